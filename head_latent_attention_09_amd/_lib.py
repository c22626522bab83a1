"""ctypes binding of libmla.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmla. PyTorch supplies device memory (tensors) and the stream
(torch.cuda.current_stream()). Loading fails loudly if the library has not
been built; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
STATUS = {0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_DTYPE",
          -4: "MLA_ERR_UNSUPPORTED", -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_ALIGN",
          -7: "MLA_ERR_SCALE", -8: "MLA_ERR_HIP"}

# (name, restype, argtypes) of every exported entry point
_c = ctypes
_vp, _i, _i64, _f, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t
SIGNATURES = [
    ("mla_status_string", _c.c_char_p, [_i]),
    ("mla_version", _i, []),
    ("mla_default_workers", _i, []),
    ("mla_absorb_q", _i, [_vp, _vp, _vp, _vp, _i64, _i, _i, _i, _i, _i, _vp]),
    ("mla_up_v", _i, [_vp, _vp, _vp, _i64, _i, _i, _i, _i, _vp]),
    ("mla_latent_decode_workspace", _sz, [_i, _i, _i, _i]),
    ("mla_latent_decode", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _i,
                               _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    ("mla_latent_decode_up_v_workspace", _sz, [_i, _i, _i, _i]),
    ("mla_latent_decode_up_v", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _i,
                                    _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    ("mla_latent_prefill_causal_workspace", _sz, [_i, _i, _i, _i, _i]),
    ("mla_latent_prefill_causal", _i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                                       _vp, _vp, _vp, _sz, _i, _vp, _vp]),
    ("mla_lse_combine", _i, [_vp, _vp, _i, _i64, _i, _i, _i, _vp, _vp, _vp]),
]


class MLAError(RuntimeError):
    def __init__(self, fn, status, lib=None):
        text = STATUS.get(status, str(status))
        if lib is not None:
            text += ": " + lib.mla_status_string(status).decode()
        super().__init__(f"{fn} failed with {text}")
        self.status = status


def load_library(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m head_latent_attention_09_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load_library()


def _check(fn, status):
    if status != 0:
        raise MLAError(fn, status, lib)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _events(timing_events):
    if timing_events is None:
        return None
    for e in timing_events:  # torch creates the underlying hipEvent_t on first record
        if not e.cuda_event:
            e.record(torch.cuda.current_stream())
    arr = (ctypes.c_void_p * 2)(timing_events[0].cuda_event, timing_events[1].cuda_event)
    return ctypes.cast(arr, ctypes.c_void_p), arr  # keep arr alive with the pointer


def default_workers() -> int:
    n = lib.mla_default_workers()
    if n <= 0:
        raise MLAError("mla_default_workers", n, lib)
    return n


# ----------------------------------------------------------------------------
def absorb_q(q_nope, q_pe, w_uk, out=None):
    """q[n,h,:d_c] = W_UK[h]^T q_nope[n,h,:]; q[n,h,d_c:] = q_pe[n,h,:].

    q_nope [N,H,d_nope], q_pe [N,H,d_r] (or None), w_uk [H,d_nope,d_c]."""
    _dev(q_nope, "q_nope"), _dev(w_uk, "w_uk")
    N, H, d_nope = q_nope.shape
    d_c = w_uk.shape[2]
    d_r = 0 if q_pe is None else q_pe.shape[2]
    if q_pe is not None:
        _dev(q_pe, "q_pe")
    if out is None:
        out = torch.empty((N, H, d_c + d_r), dtype=q_nope.dtype, device=q_nope.device)
    _check("mla_absorb_q", lib.mla_absorb_q(_ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(_dev(out, "out")),
                                            N, H, d_nope, d_c, d_r, _dtype_code(q_nope), _stream()))
    return out


def up_v(out_lat, w_uv, out=None):
    """out[n,h,i] = sum_j W_UV[h,i,j] out_lat[n,h,j]; out_lat [N,H,d_c], w_uv [H,d_v,d_c]."""
    _dev(out_lat, "out_lat"), _dev(w_uv, "w_uv")
    N, H, d_c = out_lat.shape
    d_v = w_uv.shape[1]
    if out is None:
        out = torch.empty((N, H, d_v), dtype=out_lat.dtype, device=out_lat.device)
    _check("mla_up_v", lib.mla_up_v(_ptr(out_lat), _ptr(w_uv), _ptr(_dev(out, "out")), N, H, d_c, d_v,
                                    _dtype_code(out_lat), _stream()))
    return out


def decode_workspace_bytes(batch, n_heads, d_c, num_workers=0) -> int:
    return int(lib.mla_latent_decode_workspace(batch, n_heads, d_c, num_workers))


def prefill_workspace_bytes(batch, s_q, n_heads, d_c, num_workers=0) -> int:
    return int(lib.mla_latent_prefill_causal_workspace(batch, s_q, n_heads, d_c, num_workers))


def _workspace(nbytes, device, workspace):
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def latent_decode(q, cache, seq_lens, d_c, kq_scale, block_table=None, num_pages=None, num_workers=0,
                  out=None, lse=None, want_lse=True, workspace=None, timing_events=None):
    """Absorbed decode over a dense [B,S,W] or paged [P,page,W] latent cache.

    q [B,H,W] rows [q_abs | q_pe]; seq_lens int32 [B]; block_table int32
    [B,max_pages] or None. Returns (out_lat [B,H,d_c], lse [B,H] or None)."""
    _dev(q, "q"), _dev(cache, "cache"), _dev(seq_lens, "seq_lens")
    B, H, W = q.shape
    d_r = W - d_c
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if block_table is not None:
        _dev(block_table, "block_table")
        if block_table.dtype != torch.int32:
            raise TypeError("block_table must be int32")
        page_size, max_pages = cache.shape[1], block_table.shape[1]
        num_pages = cache.shape[0] if num_pages is None else num_pages
        stride = 0
    else:
        page_size = max_pages = num_pages = 0
        stride = cache.shape[1]
    if out is None:
        out = torch.empty((B, H, d_c), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nb = decode_workspace_bytes(B, H, d_c, num_workers)
    ws = _workspace(nb, q.device, workspace)
    ev = _events(timing_events)
    _check("mla_latent_decode", lib.mla_latent_decode(
        _ptr(q), _ptr(cache), _ptr(seq_lens), _ptr(block_table), B, H, d_c, d_r, stride, page_size,
        max_pages, num_pages, float(kq_scale), _dtype_code(q), _ptr(_dev(out, "out")), _ptr(lse),
        _ptr(ws), ws.numel(), num_workers, None if ev is None else ev[0], _stream()))
    return out, lse


def decode_up_v_workspace_bytes(batch, n_heads, d_c, num_workers=0) -> int:
    return int(lib.mla_latent_decode_up_v_workspace(batch, n_heads, d_c, num_workers))


def latent_decode_up_v(q, cache, seq_lens, d_c, kq_scale, w_uv, block_table=None, num_pages=None, num_workers=0,
                       out=None, lse=None, want_lse=True, workspace=None, timing_events=None):
    """Absorbed decode and the W_UV up-projection in one call.

    As latent_decode, plus w_uv [H,d_v,d_c]. Returns (v [B,H,d_v], lse [B,H] or None)."""
    _dev(q, "q"), _dev(cache, "cache"), _dev(seq_lens, "seq_lens"), _dev(w_uv, "w_uv")
    B, H, W = q.shape
    d_r = W - d_c
    d_v = w_uv.shape[1]
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    if block_table is not None:
        _dev(block_table, "block_table")
        if block_table.dtype != torch.int32:
            raise TypeError("block_table must be int32")
        page_size, max_pages = cache.shape[1], block_table.shape[1]
        num_pages = cache.shape[0] if num_pages is None else num_pages
        stride = 0
    else:
        page_size = max_pages = num_pages = 0
        stride = cache.shape[1]
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nb = decode_up_v_workspace_bytes(B, H, d_c, num_workers)
    ws = _workspace(nb, q.device, workspace)
    ev = _events(timing_events)
    _check("mla_latent_decode_up_v", lib.mla_latent_decode_up_v(
        _ptr(q), _ptr(cache), _ptr(seq_lens), _ptr(block_table), B, H, d_c, d_r, stride, page_size,
        max_pages, num_pages, float(kq_scale), _ptr(w_uv), d_v, _dtype_code(q), _ptr(_dev(out, "out")), _ptr(lse),
        _ptr(ws), ws.numel(), num_workers, None if ev is None else ev[0], _stream()))
    return out, lse


def latent_prefill_causal(q, cache, d_c, kq_scale, num_workers=0, out=None, lse=None, want_lse=True,
                          workspace=None, timing_events=None):
    """Causal prefill: q [B,S_q,H,W], cache [B,S_kv,W]; query i sees t <= i + S_kv - S_q.
    Returns (out_lat [B,S_q,H,d_c], lse [B,S_q,H] or None)."""
    _dev(q, "q"), _dev(cache, "cache")
    B, S_q, H, W = q.shape
    S_kv = cache.shape[1]
    d_r = W - d_c
    if out is None:
        out = torch.empty((B, S_q, H, d_c), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, S_q, H), dtype=torch.float32, device=q.device)
    nb = prefill_workspace_bytes(B, S_q, H, d_c, num_workers)
    ws = _workspace(nb, q.device, workspace)
    ev = _events(timing_events)
    _check("mla_latent_prefill_causal", lib.mla_latent_prefill_causal(
        _ptr(q), _ptr(cache), B, S_q, S_kv, H, d_c, d_r, float(kq_scale), _dtype_code(q),
        _ptr(_dev(out, "out")), _ptr(lse), _ptr(ws), ws.numel(), num_workers,
        None if ev is None else ev[0], _stream()))
    return out, lse


def lse_combine(o_parts, lse_parts, dtype=torch.float32, out=None, want_lse=True):
    """Merge partial softmax results: o_parts [P,R,H,d_c] fp32, lse_parts [P,R,H] fp32."""
    _dev(o_parts, "o_parts"), _dev(lse_parts, "lse_parts")
    P, R, H, d_c = o_parts.shape
    if out is None:
        out = torch.empty((R, H, d_c), dtype=dtype, device=o_parts.device)
    lse = torch.empty((R, H), dtype=torch.float32, device=o_parts.device) if want_lse else None
    _check("mla_lse_combine", lib.mla_lse_combine(_ptr(o_parts), _ptr(lse_parts), P, R, H, d_c,
                                                  _dtype_code(out), _ptr(out), _ptr(lse), _stream()))
    return out, lse


def kq_scale_for(d_nope: int, d_r: int) -> float:
    """1/sqrt(d_nope + d_r): the width of the unabsorbed head."""
    return 1.0 / math.sqrt(d_nope + d_r)
