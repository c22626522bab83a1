"""The allocation-free decode entry (mla_latent_decode_noalloc) against the
workspace entry (mla_latent_decode), through the C ABI: the same kernels run
on the same plan, so the outputs must agree bit for bit; both are also held
to the oracle's bar. Two calls in a row, the second with a smaller input, so
that the second call runs over the scratch contents the first one left."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
import workloads as G
from gpu_util import LSE_TOL, TOL, lse_err, rel_err, to_dev, to_host64

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(M, case, workers, noalloc):
    q = to_dev(case.q, case.dtype)
    lens = torch.from_numpy(case.lens.astype(np.int32)).cuda()
    kw = dict(num_workers=workers)
    if case.page_size is None:
        cache = to_dev(case.cache, case.dtype)
    else:
        cache = to_dev(case.pages, case.dtype)
        kw["block_table"] = torch.from_numpy(case.block_table).cuda()
    fn = M.latent_decode_noalloc if noalloc else M.latent_decode
    out, lse = fn(q, cache, lens, case.d_c, case.kq_scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case):
    outs, lses = [], []
    for b in range(case.B):
        o, l = O.latent_attention(G.to_f64(case.q[b], case.dtype), G.to_f64(G.seq_rows(case, b), case.dtype),
                                  case.d_c, case.kq_scale, int(case.lens[b]))
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("dtype", [G.BF16, G.F32])
def test_noalloc_matches_workspace_entry(dtype):
    import head_latent_attention_09_amd as M
    # fp32 partials are twice the size: 32 heads at the default worker count fit the scratch
    H0 = 128 if dtype == G.BF16 else 32
    big = G.decode_case(6, H0, 512, 64, [700, 1, 0, 1500, 257, 64], dtype, seed=301, page_size=64)
    small = G.decode_case(3, H0 // 2, 512, 64, [90, 33, 400], dtype, seed=302)
    for case, workers in ((big, 0), (small, 11)):   # second call: smaller batch, heads and workers, dense
        case.kq_scale = 1.0 / math.sqrt(192)
        say(f"noalloc: dtype={dtype} B={case.B} H={case.H} lens={list(case.lens)} paged={case.page_size} "
            f"workers={workers}")
        o1, l1 = _run(M, case, workers, noalloc=True)
        o0, l0 = _run(M, case, workers, noalloc=False)
        assert torch.equal(o1, o0) and torch.equal(l1, l0), "differs from mla_latent_decode"
        ref, rlse = _oracle(case)
        e, le = rel_err(to_host64(o1), ref), lse_err(l1.cpu().numpy().astype(np.float64), rlse)
        say(f"  vs oracle: out {e:.2e} lse {le:.2e}")
        assert e <= TOL[dtype] and le <= LSE_TOL[dtype]


def test_noalloc_rejects_oversize():
    """fp32 partials of 256 workers x 128 heads x 512 dims need 128 MiB: more
    than the scratch holds, refused before any launch."""
    import head_latent_attention_09_amd as M
    assert M.noalloc_scratch_bytes(4, 128, 512, torch.float32, 256) > M.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((4, 128, 576), dtype=torch.float32, device="cuda")
    cache = torch.zeros((4, 16, 576), dtype=torch.float32, device="cuda")
    lens = torch.full((4,), 16, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MLAError) as ei:
        M.latent_decode_noalloc(q, cache, lens, 512, 0.1, num_workers=256)
    assert ei.value.status == -4
