"""Host-side checks of the Python binding's argument validation: every
wrapper compares each tensor with the query (dtype, device, shape) and
raises before calling the C ABI. Uses CPU tensors: a consistent set reaches
the final device check and is rejected there, so nothing is ever launched."""
import pytest
import torch

import head_latent_attention_09_amd as M

BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def gpu_only(fn):
    with pytest.raises(ValueError, match="CUDA"):
        fn()


def test_absorb_checks():
    qn, qp, w = z(4, 2, 8), z(4, 2, 3), z(2, 8, 16)
    gpu_only(lambda: M.absorb_q(qn, qp, w))
    with pytest.raises(TypeError):
        M.absorb_q(qn, qp, z(2, 8, 16, dtype=F32))          # weight dtype differs
    with pytest.raises(ValueError):
        M.absorb_q(qn, qp, z(3, 8, 16))                     # head count differs
    with pytest.raises(ValueError):
        M.absorb_q(qn, z(4, 1, 3), w)                       # q_pe shape
    with pytest.raises(ValueError):
        M.absorb_q(qn, qp, w, out=z(4, 2, 18))              # out too narrow
    with pytest.raises(TypeError):
        M.absorb_q(z(4, 2, 8, dtype=torch.float16), None, z(2, 8, 16, dtype=torch.float16))


def test_up_v_checks():
    lat, w = z(4, 2, 16), z(2, 8, 16)
    gpu_only(lambda: M.up_v(lat, w))
    with pytest.raises(ValueError):
        M.up_v(lat, z(2, 8, 15))
    with pytest.raises(TypeError):
        M.up_v(lat, w, out=z(4, 2, 8, dtype=F32))
    with pytest.raises(ValueError):
        M.up_v(lat, w, out=z(4, 2, 7))


def test_decode_checks():
    q, cache, lens = z(3, 4, 20), z(3, 10, 20), z(3, dtype=I32)
    gpu_only(lambda: M.latent_decode(q, cache, lens, 16, 0.3))
    with pytest.raises(ValueError):
        M.latent_decode(q, z(3, 10, 21), lens, 16, 0.3)     # cache row width
    with pytest.raises(TypeError):
        M.latent_decode(q, z(3, 10, 20, dtype=F32), lens, 16, 0.3)
    with pytest.raises(ValueError):
        M.latent_decode(q, z(2, 10, 20), lens, 16, 0.3)     # fewer dense sequences than the batch
    with pytest.raises(ValueError):
        M.latent_decode(q, cache, z(2, dtype=I32), 16, 0.3)  # seq_lens too short
    with pytest.raises(TypeError):
        M.latent_decode(q, cache, z(3, dtype=torch.int64), 16, 0.3)
    with pytest.raises(ValueError):
        M.latent_decode(q, cache, lens, 21, 0.3)            # d_c wider than the row
    with pytest.raises(ValueError):
        M.latent_decode(q, cache, lens, 16, 0.3, out=z(3, 4, 15))
    with pytest.raises(TypeError):
        M.latent_decode(q, cache, lens, 16, 0.3, lse=z(3, 4))   # lse must be fp32
    with pytest.raises(ValueError):
        M.latent_decode(q, cache, lens, 16, 0.3, lse=z(3, 5, dtype=F32))
    # paged
    pool, table = z(7, 16, 20), z(3, 2, dtype=I32)
    gpu_only(lambda: M.latent_decode(q, pool, lens, 16, 0.3, block_table=table))
    with pytest.raises(ValueError):
        M.latent_decode(q, pool, lens, 16, 0.3, block_table=z(2, 2, dtype=I32))
    with pytest.raises(ValueError):
        M.latent_decode(q, pool, lens, 16, 0.3, block_table=table, num_pages=8)
    with pytest.raises(TypeError):
        M.latent_decode(q, pool, lens, 16, 0.3, block_table=z(3, 2, dtype=torch.int64))


def test_decode_up_v_checks():
    q, cache, lens, w = z(3, 4, 20), z(3, 10, 20), z(3, dtype=I32), z(4, 8, 16)
    gpu_only(lambda: M.latent_decode_up_v(q, cache, lens, 16, 0.3, w))
    with pytest.raises(ValueError):
        M.latent_decode_up_v(q, cache, lens, 16, 0.3, z(4, 8, 20))
    with pytest.raises(ValueError):
        M.latent_decode_up_v(q, cache, lens, 16, 0.3, w, out=z(3, 4, 16))


def test_prefill_checks():
    q, cache = z(2, 5, 4, 20), z(2, 7, 20)
    gpu_only(lambda: M.latent_prefill_causal(q, cache, 16, 0.3))
    with pytest.raises(ValueError):
        M.latent_prefill_causal(q, z(1, 7, 20), 16, 0.3)
    with pytest.raises(ValueError):
        M.latent_prefill_causal(q, cache, 16, 0.3, out=z(2, 5, 4, 20))
    with pytest.raises(ValueError):
        M.latent_prefill_causal(q, cache, 16, 0.3, lse=z(2, 5, 3, dtype=F32))


def test_combine_checks():
    o, l = z(3, 2, 4, 8, dtype=F32), z(3, 2, 4, dtype=F32)
    gpu_only(lambda: M.lse_combine(o, l))
    with pytest.raises(TypeError):
        M.lse_combine(o.to(BF), l)
    with pytest.raises(ValueError):
        M.lse_combine(o, z(3, 2, 5, dtype=F32))
    with pytest.raises(ValueError):
        M.lse_combine(o, l, out=z(2, 4, 9, dtype=F32))
