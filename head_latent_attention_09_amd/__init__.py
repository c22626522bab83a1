"""Weight-absorbed Multi-head Latent Attention for MI355X (gfx950).

The computation lives in libmla.so (hand-written HIP kernels behind the C
ABI declared in include/mla.h); this package is its Python binding.
"""
from ._lib import (LIB_PATH, MLA_BF16, MLA_F32, MLAError, SIGNATURES, absorb_q,  # noqa: F401
                   decode_up_v_workspace_bytes, decode_workspace_bytes, default_workers,
                   latent_decode, latent_decode_noalloc, latent_decode_up_v, latent_prefill_causal, lib, lse_combine,
                   noalloc_scratch_bytes, NOALLOC_SCRATCH_BYTES, prefill_workspace_bytes, up_v,
                   cache_append, absorb_q_rope, prefill_unabsorbed, prefill_unabsorbed_workspace_bytes,
                   absorb_weights, absorb_q_full, out_absorbed, gated_mla)
