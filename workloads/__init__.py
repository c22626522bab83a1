"""Seeded synthetic inputs for the latent-attention path.

This package is shared by the oracle side and the HIP side. It draws random
numbers, applies the input-preparation steps that sit upstream of the path
(RMS normalisation of the latent, rotary position rotation of the rope parts,
the tiny notebook's down-projections) and stores the results in the storage
dtype (fp32, or bf16 bit patterns rounded to nearest even). It holds none of
the attention arithmetic: no scores, no softmax, no weighted sums, no
absorption and no up-projection.
"""
from .gen import *  # noqa: F401,F403
