"""The oracle: TEST INFRASTRUCTURE ONLY.

A plain float64 CPU statement of the ModernBERT-base encoder forward, used to check the GPU
path. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import it;
the product path (transformer_encoder_amd) never does.
"""
from .mbert_oracle import *  # noqa: F401,F403
from . import brute  # noqa: F401
