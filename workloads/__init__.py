"""Seeded synthetic inputs and random-init weights for the ModernBERT-base encoder.

This module is shared by the GPU path's tests/bench and by the oracle's callers. It holds
none of the encoder's arithmetic: only tensor shapes, random draws, and the rounding of
drawn values to the storage dtype of a run. Both sides receive the same rounded values, so
weight quantisation never counts as a parity error.

Recipe (every draw comes from ``numpy.random.default_rng([workload_id, stream])``):

* stream 0 = weights, drawn in float64 in this order: tok_emb, emb_norm, then per layer
  attn_norm (layers >= 1 only), Wqkv, attn_Wo, mlp_norm, Wi, mlp_Wo; final_norm last.
  Matrices ~ N(0, 0.02^2); norm weights ~ 1 + N(0, 0.02^2). Each value is then rounded
  (round-to-nearest-even) to the run dtype.
* stream 1 = sequence lengths, then token ids (uniform integers in [0, vocab)).

Shapes follow the model printed by kgptalkie, "ModernBERT-base Architecture Teardown",
§"What Is ModernBERT-base?" and the tensor list of candding, "ModernBERT", §"The tensors".
"""
from __future__ import annotations

from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

VOCAB = 50368
HIDDEN = 768
N_HEADS = 12
HEAD_DIM = 64
INTERMEDIATE = 1152
PAD_ID = 50283          # [PAD]; kgptalkie, §"How Does Text Become Tokens?"
MAX_POSITIONS = 8192    # candding, "ModernBERT", §"What it is"


@dataclass(frozen=True)
class Dims:
    """Model dimensions. The defaults are ModernBERT-base; tiny dims serve CPU-only tests."""
    n_layers: int = 22
    hidden: int = HIDDEN
    n_heads: int = N_HEADS
    head_dim: int = HEAD_DIM
    intermediate: int = INTERMEDIATE
    vocab: int = VOCAB


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    n_layers: int
    dtype: str              # "f32" | "bf16" | "f16": storage and GEMM-input dtype of the run
    layout: str             # "packed" (ids + cu_seqlens) or "padded" (ids [B,Tp] + mask)
    description: str
    n_seqs: int = 1
    fixed_len: int | None = None
    len_uniform: tuple[int, int] | None = None      # inclusive integer range
    len_loguniform: tuple[int, int] | None = None   # round(exp(U[ln a, ln b])), clamped to [a, b]
    pad_to: int | None = None
    extra: dict = field(default_factory=dict)


WORKLOADS: dict[int, Workload] = {
    1: Workload(1, "cycle3_fp32_L300", 3, "f32", "packed",
                "3-layer cycle (layer 0 global, layers 1-2 local), fp32, one 300-token sequence",
                n_seqs=1, fixed_len=300),
    2: Workload(2, "b8_L128-512_padded_bf16", 22, "bf16", "padded",
                "22 layers bf16, batch 8, lengths uniform in [128,512], right-padded to 512 and unpadded",
                n_seqs=8, len_uniform=(128, 512), pad_to=512),
    3: Workload(3, "L8192_bf16", 22, "bf16", "packed",
                "22 layers bf16, one 8192-token sequence",
                n_seqs=1, fixed_len=8192),
    4: Workload(4, "s64_loguniform32-2048_bf16", 22, "bf16", "packed",
                "22 layers bf16, 64 sequences, lengths log-uniform in [32,2048], packed",
                n_seqs=64, len_loguniform=(32, 2048)),
    5: Workload(5, "b32_L8192_fp16", 22, "f16", "packed",
                "22 layers fp16, 32 x 8192 tokens packed",
                n_seqs=32, fixed_len=8192),
}


def rng(workload_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(workload_id), int(stream)])


# ----------------------------------------------------------------------------------------
# Rounding of drawn float64 values to the storage dtype (round-to-nearest-even).
# ----------------------------------------------------------------------------------------
def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Exact RNE from float64 to bfloat16 (1 sign, 8 exponent, 7 mantissa bits), as float64."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    nz = x[x != 0]
    if nz.size and np.min(np.abs(nz)) < 1.2e-38:
        raise ValueError("value below the bfloat16 normal range; subnormal rounding not handled")
    if nz.size and np.max(np.abs(nz)) > 3.0e38:
        raise ValueError("value beyond the bfloat16 range")
    b = x.view(np.uint64)
    drop = np.uint64(45)                                  # 52 - 7 mantissa bits dropped
    lsb = (b >> drop) & np.uint64(1)
    b = b + (np.uint64((1 << 44) - 1) + lsb)
    b &= ~np.uint64((1 << 45) - 1)
    return b.view(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` and return them as float64 (exactly representable)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------------------
def make_weights(dims: Dims, dtype: str, seed_key: int, std: float = 0.02) -> dict:
    """Random-init weights, float64 arrays holding values representable in ``dtype``.

    Linear weights are stored [out, in] (row-major), as PyTorch's Linear stores them
    (kgptalkie, §"How Does ModernBERT Make Q, K and V?"). ``layers[0]['attn_norm']`` is None:
    layer 0 has no attention norm (candding, "ModernBERT", §"The tensors").
    """
    g = rng(seed_key, 0)
    D, I = dims.hidden, dims.intermediate

    def mat(rows, cols):
        return round_to(g.standard_normal((rows, cols)) * std, dtype)

    def norm_w(n):
        return round_to(1.0 + g.standard_normal(n) * std, dtype)

    w = {"tok_emb": mat(dims.vocab, D), "emb_norm": norm_w(D), "layers": []}
    for layer in range(dims.n_layers):
        lw = {"attn_norm": norm_w(D) if layer > 0 else None}
        lw["Wqkv"] = mat(3 * D, D)
        lw["attn_Wo"] = mat(D, D)
        lw["mlp_norm"] = norm_w(D)
        lw["Wi"] = mat(2 * I, D)
        lw["mlp_Wo"] = mat(D, I)
        w["layers"].append(lw)
    w["final_norm"] = norm_w(D)
    return w


def make_head_weights(dims: Dims, dtype: str, seed_key: int, n_labels: int = 4,
                      std: float = 0.02) -> dict:
    """Random-init weights of the heads on top of the encoder (kgptalkie, §"The Masked-LM
    Head", §"How Do We Put a Classifier on Top?"): the prediction head's dense [D, D] and norm
    weight [D], the decoder bias [vocab] (the decoder weight is the embedding table), and a
    classifier [n_labels, D] with bias [n_labels]. Stream 3 of the generator."""
    g = rng(seed_key, 3)
    D = dims.hidden
    return {
        "dense": round_to(g.standard_normal((D, D)) * std, dtype),
        "norm": round_to(1.0 + g.standard_normal(D) * std, dtype),
        "decoder_bias": round_to(g.standard_normal(dims.vocab) * std, dtype),
        "cls_W": round_to(g.standard_normal((n_labels, D)) * std, dtype),
        "cls_b": round_to(g.standard_normal(n_labels) * std, dtype),
    }


@lru_cache(maxsize=2)
def workload_weights(workload_id: int) -> dict:
    wl = WORKLOADS[workload_id]
    return make_weights(Dims(n_layers=wl.n_layers), wl.dtype, wl.id)


# ----------------------------------------------------------------------------------------
# Token batches
# ----------------------------------------------------------------------------------------
def draw_lengths(wl: Workload, g: np.random.Generator) -> np.ndarray:
    if wl.fixed_len is not None:
        return np.full(wl.n_seqs, wl.fixed_len, dtype=np.int64)
    if wl.len_uniform is not None:
        a, b = wl.len_uniform
        return g.integers(a, b + 1, size=wl.n_seqs).astype(np.int64)
    if wl.len_loguniform is not None:
        a, b = wl.len_loguniform
        raw = np.exp(g.uniform(np.log(a), np.log(b), size=wl.n_seqs))
        return np.clip(np.rint(raw), a, b).astype(np.int64)
    raise ValueError("workload has no length rule")


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def make_batch(wl: Workload, vocab: int = VOCAB) -> dict:
    """Token ids for a workload. Packed: ids [T], cu_seqlens [S+1]. Padded: additionally
    ids_pad [B,Tp] (pad id at the end of each row) and mask [B,Tp] (1 = real token)."""
    g = rng(wl.id, 1)
    lengths = draw_lengths(wl, g)
    cu = cu_from_lengths(lengths)
    ids = g.integers(0, vocab, size=int(cu[-1])).astype(np.int64)
    out = {"ids": ids, "cu_seqlens": cu, "lengths": lengths}
    if wl.layout == "padded":
        ids_pad, mask = pad_batch(ids, cu, wl.pad_to)
        out["ids_pad"], out["mask"] = ids_pad, mask
    return out


def pad_batch(ids: np.ndarray, cu: np.ndarray, pad_to: int, pad_id: int = PAD_ID):
    """Right-pad packed sequences to ``pad_to`` columns (pads at the end of each row)."""
    S = len(cu) - 1
    ids_pad = np.full((S, pad_to), pad_id, dtype=np.int64)
    mask = np.zeros((S, pad_to), dtype=np.int64)
    for s in range(S):
        L = int(cu[s + 1] - cu[s])
        if L > pad_to:
            raise ValueError("sequence longer than the padded width")
        ids_pad[s, :L] = ids[cu[s]:cu[s + 1]]
        mask[s, :L] = 1
    return ids_pad, mask


def random_batch(lengths, seed_key: int, vocab: int = VOCAB) -> dict:
    """Packed batch with the given lengths and uniform ids (for edge-case tests)."""
    g = rng(seed_key, 1)
    cu = cu_from_lengths(np.asarray(lengths, dtype=np.int64))
    ids = g.integers(0, vocab, size=int(cu[-1])).astype(np.int64)
    return {"ids": ids, "cu_seqlens": cu, "lengths": np.asarray(lengths, dtype=np.int64)}


def random_matrix(shape, seed_key: int, stream: int = 2, std: float = 1.0, dtype: str = "f32"):
    """Gaussian test operand (for per-step tests), rounded to ``dtype``."""
    g = rng(seed_key, stream)
    return round_to(g.standard_normal(shape) * std, dtype)
