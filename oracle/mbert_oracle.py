"""ModernBERT-base encoder forward: the oracle.

TEST INFRASTRUCTURE ONLY. A plain, slow CPU implementation in float64 of what the encoder
computes, written from the pages listed below. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code with the GPU
path (``transformer_encoder_amd``) and imports nothing from this repository.

Sources, cited by page and section:
  [KGP]  kgptalkie.com, "ModernBERT-base Architecture Teardown: Every Layer With Real Code"
  [RAY]  rayaq.ca, "Encoder-only models"
  [CAN]  candding docs, "ModernBERT"
  [SBD]  safebydesign.ai, "ModernBertModel 22L 768d"
  [NEST] nest.franknoh.dev, "modernbert-base"

Library primitives used as steps: numpy matmul (``@``), numpy exp/cos/sin/sqrt, and
``scipy.special.erf`` for the error function.

Pins (tests/test_oracle_pins.py, tests/test_oracle_brute.py): every function below is pinned
by values the pages print, by closed forms, invariants, or by an independent pure-Python
brute force (oracle/brute.py). The end-to-end 22-layer values are *parity unpinned by the
pages* (no trained weights or per-token outputs are printed): they are pinned only through
their parts, the invariants (packed == padded, pad invariance, non-causality) and the
brute force at tiny sizes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import erf as _erf


@dataclass(frozen=True)
class Config:
    """Model hyper-parameters. Defaults: ModernBERT-base ([KGP] §"What Is ModernBERT-base?":
    22 layers, 768 wide, 12 heads, MLP 1152; [CAN] §"What it is", §"The alternating
    attention", §"The two rope tables": global every 3rd layer, half window 64, bases
    160000/10000; LayerNorm eps 1e-5 from the printed model)."""
    n_layers: int = 22
    hidden: int = 768
    n_heads: int = 12
    head_dim: int = 64
    intermediate: int = 1152
    vocab: int = 50368
    global_every: int = 3
    half_window: int = 64
    theta_global: float = 160000.0
    theta_local: float = 10000.0
    eps: float = 1e-5


# ----------------------------------------------------------------------------------------
# Model structure
# ----------------------------------------------------------------------------------------
def is_global_layer(layer: int, cfg: Config = Config()) -> bool:
    """Layer i attends over the whole sequence iff i % 3 == 0, layer 0 included
    ([CAN] §"What it is"; [KGP] §"What Are Local and Global Attention?")."""
    return layer % cfg.global_every == 0


def global_layers(cfg: Config = Config()) -> list[int]:
    return [i for i in range(cfg.n_layers) if is_global_layer(i, cfg)]


def parameter_shapes(cfg: Config = Config()) -> dict[str, tuple[int, ...]]:
    """Every weight tensor of the encoder with its [out, in] shape ([CAN] §"The tensors";
    [KGP] §"Where Do the 149M Parameters Sit?"). No tensor carries a bias; layer 0 has no
    attn_norm."""
    D, I = cfg.hidden, cfg.intermediate
    shapes = {"embeddings.tok_embeddings.weight": (cfg.vocab, D),
              "embeddings.norm.weight": (D,),
              "final_norm.weight": (D,)}
    for i in range(cfg.n_layers):
        p = f"layers.{i}."
        if i > 0:
            shapes[p + "attn_norm.weight"] = (D,)
        shapes[p + "attn.Wqkv.weight"] = (3 * D, D)
        shapes[p + "attn.Wo.weight"] = (D, D)
        shapes[p + "mlp_norm.weight"] = (D,)
        shapes[p + "mlp.Wi.weight"] = (2 * I, D)
        shapes[p + "mlp.Wo.weight"] = (D, I)
    return shapes


# ----------------------------------------------------------------------------------------
# Unpadding
# ----------------------------------------------------------------------------------------
def unpad(ids_pad, mask) -> dict:
    """Strip padding before the layers run ([KGP] §"What Is ModernBERT-base?" says the model
    removes pad tokens before the layers; §"How Does Text Become Tokens?": the mask marks real
    tokens with 1). Scans the rows in order; a real token's position is its rank among the
    real tokens of its row (positions restart at 0 for every row, [CAN] §"The two rope
    tables").

    Returns ids [T], indices [T] (flat b*Tp+t of each real token, ascending), pos [T],
    cu_seqlens [B+1], max_seqlen."""
    ids_pad = np.asarray(ids_pad)
    mask = np.asarray(mask)
    B, Tp = mask.shape
    ids, indices, pos, cu = [], [], [], [0]
    for b in range(B):
        rank = 0
        for t in range(Tp):
            if mask[b, t] != 0:
                ids.append(int(ids_pad[b, t]))
                indices.append(b * Tp + t)
                pos.append(rank)
                rank += 1
        cu.append(cu[-1] + rank)
    lengths = [cu[b + 1] - cu[b] for b in range(B)]
    return {"ids": np.array(ids, dtype=np.int64),
            "indices": np.array(indices, dtype=np.int64),
            "pos": np.array(pos, dtype=np.int64),
            "cu_seqlens": np.array(cu, dtype=np.int64),
            "max_seqlen": max(lengths, default=0)}


def positions(cu_seqlens) -> np.ndarray:
    """Position of each packed token inside its own sequence: 0 .. L-1 ([CAN] §"The two rope
    tables")."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.zeros(int(cu[-1]), dtype=np.int64)
    for s in range(len(cu) - 1):
        pos[cu[s]:cu[s + 1]] = np.arange(cu[s + 1] - cu[s])
    return pos


# ----------------------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------------------
def layernorm(x, w, eps: float) -> np.ndarray:
    """Weight-only LayerNorm over the last axis: subtract the mean, divide by the square root
    of the biased (population) variance plus eps, multiply by the weight; no bias
    ([KGP] §"What Does LayerNorm Do?"; [CAN] §"The pre-norm layer and the final norm")."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * np.asarray(w, dtype=np.float64)


def gelu_erf(z) -> np.ndarray:
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)); not the tanh form
    ([CAN] §"The feed-forward halves"; [NEST] §"Why the GELU matters")."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def geglu(u, intermediate: int) -> np.ndarray:
    """GeGLU on the Wi output: the first half goes through GELU, the second half multiplies it
    ([KGP] §"What Does the GeGLU MLP Do?"; [CAN] §"The feed-forward halves";
    [NEST] §"The fused projections")."""
    u = np.asarray(u, dtype=np.float64)
    return gelu_erf(u[..., :intermediate]) * u[..., intermediate:2 * intermediate]


# ----------------------------------------------------------------------------------------
# Rotary position embedding
# ----------------------------------------------------------------------------------------
def rope_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """Turn per token of pair i: theta^(-2i/head_dim), i = 0 .. head_dim/2 - 1
    ([KGP] §"How Does RoPE Work With Two Bases?")."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(theta) ** (-2.0 * i / head_dim)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE over the full head: x [..., T, head_dim], pos [T].
    Pair (i, i + head_dim/2) turns by angle pos * theta^(-2i/head_dim)
    ([CAN] §"The two rope tables": rotate-half convention over the full 64-wide head;
    [KGP] §"How Does RoPE Work With Two Bases?")."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    angle = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(theta, hd)[None, :]
    c, s = np.cos(angle), np.sin(angle)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------
def band_allowed(pos_q, pos_k, is_global: bool, half_window: int) -> np.ndarray:
    """Which keys a query may read. Global layers: every key of the sequence. Local layers:
    key j for query i iff |i - j| <= half_window, inclusive, so an interior query reads 129
    keys ([CAN] §"The alternating attention"; [NEST] §"The sliding window";
    [KGP] §"What Are Local and Global Attention?")."""
    pq = np.asarray(pos_q)[:, None]
    pk = np.asarray(pos_k)[None, :]
    if is_global:
        return np.ones((pq.shape[0], pk.shape[1]), dtype=bool)
    return np.abs(pk - pq) <= half_window


def attention_probs(q, k, allowed) -> np.ndarray:
    """softmax(q k^T / sqrt(head_dim)) over the allowed keys of each row; disallowed keys get
    -inf, hence weight exactly 0 ([KGP] §"How Does Self-Attention Work?"; [RAY] §"Padding
    and the key padding mask" for the -inf mask). q [Lq, hd], k [Lk, hd].
    A row with no allowed key at all (only a pad query of a padded batch can have one) gets
    all-zero weights; such rows are never read."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    allowed = np.broadcast_to(np.asarray(allowed, dtype=bool), (q.shape[0], k.shape[0]))
    scores = (q @ k.T) / math.sqrt(q.shape[-1])
    scores = np.where(allowed, scores, -np.inf)
    empty = ~allowed.any(axis=-1, keepdims=True)
    m = np.where(empty, 0.0, scores.max(axis=-1, keepdims=True))
    e = np.exp(scores - m)
    z = np.where(empty, 1.0, e.sum(axis=-1, keepdims=True))
    return e / z


def attention_sequence(q, k, v, is_global: bool, half_window: int,
                       key_valid=None, chunk: int = 1024) -> np.ndarray:
    """Bidirectional attention of one sequence, every head. q, k, v: [L, H, hd] (already
    rotated). ``key_valid`` [L] (optional) masks pad keys with -inf ([RAY] §"Padding and the
    key padding mask"). Query rows are processed in chunks; for a local layer only the keys
    that can fall in a chunk's window are scored (all others would get weight exactly 0)."""
    L, H, hd = q.shape
    out = np.zeros((L, H, hd), dtype=np.float64)
    pos = np.arange(L)
    for a in range(0, L, chunk):
        b = min(L, a + chunk)
        if is_global:
            k0, k1 = 0, L
        else:
            k0, k1 = max(0, a - half_window), min(L, b + half_window)
        allowed = band_allowed(pos[a:b], pos[k0:k1], is_global, half_window)
        if key_valid is not None:
            allowed = allowed & np.asarray(key_valid[k0:k1], dtype=bool)[None, :]
        for h in range(H):
            p = attention_probs(q[a:b, h], k[k0:k1, h], allowed)
            out[a:b, h] = p @ v[k0:k1, h]
    return out


def key_ranges(cu_seqlens, is_global: bool, half_window: int):
    """For each packed token, the first and last packed token index (inclusive) its query may
    read: the whole sequence on global layers, the +-half_window band clipped to the sequence
    on local layers ([CAN] §"The alternating attention"). Returns (lo [T], hi [T])."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    lo = np.zeros(T, dtype=np.int64)
    hi = np.zeros(T, dtype=np.int64)
    for s in range(len(cu) - 1):
        s0, s1 = int(cu[s]), int(cu[s + 1])
        for t in range(s0, s1):
            if is_global:
                lo[t], hi[t] = s0, s1 - 1
            else:
                lo[t], hi[t] = max(s0, t - half_window), min(s1 - 1, t + half_window)
    return lo, hi


# ----------------------------------------------------------------------------------------
# Encoder layer and the full forward
# ----------------------------------------------------------------------------------------
def split_qkv(qkv, cfg: Config):
    """Fused Wqkv output [T, 3*D] -> q, k, v each [T, H, hd]: columns 0..D-1 are the query,
    D..2D-1 the key, 2D..3D-1 the value, each laid out head by head ([CAN] §"The tensors";
    [KGP] §"How Does ModernBERT Make Q, K and V?": view(T, 3, 12, 64))."""
    T = qkv.shape[0]
    parts = qkv.reshape(T, 3, cfg.n_heads, cfg.head_dim)
    return parts[:, 0], parts[:, 1], parts[:, 2]


def qkv_projection(h, Wqkv, pos, theta: float, cfg: Config, apply_rope: bool = True):
    """qkv = h Wqkv^T with the query and key parts rotated at each row's position
    ([KGP] §"How Does ModernBERT Make Q, K and V?"; [CAN] §"The two rope tables": q and k
    only, every head, rotate-half). Returns [T, 3D] in the fused column order."""
    qkv = np.asarray(h, dtype=np.float64) @ np.asarray(Wqkv, dtype=np.float64).T
    if not apply_rope:
        return qkv
    T = qkv.shape[0]
    q, k, v = split_qkv(qkv, cfg)
    q = rope(q.transpose(1, 0, 2), pos, theta).transpose(1, 0, 2)
    k = rope(k.transpose(1, 0, 2), pos, theta).transpose(1, 0, 2)
    return np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)


def attention_varlen(qkv, segments, is_global: bool, cfg: Config) -> np.ndarray:
    """Attention of a packed batch: each segment (start, end, key_valid or None) is one
    sequence; heads are concatenated back in order ([SBD] §"Implementing it"). Returns
    [T, D]."""
    q, k, v = split_qkv(np.asarray(qkv, dtype=np.float64), cfg)
    a = np.zeros_like(q)
    for (s0, s1, key_valid) in segments:
        if s1 > s0:
            a[s0:s1] = attention_sequence(q[s0:s1], k[s0:s1], v[s0:s1], is_global,
                                          cfg.half_window, key_valid)
    return a.reshape(q.shape[0], cfg.hidden)


def segments_of(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return [(int(cu[s]), int(cu[s + 1]), None) for s in range(len(cu) - 1)]


def residual_linear(x, a, W) -> np.ndarray:
    """x + a W^T: a bias-free Linear added back to the residual stream ([KGP] §"What Does
    LayerNorm Do?": after each block its output is added back to its input)."""
    return np.asarray(x, dtype=np.float64) + np.asarray(a, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def mlp_in_geglu(h, Wi, cfg: Config) -> np.ndarray:
    """geglu(h Wi^T) ([KGP] §"What Does the GeGLU MLP Do?")."""
    return geglu(np.asarray(h, dtype=np.float64) @ np.asarray(Wi, dtype=np.float64).T, cfg.intermediate)


def encoder_layer(x, lw: dict, layer: int, segments, pos, cfg: Config) -> np.ndarray:
    """One pre-norm block ([CAN] §"The pre-norm layer and the final norm";
    [SBD] §"Implementing it"):
        h = x (layer 0: attn_norm is the identity) or LN(x; attn_norm)
        q, k, v = split(h Wqkv^T); rotate q and k (theta by layer kind)
        a = attention per sequence; x = x + a Wo^T
        h = LN(x; mlp_norm); x = x + geglu(h Wi^T) Wo2^T
    ``segments``: list of (start, end, key_valid or None), one per sequence; attention never
    crosses a segment boundary."""
    g = is_global_layer(layer, cfg)
    if layer == 0:
        if lw.get("attn_norm") is not None:
            raise ValueError("layer 0 has no attention norm")
        h = x
    else:
        h = layernorm(x, lw["attn_norm"], cfg.eps)
    theta = cfg.theta_global if g else cfg.theta_local
    qkv = qkv_projection(h, lw["Wqkv"], pos, theta, cfg)
    a = attention_varlen(qkv, segments, g, cfg)
    x = residual_linear(x, a, lw["attn_Wo"])
    h = layernorm(x, lw["mlp_norm"], cfg.eps)
    return residual_linear(x, mlp_in_geglu(h, lw["Wi"], cfg), lw["mlp_Wo"])


def embed(ids, weights: dict, cfg: Config) -> np.ndarray:
    """Pick embedding rows, then the embedding LayerNorm; no position vector is added
    ([KGP] §"How Do Token Ids Become Vectors?"). Dropout has p = 0 and is the identity."""
    E = np.asarray(weights["tok_emb"])
    return layernorm(np.asarray(E[np.asarray(ids, dtype=np.int64)], dtype=np.float64),
                     weights["emb_norm"], cfg.eps)


def mean_pool_normalize(out, cu_seqlens, l2_eps: float = 1e-12) -> np.ndarray:
    """Mean over the real tokens of each sequence, then L2 normalisation
    ([KGP] §"How Do We Get One Vector per Text?"; [SBD] §"Implementing it": the sentence
    vector is normalize(pool(x))). An empty sequence pools to the zero vector."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.asarray(out, dtype=np.float64)
    S = len(cu) - 1
    pooled = np.zeros((S, out.shape[1]), dtype=np.float64)
    for s in range(S):
        if cu[s + 1] > cu[s]:
            v = out[cu[s]:cu[s + 1]].mean(axis=0)
            pooled[s] = v / max(float(np.sqrt((v * v).sum())), l2_eps)
    return pooled


def encode(ids, cu_seqlens, weights: dict, cfg: Config = Config(), n_layers: int | None = None,
           return_hidden: bool = False):
    """The encoder forward on a packed (unpadded) batch: embedding + LN, the layer stack,
    the final LayerNorm once ([CAN] §"The pre-norm layer and the final norm"), then mean
    pooling with L2 normalisation. Returns (out [T, D], pooled [S, D])."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = positions(cu)
    segments = [(int(cu[s]), int(cu[s + 1]), None) for s in range(len(cu) - 1)]
    x = embed(ids, weights, cfg)
    hidden = [x]
    for layer in range(cfg.n_layers if n_layers is None else n_layers):
        x = encoder_layer(x, weights["layers"][layer], layer, segments, pos, cfg)
        hidden.append(x)
    out = layernorm(x, weights["final_norm"], cfg.eps)
    pooled = mean_pool_normalize(out, cu)
    if return_hidden:
        return out, pooled, hidden
    return out, pooled


def encode_padded(ids_pad, mask, weights: dict, cfg: Config = Config()):
    """The encoder forward on a padded batch run as is: every row at its full padded width,
    positions 0 .. Tp-1, pad keys masked with -inf ([RAY] §"Padding and the key padding
    mask"; [KGP] §"How Does Text Become Tokens?"). Pad rows are computed and then zeroed.
    Returns (out [B, Tp, D] with zeros at pads, pooled [B, D] over the real tokens)."""
    ids_pad = np.asarray(ids_pad, dtype=np.int64)
    mask = np.asarray(mask)
    B, Tp = ids_pad.shape
    out = np.zeros((B, Tp, cfg.hidden), dtype=np.float64)
    pooled = np.zeros((B, cfg.hidden), dtype=np.float64)
    pos = np.arange(Tp)
    for b in range(B):
        valid = mask[b] != 0
        L = int(valid.sum())
        if L == 0:
            continue
        x = embed(ids_pad[b], weights, cfg)
        for layer in range(cfg.n_layers):
            x = encoder_layer(x, weights["layers"][layer], layer, [(0, Tp, valid)], pos, cfg)
        y = layernorm(x, weights["final_norm"], cfg.eps)
        out[b] = np.where(valid[:, None], y, 0.0)
        v = (y * valid[:, None]).sum(axis=0) / L
        pooled[b] = v / max(float(np.sqrt((v * v).sum())), 1e-12)
    return out, pooled


def repad(out, indices, B: int, Tp: int) -> np.ndarray:
    """Scatter packed rows back to [B, Tp, D], zeros at the pads (the zero-filled unpacking
    of [RAY] §"Padding and the key padding mask")."""
    out = np.asarray(out, dtype=np.float64)
    res = np.zeros((B * Tp, out.shape[1]), dtype=np.float64)
    res[np.asarray(indices, dtype=np.int64)] = out
    return res.reshape(B, Tp, out.shape[1])


# ---------------------------------------------------------------------------- heads and pooling
# The masked-LM and classification heads on top of the encoder ([KGP] §"The Masked-LM Head",
# §"How Do We Put a Classifier on Top?"): both start with the same prediction head, a Linear
# 768 -> 768 without bias, GELU, and a LayerNorm. The model's other LayerNorms carry no bias
# and the page's printout of this one names none; it is read as weight-only like the rest.

def prediction_head(x, W_dense, norm_w, eps: float) -> np.ndarray:
    """LN(gelu_erf(x W_dense^T); norm_w) ([KGP] §"The Masked-LM Head": dense, GELU, LayerNorm)."""
    u = np.asarray(x, dtype=np.float64) @ np.asarray(W_dense, dtype=np.float64).T
    return layernorm(gelu_erf(u), norm_w, eps)


def mlm_logits(x, W_dense, norm_w, tok_emb, decoder_bias, eps: float) -> np.ndarray:
    """Vocabulary scores: the prediction head, then the decoder, whose weight is the embedding
    table itself (weight tying) and which carries a bias ([KGP] §"The Masked-LM Head")."""
    h = prediction_head(x, W_dense, norm_w, eps)
    return h @ np.asarray(tok_emb, dtype=np.float64).T + np.asarray(decoder_bias, dtype=np.float64)


def mean_pool(out, cu_seqlens) -> np.ndarray:
    """Mean over each sequence's rows, not normalised (the pooling the classifier reads,
    [KGP] §"How Do We Get One Vector per Text?", §"How Do We Put a Classifier on Top?").
    An empty sequence pools to zero."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.asarray(out, dtype=np.float64)
    pooled = np.zeros((len(cu) - 1, out.shape[1]), dtype=np.float64)
    for s in range(len(cu) - 1):
        if cu[s + 1] > cu[s]:
            pooled[s] = out[cu[s]:cu[s + 1]].mean(axis=0)
    return pooled


def cls_pool(out, cu_seqlens) -> np.ndarray:
    """The first row of each sequence (CLS pooling, index 0: [CAN] §"Pooling and
    normalization"). An empty sequence pools to zero."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.asarray(out, dtype=np.float64)
    pooled = np.zeros((len(cu) - 1, out.shape[1]), dtype=np.float64)
    for s in range(len(cu) - 1):
        if cu[s + 1] > cu[s]:
            pooled[s] = out[cu[s]]
    return pooled


def l2_normalize(v, l2_eps: float = 1e-12) -> np.ndarray:
    """Each row divided by max(its L2 norm, eps) ([SBD] §"Implementing it": normalize)."""
    v = np.asarray(v, dtype=np.float64)
    n = np.sqrt((v * v).sum(axis=-1, keepdims=True))
    return v / np.maximum(n, l2_eps)


def classifier_logits(pooled, W_dense, norm_w, W_cls, b_cls, eps: float) -> np.ndarray:
    """Scores per label: the prediction head on the pooled vector, then a Linear with bias,
    one output per label ([KGP] §"How Do We Put a Classifier on Top?")."""
    h = prediction_head(pooled, W_dense, norm_w, eps)
    return h @ np.asarray(W_cls, dtype=np.float64).T + np.asarray(b_cls, dtype=np.float64)


def class_probabilities(logits) -> np.ndarray:
    """Softmax over the labels ([KGP] §"How Do We Put a Classifier on Top?")."""
    z = np.asarray(logits, dtype=np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def cross_entropy(logits, label: int) -> float:
    """Minus the log of the probability of the true label ([KGP] §"How Do We Put a Classifier
    on Top?": the loss is minus the log of that probability)."""
    return float(-np.log(class_probabilities(logits)[label]))
