"""Pure-Python brute-force encoder forward, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same import rule as mbert_oracle). A second, independent
statement of the forward described by kgptalkie, "ModernBERT-base Architecture Teardown"
(§"What Does LayerNorm Do?", §"How Does Self-Attention Work?", §"What Are Local and Global
Attention?", §"How Does RoPE Work With Two Bases?", §"What Does the GeGLU MLP Do?") and
candding, "ModernBERT" (§"The alternating attention", §"The two rope tables", §"The
feed-forward halves", §"The pre-norm layer and the final norm"): explicit loops over tokens,
heads, keys and features, with ``math`` functions only. It shares no code with
mbert_oracle.py, so a vectorisation slip there (a transposed operand, a wrong axis, a
wrong slice) shows up as a disagreement.
"""
from __future__ import annotations

import math


def _ln(row, w, eps):
    n = len(row)
    mu = sum(row) / n
    var = sum((r - mu) * (r - mu) for r in row) / n
    inv = 1.0 / math.sqrt(var + eps)
    return [(row[i] - mu) * inv * w[i] for i in range(n)]


def _matvec(W, v):
    """W given as a list of output rows (the [out, in] storage of a Linear weight)."""
    return [sum(Wr[j] * v[j] for j in range(len(v))) for Wr in W]


def _gelu(z):
    return 0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0)))


def _rotate(vec, p, theta):
    hd = len(vec)
    half = hd // 2
    out = [0.0] * hd
    for i in range(half):
        a = p * (theta ** (-(2.0 * i) / hd))
        c, s = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i + half] * c + vec[i] * s
    return out


def encode(ids, cu_seqlens, weights, *, n_layers, hidden, n_heads, head_dim, intermediate,
           global_every, half_window, theta_global, theta_local, eps):
    """Returns (out as list of rows, pooled as list of rows). ``weights`` uses the same keys
    as the workloads generator; arrays are converted to nested lists here."""
    tolist = lambda a: None if a is None else (a.tolist() if hasattr(a, "tolist") else a)
    E = weights["tok_emb"]
    emb_norm = tolist(weights["emb_norm"])
    final_norm = tolist(weights["final_norm"])
    cu = [int(c) for c in cu_seqlens]
    T = cu[-1]
    seq_of = []
    pos = []
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            seq_of.append(s)
            pos.append(t - cu[s])

    x = [_ln([float(v) for v in E[int(ids[t])]], emb_norm, eps) for t in range(T)]

    for layer in range(n_layers):
        lw = weights["layers"][layer]
        Wqkv, Wo, Wi, Wo2 = (tolist(lw[k]) for k in ("Wqkv", "attn_Wo", "Wi", "mlp_Wo"))
        mlp_norm = tolist(lw["mlp_norm"])
        glob = (layer % global_every == 0)
        theta = theta_global if glob else theta_local
        if layer == 0:
            h = [list(r) for r in x]
        else:
            attn_norm = tolist(lw["attn_norm"])
            h = [_ln(r, attn_norm, eps) for r in x]
        # projections: rows 0..D-1 query, D..2D-1 key, 2D..3D-1 value; head n = 64n..64n+63
        q = [[None] * n_heads for _ in range(T)]
        k = [[None] * n_heads for _ in range(T)]
        v = [[None] * n_heads for _ in range(T)]
        for t in range(T):
            y = _matvec(Wqkv, h[t])
            for n in range(n_heads):
                b = n * head_dim
                q[t][n] = _rotate(y[b:b + head_dim], pos[t], theta)
                k[t][n] = _rotate(y[hidden + b:hidden + b + head_dim], pos[t], theta)
                v[t][n] = y[2 * hidden + b:2 * hidden + b + head_dim]
        attn = []
        for t in range(T):
            row = []
            for n in range(n_heads):
                keys = [j for j in range(T) if seq_of[j] == seq_of[t]
                        and (glob or abs(pos[j] - pos[t]) <= half_window)]
                sc = [sum(q[t][n][d] * k[j][n][d] for d in range(head_dim)) / math.sqrt(head_dim)
                      for j in keys]
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                z = sum(ex)
                for d in range(head_dim):
                    row.append(sum(ex[i] * v[keys[i]][n][d] for i in range(len(keys))) / z)
            attn.append(row)
        x = [[x[t][i] + o for i, o in enumerate(_matvec(Wo, attn[t]))] for t in range(T)]
        new_x = []
        for t in range(T):
            u = _matvec(Wi, _ln(x[t], mlp_norm, eps))
            m = [_gelu(u[i]) * u[intermediate + i] for i in range(intermediate)]
            new_x.append([x[t][i] + o for i, o in enumerate(_matvec(Wo2, m))])
        x = new_x

    out = [_ln(r, final_norm, eps) for r in x]
    pooled = []
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L == 0:
            pooled.append([0.0] * hidden)
            continue
        mean = [sum(out[t][i] for t in range(cu[s], cu[s + 1])) / L for i in range(hidden)]
        nrm = math.sqrt(sum(m * m for m in mean))
        pooled.append([m / max(nrm, 1e-12) for m in mean])
    return out, pooled


def prediction_head(x, W_dense, norm_w, eps):
    """Dense (no bias), GELU, LayerNorm of one vector (kgptalkie, §"The Masked-LM Head")."""
    return _ln([_gelu(u) for u in _matvec(W_dense, x)], norm_w, eps)


def mlm_logits(x, W_dense, norm_w, tok_emb, decoder_bias, eps):
    """Scores of one vector against every vocabulary row (tied decoder, with bias)."""
    h = prediction_head(x, W_dense, norm_w, eps)
    return [sum(e[j] * h[j] for j in range(len(h))) + decoder_bias[v] for v, e in enumerate(tok_emb)]


def classifier_logits(pooled, W_dense, norm_w, W_cls, b_cls, eps):
    """Scores of one pooled vector per label (kgptalkie, §"How Do We Put a Classifier on Top?")."""
    h = prediction_head(pooled, W_dense, norm_w, eps)
    return [sum(Wc[j] * h[j] for j in range(len(h))) + b_cls[c] for c, Wc in enumerate(W_cls)]
