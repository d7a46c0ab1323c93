"""Thin Python binding of libmbert.so (include/mbert.h): argument marshalling only.

Every function here has the name of the C entry point it calls and forwards plain pointers
(``tensor.data_ptr()``), sizes and the HIP stream. PyTorch supplies device memory and streams;
every step of the forward runs in the library's HIP kernels. If the library is missing the
import of this module's functions raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import re
from ctypes import POINTER, Structure, c_double, c_float, c_int, c_int32, c_size_t, c_void_p
from pathlib import Path

LIB_PATH = Path(__file__).resolve().with_name("libmbert.so")
HEADER = Path(__file__).resolve().parent.parent / "include" / "mbert.h"

MBERT_OK, MBERT_EINVAL, MBERT_EUNSUPPORTED, MBERT_ERANGE, MBERT_ENOSPC, MBERT_EHIP = range(6)
MBERT_F32, MBERT_BF16, MBERT_F16 = 0, 1, 2
DTYPES = {"f32": MBERT_F32, "bf16": MBERT_BF16, "f16": MBERT_F16}
STATUS_BAD_CU, STATUS_TOO_LONG, STATUS_BAD_MASK, STATUS_BAD_ID = 1, 2, 4, 8
POOL_MEAN, POOL_CLS, POOL_L2 = 0, 1, 2
(K_EMBED_LN, K_LAYERNORM, K_QKV_ROPE, K_ATTN_GLOBAL, K_ATTN_LOCAL, K_WO_RESID, K_WI_GEGLU,
 K_WO2_RESID, K_FINAL_POOL, K_META) = range(10)
KERNEL_KINDS = {"embed_ln": 0, "layernorm": 1, "qkv_rope": 2, "attn_global": 3, "attn_local": 4,
                "wo_resid": 5, "wi_geglu": 6, "wo2_resid": 7, "final_pool": 8, "meta": 9}


class MbertError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


class mbert_config(Structure):
    _fields_ = [("n_layers", c_int), ("hidden", c_int), ("n_heads", c_int), ("head_dim", c_int),
                ("intermediate", c_int), ("vocab", c_int), ("global_every", c_int),
                ("half_window", c_int), ("max_positions", c_int), ("theta_global", c_double),
                ("theta_local", c_double), ("norm_eps", c_float)]


class mbert_layer_weights(Structure):
    _fields_ = [("attn_norm", c_void_p), ("Wqkv", c_void_p), ("attn_Wo", c_void_p),
                ("mlp_norm", c_void_p), ("Wi", c_void_p), ("mlp_Wo", c_void_p)]


class mbert_weights(Structure):
    _fields_ = [("cfg", mbert_config), ("dtype", c_int), ("tok_emb", c_void_p),
                ("emb_norm", c_void_p), ("final_norm", c_void_p),
                ("layers", POINTER(mbert_layer_weights)), ("rope", c_void_p),
                ("folded", c_void_p)]


class mbert_ws_layout(Structure):
    _fields_ = [(n, c_size_t) for n in ("resid", "h", "qkv", "meta", "partials", "ids", "indices",
                                        "rowmap", "cu", "xs", "rstats",
                                        "total_bytes")]


P, I, SZ = c_void_p, c_int, c_size_t
_SIGNATURES = {
    "mbert_version": ([], I),
    "mbert_strerror": ([I], ctypes.c_char_p),
    "mbert_default_config": ([POINTER(mbert_config)], I),
    "mbert_check_config": ([POINTER(mbert_config)], I),
    "mbert_tile_tokens": ([], I),
    "mbert_meta_ints": ([I, I], SZ),
    "mbert_dtype_size": ([I], SZ),
    "mbert_rope_table_floats": ([POINTER(mbert_config)], SZ),
    "mbert_build_rope_tables": ([POINTER(mbert_config), P, P], I),
    "mbert_pack_meta": ([P, I, I, I, P, P], I),
    "mbert_unpad": ([P, P, I, I, I, P, P, P, P, P, P], I),
    "mbert_attn_key_ranges": ([P, I, I, I, I, P, P, P], I),
    "mbert_read_status": ([P, POINTER(c_int32), P], I),
    "mbert_embed_ln": ([I, P, I, P, P, I, P, c_float, P, P, P], I),
    "mbert_layernorm": ([I, P, I, P, P, c_float, P, P], I),
    "mbert_mfma_probe": ([I, I, I, P, P], I),
    "mbert_qkv_rope": ([I, P, I, P, P, P, I, I, I, P, P], I),
    "mbert_rope": ([I, P, I, P, P, I, I, P], I),
    "mbert_attention": ([I, P, I, P, I, I, I, P, P], I),
    "mbert_linear_residual": ([I, P, I, I, P, P, P, P], I),
    "mbert_mlp_in_geglu": ([I, P, I, P, P, P, P], I),
    "mbert_linear_residual_stats": ([I, P, I, I, P, P, P, P, P, P], I),
    "mbert_fold_weight": ([I, P, P, I, P, P, P], I),
    "mbert_folded_gemm": ([I, I, P, P, I, P, P, P, c_float, P, I, I, P, P], I),
    "mbert_pool_partial_floats": ([I, I], SZ),
    "mbert_final_ln_pool": ([P, I, P, I, I, P, c_float, P, P, P, P], I),
    "mbert_repad": ([P, P, I, I, P, P], I),
    "mbert_pool": ([P, I, P, I, I, P, P, P], I),
    "mbert_attention_probs": ([I, P, I, I, I, I, I, I, P, P], I),
    "mbert_encode_padded_keymask": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P], I),
    "mbert_head_workspace_bytes": ([I, I], SZ),
    "mbert_mlm_head": ([I, P, I, P, I, P, P, c_float, P, P, I, P, SZ, P, P], I),
    "mbert_classifier_head": ([I, P, I, P, P, c_float, P, P, I, P, SZ, P, P], I),
    "mbert_workspace_bytes": ([POINTER(mbert_config), I, I, I], SZ),
    "mbert_folded_bytes": ([POINTER(mbert_config), I], SZ),
    "mbert_fold_norms": ([POINTER(mbert_weights), P, SZ, P], I),
    "mbert_workspace_layout": ([POINTER(mbert_config), I, I, I, POINTER(mbert_ws_layout)], I),
    "mbert_layer": ([POINTER(mbert_weights), I, I, I, P, SZ, P], I),
    "mbert_encode": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P], I),
    "mbert_noalloc_max_bytes": ([], SZ),
    "mbert_encode_noalloc": ([POINTER(mbert_weights), P, P, I, I, P, P, P], I),
    "mbert_encode_padded": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P], I),
    "mbert_graph_capture": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P, POINTER(P)], I),
    "mbert_graph_capture_padded": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P,
                                    POINTER(P)], I),
    "mbert_workspace_bytes_grouped": ([POINTER(mbert_config), I, I, I, I], SZ),
    "mbert_encode_padded_grouped": ([POINTER(mbert_weights), P, P, I, I, I, P, SZ, P, P, POINTER(P),
                                     P], I),
    "mbert_graph_capture_padded_grouped": ([POINTER(mbert_weights), P, P, I, I, I, P, SZ, P, P,
                                            POINTER(P), P, POINTER(P)], I),
    "mbert_graph_launch": ([P, P], I),
    "mbert_graph_destroy": ([P], I),
    "mbert_timer_create": ([I, POINTER(P)], I),
    "mbert_timer_reset": ([P], I),
    "mbert_timer_read": ([P, POINTER(c_int), POINTER(c_double)], I),
    "mbert_timer_destroy": ([P], I),
    "mbert_encode_timed": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P, I, P], I),
    "mbert_encode_padded_timed": ([POINTER(mbert_weights), P, P, I, I, P, SZ, P, P, P, I, P], I),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if libmbert.so has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with transformer_encoder_amd.build "
                               "(or __graft_entry__.build()); there is no fallback path")
        # PyTorch's HIP runtime first: the library then binds to the runtime that owns the
        # caller's device memory and streams. Loaded the other way round, the process holds
        # two HIP runtimes and the second to initialise finds no device (hipErrorNoDevice).
        import torch  # noqa: F401
        h = ctypes.CDLL(str(LIB_PATH))
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def header_functions() -> list[str]:
    """Names of every function declared in include/mbert.h."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(mbert_[a-z0-9_]+)\s*\(", text)))


def strerror(code: int) -> str:
    return lib().mbert_strerror(code).decode()


def _check(rc: int, where: str) -> None:
    if rc != MBERT_OK:
        raise MbertError(rc, where)


def ptr(t) -> int | None:
    """Device/host address of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _call(name, *args, check=True):
    rc = getattr(lib(), name)(*args)
    if check:
        _check(rc, name)
    return rc


# ---------------------------------------------------------------------------- info
def mbert_version() -> int:
    return lib().mbert_version()


def mbert_default_config() -> mbert_config:
    c = mbert_config()
    _call("mbert_default_config", ctypes.byref(c))
    return c


def mbert_check_config(cfg: mbert_config) -> int:
    return lib().mbert_check_config(ctypes.byref(cfg))


def mbert_tile_tokens() -> int:
    return lib().mbert_tile_tokens()


def mbert_meta_ints(total_max: int, n_seqs: int) -> int:
    return lib().mbert_meta_ints(total_max, n_seqs)


def mbert_dtype_size(dtype: int) -> int:
    return lib().mbert_dtype_size(dtype)


def mbert_rope_table_floats(cfg: mbert_config) -> int:
    return lib().mbert_rope_table_floats(ctypes.byref(cfg))


def mbert_build_rope_tables(cfg, table, stream=None):
    _call("mbert_build_rope_tables", ctypes.byref(cfg), ptr(table), stream_handle(stream))


# ---------------------------------------------------------------------------- meta
def mbert_pack_meta(cu_seqlens, n_seqs, total, max_positions, meta, stream=None, check=True):
    return _call("mbert_pack_meta", ptr(cu_seqlens), n_seqs, total, max_positions, ptr(meta),
                 stream_handle(stream), check=check)


def mbert_unpad(ids_pad, mask, B, Tpad, max_positions, ids, indices, rowmap, cu_seqlens, meta,
                stream=None):
    _call("mbert_unpad", ptr(ids_pad), ptr(mask), B, Tpad, max_positions, ptr(ids), ptr(indices),
          ptr(rowmap), ptr(cu_seqlens), ptr(meta), stream_handle(stream))


def mbert_attn_key_ranges(meta, total_max, n_seqs, is_global, half_window, lo, hi, stream=None):
    _call("mbert_attn_key_ranges", ptr(meta), total_max, n_seqs, int(is_global), half_window,
          ptr(lo), ptr(hi), stream_handle(stream))


def mbert_read_status(meta, stream=None) -> list[int]:
    out = (c_int32 * 4)()
    _call("mbert_read_status", ptr(meta), out, stream_handle(stream))
    return list(out)


# ---------------------------------------------------------------------------- per step
def mbert_embed_ln(dtype, ids, total, meta, tok_emb, vocab, norm_w, eps, resid, h, stream=None):
    _call("mbert_embed_ln", dtype, ptr(ids), total, ptr(meta), ptr(tok_emb), vocab, ptr(norm_w),
          eps, ptr(resid), ptr(h), stream_handle(stream))


def mbert_mfma_probe(dtype, blocks, iters, out, stream=None):
    _call("mbert_mfma_probe", dtype, blocks, iters, ptr(out), stream_handle(stream))


def mbert_layernorm(dtype, x, total, meta, w, eps, y, stream=None):
    _call("mbert_layernorm", dtype, ptr(x), total, ptr(meta), ptr(w), eps, ptr(y),
          stream_handle(stream))


def mbert_qkv_rope(dtype, h, total, meta, Wqkv, rope, max_positions, table, apply_rope, qkv,
                   stream=None):
    _call("mbert_qkv_rope", dtype, ptr(h), total, ptr(meta), ptr(Wqkv), ptr(rope), max_positions,
          table, int(apply_rope), ptr(qkv), stream_handle(stream))


def mbert_rope(dtype, qkv, total, meta, rope, max_positions, table, stream=None):
    _call("mbert_rope", dtype, ptr(qkv), total, ptr(meta), ptr(rope), max_positions, table,
          stream_handle(stream))


def mbert_attention(dtype, qkv, total, meta, n_seqs, is_global, half_window, o, stream=None):
    _call("mbert_attention", dtype, ptr(qkv), total, ptr(meta), n_seqs, int(is_global),
          half_window, ptr(o), stream_handle(stream))


def mbert_linear_residual(dtype, a, K, total, meta, W, resid, stream=None):
    _call("mbert_linear_residual", dtype, ptr(a), K, total, ptr(meta), ptr(W), ptr(resid),
          stream_handle(stream))


def mbert_mlp_in_geglu(dtype, h, total, meta, Wi, m, stream=None):
    _call("mbert_mlp_in_geglu", dtype, ptr(h), total, ptr(meta), ptr(Wi), ptr(m),
          stream_handle(stream))


FOLD_QKV_ROPE, FOLD_GEGLU = 0, 1


def mbert_linear_residual_stats(dtype, a, K, total, meta, W, resid, xs, stats, stream=None):
    _call("mbert_linear_residual_stats", dtype, ptr(a), K, total, ptr(meta), ptr(W), ptr(resid),
          ptr(xs), ptr(stats), stream_handle(stream))


def mbert_fold_weight(dtype, W, w, rows, Wf, c, stream=None):
    _call("mbert_fold_weight", dtype, ptr(W), ptr(w), rows, ptr(Wf), ptr(c), stream_handle(stream))


def mbert_folded_gemm(dtype, kind, xs, stats, total, meta, Wf, c, eps, rope, max_positions, table,
                      out, stream=None):
    _call("mbert_folded_gemm", dtype, kind, ptr(xs), ptr(stats), total, ptr(meta), ptr(Wf), ptr(c),
          eps, ptr(rope), max_positions, table, ptr(out), stream_handle(stream))


def mbert_pool_partial_floats(total_max, n_seqs) -> int:
    return lib().mbert_pool_partial_floats(total_max, n_seqs)


def mbert_final_ln_pool(resid, total, meta, n_seqs, dtype, w, eps, out, pooled, partials,
                        stream=None):
    _call("mbert_final_ln_pool", ptr(resid), total, ptr(meta), n_seqs, dtype, ptr(w), eps,
          ptr(out), ptr(pooled), ptr(partials), stream_handle(stream))


def mbert_attention_probs(dtype, qkv, total, row0, n_q, n_k, is_global, half_window, probs,
                          stream=None):
    _call("mbert_attention_probs", dtype, ptr(qkv), total, row0, n_q, n_k, int(is_global),
          half_window, ptr(probs), stream_handle(stream))


def mbert_pool(out, total, meta, n_seqs, mode, pooled, partials=None, stream=None):
    _call("mbert_pool", ptr(out), total, ptr(meta), n_seqs, mode, ptr(pooled), ptr(partials),
          stream_handle(stream))


def mbert_head_workspace_bytes(dtype, rows) -> int:
    return lib().mbert_head_workspace_bytes(dtype, rows)


def mbert_mlm_head(dtype, x, total, rows, n_rows, W_dense, norm_w, eps, decoder_w, decoder_b,
                   vocab, ws, ws_bytes, logits, stream=None):
    _call("mbert_mlm_head", dtype, ptr(x), total, ptr(rows), n_rows, ptr(W_dense), ptr(norm_w),
          eps, ptr(decoder_w), ptr(decoder_b), vocab, ptr(ws), ws_bytes, ptr(logits),
          stream_handle(stream))


def mbert_classifier_head(dtype, pooled, n_seqs, W_dense, norm_w, eps, W_cls, b_cls, n_labels,
                          ws, ws_bytes, logits, stream=None):
    _call("mbert_classifier_head", dtype, ptr(pooled), n_seqs, ptr(W_dense), ptr(norm_w), eps,
          ptr(W_cls), ptr(b_cls), n_labels, ptr(ws), ws_bytes, ptr(logits), stream_handle(stream))


def mbert_repad(out, rowmap, B, Tpad, out_pad, stream=None):
    _call("mbert_repad", ptr(out), ptr(rowmap), B, Tpad, ptr(out_pad), stream_handle(stream))


# ---------------------------------------------------------------------------- whole forward
def mbert_workspace_bytes(cfg, dtype, total_max, n_seqs) -> int:
    return lib().mbert_workspace_bytes(ctypes.byref(cfg), dtype, total_max, n_seqs)


def mbert_workspace_layout(cfg, dtype, total_max, n_seqs) -> mbert_ws_layout:
    L = mbert_ws_layout()
    _call("mbert_workspace_layout", ctypes.byref(cfg), dtype, total_max, n_seqs, ctypes.byref(L))
    return L


def mbert_folded_bytes(cfg, dtype) -> int:
    return lib().mbert_folded_bytes(ctypes.byref(cfg), dtype)


def mbert_fold_norms(weights, folded, nbytes, stream=None):
    _call("mbert_fold_norms", ctypes.byref(weights), ptr(folded), nbytes, stream_handle(stream))


def mbert_layer(weights, layer, total, n_seqs, ws, ws_bytes, stream=None):
    _call("mbert_layer", ctypes.byref(weights), layer, total, n_seqs, ptr(ws), ws_bytes,
          stream_handle(stream))


def mbert_noalloc_max_bytes() -> int:
    return lib().mbert_noalloc_max_bytes()


def mbert_encode_noalloc(weights, ids, cu_seqlens, n_seqs, total, out, pooled, stream=None,
                         check=True):
    return _call("mbert_encode_noalloc", ctypes.byref(weights), ptr(ids), ptr(cu_seqlens), n_seqs,
                 total, ptr(out), ptr(pooled), stream_handle(stream), check=check)


def mbert_encode(weights, ids, cu_seqlens, n_seqs, total, ws, ws_bytes, out, pooled,
                 stream=None, check=True):
    return _call("mbert_encode", ctypes.byref(weights), ptr(ids), ptr(cu_seqlens), n_seqs, total,
                 ptr(ws), ws_bytes, ptr(out), ptr(pooled), stream_handle(stream), check=check)


def mbert_encode_padded(weights, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                        stream=None, check=True):
    return _call("mbert_encode_padded", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B, Tpad,
                 ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled), stream_handle(stream), check=check)


def mbert_encode_padded_keymask(weights, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                                stream=None, check=True):
    return _call("mbert_encode_padded_keymask", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B,
                 Tpad, ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled), stream_handle(stream),
                 check=check)


def mbert_graph_capture(weights, ids, cu_seqlens, n_seqs, total, ws, ws_bytes, out, pooled,
                        stream) -> int:
    g = c_void_p()
    _call("mbert_graph_capture", ctypes.byref(weights), ptr(ids), ptr(cu_seqlens), n_seqs, total,
          ptr(ws), ws_bytes, ptr(out), ptr(pooled), stream_handle(stream), ctypes.byref(g))
    return g.value


def mbert_graph_capture_padded(weights, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                               stream) -> int:
    g = c_void_p()
    _call("mbert_graph_capture_padded", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B, Tpad,
          ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled), stream_handle(stream), ctypes.byref(g))
    return g.value


def _stream_array(streams):
    return (c_void_p * max(1, len(streams)))(*[stream_handle(x) for x in streams])


def mbert_workspace_bytes_grouped(cfg, dtype, B, Tpad, n_groups) -> int:
    return lib().mbert_workspace_bytes_grouped(ctypes.byref(cfg), dtype, B, Tpad, n_groups)


def mbert_encode_padded_grouped(weights, ids_pad, mask, B, Tpad, n_groups, ws, ws_bytes, out_pad,
                                pooled, streams, stream=None, check=True):
    """streams: the n_groups - 1 extra streams (torch.cuda.Stream objects)."""
    return _call("mbert_encode_padded_grouped", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B,
                 Tpad, n_groups, ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled),
                 _stream_array(streams), stream_handle(stream), check=check)


def mbert_graph_capture_padded_grouped(weights, ids_pad, mask, B, Tpad, n_groups, ws, ws_bytes,
                                       out_pad, pooled, streams, stream) -> int:
    g = c_void_p()
    _call("mbert_graph_capture_padded_grouped", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B,
          Tpad, n_groups, ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled), _stream_array(streams),
          stream_handle(stream), ctypes.byref(g))
    return g.value


def mbert_graph_launch(graph: int, stream=None):
    _call("mbert_graph_launch", graph, stream_handle(stream))


def mbert_graph_destroy(graph: int):
    _call("mbert_graph_destroy", graph)


def mbert_timer_create(max_launches: int) -> int:
    t = c_void_p()
    _call("mbert_timer_create", max_launches, ctypes.byref(t))
    return t.value


def mbert_timer_reset(timer: int):
    _call("mbert_timer_reset", timer)


def mbert_timer_read(timer: int) -> tuple[int, float]:
    n, ms = c_int(), c_double()
    _call("mbert_timer_read", timer, ctypes.byref(n), ctypes.byref(ms))
    return n.value, ms.value


def mbert_timer_destroy(timer: int):
    _call("mbert_timer_destroy", timer)


def mbert_encode_timed(weights, ids, cu_seqlens, n_seqs, total, ws, ws_bytes, out, pooled,
                       kind, timer, stream=None):
    _call("mbert_encode_timed", ctypes.byref(weights), ptr(ids), ptr(cu_seqlens), n_seqs, total,
          ptr(ws), ws_bytes, ptr(out), ptr(pooled), stream_handle(stream), kind, timer)


def mbert_encode_padded_timed(weights, ids_pad, mask, B, Tpad, ws, ws_bytes, out_pad, pooled,
                              kind, timer, stream=None):
    _call("mbert_encode_padded_timed", ctypes.byref(weights), ptr(ids_pad), ptr(mask), B, Tpad,
          ptr(ws), ws_bytes, ptr(out_pad), ptr(pooled), stream_handle(stream), kind, timer)
