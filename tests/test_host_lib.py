"""CPU-only checks of the C-ABI library: it loads, exports every function include/mbert.h
declares, and its host-side validation returns the documented error codes before anything is
enqueued (no GPU is touched)."""
import ctypes

import pytest

from transformer_encoder_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_every_declared_function_is_exported(lib):
    names = B.header_functions()
    assert len(names) >= 38
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding wraps every one of them under the same name
    assert not [n for n in names if n not in B._SIGNATURES]


def test_library_is_built_in_tree(lib):
    assert B.LIB_PATH.parent.name == "transformer_encoder_amd"
    assert B.LIB_PATH.exists()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", tmp_path / "libmbert.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        B.lib()


def test_default_config_is_modernbert_base():
    c = B.mbert_default_config()
    assert (c.n_layers, c.hidden, c.n_heads, c.head_dim, c.intermediate, c.vocab) == \
        (22, 768, 12, 64, 1152, 50368)
    assert (c.global_every, c.half_window, c.max_positions) == (3, 64, 8192)
    assert (c.theta_global, c.theta_local) == (160000.0, 10000.0)
    assert abs(c.norm_eps - 1e-5) < 1e-12
    assert B.mbert_check_config(c) == B.MBERT_OK
    assert B.mbert_tile_tokens() == 128


@pytest.mark.parametrize("field,value,code", [("hidden", 1024, B.MBERT_EUNSUPPORTED),
                                              ("n_heads", 16, B.MBERT_EUNSUPPORTED),
                                              ("intermediate", 3072, B.MBERT_EUNSUPPORTED),
                                              ("n_layers", 0, B.MBERT_EINVAL),
                                              ("max_positions", 0, B.MBERT_ERANGE),
                                              ("half_window", -1, B.MBERT_EINVAL),
                                              ("theta_local", 0.0, B.MBERT_EINVAL)])
def test_config_validation(field, value, code):
    c = B.mbert_default_config()
    setattr(c, field, value)
    assert B.mbert_check_config(c) == code
    assert B.mbert_workspace_bytes(c, B.MBERT_BF16, 100, 1) == 0


def test_strerror_and_sizes():
    assert B.strerror(B.MBERT_OK) == "ok"
    assert B.strerror(B.MBERT_ENOSPC) == "workspace too small"
    assert B.strerror(99) == "unknown error"
    assert [B.mbert_dtype_size(d) for d in (0, 1, 2, 7)] == [4, 2, 2, 0]


def test_head_workspace_bytes():
    for dt, ds in ((B.MBERT_F32, 4), (B.MBERT_BF16, 2), (B.MBERT_F16, 2)):
        for R in (0, 1, 7, 2445):
            n = B.mbert_head_workspace_bytes(dt, R)
            assert n >= R * 768 * (2 * ds + 4) and n % 256 == 0
    assert B.mbert_head_workspace_bytes(9, 4) == 0


def test_meta_and_workspace_layout():
    c = B.mbert_default_config()
    for T, S in ((0, 0), (1, 1), (300, 1), (2445, 8), (262144, 32)):
        tiles_max = -(-T // 128) + S
        off = 8 + T + S + 1
        off = (off + 3) & ~3
        assert B.mbert_meta_ints(T, S) == off + 5 * tiles_max  # tiles, then their order
        assert B.mbert_pool_partial_floats(T, S) == tiles_max * 4 * 768  # 4 partials per tile
        for dt, ds in ((B.MBERT_F32, 4), (B.MBERT_BF16, 2), (B.MBERT_F16, 2)):
            L = B.mbert_workspace_layout(c, dt, T, S)
            offs = [L.resid, L.h, L.qkv, L.meta, L.partials, L.ids, L.indices, L.rowmap, L.cu]
            sizes = [T * 768 * 4, T * 768 * ds, T * 2304 * ds, 4 * B.mbert_meta_ints(T, S),
                     4 * tiles_max * 4 * 768, 4 * T, 4 * T, 4 * T, 4 * (S + 1)]
            assert all(o % 256 == 0 for o in offs)
            for o, s, nxt in zip(offs, sizes, offs[1:] + [L.total_bytes]):
                assert o + s <= nxt
            assert B.mbert_workspace_bytes(c, dt, T, S) == L.total_bytes


def _fake_weights(n_layers=2, layer0_norm=False, dtype=B.MBERT_BF16):
    """A weights struct whose device pointers are never dereferenced: every call below fails
    validation before it launches anything."""
    c = B.mbert_default_config()
    c.n_layers = n_layers
    layers = (B.mbert_layer_weights * n_layers)()
    for i in range(n_layers):
        L = layers[i]
        L.attn_norm = 0x1000 if (i > 0 or layer0_norm) else None
        L.Wqkv = L.attn_Wo = L.mlp_norm = L.Wi = L.mlp_Wo = 0x1000
    w = B.mbert_weights()
    w.cfg = c
    w.dtype = dtype
    w.tok_emb = w.emb_norm = w.final_norm = w.rope = 0x1000
    w.layers = ctypes.cast(layers, ctypes.POINTER(B.mbert_layer_weights))
    w._layers = layers
    return w


def test_encode_validation_paths(lib):
    w = _fake_weights()
    fake = 0x2000
    need = B.mbert_workspace_bytes(w.cfg, B.MBERT_BF16, 300, 1)
    enc = lambda ww, total=300, nseq=1, ws_bytes=need, out=fake: lib.mbert_encode(
        ctypes.byref(ww), fake, fake, nseq, total, fake, ws_bytes, out, None, None)
    assert lib.mbert_encode(None, fake, fake, 1, 300, fake, need, fake, None, None) == B.MBERT_EINVAL
    assert enc(w, ws_bytes=need - 1) == B.MBERT_ENOSPC
    assert enc(w, total=-1) == B.MBERT_EINVAL
    assert enc(w, out=None) == B.MBERT_EINVAL
    assert enc(_fake_weights(layer0_norm=True)) == B.MBERT_EINVAL
    assert enc(_fake_weights(dtype=9)) == B.MBERT_EUNSUPPORTED
    bad = _fake_weights()
    bad.cfg.hidden = 512
    assert enc(bad) == B.MBERT_EUNSUPPORTED
    assert enc(w, total=10 ** 9) == B.MBERT_ERANGE
    # the padded entry point sizes its workspace for B * Tpad tokens and B sequences
    need_p = B.mbert_workspace_bytes(w.cfg, B.MBERT_BF16, 8 * 512, 8)
    assert lib.mbert_encode_padded(ctypes.byref(w), fake, fake, 8, 512, fake, need_p - 1, fake,
                                   None, None) == B.MBERT_ENOSPC
    assert lib.mbert_layer(ctypes.byref(w), 2, 300, 1, fake, need, None) == B.MBERT_EINVAL
    # grouped padded forward: workspace per group, distinct extra streams
    one = B.mbert_workspace_bytes(w.cfg, B.MBERT_BF16, 4 * 512, 4)
    assert B.mbert_workspace_bytes_grouped(w.cfg, B.MBERT_BF16, 8, 512, 2) == 2 * one
    assert B.mbert_workspace_bytes_grouped(w.cfg, B.MBERT_BF16, 8, 512, 1) == need_p
    assert B.mbert_workspace_bytes_grouped(w.cfg, B.MBERT_BF16, 8, 512, 0) == 0
    grp = lib.mbert_encode_padded_grouped
    s_main = ctypes.c_void_p(0x9000)
    same = (ctypes.c_void_p * 1)(0x9000)
    other = (ctypes.c_void_p * 1)(0xA000)
    assert grp(ctypes.byref(w), fake, fake, 8, 512, 2, fake, 2 * one, fake, None, same,
               s_main) == B.MBERT_EINVAL
    assert grp(ctypes.byref(w), fake, fake, 8, 512, 2, fake, 2 * one - 1, fake, None, other,
               s_main) == B.MBERT_ENOSPC
    assert grp(ctypes.byref(w), fake, fake, 8, 512, 0, fake, 2 * one, fake, None, other,
               s_main) == B.MBERT_EINVAL


def test_step_validation_paths(lib):
    fake = 0x3000
    assert lib.mbert_linear_residual(1, fake, 1000, 10, None, fake, fake, None) == B.MBERT_EUNSUPPORTED
    assert lib.mbert_layernorm(5, fake, 10, None, fake, 1e-5, fake, None) == B.MBERT_EUNSUPPORTED
    assert lib.mbert_attention(1, fake, 10, None, 1, 1, 64, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_qkv_rope(1, fake, 10, None, fake, fake, 8192, 0, 1, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_qkv_rope(1, fake, 10, fake, fake, fake, 8192, 2, 1, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_pack_meta(None, 1, 10, 8192, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_unpad(fake, fake, -1, 5, 8192, fake, fake, fake, fake, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_final_ln_pool(fake, 10, fake, 1, 1, fake, 1e-5, fake, fake, None, None) == B.MBERT_EINVAL
    assert lib.mbert_graph_launch(None, None) == B.MBERT_EINVAL
    # the MFMA calibration kernel: sizes and dtype checked before any launch
    assert lib.mbert_mfma_probe(1, 0, 10, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_mfma_probe(1, 1 << 17, 10, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_mfma_probe(1, 256, 0, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_mfma_probe(1, 256, 10, None, None) == B.MBERT_EINVAL
    assert lib.mbert_mfma_probe(7, 256, 10, fake, None) == B.MBERT_EUNSUPPORTED
    # pooling and heads
    assert lib.mbert_pool(fake, 10, fake, 1, 4, fake, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_pool(fake, 10, None, 1, 0, fake, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_pool(fake, 10, fake, 1, B.POOL_MEAN, fake, None, None) == B.MBERT_EINVAL
    mlm = lib.mbert_mlm_head
    assert mlm(1, fake, 10, None, 4, fake, fake, 1e-5, fake, fake, 50000, fake, 1 << 30, fake,
               None) == B.MBERT_EUNSUPPORTED  # vocabulary not a multiple of 64
    assert mlm(1, fake, 10, None, 11, fake, fake, 1e-5, fake, fake, 64, fake, 1 << 30, fake,
               None) == B.MBERT_EINVAL  # more rows than positions without a row list
    need = B.mbert_head_workspace_bytes(B.MBERT_BF16, 4)
    assert mlm(1, fake, 10, None, 4, fake, fake, 1e-5, fake, fake, 64, fake, need - 1, fake,
               None) == B.MBERT_ENOSPC
    assert mlm(7, fake, 10, None, 4, fake, fake, 1e-5, fake, fake, 64, fake, need, fake,
               None) == B.MBERT_EUNSUPPORTED
    clf = lib.mbert_classifier_head
    assert clf(1, fake, 4, fake, fake, 1e-5, fake, fake, 0, fake, need, fake, None) == B.MBERT_EINVAL
    assert clf(1, fake, 4, fake, fake, 1e-5, fake, fake, 4, fake, need - 1, fake, None) == B.MBERT_ENOSPC
    assert clf(1, fake, 0, None, None, 1e-5, None, None, 4, None, 0, None, None) == B.MBERT_OK
    assert lib.mbert_timer_create(0, ctypes.byref(ctypes.c_void_p())) == B.MBERT_EINVAL
    # the folded path's step entry points
    lrs = lib.mbert_linear_residual_stats
    assert lrs(1, fake, 1000, 10, None, fake, fake, fake, fake, None) == B.MBERT_EUNSUPPORTED
    assert lrs(1, fake, 768, 10, None, fake, fake, None, fake, None) == B.MBERT_EINVAL  # no xs
    assert lrs(1, fake, 768, 10, None, fake, fake, fake, None, None) == B.MBERT_EINVAL  # no stats
    assert lib.mbert_fold_weight(1, fake, None, 4, fake, fake, None) == B.MBERT_EINVAL
    assert lib.mbert_fold_weight(1, None, None, 0, None, None, None) == B.MBERT_OK
    fg = lib.mbert_folded_gemm
    assert fg(1, 2, fake, fake, 10, fake, fake, fake, 1e-5, fake, 8192, 0, fake, None) == B.MBERT_EINVAL
    assert fg(1, 0, fake, fake, 10, None, fake, fake, 1e-5, fake, 8192, 0, fake, None) == B.MBERT_EINVAL
    assert fg(1, 1, fake, None, 10, fake, fake, fake, 1e-5, None, 0, 0, fake, None) == B.MBERT_EINVAL
    assert fg(9, 1, fake, fake, 10, fake, fake, fake, 1e-5, None, 0, 0, fake, None) == B.MBERT_EUNSUPPORTED


def test_fold_norms_sizes_and_validation(lib):
    """Folded-norm weights: one [2304,768] weight and [2304] column sums per norm, 256-byte
    aligned, per layer, for every dtype; every failure below returns before any launch."""
    w = _fake_weights(n_layers=3)
    al = lambda n: (n + 255) // 256 * 256
    per = lambda ds: 2 * (al(2304 * 768 * ds) + al(2304 * 4))
    assert B.mbert_folded_bytes(w.cfg, B.MBERT_BF16) == 3 * per(2)
    assert B.mbert_folded_bytes(w.cfg, B.MBERT_F32) == 3 * per(4)
    assert B.mbert_folded_bytes(w.cfg, B.MBERT_F16) == 3 * per(2)
    need = B.mbert_folded_bytes(w.cfg, B.MBERT_BF16)
    fake = 0x4000
    assert lib.mbert_fold_norms(ctypes.byref(w), None, need, None) == B.MBERT_EINVAL
    assert lib.mbert_fold_norms(ctypes.byref(w), fake, need - 1, None) == B.MBERT_ENOSPC
    w16 = _fake_weights(dtype=B.MBERT_F16)
    need16 = B.mbert_folded_bytes(w16.cfg, B.MBERT_F16)
    assert need16 == 2 * per(2)
    assert lib.mbert_fold_norms(ctypes.byref(w16), fake, need16 - 1, None) == B.MBERT_ENOSPC
    assert lib.mbert_fold_norms(None, fake, need, None) == B.MBERT_EINVAL
    # the forward's workspace holds the rounded residual and its chunk statistics
    L = B.mbert_workspace_layout(w.cfg, B.MBERT_BF16, 1000, 4)
    assert L.rstats - L.xs >= 1000 * 768 * 2 and L.total_bytes - L.rstats >= 1000 * 12 * 8
