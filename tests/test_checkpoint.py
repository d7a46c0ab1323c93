"""Weights by the published tensor names (candding, 'ModernBERT', 'The tensors') and the named
configurations (safebydesign.ai, 'ModernBertModel 22L 768d', 'Implementing it'). CPU only:
synthetic safetensors files written here with tiny dimensions."""
import numpy as np
import pytest

from transformer_encoder_amd import checkpoint as C
from transformer_encoder_amd import binding as B


def _tensors(n_layers=22, V=20, D=8, I=12, seed=0, prefix="", head=False, dtype=np.float32):
    g = np.random.default_rng(seed)
    t = {}
    for name in C.tensor_names(n_layers):
        if name == "embeddings.tok_embeddings.weight":
            shape = (V, D)
        elif name.endswith("Wqkv.weight"):
            shape = (3 * D, D)
        elif name.endswith("attn.Wo.weight"):
            shape = (D, D)
        elif name.endswith("mlp.Wi.weight"):
            shape = (2 * I, D)
        elif name.endswith("mlp.Wo.weight"):
            shape = (D, I)
        else:
            shape = (D,)
        t[prefix + name] = g.standard_normal(shape).astype(dtype)
    if head:
        t["head.dense.weight"] = g.standard_normal((D, D)).astype(dtype)
        t["head.norm.weight"] = g.standard_normal(D).astype(dtype)
        t["decoder.bias"] = g.standard_normal(V).astype(dtype)
    return t


def test_134_tensor_names_for_22_layers():
    names = C.tensor_names(22)
    assert len(names) == 134 and len(set(names)) == 134
    assert "layers.0.attn_norm.weight" not in names and "layers.1.attn_norm.weight" in names
    from oracle import mbert_oracle as O
    assert set(names) == set(O.parameter_shapes(O.Config()))


def test_roundtrip_through_safetensors(tmp_path):
    from safetensors.numpy import save_file
    t = _tensors()
    save_file(t, str(tmp_path / "m.safetensors"))
    w, head = C.load_safetensors(tmp_path / "m.safetensors")
    assert head is None and len(w["layers"]) == 22
    assert np.array_equal(w["tok_emb"], t["embeddings.tok_embeddings.weight"])
    assert w["layers"][0]["attn_norm"] is None
    assert np.array_equal(w["layers"][5]["attn_norm"], t["layers.5.attn_norm.weight"])
    assert np.array_equal(w["layers"][21]["mlp_Wo"], t["layers.21.mlp.Wo.weight"])
    assert np.array_equal(w["final_norm"], t["final_norm.weight"])


def test_masked_lm_checkpoint_with_prefix_and_f16_storage(tmp_path):
    from safetensors.numpy import save_file
    t = _tensors(n_layers=3, prefix="model.", head=True, dtype=np.float16)
    save_file(t, str(tmp_path / "mlm.safetensors"))
    w, head = C.load_safetensors(tmp_path / "mlm.safetensors")
    assert len(w["layers"]) == 3 and head is not None
    assert np.array_equal(head["decoder_bias"], t["decoder.bias"].astype(np.float32))
    assert np.array_equal(w["layers"][2]["Wi"], t["model.layers.2.mlp.Wi.weight"].astype(np.float32))


def test_loader_rejects_layer0_attn_norm_missing_and_extra():
    t = _tensors(n_layers=2)
    bad = dict(t, **{"layers.0.attn_norm.weight": np.ones(8, np.float32)})
    with pytest.raises(ValueError, match="layer 0"):
        C.weights_from_tensors(bad)
    missing = dict(t)
    del missing["layers.1.mlp_norm.weight"]
    with pytest.raises(ValueError, match="missing"):
        C.weights_from_tensors(missing)
    with pytest.raises(ValueError, match="unexpected"):
        C.weights_from_tensors(dict(t, **{"pooler.weight": np.ones(8, np.float32)}))
    wrong = dict(t, **{"layers.1.attn.Wo.weight": np.ones((8, 9), np.float32)})
    with pytest.raises(ValueError, match="misshapen"):
        C.weights_from_tensors(wrong)


def test_named_configs():
    base = C.config()
    assert (base.theta_global, base.theta_local) == (160000.0, 10000.0)
    g = C.config("granite-embedding-english-r2")
    assert (g.theta_global, g.theta_local, g.half_window, g.global_every) == (80000.0, 10000.0, 64, 3)
    mm = C.config("granite-embedding-311m-multilingual-r2", vocab=1000)
    assert (mm.theta_global, mm.theta_local, mm.vocab) == (150000.0, 160000.0, 1000)
    assert B.mbert_check_config(mm) == B.MBERT_OK
    with pytest.raises(KeyError):
        C.config("bert-base")
