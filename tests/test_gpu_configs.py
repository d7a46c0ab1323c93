"""The sibling configurations end to end (safebydesign.ai, 'ModernBertModel 22L 768d',
'Implementing it': RoPE bases 80,000/10,000 and 150,000/160,000 besides ModernBERT-base's
160,000/10,000), with the weights loaded by their published names from a safetensors file:
3 layers (one global, two local), a reduced vocabulary, against the oracle at the same bases."""
import numpy as np
import pytest

from gpu_util import dev_i32, host, min_cos
from oracle import mbert_oracle as O
from workloads import Dims, cu_from_lengths, make_weights, rng

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["modernbert-base", "granite-embedding-english-r2",
                                  "granite-embedding-311m-multilingual-r2"])
def test_named_config_from_safetensors(name, tmp_path):
    from safetensors.numpy import save_file
    from transformer_encoder_amd import checkpoint as C
    from transformer_encoder_amd.model import DeviceModel
    V = 1000
    w = make_weights(Dims(n_layers=3, vocab=V), "bf16", 181)
    t = {"embeddings.tok_embeddings.weight": w["tok_emb"], "embeddings.norm.weight": w["emb_norm"],
         "final_norm.weight": w["final_norm"]}
    for i, lw in enumerate(w["layers"]):
        keys = {"attn_norm": "attn_norm.weight", "Wqkv": "attn.Wqkv.weight", "attn_Wo": "attn.Wo.weight",
                "mlp_norm": "mlp_norm.weight", "Wi": "mlp.Wi.weight", "mlp_Wo": "mlp.Wo.weight"}
        for k, n in keys.items():
            if lw[k] is not None:
                t[f"layers.{i}.{n}"] = lw[k]
    save_file({k: np.ascontiguousarray(v, dtype=np.float32) for k, v in t.items()},
              str(tmp_path / "m.safetensors"))
    wl, head = C.load_safetensors(tmp_path / "m.safetensors")
    assert head is None
    cfg = C.config(name)
    m = DeviceModel(wl, "bf16", cfg=cfg)
    cu = cu_from_lengths([300, 77])
    ids = rng(182, 1).integers(0, V, int(cu[-1]))
    out, pooled, _ = m.encode(dev_i32(ids), dev_i32(cu))
    ocfg = O.Config(n_layers=3, vocab=V, theta_global=cfg.theta_global, theta_local=cfg.theta_local)
    ref, rpool = O.encode(ids, cu, w, ocfg)
    got = host(out)
    assert np.max(np.abs(got - ref)) < 2e-2 and min_cos(got, ref) > 0.999
    assert np.max(np.abs(host(pooled) - rpool)) < 2e-2
