"""Named configurations of the family and weights by their published tensor names.

Configurations: ModernBERT-base (candding, "ModernBERT", §"The two rope tables": 160,000 on
global layers, 10,000 on local ones) and the two sibling checkpoints whose arithmetic differs
from it only in the RoPE bases (safebydesign.ai, "ModernBertModel 22L 768d", §"Implementing
it": granite-embedding-english-r2 rotates with 80,000 and 10,000,
granite-embedding-311m-multilingual-r2 with 150,000 and 160,000; a window of 128, i.e. 64 keys
either side, and every third layer global, in all three). Dimensions other than 768 / 12 x 64 / 1152 are not
supported by the kernels; the vocabulary size comes from the embedding table.

Tensor names (candding, "ModernBERT", §"The tensors"): embeddings.tok_embeddings.weight,
embeddings.norm.weight, final_norm.weight and, per layer i, layers.{i}.attn.Wqkv.weight,
attn.Wo.weight, mlp_norm.weight, mlp.Wi.weight, mlp.Wo.weight, plus layers.{i}.attn_norm.weight
on every layer but layer 0 (134 tensors for 22 layers, none with a bias). A masked-LM
checkpoint nests them under "model." and adds head.dense.weight, head.norm.weight and
decoder.bias (the decoder weight is the embedding table). Files are read with safetensors'
own reader, which executes nothing from the file; any stored float dtype is accepted and
rounded to the run dtype on upload.
"""
from __future__ import annotations

import numpy as np

from . import binding as B

CONFIGS = {
    "modernbert-base": {"theta_global": 160000.0, "theta_local": 10000.0},
    "granite-embedding-english-r2": {"theta_global": 80000.0, "theta_local": 10000.0},
    "granite-embedding-311m-multilingual-r2": {"theta_global": 150000.0, "theta_local": 160000.0},
}

_LAYER_TENSORS = ("attn.Wqkv.weight", "attn.Wo.weight", "mlp_norm.weight", "mlp.Wi.weight",
                  "mlp.Wo.weight")
_LAYER_KEYS = {"attn.Wqkv.weight": "Wqkv", "attn.Wo.weight": "attn_Wo",
               "mlp_norm.weight": "mlp_norm", "mlp.Wi.weight": "Wi", "mlp.Wo.weight": "mlp_Wo",
               "attn_norm.weight": "attn_norm"}
_HEAD_TENSORS = {"head.dense.weight": "dense", "head.norm.weight": "norm",
                 "decoder.bias": "decoder_bias"}


def config(name: str = "modernbert-base", **overrides) -> B.mbert_config:
    """The C ABI configuration of a named checkpoint, with optional field overrides."""
    if name not in CONFIGS:
        raise KeyError(f"unknown configuration {name!r}; known: {sorted(CONFIGS)}")
    c = B.mbert_default_config()
    for k, v in {**CONFIGS[name], **overrides}.items():
        if not hasattr(c, k):
            raise AttributeError(f"mbert_config has no field {k!r}")
        setattr(c, k, v)
    return c


def tensor_names(n_layers: int) -> list[str]:
    """Every encoder tensor name, in checkpoint order (layer 0 without attn_norm)."""
    names = ["embeddings.tok_embeddings.weight", "embeddings.norm.weight"]
    for i in range(n_layers):
        if i > 0:
            names.append(f"layers.{i}.attn_norm.weight")
        names += [f"layers.{i}.{t}" for t in _LAYER_TENSORS]
    names.append("final_norm.weight")
    return names


def _read(path) -> dict[str, np.ndarray]:
    from safetensors import safe_open
    out = {}
    with safe_open(str(path), framework="pt") as f:
        for k in f.keys():
            out[k] = f.get_tensor(k).float().numpy()
    return out


def weights_from_tensors(tensors: dict[str, np.ndarray]):
    """(weights, head) from a name -> array map. ``weights`` has the layout DeviceModel takes;
    ``head`` holds the masked-LM head tensors when present, else None. Raises on a missing,
    unexpected or misshapen tensor, and on a layer-0 attn_norm (layer 0 has none: the
    embedding norm has just run)."""
    t = {(k[len("model."):] if k.startswith("model.") else k): v for k, v in tensors.items()}
    layer_ids = sorted({int(k.split(".")[1]) for k in t if k.startswith("layers.")})
    n_layers = len(layer_ids)
    if layer_ids != list(range(n_layers)):
        raise ValueError(f"layer indices are not 0..{n_layers - 1}: {layer_ids}")
    if "layers.0.attn_norm.weight" in t:
        raise ValueError("layers.0.attn_norm.weight present: layer 0 has no attention norm")
    names = tensor_names(n_layers)
    missing = [n for n in names if n not in t]
    extra = sorted(set(t) - set(names) - set(_HEAD_TENSORS))
    if missing or extra:
        raise ValueError(f"missing tensors {missing[:5]}, unexpected tensors {extra[:5]}")
    E = t["embeddings.tok_embeddings.weight"]
    V, D = E.shape
    I = t["layers.0.mlp.Wo.weight"].shape[1]
    want = {"embeddings.tok_embeddings.weight": (V, D), "embeddings.norm.weight": (D,),
            "final_norm.weight": (D,)}
    for i in range(n_layers):
        p = f"layers.{i}."
        if i > 0:
            want[p + "attn_norm.weight"] = (D,)
        want.update({p + "attn.Wqkv.weight": (3 * D, D), p + "attn.Wo.weight": (D, D),
                     p + "mlp_norm.weight": (D,), p + "mlp.Wi.weight": (2 * I, D),
                     p + "mlp.Wo.weight": (D, I)})
    bad = [f"{n} {t[n].shape} != {s}" for n, s in want.items() if tuple(t[n].shape) != s]
    if bad:
        raise ValueError("misshapen tensors: " + "; ".join(bad[:5]))
    w = {"tok_emb": E, "emb_norm": t["embeddings.norm.weight"],
         "final_norm": t["final_norm.weight"], "layers": []}
    for i in range(n_layers):
        lw = {"attn_norm": None}
        for suffix, key in _LAYER_KEYS.items():
            name = f"layers.{i}.{suffix}"
            if name in t:
                lw[key] = t[name]
        w["layers"].append(lw)
    head = None
    present = [n for n in _HEAD_TENSORS if n in t]
    if present:
        if len(present) != len(_HEAD_TENSORS):
            raise ValueError(f"incomplete masked-LM head: {present}")
        head = {_HEAD_TENSORS[n]: t[n] for n in _HEAD_TENSORS}
        if head["dense"].shape != (D, D) or head["norm"].shape != (D,) or head["decoder_bias"].shape != (V,):
            raise ValueError("misshapen masked-LM head tensors")
    return w, head


def load_safetensors(path):
    """(weights, head) from a .safetensors file of the family (see weights_from_tensors)."""
    return weights_from_tensors(_read(path))
