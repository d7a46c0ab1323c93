"""Device weights and convenience calls over the C ABI.

``DeviceModel`` uploads a weight set to the GPU with PyTorch (device memory only), builds the
RoPE tables with the library, fills the ``mbert_weights`` struct and runs the forward through
``mbert_encode`` / ``mbert_encode_padded``. No arithmetic of the encoder happens here.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import binding as B

_TORCH_DTYPES = None


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload values already representable in ``dtype`` (exact through float32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32)))
    return t.to(device=device).to(torch_dtype(dtype))


def int32_device(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(device)


class DeviceModel:
    def __init__(self, weights: dict, dtype: str, device="cuda", cfg: B.mbert_config | None = None,
                 stream=None, fold: bool = True):
        import torch
        self.dtype_name = dtype
        self.dtype = B.DTYPES[dtype]
        self.device = device
        self.cfg = cfg if cfg is not None else B.mbert_default_config()
        self.cfg.n_layers = len(weights["layers"])
        self.cfg.vocab = int(weights["tok_emb"].shape[0])
        self._keep = []

        def up(a):
            t = to_device(a, dtype, device)
            self._keep.append(t)
            return t

        self.tok_emb = up(weights["tok_emb"])
        self.emb_norm = up(weights["emb_norm"])
        self.final_norm = up(weights["final_norm"])
        n = self.cfg.n_layers
        self.layers_c = (B.mbert_layer_weights * n)()
        self.layers = []
        for i, lw in enumerate(weights["layers"]):
            d = {k: (up(v) if v is not None else None) for k, v in lw.items()}
            self.layers.append(d)
            L = self.layers_c[i]
            L.attn_norm = B.ptr(d["attn_norm"])
            L.Wqkv, L.attn_Wo = B.ptr(d["Wqkv"]), B.ptr(d["attn_Wo"])
            L.mlp_norm, L.Wi, L.mlp_Wo = B.ptr(d["mlp_norm"]), B.ptr(d["Wi"]), B.ptr(d["mlp_Wo"])
        self.rope = torch.empty(B.mbert_rope_table_floats(self.cfg), dtype=torch.float32,
                                device=device)
        B.mbert_build_rope_tables(self.cfg, self.rope, stream)
        self.w = B.mbert_weights()
        self.w.cfg = self.cfg
        self.w.dtype = self.dtype
        self.w.tok_emb, self.w.emb_norm = B.ptr(self.tok_emb), B.ptr(self.emb_norm)
        self.w.final_norm = B.ptr(self.final_norm)
        self.w.layers = ctypes.cast(self.layers_c, ctypes.POINTER(B.mbert_layer_weights))
        self.w.rope = B.ptr(self.rope)
        # LayerNorms folded into the following GEMMs (every dtype; fold=False runs them apart)
        self.folded = None
        nb = B.mbert_folded_bytes(self.cfg, self.dtype)
        if fold and nb > 0:
            self.folded = torch.empty(nb, dtype=torch.uint8, device=device)
            B.mbert_fold_norms(self.w, self.folded, nb, stream)
            self.w.folded = B.ptr(self.folded)

    def set_fold(self, on: bool):
        """Switch the forward between folded and separate LayerNorms (if folded weights exist)."""
        self.w.folded = B.ptr(self.folded) if (on and self.folded is not None) else None

    def workspace(self, total_max: int, n_seqs: int):
        import torch
        nbytes = B.mbert_workspace_bytes(self.cfg, self.dtype, total_max, n_seqs)
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)

    def layout(self, total_max: int, n_seqs: int) -> B.mbert_ws_layout:
        return B.mbert_workspace_layout(self.cfg, self.dtype, total_max, n_seqs)

    def encode(self, ids, cu_seqlens, total: int | None = None, ws=None, pooled=True, stream=None):
        """Packed batch: ids [T] and cu_seqlens [S+1] int32 device tensors."""
        import torch
        S = int(cu_seqlens.numel()) - 1
        T = int(ids.numel()) if total is None else total
        ws = ws if ws is not None else self.workspace(T, S)
        out = torch.empty((T, 768), dtype=torch.float32, device=self.device)
        pool = torch.empty((S, 768), dtype=torch.float32, device=self.device) if pooled else None
        B.mbert_encode(self.w, ids, cu_seqlens, S, T, ws, ws.numel(), out, pool, stream)
        return out, pool, ws

    def encode_padded_keymask(self, ids_pad, mask, ws=None, stream=None):
        """Padded batch run at full width without unpadding (pad keys masked)."""
        import torch
        Bn, Tp = ids_pad.shape
        ws = ws if ws is not None else self.workspace(Bn * Tp, Bn)
        out = torch.empty((Bn, Tp, 768), dtype=torch.float32, device=self.device)
        pool = torch.empty((Bn, 768), dtype=torch.float32, device=self.device)
        B.mbert_encode_padded_keymask(self.w, ids_pad, mask, Bn, Tp, ws, ws.numel(), out, pool,
                                      stream)
        return out, pool, ws

    def encode_padded(self, ids_pad, mask, ws=None, stream=None):
        """Padded batch: ids_pad, mask [B, Tpad] int32 device tensors."""
        import torch
        Bn, Tp = ids_pad.shape
        ws = ws if ws is not None else self.workspace(Bn * Tp, Bn)
        out = torch.empty((Bn, Tp, 768), dtype=torch.float32, device=self.device)
        pool = torch.empty((Bn, 768), dtype=torch.float32, device=self.device)
        B.mbert_encode_padded(self.w, ids_pad, mask, Bn, Tp, ws, ws.numel(), out, pool, stream)
        return out, pool, ws
