"""Helpers shared by the GPU tests: device upload of seeded inputs and error measures."""
from __future__ import annotations

import numpy as np

TOL_STEP = {"f32": 3e-5, "bf16": 1e-2, "f16": 2e-3}   # per-step, max |err| / max |ref|


def torch():
    import torch as t
    return t


def dev_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def dev(a, dtype):
    from transformer_encoder_amd.model import to_device
    return to_device(a, dtype, "cuda")


def host(t) -> np.ndarray:
    torch().cuda.synchronize()
    return t.detach().float().cpu().double().numpy() if t.dtype != torch().int32 else t.cpu().numpy()


def rel_err(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def min_cos(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    num = np.sum(got * ref, axis=-1)
    den = np.linalg.norm(got, axis=-1) * np.linalg.norm(ref, axis=-1)
    return float(np.min(num / np.maximum(den, 1e-300)))


def meta_for(cu, total, max_pos=8192):
    """Packed-batch meta buffer built by the library from device cu_seqlens."""
    from transformer_encoder_amd import binding as B
    t = torch()
    S = len(cu) - 1
    meta = t.full((B.mbert_meta_ints(total, S),), -7, dtype=t.int32, device="cuda")
    B.mbert_pack_meta(dev_i32(cu), S, total, max_pos, meta)
    return meta


def expected_tiles(cu, tile):
    tiles, first = [], []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        first.append(len(tiles))
        for q0 in range(a, b, tile):
            tiles.append((q0, min(tile, b - q0), a, b))
    first.append(len(tiles))
    return np.array(tiles, dtype=np.int64).reshape(-1, 4), np.array(first)


def meta_order(meta_np, total_max, S):
    """The attention's tile dispatch order stored after the work tiles."""
    off = 8 + total_max + S + 1
    off = (off + 3) & ~3
    tiles_max = -(-total_max // 128) + S
    n_tiles = int(meta_np[2])
    return meta_np[off + 4 * tiles_max:off + 4 * tiles_max + n_tiles]


def split_meta(meta_np, total_max, S):
    counts = meta_np[:8]
    pos = meta_np[8:8 + total_max]
    first = meta_np[8 + total_max:8 + total_max + S + 1]
    off = 8 + total_max + S + 1
    off = (off + 3) & ~3
    n_tiles = counts[2]
    tiles = meta_np[off:off + 4 * n_tiles].reshape(-1, 4)
    return counts, pos, first, tiles
