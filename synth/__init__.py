"""Seeded synthetic inputs and the workload table for the MoDA forward.

This module holds input generation only: shapes, seeds and random draws.  It
contains none of the method's arithmetic, so both the oracle side (tests) and
the HIP side (tests, bench) may use it.

Recipe (the same for every workload): i.i.d. standard normal draws, times a
per-workload scale, rounded to the input dtype by round-to-nearest-even.
Tensor ids: Q=0, K=1, V=2, K_depth=3, V_depth=4; tensor ``i`` of a workload
with seed ``s`` is drawn from seed ``s + i``.

Layouts: Q [B,Hq,T,d]; K, V [B,Hkv,T,d]; K_depth, V_depth [B,Hkv,T,L,d].
"""
from __future__ import annotations

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "kd": 3, "vd": 4}

# Named workloads.  "tiny" is small enough for a full fp64 CPU check; the
# others are the shapes used for parity sampling and timing.
WORKLOADS = {
    # B=1 Hq=2 Hkv=1 T=64 d=32 L=4, fp32
    "tiny": dict(B=1, Hq=2, Hkv=1, T=64, L=4, d=32, dtype="f32", scale=1.0, seed=1000),
    # 1.5B-model mid-stack layer: one depth entry per preceding layer
    "layer_1p5b": dict(B=2, Hq=16, Hkv=4, T=4096, L=24, d=128, dtype="bf16", scale=0.5,
                       seed=2000),
    # 64K context, GQA G=4, 32 depth entries
    "long_64k": dict(B=1, Hq=16, Hkv=4, T=65536, L=32, d=128, dtype="bf16", scale=1.0,
                     seed=3000),
    # 64 layers x (attention + FFN) depth entries: depth traffic ~ sequence traffic
    "depth_heavy": dict(B=4, Hq=32, Hkv=8, T=8192, L=128, d=128, dtype="bf16", scale=1.0,
                        seed=4000),
}

SWEEP_T = (4096, 16384, 65536)
SWEEP_L = (0, 8, 32, 96)
SWEEP_G = (1, 4, 8)


def sweep_points():
    """The T x L x G sweep at B=1, Hq=16, d=128, bf16 (Hkv = 16 / G)."""
    pts = []
    idx = 0
    for T in SWEEP_T:
        for L in SWEEP_L:
            for G in SWEEP_G:
                pts.append(dict(B=1, Hq=16, Hkv=16 // G, T=T, L=L, d=128, dtype="bf16",
                                scale=1.0, seed=5000 + 100 * idx,
                                name=f"sweep_T{T}_L{L}_G{G}"))
                idx += 1
    return pts


def shapes(cfg):
    B, Hq, Hkv, T, L, d = (cfg[x] for x in ("B", "Hq", "Hkv", "T", "L", "d"))
    return {"q": (B, Hq, T, d), "k": (B, Hkv, T, d), "v": (B, Hkv, T, d),
            "kd": (B, Hkv, T, L, d), "vd": (B, Hkv, T, L, d)}


# ---------------------------------------------------------------- numpy (CPU)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def numpy_inputs(cfg, seed=None):
    """Host tensors for a workload dict (needs B,Hq,Hkv,T,L,d,dtype,scale).

    Returns a dict name -> ndarray: float32 for dtype "f32", float64 for
    "f64", uint16 bf16 bit patterns for "bf16".
    """
    seed = cfg.get("seed", 0) if seed is None else seed
    out = {}
    for name, shp in shapes(cfg).items():
        rng = np.random.Generator(np.random.PCG64(seed + TENSOR_IDS[name]))
        x = rng.standard_normal(shp) * cfg.get("scale", 1.0)
        if cfg["dtype"] == "f64":
            out[name] = x.astype(np.float64)
        elif cfg["dtype"] == "f32":
            out[name] = x.astype(np.float32)
        elif cfg["dtype"] == "bf16":
            out[name] = f32_to_bf16_bits(x.astype(np.float32))
        else:
            raise ValueError(cfg["dtype"])
    return out


# ---------------------------------------------------------------- torch (device)

def torch_inputs(cfg, device, seed=None):
    """Device tensors for a workload: torch's counter-based generator on
    ``device``, fp32 draws, scaled, then cast (RNE) to the workload dtype."""
    import torch
    seed = cfg.get("seed", 0) if seed is None else seed
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[cfg["dtype"]]
    out = {}
    for name, shp in shapes(cfg).items():
        g = torch.Generator(device=device)
        g.manual_seed(seed + TENSOR_IDS[name])
        n = int(np.prod(shp))
        if n == 0:
            out[name] = torch.empty(shp, dtype=dt, device=device)
            continue
        x = torch.empty(shp, dtype=dt, device=device)
        # draw in slabs over the two leading axes to bound the fp32 temporary
        flat = x.view(shp[0] * shp[1], -1)
        for i in range(flat.shape[0]):
            tmp = torch.randn(flat.shape[1], generator=g, device=device, dtype=torch.float32)
            sc = cfg.get("scale", 1.0)
            if sc != 1.0:
                tmp.mul_(sc)
            flat[i].copy_(tmp)
            del tmp
        out[name] = x
    return out
