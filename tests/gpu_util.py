"""Helpers for the GPU tests: host<->device marshalling and oracle checks.

The oracle always consumes bytes downloaded from the device (or the same
host arrays that were uploaded), so both sides see bit-identical inputs.
"""
from __future__ import annotations

import numpy as np

import oracle
from synth import numpy_inputs, torch_inputs

BF16_TOL = 2e-2   # max-abs on O, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs on O, fp32 inputs
LSE_TOL_BF16 = 1e-3
LSE_TOL_F32 = 1e-5


def to_np(t):
    """Device/host torch tensor -> numpy in the oracle's input encoding."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def out_to_f64(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 \
        else t.detach().cpu().numpy().astype(np.float64)


def to_dev(a, dtype, device):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_case(cfg, device):
    """numpy inputs (oracle encoding) and their device copies."""
    h = numpy_inputs(cfg)
    d = {n: to_dev(a, cfg["dtype"], device) for n, a in h.items()}
    return h, d


def device_case(cfg, device):
    return torch_inputs(cfg, device)


def tile_rows(variant):
    """Query rows (token x head pairs) of one workgroup tile of a forward variant
    (moda_fwd_variant's name): 256 for the 8-wave d = 128 kernel, 128 for its
    4-wave and key-split forms and for the kernel of the other head dims and fp32."""
    if variant.endswith("_w8"):
        return 256
    if variant.endswith("_w4") or variant.endswith("_ks"):
        return 128
    if variant in ("mfma_bf16_d32", "mfma_bf16_d64", "mfma_f32_d32", "mfma_f32_d64",
                   "mfma_f32_d128"):
        return 128
    raise ValueError(f"no MFMA tile for variant {variant!r}")


def seam_tokens(T, G, rows_per_tile):
    """Tokens on both sides of the kernel's real seams: the first and last tile
    seams (tiles hold rows_per_tile // G tokens), the seam in the middle of the
    sequence, one wave seam (32 // G tokens per wave), the start of the last
    (possibly ragged) tile, and the first and last tokens."""
    tq = max(1, rows_per_tile // G)
    wq = max(1, 32 // G)
    last = ((T - 1) // tq) * tq           # first token of the last tile
    mid = ((T // 2) // tq) * tq           # a tile seam near the middle
    ts = {0, 1, T - 1, T // 2}
    for s in (tq, mid, last, T - tq, wq):
        ts |= {s - 1, s, s + 1}
    return {t for t in ts if 0 <= t < T}


def sample_rows(cfg, n_random=64, seed=0, rows_per_tile=256):
    """Per (b, h): the rows on both sides of the forward kernel's tile and wave
    seams (``rows_per_tile`` from tile_rows of the variant the shape runs)
    plus n_random seeded rows."""
    B, Hq, Hkv, T = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"]
    G = Hq // Hkv
    fixed = seam_tokens(T, G, rows_per_tile)
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(B):
        for h in range(Hq):
            ts = {t for t in fixed if 0 <= t < T}
            ts |= set(int(x) for x in rng.integers(0, T, size=n_random))
            rows.extend((b, h, t) for t in sorted(ts))
    return np.array(rows, np.int64)


def oracle_rows_from_device(cfg, dev_in, rows):
    """Run the oracle on selected rows, fed from the device tensors."""
    import torch
    B, Hq, Hkv, T, L, d = (cfg[x] for x in ("B", "Hq", "Hkv", "T", "L", "d"))
    G = Hq // Hkv
    rt = torch.from_numpy(rows).to(dev_in["q"].device)
    b, h, t = rt[:, 0], rt[:, 1], rt[:, 2]
    q_rows = to_np(dev_in["q"][b, h, t])
    k, v = to_np(dev_in["k"]), to_np(dev_in["v"])
    if L:
        kd_rows = to_np(dev_in["kd"][b, h // G, t])
        vd_rows = to_np(dev_in["vd"][b, h // G, t])
    else:
        kd_rows = vd_rows = None
    return oracle.moda_rows(rows, (B, Hq, Hkv, T, L, d), q_rows, k, v, kd_rows, vd_rows)


def gather_rows(t, rows):
    import torch
    rt = torch.from_numpy(rows).to(t.device)
    return t[rt[:, 0], rt[:, 1], rt[:, 2]]


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert np.all(np.isfinite(a)), "non-finite GPU output"
    return float(np.max(np.abs(a - b))) if a.size else 0.0
