"""GPU parity across the sweep of sequence length, depth and group size, and
at the 64K-token shape in the causal-only mode.

The sweep is B=1, Hq=16, d=128, bf16 N(0,1) inputs, T in {4096, 16384, 65536}
x L in {0, 8, 32, 96} x G in {1, 4, 8} (Hkv = 16 / G): the shape of the
scaling claim on the hyper.ai page on arXiv 2603.15619, section
"Experiments" (overhead shrinks as T and the depth utilisation grow).

- T = 4096: every row of O and LSE against the fp64 oracle (the 4-wave,
  128-row tiles the forward uses for these small grids).
- T = 16384 and 65536: sampled rows per head against the oracle, including
  both sides of the 8-wave kernel's real tile and wave seams.
- The causal-only mode (moda_causal_fwd) at B1 Hq16 Hkv4 T65536: sampled rows
  against the oracle with no depth entries.
- An 8-wave tile whose G does not divide its 256 rows (G = 3: 85 tokens per
  tile, one idle row), sampled.

Tolerances: max-abs 2e-2 on O and 1e-3 on the LSE (bf16 inputs, fp32
accumulation), over every checked element.
"""
import pytest

import oracle
from gpu_util import (BF16_TOL, LSE_TOL_BF16, device_case, gather_rows, max_err,
                      oracle_rows_from_device, out_to_f64, sample_rows, seam_tokens, tile_rows,
                      to_np)
from synth import sweep_points

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SWEEP = sweep_points()
SWEEP_FULL = [c for c in SWEEP if c["T"] == 4096]
SWEEP_SAMPLED = [c for c in SWEEP if c["T"] > 4096]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def m():
    from depth_wise_kv_amd import moda
    return moda


def variant(m, cfg):
    return m.moda_fwd_variant(m.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["L"],
                                           cfg["d"], cfg["dtype"]))


def forward(m, d_in, L):
    kd, vd = (d_in["kd"], d_in["vd"]) if L else (None, None)
    out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], kd, vd, with_lse=True)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("cfg", SWEEP_FULL, ids=[c["name"] for c in SWEEP_FULL])
def test_sweep_full(m, dev, cfg):
    """Every row of a T = 4096 sweep point against the oracle."""
    print(f"[sweep] {cfg['name']} variant={variant(m, cfg)}", flush=True)
    d_in = device_case(cfg, dev)
    out, lse = forward(m, d_in, cfg["L"])
    L = cfg["L"]
    ref, rlse = oracle.moda_forward(to_np(d_in["q"]), to_np(d_in["k"]), to_np(d_in["v"]),
                                    to_np(d_in["kd"]) if L else None,
                                    to_np(d_in["vd"]) if L else None)
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[sweep] {cfg['name']} all rows max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    del d_in, out, lse
    torch.cuda.empty_cache()
    assert e_o <= BF16_TOL, f"O error {e_o}"
    assert e_l <= LSE_TOL_BF16, f"LSE error {e_l}"


def sampled(m, dev, cfg, n_random, causal_only=False):
    v = variant(m, cfg)
    print(f"[sweep] {cfg['name']} variant={v}", flush=True)
    d_in = device_case(cfg, dev)
    if causal_only:
        out, lse = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
        torch.cuda.synchronize()
    else:
        out, lse = forward(m, d_in, cfg["L"])
    rows = sample_rows(cfg, n_random=n_random, seed=cfg["seed"], rows_per_tile=tile_rows(v))
    # every seam token of the kernel's tiles is among the sampled rows of every head
    seams = seam_tokens(cfg["T"], cfg["Hq"] // cfg["Hkv"], tile_rows(v))
    assert seams <= set(int(t) for t in rows[rows[:, 1] == cfg["Hq"] - 1][:, 2])
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    e_o = max_err(out_to_f64(gather_rows(out, rows)), ref)
    e_l = max_err(gather_rows(lse, rows).cpu().numpy(), rlse)
    print(f"[sweep] {cfg['name']} rows={len(rows)} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}",
          flush=True)
    del d_in, out, lse
    torch.cuda.empty_cache()
    assert e_o <= BF16_TOL, f"O error {e_o}"
    assert e_l <= LSE_TOL_BF16, f"LSE error {e_l}"


@pytest.mark.parametrize("cfg", SWEEP_SAMPLED, ids=[c["name"] for c in SWEEP_SAMPLED])
def test_sweep_sampled(m, dev, cfg):
    """T = 16384 and 65536 sweep points: seam rows (of whichever MFMA kernel the
    shape runs) plus 24 random rows per head."""
    assert variant(m, cfg).startswith("mfma_bf16_d128_")
    sampled(m, dev, cfg, n_random=24)


def test_causal_only_long_64k_sampled(m, dev):
    """The causal-only mode at B1 Hq16 Hkv4 T65536 (the shape the MoDA / causal
    time ratio is taken at): sampled rows against the oracle with L = 0."""
    cfg = dict(B=1, Hq=16, Hkv=4, T=65536, L=0, d=128, dtype="bf16", scale=1.0, seed=3000,
               name="long_64k_causal_only")
    sampled(m, dev, cfg, n_random=48, causal_only=True)


@pytest.mark.parametrize("T,L", [(16384, 8), (20000, 5)])
def test_w8_group_not_dividing_tile(m, dev, T, L):
    """G = 3 on the 8-wave kernel: 85 tokens per 256-row tile (one idle row),
    sampled rows on both sides of its seams; T = 20000 leaves a ragged last tile."""
    cfg = dict(B=1, Hq=12, Hkv=4, T=T, L=L, d=128, dtype="bf16", scale=1.0, seed=5900 + L,
               name=f"G3_T{T}_L{L}")
    assert variant(m, cfg) == "mfma_bf16_d128_w8"
    sampled(m, dev, cfg, n_random=32)
