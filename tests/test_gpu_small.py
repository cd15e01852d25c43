"""GPU parity of the matrix-core forward for the shapes outside the bf16,
d = 128 kernel: bf16 with d in {32, 64} and fp32 with d in {32, 64, 128}
(moda_fwd_small.hip), in its three modes, against the fp64 oracle.

Tolerances (max-abs on every element of O): 1e-5 for fp32, 2e-2 for bf16;
on the LSE 1e-5 and 1e-3.
"""
import pytest

import oracle
from gpu_util import (BF16_TOL, F32_TOL, LSE_TOL_BF16, LSE_TOL_F32, host_case, max_err,
                      out_to_f64)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def m():
    from depth_wise_kv_amd import moda
    return moda


def cfg_of(B, Hq, Hkv, T, L, d, dt, seed):
    return dict(B=B, Hq=Hq, Hkv=Hkv, T=T, L=L, d=d, dtype=dt, scale=1.0, seed=seed)


def tols(dt):
    return (F32_TOL, LSE_TOL_F32) if dt == "f32" else (BF16_TOL, LSE_TOL_BF16)


# (B, Hq, Hkv, T, L, d, dtype): every (dtype, d) pair; T ragged and spanning
# several 32-key tiles and several 128-row workgroups; G from 1 to 128 (G = 3,
# 5, 6 and 24 leave idle rows in each tile); L in {0, 1, 3, 7, 33}.
SMALL_SHAPES = [
    (1, 2, 1, 1, 0, 32, "f32"), (1, 2, 1, 1, 3, 32, "f32"), (1, 2, 1, 64, 4, 32, "f32"),
    (1, 4, 2, 33, 3, 64, "f32"), (2, 4, 1, 70, 0, 128, "f32"), (1, 3, 1, 257, 7, 128, "f32"),
    (1, 8, 8, 100, 1, 64, "f32"), (2, 16, 2, 45, 33, 32, "f32"), (1, 128, 1, 9, 2, 64, "f32"),
    (1, 6, 2, 130, 5, 64, "bf16"), (1, 2, 2, 45, 2, 32, "bf16"), (1, 5, 1, 300, 3, 64, "bf16"),
    (2, 8, 1, 1000, 7, 32, "bf16"), (1, 24, 1, 77, 33, 64, "bf16"), (1, 64, 2, 40, 1, 32, "bf16"),
    (1, 128, 1, 3, 4, 64, "bf16"), (1, 4, 4, 513, 0, 64, "bf16"), (1, 32, 4, 129, 9, 32, "bf16"),
]
IDS = [f"B{b}Hq{hq}Hkv{hk}T{t}L{l}d{d}{dt}" for b, hq, hk, t, l, d, dt in SMALL_SHAPES]


def variant_name(d, dt):
    return f"mfma_{dt}_d{d}"


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", SMALL_SHAPES, ids=IDS)
def test_small_fwd(m, dev, B, Hq, Hkv, T, L, d, dt):
    """moda_fwd (sequence and depth) on every row against the oracle."""
    cfg = cfg_of(B, Hq, Hkv, T, L, d, dt, seed=31 + T + 3 * L + d)
    assert m.moda_fwd_variant(m.make_shape(B, Hq, Hkv, T, L, d, dt)) == variant_name(d, dt)
    h_in, d_in = host_case(cfg, dev)
    kd, vd = (d_in["kd"], d_in["vd"]) if L else (None, None)
    out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], kd, vd, with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"],
                                    h_in["kd"] if L else None, h_in["vd"] if L else None)
    tol, ltol = tols(dt)
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] small fwd {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= tol and e_l <= ltol


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", SMALL_SHAPES[::2], ids=IDS[::2])
def test_small_causal(m, dev, B, Hq, Hkv, T, L, d, dt):
    """moda_causal_fwd (the depth entries left out) against the oracle with L = 0."""
    cfg = cfg_of(B, Hq, Hkv, T, 0, d, dt, seed=500 + T + d)
    h_in, d_in = host_case(cfg, dev)
    out, lse = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"])
    tol, ltol = tols(dt)
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] small causal {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= tol and e_l <= ltol


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", [s for s in SMALL_SHAPES if s[4] > 0],
                         ids=[i for s, i in zip(SMALL_SHAPES, IDS) if s[4] > 0])
def test_small_depth_only(m, dev, B, Hq, Hkv, T, L, d, dt):
    """moda_depth_fwd against the oracle's depth attention, every row."""
    cfg = cfg_of(B, Hq, Hkv, T, L, d, dt, seed=700 + T + L + d)
    h_in, d_in = host_case(cfg, dev)
    out, lse = m.depth_forward(d_in["q"], d_in["kd"], d_in["vd"], with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.depth_forward(h_in["q"], h_in["kd"], h_in["vd"])
    tol, ltol = tols(dt)
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] small depth-only {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= tol and e_l <= ltol


@pytest.mark.parametrize("d,dt", [(32, "f32"), (64, "bf16")])
def test_small_l0_equals_causal_bitwise(m, dev, d, dt):
    """With L = 0, moda_fwd and moda_causal_fwd take the same path: equal bits."""
    cfg = cfg_of(1, 8, 2, 300, 0, d, dt, seed=41)
    _, d_in = host_case(cfg, dev)
    o1, l1 = m.fwd(d_in["q"], d_in["k"], d_in["v"], None, 0, with_lse=True)
    o2, l2 = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_small_merge_identity(m, dev):
    """fp32: causal attention and depth attention alone, merged through their
    LSEs, give moda_fwd (one softmax over the union of the two key sets)."""
    cfg = cfg_of(1, 8, 2, 200, 6, 64, "f32", seed=43)
    _, d_in = host_case(cfg, dev)
    out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                              with_lse=True)
    o_s, l_s = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
    o_d, l_d = m.depth_forward(d_in["q"], d_in["kd"], d_in["vd"], with_lse=True)
    l_s, l_d = l_s.double(), l_d.double()
    mm = torch.maximum(l_s, l_d)
    a, c = torch.exp(l_s - mm), torch.exp(l_d - mm)
    merged = (a[..., None] * o_s.double() + c[..., None] * o_d.double()) / (a + c)[..., None]
    e_o = (merged - out.double()).abs().max().item()
    e_l = (mm + torch.log(a + c) - lse.double()).abs().max().item()
    assert e_o <= F32_TOL and e_l <= LSE_TOL_F32


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", [(1, 16, 4, 16384, 8, 64, "bf16"),
                                               (1, 8, 8, 8192, 24, 32, "bf16"),
                                               (1, 16, 2, 4096, 16, 128, "f32")],
                         ids=["T16384d64bf16", "T8192d32bf16G1", "T4096d128f32G8"])
def test_small_sampled_large(m, dev, B, Hq, Hkv, T, L, d, dt):
    """Larger shapes on sampled rows: the seams of the kernel's 128-row tiles
    and of its waves, plus seeded random rows, against the oracle row by row."""
    from gpu_util import device_case, gather_rows, oracle_rows_from_device, sample_rows, tile_rows
    cfg = cfg_of(B, Hq, Hkv, T, L, d, dt, seed=77 + T + d)
    v = m.moda_fwd_variant(m.make_shape(B, Hq, Hkv, T, L, d, dt))
    assert v == variant_name(d, dt)
    d_in = device_case(cfg, dev)
    out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                              with_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, n_random=16, seed=3, rows_per_tile=tile_rows(v))
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    got = out_to_f64(gather_rows(out, rows))
    glse = gather_rows(lse, rows).cpu().numpy()
    tol, ltol = tols(dt)
    e_o, e_l = max_err(got, ref), max_err(glse, rlse)
    print(f"[parity] small sampled {cfg} rows={len(rows)} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}",
          flush=True)
    assert e_o <= tol and e_l <= ltol
