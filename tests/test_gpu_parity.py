"""GPU parity: libmoda (through its C ABI) against the fp64 oracle, plus
invariants that need no oracle.  Runs only on an MI355X (pytest -m gpu).

Tolerances (max-abs on O over every checked element): 1e-5 for fp32 inputs,
2e-2 for bf16 inputs with fp32 accumulation.
"""
import numpy as np
import pytest

import oracle
from gpu_util import (BF16_TOL, F32_TOL, LSE_TOL_BF16, LSE_TOL_F32, device_case, gather_rows,
                      host_case, max_err, oracle_rows_from_device, out_to_f64, sample_rows,
                      tile_rows, to_np)
from synth import WORKLOADS

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


def run_full(m, d_in, L, with_lse=True):
    kd, vd = (d_in["kd"], d_in["vd"]) if L else (None, None)
    out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], kd, vd, with_lse=True)
    torch.cuda.synchronize()
    return out, lse


def check_full(m, cfg, dev, tol=None, lse_tol=None):
    h_in, d_in = host_case(cfg, dev)
    out, lse = run_full(m, d_in, cfg["L"])
    L = cfg["L"]
    ref, rlse = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"],
                                    h_in["kd"] if L else None, h_in["vd"] if L else None)
    f32 = cfg["dtype"] == "f32"
    tol = tol or (F32_TOL if f32 else BF16_TOL)
    lse_tol = lse_tol or (LSE_TOL_F32 if f32 else LSE_TOL_BF16)
    e_o = max_err(out_to_f64(out), ref)
    e_l = max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= tol, f"O error {e_o} > {tol}"
    assert e_l <= lse_tol, f"LSE error {e_l} > {lse_tol}"
    return out, lse


def shape_cfg(B, Hq, Hkv, T, L, d=128, dtype="bf16", scale=1.0, seed=7):
    return dict(B=B, Hq=Hq, Hkv=Hkv, T=T, L=L, d=d, dtype=dtype, scale=scale, seed=seed)


def kernel_rows(m, cfg):
    """Sampled rows of a shape, with the seams of the tile the forward runs it on."""
    v = m.moda_fwd_variant(m.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["L"],
                                        cfg["d"], cfg["dtype"]))
    return tile_rows(v)


# ------------------------------------------------------------------ full-oracle parity

def test_tiny_workload_fp32(m, dev):
    """B1 Hq2 Hkv1 T64 d32 L4, fp32 (matrix-core fp32 kernel), whole tensor."""
    check_full(m, WORKLOADS["tiny"], dev)


MFMA_SHAPES = [
    # (B, Hq, Hkv, T, L): ragged T, L in {0,1,3,24}, G in {1,2,3,4,8,16,24,32}
    (1, 2, 1, 1, 0), (1, 2, 1, 1, 3), (1, 4, 1, 17, 1), (1, 4, 2, 129, 3),
    (2, 8, 2, 1000, 24), (1, 16, 4, 200, 0), (1, 3, 1, 50, 5), (1, 4, 4, 77, 2),
    (1, 32, 2, 130, 4), (1, 64, 2, 40, 3), (1, 24, 1, 33, 2), (1, 8, 1, 300, 40),
    (1, 16, 4, 64, 32), (2, 4, 1, 65, 7), (1, 16, 4, 70, 100), (1, 4, 4, 9, 129),
    (1, 8, 1, 40, 65),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,L", MFMA_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in MFMA_SHAPES])
def test_mfma_path_small(m, dev, B, Hq, Hkv, T, L):
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=11 + T + 7 * L)
    assert m.moda_fwd_variant(m.make_shape(B, Hq, Hkv, T, L, 128, "bf16")).startswith(
        "mfma_bf16_d128")
    check_full(m, cfg, dev)


@pytest.mark.parametrize("variant", ["w4", "w8", "ks"])
@pytest.mark.parametrize("B,Hq,Hkv,T,L", [(2, 8, 2, 1000, 24), (1, 16, 4, 70, 100),
                                          (1, 8, 1, 300, 40), (1, 32, 4, 513, 0),
                                          (1, 12, 4, 700, 9), (1, 2, 1, 257, 3),
                                          (1, 128, 1, 40, 5), (2, 3, 1, 131, 1)])
def test_both_wave_counts(m, dev, monkeypatch, variant, B, Hq, Hkv, T, L):
    """The 4-wave (128-row), 8-wave (256-row) and key-split (8 waves on 128 rows)
    kernels on the same shapes, whichever the shape would get by default,
    against the full oracle."""
    monkeypatch.setenv("MODA_FWD_VARIANT", variant)
    assert m.moda_fwd_variant(m.make_shape(B, Hq, Hkv, T, L, 128, "bf16")) == \
        f"mfma_bf16_d128_{variant}"
    check_full(m, shape_cfg(B, Hq, Hkv, T, L, seed=57 + T + L), dev)


GENERIC_SHAPES = [  # G above 128: the one-wave-per-row VALU kernel
    (1, 256, 1, 4, 2, 32, "f32"), (1, 256, 1, 3, 0, 64, "bf16"), (1, 512, 2, 3, 1, 128, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", GENERIC_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}d{d}{dt}" for b, hq, hk, t, l, d, dt
                              in GENERIC_SHAPES])
def test_generic_path(m, dev, B, Hq, Hkv, T, L, d, dt):
    cfg = shape_cfg(B, Hq, Hkv, T, L, d=d, dtype=dt, seed=3 + T)
    assert m.moda_fwd_variant(m.make_shape(B, Hq, Hkv, T, L, d, dt)) == "generic"
    check_full(m, cfg, dev)


def test_layer_1p5b_full(m, dev):
    """B2 Hq16 Hkv4 T4096 d128 L24, bf16 N(0,1)*0.5: every row against the oracle."""
    cfg = WORKLOADS["layer_1p5b"]
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, cfg["L"])
    ref, rlse = oracle.moda_forward(*(to_np(d_in[n]) for n in ("q", "k", "v", "kd", "vd")))
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] layer_1p5b max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


def sampled_check(m, cfg, dev, n_random=64):
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, cfg["L"])
    rows = sample_rows(cfg, n_random=n_random, seed=cfg["seed"], rows_per_tile=kernel_rows(m, cfg))
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    got = out_to_f64(gather_rows(out, rows))
    got_l = gather_rows(lse, rows).cpu().numpy()
    e_o, e_l = max_err(got, ref), max_err(got_l, rlse)
    print(f"[parity] {cfg.get('name', cfg)} rows={len(rows)} max|dO|={e_o:.3e} "
          f"max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    del d_in, out, lse
    torch.cuda.empty_cache()


def test_long_64k_sampled(m, dev):
    """B1 Hq16 Hkv4 T65536 d128 L32: 73 sampled rows per head."""
    sampled_check(m, WORKLOADS["long_64k"], dev)


def test_depth_heavy_sampled(m, dev):
    """B4 Hq32 Hkv8 T8192 d128 L128: 73 sampled rows per (b, head)."""
    sampled_check(m, WORKLOADS["depth_heavy"], dev)


def adversarial_inputs(kind, B=1, Hq=8, Hkv=2, T=700, L=5, seed=21):
    """bf16 inputs whose scores force the online softmax to move its reference
    max often: sequence scores that rise (or fall) steeply along the key axis,
    and depth entries that dominate every even token's row."""
    from synth import f32_to_bf16_bits
    rng = np.random.default_rng(seed)
    d = 128
    j = np.arange(T, dtype=np.float64)
    s = 0.05 + 8.0 * j / T if kind == "rising" else 8.0 - 7.9 * j / T
    q = rng.standard_normal((B, Hq, T, d)) * 0.5 + 1.0
    k = (rng.standard_normal((B, Hkv, T, d)) * 0.5 + 1.0) * s[None, None, :, None]
    v = rng.standard_normal((B, Hkv, T, d))
    kd = rng.standard_normal((B, Hkv, T, L, d)) * 0.5 + 1.0
    kd *= np.where(np.arange(T) % 2 == 0, 10.0, 0.1)[None, None, :, None, None]
    vd = rng.standard_normal((B, Hkv, T, L, d))
    return {n: f32_to_bf16_bits(a.astype(np.float32))
            for n, a in dict(q=q, k=k, v=v, kd=kd, vd=vd).items()}


@pytest.mark.parametrize("kind,Hq,Hkv", [("rising", 8, 2), ("falling", 8, 2), ("rising", 4, 4),
                                         ("rising", 32, 4)])
def test_rescale_paths(m, dev, kind, Hq, Hkv):
    """Steep score ramps and dominant depth entries: many reference-max moves
    inside the key loop and in the depth part, against the oracle."""
    from gpu_util import to_dev
    h = adversarial_inputs(kind, Hq=Hq, Hkv=Hkv)
    d_in = {n: to_dev(a, "bf16", dev) for n, a in h.items()}
    out, lse = run_full(m, d_in, 5)
    ref, rlse = oracle.moda_forward(h["q"], h["k"], h["v"], h["kd"], h["vd"])
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] rescale {kind} Hq{Hq} Hkv{Hkv} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}",
          flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


# ------------------------------------------------------------------ natural depth layout

NATURAL_SHAPES = [(1, 16, 4, 70, 5), (2, 4, 4, 9, 33), (1, 8, 1, 40, 65), (1, 32, 8, 300, 128),
                  (1, 6, 2, 257, 3), (1, 16, 4, 1000, 24)]


@pytest.mark.parametrize("B,Hq,Hkv,T,L", NATURAL_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in NATURAL_SHAPES])
def test_fwd_natural_parity(m, dev, B, Hq, Hkv, T, L):
    """moda_fwd_natural (depth K/V read in their natural layout) and the packed
    path both match the full oracle.  (They visit a row's depth entries in
    different blocks, so they differ in rounding, not in what they compute.)"""
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=700 + T + L)
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, L)
    out_n, lse_n = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                 with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.moda_forward(*(to_np(d_in[n]) for n in ("q", "k", "v", "kd", "vd")))
    for name, o, l in (("packed", out, lse), ("natural", out_n, lse_n)):
        e_o, e_l = max_err(out_to_f64(o), ref), max_err(l.cpu().numpy(), rlse)
        print(f"[parity] {name} {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
        assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


def layer_major(t):
    """[B,Hkv,T,L,d] -> [L,B,Hkv,T,d]: entry i of every token in one slice."""
    return t.permute(3, 0, 1, 2, 4).contiguous()


@pytest.mark.parametrize("B,Hq,Hkv,T,L", NATURAL_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in NATURAL_SHAPES])
def test_fwd_layers_matches_natural(m, dev, B, Hq, Hkv, T, L):
    """moda_fwd_layers (depth stream as per-layer slices [L,B,Hkv,T,d]) gives
    the natural-layout forward's O and LSE bit for bit: the same depth rows
    reach the same operand registers in the same order."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=800 + T + L)
    d_in = device_case(cfg, dev)
    out, lse = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                             with_lse=True)
    out_l, lse_l = m.fwd_layers(d_in["q"], d_in["k"], d_in["v"], layer_major(d_in["kd"]),
                                layer_major(d_in["vd"]), with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_l) and torch.equal(lse, lse_l)


def test_fwd_near_size_limit(m, dev):
    """T*L just under its 2^23 limit (T = 65536, L = 127, G = 4): the packed
    and the natural-layout forwards against the oracle on sampled rows, and the
    layer-major forward, whose depth reads span all T*L rows like the natural
    one's, equal to the natural one bit for bit."""
    cfg = dict(B=1, Hq=4, Hkv=1, T=65536, L=127, d=128, dtype="bf16", scale=1.0, seed=6100,
               name="T65536_L127")
    assert cfg["T"] * cfg["L"] < 1 << 23
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, cfg["L"])
    rows = sample_rows(cfg, n_random=64, seed=cfg["seed"], rows_per_tile=kernel_rows(m, cfg))
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    e_o = max_err(out_to_f64(gather_rows(out, rows)), ref)
    e_l = max_err(gather_rows(lse, rows).cpu().numpy(), rlse)
    print(f"[parity] {cfg['name']} rows={len(rows)} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}",
          flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    del out, lse
    out_n, lse_n = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                 with_lse=True)
    torch.cuda.synchronize()
    e_o = max_err(out_to_f64(gather_rows(out_n, rows)), ref)
    e_l = max_err(gather_rows(lse_n, rows).cpu().numpy(), rlse)
    print(f"[parity] {cfg['name']} natural max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    out_l, lse_l = m.fwd_layers(d_in["q"], d_in["k"], d_in["v"], layer_major(d_in["kd"]),
                                layer_major(d_in["vd"]), with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_l) and torch.equal(lse_n, lse_l)
    del d_in, out_n, lse_n, out_l, lse_l
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,Hq,Hkv,T,L", NATURAL_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in NATURAL_SHAPES])
def test_fwd_masked_scan_matches_natural(m, dev, B, Hq, Hkv, T, L):
    """The masked-scan ablation (every earlier token's depth entries scanned,
    all but the row's own masked out) gives the natural-layout forward's O and
    LSE bit for bit: the extra blocks carry zero weight."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=900 + T + L)
    d_in = device_case(cfg, dev)
    out_n, lse_n = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                 with_lse=True)
    out_s, lse_s = m.fwd_masked_scan(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                     with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_s) and torch.equal(lse_n, lse_s)


def test_depth_layouts_at_the_index_limit(m, dev):
    """T * L just below 2^23: the largest depth stream the row-by-row layouts
    take (a 32-bit flat index; a 2 GiB buffer range for the natural layout's
    V loads).  The natural and layer-major forwards agree bit for bit, and
    sampled rows (the last tokens included) of both them and the packed path
    match the oracle."""
    B, Hq, Hkv, T, L = 1, 4, 1, 65535, 128
    assert T * L < (1 << 23) and T * L * 256 > (1 << 30)
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=1234)
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, L)
    out_n, lse_n = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                 with_lse=True)
    kl, vl = layer_major(d_in["kd"]), layer_major(d_in["vd"])
    out_l, lse_l = m.fwd_layers(d_in["q"], d_in["k"], d_in["v"], kl, vl, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_n, out_l) and torch.equal(lse_n, lse_l)
    del kl, vl, out_l, lse_l
    rows = sample_rows(cfg, n_random=24, seed=9, rows_per_tile=kernel_rows(m, cfg))
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    for name, o, l in (("packed", out, lse), ("natural", out_n, lse_n)):
        e_o = max_err(out_to_f64(gather_rows(o, rows)), ref)
        e_l = max_err(gather_rows(l, rows).cpu().numpy(), rlse)
        print(f"[limit] {name} T*L={T * L} rows={len(rows)} max|dO|={e_o:.3e} "
              f"max|dLSE|={e_l:.3e}", flush=True)
        assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    del d_in, out, lse, out_n, lse_n
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,Hq,Hkv,T,L", NATURAL_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in NATURAL_SHAPES])
def test_fwd_capacity_matches_natural(m, dev, B, Hq, Hkv, T, L):
    """A natural-layout stream with room for 7 more entries per token (the
    spare slots hold NaN): the strided forward over its first L entries gives
    the natural-layout forward's O and LSE bit for bit."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=820 + T + L)
    d_in = device_case(cfg, dev)
    out, lse = m.fwd_natural(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                             with_lse=True)
    cap = L + 7
    kc = torch.full((B, Hkv, T, cap, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    vc = torch.full_like(kc, float("nan"))
    kc[:, :, :, :L], vc[:, :, :, :L] = d_in["kd"], d_in["vd"]
    out_c, lse_c = m.fwd_capacity(d_in["q"], d_in["k"], d_in["v"], kc, vc, L, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_c) and torch.equal(lse, lse_c)


def test_fwd_layers_stream_prefix(m, dev):
    """A layer reads only the first l slices of a longer stream: the forward
    with L = l over a 40-slice stream equals the oracle on those l entries,
    and the slices past l are never read (they hold NaN here)."""
    B, Hq, Hkv, T, Lcap, l = 1, 16, 4, 1500, 40, 13
    cfg = shape_cfg(B, Hq, Hkv, T, l, seed=901)
    d_in = device_case(cfg, dev)
    kl = torch.full((Lcap, B, Hkv, T, 128), float("nan"), dtype=torch.bfloat16, device=dev)
    vl = torch.full_like(kl, float("nan"))
    kl[:l], vl[:l] = layer_major(d_in["kd"]), layer_major(d_in["vd"])
    out, lse = m.fwd_layers(d_in["q"], d_in["k"], d_in["v"], kl, vl, l, with_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, n_random=16, seed=5, rows_per_tile=kernel_rows(m, cfg))
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    e_o = max_err(out_to_f64(gather_rows(out, rows)), ref)
    e_l = max_err(gather_rows(lse, rows).cpu().numpy(), rlse)
    print(f"[layers] prefix l={l} of {Lcap}: max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


# ------------------------------------------------------------------ depth attention alone

DEPTH_SHAPES = [  # (B, Hq, Hkv, T, L, d, dtype): MFMA path and generic path, ragged sizes
    (1, 16, 4, 70, 5, 128, "bf16"), (2, 4, 4, 9, 33, 128, "bf16"), (1, 8, 1, 40, 65, 128, "bf16"),
    (1, 32, 8, 300, 128, 128, "bf16"), (1, 2, 1, 64, 4, 32, "f32"), (1, 6, 2, 30, 3, 64, "bf16"),
    (2, 4, 2, 17, 1, 128, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", DEPTH_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}d{d}{dt}"
                              for b, hq, hk, t, l, d, dt in DEPTH_SHAPES])
def test_depth_only_parity(m, dev, B, Hq, Hkv, T, L, d, dt):
    """moda_depth_fwd against the oracle's depth attention, every row."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, d=d, dtype=dt, seed=900 + T + L)
    h_in, d_in = host_case(cfg, dev)
    out, lse = m.depth_forward(d_in["q"], d_in["kd"], d_in["vd"], with_lse=True)
    torch.cuda.synchronize()
    ref, rlse = oracle.depth_forward(h_in["q"], h_in["kd"], h_in["vd"])
    tol, ltol = (F32_TOL, LSE_TOL_F32) if dt == "f32" else (BF16_TOL, LSE_TOL_BF16)
    e_o, e_l = max_err(out_to_f64(out), ref), max_err(lse.cpu().numpy(), rlse)
    print(f"[parity] depth-only {cfg} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= tol and e_l <= ltol


def test_depth_only_merges_with_causal(m, dev):
    """GPU causal attention and GPU depth attention alone, merged through
    their LSEs, reproduce the GPU MoDA forward (one softmax over the union)."""
    cfg = shape_cfg(1, 16, 4, 600, 24, seed=77)
    d_in = device_case(cfg, dev)
    out, lse = run_full(m, d_in, cfg["L"])
    o_s, l_s = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
    o_d, l_d = m.depth_forward(d_in["q"], d_in["kd"], d_in["vd"], with_lse=True)
    l_s, l_d = l_s.double(), l_d.double()
    mm = torch.maximum(l_s, l_d)
    a, c = torch.exp(l_s - mm), torch.exp(l_d - mm)
    merged = (a[..., None] * o_s.double() + c[..., None] * o_d.double()) / (a + c)[..., None]
    e_o = (merged - out.double()).abs().max().item()
    e_l = (mm + torch.log(a + c) - lse.double()).abs().max().item()
    print(f"[parity] causal+depth merge max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


# ------------------------------------------------------------------ invariants

def test_l0_equals_causal_bitwise(m, dev):
    cfg = shape_cfg(1, 16, 4, 1000, 0, seed=5)
    _, d_in = host_case(cfg, dev)
    o1, l1 = m.fwd(d_in["q"], d_in["k"], d_in["v"], None, 0, with_lse=True)
    o2, l2 = m.causal_fwd(d_in["q"], d_in["k"], d_in["v"], with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_causal_mode_ignores_depth(m, dev):
    """moda_causal_fwd on a shape with L > 0 equals causal attention (oracle, L=0)."""
    cfg = shape_cfg(1, 8, 2, 257, 0, seed=9)
    h_in, d_in = host_case(cfg, dev)
    shape = m.make_shape(1, 8, 2, 257, 5, 128, "bf16")
    out = torch.empty_like(d_in["q"])
    st = m.moda_causal_fwd(shape, m._ptr(d_in["q"]), m._ptr(d_in["k"]), m._ptr(d_in["v"]),
                           m._ptr(out), None, m._stream_ptr(out))
    assert st == m.MODA_OK
    torch.cuda.synchronize()
    ref, _ = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"])
    assert max_err(out_to_f64(out), ref) <= BF16_TOL


def test_deterministic(m, dev):
    cfg = shape_cfg(2, 8, 2, 777, 9, seed=13)
    _, d_in = host_case(cfg, dev)
    o1, l1 = run_full(m, d_in, 9)
    o2, l2 = run_full(m, d_in, 9)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_all_ones_values(m, dev):
    """Weights sum to one: V = Vd = 1 gives O = 1 (within bf16 rounding)."""
    cfg = shape_cfg(1, 8, 2, 300, 6, seed=17)
    _, d_in = host_case(cfg, dev)
    d_in["v"].fill_(1.0)
    d_in["vd"].fill_(1.0)
    out, _ = run_full(m, d_in, 6)
    assert float((out.float() - 1.0).abs().max()) <= BF16_TOL


def test_depth_permutation(m, dev):
    cfg = shape_cfg(1, 8, 2, 150, 7, seed=19)
    _, d_in = host_case(cfg, dev)
    o1, _ = run_full(m, d_in, 7)
    perm = torch.randperm(7, generator=torch.Generator().manual_seed(3)).to(dev)
    d_in["kd"] = d_in["kd"][:, :, :, perm].contiguous()
    d_in["vd"] = d_in["vd"][:, :, :, perm].contiguous()
    o2, _ = run_full(m, d_in, 7)
    assert float((o1.float() - o2.float()).abs().max()) <= BF16_TOL


def test_locality_bitwise(m, dev):
    """Row t ignores keys after t and other tokens' depth entries, exactly."""
    cfg = shape_cfg(1, 8, 2, 200, 4, seed=23)
    _, d_in = host_case(cfg, dev)
    o1, l1 = run_full(m, d_in, 4)
    t = 97
    d_in["k"][:, :, t + 1:] += 3.0
    d_in["v"][:, :, t + 1:] -= 2.0
    keep_kd, keep_vd = d_in["kd"][:, :, t].clone(), d_in["vd"][:, :, t].clone()
    d_in["kd"].mul_(-1.5)
    d_in["vd"].add_(4.0)
    d_in["kd"][:, :, t] = keep_kd
    d_in["vd"][:, :, t] = keep_vd
    o2, l2 = run_full(m, d_in, 4)
    assert torch.equal(o1[:, :, t], o2[:, :, t]) and torch.equal(l1[:, :, t], l2[:, :, t])


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 32)])
def test_guard_bands(m, dev, dt, d):
    """Every output row is written and nothing outside the output is touched."""
    cfg = shape_cfg(1, 4, 2, 131, 3, d=d, dtype=dt, seed=29)
    _, d_in = host_case(cfg, dev)
    n = d_in["q"].numel()
    pad = 1024
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=d_in["q"].dtype, device=dev)
    out = buf[pad:pad + n].view_as(d_in["q"])
    lbuf = torch.full((4 * 131 + 2 * 64,), float("nan"), dtype=torch.float32, device=dev)
    lse = lbuf[64:64 + 4 * 131].view(1, 4, 131)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"])
    m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, 3, out=out, lse=lse, with_lse=True)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()
    assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[pad + n:]).all()
    assert torch.isnan(lbuf[:64]).all() and torch.isnan(lbuf[64 + 4 * 131:]).all()


def unpack_mfma(packed, B, Hkv, T, L):
    """Decode the bf16/d=128 packed layout on the host (uint16 bit patterns)
    into natural order [B*Hkv, Tp, Lp, 128], Tp = T rounded up to 8 tokens and
    Lp = L rounded up to 4 entries (the padding must be zero).  The layout, per
    (b, kv head): blocks of 8 tokens x 4 entries, block tg * ceil(L/4) + eg of
    16 KiB (K half, then V half); block row r is token
    8tg + ((r & 3) | ((r >> 3) & 1) << 2), entry 4eg + 2(r >> 4) + ((r >> 2) & 1).
    K half: lane l of k-step ks holds row l % 32, dims 64(l/32) + 8ks .. +7.
    V half: lane l of (nb, kk) holds dim 32nb + l % 32 of rows
    16kk + 8(j/4) + 4(l/32) + j%4, j = 0..7."""
    BH, ng, ne = B * Hkv, -(-T // 8), -(-L // 4)
    nblk = ng * ne
    P = to_np(packed).view(np.uint16).reshape(BH, nblk, 2, 4096)
    K = P[:, :, 0].reshape(BH, nblk, 8, 2, 32, 8)        # ks, lh, row, j
    K = K.transpose(0, 1, 4, 3, 2, 5).reshape(BH, nblk, 32, 128)
    V = P[:, :, 1].reshape(BH, nblk, 4, 2, 2, 32, 2, 4)  # nb, kk, lh, li, ja, jc
    V = V.transpose(0, 1, 3, 6, 4, 7, 2, 5).reshape(BH, nblk, 32, 128)  # row = (kk, ja, lh, jc)
    r = np.arange(32)
    tok = (r & 3) | (((r >> 3) & 1) << 2)
    ent = 2 * (r >> 4) + ((r >> 2) & 1)
    out = []
    for X in (K, V):
        X = X.reshape(BH, ng, ne, 32, 128)
        N = np.zeros((BH, ng, 8, ne, 4, 128), np.uint16)
        N[:, :, tok, :, ent] = X.transpose(3, 0, 1, 2, 4)  # row r -> (token, entry)
        out.append(N.reshape(BH, ng * 8, ne * 4, 128))
    return out


def check_unpacked(K, V, kd, vd, T, L):
    """Decoded cache equals the natural tensors, and every padding row is zero."""
    BH = K.shape[0]
    assert np.array_equal(K[:, :T, :L], kd.reshape(BH, T, L, 128))
    assert np.array_equal(V[:, :T, :L], vd.reshape(BH, T, L, 128))
    for X in (K, V):
        assert not X[:, T:].any() and not X[:, :, L:].any()


@pytest.mark.parametrize("T,L", [(37, 3), (64, 32), (5, 1), (100, 24), (9, 5), (16, 4)])
def test_repack_round_trip(m, dev, T, L):
    cfg = shape_cfg(2, 4, 2, T, L, seed=31 + T)
    h_in, d_in = host_case(cfg, dev)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"])
    torch.cuda.synchronize()
    K, V = unpack_mfma(packed, 2, 2, T, L)
    check_unpacked(K, V, h_in["kd"], h_in["vd"], T, L)


def test_generic_repack_round_trip(m, dev):
    cfg = shape_cfg(1, 2, 1, 19, 3, d=32, dtype="f32", seed=37)
    h_in, d_in = host_case(cfg, dev)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"])
    torch.cuda.synchronize()
    raw = to_np(packed).view(np.float32)
    n = h_in["kd"].size
    assert np.array_equal(raw[:n], h_in["kd"].ravel()) and np.array_equal(raw[n:], h_in["vd"].ravel())


def test_runs_on_nondefault_stream(m, dev):
    cfg = shape_cfg(1, 8, 2, 333, 5, seed=41)
    h_in, d_in = host_case(cfg, dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = m.moda_forward(d_in["q"], d_in["k"], d_in["v"], d_in["kd"], d_in["vd"],
                                  with_lse=True)
    s.synchronize()
    ref, _ = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"], h_in["kd"], h_in["vd"])
    assert max_err(out_to_f64(out), ref) <= BF16_TOL


# ------------------------------------------------------------------ backward

BWD_SHAPES = [  # (B, Hq, Hkv, T, L): G = 1, 2, 3, 4, 8, 32, 64; ragged T
    (1, 4, 4, 70, 0), (1, 8, 2, 130, 0), (2, 16, 4, 257, 0), (1, 8, 1, 100, 0), (1, 6, 2, 65, 0),
    (1, 2, 2, 1, 0), (1, 64, 1, 150, 0),
    (1, 4, 4, 70, 5), (1, 8, 2, 130, 24), (1, 8, 1, 100, 33), (1, 6, 2, 65, 3), (2, 16, 4, 96, 1),
    (1, 32, 1, 40, 2), (1, 2, 2, 1, 7),
]
BWD_TOL = 2e-2  # max-abs error relative to max(1, max |reference|) of each gradient


def bwd_check(m, dev, B, Hq, Hkv, T, L, seed, split=True):
    from synth import f32_to_bf16_bits
    from gpu_util import to_dev
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=seed)
    h_in, d_in = host_case(cfg, dev)
    rng = np.random.default_rng(seed + 1)
    h_do = f32_to_bf16_bits(rng.standard_normal((B, Hq, T, 128)).astype(np.float32))
    d_do = to_dev(h_do, "bf16", dev)
    kd, vd = (d_in["kd"], d_in["vd"]) if L else (None, None)
    packed = m.pack_depth_cache(kd, vd, m.make_shape(B, Hq, Hkv, T, L, 128, "bf16")) if L else None
    out, lse = m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, with_lse=True)
    grads = m.bwd(d_in["q"], d_in["k"], d_in["v"], out, lse, d_do, kd, vd, packed, split=split)
    torch.cuda.synchronize()
    ref = oracle.moda_backward(h_in["q"], h_in["k"], h_in["v"], h_in["kd"] if L else None,
                               h_in["vd"] if L else None, h_do)
    for name, g, r in zip(("dq", "dk", "dv", "dkd", "dvd"), grads, ref):
        if r is None:
            continue
        scale = max(1.0, float(np.max(np.abs(r))))
        e = max_err(out_to_f64(g), r)
        print(f"[parity] bwd {B,Hq,Hkv,T,L} {name} max|err|={e:.3e} max|ref|={scale:.3e}",
              flush=True)
        assert e <= BWD_TOL * scale, f"{name}: {e} > {BWD_TOL} * {scale}"
    return grads


@pytest.mark.parametrize("B,Hq,Hkv,T,L", BWD_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in BWD_SHAPES])
def test_bwd_parity(m, dev, B, Hq, Hkv, T, L):
    """moda_bwd against the oracle's backward, every element of every gradient."""
    bwd_check(m, dev, B, Hq, Hkv, T, L, seed=300 + T + 7 * Hq)


SPLIT_SHAPES = [(2, 16, 4, 257, 0), (1, 8, 2, 130, 24), (1, 16, 2, 700, 8)]


@pytest.mark.parametrize("B,Hq,Hkv,T,L", SPLIT_SHAPES,
                         ids=[f"B{b}Hq{hq}Hkv{hk}T{t}L{l}" for b, hq, hk, t, l in SPLIT_SHAPES])
def test_bwd_split_and_unsplit(m, dev, B, Hq, Hkv, T, L):
    """Shapes whose dK/dV work moda_bwd_ws splits over several workgroups: the
    unsplit moda_bwd against the oracle too, and the two within two bf16 ulps
    of each other, floored at 2^-12 of the gradient's largest entry (they differ
    only in the order fp32 terms are summed)."""
    shape = m.make_shape(B, Hq, Hkv, T, L, 128, "bf16")
    assert m.moda_bwd_workspace_bytes(shape) > 0
    seed = 300 + T + 7 * Hq
    g_split = bwd_check(m, dev, B, Hq, Hkv, T, L, seed, split=True)
    g_plain = bwd_check(m, dev, B, Hq, Hkv, T, L, seed, split=False)
    for name, a, b in zip(("dq", "dk", "dv", "dkd", "dvd"), g_split, g_plain):
        if a is None:
            continue
        a, b = out_to_f64(a), out_to_f64(b)
        # two bf16 ulps, with a floor for entries near zero (where summation
        # order moves the result by much more than its own ulp)
        bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -12 * np.max(np.abs(a))
        assert np.all(np.abs(a - b) <= bound), f"{name}: split and unsplit differ"


def bwd_sampled_check(m, cfg, dev, n_rows=16, n_tokens=4, n_end=3):
    """The backward at a full workload size, launched as the bench times it.

    Against the oracle's row-restricted backward: sampled dQ rows, every depth
    entry of sampled tokens (dKd, dVd: all G rows of the token), and dK, dV of
    the last n_end keys of one (b, kv head) (every row that reads them).  Over
    all keys, the identity each row's weights (summing to one) give: per
    (b, kv head) and dim, sum dV + sum dVd = sum of the group's dO rows.  (The
    matching identity for keys, sum dK + sum dKd = 0, has no tolerance that
    the device can compute and that is tight enough to catch a missing term,
    so dK of the bulk of the keys is covered element by element at the 1.5B
    layer's full size instead.)
    """
    import math
    from gpu_util import to_np
    from synth import bf16_bits_to_f32
    B, Hq, Hkv, T, L, d = (cfg[x] for x in ("B", "Hq", "Hkv", "T", "L", "d"))
    G = Hq // Hkv
    s = 1.0 / math.sqrt(d)
    d_in = device_case(cfg, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg["seed"] + 77)
    dout = torch.randn((B, Hq, T, d), generator=gen, device=dev).to(torch.bfloat16)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"], m.make_shape(B, Hq, Hkv, T, L, d, "bf16"))
    out, lse = m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, with_lse=True)
    dq, dk, dv, dkd, dvd = m.bwd(d_in["q"], d_in["k"], d_in["v"], out, lse, dout, d_in["kd"],
                                 d_in["vd"], packed)
    torch.cuda.synchronize()
    del out, lse, packed

    rng = np.random.default_rng(cfg["seed"] + 78)
    qrows = {(int(rng.integers(B)), int(rng.integers(Hq)), int(t))
             for t in rng.integers(0, T, n_rows)} | {(0, 0, 0), (B - 1, Hq - 1, T - 1)}
    toks = {(int(rng.integers(B)), int(rng.integers(Hkv)), int(t))
            for t in rng.integers(0, T, n_tokens)} | {(0, 0, 0), (B - 1, Hkv - 1, T - 1)}
    eb, eg = int(rng.integers(B)), int(rng.integers(Hkv))
    need = set(qrows) | {(b, g * G + j, t) for b, g, t in toks for j in range(G)}
    need |= {(eb, eg * G + j, t) for t in range(T - n_end, T) for j in range(G)}
    rows = np.array(sorted(need), np.int64)
    at = {tuple(r): i for i, r in enumerate(rows.tolist())}
    rt = torch.from_numpy(rows).to(dev)
    bi, hi, ti = rt[:, 0], rt[:, 1], rt[:, 2]
    q_rows, do_rows = to_np(d_in["q"][bi, hi, ti]), to_np(dout[bi, hi, ti])
    rdq, p, ds = oracle.moda_backward_rows(
        rows, (B, Hq, Hkv, T, L, d), q_rows, do_rows, to_np(d_in["k"]), to_np(d_in["v"]),
        to_np(d_in["kd"][bi, hi // G, ti]), to_np(d_in["vd"][bi, hi // G, ti]))
    qf = bf16_bits_to_f32(q_rows).astype(np.float64)
    df = bf16_bits_to_f32(do_rows).astype(np.float64)

    def check(name, got, ref):
        scale = max(1.0, float(np.max(np.abs(ref))))
        e = max_err(got, ref)
        print(f"[parity] bwd {cfg.get('name', '')} {name} max|err|={e:.3e} max|ref|={scale:.3e}",
              flush=True)
        assert e <= BWD_TOL * scale, f"{name}: {e} > {BWD_TOL} * {scale}"

    sel = [at[r] for r in sorted(qrows)]
    qr = torch.from_numpy(rows[sel]).to(dev)
    check(f"dq ({len(sel)} rows)", out_to_f64(dq[qr[:, 0], qr[:, 1], qr[:, 2]]), rdq[sel])
    got_kd, got_vd, ref_kd, ref_vd = [], [], [], []
    for b, g, t in sorted(toks):
        rs = [at[(b, g * G + j, t)] for j in range(G)]
        ref_kd.append(sum(s * ds[r, t + 1:t + 1 + L, None] * qf[r] for r in rs))
        ref_vd.append(sum(p[r, t + 1:t + 1 + L, None] * df[r] for r in rs))
        got_kd.append(out_to_f64(dkd[b, g, t]))
        got_vd.append(out_to_f64(dvd[b, g, t]))
    check(f"dkd ({len(toks)} tokens)", np.stack(got_kd), np.stack(ref_kd))
    check(f"dvd ({len(toks)} tokens)", np.stack(got_vd), np.stack(ref_vd))
    ref_k, ref_v = [], []
    for j in range(T - n_end, T):
        rs = [at[(eb, eg * G + h, t)] for t in range(j, T) for h in range(G)]
        ref_k.append(sum(s * ds[r, j] * qf[r] for r in rs))
        ref_v.append(sum(p[r, j] * df[r] for r in rs))
    check(f"dk (last {n_end} keys)", out_to_f64(dk[eb, eg, T - n_end:]), np.stack(ref_k))
    check(f"dv (last {n_end} keys)", out_to_f64(dv[eb, eg, T - n_end:]), np.stack(ref_v))

    # The identity over all keys, per (b, kv head) and dim, in fp64 on the
    # device.  Each term carries independent round-to-nearest-even errors, so
    # the sum's error is a random walk; the tolerance is 10 standard
    # deviations, from root-sums-of-squares: each row's weights are rounded
    # (2^-9 relative: their sum, 1, errs by at most 2^-9, times dO_t) and every
    # stored dV, dVd by 2^-9.
    f = lambda x: x.double()
    rss = lambda x, dims: x.square().sum(dims).sqrt()
    do_g = f(dout).view(B, Hkv, G, T, d)
    gv, gvd = f(dv), f(dvd)
    err_v = (gv.sum(2) + gvd.sum((2, 3)) - do_g.sum((2, 3))).abs()
    sig_v = 2.0 ** -9 * (rss(do_g, (2, 3)) + rss(gv, 2) + rss(gvd, (2, 3)))
    r_v = float((err_v / (10 * sig_v)).max())
    # what the check would read if the depth entries' dV were missing
    miss_v = float(((gv.sum(2) - do_g.sum((2, 3))).abs() / (10 * sig_v)).max())
    print(f"[parity] bwd {cfg.get('name', '')} sum dV + sum dVd vs sum dO: error / 10 sigma "
          f"{r_v:.3f} (without the depth terms: {miss_v:.1f})", flush=True)
    assert r_v <= 1.0
    del d_in, dout, dq, dk, dv, dkd, dvd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["long_64k", "depth_heavy"])
def test_bwd_full_size_sampled(m, dev, name):
    """The backward at the 64K-token and depth-heavy workloads (sampled outputs
    against the oracle's row-restricted backward, identities over all keys)."""
    bwd_sampled_check(m, dict(WORKLOADS[name], name=name), dev)


def test_bwd_near_size_limit_sampled(m, dev):
    """The backward with T*L just under its 2^23 limit (T = 65536, L = 127,
    G = 4): every flat depth-entry offset and per-head extent at its largest,
    sampled against the oracle as above."""
    cfg = dict(B=1, Hq=4, Hkv=1, T=65536, L=127, d=128, dtype="bf16", scale=1.0, seed=6000,
               name="T65536_L127")
    assert cfg["T"] * cfg["L"] < 1 << 23
    bwd_sampled_check(m, cfg, dev)


def test_bwd_layer_1p5b_full(m, dev):
    """B2 Hq16 Hkv4 T4096 d128 L24 (bf16 N(0,1)*0.5 inputs, N(0,1) dO): every
    element of every gradient against the oracle's backward."""
    from synth import f32_to_bf16_bits
    from gpu_util import to_dev
    cfg = WORKLOADS["layer_1p5b"]
    d_in = device_case(cfg, dev)
    B, Hq, Hkv, T, L = (cfg[x] for x in ("B", "Hq", "Hkv", "T", "L"))
    h_do = f32_to_bf16_bits(np.random.default_rng(2024).standard_normal((B, Hq, T, 128))
                            .astype(np.float32))
    d_do = to_dev(h_do, "bf16", dev)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"], m.make_shape(B, Hq, Hkv, T, L, 128, "bf16"))
    out, lse = m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, with_lse=True)
    grads = m.bwd(d_in["q"], d_in["k"], d_in["v"], out, lse, d_do, d_in["kd"], d_in["vd"], packed)
    torch.cuda.synchronize()
    ref = oracle.moda_backward(*(to_np(d_in[n]) for n in ("q", "k", "v", "kd", "vd")), h_do)
    for name, g, r in zip(("dq", "dk", "dv", "dkd", "dvd"), grads, ref):
        scale = max(1.0, float(np.max(np.abs(r))))
        e = max_err(out_to_f64(g), r)
        print(f"[parity] bwd layer_1p5b {name} max|err|={e:.3e} max|ref|={scale:.3e}", flush=True)
        assert e <= BWD_TOL * scale


# ------------------------------------------------------------------ decode step

DECODE_SHAPES = [  # (B, Hq, Hkv, T, L): T = cache length with the new token; ragged, G 1..32
    (1, 2, 1, 1, 0), (1, 4, 4, 1, 3), (2, 8, 2, 37, 5), (3, 8, 8, 1000, 1), (1, 32, 1, 300, 24),
    (2, 12, 4, 2050, 33), (1, 2, 1, 513, 128), (1, 16, 4, 4096, 24), (1, 8, 2, 9000, 0),
    (2, 4, 1, 257, 65),
]


def decode_case(cfg, dev):
    """Decode inputs cut from a forward case: the last token's query and depth
    rows, the whole K/V as the cache."""
    d_in = device_case(cfg, dev)
    T, L = cfg["T"], cfg["L"]
    q = d_in["q"][:, :, T - 1].contiguous()
    kd = d_in["kd"][:, :, T - 1].contiguous() if L else None
    vd = d_in["vd"][:, :, T - 1].contiguous() if L else None
    return d_in, q, kd, vd


def decode_check(m, cfg, dev):
    d_in, q, kd, vd = decode_case(cfg, dev)
    out, lse = m.decode(q, d_in["k"], d_in["v"], kd, vd, with_lse=True)
    torch.cuda.synchronize()
    B, Hq, T = cfg["B"], cfg["Hq"], cfg["T"]
    rows = np.array([(b, h, T - 1) for b in range(B) for h in range(Hq)], np.int64)
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    e_o = max_err(out_to_f64(out).reshape(B * Hq, -1), ref)
    e_l = max_err(lse.cpu().numpy().reshape(-1), rlse)
    print(f"[decode] {cfg.get('name', cfg)} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    return d_in, q, kd, vd, out, lse


@pytest.mark.parametrize("B,Hq,Hkv,T,L", DECODE_SHAPES,
                         ids=[f"B{b}_Hq{h}_Hkv{k}_T{t}_L{l}" for b, h, k, t, l in DECODE_SHAPES])
def test_decode_parity(m, dev, B, Hq, Hkv, T, L):
    """The decode step against the oracle's row t = T-1 of every (b, head)."""
    decode_check(m, shape_cfg(B, Hq, Hkv, T, L, seed=B * 1000 + T + L), dev)


@pytest.mark.parametrize("name", ["long_64k", "depth_heavy"])
def test_decode_full_size(m, dev, name):
    """Decode over the full-size caches (64K entries; 8K entries x 32 heads)."""
    decode_check(m, dict(WORKLOADS[name], name=name), dev)
    torch.cuda.empty_cache()


def test_decode_matches_forward_last_row(m, dev):
    """Decode equals the forward's last query row up to summation order."""
    cfg = shape_cfg(2, 16, 4, 3000, 24, scale=0.5, seed=77)
    d_in, q, kd, vd, out, lse = decode_check(m, cfg, dev)
    f_out, f_lse = run_full(m, d_in, cfg["L"])
    e_o = (out.float() - f_out[:, :, -1].float()).abs().max().item()
    e_l = (lse - f_lse[:, :, -1]).abs().max().item()
    print(f"[decode] vs forward last row max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


def test_decode_workspace_reuse(m, dev):
    """One workspace serves calls of different shapes in a row; its contents
    from an earlier call never leak into a later result."""
    big = shape_cfg(1, 16, 4, 5000, 24, seed=91)
    small = shape_cfg(1, 8, 2, 700, 3, seed=92)
    sb = m.make_shape(1, 16, 4, 5000, 24, 128, "bf16")
    ws = torch.full((m.moda_decode_workspace_bytes(sb),), 0x7F, dtype=torch.uint8, device=dev)
    for cfg in (big, small, big):
        d_in, q, kd, vd = decode_case(cfg, dev)
        ref_out = m.decode(q, d_in["k"], d_in["v"], kd, vd)
        out = m.decode(q, d_in["k"], d_in["v"], kd, vd, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)


@pytest.mark.parametrize("B,Hq,Hkv,T,L", [(5, 16, 4, 3000, 5), (3, 8, 8, 700, 0), (2, 32, 1, 5000, 24),
                                          (4, 6, 2, 129, 128)],
                         ids=["B5_G4_L5", "B3_G1_L0", "B2_G32_L24", "B4_G3_L128"])
def test_decode_varlen_parity(m, dev, B, Hq, Hkv, T, L):
    """Sequences of different cache lengths in one call (T is the capacity):
    row (b, h) against the oracle's row t = len_b - 1.  The slots past each
    length hold NaN and are never read."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=1500 + T + L)
    d_in = device_case(cfg, dev)
    rng = np.random.default_rng(T + L)
    lens = np.concatenate([[1, T], rng.integers(1, T + 1, size=B)])[:B].astype(np.int32)
    k, v = d_in["k"].clone(), d_in["v"].clone()
    for b in range(B):
        k[b, :, int(lens[b]):] = float("nan")
        v[b, :, int(lens[b]):] = float("nan")
    bi = torch.arange(B, device=dev)
    tl = torch.from_numpy(lens.astype(np.int64) - 1).to(dev)
    q = d_in["q"][bi, :, tl].contiguous()                               # [B, Hq, d]
    kd = d_in["kd"][bi, :, tl].contiguous() if L else None              # [B, Hkv, L, d]
    vd = d_in["vd"][bi, :, tl].contiguous() if L else None
    out, lse = m.decode(q, k, v, kd, vd, with_lse=True,
                        cache_lens=torch.from_numpy(lens).to(dev))
    torch.cuda.synchronize()
    rows = np.array([(b, h, int(lens[b]) - 1) for b in range(B) for h in range(Hq)], np.int64)
    ref, rlse = oracle_rows_from_device(cfg, d_in, rows)
    e_o = max_err(out_to_f64(out).reshape(B * Hq, -1), ref)
    e_l = max_err(lse.cpu().numpy().reshape(-1), rlse)
    print(f"[decode varlen] lens={lens.tolist()} max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}", flush=True)
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16


def test_decode_varlen_edges(m, dev):
    """Length 0 leaves the depth entries alone (depth attention over the L
    entries); length 0 with L = 0 gives O = 0 and LSE = -inf; lengths all equal
    to T give moda_decode's result bit for bit."""
    B, Hq, Hkv, T, L = 3, 8, 2, 400, 6
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=1601)
    d_in, q, kd, vd = decode_case(cfg, dev)
    full = torch.full((B,), T, dtype=torch.int32, device=dev)
    o_full = m.decode(q, d_in["k"], d_in["v"], kd, vd, cache_lens=full)
    o_ref = m.decode(q, d_in["k"], d_in["v"], kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o_full, o_ref)
    zero = torch.tensor([0, T, 0], dtype=torch.int32, device=dev)
    out, lse = m.decode(q, d_in["k"], d_in["v"], kd, vd, with_lse=True, cache_lens=zero)
    torch.cuda.synchronize()
    G = Hq // Hkv
    q1 = to_np(q[0::2].unsqueeze(2))                                  # rows of b = 0, 2 as T = 1
    kd1 = to_np(kd[0::2].unsqueeze(2))
    vd1 = to_np(vd[0::2].unsqueeze(2))
    ref, rlse = oracle.depth_forward(q1, kd1, vd1)
    e_o = max_err(out_to_f64(out[0::2]), ref[:, :, 0])
    e_l = max_err(lse[0::2].cpu().numpy(), rlse[:, :, 0])
    assert e_o <= BF16_TOL and e_l <= LSE_TOL_BF16
    assert torch.equal(out[1], o_ref[1])
    out0, lse0 = m.decode(q, d_in["k"], d_in["v"], with_lse=True, cache_lens=zero)
    torch.cuda.synchronize()
    assert not out0[0::2].float().abs().any() and torch.isneginf(lse0[0::2]).all()
    assert torch.isfinite(lse0[1]).all()


def test_decode_per_token_loop_is_the_forward(m, dev):
    """Decoding every token in turn (cache length t+1 within the full cache,
    the token's own depth entries) gives the forward's rows: each against the
    full fp64 oracle."""
    B, Hq, Hkv, T, L = 2, 8, 2, 70, 5
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=1701)
    h_in, d_in = host_case(cfg, dev)
    out = torch.empty_like(d_in["q"])
    for t in range(T):
        lens = torch.full((B,), t + 1, dtype=torch.int32, device=dev)
        out[:, :, t] = m.decode(d_in["q"][:, :, t].contiguous(), d_in["k"], d_in["v"],
                                d_in["kd"][:, :, t].contiguous(), d_in["vd"][:, :, t].contiguous(),
                                cache_lens=lens)
    torch.cuda.synchronize()
    ref, _ = oracle.moda_forward(h_in["q"], h_in["k"], h_in["v"], h_in["kd"], h_in["vd"])
    e_o = max_err(out_to_f64(out), ref)
    print(f"[decode loop] T={T} max|dO|={e_o:.3e}", flush=True)
    assert e_o <= BF16_TOL


def test_decode_graph_replay(m, dev):
    """The decode step captured in a HIP graph: every replay, with eager work
    and synchronisations between them, equals the eager result bit for bit."""
    cfg = shape_cfg(2, 16, 4, 6000, 24, seed=93)
    d_in, q, kd, vd = decode_case(cfg, dev)
    sb = m.make_shape(2, 16, 4, 6000, 24, 128, "bf16")
    ws = torch.empty(m.moda_decode_workspace_bytes(sb), dtype=torch.uint8, device=dev)
    ref = m.decode(q, d_in["k"], d_in["v"], kd, vd, workspace=ws)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.decode(q, d_in["k"], d_in["v"], kd, vd, out=out, workspace=ws)
    for i in range(4):
        out.zero_()
        ws.fill_(0x55)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("B,Hq,Hkv,T,L,d,dt", [(1, 16, 4, 3000, 24, 128, "bf16"),
                                               (1, 8, 2, 700, 5, 64, "f32")],
                         ids=["bf16d128", "f32d64"])
def test_forward_graph_replay(m, dev, B, Hq, Hkv, T, L, d, dt):
    """The depth-cache repack and the forward captured in one HIP graph: every
    replay, with eager work and synchronisations between replays, equals the
    eager result bit for bit (O and LSE)."""
    cfg = shape_cfg(B, Hq, Hkv, T, L, d=d, dtype=dt, seed=95 + T)
    _, d_in = host_case(cfg, dev)
    shape = m.make_shape(B, Hq, Hkv, T, L, d, dt)
    packed = m.pack_depth_cache(d_in["kd"], d_in["vd"], shape)
    ref, rlse = m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, with_lse=True)
    out = torch.empty_like(ref)
    lse = torch.empty_like(rlse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.pack_depth_cache(d_in["kd"], d_in["vd"], shape, out=packed)
        m.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, out=out, lse=lse)
    for i in range(3):
        out.zero_()
        lse.fill_(7.0)
        packed.fill_(0x33)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, rlse), f"replay {i} differs"


# ------------------------------------------------------------------ depth-stream write

APPEND_SHAPES = [  # (B, Hkv, T, L, group sizes n of the writes, in order of entries)
    (2, 2, 37, 3, (1, 1, 1)), (1, 4, 100, 24, (2,) * 12), (2, 1, 5, 1, (1,)),
    (1, 2, 64, 32, (1, 2, 3, 26)), (3, 2, 33, 7, (2, 1, 2, 2)), (1, 1, 1000, 128, (2,) * 64),
]


def write_order(groups, seed):
    """The groups' entry ranges [first, first + n), in a seeded random order."""
    firsts = np.cumsum((0,) + tuple(groups))[:-1]
    order = np.random.default_rng(seed).permutation(len(groups))
    return [(int(firsts[i]), int(groups[i])) for i in order]


@pytest.mark.parametrize("B,Hkv,T,L,groups", APPEND_SHAPES,
                         ids=[f"B{b}_Hkv{h}_T{t}_L{l}_w{len(g)}" for b, h, t, l, g in APPEND_SHAPES])
def test_append_builds_the_cache(m, dev, B, Hkv, T, L, groups):
    """Writing every entry into a zero-filled cache, in any order and group
    size, gives the packed layout of the natural depth tensor: decoded on the
    host it is that tensor bit for bit, with zero padding, and it equals
    moda_pack_depth_cache's bytes."""
    cfg = shape_cfg(B, 2 * Hkv, Hkv, T, L, seed=500 + T + L)
    h_in, d_in = host_case(cfg, dev)
    shape = m.make_shape(B, 2 * Hkv, Hkv, T, L, 128, "bf16")
    cache = torch.zeros(m.moda_depth_cache_bytes(shape), dtype=torch.uint8, device=dev)
    for first, n in write_order(groups, seed=T):
        m.append_depth(cache, shape, first, d_in["kd"][:, :, :, first:first + n].contiguous(),
                       d_in["vd"][:, :, :, first:first + n].contiguous())
    ref = m.pack_depth_cache(d_in["kd"], d_in["vd"], shape)
    torch.cuda.synchronize()
    K, V = unpack_mfma(cache, B, Hkv, T, L)
    check_unpacked(K, V, h_in["kd"], h_in["vd"], T, L)
    assert torch.equal(cache, ref)


def test_append_near_size_limit(m, dev):
    """T*L just under its 2^23 limit (T = 65536, L = 127): writing the last
    entry of every token into a cache packed without it gives the repack of
    the whole stream byte for byte (compared on the device)."""
    B, Hkv, T, L = 1, 1, 65536, 127
    cfg = dict(B=B, Hq=4, Hkv=Hkv, T=T, L=L, d=128, dtype="bf16", scale=1.0, seed=6200)
    d_in = device_case(cfg, dev)
    shape = m.make_shape(B, 4, Hkv, T, L, 128, "bf16")
    kd0, vd0 = d_in["kd"].clone(), d_in["vd"].clone()
    kd0[:, :, :, L - 1] = 0
    vd0[:, :, :, L - 1] = 0
    cache = m.pack_depth_cache(kd0, vd0, shape)
    del kd0, vd0
    m.append_depth(cache, shape, L - 1, d_in["kd"][:, :, :, L - 1:].contiguous(),
                   d_in["vd"][:, :, :, L - 1:].contiguous())
    ref = m.pack_depth_cache(d_in["kd"], d_in["vd"], shape)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref)
    del d_in, cache, ref
    torch.cuda.empty_cache()


def test_append_replaces_one_entry(m, dev):
    """Writing entry i over a packed cache changes exactly entry i of every
    token: the forward on it equals the forward on a fresh repack of the
    natural tensor with that entry replaced, bit for bit."""
    B, Hq, Hkv, T, L, i = 1, 8, 2, 300, 6, 4
    cfg = shape_cfg(B, Hq, Hkv, T, L, seed=611)
    d_in = device_case(cfg, dev)
    shape = m.make_shape(B, Hq, Hkv, T, L, 128, "bf16")
    cache = m.pack_depth_cache(d_in["kd"], d_in["vd"], shape)
    g = torch.Generator(device=dev)
    g.manual_seed(612)
    k_new = torch.randn(B, Hkv, T, 128, generator=g, device=dev).to(torch.bfloat16)
    v_new = torch.randn(B, Hkv, T, 128, generator=g, device=dev).to(torch.bfloat16)
    m.append_depth(cache, shape, i, k_new, v_new)
    kd2, vd2 = d_in["kd"].clone(), d_in["vd"].clone()
    kd2[:, :, :, i], vd2[:, :, :, i] = k_new, v_new
    ref = m.pack_depth_cache(kd2, vd2, shape)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref)
    o1 = m.fwd(d_in["q"], d_in["k"], d_in["v"], cache, L)
    o2 = m.fwd(d_in["q"], d_in["k"], d_in["v"], ref, L)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("d,dt", [(32, "f32"), (64, "bf16"), (128, "f32")])
def test_append_generic_layout(m, dev, d, dt):
    """The generic layout (natural Kd then natural Vd): writes of every entry
    into a zero-filled cache reproduce the natural tensors bit for bit."""
    B, Hkv, T, L = 2, 2, 19, 5
    cfg = shape_cfg(B, 2 * Hkv, Hkv, T, L, d=d, dtype=dt, seed=700 + d)
    h_in, d_in = host_case(cfg, dev)
    shape = m.make_shape(B, 2 * Hkv, Hkv, T, L, d, dt)
    cache = torch.zeros(m.moda_depth_cache_bytes(shape), dtype=torch.uint8, device=dev)
    for first, n in write_order((2, 1, 2), seed=d):
        m.append_depth(cache, shape, first, d_in["kd"][:, :, :, first:first + n].contiguous(),
                       d_in["vd"][:, :, :, first:first + n].contiguous())
    torch.cuda.synchronize()
    raw = to_np(cache).view(h_in["kd"].dtype)
    n = h_in["kd"].size
    assert np.array_equal(raw[:n], h_in["kd"].ravel()) and np.array_equal(raw[n:], h_in["vd"].ravel())
