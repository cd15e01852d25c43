"""The allocation-free decode (moda_decode_noalloc) against the decode with a
workspace (moda_decode, moda_decode_varlen), through the C ABI, on two calls in
a row, the second with a smaller input: equal bit for bit (same kernels, same
split), which is stronger than the 2e-2 parity bar.  The calls must not
allocate: torch's allocator counts no new allocation across them."""
import numpy as np
import pytest

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


def inputs(B, Hq, Hkv, T, L, seed, dev):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    r = lambda *sh: torch.randn(*sh, generator=g, device=dev).to(torch.bfloat16)
    q, k, v = r(B, Hq, 128), r(B, Hkv, T, 128), r(B, Hkv, T, 128)
    kd, vd = (r(B, Hkv, L, 128), r(B, Hkv, L, 128)) if L else (None, None)
    return q, k, v, kd, vd


def allocations():
    return torch.cuda.memory_stats()["allocation.all.allocated"]


@pytest.mark.parametrize("varlen", [False, True])
def test_decode_noalloc_matches_decode(m, dev, varlen):
    # first call: a larger shape; second: a smaller one (the scratch keeps the
    # first call's partial states, which the second must not read)
    for (B, Hq, Hkv, T, L, seed) in [(3, 32, 8, 5000, 24, 71), (1, 8, 2, 700, 5, 72)]:
        print(f"[noalloc] varlen={varlen} B{B} Hq{Hq} Hkv{Hkv} T{T} L{L}", flush=True)
        q, k, v, kd, vd = inputs(B, Hq, Hkv, T, L, seed, dev)
        lens = (torch.tensor([T - 7 * b for b in range(B)], dtype=torch.int32, device=dev)
                if varlen else None)
        ref, ref_lse = m.decode(q, k, v, kd, vd, with_lse=True, cache_lens=lens)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        before = allocations()
        m.decode_noalloc(q, k, v, kd, vd, out=out, lse=lse, cache_lens=lens)
        torch.cuda.synchronize()
        assert allocations() == before, "the allocation-free decode allocated through torch"
        assert torch.equal(out, ref), "O differs from moda_decode's"
        assert torch.equal(lse, ref_lse), "LSE differs from moda_decode's"
        e = float((out.float() - ref.float()).abs().max())
        assert np.isfinite(e) and e <= 2e-2


def test_decode_noalloc_refuses_big_shape(m, dev):
    B, Hq, Hkv, T = 4096, 128, 4, 64
    shape = m.make_shape(B, Hq, Hkv, T, 0, 128, "bf16")
    assert m.moda_decode_workspace_bytes(shape) > 8 << 20
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(B, Hkv, T, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(m.ModaError):
        m.decode_noalloc(q, k, k, out=torch.empty_like(q))
