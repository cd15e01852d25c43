"""The C-ABI library loads, exports what include/moda.h declares, and rejects
bad arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moda.h")


@pytest.fixture(scope="module")
def m():
    from depth_wise_kv_amd import moda
    return moda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moda_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(m.lib, n), f"libmoda.so does not export {n}"
    assert sorted(m.EXPORTS) == names


def shape(m, **kw):
    base = dict(B=1, Hq=16, Hkv=4, T=4096, L=24, d=128, dtype="bf16")
    base.update(kw)
    return m.make_shape(**base)


def test_check_shape(m):
    assert m.moda_check_shape(shape(m)) == m.MODA_OK
    assert m.moda_check_shape(shape(m, Hq=15)) == m.MODA_ERR_INVALID_ARG
    assert m.moda_check_shape(shape(m, T=0)) == m.MODA_ERR_INVALID_ARG
    assert m.moda_check_shape(shape(m, L=-1)) == m.MODA_ERR_INVALID_ARG
    assert m.moda_check_shape(shape(m, d=96)) == m.MODA_ERR_UNSUPPORTED
    assert m.moda_check_shape(shape(m, Hq=512, Hkv=1)) == m.MODA_ERR_UNSUPPORTED
    assert m.moda_check_shape(shape(m, T=1 << 40, L=1 << 20)) == m.MODA_ERR_INVALID_ARG
    s = shape(m)
    s.dtype = 7
    assert m.moda_check_shape(s) == m.MODA_ERR_INVALID_ARG
    assert "multiple" in (m.moda_check_shape(shape(m, Hq=15)) and m.moda_last_error())


def test_depth_cache_bytes(m):
    # bf16, d=128: 32-entry blocks of 16 KiB per (b, kv head)
    assert m.moda_depth_cache_bytes(shape(m)) == 4 * (4096 * 24 // 32) * 16384
    assert m.moda_depth_cache_bytes(shape(m, T=5, L=3)) == 4 * 1 * 16384
    assert m.moda_depth_cache_bytes(shape(m, L=0)) == 0
    # same layout whatever G is
    assert m.moda_depth_cache_bytes(shape(m, Hq=4)) == m.moda_depth_cache_bytes(shape(m, Hq=32))
    # generic path: Kd then Vd in natural layout
    assert m.moda_depth_cache_bytes(shape(m, dtype="f32", d=32, T=64, L=4, Hkv=1, Hq=2)) == \
        2 * 64 * 4 * 32 * 4
    assert m.moda_depth_cache_bytes(shape(m, Hq=15)) == 0
    # the key-split form when the 128-row grid fills the chip's 512 slots at most
    # once (B1 Hkv4 T4096 G4: 512 tiles); 4-wave workgroups when the 256-row grid
    # fills it at most twice over
    assert m.moda_fwd_variant(shape(m)) == "mfma_bf16_d128_ks"
    assert m.moda_fwd_variant(shape(m, T=4097)) == "mfma_bf16_d128_w4"
    assert m.moda_fwd_variant(shape(m, B=2)) == "mfma_bf16_d128_w4"
    assert m.moda_fwd_variant(shape(m, T=8192)) == "mfma_bf16_d128_w4"
    assert m.moda_fwd_variant(shape(m, T=8193)) == "mfma_bf16_d128_w8"
    assert m.moda_fwd_variant(shape(m, T=65536)) == "mfma_bf16_d128_w8"
    assert m.moda_fwd_variant(shape(m, Hq=256, Hkv=1)) == "mfma_bf16_d128_w8"   # G > 128
    # the matrix-core kernel for the other head dims and fp32, G <= 128
    assert m.moda_fwd_variant(shape(m, dtype="f32")) == "mfma_f32_d128"
    assert m.moda_fwd_variant(shape(m, dtype="f32", d=64)) == "mfma_f32_d64"
    assert m.moda_fwd_variant(shape(m, dtype="f32", d=32)) == "mfma_f32_d32"
    assert m.moda_fwd_variant(shape(m, d=64)) == "mfma_bf16_d64"
    assert m.moda_fwd_variant(shape(m, d=32)) == "mfma_bf16_d32"
    assert m.moda_fwd_variant(shape(m, d=32, Hq=128, Hkv=1)) == "mfma_bf16_d32"
    # one-wave-per-row VALU kernel above G = 128
    assert m.moda_fwd_variant(shape(m, d=32, Hq=256, Hkv=1)) == "generic"
    assert m.moda_fwd_variant(shape(m, dtype="f32", Hq=256, Hkv=1)) == "generic"


def test_status_strings(m):
    for st, name in [(0, "MODA_OK"), (1, "MODA_ERR_INVALID_ARG"), (2, "MODA_ERR_UNSUPPORTED"),
                     (3, "MODA_ERR_HIP")]:
        assert m.moda_status_string(st) == name


def test_fwd_rejects_before_launch(m):
    """Argument errors return a status without any device call (no GPU here)."""
    s = shape(m)
    p = ctypes.c_void_p(4096)       # never dereferenced: validation fails first
    mis = ctypes.c_void_p(4096 + 8)
    nb = m.moda_depth_cache_bytes(s)
    assert m.moda_fwd(s, None, p, p, p, nb, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd(s, mis, p, p, p, nb, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert "aligned" in m.moda_last_error()
    assert m.moda_fwd(s, p, p, p, None, 0, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd(s, p, p, p, p, nb - 1, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert "too small" in m.moda_last_error()
    s0 = shape(m, L=0)
    assert m.moda_fwd(s0, p, p, p, p, 16, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd(shape(m, d=96), p, p, p, p, nb, p, None, None) == m.MODA_ERR_UNSUPPORTED
    assert m.moda_causal_fwd(s, p, None, p, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_causal_fwd(None, p, p, p, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_pack_depth_cache(s, p, p, p, nb - 16, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_pack_depth_cache(s0, p, p, p, 0, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_pack_depth_cache(s, p, None, p, nb, None) == m.MODA_ERR_INVALID_ARG
    # depth attention alone: needs L >= 1, q, out and a large enough packed cache
    assert m.moda_depth_fwd(s0, p, p, 16, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert "L >= 1" in m.moda_last_error()
    assert m.moda_depth_fwd(s, None, p, nb, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_depth_fwd(s, p, p, nb, None, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_depth_fwd(s, p, None, nb, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_depth_fwd(s, p, p, nb - 1, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_depth_fwd(s, p, p, nb, mis, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_depth_fwd(None, p, p, nb, p, None, None) == m.MODA_ERR_INVALID_ARG


def test_decode_workspace_and_rejects(m):
    """Decode: workspace size is a host-side function of the shape; argument
    errors come back as statuses before any device call."""
    s = shape(m, T=65536, L=32)
    ws = m.moda_decode_workspace_bytes(s)
    rec = 132 * 4  # one record (O, max, sum, padding) per query row and workgroup part
    # parts per (b, kv head): 256 8-wave workgroups in all, but at least 8 blocks of 32
    # entries each; where that fills at most 128 units, 4-wave parts of at least 4 blocks
    # each, up to 512
    assert ws == 16 * 64 * rec
    assert m.moda_decode_workspace_bytes(shape(m, T=65536, L=0)) == 16 * 64 * rec
    # 129 blocks: 16 8-wave parts (64 workgroups), so 32 4-wave parts
    assert m.moda_decode_workspace_bytes(shape(m, T=4096, L=24)) == 16 * 32 * rec
    assert m.moda_decode_workspace_bytes(shape(m, B=64, T=4096)) == 64 * 16 * 1 * rec
    # 13 blocks per (b, kv head), 48 KV heads in all: 1 8-wave part (48 workgroups), so 3 4-wave parts
    assert m.moda_decode_workspace_bytes(shape(m, B=12, T=384)) == 12 * 16 * 3 * rec
    assert m.moda_decode_workspace_bytes(shape(m, T=1, L=0)) == 16 * 1 * rec
    s0 = shape(m, T=65536, L=0)
    assert m.moda_decode_workspace_bytes(shape(m, dtype="f32")) == 0
    assert m.moda_decode_workspace_bytes(shape(m, Hq=64, Hkv=1)) == 0   # G = 64
    assert m.moda_decode_workspace_bytes(shape(m, Hq=32, Hkv=1)) > 0    # G = 32
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    ok = (p, p, p, p, p, p, None, p, ws, None)
    assert m.moda_decode(None, *ok) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(shape(m, dtype="f32"), *ok) == m.MODA_ERR_UNSUPPORTED
    assert m.moda_decode(shape(m, Hq=64, Hkv=1), *ok) == m.MODA_ERR_UNSUPPORTED
    assert m.moda_decode(s, None, p, p, p, p, p, None, p, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s, p, p, p, None, p, p, None, p, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s0, p, p, p, p, p, p, None, p, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s, p, p, p, p, mis, p, None, p, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s, p, p, p, p, p, p, None, None, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s, p, p, p, p, p, p, None, mis, ws, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_decode(s, p, p, p, p, p, p, None, p, ws - 1, None) == m.MODA_ERR_INVALID_ARG
    assert "too small" in m.moda_last_error()
    # the ragged form also needs its length array (device int32, 4-byte aligned)
    odd = ctypes.c_void_p(4096 + 2)
    assert m.moda_decode_varlen(s, None, p, p, p, p, p, p, None, p, ws, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_decode_varlen(s, odd, p, p, p, p, p, p, None, p, ws, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_decode_varlen(s, p, p, p, p, p, p, p, None, p, ws - 1, None) == \
        m.MODA_ERR_INVALID_ARG


def test_bwd_workspace_and_rejects(m):
    """Backward: the dK/dV split's workspace is a host-side function of the
    shape (0 where 128-key workgroups already fill the GPU twice over), and a
    missing or short workspace comes back as a status before any device call."""
    part = 4096 * 128 * 4  # one fp32 partial of one (b, kv head)'s dK or dV at T = 4096
    # 32 key tiles x 4 KV heads = 128 workgroups: 4 parts
    assert m.moda_bwd_workspace_bytes(shape(m, T=4096, L=24)) == 2 * 4 * 4 * part
    # B = 2: 256 workgroups, 2 parts; two KV heads: 64, 8 parts
    assert m.moda_bwd_workspace_bytes(shape(m, B=2, T=4096, L=24)) == 2 * 2 * 8 * part
    assert m.moda_bwd_workspace_bytes(shape(m, Hkv=2, T=4096, L=0)) == 2 * 8 * 2 * part
    # enough workgroups, or too few query tiles to split, or a shape moda_bwd refuses
    assert m.moda_bwd_workspace_bytes(shape(m, T=65536, L=32)) == 0
    assert m.moda_bwd_workspace_bytes(shape(m, T=70, L=5)) == 0
    assert m.moda_bwd_workspace_bytes(shape(m, dtype="f32")) == 0
    assert m.moda_bwd_workspace_bytes(shape(m, Hq=64, Hkv=1, L=24)) == 0
    assert m.moda_bwd_workspace_bytes(None) == 0
    s = shape(m, T=4096, L=24)
    need = m.moda_bwd_workspace_bytes(s)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    args = (p, p, p, p, p, p, 1 << 30, p, p, p, p, p, p, p, p, p)
    assert m.moda_bwd_ws(s, *args, p, need - 1, None) == m.MODA_ERR_INVALID_ARG
    assert "too small" in m.moda_last_error()
    assert m.moda_bwd_ws(s, *args, None, need, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_bwd_ws(s, *args, mis, need, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_bwd_ws(shape(m, dtype="f32"), *args, p, need, None) == m.MODA_ERR_UNSUPPORTED


def test_append_rejects_before_launch(m):
    s = shape(m, T=100, L=24)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    nb = m.moda_depth_cache_bytes(s)
    bad = [(s, -1, 1, p, p, p, nb), (s, 0, 0, p, p, p, nb), (s, 23, 2, p, p, p, nb),
           (s, 24, 1, p, p, p, nb), (s, 0, 1, None, p, p, nb), (s, 0, 1, p, None, p, nb),
           (s, 0, 1, p, p, None, nb), (s, 0, 1, mis, p, p, nb), (s, 0, 1, p, p, p, nb - 1),
           (shape(m, L=0), 0, 1, p, p, p, nb), (None, 0, 1, p, p, p, nb)]
    for args in bad:
        assert m.moda_append_depth(*args, None) == m.MODA_ERR_INVALID_ARG, args
    assert m.moda_append_depth(shape(m, d=96), 0, 1, p, p, p, nb, None) == m.MODA_ERR_UNSUPPORTED


def test_fwd_layers_rejects_before_launch(m):
    s = shape(m, T=100, L=24)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    bad = [(s, None, p, p, p, p, p, None), (s, p, p, p, None, p, p, None),
           (s, p, p, p, p, mis, p, None), (s, p, p, p, p, p, None, None),
           (shape(m, L=0), p, p, p, p, p, p, None), (None, p, p, p, p, p, p, None)]
    for args in bad:
        assert m.moda_fwd_layers(*args, None) == m.MODA_ERR_INVALID_ARG, args
    assert m.moda_fwd_layers(shape(m, dtype="f32"), p, p, p, p, p, p, None, None) == \
        m.MODA_ERR_UNSUPPORTED
    assert m.moda_fwd_layers(shape(m, T=1 << 20, L=8), p, p, p, p, p, p, None, None) == \
        m.MODA_ERR_UNSUPPORTED


def test_fwd_masked_scan_rejects_before_launch(m):
    s = shape(m, T=100, L=24)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    for args in [(s, None, p, p, p, p, p, None), (s, p, p, p, None, p, p, None),
                 (s, p, p, p, p, mis, p, None), (None, p, p, p, p, p, p, None)]:
        assert m.moda_fwd_masked_scan(*args, None) == m.MODA_ERR_INVALID_ARG, args
    for s2 in (shape(m, L=0), shape(m, dtype="f32"), shape(m, T=1 << 20, L=8)):
        assert m.moda_fwd_masked_scan(s2, p, p, p, p, p, p, None, None) == m.MODA_ERR_UNSUPPORTED


def test_fwd_strided_rejects_before_launch(m):
    s = shape(m, T=100, L=24)
    p = ctypes.c_void_p(4096)
    mis = ctypes.c_void_p(4096 + 8)
    ok = (100 * 24, 24, 1)
    assert m.moda_fwd_strided(s, p, p, p, None, p, *ok, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd_strided(s, p, p, p, mis, p, *ok, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd_strided(s, p, p, p, p, p, -1, 24, 1, p, None, None) == m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd_strided(s, p, p, p, p, p, 1 << 60, 24, 1, p, None, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd_strided(shape(m, T=100, L=0), p, p, p, p, p, *ok, p, None, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_fwd_strided(shape(m, dtype="f32"), p, p, p, p, p, *ok, p, None, None) == \
        m.MODA_ERR_UNSUPPORTED
    assert m.moda_fwd_strided(None, p, p, p, p, p, *ok, p, None, None) == m.MODA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors(m):
    import torch
    q = torch.zeros(1, 2, 4, 32)
    with pytest.raises(ValueError):
        m.fwd(q, q[:, :1], q[:, :1])


def test_binding_checks_shapes_and_dtypes(m):
    """The torch conveniences refuse tensors whose shape, dtype or device does
    not match before anything reaches the C ABI, which gets bare pointers and
    could not tell a short or mistyped buffer from a good one."""
    import torch
    bf = torch.bfloat16
    B, Hq, Hkv, T, L, d = 1, 8, 2, 16, 3, 128
    q = torch.zeros(B, Hq, T, d, dtype=bf)
    k = torch.zeros(B, Hkv, T, d, dtype=bf)
    v = torch.zeros(B, Hkv, T, d, dtype=bf)
    kd = torch.zeros(B, Hkv, T, L, d, dtype=bf)
    vd = torch.zeros(B, Hkv, T, L, d, dtype=bf)
    short_v = torch.zeros(B, Hkv, T - 1, d, dtype=bf)
    f32_k = torch.zeros(B, Hkv, T, d, dtype=torch.float32)
    lse = torch.zeros(B, Hq, T, dtype=torch.float32)
    cases = [
        lambda: m.fwd(q, k, short_v),
        lambda: m.fwd(q, f32_k, v),
        lambda: m.fwd(q, k, v, out=torch.zeros(B, Hq, T, 64, dtype=bf)),
        lambda: m.fwd(q, k, v, lse=torch.zeros(B, Hq, T, dtype=bf)),
        lambda: m.causal_fwd(q, k, short_v),
        lambda: m.causal_fwd(q, k[:, :, :, :64].contiguous(), v),
        lambda: m.fwd_natural(q, k, v, kd, vd[:, :, :, :2].contiguous()),
        lambda: m.fwd_natural(q, k, v, kd.float(), vd),
        lambda: m.fwd_masked_scan(q, k, v, kd, None),
        lambda: m.fwd_capacity(q, k, v, kd, vd, L=L + 1),
        lambda: m.fwd_layers(q, k, v, kd.permute(3, 0, 1, 2, 4).contiguous(),
                             vd.permute(3, 0, 1, 2, 4).contiguous()[:2]),
        lambda: m.depth_fwd(q[0], None, Hkv, L),
        lambda: m.bwd(q, k, v, q, lse, short_v),
        lambda: m.bwd(q, k, v, q, lse.to(bf), q),
        lambda: m.bwd(q, k, v, q, lse, q, kd, vd[:, :1].contiguous()),
        lambda: m.bwd(q, k, v, q, lse, q, grads=(q, k, short_v, None, None)),
        lambda: m.pack_depth_cache(kd, vd[:, :, :1].contiguous()),
        lambda: m.pack_depth_cache(kd, vd, m.make_shape(B, Hq, Hkv, T + 1, L, d, "bf16")),
        lambda: m.append_depth(torch.zeros(8, dtype=torch.uint8),
                               m.make_shape(B, Hq, Hkv, T, L, d, "bf16"), 0,
                               k[:, :, :-1].contiguous(), v[:, :, :-1].contiguous()),
        lambda: m.append_depth(torch.zeros(8, dtype=torch.uint8),
                               m.make_shape(B, Hq, Hkv, T, L, d, "f32"), 0, k, v),
        lambda: m.decode(q[:, :, 0], k, short_v),
        lambda: m.decode(q[:, :, 0], k, v, kd[:, :, 0], vd[:, :, 0, :2].contiguous()),
        lambda: m.decode(q[:, :, 0], k, v, out=torch.zeros(B, Hq, 64, dtype=bf)),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(ValueError):
            c()


def test_decode_noalloc_rejects_before_launch(m):
    """moda_decode_noalloc validates on the host like moda_decode, and refuses a
    shape whose partial states outgrow its fixed 8 MiB scratch, before any GPU call."""
    p = ctypes.c_void_p(1 << 20)
    good = m.make_shape(2, 16, 4, 3000, 24, 128, "bf16")
    assert m.moda_decode_noalloc(None, None, p, p, p, p, p, p, None, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_decode_noalloc(good, None, None, p, p, p, p, p, None, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_decode_noalloc(good, None, p, p, p, None, p, p, None, None) == \
        m.MODA_ERR_INVALID_ARG
    assert m.moda_decode_noalloc(good, ctypes.c_void_p((1 << 20) + 2), p, p, p, p, p, p, None,
                                 None) == m.MODA_ERR_INVALID_ARG
    big = m.make_shape(4096, 128, 4, 64, 0, 128, "bf16")
    assert m.moda_decode_workspace_bytes(big) > 8 << 20
    assert m.moda_decode_noalloc(big, None, p, p, p, None, None, p, None, None) == \
        m.MODA_ERR_UNSUPPORTED
    assert "scratch" in m.moda_last_error()
    f32 = m.make_shape(2, 16, 4, 3000, 24, 128, "f32")
    assert m.moda_decode_noalloc(f32, None, p, p, p, p, p, p, None, None) == \
        m.MODA_ERR_UNSUPPORTED


LOG_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
from depth_wise_kv_amd import moda as m
s = m.make_shape(1, 8, 2, 300, 6, 128, "bf16")
p = ctypes.c_void_p(4096)
rc = m.moda_fwd(s, None, p, p, p, m.moda_depth_cache_bytes(s), p, None, None)
err = m.moda_last_error()
assert rc == m.MODA_ERR_INVALID_ARG, rc
rc = m.moda_causal_fwd(None, p, p, p, p, None, None)
assert rc == m.MODA_ERR_INVALID_ARG, rc
print(err)
"""


def run_logged(env_value):
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("MODA_LOG", None)
    if env_value is not None:
        env["MODA_LOG"] = env_value
    p = subprocess.run([sys.executable, "-c", LOG_SCRIPT, ROOT], capture_output=True, text=True,
                       env=env, timeout=120)
    assert p.returncode == 0, p.stderr
    return p.stdout.strip(), [l for l in p.stderr.splitlines() if l.startswith("moda: ")]


def test_dispatch_log():
    """MODA_LOG=1: one stderr line per call that would enqueue work, naming the
    entry point, the shape, the kernel variant and the result; the call's own
    error text stays what moda_last_error() returns.  Unset or "0": silent."""
    err, lines = run_logged("1")
    assert len(lines) == 2, lines
    assert lines[0].startswith("moda: moda_fwd B=1 Hq=8 Hkv=2 T=300 L=6 d=128 bf16 [mfma_bf16_d128_")
    assert lines[0].endswith(": " + err) and err
    assert lines[1] == "moda: moda_causal_fwd (no shape): shape is NULL"
    for v in (None, "0"):
        err2, lines2 = run_logged(v)
        assert lines2 == [] and err2 == err
