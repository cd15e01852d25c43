"""ctypes binding of libmoda (include/moda.h): argument marshalling only.

Every step of the MoDA forward runs in libmoda's HIP kernels.  PyTorch only
supplies device memory and the current stream.  The C entry points keep their
names (``moda_fwd`` ...); ``pack_depth_cache``, ``fwd`` and ``causal_fwd`` are
conveniences that allocate outputs with torch and call them.

If libmoda.so is missing or cannot be loaded, importing this module raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# MODA_LIBRARY may point at another build of the same library (e.g. an
# instrumented one); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MODA_LIBRARY") or os.path.join(_HERE, "libmoda.so")

MODA_OK, MODA_ERR_INVALID_ARG, MODA_ERR_UNSUPPORTED, MODA_ERR_HIP = 0, 1, 2, 3
MODA_F32, MODA_BF16 = 0, 1

# every symbol include/moda.h declares
EXPORTS = ("moda_check_shape", "moda_depth_cache_bytes", "moda_pack_depth_cache", "moda_fwd",
           "moda_causal_fwd", "moda_depth_fwd", "moda_fwd_natural", "moda_bwd",
           "moda_bwd_workspace_bytes", "moda_bwd_ws",
           "moda_decode_workspace_bytes", "moda_decode", "moda_append_depth",
           "moda_fwd_layers", "moda_fwd_masked_scan", "moda_decode_varlen",
           "moda_fwd_strided", "moda_decode_noalloc",
           "moda_status_string", "moda_last_error", "moda_fwd_variant")


class ModaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Hq", ctypes.c_int64), ("Hkv", ctypes.c_int64),
                ("T", ctypes.c_int64), ("L", ctypes.c_int64), ("d", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


class ModaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmoda.so not built at {LIB_PATH}; run "
                          "`python -m depth_wise_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sp, vp, sz = ctypes.POINTER(ModaShape), ctypes.c_void_p, ctypes.c_size_t
    lib.moda_check_shape.argtypes = [sp]
    lib.moda_check_shape.restype = ctypes.c_int
    lib.moda_depth_cache_bytes.argtypes = [sp]
    lib.moda_depth_cache_bytes.restype = sz
    lib.moda_pack_depth_cache.argtypes = [sp, vp, vp, vp, sz, vp]
    lib.moda_pack_depth_cache.restype = ctypes.c_int
    lib.moda_fwd.argtypes = [sp, vp, vp, vp, vp, sz, vp, vp, vp]
    lib.moda_fwd.restype = ctypes.c_int
    lib.moda_causal_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp]
    lib.moda_causal_fwd.restype = ctypes.c_int
    lib.moda_depth_fwd.argtypes = [sp, vp, vp, sz, vp, vp, vp]
    lib.moda_depth_fwd.restype = ctypes.c_int
    lib.moda_fwd_natural.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moda_fwd_natural.restype = ctypes.c_int
    lib.moda_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                             vp]
    lib.moda_bwd.restype = ctypes.c_int
    lib.moda_bwd_workspace_bytes.argtypes = [sp]
    lib.moda_bwd_workspace_bytes.restype = sz
    lib.moda_bwd_ws.argtypes = [sp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp,
                                vp, vp, sz, vp]
    lib.moda_bwd_ws.restype = ctypes.c_int
    lib.moda_decode_workspace_bytes.argtypes = [sp]
    lib.moda_decode_workspace_bytes.restype = sz
    lib.moda_decode.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moda_decode.restype = ctypes.c_int
    lib.moda_append_depth.argtypes = [sp, ctypes.c_int64, ctypes.c_int64, vp, vp, vp, sz, vp]
    lib.moda_append_depth.restype = ctypes.c_int
    lib.moda_fwd_layers.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moda_fwd_layers.restype = ctypes.c_int
    lib.moda_decode_varlen.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moda_decode_varlen.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.moda_fwd_strided.argtypes = [sp, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.moda_fwd_strided.restype = ctypes.c_int
    lib.moda_decode_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moda_decode_noalloc.restype = ctypes.c_int
    lib.moda_fwd_masked_scan.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moda_fwd_masked_scan.restype = ctypes.c_int
    lib.moda_status_string.argtypes = [ctypes.c_int]
    lib.moda_status_string.restype = ctypes.c_char_p
    lib.moda_last_error.argtypes = []
    lib.moda_last_error.restype = ctypes.c_char_p
    lib.moda_fwd_variant.argtypes = [sp]
    lib.moda_fwd_variant.restype = ctypes.c_char_p
    return lib


lib = _load()


def make_shape(B, Hq, Hkv, T, L, d, dtype) -> ModaShape:
    code = {"f32": MODA_F32, "bf16": MODA_BF16, MODA_F32: MODA_F32, MODA_BF16: MODA_BF16}
    if not isinstance(dtype, (str, int)):
        dtype = str(dtype).replace("torch.", "")
        dtype = {"float32": "f32", "bfloat16": "bf16"}.get(dtype, dtype)
    return ModaShape(int(B), int(Hq), int(Hkv), int(T), int(L), int(d), code[dtype])


def _check(status: int, where: str):
    if status != MODA_OK:
        detail = lib.moda_last_error().decode() or lib.moda_status_string(status).decode()
        raise ModaError(status, where, detail)


# ---------------------------------------------------------------- C entry points

def _sref(shape):
    return None if shape is None else ctypes.byref(shape)


def moda_check_shape(shape: ModaShape) -> int:
    return lib.moda_check_shape(_sref(shape))


def moda_depth_cache_bytes(shape: ModaShape) -> int:
    return int(lib.moda_depth_cache_bytes(_sref(shape)))


def moda_fwd_variant(shape: ModaShape) -> str:
    return lib.moda_fwd_variant(_sref(shape)).decode()


def moda_pack_depth_cache(shape, k_depth_ptr, v_depth_ptr, packed_ptr, packed_bytes, stream):
    return lib.moda_pack_depth_cache(_sref(shape), k_depth_ptr, v_depth_ptr, packed_ptr,
                                     packed_bytes, stream)


def moda_fwd(shape, q_ptr, k_ptr, v_ptr, packed_ptr, packed_bytes, out_ptr, lse_ptr, stream):
    return lib.moda_fwd(_sref(shape), q_ptr, k_ptr, v_ptr, packed_ptr, packed_bytes,
                        out_ptr, lse_ptr, stream)


def moda_causal_fwd(shape, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, stream):
    return lib.moda_causal_fwd(_sref(shape), q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, stream)


def moda_depth_fwd(shape, q_ptr, packed_ptr, packed_bytes, out_ptr, lse_ptr, stream):
    return lib.moda_depth_fwd(_sref(shape), q_ptr, packed_ptr, packed_bytes, out_ptr, lse_ptr,
                              stream)


def moda_fwd_natural(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr, stream):
    return lib.moda_fwd_natural(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr,
                                lse_ptr, stream)


def moda_bwd(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, packed_ptr, packed_bytes, out_ptr,
             lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr, dkd_ptr, dvd_ptr, delta_ptr, stream):
    return lib.moda_bwd(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, packed_ptr, packed_bytes,
                        out_ptr, lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr, dkd_ptr, dvd_ptr,
                        delta_ptr, stream)


def moda_bwd_workspace_bytes(shape: ModaShape) -> int:
    return int(lib.moda_bwd_workspace_bytes(_sref(shape)))


def moda_bwd_ws(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, packed_ptr, packed_bytes, out_ptr,
                lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr, dkd_ptr, dvd_ptr, delta_ptr, ws_ptr,
                ws_bytes, stream):
    return lib.moda_bwd_ws(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, packed_ptr,
                           packed_bytes, out_ptr, lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr,
                           dkd_ptr, dvd_ptr, delta_ptr, ws_ptr, ws_bytes, stream)


def moda_decode_workspace_bytes(shape: ModaShape) -> int:
    return int(lib.moda_decode_workspace_bytes(_sref(shape)))


def moda_decode(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr, ws_ptr, ws_bytes,
                stream):
    return lib.moda_decode(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr,
                           ws_ptr, ws_bytes, stream)


def moda_append_depth(shape, first, n, k_ptr, v_ptr, packed_ptr, packed_bytes, stream):
    return lib.moda_append_depth(_sref(shape), int(first), int(n), k_ptr, v_ptr, packed_ptr,
                                 packed_bytes, stream)


def moda_fwd_layers(shape, q_ptr, k_ptr, v_ptr, kl_ptr, vl_ptr, out_ptr, lse_ptr, stream):
    return lib.moda_fwd_layers(_sref(shape), q_ptr, k_ptr, v_ptr, kl_ptr, vl_ptr, out_ptr,
                               lse_ptr, stream)


def moda_decode_varlen(shape, lens_ptr, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr,
                       ws_ptr, ws_bytes, stream):
    return lib.moda_decode_varlen(_sref(shape), lens_ptr, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr,
                                  out_ptr, lse_ptr, ws_ptr, ws_bytes, stream)


def moda_decode_noalloc(shape, lens_ptr, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr,
                        stream):
    return lib.moda_decode_noalloc(_sref(shape), lens_ptr, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr,
                                   out_ptr, lse_ptr, stream)


def moda_fwd_strided(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, s_bh, s_t, s_i, out_ptr, lse_ptr,
                     stream):
    return lib.moda_fwd_strided(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, int(s_bh),
                                int(s_t), int(s_i), out_ptr, lse_ptr, stream)


def moda_fwd_masked_scan(shape, q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr, lse_ptr, stream):
    return lib.moda_fwd_masked_scan(_sref(shape), q_ptr, k_ptr, v_ptr, kd_ptr, vd_ptr, out_ptr,
                                    lse_ptr, stream)


def moda_status_string(status: int) -> str:
    return lib.moda_status_string(status).decode()


def moda_last_error() -> str:
    return lib.moda_last_error().decode()


# ---------------------------------------------------------------- torch conveniences

def _stream_ptr(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def shape_of(q, k, kd=None) -> ModaShape:
    B, Hq, T, d = q.shape
    L = 0 if kd is None else kd.shape[3]
    return make_shape(B, Hq, k.shape[1], T, L, d, q.dtype)


def _check_tensors(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libmoda takes device tensors")
        if not t.is_contiguous():
            raise ValueError("libmoda takes contiguous tensors")


def _expect(name, t, shape, dtype=None, device=None):
    """Raise ValueError unless tensor t has exactly this shape (and dtype and
    device, when given).  The C ABI receives bare pointers and cannot check
    these itself: a short or mistyped tensor would be read past its end."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_qkv(q, k, v):
    """q [B,Hq,T,d]; k, v [B,Hkv,T,d] of q's dtype and device.  Returns B, Hq, Hkv, T, d."""
    if q is None or k is None or v is None:
        raise ValueError("q, k and v are required")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D: [B,Hq,T,d] and [B,Hkv,T,d]")
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    _expect("k", k, (B, Hkv, T, d), q.dtype, q.device)
    _expect("v", v, (B, Hkv, T, d), q.dtype, q.device)
    return B, Hq, Hkv, T, d


def _check_out(q, out, lse, lse_shape):
    if out is not None:
        _expect("out", out, q.shape, q.dtype, q.device)
    if lse is not None:
        import torch
        _expect("lse", lse, lse_shape, torch.float32, q.device)


def pack_depth_cache(kd, vd, shape: ModaShape | None = None, out=None):
    """Repack Kd, Vd [B,Hkv,T,L,d] into a new (or given) uint8 device buffer."""
    import torch
    if kd is None or kd.dim() != 5:
        raise ValueError("kd must be 5-D: [B,Hkv,T,L,d]")
    _expect("vd", vd, kd.shape, kd.dtype, kd.device)
    if shape is not None:
        _expect("kd", kd, (shape.B, shape.Hkv, shape.T, shape.L, shape.d))
    _check_tensors(kd, vd)
    if shape is None:
        B, Hkv, T, L, d = kd.shape
        shape = make_shape(B, Hkv, Hkv, T, L, d, kd.dtype)
    n = moda_depth_cache_bytes(shape)
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=kd.device)
    _check(moda_pack_depth_cache(shape, _ptr(kd), _ptr(vd), _ptr(out), out.numel(),
                                 _stream_ptr(kd)), "moda_pack_depth_cache")
    return out


def fwd(q, k, v, packed=None, L: int = 0, *, with_lse: bool = False, out=None, lse=None):
    """MoDA forward.  ``packed`` comes from pack_depth_cache with the same
    shape (the Hq of the pack shape does not matter; only B, Hkv, T, L, d)."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    _check_out(q, out, lse, (B, Hq, T))
    if packed is not None and packed.device != q.device:
        raise ValueError("packed must be on q's device")
    _check_tensors(q, k, v, packed)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    nbytes = 0 if packed is None else packed.numel() * packed.element_size()
    _check(moda_fwd(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(packed), nbytes, _ptr(out), _ptr(lse),
                    _stream_ptr(q)), "moda_fwd")
    return (out, lse) if with_lse else out


def causal_fwd(q, k, v, *, with_lse: bool = False, out=None, lse=None):
    """Causal-only attention (the same kernel without the depth part)."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, k, v)
    shape = make_shape(B, Hq, Hkv, T, 0, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(moda_causal_fwd(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                           _stream_ptr(q)), "moda_causal_fwd")
    return (out, lse) if with_lse else out


def depth_fwd(q, packed, Hkv: int, L: int, *, with_lse: bool = False, out=None, lse=None):
    """Depth attention alone over a packed depth cache (the same packed
    buffer moda_fwd reads; Hkv and L are those of the pack shape)."""
    import torch
    if q is None or q.dim() != 4:
        raise ValueError("q must be 4-D: [B,Hq,T,d]")
    B, Hq, T, d = q.shape
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, packed)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    nbytes = 0 if packed is None else packed.numel() * packed.element_size()
    _check(moda_depth_fwd(shape, _ptr(q), _ptr(packed), nbytes, _ptr(out), _ptr(lse),
                          _stream_ptr(q)), "moda_depth_fwd")
    return (out, lse) if with_lse else out


def depth_forward(q, kd, vd, *, with_lse: bool = False):
    """Pack then depth attention alone."""
    B, Hq, T, d = q.shape
    Hkv, L = kd.shape[1], kd.shape[3]
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    packed = pack_depth_cache(kd, vd, shape)
    return depth_fwd(q, packed, Hkv, L, with_lse=with_lse)


def fwd_natural(q, k, v, kd=None, vd=None, *, with_lse: bool = False, out=None, lse=None):
    """MoDA forward straight from the natural depth layout (no repack)."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    L = 0 if kd is None else kd.shape[3]
    if kd is not None:
        _expect("kd", kd, (B, Hkv, T, L, d), q.dtype, q.device)
        _expect("vd", vd, (B, Hkv, T, L, d), q.dtype, q.device)
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, k, v, kd, vd)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(moda_fwd_natural(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kd if L else None),
                            _ptr(vd if L else None), _ptr(out), _ptr(lse), _stream_ptr(q)),
           "moda_fwd_natural")
    return (out, lse) if with_lse else out


def fwd_masked_scan(q, k, v, kd, vd, *, with_lse: bool = False, out=None, lse=None):
    """Layout ablation: moda_fwd_natural's result, with every query tile
    scanning the flattened depth axis from entry 0 under the own-token mask."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    if kd is None or kd.dim() != 5:
        raise ValueError("kd must be 5-D: [B,Hkv,T,L,d]")
    L = kd.shape[3]
    _expect("kd", kd, (B, Hkv, T, L, d), q.dtype, q.device)
    _expect("vd", vd, (B, Hkv, T, L, d), q.dtype, q.device)
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, k, v, kd, vd)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(moda_fwd_masked_scan(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kd), _ptr(vd), _ptr(out),
                                _ptr(lse), _stream_ptr(q)), "moda_fwd_masked_scan")
    return (out, lse) if with_lse else out


def fwd_capacity(q, k, v, kd=None, vd=None, L=None, *, with_lse: bool = False, out=None,
                 lse=None):
    """MoDA forward over a natural-layout depth stream with room for more
    entries: kd, vd [B,Hkv,T,Lcap,d], of which the first L (default: all) are
    the depth entries (moda_fwd_strided with strides (T*Lcap, Lcap, 1))."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    Lcap = 0 if kd is None else kd.shape[3]
    L = Lcap if L is None else L
    if kd is not None:
        _expect("kd", kd, (B, Hkv, T, Lcap, d), q.dtype, q.device)
        _expect("vd", vd, (B, Hkv, T, Lcap, d), q.dtype, q.device)
    if not 0 <= L <= Lcap:
        raise ValueError(f"L = {L} must lie in [0, {Lcap}]")
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, k, v, kd, vd)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(moda_fwd_strided(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kd if L else None),
                            _ptr(vd if L else None), T * Lcap, Lcap, 1, _ptr(out), _ptr(lse),
                            _stream_ptr(q)), "moda_fwd_strided")
    return (out, lse) if with_lse else out


def fwd_layers(q, k, v, kl=None, vl=None, L=None, *, with_lse: bool = False, out=None,
               lse=None):
    """MoDA forward over a layer-major depth stream kl, vl [Lcap,B,Hkv,T,d]: the
    first L slices (default: all) are the depth entries."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    if kl is None:
        L = 0
    else:
        Lcap = kl.shape[0]
        _expect("kl", kl, (Lcap, B, Hkv, T, d), q.dtype, q.device)
        _expect("vl", vl, (Lcap, B, Hkv, T, d), q.dtype, q.device)
        L = Lcap if L is None else L
        if not 0 <= L <= Lcap:
            raise ValueError(f"L = {L} must lie in [0, {Lcap}]")
    _check_out(q, out, lse, (B, Hq, T))
    _check_tensors(q, k, v, kl, vl)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(moda_fwd_layers(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kl if L else None),
                           _ptr(vl if L else None), _ptr(out), _ptr(lse), _stream_ptr(q)),
           "moda_fwd_layers")
    return (out, lse) if with_lse else out


def bwd(q, k, v, out, lse, dout, kd=None, vd=None, packed=None, *, grads=None, delta=None,
        workspace=None, split: bool = True):
    """MoDA backward.  ``out`` and ``lse`` come from fwd(..., with_lse=True) on
    the same inputs.  Returns (dq, dk, dv, dkd, dvd); dkd, dvd are None when
    L = 0.  ``grads`` may pass the five output tensors to fill.  With ``split``
    (moda_bwd_ws) a shape whose dK/dV work would not fill the GPU gets its
    split, with ``workspace`` (a uint8 device tensor of at least
    moda_bwd_workspace_bytes bytes) or one allocated here; without it, moda_bwd."""
    import torch
    B, Hq, Hkv, T, d = _check_qkv(q, k, v)
    L = 0 if kd is None else kd.shape[3]
    _expect("out", out, q.shape, q.dtype, q.device)
    _expect("dout", dout, q.shape, q.dtype, q.device)
    _expect("lse", lse, (B, Hq, T), torch.float32, q.device)
    if kd is not None:
        _expect("kd", kd, (B, Hkv, T, L, d), q.dtype, q.device)
        _expect("vd", vd, (B, Hkv, T, L, d), q.dtype, q.device)
    if delta is not None:
        _expect("delta", delta, (B, Hq, T), torch.float32, q.device)
    if grads is not None:
        want = (q.shape, k.shape, v.shape, kd.shape if L else None, vd.shape if L else None)
        for nm, g, w in zip(("dq", "dk", "dv", "dkd", "dvd"), grads, want):
            if w is None:
                if g is not None:
                    raise ValueError(f"{nm} must be None when L = 0")
            else:
                _expect(nm, g, w, q.dtype, q.device)
    _check_tensors(q, k, v, out, lse, dout, kd, vd, packed)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(kd) if L else None, torch.empty_like(vd) if L else None)
    if delta is None:
        delta = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    nbytes = 0 if packed is None else packed.numel() * packed.element_size()
    dq, dk, dv, dkd, dvd = grads
    if not split:
        _check(moda_bwd(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kd), _ptr(vd), _ptr(packed),
                        nbytes, _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(dkd), _ptr(dvd), _ptr(delta), _stream_ptr(q)), "moda_bwd")
        return grads
    need = moda_bwd_workspace_bytes(shape)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(moda_bwd_ws(shape, _ptr(q), _ptr(k), _ptr(v), _ptr(kd), _ptr(vd), _ptr(packed), nbytes,
                       _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkd),
                       _ptr(dvd), _ptr(delta), _ptr(workspace), ws_bytes, _stream_ptr(q)),
           "moda_bwd_ws")
    return grads


def append_depth(packed, shape: ModaShape, first: int, k_new, v_new):
    """Write entries [first, first + n) of every token into ``packed`` in place;
    k_new, v_new [B,Hkv,T,n,d] (a [B,Hkv,T,d] pair is taken as n = 1)."""
    if k_new is None or v_new is None or k_new.dim() not in (4, 5):
        raise ValueError("k_new, v_new must be [B,Hkv,T,d] or [B,Hkv,T,n,d]")
    if k_new.dim() == 4:
        k_new, v_new = k_new.unsqueeze(3), v_new.unsqueeze(3)
    n = k_new.shape[3]
    want = (shape.B, shape.Hkv, shape.T, n, shape.d)
    _expect("k_new", k_new, want)
    _expect("v_new", v_new, want, k_new.dtype, k_new.device)
    if (shape.dtype == MODA_BF16) != (str(k_new.dtype) == "torch.bfloat16"):
        raise ValueError(f"k_new dtype {k_new.dtype} does not match the cache shape's dtype")
    _check_tensors(packed, k_new, v_new)
    _check(moda_append_depth(shape, first, n, _ptr(k_new), _ptr(v_new), _ptr(packed),
                             packed.numel() * packed.element_size(), _stream_ptr(k_new)),
           "moda_append_depth")
    return packed


def decode(q, k, v, kd=None, vd=None, *, with_lse: bool = False, out=None, lse=None,
           workspace=None, cache_lens=None):
    """Decode step: q [B,Hq,d] of the new token over the cache k, v [B,Hkv,T,d]
    (the new token's own K, V last) and its depth entries kd, vd [B,Hkv,L,d].
    ``cache_lens`` (int32 device tensor [B]) gives each sequence's cache length
    (T is then the capacity).  ``workspace`` may pass a uint8 device tensor of
    at least moda_decode_workspace_bytes bytes."""
    import torch
    if q is None or q.dim() != 3 or k is None or k.dim() != 4:
        raise ValueError("q must be [B,Hq,d] and k [B,Hkv,T,d]")
    B, Hq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    _expect("k", k, (B, Hkv, T, d), q.dtype, q.device)
    _expect("v", v, (B, Hkv, T, d), q.dtype, q.device)
    L = 0 if kd is None else kd.shape[2]
    if kd is not None:
        _expect("kd", kd, (B, Hkv, L, d), q.dtype, q.device)
        _expect("vd", vd, (B, Hkv, L, d), q.dtype, q.device)
    _check_out(q, out, lse, (B, Hq))
    _check_tensors(q, k, v, kd, vd, cache_lens)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    need = moda_decode_workspace_bytes(shape)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if with_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(kd if L else None), _ptr(vd if L else None),
            _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_ptr(q))
    if cache_lens is None:
        _check(moda_decode(shape, *args), "moda_decode")
    else:
        if cache_lens.dtype != torch.int32 or cache_lens.numel() != B:
            raise ValueError("cache_lens must be an int32 tensor of B elements")
        _check(moda_decode_varlen(shape, _ptr(cache_lens), *args), "moda_decode_varlen")
    return (out, lse) if with_lse else out


def decode_noalloc(q, k, v, kd=None, vd=None, *, out, lse=None, cache_lens=None):
    """The decode step through moda_decode_noalloc: the library's fixed device
    scratch instead of a workspace.  ``out`` (and ``lse``, if wanted) must be
    given, so that the call allocates nothing."""
    if q is None or q.dim() != 3 or k is None or k.dim() != 4:
        raise ValueError("q must be [B,Hq,d] and k [B,Hkv,T,d]")
    B, Hq, d = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    _expect("k", k, (B, Hkv, T, d), q.dtype, q.device)
    _expect("v", v, (B, Hkv, T, d), q.dtype, q.device)
    L = 0 if kd is None else kd.shape[2]
    if kd is not None:
        _expect("kd", kd, (B, Hkv, L, d), q.dtype, q.device)
        _expect("vd", vd, (B, Hkv, L, d), q.dtype, q.device)
    _check_out(q, out, lse, (B, Hq))
    if out is None:
        raise ValueError("out is required")
    if cache_lens is not None and (str(cache_lens.dtype) != "torch.int32" or
                                   cache_lens.numel() != B):
        raise ValueError("cache_lens must be an int32 tensor of B elements")
    _check_tensors(q, k, v, kd, vd, out, lse, cache_lens)
    shape = make_shape(B, Hq, Hkv, T, L, d, q.dtype)
    _check(moda_decode_noalloc(shape, _ptr(cache_lens), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(kd if L else None), _ptr(vd if L else None), _ptr(out),
                               _ptr(lse), _stream_ptr(q)), "moda_decode_noalloc")
    return out


def moda_forward(q, k, v, kd=None, vd=None, *, with_lse: bool = False):
    """Pack (when L > 0) then forward: the whole MoDA path in two launches."""
    if kd is None or kd.shape[3] == 0:
        return fwd(q, k, v, None, 0, with_lse=with_lse)
    B, Hq, T, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], T, kd.shape[3], d, q.dtype)
    packed = pack_depth_cache(kd, vd, shape)
    return fwd(q, k, v, packed, kd.shape[3], with_lse=with_lse)
