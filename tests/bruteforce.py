"""Second, independent MoDA formulation: concatenate-then-softmax, NumPy fp64.

Test helper only.  Where the C oracle walks one query row at a time over an
explicit score list, this builds whole score matrices: sequence scores
s*Q K^T with -inf above the diagonal, depth scores s*<q_t, Kd_{t,i}>, one
softmax over their concatenation along the key axis, then P_seq V + P_dep Vd.
Same definition (hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths
Attention (MoDA)": sequence and own-token depth entries under one joint
normalisation), different arithmetic order and language.
"""
import numpy as np


def moda_bruteforce(q, k, v, kd=None, vd=None):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    ke = np.repeat(k, G, axis=1)
    ve = np.repeat(v, G, axis=1)
    s = 1.0 / np.sqrt(d)
    seq = s * np.matmul(q, np.swapaxes(ke, -1, -2))           # [B,Hq,T,T]
    future = np.triu(np.ones((T, T), bool), k=1)
    seq = np.where(future, -np.inf, seq)
    if kd is not None and kd.shape[3] > 0:
        kde = np.repeat(np.asarray(kd, np.float64), G, axis=1)
        vde = np.repeat(np.asarray(vd, np.float64), G, axis=1)
        dep = s * np.einsum("bhtd,bhtld->bhtl", q, kde)
        scores = np.concatenate([seq, dep], axis=-1)
    else:
        scores = seq
    m = scores.max(axis=-1, keepdims=True)
    w = np.exp(scores - m)
    Z = w.sum(axis=-1, keepdims=True)
    p = w / Z
    out = np.matmul(p[..., :T], ve)
    if scores.shape[-1] > T:
        out = out + np.einsum("bhtl,bhtld->bhtd", p[..., T:], vde)
    lse = (m + np.log(Z))[..., 0]
    return out, lse


def depth_bruteforce(q, kd, vd):
    """Depth attention alone in matrix form (NumPy fp64): scores
    s*<q_t, Kd_{t,i}> over the L entries of token t, softmax along i, then the
    weighted sum of Vd_{t,i}.  Same definition as the oracle's depth
    attention (hyper.ai page on arXiv 2603.15619, section "Depth stream
    mechanism"), written with einsum over whole tensors."""
    q = np.asarray(q, np.float64)
    B, Hq, T, d = q.shape
    G = Hq // kd.shape[1]
    kde = np.repeat(np.asarray(kd, np.float64), G, axis=1)
    vde = np.repeat(np.asarray(vd, np.float64), G, axis=1)
    sc = np.einsum("bhtd,bhtld->bhtl", q, kde) / np.sqrt(d)
    m = sc.max(axis=-1, keepdims=True)
    w = np.exp(sc - m)
    Z = w.sum(axis=-1, keepdims=True)
    out = np.einsum("bhtl,bhtld->bhtd", w / Z, vde)
    return out, (m + np.log(Z))[..., 0]
