"""Pins for the fp64 MoDA oracle: facts fixed by the pages and by mathematics.

Each pin takes the loaded oracle library (so the same battery can run against
deliberately broken copies of the oracle, see test_oracle_mutants.py) and
raises AssertionError when the fact does not hold.

Sources of the facts:
  * hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths Attention
    (MoDA)": each token attends to the sequence entries and to its own depth
    entries, jointly normalised.  -> pins b, c, f, h, i, k
  * same page, section "Depth stream mechanism": the depth set is a set of
    per-token entries {K_i, V_i}, i < l (order carries no meaning in a softmax
    over a set).  -> pin d
  * same page, section "Hardware-efficient implementation": G is the GQA
    group count; query heads of a group read one KV head.  -> pin j
  * the causal sequence part alone is ordinary causal attention, a library
    routine.  -> pin a
  * a second formulation in another language (tests/bruteforce.py).  -> pin e
  * same page, section "Depth stream mechanism": depth attention alone reads
    the token's own depth entries under one softmax.  -> pins o to s (the
    oracle's standalone depth attention)
  * the backward is calculus on the forward: central finite differences of
    the (pinned) forward oracle and PyTorch autograd through an independent
    fp64 formulation.  -> pins t to w
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from bruteforce import depth_bruteforce, moda_bruteforce
from synth import bf16_bits_to_f32, f32_to_bf16_bits

TOL = 1e-12


def _case(B, Hq, Hkv, T, L, d, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    kd = rng.standard_normal((B, Hkv, T, L, d))
    vd = rng.standard_normal((B, Hkv, T, L, d))
    return q, k, v, kd, vd


def _fwd(lib, q, k, v, kd, vd):
    if kd is not None and kd.shape[3] == 0:
        kd = vd = None
    return oracle.moda_forward(q, k, v, kd, vd, lib=lib)


def _close(a, b, tol=TOL, what=""):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


def pin_a_causal_limit(lib):
    """L = 0: MoDA is causal GQA attention (torch SDPA, fp64, CPU)."""
    import torch
    import torch.nn.functional as F
    for (B, Hq, Hkv, T, d, seed) in [(1, 2, 1, 7, 8, 1), (2, 4, 2, 13, 16, 2),
                                     (1, 8, 1, 5, 3, 3), (1, 4, 4, 33, 32, 4)]:
        q, k, v, _, _ = _case(B, Hq, Hkv, T, 0, d, seed)
        out, lse = _fwd(lib, q, k, v, None, None)
        G = Hq // Hkv
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk.repeat_interleave(G, 1),
                                             tv.repeat_interleave(G, 1), is_causal=True)
        _close(out, ref.numpy(), what=f"L=0 vs SDPA {B,Hq,Hkv,T,d}")
        # LSE of a causal row: log-sum-exp of the scaled scores (scipy routine)
        from scipy.special import logsumexp
        s = np.matmul(q, np.swapaxes(np.repeat(k, G, 1), -1, -2)) / math.sqrt(d)
        s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
        _close(lse, logsumexp(s, axis=-1), what="L=0 lse")


def pin_b_single_token(lib):
    """T = 1: the one query sees key 0 and its L depth entries -> depth
    attention over L+1 per-token entries (closed form, plain Python)."""
    # hand case: d=1, L=1, q=1, K0=0, V0=0, Kd=c, Vd=w  ->  O = w e^c / (1 + e^c)
    c, w = 0.7, -1.3
    q = np.array([[[[1.0]]]]); k = np.array([[[[0.0]]]]); v = np.array([[[[0.0]]]])
    kd = np.array([[[[[c]]]]]); vd = np.array([[[[[w]]]]])
    out, lse = _fwd(lib, q, k, v, kd, vd)
    _close(out[0, 0, 0, 0], w * math.exp(c) / (1.0 + math.exp(c)), what="hand T=1")
    _close(lse[0, 0, 0], math.log(1.0 + math.exp(c)), what="hand T=1 lse")
    # general T=1: softmax over the stack [K0, Kd_0..Kd_{L-1}] per query head
    B, Hq, Hkv, L, d = 2, 4, 2, 5, 4
    q, k, v, kd, vd = _case(B, Hq, Hkv, 1, L, d, 11)
    out, _ = _fwd(lib, q, k, v, kd, vd)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            keys = [k[b, g, 0]] + [kd[b, g, 0, i] for i in range(L)]
            vals = [v[b, g, 0]] + [vd[b, g, 0, i] for i in range(L)]
            logit = [sum(float(a) * float(bb) for a, bb in zip(q[b, h, 0], kk)) / math.sqrt(d)
                     for kk in keys]
            mx = max(logit)
            e = [math.exp(x - mx) for x in logit]
            Z = sum(e)
            expect = [sum(e[n] * float(vals[n][c]) for n in range(L + 1)) / Z for c in range(d)]
            _close(out[b, h, 0], expect, what=f"T=1 row b={b} h={h}")


def pin_c_weights_sum_to_one(lib):
    """Joint normalisation: the explicit weights of every row sum to 1, are
    non-negative and cover t+1 sequence plus L depth entries."""
    B, Hq, Hkv, T, L, d = 1, 4, 2, 9, 3, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 21)
    full, _ = _fwd(lib, q, k, v, kd, vd)
    G = Hq // Hkv
    for (b, h, t) in [(0, 0, 0), (0, 1, 4), (0, 3, 8), (0, 2, 5)]:
        p, o = oracle.moda_row_weights(q, k, v, kd, vd, b, h, t, lib=lib)
        assert p.shape == (t + 1 + L,)
        assert np.all(p >= 0.0), "negative weight"
        assert abs(p.sum() - 1.0) <= TOL, f"weights sum {p.sum()!r}"
        # the weights are the ones the output is built from, for this row
        vals = np.concatenate([v[b, h // G, :t + 1], vd[b, h // G, t]], axis=0)
        _close(p @ vals, o, what="weights vs output")
        _close(o, full[b, h, t], what="weights entry vs full forward")
    # GPU-style form of the same fact: all values equal to one -> output one
    v1, vd1 = np.ones_like(v), np.ones_like(vd)
    out, _ = _fwd(lib, q, k, v1, kd, vd1)
    _close(out, np.ones_like(out), what="all-ones V")


def pin_d_depth_permutation(lib):
    """Depth entries form a set: permuting them jointly changes nothing."""
    B, Hq, Hkv, T, L, d = 1, 4, 1, 11, 7, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 31)
    perm = np.random.default_rng(5).permutation(L)
    out1, lse1 = _fwd(lib, q, k, v, kd, vd)
    out2, lse2 = _fwd(lib, q, k, v, kd[:, :, :, perm], vd[:, :, :, perm])
    _close(out1, out2, what="depth permutation")
    _close(lse1, lse2, what="depth permutation lse")
    # a permutation that is not joint (keys only) must change the result
    out3, _ = _fwd(lib, q, k, v, kd[:, :, :, perm], vd)
    assert np.max(np.abs(out3 - out1)) > 1e-6, "keys and values of depth are not paired"


def pin_e_bruteforce(lib):
    """Concatenate-then-softmax matrix form (NumPy) agrees to 1e-12."""
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 2, 1, 17, 3, 8, 41), (2, 4, 4, 9, 1, 1, 42),
                                        (1, 8, 2, 13, 5, 32, 43), (1, 8, 1, 6, 24, 8, 44),
                                        (1, 2, 2, 1, 2, 3, 45), (1, 4, 2, 20, 0, 8, 46)]:
        q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, seed)
        out, lse = _fwd(lib, q, k, v, kd, vd)
        ref, rlse = moda_bruteforce(q, k, v, kd if L else None, vd if L else None)
        _close(out, ref, what=f"bruteforce {B,Hq,Hkv,T,L,d}")
        _close(lse, rlse, what=f"bruteforce lse {B,Hq,Hkv,T,L,d}")


def pin_f_split_merge(lib):
    """One softmax over the union equals the log-sum-exp merge of the two
    partial softmaxes (sequence-only and depth-only)."""
    B, Hq, Hkv, T, L, d = 1, 4, 2, 12, 6, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 51)
    out, lse = _fwd(lib, q, k, v, kd, vd)
    o_s, l_s = _fwd(lib, q, k, v, None, None)
    G = Hq // Hkv
    kde, vde = np.repeat(kd, G, 1), np.repeat(vd, G, 1)
    sd = np.einsum("bhtd,bhtld->bhtl", q, kde) / math.sqrt(d)
    md = sd.max(-1, keepdims=True)
    wd = np.exp(sd - md)
    o_d = np.einsum("bhtl,bhtld->bhtd", wd / wd.sum(-1, keepdims=True), vde)
    l_d = (md + np.log(wd.sum(-1, keepdims=True)))[..., 0]
    mm = np.maximum(l_s, l_d)
    a, c = np.exp(l_s - mm), np.exp(l_d - mm)
    merged = (a[..., None] * o_s + c[..., None] * o_d) / (a + c)[..., None]
    _close(out, merged, what="split-merge")
    _close(lse, mm + np.log(a + c), what="split-merge lse")


def pin_g_constant_values(lib):
    """Every value row (sequence and depth) of a KV head equal to c -> O = c."""
    B, Hq, Hkv, T, L, d = 2, 4, 2, 10, 3, 5
    q, k, _, kd, _ = _case(B, Hq, Hkv, T, L, d, 61)
    c = np.random.default_rng(62).standard_normal((B, Hkv, d))
    v = np.broadcast_to(c[:, :, None, :], (B, Hkv, T, d)).copy()
    vd = np.broadcast_to(c[:, :, None, None, :], (B, Hkv, T, L, d)).copy()
    out, _ = _fwd(lib, q, k, v, kd, vd)
    G = Hq // Hkv
    expect = np.broadcast_to(np.repeat(c, G, 1)[:, :, None, :], out.shape)
    _close(out, expect, what="constant V")


def pin_h_zero_query(lib):
    """Q = 0: all logits 0, uniform weights over the t+1+L entries."""
    B, Hq, Hkv, T, L, d = 1, 2, 1, 8, 4, 6
    _, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 71)
    q = np.zeros((B, Hq, T, d))
    out, lse = _fwd(lib, q, k, v, kd, vd)
    for t in range(T):
        expect = (v[0, 0, :t + 1].sum(0) + vd[0, 0, t].sum(0)) / (t + 1 + L)
        _close(out[0, 0, t], expect, what=f"zero Q t={t}")
        _close(out[0, 1, t], expect, what=f"zero Q t={t} h=1")
        _close(lse[0, :, t], [math.log(t + 1 + L)] * 2, what="zero Q lse")


def pin_i_locality(lib):
    """Row t reads only keys 0..t and token t's own depth entries."""
    B, Hq, Hkv, T, L, d = 1, 2, 1, 9, 3, 4
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 81)
    out, _ = _fwd(lib, q, k, v, kd, vd)
    t = 4
    k2, v2, kd2, vd2 = k.copy(), v.copy(), kd.copy(), vd.copy()
    k2[:, :, t + 1:] += 3.0
    v2[:, :, t + 1:] -= 2.0
    for tp in range(T):
        if tp != t:
            kd2[:, :, tp] *= -1.5
            vd2[:, :, tp] += 4.0
    out2, _ = _fwd(lib, q, k2, v2, kd2, vd2)
    assert np.array_equal(out[:, :, t], out2[:, :, t]), "row depends on other tokens"
    # and it does depend on its own depth entries and on key t
    kd3 = kd.copy(); kd3[:, :, t] += 1.0
    out3, _ = _fwd(lib, q, k, v, kd3, vd)
    assert np.max(np.abs(out3[:, :, t] - out[:, :, t])) > 1e-6, "own depth ignored"
    k4 = k.copy(); k4[:, :, t] += 1.0
    out4, _ = _fwd(lib, q, k4, v, kd, vd)
    assert np.max(np.abs(out4[:, :, t] - out[:, :, t])) > 1e-6, "diagonal key ignored"


def pin_j_gqa_expansion(lib):
    """GQA equals multi-head attention on KV (and depth) repeated G times."""
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 4, 2, 7, 3, 8, 91), (2, 8, 2, 5, 2, 4, 92)]:
        q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, seed)
        G = Hq // Hkv
        out, lse = _fwd(lib, q, k, v, kd, vd)
        out2, lse2 = _fwd(lib, q, *(np.repeat(x, G, 1) for x in (k, v, kd, vd)))
        _close(out, out2, tol=1e-15, what="GQA expansion")
        _close(lse, lse2, tol=1e-15, what="GQA expansion lse")


def pin_k_dominance(lib):
    """A depth key aligned with the query and far larger than every other
    logit takes all the weight: O_t -> Vd[t, i*]."""
    B, Hq, Hkv, T, L, d = 1, 1, 1, 6, 4, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 101)
    istar = 2
    kd = kd.copy()
    lam = 400.0 / np.maximum((q[0, 0] ** 2).sum(-1), 1e-3)  # logit ~ 400/sqrt(d)
    kd[0, 0, :, istar] = lam[:, None] * q[0, 0]
    out, lse = _fwd(lib, q, k, v, kd, vd)
    _close(out[0, 0], vd[0, 0, :, istar], tol=1e-12, what="dominance")


def pin_l_input_decoding(lib):
    """fp32 and bf16 inputs are read exactly: same result as the oracle on
    the fp64 values of the same numbers, bit for bit."""
    B, Hq, Hkv, T, L, d = 1, 2, 1, 6, 2, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 111)
    f32 = [x.astype(np.float32) for x in (q, k, v, kd, vd)]
    o32, _ = _fwd(lib, *f32)
    o64, _ = _fwd(lib, *(x.astype(np.float64) for x in f32))
    assert np.array_equal(o32, o64), "fp32 input decoding"
    b16 = [f32_to_bf16_bits(x) for x in f32]
    ob, _ = _fwd(lib, *b16)
    ob64, _ = _fwd(lib, *(bf16_bits_to_f32(x).astype(np.float64) for x in b16))
    assert np.array_equal(ob, ob64), "bf16 input decoding"
    # bf16 bits: 0x3F80 is 1.0, 0xC040 is -3.0 (IEEE binary32 upper halves)
    assert bf16_bits_to_f32(np.array([0x3F80, 0xC040], np.uint16)).tolist() == [1.0, -3.0]


def pin_m_hand_example(lib):
    """A worked example by hand (d=2, T=2, L=1, one head), closed form.

    row 0: logits s*[<q0,K0>, <q0,Kd0>] = s*[2, 0]
    row 1: logits s*[<q1,K0>, <q1,K1>, <q1,Kd1>] = s*[1, 2, 2]
    """
    q = np.array([[2.0, 0.0], [1.0, 1.0]])[None, None]
    k = np.array([[1.0, 0.0], [0.0, 2.0]])[None, None]
    v = np.array([[1.0, 2.0], [3.0, 4.0]])[None, None]
    kd = np.array([[[0.0, 1.0]], [[1.0, 1.0]]])[None, None]
    vd = np.array([[[5.0, 6.0]], [[7.0, 8.0]]])[None, None]
    out, lse = _fwd(lib, q, k, v, kd, vd)
    s = 1.0 / math.sqrt(2.0)
    e2, e1 = math.exp(2 * s), math.exp(s)
    o0 = [(e2 * 1 + 5) / (e2 + 1), (e2 * 2 + 6) / (e2 + 1)]
    Z1 = e1 + 2 * e2
    o1 = [(e1 * 1 + e2 * 3 + e2 * 7) / Z1, (e1 * 2 + e2 * 4 + e2 * 8) / Z1]
    _close(out[0, 0], [o0, o1], what="hand example")
    _close(lse[0, 0], [math.log(e2 + 1), math.log(Z1)], what="hand example lse")


def pin_n_rows_entry(lib):
    """The selected-rows entry point returns exactly the full forward's rows."""
    B, Hq, Hkv, T, L, d = 2, 4, 2, 10, 3, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 121)
    out, lse = _fwd(lib, q, k, v, kd, vd)
    rows = np.array([[0, 0, 0], [1, 3, 9], [0, 2, 5], [1, 1, 7]], np.int64)
    G = Hq // Hkv
    qr = np.stack([q[b, h, t] for b, h, t in rows])
    kdr = np.stack([kd[b, h // G, t] for b, h, t in rows])
    vdr = np.stack([vd[b, h // G, t] for b, h, t in rows])
    o2, l2 = oracle.moda_rows(rows, (B, Hq, Hkv, T, L, d), qr, k, v, kdr, vdr, lib=lib)
    for i, (b, h, t) in enumerate(rows):
        assert np.array_equal(o2[i], out[b, h, t]) and l2[i] == lse[b, h, t]


def _depth(lib, q, kd, vd):
    return oracle.depth_forward(q, kd, vd, lib=lib)


def pin_o_depth_hand_example(lib):
    """Depth attention alone, worked by hand (d=1, T=2, L=2, one head).

    token 0: logits [1.5*0.5, 1.5*(-1)] = [0.75, -1.5], values [2, -3]
    token 1: logits [-0.5*2, -0.5*1] = [-1, -0.5], values [1, 4]
    """
    q = np.array([[1.5], [-0.5]])[None, None]
    kd = np.array([[[0.5], [-1.0]], [[2.0], [1.0]]])[None, None]
    vd = np.array([[[2.0], [-3.0]], [[1.0], [4.0]]])[None, None]
    out, lse = _depth(lib, q, kd, vd)
    a, b = math.exp(0.75), math.exp(-1.5)
    c, e = math.exp(-1.0), math.exp(-0.5)
    _close(out[0, 0, :, 0], [(2 * a - 3 * b) / (a + b), (c + 4 * e) / (c + e)],
           what="depth hand example")
    _close(lse[0, 0], [math.log(a + b), math.log(c + e)], what="depth hand example lse")


def pin_p_depth_bruteforce(lib):
    """Depth attention alone against the NumPy matrix form, including GQA,
    one entry, and fp32 / bf16 inputs read exactly."""
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 2, 1, 7, 3, 8, 131), (2, 8, 2, 5, 1, 4, 132),
                                        (1, 4, 4, 3, 17, 16, 133), (1, 6, 3, 9, 5, 32, 134)]:
        q, _, _, kd, vd = _case(B, Hq, Hkv, T, L, d, seed)
        out, lse = _depth(lib, q, kd, vd)
        ref, rlse = depth_bruteforce(q, kd, vd)
        _close(out, ref, what=f"depth bruteforce {B,Hq,Hkv,T,L,d}")
        _close(lse, rlse, what=f"depth bruteforce lse {B,Hq,Hkv,T,L,d}")
    q, _, _, kd, vd = _case(1, 4, 2, 6, 4, 8, 135)
    for enc, dec in ((lambda x: x.astype(np.float32), lambda x: x.astype(np.float64)),
                     (lambda x: f32_to_bf16_bits(x.astype(np.float32)),
                      lambda x: bf16_bits_to_f32(x).astype(np.float64))):
        xs = [enc(x) for x in (q, kd, vd)]
        out, lse = _depth(lib, *xs)
        ref, rlse = depth_bruteforce(*(dec(x) for x in xs))
        _close(out, ref, what="depth bruteforce, narrow inputs")
        _close(lse, rlse, what="depth bruteforce lse, narrow inputs")


def pin_q_depth_merge(lib):
    """MoDA is the log-sum-exp merge of causal attention and depth attention
    alone: ties the standalone depth attention to the MoDA oracle."""
    B, Hq, Hkv, T, L, d = 2, 6, 2, 9, 4, 8
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, 141)
    out, lse = _fwd(lib, q, k, v, kd, vd)
    o_s, l_s = _fwd(lib, q, k, v, None, None)
    o_d, l_d = _depth(lib, q, kd, vd)
    mm = np.maximum(l_s, l_d)
    a, c = np.exp(l_s - mm), np.exp(l_d - mm)
    _close(out, (a[..., None] * o_s + c[..., None] * o_d) / (a + c)[..., None],
           what="causal + depth merge")
    _close(lse, mm + np.log(a + c), what="causal + depth merge lse")


def pin_r_depth_single_entry(lib):
    """With one depth entry its weight is exactly 1: O_t = Vd[t, 0] bit for
    bit, and LSE is that entry's logit."""
    B, Hq, Hkv, T, L, d = 1, 4, 2, 5, 1, 8
    q, _, _, kd, vd = _case(B, Hq, Hkv, T, L, d, 151)
    out, lse = _depth(lib, q, kd, vd)
    G = Hq // Hkv
    assert np.array_equal(out, np.repeat(vd[:, :, :, 0], G, axis=1)), "single depth entry"
    logit = np.einsum("bhtd,bhtd->bht", q, np.repeat(kd[:, :, :, 0], G, axis=1)) / math.sqrt(d)
    _close(lse, logit, what="single depth entry lse")


def pin_s_depth_dominance(lib):
    """A depth key aligned with the query with a logit of 1000 (exp of it
    overflows a double) takes all the weight: O_t = Vd[t, i*]."""
    B, Hq, Hkv, T, L, d = 1, 1, 1, 5, 3, 8
    q, _, _, kd, vd = _case(B, Hq, Hkv, T, L, d, 161)
    kd = kd.copy()
    lam = 1000.0 * math.sqrt(d) / (q[0, 0] ** 2).sum(-1)
    kd[0, 0, :, 1] = lam[:, None] * q[0, 0]
    out, lse = _depth(lib, q, kd, vd)
    _close(out[0, 0], vd[0, 0, :, 1], tol=1e-12, what="depth dominance")
    _close(lse[0, 0], np.full(T, 1000.0), tol=1e-9, what="depth dominance lse")


def _bwd_case(B, Hq, Hkv, T, L, d, seed):
    q, k, v, kd, vd = _case(B, Hq, Hkv, T, L, d, seed)
    dout = np.random.default_rng(seed + 1).standard_normal(q.shape)
    return q, k, v, kd, vd, dout


def _bwd(lib, q, k, v, kd, vd, dout):
    if kd is not None and kd.shape[3] == 0:
        kd = vd = None
    return oracle.moda_backward(q, k, v, kd, vd, dout, lib=lib)


def pin_t_bwd_finite_differences(lib):
    """Each gradient matches the central difference of the forward oracle's
    loss sum(dO * O) along a random direction (step 1e-5: error ~1e-10)."""
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 4, 2, 5, 3, 4, 171), (2, 2, 2, 3, 0, 8, 172),
                                        (1, 4, 1, 1, 4, 3, 173), (1, 8, 2, 6, 2, 5, 174)]:
        q, k, v, kd, vd, dout = _bwd_case(B, Hq, Hkv, T, L, d, seed)
        grads = _bwd(lib, q, k, v, kd, vd, dout)
        xs = [q, k, v, kd, vd]
        rng = np.random.default_rng(seed + 2)

        def loss(args):
            o, _ = _fwd(lib, *args)
            return float((o * dout).sum())

        for i in range(5 if L else 3):
            u = rng.standard_normal(xs[i].shape)
            eps = 1e-5
            xp, xm = list(xs), list(xs)
            xp[i], xm[i] = xs[i] + eps * u, xs[i] - eps * u
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            an = float((grads[i] * u).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), \
                f"finite difference of input {i} {B,Hq,Hkv,T,L,d}: {fd} vs {an}"


def pin_u_bwd_autograd(lib):
    """Gradients agree with PyTorch autograd (fp64, CPU) through the
    concatenate-then-softmax formulation written with torch ops."""
    import torch
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 4, 2, 7, 3, 8, 181), (2, 2, 1, 5, 1, 4, 182),
                                        (1, 2, 2, 6, 0, 8, 183)]:
        q, k, v, kd, vd, dout = _bwd_case(B, Hq, Hkv, T, L, d, seed)
        tq, tk, tv, tkd, tvd = (torch.tensor(x, dtype=torch.float64, requires_grad=True)
                                for x in (q, k, v, kd, vd))
        G = Hq // Hkv
        ke, ve = tk.repeat_interleave(G, 1), tv.repeat_interleave(G, 1)
        sc = torch.matmul(tq, ke.transpose(-1, -2)) / math.sqrt(d)
        sc = sc.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
        if L:
            kde, vde = tkd.repeat_interleave(G, 1), tvd.repeat_interleave(G, 1)
            sd = torch.einsum("bhtd,bhtld->bhtl", tq, kde) / math.sqrt(d)
            p = torch.softmax(torch.cat([sc, sd], -1), -1)
            o = torch.matmul(p[..., :T], ve) + torch.einsum("bhtl,bhtld->bhtd", p[..., T:], vde)
        else:
            o = torch.matmul(torch.softmax(sc, -1), ve)
        (o * torch.tensor(dout)).sum().backward()
        got = _bwd(lib, q, k, v, kd, vd, dout)
        for name, g, t in zip("q k v kd vd".split(), got, (tq, tk, tv, tkd, tvd)):
            if g is None:
                continue
            _close(g, t.grad.numpy(), tol=1e-10, what=f"autograd d{name} {B,Hq,Hkv,T,L,d}")


def pin_v_bwd_zero_upstream(lib):
    """dO = 0 gives exactly zero gradients."""
    q, k, v, kd, vd, dout = _bwd_case(1, 4, 2, 6, 3, 8, 191)
    for g in _bwd(lib, q, k, v, kd, vd, np.zeros_like(dout)):
        assert not np.any(g), "nonzero gradient from a zero upstream gradient"


def pin_w_bwd_input_decoding(lib):
    """fp32 and bf16 inputs (dO included) are read exactly by the backward."""
    q, k, v, kd, vd, dout = _bwd_case(1, 2, 1, 5, 2, 8, 201)
    xs = [x.astype(np.float32) for x in (q, k, v, kd, vd, dout)]
    g32 = _bwd(lib, *xs)
    g64 = _bwd(lib, *(x.astype(np.float64) for x in xs))
    for a, b in zip(g32, g64):
        assert np.array_equal(a, b), "fp32 decoding in the backward"
    xb = [f32_to_bf16_bits(x) for x in xs]
    gb = _bwd(lib, *xb)
    gb64 = _bwd(lib, *(bf16_bits_to_f32(x).astype(np.float64) for x in xb))
    for a, b in zip(gb, gb64):
        assert np.array_equal(a, b), "bf16 decoding in the backward"


def pin_x_bwd_rows_assemble(lib):
    """The row-restricted backward, summed over every row that reads each key
    (p * dO for values, s * ds * q for keys), rebuilds the full backward
    (pinned above by finite differences and autograd), and its dQ rows match."""
    for (B, Hq, Hkv, T, L, d, seed) in [(1, 4, 2, 6, 3, 8, 211), (2, 2, 1, 5, 0, 4, 212),
                                        (1, 6, 2, 4, 2, 5, 213)]:
        q, k, v, kd, vd, dout = _bwd_case(B, Hq, Hkv, T, L, d, seed)
        want = _bwd(lib, q, k, v, kd, vd, dout)
        G = Hq // Hkv
        rows = np.array([(b, h, t) for b in range(B) for h in range(Hq) for t in range(T)],
                        dtype=np.int64)
        bi, hi, ti = rows[:, 0], rows[:, 1], rows[:, 2]
        kd_rows = kd[bi, hi // G, ti] if L else None
        vd_rows = vd[bi, hi // G, ti] if L else None
        dq, p, ds = oracle.moda_backward_rows(rows, (B, Hq, Hkv, T, L, d), q[bi, hi, ti],
                                              dout[bi, hi, ti], k, v, kd_rows, vd_rows, lib=lib)
        s = 1.0 / math.sqrt(d)
        dk, dv = np.zeros_like(k), np.zeros_like(v)
        dkd = np.zeros_like(kd) if L else None
        dvd = np.zeros_like(vd) if L else None
        for r, (b, h, t) in enumerate(rows):
            g = h // G
            assert not np.any(p[r, t + 1 + L:]) and not np.any(ds[r, t + 1 + L:])
            dk[b, g, :t + 1] += s * ds[r, :t + 1, None] * q[b, h, t]
            dv[b, g, :t + 1] += p[r, :t + 1, None] * dout[b, h, t]
            if L:
                dkd[b, g, t] += s * ds[r, t + 1:t + 1 + L, None] * q[b, h, t]
                dvd[b, g, t] += p[r, t + 1:t + 1 + L, None] * dout[b, h, t]
        _close(dq.reshape(B, Hq, T, d), want[0], tol=1e-12, what="rows dq")
        for name, got, ref in zip(("dk", "dv", "dkd", "dvd"), (dk, dv, dkd, dvd), want[1:]):
            if ref is not None:
                _close(got, ref, tol=1e-12, what=f"rows {name} {B,Hq,Hkv,T,L,d}")


PINS = [(name, fn) for name, fn in sorted(globals().items()) if name.startswith("pin_")]
