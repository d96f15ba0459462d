"""Pins of the fp64 oracle against things other than itself: numbers printed on the pages
(tests/golden, each with its citation), closed forms, textbook special cases, brute force
with pure-Python loops, independent library routines (scipy.special) and the method's
invariants.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle as O
from dit_amd import workloads as WL


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- constants -----------
def test_printed_constants(golden_dir):
    for case in _load(golden_dir, "printed_constants.json")["cases"]:
        L, C, W, gate = O.constants(case["n"])
        assert W == case["W"], case["cite"]
        assert gate == case["gate"], case["cite"]
        if "C" in case:
            assert C == case["C"], case["cite"]


def test_ceil_log2_bruteforce():
    for n in list(range(1, 5000)) + [2**k + d for k in range(13, 40) for d in (-1, 0, 1)]:
        L = 0
        while (1 << L) < n:
            L += 1
        assert O.ceil_log2(n) == L, n
    with pytest.raises(ValueError):
        O.ceil_log2(0)


def test_constants_closed_form():
    for n in [1, 2, 3, 255, 256, 257, 4096, 37800, 75600, 131072, 131073]:
        L, C, W, gate = O.constants(n)
        assert C == 127 - L - 8 and W == C + 125 and gate == W // 2
        # fp32 headroom: N * 2^C * Vmax <= 2^127 < the largest fp32
        assert n * 2.0**C * O.VMAX <= 2.0**127


def test_gate_is_tight_window_sweep():
    """Every U <= gate keeps the worst shifted exponent >= -125, and every U just above
    the gate breaks it ([FM] Summary inequality): floor(W/2) is exactly the largest
    admissible integer bound."""
    for n in [256, 4096, 37800, 75600]:
        L, C, W, gate = O.constants(n)
        for u in np.arange(0.0, gate + 1e-9, 1e-3):
            assert O.window_lower_edge(float(u), C) >= -125.0
        for eps in (1e-6, 1e-3, 0.5, 1.0):
            assert O.window_lower_edge(gate + eps, C) < -125.0


# ---------------------------------------------------------------- soundness cases -----
def test_raw_key_bound_unsound(golden_dir):
    g = _load(golden_dir, "raw_key_unsound.json")
    r = O.raw_key_unsound_case(g["n_keys"], g["key_norm"])
    assert r["raw_u"] == g["raw_bound"] and r["gate"] == g["gate"]
    assert r["raw_passes_gate"]
    assert abs(r["centred_max_logit"] - g["centred_max_logit_approx"]) <= g["centred_max_logit_abs_tol"]
    assert r["max_exponent"] > g["min_shifted_exponent_exceeds"]
    assert r["verdict"] == "rejected"
    # the sound pairing: the bound measured on the centred keys fails the gate
    assert not r["centred_passes_gate"] and r["centred_u"] > g["gate"]


def test_adversarial_query_fails_halved_gate(golden_dir):
    g = _load(golden_dir, "adversarial_gate.json")
    rng = np.random.default_rng(7)
    n, d = g["n_keys"], 16
    keys = rng.standard_normal((n, d))
    keys -= keys.mean(axis=0)
    keys /= np.linalg.norm(keys, axis=1).max()
    scale = 0.25
    alpha = O.alpha_of(scale)
    qdir = rng.standard_normal((8, d))
    q = qdir / np.linalg.norm(qdir, axis=1, keepdims=True) * (g["query_base2_norm"] / alpha)
    b = O.bounds(q[None, :, None, :], [keys[None, :, None, :]], [np.zeros((1, n, 1, d))],
                 scale=scale, q_block=8, center="none", dtype="fp32")
    assert (b.W, b.gate) == (g["W"], g["gate"])
    u = float(b.u[0, 0, 0])
    assert abs(u - g["query_base2_norm"]) < 1e-9
    assert u <= b.W            # would pass a full-W gate
    assert not b.elig[0, 0, 0]  # the halved gate rejects it
    assert int(b.m[0, 0, 0]) == math.ceil(u) - b.C == 125


# ---------------------------------------------------------------- bounds --------------
def _bounds_bruteforce(q, kc, vc, scale, q_block, kbar):
    """Pure-Python loops over the same definition (fsum for the k mean)."""
    B, Sq, H, D = q.shape
    keys = np.concatenate(kc, axis=1)
    N = keys.shape[1]
    out = {}
    for b in range(B):
        for h in range(H):
            k2 = 0.0
            for j in range(N):
                s = 0.0
                for d in range(D):
                    t = float(keys[b, j, h, d]) - float(kbar[b, h, d])
                    s += t * t
                k2 = max(k2, s)
            for beta in range(-(-Sq // q_block)):
                q2 = 0.0
                for i in range(beta * q_block, min((beta + 1) * q_block, Sq)):
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, i, h, d]) ** 2
                    q2 = max(q2, s)
                u = float(np.float32(scale)) * 1.4426950408889634 * math.sqrt(q2 * k2)
                out[(b, h, beta)] = (q2, k2, u)
    return out


@pytest.mark.parametrize("center", ["none", "compute", "supplied"])
def test_bounds_bruteforce(center):
    inp = WL.generic_inputs(11, "bf16", 2, 3, 8, 21, (7, 6), q_block=8, center=center,
                            k_offset=2.0 if center != "none" else 0.0)
    q, kc, vc = inp.q, inp.k, inp.v
    scale = 0.3
    kmean = inp.k_mean if center == "supplied" else None
    b = O.bounds(q, kc, vc, scale=scale, q_block=8, center=center, k_mean=kmean)
    keys = np.concatenate(kc, axis=1).astype(np.float64)
    N = keys.shape[1]
    if center == "compute":
        exact = np.zeros(b.k_mean.shape, dtype=np.float32)
        for bb in range(2):
            for h in range(3):
                for d in range(8):
                    col = [Fraction(float(x)) for x in keys[bb, :, h, d]]
                    exact[bb, h, d] = np.float32(float(sum(col)) / N)
        assert np.array_equal(exact, b.k_mean)
        kbar = exact
    elif center == "supplied":
        kbar = inp.k_mean
        assert np.array_equal(b.k_mean, kbar)
    else:
        kbar = np.zeros((2, 3, 8), np.float32)
        assert not b.k_mean.any()
    ref = _bounds_bruteforce(q, kc, vc, scale, 8, kbar)
    L, C, W, gate = O.constants(N)
    for (bb, h, beta), (q2, k2, u) in ref.items():
        assert b.q2[bb, h, beta] == q2
        assert b.k2[bb, h] == k2
        assert b.u[bb, h, beta] == u
        assert b.m[bb, h, beta] == math.ceil(u) - C
        assert bool(b.elig[bb, h, beta]) == (u <= gate)


@pytest.mark.parametrize("center", ["none", "compute"])
def test_row_bounds_bruteforce(center):
    """Per-row shifts ([CM] "Picking a max that is safe without measuring it": each query
    row's own norm times the largest key norm) against pure-Python loops."""
    inp = WL.generic_inputs(12, "bf16", 1, 2, 8, 19, (9, 5), q_block=8, center=center,
                            k_offset=1.5 if center != "none" else 0.0)
    q, kc, vc = inp.q, inp.k, inp.v
    scale = 0.3
    b = O.bounds(q, kc, vc, scale=scale, q_block=8, center=center, shift="row")
    L, C, W, gate = O.constants(14)
    for h in range(2):
        k2 = b.k2[0, h]
        for i in range(19):
            s = 0.0
            for d in range(8):
                s += float(q[0, i, h, d]) ** 2
            u = float(np.float32(scale)) * 1.4426950408889634 * math.sqrt(s * k2)
            assert b.q2_row[0, h, i] == s
            assert b.u_row[0, h, i] == u
            assert b.m_row[0, h, i] == math.ceil(u) - C


@pytest.mark.parametrize("q_block", [64, 128, 256])
def test_row_shift_max_over_block_is_block_shift(q_block):
    """ceil, sqrt and products are monotone, so the block's bound is its loudest row's bound:
    max over a block's rows of U_i and m_i equal the block's U and m exactly, and the
    eligibility (decided per block) is the same in both modes."""
    inp = WL.generic_inputs(13, "bf16", 2, 3, 32, 300, (130, 77), q_block=q_block,
                            center="compute", k_offset=2.0, q_scale=1.7)
    q = inp.q.astype(np.float64)
    q[:, 40:50, 1] *= 9.0                   # a few loud rows in one head
    blk = O.bounds(q, inp.k, inp.v, scale=0.2, q_block=q_block, center="compute")
    row = O.bounds(q, inp.k, inp.v, scale=0.2, q_block=q_block, center="compute", shift="row")
    assert np.array_equal(blk.m, row.m) and np.array_equal(blk.elig, row.elig)
    for beta in range(blk.m.shape[2]):
        lo, hi = beta * q_block, min((beta + 1) * q_block, 300)
        assert np.array_equal(row.u_row[:, :, lo:hi].max(axis=2), blk.u[:, :, beta])
        assert np.array_equal(row.m_row[:, :, lo:hi].max(axis=2), blk.m[:, :, beta])
    assert (row.m_row <= np.repeat(blk.m, q_block, axis=2)[:, :, :300]).all()


def test_row_shift_closed_form_and_headroom():
    """Rows along one direction with norms n_i against keys +-e0 (max norm 1, no centring):
    U_i = alpha n_i, m_i = ceil(alpha n_i) - C, and each row's largest shifted exponent
    alpha n_i - m_i lies in (C - 1, C]; under the block shift the quiet rows sit
    ceil(U_max) - ceil(U_i) further down (the overshoot [CM] Best practices warns about)."""
    D, norms = 4, [0.5, 3.25, 17.0, 60.5]
    scale = 0.125
    alpha = float(np.float32(scale)) * 1.4426950408889634
    q = np.zeros((1, len(norms), 1, D))
    for i, n in enumerate(norms):
        q[0, i, 0, 0] = n
    k = np.zeros((1, 2, 1, D))
    k[0, 0, 0, 0], k[0, 1, 0, 0] = 1.0, -1.0
    v = np.ones((1, 2, 1, D))
    row = O.bounds(q, [k], [v], scale=scale, q_block=64, shift="row", dtype="fp32")
    L, C, W, gate = O.constants(2)
    assert row.C == C
    for i, n in enumerate(norms):
        assert row.m_row[0, 0, i] == math.ceil(alpha * n) - C
    o, lse, windows = O.method_forward(q, [k], [v], row, scale=scale, q_block=64)
    _, _, e0, e1 = O.fixed_m_emulate(q[0, :, 0], [k[0, :, 0]], [v[0, :, 0]], scale=scale,
                                     k_mean=np.zeros(D), m=row.m_row[0, 0], C=C)
    assert C - 1 < e1 <= C
    for i, n in enumerate(norms):
        e_top = alpha * n - row.m_row[0, 0, i]
        assert C - 1 < e_top <= C
        e_blk = alpha * n - row.m[0, 0, 0]
        assert e_blk == pytest.approx(e_top - (row.m[0, 0, 0] - row.m_row[0, 0, i]))
    ref, lse_ref = O.attention(q, k, v, scale)
    assert np.max(np.abs(o - ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12


def test_v_bound_inclusive_and_nan():
    q = np.ones((1, 4, 1, 4))
    k = [np.ones((1, 5, 1, 4))]
    for vmax, ok in [(256.0, True), (np.nextafter(256.0, 1e9), False), (-256.0, True), (-257.0, False)]:
        v = np.zeros((1, 5, 1, 4))
        v[0, 2, 0, 1] = vmax
        b = O.bounds(q, k, [v], scale=0.5, q_block=64)
        assert b.v_ok == ok and bool(b.elig.all()) == ok
    v = np.zeros((1, 5, 1, 4))
    v[0, 0, 0, 0] = np.nan
    b = O.bounds(q, k, [v], scale=0.5, q_block=64)
    assert not b.v_ok and not b.elig.any()


def test_dtype_and_nonfinite():
    q = np.ones((1, 4, 1, 4))
    k = [np.ones((1, 5, 1, 4))]
    v = [np.zeros((1, 5, 1, 4))]
    assert not O.bounds(q, k, v, scale=0.5, q_block=64, dtype="fp16").elig.any()
    assert O.bounds(q, k, v, scale=0.5, q_block=64, dtype="fp32").elig.all()
    qi = q.copy()
    qi[0, 1, 0, 2] = np.inf
    b = O.bounds(qi, k, v, scale=0.5, q_block=64)
    assert not b.elig.any() and b.m[0, 0, 0] == O.INT32_MAX


# ---------------------------------------------------------------- attention -----------
def test_attention_bruteforce_and_scipy():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 5, 3, 4))
    k = rng.standard_normal((2, 7, 3, 4))
    v = rng.standard_normal((2, 7, 3, 4))
    o, lse = O.attention(q, k, v, 0.7)
    ob = O.attention_bruteforce(q, k, v, 0.7)
    assert np.max(np.abs(o - ob)) < 1e-13
    s = float(np.float32(0.7)) * np.einsum("bqhd,bkhd->bhqk", q, k)
    w = scipy.special.softmax(s, axis=-1)
    oref = np.einsum("bhqk,bkhd->bqhd", w, v)
    assert np.max(np.abs(o - oref)) < 1e-13
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=-1))) < 1e-12


def test_attention_rows_bruteforce():
    """attention_rows (the checker of the sampled rows at full sizes) against the pure-Python
    triple loop on the same rows: rows given out of order, repeated, across two batches and
    three heads, and including the last row of a ragged last q-block (Sq = 11 with q-blocks of
    4).  A mistake in the row indexing (wrong axis, sorting, dropping a repeat) fails here."""
    rng = np.random.default_rng(31)
    q = rng.standard_normal((2, 11, 3, 4))
    k = rng.standard_normal((2, 6, 3, 4))
    v = rng.standard_normal((2, 6, 3, 4))
    rows = np.array([10, 0, 7, 7, 3, 8])
    o, lse = O.attention_rows(q, k, v, 0.6, rows)
    assert o.shape == (2, len(rows), 3, 4) and lse.shape == (2, 3, len(rows))
    ob = O.attention_bruteforce(q[:, rows], k, v, 0.6)
    assert np.max(np.abs(o - ob)) < 1e-13
    s = float(np.float32(0.6)) * np.einsum("bqhd,bkhd->bhqk", q[:, rows], k)
    assert np.max(np.abs(lse - scipy.special.logsumexp(s, axis=-1))) < 1e-12
    # closed form: a zero query row gives the mean of v wherever it sits in the list
    qz = q.copy()
    qz[:, 8] = 0.0
    oz, lz = O.attention_rows(qz, k, v, 0.6, rows)
    assert np.allclose(oz[:, 5], v.mean(axis=1), atol=1e-14)
    assert np.allclose(lz[:, :, 5], math.log(6), atol=1e-14)


def test_default_scale_closed_form():
    """softmax_scale defaults to 1/sqrt(d) ([CM] Interface table), held as an fp32: exact
    powers of two where d is a power of 4, and otherwise the fp32 nearest to 1/sqrt(d)."""
    assert O.default_scale(64) == 0.125
    assert O.default_scale(16) == 0.25 and O.default_scale(256) == 0.0625
    for d in (128, 96, 80, 72):
        s = O.default_scale(d)
        exact = Fraction(1) / Fraction(math.isqrt(d * 10**40)) * 10**20   # 1/sqrt(d) to ~1e-20
        f = np.float32(s)
        assert float(f) == s
        lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1))
        # the neighbours of s are both further from 1/sqrt(d) than s is
        assert abs(Fraction(float(s)) - exact) < abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(s)) - exact) < abs(Fraction(float(hi)) - exact)
    assert O.default_scale(128) == float(np.float32(2.0**-3.5))


def test_attention_special_cases(golden_dir):
    rng = np.random.default_rng(4)
    k = rng.standard_normal((1, 9, 2, 4))
    v = rng.standard_normal((1, 9, 2, 4))
    # q = 0: every weight equal, O = mean of v
    o, lse = O.attention(np.zeros((1, 3, 2, 4)), k, v, 1.0)
    assert np.allclose(o, v.mean(axis=1, keepdims=True), atol=1e-14)
    assert np.allclose(lse, math.log(9), atol=1e-14)
    # a single key: O = v
    q = rng.standard_normal((1, 3, 2, 4))
    o, _ = O.attention(q, k[:, :1], v[:, :1], 1.0)
    assert np.allclose(o, np.broadcast_to(v[:, :1], o.shape), atol=1e-14)
    # identical keys: O = mean of v
    kk = np.broadcast_to(k[:, :1], k.shape)
    o, _ = O.attention(q, kk, v, 1.0)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-13)
    # the printed layout example: two heads, 3 tokens, head_dim 1
    g = _load(golden_dir, "layout_example.json")
    vals = np.array(g["values_per_head"]).T[None, :, :, None]      # [1, 3, 2, 1]
    o, _ = O.attention(np.zeros((1, 3, 2, 1)), np.zeros((1, 3, 2, 1)), vals, 1.0)
    assert np.allclose(o[0, :, :, 0], np.array(g["expected_per_head"])[None, :], atol=1e-14)
    assert not np.allclose(o[0, 0, :, 0], g["buggy_per_head"])


def test_mass_is_one_per_row():
    inp = WL.make_inputs(1)
    q = inp.q[0, :, 0].astype(np.float64)
    k = np.concatenate(inp.k, axis=1)[0, :, 0].astype(np.float64)
    v = np.concatenate(inp.v, axis=1)[0, :, 0].astype(np.float64)
    _, lse = O.attention(q[None, :, None], k[None, :, None], v[None, :, None], inp.wl.scale)
    mass = O.softmax_mass(q, k, inp.wl.scale, lse[0, 0])
    assert np.max(np.abs(mass - 1.0)) < 1e-12


# ---------------------------------------------------------------- the two bodies ------
def _cfg1_head():
    inp = WL.make_inputs(1)
    q = inp.q[0, :, 0].astype(np.float64)
    kc = [c[0, :, 0].astype(np.float64) for c in inp.k]
    vc = [c[0, :, 0].astype(np.float64) for c in inp.v]
    return inp, q, kc, vc


def test_fixed_m_body_equals_softmax_and_is_shift_invariant():
    inp, q, kc, vc = _cfg1_head()
    scale = inp.wl.scale
    b = O.bounds(q[None, :, None], [c[None, :, None] for c in kc], [c[None, :, None] for c in vc],
                 scale=scale, q_block=256)
    assert b.elig.all()
    ref, lse_ref = O.attention(q[None, :, None], np.concatenate(kc)[None, :, None],
                               np.concatenate(vc)[None, :, None], scale)
    ref, lse_ref = ref[0, :, 0], lse_ref[0, 0]
    m = int(b.m[0, 0, 0])
    o, lse, e0, e1 = O.fixed_m_emulate(q, kc, vc, scale=scale, k_mean=np.zeros(64), m=m, C=b.C)
    assert -125 <= e0 and e1 <= b.C
    assert np.max(np.abs(o - ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    for dm in (-3, 3):
        o2, lse2, _, _ = O.fixed_m_emulate(q, kc, vc, scale=scale, k_mean=np.zeros(64),
                                           m=m + dm, C=b.C, check_window=False)
        assert np.max(np.abs(o2 - ref)) < 1e-12 and np.max(np.abs(lse2 - lse_ref)) < 1e-12
    kbar = np.random.default_rng(5).standard_normal(64).astype(np.float32)
    o3, lse3, _, _ = O.fixed_m_emulate(q, kc, vc, scale=scale, k_mean=kbar, m=m, C=b.C,
                                       check_window=False)
    assert np.max(np.abs(o3 - ref)) < 1e-12 and np.max(np.abs(lse3 - lse_ref)) < 1e-12
    # chunk order does not matter (pure addition)
    o4, _, _, _ = O.fixed_m_emulate(q, kc[::-1], vc[::-1], scale=scale, k_mean=np.zeros(64), m=m, C=b.C)
    assert np.max(np.abs(o4 - ref)) < 1e-12


@pytest.mark.parametrize("block", [1, 7, 64, 1000])
def test_online_body_equals_softmax(block):
    inp, q, kc, vc = _cfg1_head()
    ref, lse_ref = O.attention(q[None, :, None], np.concatenate(kc)[None, :, None],
                               np.concatenate(vc)[None, :, None], inp.wl.scale)
    o, lse = O.online_softmax_emulate(q, kc, vc, scale=inp.wl.scale, block=block)
    assert np.max(np.abs(o - ref[0, :, 0])) < 1e-12
    assert np.max(np.abs(lse - lse_ref[0, 0])) < 1e-12


@pytest.mark.parametrize("q_block", [64, 256])
def test_method_forward_tiny_config(q_block):
    inp = WL.make_inputs(1)
    wl = inp.wl
    b = O.bounds(inp.q, inp.k, inp.v, scale=wl.scale, q_block=q_block, center=wl.center)
    o, lse, windows = O.method_forward(inp.q, inp.k, inp.v, b, scale=wl.scale, q_block=q_block)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), wl.scale)
    assert np.max(np.abs(o - ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    assert len(windows) == b.elig.sum() > 0
    for (_, _, _, e0, e1) in windows:
        assert e0 >= -125 and e1 <= b.C


def test_method_forward_mixed_bodies_and_centring():
    """Offset keys with centring on, one adversarial head that must fall back."""
    inp = WL.generic_inputs(21, "fp32", 1, 3, 16, 70, (40, 33), q_block=64, k_offset=3.0)
    q = inp.q.astype(np.float64)
    q[:, :, 2] *= 60.0                      # head 2 loud: fails the gate
    scale = 0.25
    b = O.bounds(q, inp.k, inp.v, scale=scale, q_block=64, center="compute", dtype="fp32")
    assert b.elig[0, :2].all() and not b.elig[0, 2].any()
    o, lse, windows = O.method_forward(q, inp.k, inp.v, b, scale=scale, q_block=64, block=16)
    ref, lse_ref = O.attention(q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), scale)
    assert np.max(np.abs(o - ref)) < 1e-11 and np.max(np.abs(lse - lse_ref)) < 1e-11


@pytest.mark.parametrize("q_block", [64, 256])
def test_method_forward_row_shift(q_block):
    """The whole method with per-row shifts equals softmax attention, and every eligible
    row's shifted exponents stay inside [-125, C], on the tiny config and on offset keys with
    centring and a loud head that falls back."""
    inp = WL.make_inputs(1)
    wl = inp.wl
    b = O.bounds(inp.q, inp.k, inp.v, scale=wl.scale, q_block=q_block, shift="row")
    o, lse, windows = O.method_forward(inp.q, inp.k, inp.v, b, scale=wl.scale, q_block=q_block)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), wl.scale)
    assert np.max(np.abs(o - ref)) < 1e-12 and np.max(np.abs(lse - lse_ref)) < 1e-12
    assert len(windows) == b.elig.sum() > 0
    for (_, _, _, e0, e1) in windows:
        assert e0 >= -125 and e1 <= b.C
    inp = WL.generic_inputs(21, "fp32", 1, 3, 16, 70, (40, 33), q_block=64, k_offset=3.0)
    q = inp.q.astype(np.float64)
    q[:, :, 2] *= 60.0
    q[:, 5:9, 0] *= 4.0
    b = O.bounds(q, inp.k, inp.v, scale=0.25, q_block=64, center="compute", dtype="fp32", shift="row")
    assert b.elig[0, :2].all() and not b.elig[0, 2].any()
    assert len(set(b.m_row[0, 0].tolist())) > 1
    o, lse, _ = O.method_forward(q, inp.k, inp.v, b, scale=0.25, q_block=64, block=16)
    ref, lse_ref = O.attention(q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), 0.25)
    assert np.max(np.abs(o - ref)) < 1e-11 and np.max(np.abs(lse - lse_ref)) < 1e-11


def test_empty_chunk_changes_nothing():
    """A ring step with no keys: the bounds and the method's output equal those of the same
    keys without it (the maxima and sums run over real keys only)."""
    inp = WL.generic_inputs(22, "fp32", 1, 2, 16, 40, (30, 0, 25), q_block=32, k_offset=1.0)
    kk = [inp.k[0], inp.k[2]]
    vv = [inp.v[0], inp.v[2]]
    scale = 0.25
    b0 = O.bounds(inp.q, inp.k, inp.v, scale=scale, q_block=32, center="compute", dtype="fp32")
    b1 = O.bounds(inp.q, kk, vv, scale=scale, q_block=32, center="compute", dtype="fp32")
    for f in ("m", "elig", "q2", "k2", "k_mean"):
        assert np.array_equal(getattr(b0, f), getattr(b1, f)), f
    o0, l0, _ = O.method_forward(inp.q, inp.k, inp.v, b0, scale=scale, q_block=32, block=16)
    o1, l1, _ = O.method_forward(inp.q, kk, vv, b1, scale=scale, q_block=32, block=16)
    ref, lse_ref = O.attention(inp.q, np.concatenate(kk, 1), np.concatenate(vv, 1), scale)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    assert np.max(np.abs(o0 - ref)) < 1e-12 and np.max(np.abs(l0 - lse_ref)) < 1e-12


# ---------------------------------------------------------------- planted mistakes ----
def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    """Mistakes planted in the oracle (on the CPU) trip the pins above."""
    mod = O.fixedm_oracle
    cases = _load(golden_dir, "printed_constants.json")["cases"]
    real_constants = mod.constants
    # 1. floor instead of ceil for log2 N: the printed W values no longer match
    monkeypatch.setattr(mod, "ceil_log2", lambda n: max(n.bit_length() - 1, 0))
    assert any(mod.constants(c["n"])[2] != c["W"] for c in cases)
    monkeypatch.undo()
    # 2. the full window W used as the gate: the adversarial query becomes eligible
    monkeypatch.setattr(mod, "constants", lambda n, vmax=O.VMAX: real_constants(n, vmax)[:3]
                        + (real_constants(n, vmax)[2],))
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((4096, 16))
    keys -= keys.mean(axis=0)
    keys /= np.linalg.norm(keys, axis=1).max()
    q = np.ones((1, 4, 1, 16)) / 4.0 * (231.01 / mod.alpha_of(0.25))
    b = mod.bounds(q, [keys[None, :, None]], [np.zeros((1, 4096, 1, 16))], scale=0.25, q_block=64)
    assert b.elig.all()          # test_adversarial_query_fails_halved_gate would fail
    monkeypatch.undo()
    # 3. a sign error in the fixed-m exponent: the body no longer equals softmax
    inp, qh, kc, vc = _cfg1_head()
    ref, _ = O.attention(qh[None, :, None], np.concatenate(kc)[None, :, None],
                         np.concatenate(vc)[None, :, None], inp.wl.scale)
    o_bad, _, _, _ = O.fixed_m_emulate(-qh, kc, vc, scale=inp.wl.scale, k_mean=np.zeros(64),
                                       m=0, C=200, check_window=False)
    assert np.max(np.abs(o_bad - ref[0, :, 0])) > 1e-3
    # 4. a transposed operand (keys used as values) is caught by the brute-force pin
    rng = np.random.default_rng(3)
    qq, kk, vv = (rng.standard_normal((1, 5, 1, 4)) for _ in range(3))
    assert np.max(np.abs(O.attention(qq, kk, kk, 0.7)[0] - O.attention_bruteforce(qq, kk, vv, 0.7))) > 1e-3


# ---------------------------------------------------------------- exact key sum --------
def _fraction_sum(col):
    """The exact sum of fp64 numbers as a Fraction, rounded once to fp64 (Fraction -> float
    rounds to nearest, ties to even)."""
    return float(sum((Fraction(float(x)) for x in col), Fraction(0)))


def _wide_fp32(rng, shape, lo_exp, hi_exp):
    """fp32 values with random signs, mantissas and exponents in [lo_exp, hi_exp]."""
    m = rng.uniform(1.0, 2.0, size=shape)
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    s = rng.choice([-1.0, 1.0], size=shape)
    return (s * np.ldexp(m, e)).astype(np.float32)


@pytest.mark.parametrize("lo_exp,hi_exp", [(-20, 20), (-60, 60), (-149, -120), (100, 127)])
def test_exact_key_sum_against_fractions(lo_exp, hi_exp):
    """exact_sum_f64 equals the exact rational sum rounded once to fp64, on fp32 keys whose
    magnitudes span many binades (where a running fp64 sum loses bits), fp32 denormals, and
    values near the top of the fp32 range; chunked unevenly."""
    rng = np.random.default_rng(lo_exp + 1000)
    k = _wide_fp32(rng, (2, 301, 2, 3), lo_exp, hi_exp)
    k[0, 5, 0, 0] = 0.0
    got = O.exact_sum_f64([k[:, :100], k[:, 100:101], k[:, 101:]])
    for b in range(2):
        for h in range(2):
            for d in range(3):
                assert got[b, h, d] == _fraction_sum(k[b, :, h, d].astype(np.float64)), (b, h, d)


def test_exact_key_sum_cancellation_and_order():
    """A sum a running fp64 sum gets wrong (2^60 + 1 - 2^60 = 1, not 0), the same keys in
    every order and chunking giving the same bits, bf16 keys, and math.fsum agreeing on
    ordinary data."""
    k = np.zeros((1, 3, 1, 1), np.float32)
    k[0, :, 0, 0] = [2.0**60, 1.0, -(2.0**60)]
    assert O.exact_sum_f64([k])[0, 0, 0] == 1.0
    naive = 0.0
    for x in k[0, :, 0, 0].astype(np.float64):
        naive += x
    assert naive == 0.0                                      # the running sum drops the 1
    rng = np.random.default_rng(8)
    k = _wide_fp32(rng, (1, 500, 3, 4), -40, 40)
    ref = O.exact_sum_f64([k])
    perm = rng.permutation(500)
    assert np.array_equal(O.exact_sum_f64([k[:, perm[:123]], k[:, perm[123:]]]), ref)
    kb = WL.f32_from_bf16_bits(WL.bf16_bits_from_f32(_wide_fp32(rng, (1, 400, 2, 5), -30, 30)))
    got = O.exact_sum_f64([kb])
    for h in range(2):
        for d in range(5):
            assert got[0, h, d] == _fraction_sum(kb[0, :, h, d].astype(np.float64))
    kn = rng.standard_normal((1, 5000, 2, 4)).astype(np.float32)
    got = O.exact_sum_f64([kn])
    for h in range(2):
        for d in range(4):
            assert got[0, h, d] == math.fsum(kn[0, :, h, d].astype(np.float64))


def test_exact_key_sum_nonfinite():
    """NaN anywhere, or both infinities, give NaN; one infinity gives itself (IEEE sums)."""
    k = np.ones((1, 4, 1, 4), np.float32)
    k[0, 1, 0, 0] = np.nan
    k[0, 0, 0, 1], k[0, 2, 0, 1] = np.inf, -np.inf
    k[0, 3, 0, 2] = np.inf
    k[0, 3, 0, 3] = -np.inf
    got = O.exact_sum_f64([k])[0, 0]
    assert np.isnan(got[0]) and np.isnan(got[1]) and got[2] == np.inf and got[3] == -np.inf
    km = O.k_mean_of([k])[0, 0]
    assert np.isnan(km[0]) and km[2] == np.inf and km[3] == -np.inf
