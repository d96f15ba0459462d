"""Helpers for the GPU parity tests: move seeded inputs to the device, run the C ABI path,
and compare with the oracle.  Tolerances (stated in the spec acceptance criteria):
m and the eligibility mask bit-exact; bf16 inputs max |dO| <= 1e-2 and mean |dO| <= 1e-3;
fp32 inputs max |dO| <= 1e-5."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

TOL = {"bf16": {"max": 1e-2, "mean": 1e-3}, "fp32": {"max": 1e-5, "mean": 1e-5}}
# lse = ln2 (r + log2 l).  On the bf16 path l sums fp32 probabilities, and the logits come
# from bf16(alpha q) (one rounding, relative <= 2^-8 per element).  Over thousands of keys of
# Wan-like rows the rounding's effect averages out far below the worst case; 2.5e-3 is the
# tolerance set on those rows (measured errors ~1e-3).  Rows far louder than that are
# checked against lse_bound_bf16, the worst case of the same arithmetic.  The fp32 path forms
# logits and probabilities in fp64 and fp32.
LSE_TOL = {"bf16": 2.5e-3, "fp32": 1e-5}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda")


def device_inputs(inp):
    dt = inp.wl.dtype
    q = to_dev(inp.q_store, dt)
    ks = [to_dev(c, dt) for c in inp.k_store]
    vs = [to_dev(c, dt) for c in inp.v_store]
    km = None
    if inp.k_mean is not None:
        import torch
        km = torch.from_numpy(np.ascontiguousarray(inp.k_mean, np.float32)).to("cuda")
    return q, ks, vs, km


def gpu_bounds_dict(desc, buf):
    from dit_amd import fixedm as F
    d = F.read_bounds(desc, buf)
    return {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in d.items()}


def check_bounds(gb: dict, ob: "O.Bounds"):
    """Bit-exact comparison of the GPU bounds with the oracle's."""
    assert (gb["C"], gb["W"], gb["gate"], gb["log2_n"]) == (ob.C, ob.W, ob.gate, ob.L)
    # k_mean bit for bit; where the oracle's is NaN (a NaN key, or both infinities, in that
    # element's keys) the GPU's must be NaN too (the payload is not compared)
    okm, gkm = ob.k_mean, gb["k_mean"]
    fin = ~np.isnan(okm)
    assert np.array_equal(gkm[fin].view(np.uint32), okm[fin].view(np.uint32)), "k_mean bits"
    assert np.isnan(gkm[~fin]).all(), "k_mean NaN"
    assert np.array_equal(gb["k2"], ob.k2, equal_nan=True), "K2"
    assert np.array_equal(gb["q2"], ob.q2, equal_nan=True), "Q2"
    # U is alpha * sqrt(Q2 * K2) in fp64 on both sides: equal value for value, NaN where the
    # oracle has NaN (a non-finite query or key) and nowhere else
    assert np.array_equal(gb["u"], ob.u, equal_nan=True), "U"
    assert np.array_equal(gb["m"].astype(np.int64), ob.m), "m"
    assert np.array_equal(gb["elig"].astype(bool), ob.elig), "eligibility mask"
    assert bool(gb["v_bad"][0] == 0) == ob.v_ok
    assert ("m_row" in gb) == (ob.m_row is not None), "shift granularity"
    if ob.m_row is not None:
        assert np.array_equal(gb["q2_row"], ob.q2_row), "Q2 per row"
        assert np.array_equal(gb["u_row"], ob.u_row), "U per row"
        assert np.array_equal(gb["m_row"].astype(np.int64), ob.m_row), "m per row"


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.mean())


def error_quantiles(got, ref, qs=(0.5, 0.9, 0.99, 0.999, 1.0)) -> dict:
    """Distribution of |got - ref| (element-wise, fp64): the given quantiles."""
    d = np.abs(np.asarray(got, np.float64) - ref).ravel()
    return {q: float(np.quantile(d, q)) for q in qs}


def check_output(got, ref, dtype: str, what: str = "O"):
    mx, mn = err_stats(got, ref)
    say(f"  {what}: max|d|={mx:.3e} mean|d|={mn:.3e} (tol {TOL[dtype]})")
    eq = error_quantiles(got, ref)
    say("  |d| quantiles: " + "  ".join(f"p{100 * q:g}={v:.2e}" for q, v in eq.items()))
    assert np.isfinite(got).all(), f"{what} has non-finite values"
    assert mx <= TOL[dtype]["max"], f"{what} max abs error {mx}"
    assert mn <= TOL[dtype]["mean"], f"{what} mean abs error {mn}"
    return mx, mn


def lse_bound_bf16(q, k_all, scale: float) -> np.ndarray:
    """Worst-case lse error of the bf16 path per row, [B, H, Sq]: the fixed-m body forms
    logits from bf16(alpha q) (one round-to-nearest-even, relative error <= 2^-8 per element),
    so a base-2 logit moves by at most 2^-8 sum_d |alpha q_d k_d| and lse by ln 2 times that;
    ln(1 + 2^-8) more covers the fp32 summation of l and the online body's bf16 path with
    ample margin.  Used for rows far louder than the Wan-like ones LSE_TOL was set on."""
    alpha = float(np.float32(scale)) * O.LOG2E
    qa = np.abs(alpha * np.asarray(q, np.float64))
    ka = np.abs(np.asarray(k_all, np.float64))
    B, Sq, H, D = qa.shape
    out = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            out[b, h] = (qa[b, :, h] @ ka[b, :, h].T).max(axis=1)
    return np.log(2.0) * 2.0**-8 * out + np.log1p(2.0**-8) + 1e-5


def out_bound_bf16(q, k_all, v_all, scale: float, ref) -> np.ndarray:
    """Worst-case |O - ref| of the bf16 path per element, [B, Sq, H, D], for rows over few keys,
    where the errors do not average out: each probability enters the PV product rounded to bf16
    (relative <= 2^-8, l sums the fp32 values), which moves O by at most 2^-8 max_j |v_jd|; the
    logits come from bf16(alpha q), so each moves by at most E = 2^-8 max_j sum_d |alpha q_d k_jd|
    (base 2) and every normalised weight by a factor within 2^(+-2E), which moves O by at most
    (2^(2E) - 1) max_j |v_jd - ref_d|.  1e-5 covers the fp32 accumulation.  Holds O(Sq N) memory
    per (b, h): meant for short key sets."""
    alpha = float(np.float32(scale)) * O.LOG2E
    qa = np.abs(alpha * np.asarray(q, np.float64))
    ka = np.abs(np.asarray(k_all, np.float64))
    va = np.asarray(v_all, np.float64)
    ref = np.asarray(ref, np.float64)
    e = 2.0**-8 * np.einsum("bihd,bjhd->bhij", qa, ka).max(axis=3)        # [B, H, Sq]
    grow = np.exp2(2.0 * e) - 1.0
    vmax = np.abs(va).max(axis=1)                                            # [B, H, D]
    out = np.empty_like(ref)
    for i in range(ref.shape[1]):
        spread = np.abs(va - ref[:, i:i + 1]).max(axis=1)                    # [B, H, D]
        out[:, i] = 2.0**-8 * vmax + grow[:, :, i, None] * spread + 1e-5
    return out


def bf16_rne_bits(x_f32: np.ndarray) -> np.ndarray:
    from dit_amd.workloads import bf16_bits_from_f32
    return bf16_bits_from_f32(x_f32)


def assert_bf16_is_rne(bits: np.ndarray, x_f32: np.ndarray):
    """bf16 output bits are the round-to-nearest-even of the fp32 output wherever that is not a
    NaN; where it is a NaN they are a NaN too (the payload is not fixed)."""
    nan = np.isnan(x_f32)
    assert np.array_equal(bits[~nan], bf16_rne_bits(x_f32)[~nan])
    b = bits[nan].astype(np.uint32)
    assert np.all(((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0))
