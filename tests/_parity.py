"""Helpers for the GPU parity tests: move seeded inputs to the device, run the C ABI path,
and compare with the oracle.  Tolerances (stated in the spec acceptance criteria):
m and the eligibility mask bit-exact; bf16 inputs max |dO| <= 1e-2 and mean |dO| <= 1e-3;
fp32 inputs max |dO| <= 1e-5."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O

TOL = {"bf16": {"max": 1e-2, "mean": 1e-3}, "fp32": {"max": 1e-5, "mean": 1e-5}}
# lse = ln2 (r + log2 l).  On the bf16 path l sums the bf16-rounded probabilities that the
# PV product uses (relative rounding <= 2^-9 each), so |d lse| <= ln(1 + 2^-9) < 2e-3 plus
# fp32 rounding; 2.5e-3 is that bound with margin.  The fp32 path keeps fp32 probabilities.
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
    assert np.array_equal(gb["k_mean"].view(np.uint32), ob.k_mean.view(np.uint32)), "k_mean bits"
    assert np.array_equal(gb["k2"], ob.k2), "K2"
    assert np.array_equal(gb["q2"], ob.q2), "Q2"
    assert np.array_equal(gb["u"], ob.u) or np.array_equal(np.isnan(gb["u"]), np.isnan(ob.u)), "U"
    assert np.array_equal(gb["m"].astype(np.int64), ob.m), "m"
    assert np.array_equal(gb["elig"].astype(bool), ob.elig), "eligibility mask"
    assert bool(gb["v_bad"][0] == 0) == ob.v_ok


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got.astype(np.float64) - ref)
    return float(d.max()), float(d.mean())


def check_output(got, ref, dtype: str, what: str = "O"):
    mx, mn = err_stats(got, ref)
    say(f"  {what}: max|d|={mx:.3e} mean|d|={mn:.3e} (tol {TOL[dtype]})")
    assert np.isfinite(got).all(), f"{what} has non-finite values"
    assert mx <= TOL[dtype]["max"], f"{what} max abs error {mx}"
    assert mn <= TOL[dtype]["mean"], f"{what} mean abs error {mn}"
    return mx, mn


def bf16_rne_bits(x_f32: np.ndarray) -> np.ndarray:
    from dit_amd.workloads import bf16_bits_from_f32
    return bf16_bits_from_f32(x_f32)
