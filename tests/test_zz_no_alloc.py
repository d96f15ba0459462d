"""fixedm_bounds_static, the entry point that allocates nothing (its scratch is a static device
array), against fixedm_bounds through the C ABI: identical bounds on two calls in a row, the
second with a smaller problem (the array keeps the first call's contents), and attention
outputs computed from its descriptor identical to those from fixedm_bounds's."""
import numpy as np
import pytest

import oracle as O
from dit_amd import workloads as WL

from _parity import check_bounds, device_inputs, gpu_bounds_dict, say

pytestmark = pytest.mark.gpu

KEYS = ("k_mean", "k2", "q2", "u", "m", "elig", "v_bad")


@pytest.fixture(scope="module")
def F():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dit_amd import fixedm
    fixedm.lib()
    return fixedm


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_static_bounds_match_the_allocating_call(F, dtype, D):
    import torch
    cases = [(2, 5, 700, (3000, 2111), "compute"), (1, 3, 130, (600, 77), "compute")]
    for seed, (B, H, Sq, chunks, center) in enumerate(cases):
        say(f"static bounds: {dtype} B={B} H={H} Sq={Sq} chunks={chunks}")
        inp = WL.generic_inputs(90 + seed, dtype, B, H, D, Sq, chunks, q_block=64, center=center,
                                k_offset=2.0)
        inp.k_mean = None
        q, ks, vs, _ = device_inputs(inp)
        p = F.make_problem(dtype, B, H, D, Sq, sum(chunks), 64, 0.0, center)
        d1, b1 = F.bounds(p, q, ks, vs)
        d2, b2 = F.bounds_static(p, q, ks, vs)
        torch.cuda.synchronize()
        g1, g2 = gpu_bounds_dict(d1, b1), gpu_bounds_dict(d2, b2)
        for k in KEYS:
            assert np.array_equal(np.asarray(g1[k]), np.asarray(g2[k]), equal_nan=True), k
        ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(D), q_block=64, center=center, dtype=dtype)
        check_bounds(g2, ob)
        outs = []
        for d in (d1, d2):
            ws = F.alloc_workspace(p, q.device)
            out = torch.empty_like(q, dtype=torch.float32)
            F.attn_fwd_final(d, F.run_init(d), q, ks, vs, ws, out)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
