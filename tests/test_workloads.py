"""The seeded input generators: deterministic, right shapes, and the stated recipes."""
import numpy as np

from dit_amd import workloads as WL


def test_bf16_rounding_rne():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even pattern (1.0);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties go to 1 + 2^-6
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, np.inf],
                 dtype=np.float32)
    back = WL.f32_from_bf16_bits(WL.bf16_bits_from_f32(x))
    assert back.tolist() == [1.0, 1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, np.inf]
    # every finite bf16 pattern survives widening then rounding
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    f = WL.f32_from_bf16_bits(bits)
    finite = np.isfinite(f)
    assert np.array_equal(WL.bf16_bits_from_f32(f[finite]), bits[finite])


def test_tiny_config_deterministic():
    a, b = WL.make_inputs(1), WL.make_inputs(1)
    assert np.array_equal(a.q, b.q) and all(np.array_equal(x, y) for x, y in zip(a.k, b.k))
    assert a.q.shape == (1, 256, 1, 64) and [c.shape[1] for c in a.k] == [128, 128]


def test_adversarial_recipe():
    inp = WL.make_inputs(5)
    wl = inp.wl
    q = inp.q.astype(np.float64)
    alpha = float(np.float32(wl.scale)) * 1.4426950408889634
    qn = np.linalg.norm(q[0, :, 4:], axis=-1) * alpha
    assert np.allclose(qn, 231.01, rtol=1e-6)
    k = np.concatenate(inp.k, axis=1).astype(np.float64)[0, :, 4:]
    assert np.allclose(k.mean(axis=0), 0.0, atol=1e-7)
    assert np.allclose(np.linalg.norm(k, axis=-1).max(axis=0), 1.0, rtol=1e-6)


def test_ragged_recipe_small_draw():
    inp = WL.generic_inputs(3, "bf16", 1, 2, 8, 9, (5, 4), k_offset=3.0)
    assert np.allclose(np.linalg.norm(inp.k_mean, axis=-1), 3.0, rtol=1e-6)
    assert inp.q_store.dtype == np.uint16 and inp.q.dtype == np.float32
