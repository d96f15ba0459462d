"""GPU parity: the HIP path through the C ABI against the fp64 oracle on seeded inputs.

Bounds (k_mean, Q2, K2, U, m, eligibility) are compared bit for bit on every config; the
output within the acceptance tolerances (_parity.TOL).  Configs 1, 2 and 5 are compared in
full; configs 3 and 4 (the Wan 720p rank share and the ragged one) on sampled rows of every
head, including the ragged last q-block, at the full sizes.  Config 3 runs both as a ring
rank sees it (bounds + one fixedm_attn_fwd per ring chunk + finalize) and in the launch
configuration the benchmark times (bounds + one fixedm_attn_fwd_final over the four chunks
in ring order).  The fused and multi-chunk paths are also run on the edge cases."""
import numpy as np
import pytest

import oracle as O
from dit_amd import workloads as WL

from _parity import (LSE_TOL, assert_bf16_is_rne, check_bounds, check_output, device_inputs,
                     gpu_bounds_dict, lse_bound_bf16, out_bound_bf16, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dit_amd import fixedm
    fixedm.lib()   # raises if the library is missing: no fallback exists
    return fixedm


def _run(F, inp, *, q_block=None, order=None, out_dtype=None, want_lse=True, **fwd):
    import torch
    wl = inp.wl
    q, ks, vs, km = device_inputs(inp)
    if order is not None:
        ks, vs = [ks[i] for i in order], [vs[i] for i in order]
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=q_block or wl.q_block, center=wl.center,
                                    k_mean=km, out_dtype=out_dtype or torch.float32,
                                    want_lse=want_lse, **fwd)
    torch.cuda.synchronize()
    return out, lse, desc, buf, (q, ks, vs, km)


def _oracle_bounds(inp, q_block=None, shift="block"):
    wl = inp.wl
    return O.bounds(inp.q, inp.k, inp.v, scale=wl.scale, q_block=q_block or wl.q_block,
                    center=wl.center, k_mean=inp.k_mean, dtype=wl.dtype, shift=shift)


# ------------------------------------------------------------------ full configs ------
@pytest.mark.parametrize("q_block", [64, 256])
def test_config1_tiny_fp32(F, q_block):
    say(f"config 1 q_block={q_block}")
    inp = WL.make_inputs(1)
    out, lse, desc, buf, _ = _run(F, inp, q_block=q_block)
    # softmax_scale 0 resolves to fp32(1/sqrt(d)), the [CM] Interface table default
    assert desc.p.softmax_scale == O.default_scale(64) == inp.wl.scale
    ob = _oracle_bounds(inp, q_block)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    check_output(out.cpu().numpy(), ref, "fp32")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["fp32"]


def test_config2_wan_block_bf16(F):
    import torch
    say("config 2")
    inp = WL.make_inputs(2)
    out, lse, desc, buf, dev = _run(F, inp)
    ob = _oracle_bounds(inp)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert ob.elig.all()
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    got = out.cpu().numpy()
    check_output(got, ref, "bf16")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["bf16"]
    # bf16 output is the round-to-nearest-even of the fp32 output, bit for bit
    out16, _, _, _ = F.forward(dev[0], dev[1], dev[2], q_block=256, center="none",
                               out_dtype=torch.bfloat16)
    bits = out16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert_bf16_is_rne(bits, got)


def _sample_rows(sq, q_block, seed=7):
    """Query rows checked at the full sizes: wave 0 of the first 256-row tile, the last 64
    rows (the ragged last q-block and tile), one seeded row of every 256-row tile, and one
    seeded row of each of the four 64-row waves in three middle tiles (every tile runs the
    long-chunk loop schedule on its own workgroup, XCD-remapped)."""
    last_lo = ((sq - 1) // q_block) * q_block
    rows = list(range(0, 64)) + list(range(max(sq - 64, last_lo), sq))
    rng = np.random.default_rng(seed)
    n_tiles = -(-sq // 256)
    for t in range(n_tiles):
        rows.append(t * 256 + int(rng.integers(0, min(256, sq - t * 256))))
    for t in sorted({n_tiles // 4, n_tiles // 2, (3 * n_tiles) // 4}):
        for w in range(4):
            lo = t * 256 + 64 * w
            if lo < sq:
                rows.append(lo + int(rng.integers(0, min(64, sq - lo))))
    return np.array(sorted(set(rows)))


@pytest.fixture(scope="module")
def cfg3(F):
    say("config 3: drawing inputs")
    return WL.make_inputs(3)


def test_config3_bounds_bitexact(F, cfg3):
    say("config 3 bounds")
    inp = cfg3
    import torch
    q, ks, vs, km = device_inputs(inp)
    p = F.make_problem("bf16", 1, 40, 128, inp.wl.sq, inp.wl.sk, 256, 0.0, "compute")
    desc, buf = F.bounds(p, q, ks, vs)
    torch.cuda.synchronize()
    ob = _oracle_bounds(inp)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert ob.elig.all() and (ob.C, ob.gate) == (102, 113)
    say(f"  U range {ob.u.min():.3f}..{ob.u.max():.3f}, m range {ob.m.min()}..{ob.m.max()}")


def test_config3_output_sampled_rows(F, cfg3):
    say("config 3 output (ring order 0,3,2,1)")
    inp = cfg3
    out, lse, desc, buf, _ = _run(F, inp, order=(0, 3, 2, 1))
    rows = _sample_rows(inp.wl.sq, 256)
    ref, lse_ref = O.attention_rows(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1),
                                    inp.wl.scale, rows)
    check_output(out.cpu().numpy()[:, rows], ref, "bf16")
    assert np.abs(lse.cpu().numpy()[:, :, rows] - lse_ref).max() <= LSE_TOL["bf16"]
    assert np.isfinite(out.cpu().numpy()).all()


def test_config4_ragged_offset(F):
    say("config 4")
    inp = WL.make_inputs(4)
    out, lse, desc, buf, _ = _run(F, inp)
    ob = _oracle_bounds(inp)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert ob.elig.all()
    rows = _sample_rows(inp.wl.sq, 256)
    ref, lse_ref = O.attention_rows(inp.q, inp.k[0], inp.v[0], inp.wl.scale, rows)
    check_output(out.cpu().numpy()[:, rows], ref, "bf16")
    assert np.abs(lse.cpu().numpy()[:, :, rows] - lse_ref).max() <= LSE_TOL["bf16"]


def test_config5_adversarial_fp32(F):
    say("config 5")
    inp = WL.make_inputs(5)
    out, lse, desc, buf, _ = _run(F, inp)
    ob = _oracle_bounds(inp)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert ob.elig[0, :4].all() and not ob.elig[0, 4:].any()
    assert (ob.m[0, 4:] == 125).all()
    kall = np.concatenate(inp.k, 1)
    ref, lse_ref = O.attention(inp.q, kall, np.concatenate(inp.v, 1), inp.wl.scale)
    check_output(out.cpu().numpy(), ref, "fp32")
    lse_g = lse.cpu().numpy()
    for h in range(8):
        mass = O.softmax_mass(inp.q[0, :, h], kall[0, :, h], inp.wl.scale, lse_g[0, h])
        assert np.abs(mass - 1.0).max() <= 1e-5, (h, np.abs(mass - 1.0).max())


# ------------------------------------------------------------------ edge cases --------
def _generic(F, seed, dtype, B, H, D, Sq, chunks, q_block=64, center="none", q_scale=1.0,
             k_offset=0.0, v_poke=None, loud_rows=None, shift="block", lse_worst_case=False,
             few_keys=False, scale=None, **fwd):
    """One seeded edge case through the C ABI against the oracle.  scale: an explicit
    softmax scale handed to the ABI (None: the ABI's default, 0, which resolves to the
    oracle's default_scale(D))."""
    import torch
    inp = WL.generic_inputs(seed, dtype, B, H, D, Sq, chunks, q_block=q_block, center=center,
                            q_scale=q_scale, k_offset=k_offset)
    oscale = O.default_scale(D) if scale is None else float(np.float32(scale))
    if loud_rows is not None:                      # (head, lo, hi, factor): a loud q-block
        h, lo, hi, fac = loud_rows
        qf = inp.q.copy()
        qf[:, lo:hi, h] *= np.float32(fac)
        inp.q_store = WL.bf16_bits_from_f32(qf) if dtype == "bf16" else qf
    if v_poke is not None:
        c, idx, val = v_poke
        if dtype == "bf16":
            inp.v_store[c][idx] = WL.bf16_bits_from_f32(np.array([val], np.float32))[0]
        else:
            inp.v_store[c][idx] = val
    kmean = inp.k_mean if center == "supplied" else None
    if center != "supplied":
        inp.k_mean = None
    q, ks, vs, km = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=q_block, center=center, k_mean=km,
                                    out_dtype=torch.float32, want_lse=True, shift=shift,
                                    softmax_scale=0.0 if scale is None else scale, **fwd)
    torch.cuda.synchronize()
    assert desc.p.softmax_scale == oscale, (desc.p.softmax_scale, oscale)
    assert desc.alpha == np.float32(O.alpha_of(oscale))
    ob = O.bounds(inp.q, inp.k, inp.v, scale=oscale, q_block=q_block, center=center,
                  k_mean=kmean, dtype=dtype, shift=shift)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), oscale)
    got = out.cpu().numpy()
    if few_keys and dtype == "bf16":
        # rows over a handful of keys: the bf16 roundings do not average out, so each element
        # is held to the worst case of the bf16 arithmetic instead of the many-key tolerance
        bound = out_bound_bf16(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), oscale, ref)
        assert np.isfinite(got).all()
        assert (np.abs(got - ref) <= bound).all(), float((np.abs(got - ref) / bound).max())
    elif v_poke is None:
        check_output(got, ref, dtype)
    else:
        # bf16 probability rounding scales the error with |v|: the poked (head, dim) column
        # holds one value of magnitude |val|, so its tolerance scales by |val| / 4
        c, (b0, j0, h0, d0), val = v_poke
        keep = np.ones(got.shape, bool)
        keep[:, :, h0, d0] = False
        check_output(got[keep], ref[keep], dtype, "O (other columns)")
        col = np.abs(got[:, :, h0, d0] - ref[:, :, h0, d0]).max()
        assert col <= 1e-2 * abs(val) / 4.0, col
    if (lse_worst_case or few_keys) and dtype == "bf16":
        bound = lse_bound_bf16(inp.q, np.concatenate(inp.k, 1), oscale)
        assert (np.abs(lse.cpu().numpy() - lse_ref) <= bound).all()
    else:
        assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL[dtype]
    return ob, out


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64), ("fp32", 128)])
def test_single_query_single_key(F, dtype, D):
    say(f"edge: 1x1 {dtype} D={D}")
    _generic(F, 31, dtype, 1, 2, D, 1, (1,))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_ragged_everything(F, dtype, D):
    say(f"edge: ragged {dtype}")
    _generic(F, 32, dtype, 2, 3, D, 300, (1, 63, 64, 65, 130), q_block=64, center="compute",
             k_offset=2.0)


def test_supplied_centre_bf16(F):
    say("edge: supplied k_mean")
    _generic(F, 33, "bf16", 1, 4, 128, 513, (700, 300), q_block=128, center="supplied", k_offset=3.0)


def test_mixed_bodies_in_one_workgroup(F):
    """q_block 64 with a loud query block: four waves of one workgroup take different bodies."""
    say("edge: mixed bodies")
    ob, _ = _generic(F, 34, "bf16", 1, 2, 128, 256, (400, 300), q_block=64,
                     loud_rows=(0, 64, 128, 14.0))
    assert ob.elig.any() and not ob.elig.all()


def test_mixed_bodies_with_assembly_loop(F):
    """Long chunks (the fixed-m waves run the assembly main loop) next to online-softmax waves
    of the same workgroups: both bodies must meet at the same ring barriers."""
    say("edge: mixed bodies, long chunks")
    ob, _ = _generic(F, 39, "bf16", 1, 2, 128, 256, (1000, 737), q_block=64,
                     loud_rows=(1, 128, 192, 14.0))
    assert ob.elig.any() and not ob.elig.all()


def test_split_grid_tail(F):
    """37 heads x 8 query tiles = 296 tiles: on a 256-CU device the last 40 run as 6 key-range
    parts each.  In the per-chunk runs the first chunk (60 keys, 2 tiles) leaves parts 0, 1, 3
    and 4 of every split tile empty on the visit that initialises the workspace, and a loud
    query block puts online-softmax waves into split tiles (tail tiles belong to heads 32-36),
    so the finalize merges both kinds."""
    say("edge: split grid tail")
    ob, _ = _generic(F, 47, "bf16", 1, 37, 128, 2048, (60, 700, 1301), q_block=64,
                     loud_rows=(35, 0, 64, 14.0))
    assert ob.elig.any() and not ob.elig.all()


def test_split_part_without_keys_in_a_later_call(F):
    """The split grid tail again (37 heads x 8 query tiles: the last 40 tiles in 6 parts on a
    256-CU device), with a 60-key chunk (2 tiles) as the second of three per-chunk calls: parts
    0, 1, 3 and 4 of every split tile (key tiles [2 p / 6, 2 (p + 1) / 6)) get none in a call that continues the run,
    so they take their saved state and store it back unchanged; the result must still be the
    whole sequence's (loud rows put online-softmax waves into those parts too)."""
    say("edge: a split part with no keys in a continuing call")
    ob, _ = _generic(F, 48, "bf16", 1, 37, 128, 2048, (700, 60, 1301), q_block=64,
                     loud_rows=(35, 0, 64, 14.0))
    assert ob.elig.any() and not ob.elig.all()


@pytest.mark.parametrize("chunks", [
    (448, 480, 481),          # 14, 15 and 15 + 1 tiles: no assembly group, one group, one + partial
    (735, 0, 736, 1000),      # 22 and 23 full tiles (one / two groups) and an empty chunk
    (32 * (7 + 8 * 3) + 31,), # three groups and a 31-key last tile
])
def test_assembly_loop_boundaries(F, chunks):
    say(f"edge: assembly-loop boundaries {chunks}")
    _generic(F, 40 + len(chunks), "bf16", 1, 2, 128, 300, chunks, q_block=64, center="compute")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_no_reads_past_a_chunk(F, dtype):
    """Every chunk is a view into a larger buffer whose rows past the chunk are NaN: a load
    past a chunk's last key (or a misplaced last window) would put NaN into the output."""
    import torch
    say(f"edge: NaN past each chunk ({dtype})")
    chunks = (737, 1000, 481, 33)               # last tiles of 1, 8, 1 and 1 keys; fast groups
    D = 128
    inp = WL.generic_inputs(45, dtype, 1, 2, D, 200, chunks, q_block=64)
    q, ks, vs, _ = device_inputs(inp)
    kp, vp = [], []
    for k, v in zip(ks, vs):
        pad = 64
        kb = torch.full((1, k.shape[1] + pad, 2, D), float("nan"), device="cuda", dtype=k.dtype)
        vb = torch.full_like(kb, float("nan"))
        kb[:, :k.shape[1]] = k
        vb[:, :v.shape[1]] = v
        kp.append(kb[:, :k.shape[1]])
        vp.append(vb[:, :v.shape[1]])
    out, lse, desc, buf = F.forward(q, kp, vp, q_block=64, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    check_output(out.cpu().numpy(), ref, dtype)
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL[dtype]


def test_offsets_past_4gib(F):
    """A chunk whose key rows lie 16 KiB apart (a view of the first 2 of 64 NaN-filled heads),
    so its last keys sit past 4 GiB from its base, followed by a small chunk: every address
    the bounds and attention kernels form stays 64-bit, and no read leaves the view."""
    import torch
    say("edge: key offsets past 4 GiB (bf16)")
    chunks = (262_200, 1000)
    inp = WL.generic_inputs(63, "bf16", 1, 2, 128, 16, chunks, q_block=64, center="compute")
    q, ks, vs, _ = device_inputs(inp)
    big = []
    for t in (ks[0], vs[0]):
        pad = torch.full((1, chunks[0], 64, 128), float("nan"), device="cuda", dtype=t.dtype)
        pad[:, :, :2] = t
        big.append(pad[:, :, :2])
    del ks[0], vs[0]
    assert big[0].stride(1) * (chunks[0] - 1) * 2 >= 2**32
    ks.insert(0, big[0])
    vs.insert(0, big[1])
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, center="compute", out_dtype=torch.float32,
                                    want_lse=True)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=inp.wl.scale, q_block=64, center="compute", dtype="bf16")
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    check_output(out.cpu().numpy(), ref, "bf16")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["bf16"]


def test_v_magnitude_forces_fallback(F):
    say("edge: |v| > 256")
    ob, _ = _generic(F, 35, "bf16", 1, 2, 128, 200, (150, 100), q_block=64,
                     v_poke=(1, (0, 7, 1, 3), 300.0))
    assert not ob.v_ok and not ob.elig.any()


# (chunk, (b, key in chunk, h, d)) over 521 keys in chunks of 300 and 221: the first key,
# the first key of the second wave, the last key of a 256-key work item, the first and
# the last key of the second chunk, and the last key of the ragged tail.
V_POKES = [(0, (0, 0, 0, 0)), (0, (0, 64, 2, 5)), (0, (0, 255, 1, -1)), (1, (0, 0, 2, 3)),
           (1, (0, 211, 0, -1)), (1, (0, 220, 2, -1))]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64), ("fp32", 128)])
@pytest.mark.parametrize("val", [300.0, -258.0, float("nan"), 256.0, -256.0])
def test_v_check_anywhere(F, dtype, D, val):
    """One value row element set to val, at each of V_POKES in turn: the check fails for
    |val| > 256 and NaN and passes at exactly 256, wherever the element lies."""
    import torch
    say(f"edge: V check, {dtype} D={D}, v={val}")
    B, H, Sq, chunks = 1, 3, 100, (300, 221)
    p = F.make_problem(dtype, B, H, D, Sq, sum(chunks), 64)
    for c, (b0, j0, h0, d0) in V_POKES:
        inp = WL.generic_inputs(51, dtype, B, H, D, Sq, chunks, q_block=64)
        d0 = d0 % D
        if dtype == "bf16":
            inp.v_store[c][b0, j0, h0, d0] = WL.bf16_bits_from_f32(np.array([val], np.float32))[0]
        else:
            inp.v_store[c][b0, j0, h0, d0] = val
        q, ks, vs, _ = device_inputs(inp)
        desc, buf = F.bounds(p, q, ks, vs)
        torch.cuda.synchronize()
        ob = O.bounds(inp.q, inp.k, inp.v, scale=inp.wl.scale, q_block=64, dtype=dtype)
        assert ob.v_ok == (abs(val) <= 256.0), (c, j0, val)
        check_bounds(gpu_bounds_dict(desc, buf), ob)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_most_heads(F, dtype, D):
    """batch x heads at the ABI's maximum (3 x 21,845 = 65,535), one query row against two
    one-key chunks: every grid that spans batch x heads reaches its limit.  Two keys a row:
    bf16 output and lse are held to the per-element worst case of their arithmetic (over 8.4M
    outputs the rounding of a probability times |v| ~ 4 reaches ~0.016, and a logit's rounding
    moves lse by up to ~0.007)."""
    say(f"edge: 65,535 (batch, head) pairs ({dtype})")
    _generic(F, 61, dtype, 3, 21845, D, 1, (1, 1), q_block=64, few_keys=True)


def test_every_element_written_and_deterministic(F):
    import torch
    say("edge: NaN sentinel + determinism")
    inp = WL.generic_inputs(36, "bf16", 1, 5, 128, 700, (333, 444), q_block=64)
    q, ks, vs, _ = device_inputs(inp)
    N = 777
    p = F.make_problem("bf16", 1, 5, 128, 700, N, 64)
    outs = []
    for _ in range(2):
        desc, buf = F.bounds(p, q, ks, vs)
        ws = F.alloc_workspace(p, q.device)
        run = F.run_init(desc)
        for k, v in zip(ks, vs):
            F.attn_fwd(desc, run, q, [k], [v], ws)
        out = torch.full((1, 700, 5, 128), float("nan"), device="cuda")
        F.finalize(desc, run, ws, out)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])


def test_strided_layout_and_chunk_order(F):
    """[B, H, S, D]-strided views give the same result; chunk order changes only rounding."""
    import torch
    say("edge: strides + order")
    inp = WL.generic_inputs(37, "bf16", 1, 3, 128, 260, (100, 90, 70), q_block=64)
    q, ks, vs, _ = device_inputs(inp)
    base, _, _, _ = F.forward(q, ks, vs, q_block=64, out_dtype=torch.float32)
    qt = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)     # stride_s = D, stride_h = S*D
    kt = [k.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for k in ks]
    vt = [v.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for v in vs]
    o2, _, _, _ = F.forward(qt, kt, vt, q_block=64, out_dtype=torch.float32)
    assert torch.equal(base, o2)
    o3, _, _, _ = F.forward(q, ks[::-1], vs[::-1], q_block=64, out_dtype=torch.float32)
    assert (base - o3).abs().max().item() < 1e-5


def test_state_contracts(F):
    import torch
    say("edge: state contracts")
    inp = WL.generic_inputs(38, "bf16", 1, 2, 128, 64, (64, 64), q_block=64)
    q, ks, vs, _ = device_inputs(inp)
    p = F.make_problem("bf16", 1, 2, 128, 64, 128, 64)
    desc, buf = F.bounds(p, q, ks, vs)
    ws = F.alloc_workspace(p, q.device)
    run = F.run_init(desc)
    F.attn_fwd(desc, run, q, ks[:1], vs[:1], ws)
    out = torch.empty((1, 64, 2, 128), device="cuda")
    with pytest.raises(F.FixedmError) as e:
        F.finalize(desc, run, ws, out)                 # only half the keys visited
    assert e.value.status == -5
    # the C ABI itself rejects a workspace smaller than fixedm_workspace_bytes, before any launch
    import ctypes
    kk, vv, lens, nch = F._chunk_arrays(ks[1:], vs[1:])
    short = F.workspace_bytes(p) - 1
    assert F.lib().fixedm_attn_fwd(ctypes.byref(desc), ctypes.byref(run), F.tensor_desc(q), kk, vv, lens, nch,
                                   F._ptr(ws), short, F._stream(None)) == -1
    assert F.lib().fixedm_finalize(ctypes.byref(desc), ctypes.byref(run), F._ptr(ws), short,
                                   F.tensor_desc(out), F.F32, None, F._stream(None)) == -1
    assert run.kv_visited == 64
    run.kv_visited = 2**63 - 10                        # a forged count: rejected, no wrap-around
    with pytest.raises(F.FixedmError) as e:
        F.attn_fwd(desc, run, q, ks[1:], vs[1:], ws)
    assert e.value.status == -5
    run.kv_visited = 64
    F.attn_fwd(desc, run, q, ks[1:], vs[1:], ws)
    with pytest.raises(F.FixedmError) as e:
        F.attn_fwd(desc, run, q, ks[1:], vs[1:], ws)   # more keys than sk_total
    assert e.value.status == -5
    F.finalize(desc, run, ws, out)
    out16 = torch.empty((1, 64, 2, 128), device="cuda", dtype=torch.bfloat16)
    F.finalize(desc, run, ws, out16)                   # finalize again, other dtype
    torch.cuda.synchronize()
    assert torch.equal(out16, out.to(torch.bfloat16))
    other, _ = F.bounds(p, q, ks, vs)
    with pytest.raises(F.FixedmError) as e:
        F.attn_fwd(other, run, q, ks[:1], vs[:1], ws)  # run state of another descriptor
    assert e.value.status == -4
    desc.gate += 1                                     # a modified descriptor
    with pytest.raises(F.FixedmError) as e:
        F.run_init(desc)
    assert e.value.status == -4


# ------------------------------------------------------------------ fused final step --
# One fixedm_attn_fwd_final over every chunk: the accumulators stay in registers across the
# chunks and the whole query tiles write O and lse themselves.
FUSED = dict(chunks_per_call=8, fused_final=True)


def test_config3_fused_sampled_rows(F, cfg3):
    """The benchmark's launch configuration: bounds + fixedm_attn_fwd_final over the four ring
    chunks in rank 0's order (0, 3, 2, 1)."""
    say("config 3 output, fused final step over the 4 chunks")
    inp = cfg3
    out, lse, desc, buf, _ = _run(F, inp, order=(0, 3, 2, 1), **FUSED)
    check_bounds(gpu_bounds_dict(desc, buf), _oracle_bounds(inp))
    rows = _sample_rows(inp.wl.sq, 256)
    ref, lse_ref = O.attention_rows(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1),
                                    inp.wl.scale, rows)
    got = out.cpu().numpy()
    check_output(got[:, rows], ref, "bf16")
    assert np.abs(lse.cpu().numpy()[:, :, rows] - lse_ref).max() <= LSE_TOL["bf16"]
    assert np.isfinite(got).all()


def test_config2_fused(F):
    import torch
    say("config 2, fused final step")
    inp = WL.make_inputs(2)
    out, lse, desc, buf, dev = _run(F, inp, **FUSED)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    got = out.cpu().numpy()
    check_output(got, ref, "bf16")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["bf16"]
    # the fused bf16 output is the round-to-nearest-even of the fused fp32 output
    out16, _, _, _ = F.forward(dev[0], dev[1], dev[2], q_block=256, out_dtype=torch.bfloat16, **FUSED)
    bits = out16.cpu().view(torch.int16).numpy().view(np.uint16)
    assert_bf16_is_rne(bits, got)
    # per-chunk folds through the workspace: the same result up to fp32 summation order
    unfused, _, _, _ = F.forward(dev[0], dev[1], dev[2], q_block=256, out_dtype=torch.float32)
    assert np.abs(unfused.cpu().numpy() - got).max() <= 1e-5


@pytest.mark.parametrize("name,args,fwd", [
    ("ragged, all chunks fused", (32, "bf16", 2, 3, 128, 300, (1, 63, 64, 65, 130)),
     dict(center="compute", k_offset=2.0, **FUSED)),
    ("ragged, last chunk fused onto folds", (32, "bf16", 2, 3, 128, 300, (1, 63, 64, 65, 130)),
     dict(center="compute", k_offset=2.0, chunks_per_call=1, fused_final=True)),
    ("mixed bodies, long chunks", (39, "bf16", 1, 2, 128, 256, (1000, 737)),
     dict(loud_rows=(1, 128, 192, 14.0), **FUSED)),
    ("split tail, all chunks fused", (47, "bf16", 1, 37, 128, 2048, (60, 700, 1301)),
     dict(loud_rows=(35, 0, 64, 14.0), **FUSED)),
    ("split tail, two per call", (47, "bf16", 1, 37, 128, 2048, (60, 700, 1301)),
     dict(loud_rows=(35, 0, 64, 14.0), chunks_per_call=2, fused_final=True)),
    ("loop boundaries and an empty chunk", (44, "bf16", 1, 2, 128, 300, (735, 0, 736, 1000)),
     dict(center="compute", **FUSED)),
    ("single key", (31, "bf16", 1, 2, 128, 1, (1,)), FUSED),
    ("fp32 path", (32, "fp32", 2, 3, 64, 300, (1, 63, 64, 65, 130)),
     dict(center="compute", k_offset=2.0, **FUSED)),
])
def test_fused_and_multichunk_edges(F, name, args, fwd):
    say(f"fused: {name}")
    _generic(F, *args, **fwd)


def test_more_chunks_than_one_launch(F):
    """11 chunks in one call: launches of 8 and 3 chunks; the fused call folds the first 8 into
    the workspace and finishes with the last 3."""
    import torch
    say("fused: 11 chunks in one call")
    chunks = (100, 37, 0, 250, 64, 1, 33, 500, 129, 70, 300)
    for fwd in (dict(chunks_per_call=11), dict(chunks_per_call=11, fused_final=True)):
        ob, out = _generic(F, 48, "bf16", 1, 3, 128, 333, chunks, center="compute", **fwd)
        assert torch.isfinite(out).all()


def test_fused_state_sentinel_and_determinism(F):
    import torch
    say("fused: state contracts, NaN sentinel, determinism")
    inp = WL.generic_inputs(49, "bf16", 1, 5, 128, 700, (333, 444), q_block=64)
    q, ks, vs, _ = device_inputs(inp)
    p = F.make_problem("bf16", 1, 5, 128, 700, 777, 64)
    outs = []
    for _ in range(2):
        desc, buf = F.bounds(p, q, ks, vs)
        ws = F.alloc_workspace(p, q.device)
        run = F.run_init(desc)
        out = torch.full((1, 700, 5, 128), float("nan"), device="cuda")
        lse = torch.full((1, 5, 700), float("nan"), device="cuda")
        with pytest.raises(F.FixedmError) as e:
            F.attn_fwd_final(desc, run, q, ks[:1], vs[:1], ws, out, lse)   # keys missing
        assert e.value.status == -5
        F.attn_fwd_final(desc, run, q, ks, vs, ws, out, lse)
        assert run.finalized == 1 and run.kv_visited == 777
        with pytest.raises(F.FixedmError) as e:
            F.finalize(desc, run, ws, out)                                  # run already complete
        assert e.value.status == -5
        with pytest.raises(F.FixedmError) as e:
            F.attn_fwd(desc, run, q, ks[:1], vs[:1], ws)
        assert e.value.status == -5
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        outs.append((out, lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # all keys folded by fixedm_attn_fwd, then a fused call with no chunk: the finalize alone
    desc, buf = F.bounds(p, q, ks, vs)
    ws = F.alloc_workspace(p, q.device)
    run = F.run_init(desc)
    F.attn_fwd(desc, run, q, ks, vs, ws)
    out2 = torch.full((1, 700, 5, 128), float("nan"), device="cuda")
    F.attn_fwd_final(desc, run, q, [], [], ws, out2)
    ref = torch.full_like(out2, float("nan"))
    run2 = F.run_init(desc)
    F.attn_fwd(desc, run2, q, ks, vs, ws)
    F.finalize(desc, run2, ws, ref)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref)


# ------------------------------------------------------------------ per-row shifts ----
# One shift per query row (the per-query-row bound, in the same integer form): Q2, U and m
# per row bit-exact, eligibility per q-block as before, output within the same tolerances.
@pytest.mark.parametrize("cid", [1, 2, 4, 5])
def test_row_shift_configs(F, cid):
    say(f"per-row shift: config {cid}")
    inp = WL.make_inputs(cid)
    wl = inp.wl
    out, lse, desc, buf, _ = _run(F, inp, shift="row", **FUSED)
    ob = _oracle_bounds(inp, shift="row")
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert np.array_equal(ob.elig, _oracle_bounds(inp).elig)
    say(f"  m per row {ob.m_row.min()}..{ob.m_row.max()}, per block {ob.m.min()}..{ob.m.max()}")
    kall, vall = np.concatenate(inp.k, 1), np.concatenate(inp.v, 1)
    if cid == 4:
        rows = _sample_rows(wl.sq, 256)
        ref, lse_ref = O.attention_rows(inp.q, kall, vall, wl.scale, rows)
        got, lse_g = out.cpu().numpy()[:, rows], lse.cpu().numpy()[:, :, rows]
    else:
        ref, lse_ref = O.attention(inp.q, kall, vall, wl.scale)
        got, lse_g = out.cpu().numpy(), lse.cpu().numpy()
    check_output(got, ref, wl.dtype)
    assert np.abs(lse_g - lse_ref).max() <= LSE_TOL[wl.dtype]


@pytest.mark.parametrize("shift,q_block", [("row", 256), ("block", 18944)])
def test_config3_granularity_fused(F, cfg3, shift, q_block):
    """Config 3 in the benchmark's launch configuration with per-row shifts, and with one
    shift per head (q_block >= Sq)."""
    say(f"config 3 fused, shift={shift} q_block={q_block}")
    inp = cfg3
    out, lse, desc, buf, _ = _run(F, inp, order=(0, 3, 2, 1), q_block=q_block, shift=shift, **FUSED)
    ob = _oracle_bounds(inp, q_block=q_block, shift=shift)
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    assert ob.elig.all()
    rows = _sample_rows(inp.wl.sq, 256)
    ref, lse_ref = O.attention_rows(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1),
                                    inp.wl.scale, rows)
    check_output(out.cpu().numpy()[:, rows], ref, "bf16")
    assert np.abs(lse.cpu().numpy()[:, :, rows] - lse_ref).max() <= LSE_TOL["bf16"]


@pytest.mark.parametrize("name,args,kw", [
    ("ragged, centred", (32, "bf16", 2, 3, 128, 300, (1, 63, 64, 65, 130)),
     dict(center="compute", k_offset=2.0)),
    ("mixed bodies, long chunks", (39, "bf16", 1, 2, 128, 256, (1000, 737)),
     dict(loud_rows=(1, 128, 192, 14.0))),
    # rows with 4x the norm: their logits (and the bf16 rounding of alpha q in them) are 4x
    # larger, so lse is held to the worst-case bound of the bf16 arithmetic
    ("loud rows inside eligible blocks", (50, "bf16", 1, 2, 128, 320, (500, 333)),
     dict(q_block=128, loud_rows=(0, 70, 90, 4.0), lse_worst_case=True)),
    ("split tail", (47, "bf16", 1, 37, 128, 2048, (60, 700, 1301)),
     dict(loud_rows=(35, 0, 64, 14.0))),
    ("fp32 ragged", (32, "fp32", 2, 3, 64, 300, (1, 63, 64, 65, 130)),
     dict(center="compute", k_offset=2.0)),
])
def test_row_shift_edges(F, name, args, kw):
    say(f"per-row shift: {name}")
    for fwd in (dict(chunks_per_call=1), FUSED):
        _generic(F, *args, shift="row", **kw, **fwd)


# ------------------------------------------------------------------ degenerate inputs -
@pytest.mark.parametrize("mode", ["fused", "per_chunk"])
def test_online_fallback_with_huge_values_stays_finite(F, mode):
    """V elements of 2^110 (beyond the V bound: every block takes the online body) over 4096
    keys, whose scores are 0 in the first 32-key tile and about 7 (base 2) after it.  Exact
    online softmax keeps every probability <= 1 and sums to about 2^122; a reference allowed
    to lag 8 behind the row maximum would sum 2^7 per key and overflow fp32.  The V check
    records max|v| bit for bit, the body lets the reference lag at most
    127 - ceil(log2 N) - ceil(log2 max|v|) = 5, and the output is 2^110 as softmax's is."""
    import torch
    say(f"degenerate: |v| = 2^110 on the online body ({mode})")
    B, H, D, Sq, chunks = 1, 2, 128, 200, (2048, 2048)
    inp = WL.generic_inputs(57, "bf16", B, H, D, Sq, chunks, q_block=64)
    scale = O.default_scale(D)
    qf = np.zeros_like(inp.q)
    qf[..., 0] = 1.0
    ks, vs = [], []
    for c, n in enumerate(chunks):
        k = np.zeros((B, n, H, D), np.float32)
        k[:, 32 if c == 0 else 0:, :, 0] = 55.0            # alpha 55 = 7.01 with the default scale
        ks.append(k)
        vs.append(np.full((B, n, H, D), 2.0 ** 110, np.float32))
    inp.q_store = WL.bf16_bits_from_f32(qf)
    inp.k_store = [WL.bf16_bits_from_f32(k) for k in ks]
    inp.v_store = [WL.bf16_bits_from_f32(v) for v in vs]
    q, kd, vd, _ = device_inputs(inp)
    kw = FUSED if mode == "fused" else {}
    out, _, desc, buf = F.forward(q, kd, vd, q_block=64, out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    gb = gpu_bounds_dict(desc, buf)
    assert int(gb["v_bad"][0]) == int(np.float32(2.0 ** 110).view(np.int32))
    assert not gb["elig"].any()
    ref, _ = O.attention(qf, np.concatenate(ks, 1), np.concatenate(vs, 1), scale)
    assert np.allclose(ref, 2.0 ** 110, rtol=1e-12)
    got = out.cpu().numpy()
    assert np.isfinite(got).all(), "the online body overflowed"
    rel = np.abs(got / 2.0 ** 110 - 1.0).max()
    say(f"  max relative error {rel:.3e}")
    assert rel <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_nonfinite_query_takes_fallback(F, dtype):
    """An infinite query element makes its block's bound non-finite: the block is ineligible
    with m = INT32_MAX (bit-exact), takes the online body, and its poisoned row comes out
    non-finite as softmax's does; every other row matches the oracle."""
    import torch
    say(f"degenerate: inf in a query ({dtype})")
    D = 128 if dtype == "bf16" else 64
    inp = WL.generic_inputs(51, dtype, 1, 2, D, 200, (150, 170), q_block=64)
    qf = inp.q.copy()
    qf[0, 5, 1, 7] = np.inf
    inp.q_store = WL.bf16_bits_from_f32(qf) if dtype == "bf16" else qf
    q, ks, vs, _ = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, out_dtype=torch.float32, want_lse=True, **FUSED)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=inp.wl.scale, q_block=64, dtype=dtype)
    assert not ob.elig[0, 1, 0] and ob.m[0, 1, 0] == O.INT32_MAX and ob.elig[0, 0].all()
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, _ = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    got = out.cpu().numpy()
    assert not np.isfinite(ref[0, 5, 1]).any() and not np.isfinite(got[0, 5, 1]).any()
    keep = np.ones(got.shape[:3], bool)
    keep[0, 5, 1] = False
    check_output(got[keep], ref[keep], dtype, "O (other rows)")


@pytest.mark.parametrize("shift", ["block", "row"])
def test_zero_query_rows_give_the_mean_of_v(F, shift):
    """Query rows that are all zero: U = 0, m = -C, every key's exponent is exactly C, so the
    block stays eligible and its rows equal the mean of V (the textbook special case)."""
    import torch
    say(f"degenerate: zero query rows (shift={shift})")
    inp = WL.generic_inputs(52, "bf16", 1, 2, 128, 256, (300, 211), q_block=64, center="compute",
                            k_offset=2.0)
    qf = inp.q.copy()
    qf[0, 64:128, 0] = 0.0
    inp.q_store = WL.bf16_bits_from_f32(qf)
    q, ks, vs, _ = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, center="compute", out_dtype=torch.float32,
                                    want_lse=True, shift=shift, **FUSED)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=inp.wl.scale, q_block=64, center="compute", shift=shift)
    assert ob.elig.all() and ob.u[0, 0, 1] == 0.0 and ob.m[0, 0, 1] == -ob.C
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    mean_v = np.concatenate(inp.v, 1)[0, :, 0].astype(np.float64).mean(axis=0)
    got = out.cpu().numpy()
    assert np.abs(got[0, 64:128, 0] - mean_v[None, :]).max() <= 1e-5
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), inp.wl.scale)
    check_output(got, ref, "bf16")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["bf16"]


def test_combined_options(F):
    """Batch 2, five heads, q_block 192 (three waves' rows per block, blocks straddling
    workgroups), supplied centring on offset keys, per-row shifts, an empty and a one-key
    chunk, a loud block that falls back, all chunks in one fused call."""
    say("combined: B=2 H=5 q_block=192 supplied row-shift fused")
    ob, _ = _generic(F, 53, "bf16", 2, 5, 128, 700, (333, 0, 1200, 1, 47), q_block=192,
                     center="supplied", k_offset=3.0, loud_rows=(3, 192, 384, 14.0), shift="row",
                     **FUSED)
    assert ob.elig.any() and not ob.elig[:, 3, 1].any()


# A query row whose bound is exactly the gate at N = 4096 (C = 107, W = 232 even, gate 116)
# against keys k = -2^-10 q: in-order fp64 sums give Q2 * K2 = Q2^2 2^-20, so
# U = alpha * Q2 * 2^-10 = 116.0 exactly with alpha = fp32(1/sqrt(128)) log2 e.  These bf16
# components were found by a greedy search for that fp64 value (the test re-checks U).
GATE_EDGE_Q = [964.0, 47.0, 2.609375, 0.26953125, 0.031005859375, 0.0024261474609375,
               0.0002346038818359375, 1.52587890625e-05]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shift", ["block", "row"])
def test_bound_exactly_at_the_gate(F, dtype, shift):
    """The lower edge of the fixed-m window ([FM] Summary inequality: exponents >= C - (U +
    ceil U) >= -125).  With U = 116 = gate and m = ceil(U) - C = 9, every key of head 0 is
    anti-aligned with the loud query row at full norm, so that row's exponents all sit at
    C - 2 gate = -125 (on the bf16 path the rounding of alpha q moves a logit by at most 2^-8 of
    sum_d |alpha q_d k_d| = 116, to no lower than about -125.45: still a normal fp32).  The
    block's other rows are the loud row scaled by 2^-s (exponents from -125 up to -9) and a few
    N(0,1) rows.  The block is eligible, every probability is normal, and the output matches
    the oracle; the loud row, whose keys are identical, is the mean of V.  Head 1 holds
    ordinary N(0,1) data."""
    import torch
    say(f"edge: U exactly at the gate ({dtype}, shift={shift})")
    B, H, D, Sq, chunks = 1, 2, 128, 64, (2048, 2048)
    inp = WL.generic_inputs(71, dtype, B, H, D, Sq, chunks, q_block=64)
    qf, kf = inp.q.copy(), np.concatenate(inp.k, 1).copy()
    loud = np.zeros(D, np.float32)
    loud[:len(GATE_EDGE_Q)] = GATE_EDGE_Q
    for i in range(48):
        qf[0, i, 0] = loud * np.float32(2.0 ** -(i % 8))
    kf[0, :, 0] = -(2.0 ** -10) * loud
    store = (lambda x: WL.bf16_bits_from_f32(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    assert np.array_equal(WL.f32_from_bf16_bits(store(qf)) if dtype == "bf16" else qf, qf)
    inp.q_store = store(qf)
    inp.k_store = [np.ascontiguousarray(store(kf)[:, :2048]), np.ascontiguousarray(store(kf)[:, 2048:])]
    q, ks, vs, _ = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, out_dtype=torch.float32, want_lse=True,
                                    shift=shift, **FUSED)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(D), q_block=64, dtype=dtype, shift=shift)
    assert (ob.C, ob.W, ob.gate) == (107, 232, 116)
    assert ob.u[0, 0, 0] == 116.0 and ob.m[0, 0, 0] == 9 and ob.elig.all()
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), O.default_scale(D))
    got = out.cpu().numpy()
    mean_v = np.concatenate(inp.v, 1)[0, :, 0].astype(np.float64).mean(axis=0)
    say(f"  loud row vs mean of V: {np.abs(got[0, 0, 0] - mean_v).max():.3e}")
    check_output(got, ref, dtype)
    assert np.abs(got[0, 0, 0] - mean_v).max() <= (1e-3 if dtype == "bf16" else 5e-6)
    # Head 0's keys are identical, so a row's l is the fp32 sum of 4,096 equal terms, whose
    # rounding errors do not cancel: its relative error is bounded by (N - 1) 2^-24, and lse
    # = ln l + const moves by as much.  (The bf16 tolerance covers it already.)
    lse_tol = max(LSE_TOL[dtype], sum(chunks) * 2.0**-24 + 1e-5)
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= lse_tol


@pytest.mark.parametrize("dtype,D,scale", [("bf16", 128, 0.05), ("bf16", 128, 0.13), ("fp32", 64, 0.3)])
def test_explicit_softmax_scale(F, dtype, D, scale):
    """A softmax scale given by the caller (not the 1/sqrt(d) default): the descriptor holds
    its fp32 value and alpha = fp32(scale log2 e); bounds bit-exact, output within tolerance,
    on the fused and the per-chunk paths."""
    say(f"edge: softmax scale {scale} ({dtype})")
    _generic(F, 72, dtype, 1, 3, D, 300, (257, 190), q_block=64, scale=scale, **FUSED)
    _generic(F, 73, dtype, 1, 3, D, 300, (257, 190), q_block=128, scale=scale, center="compute",
             k_offset=2.0)


@pytest.mark.parametrize("fwd", [FUSED, dict(chunks_per_call=1)], ids=["fused", "per_chunk"])
def test_three_bodies_in_one_workgroup(F, fwd):
    """q_block 64 puts four blocks in one 256-row workgroup; the query rows of each are scaled
    so the waves take different bodies: U <= 32 (fixed-m assembly loop, logits from
    bf16(alpha q)), 32 < U <= gate (eligible, fixed-m with alpha applied in fp32), U > gate
    (online softmax), and U <= 32 again.  Loud eligible rows are where the bf16 rounding of
    alpha q would matter (a base-2 logit moves by up to 2^-8 U), so they are held to the
    flat bf16 tolerance like every other row.  Both heads, ragged Sq and chunk lengths."""
    import torch
    say(f"edge: three bodies in one workgroup ({'fused' if fwd is FUSED else 'per chunk'})")
    inp = WL.generic_inputs(74, "bf16", 1, 2, 128, 300, (700, 333), q_block=64)
    qf = inp.q.copy()
    for lo, fac in ((64, 4.5), (128, 8.0), (256, 4.0)):
        qf[0, lo:lo + 64] *= np.float32(fac)
    inp.q_store = WL.bf16_bits_from_f32(qf)
    q, ks, vs, _ = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, out_dtype=torch.float32, want_lse=True, **fwd)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(128), q_block=64, dtype="bf16")
    say(f"  U per block (head 0): {np.round(ob.u[0, 0], 2).tolist()}, gate {ob.gate}")
    u0 = ob.u[0, 0]
    assert u0[0] <= 32 and 32 < u0[1] <= ob.gate and u0[2] > ob.gate and u0[3] <= 32 < u0[4] <= ob.gate
    assert ob.elig[0, 0].tolist() == [True, True, False, True, True]
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    ref, lse_ref = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), O.default_scale(128))
    got = out.cpu().numpy()
    check_output(got, ref, "bf16")
    for lo, hi in ((64, 128), (256, 300)):
        say(f"  loud eligible rows {lo}..{hi}: max|d| {np.abs(got[0, lo:hi] - ref[0, lo:hi]).max():.2e}")
    assert np.abs(lse.cpu().numpy() - lse_ref).max() <= LSE_TOL["bf16"]


def _keys_wide(rng, shape, lo_exp, hi_exp, dtype):
    m = rng.uniform(1.0, 2.0, size=shape)
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    x = (rng.choice([-1.0, 1.0], size=shape) * np.ldexp(m, e)).astype(np.float32)
    return WL.bf16_bits_from_f32(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype,D,lo,hi", [("fp32", 64, -20, 20), ("fp32", 128, -60, 60),
                                           ("bf16", 128, -40, 40), ("fp32", 64, -149, -80)])
def test_key_mean_is_the_rounded_exact_sum(F, dtype, D, lo, hi):
    """COMPUTE centring on keys whose magnitudes span many binades (fp32 2^+-20 and 2^+-60,
    bf16 2^+-40, fp32 denormals): running fp64 sums of such keys round, so the key mean is
    defined as the exact sum rounded once to fp64, divided by N in fp64, rounded to fp32
    (every bit independent of summation order).  The GPU's slab partial sums detect the
    rounding and re-sum those elements exactly; k_mean, K2, U, m and the mask must equal the
    oracle's bit for bit.  Ragged chunks, several heads, batch 2."""
    import torch
    say(f"key mean: {dtype} D={D} keys 2^{lo}..2^{hi}")
    B, H, Sq, chunks = 2, 3, 70, (901, 77, 1500)
    inp = WL.generic_inputs(81, dtype, B, H, D, Sq, chunks, q_block=64, center="compute")
    rng = np.random.default_rng(82 + abs(lo))
    inp.k_store = [np.ascontiguousarray(_keys_wide(rng, (B, n, H, D), lo, hi, dtype)) for n in chunks]
    q, ks, vs, _ = device_inputs(inp)
    p = F.make_problem(dtype, B, H, D, Sq, sum(chunks), 64, 0.0, "compute")
    desc, buf = F.bounds(p, q, ks, vs)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(D), q_block=64, center="compute", dtype=dtype)
    # the case is meant to need the exact sum: a running fp64 sum differs from it somewhere
    run = np.zeros((B, H, D))
    for c in inp.k:
        for j in range(c.shape[1]):
            run += c[:, j].astype(np.float64)
    assert not np.array_equal(run, O.exact_sum_f64(inp.k))
    check_bounds(gpu_bounds_dict(desc, buf), ob)


def test_key_mean_fp32_gaussian_many_keys(F):
    """fp32 N(0,1) keys over 20,000 keys under COMPUTE centring (a running fp64 sum of these
    rounds for some elements); bounds bit-exact and the output within tolerance."""
    say("key mean: fp32 N(0,1), 20,000 keys")
    _generic(F, 83, "fp32", 1, 4, 64, 130, (12000, 8000), q_block=64, center="compute", k_offset=1.5)


def test_key_mean_nonfinite_keys(F):
    """A NaN key element, and an element holding both infinities, make that element's key
    mean NaN; one holding +inf only makes it +inf.  Those heads' K2, U are NaN and their
    blocks ineligible with m = INT32_MAX; the other heads are untouched (bit-exact)."""
    import torch
    say("key mean: non-finite keys")
    B, H, D, Sq, chunks = 1, 4, 64, 70, (300, 211)
    inp = WL.generic_inputs(84, "fp32", B, H, D, Sq, chunks, q_block=64, center="compute")
    k0, k1 = inp.k_store[0].copy(), inp.k_store[1].copy()
    k0[0, 3, 0, 5] = np.nan
    k0[0, 7, 1, 2], k1[0, 9, 1, 2] = np.inf, -np.inf
    k1[0, 200, 2, 9] = np.inf
    inp.k_store = [k0, k1]
    q, ks, vs, _ = device_inputs(inp)
    p = F.make_problem("fp32", B, H, D, Sq, sum(chunks), 64, 0.0, "compute")
    desc, buf = F.bounds(p, q, ks, vs)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(D), q_block=64, center="compute", dtype="fp32")
    assert np.isnan(ob.k_mean[0, 0, 5]) and np.isnan(ob.k_mean[0, 1, 2]) and ob.k_mean[0, 2, 9] == np.inf
    assert not ob.elig[0, :3].any() and ob.elig[0, 3].all()
    check_bounds(gpu_bounds_dict(desc, buf), ob)


def _bf16_keys_test(F, seed, chunks, make_keys, H=2, Sq=96, check_out=True):
    """bf16, COMPUTE centring, keys from make_keys(rng, shape) (fp32, rounded to bf16): the
    bounds (k_mean, K2, U, m, mask) bit-exact against the oracle, and the output within
    tolerance where check_out."""
    import torch
    B, D = 1, 128
    inp = WL.generic_inputs(seed, "bf16", B, H, D, Sq, chunks, q_block=64, center="compute")
    rng = np.random.default_rng(seed + 1000)
    k = make_keys(rng, (B, sum(chunks), H, D)).astype(np.float32)
    kb = WL.bf16_bits_from_f32(k)
    inp.k_store = [np.ascontiguousarray(c) for c in np.split(kb, np.cumsum(chunks)[:-1], axis=1)]
    q, ks, vs, _ = device_inputs(inp)
    out, lse, desc, buf = F.forward(q, ks, vs, q_block=64, center="compute", out_dtype=torch.float32,
                                    want_lse=True)
    torch.cuda.synchronize()
    ob = O.bounds(inp.q, inp.k, inp.v, scale=O.default_scale(D), q_block=64, center="compute", dtype="bf16")
    check_bounds(gpu_bounds_dict(desc, buf), ob)
    if check_out:
        ref, _ = O.attention(inp.q, np.concatenate(inp.k, 1), np.concatenate(inp.v, 1), O.default_scale(D))
        check_output(out.cpu().numpy(), ref, "bf16")
    return ob


def test_k2_keys_at_one_distance(F):
    """bf16 keys all at (nearly) the same distance from their mean, as RMS-normalised keys are:
    the largest centred norm is decided by the last bits of the fp64 sums; k_mean, K2, U, m and
    the mask bit-exact, the output within tolerance."""
    say("K2: keys at one distance from the mean")

    def keys(rng, shape):
        u = rng.standard_normal(shape)
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        return 0.5 + 8.0 * u

    _bf16_keys_test(F, 91, (9000, 7000), keys)


def test_k2_keys_with_a_shifted_first_part(F):
    """The first 2,048 keys sit 3 units above the rest in every dimension (a mean far from both
    groups, the largest centred norms in the first group): bounds bit-exact, output within
    tolerance."""
    say("K2: keys with a shifted first part")

    def keys(rng, shape):
        k = rng.standard_normal(shape)
        k[:, :2048] += 3.0
        return k

    _bf16_keys_test(F, 92, (3000, 2500), keys)


def test_k2_nonfinite_bf16_keys(F):
    """bf16 keys with a NaN (head 0) and an infinity (head 1) under COMPUTE centring: those
    heads' key means and K2 are not finite, as the oracle has them; head 2 is finite: bounds
    bit-exact, its blocks eligible."""
    say("K2: non-finite bf16 keys")

    def keys(rng, shape):
        k = rng.standard_normal(shape)
        k[0, 100, 0, 7] = np.nan
        k[0, 3000, 1, 40] = np.inf
        return k

    ob = _bf16_keys_test(F, 93, (2500, 1700), keys, H=3, check_out=False)
    assert not np.isfinite(ob.k2[0, 0]) and not np.isfinite(ob.k2[0, 1]) and np.isfinite(ob.k2[0, 2])
    assert ob.elig[0, 2].all()
