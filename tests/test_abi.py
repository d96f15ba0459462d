"""The C ABI without a GPU: the library loads, exports every declared function, and its
host logic (constants, sizes, argument validation) answers before any launch."""
import ctypes

import pytest

import oracle as O
from dit_amd import fixedm as F


@pytest.fixture(scope="module")
def L():
    return F.lib()


def test_exports_every_declared_function(L):
    names = F.declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code, name in F.STATUS.items():
        assert L.fixedm_status_string(code).decode() == name
    assert L.fixedm_status_string(17).decode() == "FIXEDM_UNKNOWN_STATUS"


@pytest.mark.parametrize("n", [1, 2, 3, 255, 256, 257, 4096, 37800, 75600, 2**31, 2**40 + 1])
def test_constants_match_oracle(n):
    assert F.constants(n) == O.constants(n)


def test_constants_rejects_nonpositive(L):
    assert L.fixedm_constants(0, None, None, None, None) == -1
    assert L.fixedm_constants(-5, None, None, None, None) == -1
    assert L.fixedm_constants(1, None, None, None, None) == 0


def _p(**kw):
    base = dict(dtype="bf16", batch=1, heads=40, head_dim=128, sq=18900, sk_total=75600,
                q_block=256, softmax_scale=0.0, center="compute")
    base.update(kw)
    return F.make_problem(**base)


def test_sizes_of_valid_problems():
    p = _p()
    lay = F.bounds_layout(p)
    offs = [lay.m, lay.elig, lay.u, lay.q2, lay.k2, lay.k_mean, lay.v_bad, lay.scratch, lay.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert F.bounds_bytes(p) == lay.total
    nqt = -(-18900 // 256)
    rows = 40 * nqt * 256
    ws = F.workspace_bytes(p)
    assert ws >= rows * (128 + 2) * 4 and ws % 256 == 0
    assert F.bounds_bytes(_p(dtype="fp32", head_dim=64, center="none")) > 0
    assert (lay.m_row, lay.q2_row, lay.u_row) == (lay.scratch,) * 3      # block mode: empty
    r = F.bounds_layout(_p(shift="row"))
    assert r.q2_row - r.m_row >= 40 * 18900 * 4 and r.u_row - r.q2_row >= 40 * 18900 * 8
    assert r.scratch - r.u_row >= 40 * 18900 * 8 and all(o % 256 == 0 for o in (r.m_row, r.q2_row, r.u_row))
    assert F.workspace_bytes(_p(shift="row")) == ws
    assert F.bounds_bytes(_p(batch=3, heads=21845, sq=1, sk_total=2, q_block=64)) > 0   # the most heads
    assert F.bounds_bytes(_p(sk_total=2**35)) > 0
    assert F.bounds_bytes(_p(dtype="fp32", head_dim=64, center="none", sk_total=2**38)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), -2),                      # fp16-like: no such dtype in the ABI
    (dict(dtype=0), -2),
    (dict(head_dim=64), -3),                  # bf16 path is head_dim 128
    (dict(dtype="fp32", head_dim=96), -3),
    (dict(q_block=100), -3),
    (dict(q_block=32), -3),
    (dict(q_block=0), -3),
    (dict(batch=0), -1),
    (dict(sq=-1), -1),
    (dict(sk_total=0), -1),
    (dict(center=5), -1),
    (dict(shift=2), -1),
    (dict(shift=-1), -1),
    (dict(softmax_scale=-0.1), -1),
    (dict(softmax_scale=float("nan")), -1),
    (dict(batch=2, heads=40000), -3),
    (dict(batch=1, heads=65536), -3),         # batch x heads above 65,535
    (dict(batch=2**40, heads=2**40), -3),     # no overflow in the product check
    (dict(sk_total=2**38 + 1), -3),
    (dict(sk_total=2**35 + 1), -3),           # bf16: a launch's key tiles are counted in 32 bits
])
def test_invalid_problems(kw, code):
    p = _p(**kw)
    assert F.bounds_bytes(p) == 0
    assert F.workspace_bytes(p) == 0
    with pytest.raises(F.FixedmError) as e:
        F.bounds_layout(p)
    assert e.value.status == code


@pytest.mark.parametrize("version", [1, F.ABI_VERSION + 1, 0])
def test_bad_abi_version(version):
    p = _p()
    p.abi_version = version
    assert F.bounds_bytes(p) == 0


def _call_bounds(L, p, q=None, kc=None, vc=None, lens=None, n=1, kmean=None, dev=0x10000,
                 out=True, nbytes=None):
    T = F.Tensor
    q = q if q is not None else T(0x20000, 0, 40 * 128, 128)
    kc = kc if kc is not None else (T * 1)(T(0x40000, 0, 40 * 128, 128))
    vc = vc if vc is not None else (T * 1)(T(0x80000, 0, 40 * 128, 128))
    lens = lens if lens is not None else (ctypes.c_int64 * 1)(p.sk_total)
    desc = F.BoundsDesc()
    nbytes = nbytes if nbytes is not None else max(F.bounds_bytes(p), 1)
    return L.fixedm_bounds(ctypes.byref(p), q, kc, vc, lens, n, kmean, dev, nbytes,
                           ctypes.byref(desc) if out else None, None)


def test_bounds_argument_errors_before_launch(L):
    p = _p(sk_total=1000, sq=100)
    T = F.Tensor
    assert _call_bounds(L, p, out=False) == -1                              # no descriptor
    assert _call_bounds(L, p, dev=0) == -1                                  # no buffer
    assert _call_bounds(L, p, dev=0x10010) == -1                            # buffer not 256-aligned
    assert _call_bounds(L, p, nbytes=F.bounds_bytes(p) - 1) == -1            # buffer too small
    assert _call_bounds(L, p, nbytes=0) == -1
    assert _call_bounds(L, p, q=T(0, 0, 5120, 128)) == -1                   # null q
    assert _call_bounds(L, p, q=T(0x20008, 0, 5120, 128)) == -3             # q not 16-aligned
    assert _call_bounds(L, p, q=T(0x20000, 0, 5121, 128)) == -3             # stride not 8-multiple
    # bf16 sequence strides up to 2^26 elements pass; beyond, the attention kernel's 32-bit
    # lane offsets (31 rows x stride x 2 bytes) could wrap, so the ABI rejects them
    assert _call_bounds(L, p, q=T(0x20000, 0, 2**26 + 8, 128)) == -3
    kbig = (T * 1)(T(0x40000, 0, 2**26 + 8, 128))
    assert _call_bounds(L, p, kc=kbig) == -3 and _call_bounds(L, p, vc=kbig) == -3
    # fp32 has no such limit: the same stride passes the tensor checks and the call fails
    # only later, on the chunk lengths that do not sum to sk_total
    assert _call_bounds(L, _p(dtype="fp32", head_dim=64, sk_total=1000, sq=100),
                        q=T(0x20000, 0, 2**26 + 8, 64), lens=(ctypes.c_int64 * 1)(999)) == -1
    assert _call_bounds(L, p, lens=(ctypes.c_int64 * 1)(999)) == -1         # sum != sk_total
    assert _call_bounds(L, p, lens=(ctypes.c_int64 * 1)(-1)) == -1
    big = 2**62                                                            # four lengths summing to
    kc4 = (T * 4)(*([T(0x40000, 0, 40 * 128, 128)] * 4))                  # 2^64 + 1000 would wrap
    lens4 = (ctypes.c_int64 * 4)(big, big, big, big + 1000)                # to sk_total
    assert _call_bounds(L, p, kc=kc4, vc=kc4, lens=lens4, n=4) == -1
    assert _call_bounds(L, p, lens=(ctypes.c_int64 * 1)(2**38 + 1)) == -1
    assert _call_bounds(L, p, n=0) == -1
    assert _call_bounds(L, p, n=33) == -3                                   # too many chunks
    ps = _p(sk_total=1000, sq=100, center="supplied")
    assert _call_bounds(L, ps) == -1                                        # k_mean missing
    assert _call_bounds(L, _p(dtype=3)) == -2


def test_forged_descriptor_is_rejected(L):
    d = F.BoundsDesc()
    run = F.RunState()
    assert L.fixedm_run_init(ctypes.byref(d), ctypes.byref(run)) == -4       # zeroed descriptor
    d.p = _p()
    d.dev = 0x10000
    d.token = 12345
    assert L.fixedm_run_init(ctypes.byref(d), ctypes.byref(run)) == -4       # token does not match
    T = F.Tensor
    kc = (T * 1)(T(0x40000, 0, 5120, 128))
    lens = (ctypes.c_int64 * 1)(10)
    big = 1 << 40
    assert L.fixedm_attn_fwd(ctypes.byref(d), ctypes.byref(run), T(0x20000, 0, 5120, 128), kc, kc,
                             lens, 1, 0x100000, big, None) == -4
    assert L.fixedm_finalize(ctypes.byref(d), ctypes.byref(run), 0x100000, big, T(0x20000, 0, 5120, 128),
                             1, None, None) == -4
    assert L.fixedm_attn_fwd_final(ctypes.byref(d), ctypes.byref(run), T(0x20000, 0, 5120, 128), kc, kc,
                                   lens, 1, 0x100000, big, T(0x20000, 0, 5120, 128), 1, None, None) == -4
    assert L.fixedm_attn_fwd_final(None, ctypes.byref(run), T(0x20000, 0, 5120, 128), kc, kc, lens, 1,
                                   0x100000, big, T(0x20000, 0, 5120, 128), 1, None, None) == -1
    assert L.fixedm_attn_fwd(None, ctypes.byref(run), T(0x20000, 0, 5120, 128), kc, kc, lens, 1,
                             0x100000, big, None) == -1


def test_binding_checks_sizes_and_shapes():
    """The C ABI takes bare device pointers; the binding rejects buffers smaller than the
    problem needs and tensors of the wrong shape before any call (CPU tensors suffice)."""
    import torch
    p = _p(sq=100, sk_total=1000)
    q = torch.empty((1, 100, 40, 128), dtype=torch.bfloat16)
    k = [torch.empty((1, 1000, 40, 128), dtype=torch.bfloat16)]
    with pytest.raises(ValueError, match="bounds buffer"):
        F.bounds(p, q, k, k, buf=torch.empty(16, dtype=torch.uint8))
    buf = torch.empty(F.bounds_bytes(p), dtype=torch.uint8)
    with pytest.raises(ValueError, match="q has shape"):
        F.bounds(p, q[:, :50], k, k, buf=buf)
    with pytest.raises(ValueError, match=r"k_chunks\[0\]"):
        F.bounds(p, q, [k[0][:, :, :20]], k, buf=buf)
    ps = _p(sq=100, sk_total=1000, center="supplied")
    with pytest.raises(ValueError, match="k_mean"):
        F.bounds(ps, q, k, k, k_mean=torch.empty(40, 128), buf=torch.empty(F.bounds_bytes(ps), dtype=torch.uint8))
    d = F.BoundsDesc()
    d.p = p
    run = F.RunState()
    with pytest.raises(ValueError, match="workspace"):
        F.attn_fwd(d, run, q, k, k, torch.empty(8, dtype=torch.uint8))
    ws = torch.empty(F.workspace_bytes(p), dtype=torch.uint8)
    out = torch.empty((1, 100, 40, 128), dtype=torch.float32)
    with pytest.raises(ValueError, match="out has shape"):
        F.finalize(d, run, ws, out[:, :10])
    with pytest.raises(ValueError, match="lse"):
        F.finalize(d, run, ws, out, lse=torch.empty((1, 40, 100), dtype=torch.float64))
    with pytest.raises(ValueError, match="workspace"):
        F.attn_fwd_final(d, run, q, k, k, torch.empty(8, dtype=torch.uint8), out)


def test_static_bounds_argument_errors_before_launch(L):
    """fixedm_bounds_static checks like fixedm_bounds, wants only the output arrays of the
    buffer, and rejects problems whose key-mean partial sums cannot fit its static array."""
    p = _p(sk_total=1000, sq=100)
    T = F.Tensor
    kc = (T * 1)(T(0x40000, 0, 40 * 128, 128))
    lens = (ctypes.c_int64 * 1)(1000)
    lay = F.bounds_layout(p)
    d = F.BoundsDesc()

    def call(p_, dev=0x10000, nbytes=lay.scratch, out=True, q=T(0x20000, 0, 40 * 128, 128), ln=lens):
        return L.fixedm_bounds_static(ctypes.byref(p_), q, kc, kc, ln, 1, None, dev, nbytes,
                                      ctypes.byref(d) if out else None, None)
    assert call(p, out=False) == -1 and call(p, dev=0) == -1 and call(p, dev=0x10010) == -1
    assert call(p, nbytes=lay.scratch - 1) == -1
    assert call(p, q=T(0x20008, 0, 5120, 128)) == -3
    assert call(p, ln=(ctypes.c_int64 * 1)(999)) == -1
    # 65,535 (batch, head) pairs x 128 dims: one slab of fp64 partial sums is 64 MiB
    big = _p(batch=3, heads=21845, sk_total=1000, sq=100)
    assert call(big, nbytes=F.bounds_layout(big).scratch) == -3
    assert call(_p(dtype=3)) == -2
