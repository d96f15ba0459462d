"""ctypes binding of libfixedm (include/fixedm.h): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI.  PyTorch is used
for device memory and streams.  If the library has not been built, or no GPU is present,
the calls fail loudly; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfixedm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fixedm.h")

ABI_VERSION = 2
BF16, F32 = 1, 2
CENTER = {"none": 0, "supplied": 1, "compute": 2}
SHIFT = {"block": 0, "row": 1}
STATUS = {
    0: "FIXEDM_OK", -1: "FIXEDM_ERR_INVALID_ARGUMENT", -2: "FIXEDM_ERR_UNSUPPORTED_DTYPE",
    -3: "FIXEDM_ERR_UNSUPPORTED_SHAPE", -4: "FIXEDM_ERR_BOUNDS_MISMATCH", -5: "FIXEDM_ERR_STATE",
    -6: "FIXEDM_ERR_HIP",
}


class FixedmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class Problem(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("sq", ctypes.c_int64),
                ("sk_total", ctypes.c_int64), ("q_block", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float), ("center", ctypes.c_int32),
                ("shift", ctypes.c_int32)]


class BoundsDesc(ctypes.Structure):
    _fields_ = [("p", Problem), ("log2_n", ctypes.c_int32), ("C", ctypes.c_int32),
                ("W", ctypes.c_int32), ("gate", ctypes.c_int32), ("n_qblocks", ctypes.c_int64),
                ("alpha", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("dev", ctypes.c_void_p), ("token", ctypes.c_uint64)]


class RunState(ctypes.Structure):
    _fields_ = [("token", ctypes.c_uint64), ("kv_visited", ctypes.c_int64),
                ("calls", ctypes.c_int32), ("finalized", ctypes.c_int32)]


class BoundsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("m", "elig", "u", "q2", "k2", "k_mean", "v_bad", "m_row", "q2_row", "u_row",
                 "scratch", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads dit_amd/libfixedm.so (built by dit_amd.build / __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m dit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.fixedm_status_string.restype = ctypes.c_char_p
    L.fixedm_status_string.argtypes = [ctypes.c_int]
    L.fixedm_constants.restype = ctypes.c_int
    L.fixedm_constants.argtypes = [ctypes.c_int64] + [P(ctypes.c_int32)] * 4
    L.fixedm_bounds_bytes.restype = ctypes.c_size_t
    L.fixedm_bounds_bytes.argtypes = [P(Problem)]
    L.fixedm_bounds_layout.restype = ctypes.c_int
    L.fixedm_bounds_layout.argtypes = [P(Problem), P(BoundsLayout)]
    L.fixedm_workspace_bytes.restype = ctypes.c_size_t
    L.fixedm_workspace_bytes.argtypes = [P(Problem)]
    L.fixedm_bounds.restype = ctypes.c_int
    L.fixedm_bounds.argtypes = [P(Problem), Tensor, P(Tensor), P(Tensor), P(ctypes.c_int64),
                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                P(BoundsDesc), ctypes.c_void_p]
    L.fixedm_bounds_static.restype = ctypes.c_int
    L.fixedm_bounds_static.argtypes = L.fixedm_bounds.argtypes
    L.fixedm_run_init.restype = ctypes.c_int
    L.fixedm_run_init.argtypes = [P(BoundsDesc), P(RunState)]
    L.fixedm_attn_fwd.restype = ctypes.c_int
    L.fixedm_attn_fwd.argtypes = [P(BoundsDesc), P(RunState), Tensor, P(Tensor), P(Tensor),
                                  P(ctypes.c_int64), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]
    L.fixedm_attn_fwd_final.restype = ctypes.c_int
    L.fixedm_attn_fwd_final.argtypes = [P(BoundsDesc), P(RunState), Tensor, P(Tensor), P(Tensor),
                                        P(ctypes.c_int64), ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                        Tensor, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    L.fixedm_finalize.restype = ctypes.c_int
    L.fixedm_finalize.argtypes = [P(BoundsDesc), P(RunState), ctypes.c_void_p, ctypes.c_size_t, Tensor,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    _lib = L
    return L


def declared_functions() -> list[str]:
    """Names of the functions include/fixedm.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(fixedm_[a-z_0-9]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != 0:
        raise FixedmError(status, where)


# ----------------------------------------------------------------------- host-only calls
def constants(n: int):
    L = lib()
    out = [ctypes.c_int32() for _ in range(4)]
    _check(L.fixedm_constants(n, *[ctypes.byref(o) for o in out]), "fixedm_constants")
    return tuple(o.value for o in out)


def make_problem(dtype, batch, heads, head_dim, sq, sk_total, q_block=256, softmax_scale=0.0,
                 center="none", shift="block") -> Problem:
    dt = {"bf16": BF16, "fp32": F32}.get(dtype, dtype)
    c = CENTER.get(center, center)
    sh = SHIFT.get(shift, shift)
    return Problem(ABI_VERSION, dt, batch, heads, head_dim, sq, sk_total, q_block,
                   softmax_scale, c, sh)


def bounds_bytes(p: Problem) -> int:
    return lib().fixedm_bounds_bytes(ctypes.byref(p))


def workspace_bytes(p: Problem) -> int:
    return lib().fixedm_workspace_bytes(ctypes.byref(p))


def bounds_layout(p: Problem) -> BoundsLayout:
    out = BoundsLayout()
    _check(lib().fixedm_bounds_layout(ctypes.byref(p), ctypes.byref(out)), "fixedm_bounds_layout")
    return out


# ----------------------------------------------------------------------- tensor helpers
def tensor_desc(t) -> Tensor:
    """fixedm_tensor for a torch tensor of shape [B, S, H, D] with stride 1 along D."""
    if t is None:
        return Tensor(None, 0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, S, H, D] tensor with a contiguous head_dim")
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _chunk_arrays(k_chunks, v_chunks):
    n = len(k_chunks)
    if len(v_chunks) != n:
        raise ValueError("k_chunks and v_chunks differ in length")
    KT, VT, LN = Tensor * max(n, 1), Tensor * max(n, 1), ctypes.c_int64 * max(n, 1)
    ks = KT(*[tensor_desc(k) for k in k_chunks])
    vs = VT(*[tensor_desc(v) for v in v_chunks])
    lens = LN(*[int(k.shape[1]) for k in k_chunks])
    return ks, vs, lens, n


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# The C ABI takes device buffers as bare pointers (their sizes are the caller's contract);
# the binding checks sizes and shapes against the problem before any call, so a PyTorch
# caller gets an exception instead of a launch that reads or writes past a buffer.
def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _need_bytes(t, nbytes: int, what: str):
    if t is None:
        raise ValueError(f"{what} is required")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes; the problem needs {nbytes}")


def _need_shape(t, shape, what: str):
    if t is None or tuple(t.shape) != tuple(shape):
        got = None if t is None else tuple(t.shape)
        raise ValueError(f"{what} has shape {got}; the problem needs {tuple(shape)}")


def _check_qkv(p: Problem, q, k_chunks, v_chunks):
    _need_shape(q, (p.batch, p.sq, p.heads, p.head_dim), "q")
    for i, (k, v) in enumerate(zip(k_chunks, v_chunks)):
        want = (p.batch, int(k.shape[1]), p.heads, p.head_dim)
        _need_shape(k, want, f"k_chunks[{i}]")
        _need_shape(v, want, f"v_chunks[{i}]")


def _check_out(p: Problem, out, lse):
    import torch
    _need_shape(out, (p.batch, p.sq, p.heads, p.head_dim), "out")
    if lse is not None:
        _need_shape(lse, (p.batch, p.heads, p.sq), "lse")
        if lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 tensor")


# ----------------------------------------------------------------------- device calls
def bounds(p: Problem, q, k_chunks, v_chunks, k_mean=None, buf=None, stream=None):
    """fixedm_bounds: returns (BoundsDesc, device buffer).  buf: optional uint8 CUDA tensor
    of at least bounds_bytes(p) bytes (256-byte aligned)."""
    import torch
    nbytes = bounds_bytes(p)
    if nbytes == 0:
        raise FixedmError(-1, "fixedm_bounds_bytes")
    if buf is None:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _need_bytes(buf, nbytes, "bounds buffer")
    _check_qkv(p, q, k_chunks, v_chunks)
    if p.center == CENTER["supplied"]:
        _need_shape(k_mean, (p.batch, p.heads, p.head_dim), "k_mean")
    ks, vs, lens, n = _chunk_arrays(k_chunks, v_chunks)
    desc = BoundsDesc()
    st = lib().fixedm_bounds(ctypes.byref(p), tensor_desc(q), ks, vs, lens, n, _ptr(k_mean),
                             _ptr(buf), _nbytes(buf), ctypes.byref(desc), _stream(stream))
    _check(st, "fixedm_bounds")
    return desc, buf


def bounds_static(p: Problem, q, k_chunks, v_chunks, k_mean=None, buf=None, stream=None):
    """fixedm_bounds_static: as bounds(), with the scratch in the library's static device
    array; buf needs only the output arrays (bounds_layout(p).scratch bytes)."""
    import torch
    nbytes = bounds_layout(p).scratch
    if buf is None:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _need_bytes(buf, nbytes, "bounds buffer")
    _check_qkv(p, q, k_chunks, v_chunks)
    if p.center == CENTER["supplied"]:
        _need_shape(k_mean, (p.batch, p.heads, p.head_dim), "k_mean")
    ks, vs, lens, n = _chunk_arrays(k_chunks, v_chunks)
    desc = BoundsDesc()
    st = lib().fixedm_bounds_static(ctypes.byref(p), tensor_desc(q), ks, vs, lens, n, _ptr(k_mean),
                                    _ptr(buf), _nbytes(buf), ctypes.byref(desc), _stream(stream))
    _check(st, "fixedm_bounds_static")
    return desc, buf


def run_init(desc: BoundsDesc) -> RunState:
    run = RunState()
    _check(lib().fixedm_run_init(ctypes.byref(desc), ctypes.byref(run)), "fixedm_run_init")
    return run


def attn_fwd(desc: BoundsDesc, run: RunState, q, k_chunks, v_chunks, workspace, stream=None):
    _check_qkv(desc.p, q, k_chunks, v_chunks)
    _need_bytes(workspace, workspace_bytes(desc.p), "workspace")
    ks, vs, lens, n = _chunk_arrays(k_chunks, v_chunks)
    st = lib().fixedm_attn_fwd(ctypes.byref(desc), ctypes.byref(run), tensor_desc(q), ks, vs,
                               lens, n, _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "fixedm_attn_fwd")


def attn_fwd_final(desc: BoundsDesc, run: RunState, q, k_chunks, v_chunks, workspace, out, lse=None,
                   stream=None):
    import torch
    dt = {torch.bfloat16: BF16, torch.float32: F32}[out.dtype]
    _check_qkv(desc.p, q, k_chunks, v_chunks)
    _need_bytes(workspace, workspace_bytes(desc.p), "workspace")
    _check_out(desc.p, out, lse)
    ks, vs, lens, n = _chunk_arrays(k_chunks, v_chunks)
    st = lib().fixedm_attn_fwd_final(ctypes.byref(desc), ctypes.byref(run), tensor_desc(q), ks, vs,
                                     lens, n, _ptr(workspace), _nbytes(workspace), tensor_desc(out), dt,
                                     _ptr(lse), _stream(stream))
    _check(st, "fixedm_attn_fwd_final")


def finalize(desc: BoundsDesc, run: RunState, workspace, out, lse=None, stream=None):
    import torch
    dt = {torch.bfloat16: BF16, torch.float32: F32}[out.dtype]
    _need_bytes(workspace, workspace_bytes(desc.p), "workspace")
    _check_out(desc.p, out, lse)
    st = lib().fixedm_finalize(ctypes.byref(desc), ctypes.byref(run), _ptr(workspace),
                               _nbytes(workspace), tensor_desc(out), dt, _ptr(lse), _stream(stream))
    _check(st, "fixedm_finalize")


def read_bounds(desc: BoundsDesc, buf) -> dict:
    """Views of the arrays fixedm_bounds wrote (device tensors sharing buf's memory)."""
    import torch
    p = desc.p
    lay = bounds_layout(p)
    bh, nqb, D = p.batch * p.heads, desc.n_qblocks, p.head_dim

    def view(off, n, dtype):
        width = torch.tensor([], dtype=dtype).element_size()
        return buf[off:off + n * width].view(dtype)

    rows = {}
    if p.shift == SHIFT["row"]:
        n = bh * p.sq
        rows = {
            "m_row": view(lay.m_row, n, torch.int32).view(p.batch, p.heads, p.sq),
            "q2_row": view(lay.q2_row, n, torch.float64).view(p.batch, p.heads, p.sq),
            "u_row": view(lay.u_row, n, torch.float64).view(p.batch, p.heads, p.sq),
        }
    return {
        **rows,
        "m": view(lay.m, bh * nqb, torch.int32).view(p.batch, p.heads, nqb),
        "elig": view(lay.elig, bh * nqb, torch.uint8).view(p.batch, p.heads, nqb),
        "u": view(lay.u, bh * nqb, torch.float64).view(p.batch, p.heads, nqb),
        "q2": view(lay.q2, bh * nqb, torch.float64).view(p.batch, p.heads, nqb),
        "k2": view(lay.k2, bh, torch.float64).view(p.batch, p.heads),
        "k_mean": view(lay.k_mean, bh * D, torch.float32).view(p.batch, p.heads, D),
        "v_bad": view(lay.v_bad, 1, torch.int32),
        "C": desc.C, "W": desc.W, "gate": desc.gate, "log2_n": desc.log2_n,
    }


def alloc_workspace(p: Problem, device):
    import torch
    return torch.empty(workspace_bytes(p), dtype=torch.uint8, device=device)


def forward(q, k_chunks, v_chunks, *, q_block=256, center="none", k_mean=None,
            softmax_scale=0.0, out_dtype=None, want_lse=False, chunks_per_call=1,
            fused_final=False, shift="block", stream=None):
    """The whole sequence for one rank: bounds, one fixedm_attn_fwd per ring step (each
    with `chunks_per_call` chunks), finalize; with `fused_final` the last step is
    fixedm_attn_fwd_final instead of fixedm_attn_fwd + fixedm_finalize.
    Returns (out, lse or None, desc, bounds buf)."""
    import torch
    B, Sq, H, D = q.shape
    dtype = {torch.bfloat16: "bf16", torch.float32: "fp32"}[q.dtype]
    N = sum(int(k.shape[1]) for k in k_chunks)
    p = make_problem(dtype, B, H, D, Sq, N, q_block, softmax_scale, center, shift)
    desc, buf = bounds(p, q, k_chunks, v_chunks, k_mean=k_mean, stream=stream)
    ws = alloc_workspace(p, q.device)
    run = run_init(desc)
    out = torch.empty((B, Sq, H, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if want_lse else None
    starts = list(range(0, len(k_chunks), chunks_per_call)) or [0]
    for i in starts:
        ks, vs = k_chunks[i:i + chunks_per_call], v_chunks[i:i + chunks_per_call]
        if fused_final and i == starts[-1]:
            attn_fwd_final(desc, run, q, ks, vs, ws, out, lse, stream=stream)
        else:
            attn_fwd(desc, run, q, ks, vs, ws, stream=stream)
    if not fused_final:
        finalize(desc, run, ws, out, lse, stream=stream)
    return out, lse, desc, buf
