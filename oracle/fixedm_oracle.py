"""Plain fp64 CPU oracle for fixed-m ("const-max") attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares no code,
header, table or constant generator with the HIP library under ``dit_amd/``, and it
imports nothing from it.  Every function is slow on purpose: no blocking, fusion or
reordering beyond what the cited definition states.

Sources (cited by title and section; the pages are the authority on what is computed):

  [CM]  "Kernel reference: ring_attention_const_max_fwd const-max ring attention"
        (AWS Neuron documentation page for Trainium2/3)
  [FM]  "feat(attention): fixed-m splash attention kernel with dynamic bounds and
        safety fallbacks" (maxdiffusion pull request #477)
  [UR]  "feat(attention): 2D Ulysses+Ring attention with Global Virtual K-Centering"
        (maxdiffusion pull request #478)

Layouts: q is [B, Sq, H, D]; each K/V chunk is [B, Sc, H, D] (token-major, as in the
[CM] Interface table).  All arithmetic is fp64 after an exact upcast of the inputs.

Readings taken where the pages leave a step open (listed again in the design doc):
  * exponent units: U bounds the argument of exp2, so U = alpha*||q||*||k|| with
    alpha = softmax_scale * log2(e)  (the base-2 logit rescale of [FM] Summary);
  * N is the total real KV length over all chunks (the ring length, unpadded);
  * Vmax = 256, so ceil(log2 Vmax) = 8 ([FM] review thread on the V check);
  * the gate test is inclusive: U <= gate;
  * q-blocks are consecutive runs of ``q_block`` real query rows; the last one is short;
  * sums over d run in index order (fp64);
  * k_mean is fp32(fl64(sum_j k_j) / N): the exact sum of the keys rounded once to fp64
    (so no summation order enters), the division in fp64, one rounding to fp32;
  * non-finite U: ineligible and m = INT32_MAX;
  * per-row shifts (the per-query-row bound of [CM]): m_i = ceil(U_i) - C(N) with
    U_i = alpha * sqrt(||q_i||^2 * K2); eligibility stays per q-block (every row of the
    block must pass the same gate, i.e. the block's loudest row decides).

Parity status: every public function below is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` (printed constants, closed forms, brute force, invariants).
The 0.882 softmax-mass figure of the [FM] gate discussion is *parity unpinned*: the pages
do not print the key set that produced it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "LOG2E", "VMAX", "INT32_MAX", "ceil_log2", "constants", "default_scale", "alpha_of",
    "Bounds", "exact_sum_f64", "k_mean_of", "bounds", "attention", "attention_rows", "attention_bruteforce",
    "fixed_m_emulate", "online_softmax_emulate", "method_forward", "max_shifted_exponent",
    "raw_key_unsound_case", "window_lower_edge", "softmax_mass",
]

LOG2E = 1.4426950408889634          # log2(e) to fp64 precision
VMAX = 256                          # DEFAULT_MAX_V_BOUND, [FM] review thread on the V check
INT32_MAX = 2**31 - 1


# --------------------------------------------------------------------------------------
# Constants  ([FM] Summary, "Dynamic eligibility bounding" equation)
# --------------------------------------------------------------------------------------
def ceil_log2(n: int) -> int:
    """ceil(log2 n) for an integer n >= 1, exactly (integer arithmetic, no float log)."""
    if n < 1:
        raise ValueError("ceil_log2 needs n >= 1")
    return (n - 1).bit_length()


def constants(n_keys: int, vmax: int = VMAX) -> tuple[int, int, int, int]:
    """(ceil(log2 N), C(N), W(N), gate) of [FM] Summary:

    C(N) = 127 - ceil(log2 N) - ceil(log2 Vmax);  W(N) = C(N) + 125;  gate = floor(W/2).
    The gate is floor(W/2) whatever the centring or ring mode ([FM] "Why the gate is halved").
    """
    L = ceil_log2(n_keys)
    C = 127 - L - ceil_log2(vmax)
    W = C + 125
    return L, C, W, W // 2


def default_scale(head_dim: int) -> float:
    """softmax_scale default 1/sqrt(d) ([CM] Interface table), rounded to fp32."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def alpha_of(scale: float) -> float:
    """Base-2 logit factor: the fp32 softmax scale, upcast, times log2(e), in fp64."""
    return float(np.float32(scale)) * LOG2E


# --------------------------------------------------------------------------------------
# Bounds: k_mean, Q/K norms, U, m, eligibility  ([FM] Summary; [UR] Summary;
# [CM] "Picking a max that is safe without measuring it")
# --------------------------------------------------------------------------------------
@dataclass
class Bounds:
    L: int
    C: int
    W: int
    gate: int
    n_keys: int
    k_mean: np.ndarray     # [B, H, D] float32 (zeros when centring is off)
    q2: np.ndarray         # [B, H, nQB] float64: max over the block's rows of sum_d q^2
    k2: np.ndarray         # [B, H] float64: max over all keys of sum_d (k - k_mean)^2
    u: np.ndarray          # [B, H, nQB] float64: alpha * sqrt(q2 * k2)
    m: np.ndarray          # [B, H, nQB] int64 (values fit int32): ceil(u) - C
    elig: np.ndarray       # [B, H, nQB] bool
    v_ok: bool
    v_absmax: float
    shift: str = "block"   # "block": one shift per (b, h, q-block); "row": one per query row
    q2_row: np.ndarray | None = None   # [B, H, Sq] float64: sum_d q_id^2 (shift == "row")
    u_row: np.ndarray | None = None    # [B, H, Sq] float64: alpha * sqrt(q2_row * k2)
    m_row: np.ndarray | None = None    # [B, H, Sq] int64: ceil(u_row) - C


_EXP_LO = -172          # every fp32 (hence bf16) value is an integer multiple of 2^-149; with
                        # frexp's 24-bit integer mantissas the lowest weight is 2^(-148-24)
_N_BINS = 104 + 24 - _EXP_LO + 1     # frexp exponents of fp32 values lie in [-148, 128]


def exact_sum_f64(k_chunks) -> np.ndarray:
    """sum_j k_j over the real keys of every chunk, as the fp64 number nearest the EXACT sum
    (round to nearest, ties to even), for bf16 / fp32 keys; [B, H, D].

    Each key element is an integer mantissa times a power of two (frexp: x = m 2^e,
    M = m 2^24 an integer below 2^24 in magnitude).  The integer mantissas are added per
    (element, exponent) in fp64, which is exact (fewer than 2^29 keys, so every such sum
    stays below 2^53); the bins are then combined as Python integers, exactly, and the
    integer is rounded once to fp64 (int to float conversion rounds to nearest, ties to
    even).  A NaN, or both infinities, give NaN; otherwise an infinity gives itself.
    Order of the keys plays no part: the sum is exact before its one rounding."""
    chunks = [np.asarray(c, dtype=np.float64) for c in k_chunks]
    B, _, H, D = chunks[0].shape
    E = B * H * D
    assert sum(c.shape[1] for c in chunks) < 2**29, "bin sums would leave the exact fp64 range"
    bins = np.zeros(E * _N_BINS, dtype=np.float64)
    any_nan = np.zeros(E, bool)
    pos_inf = np.zeros(E, bool)
    neg_inf = np.zeros(E, bool)
    elem = np.arange(E, dtype=np.int64)
    for c in chunks:
        for j in range(c.shape[1]):
            x = c[:, j].reshape(E)
            any_nan |= np.isnan(x)
            pos_inf |= x == np.inf
            neg_inf |= x == -np.inf
            fin = np.isfinite(x) & (x != 0.0)
            m, e = np.frexp(np.where(fin, x, 0.0))
            M = np.ldexp(m, 24)                      # integer-valued, |M| < 2^24
            assert np.array_equal(M, np.round(M)), "keys must be fp32-representable"
            idx = elem * _N_BINS + (e.astype(np.int64) - 24 - _EXP_LO)
            np.add.at(bins, idx[fin], M[fin])
    bins = bins.reshape(E, _N_BINS)
    out = np.empty(E, dtype=np.float64)
    for i in range(E):
        if any_nan[i] or (pos_inf[i] and neg_inf[i]):
            out[i] = np.nan
        elif pos_inf[i] or neg_inf[i]:
            out[i] = np.inf if pos_inf[i] else -np.inf
        else:
            total = 0
            for t in np.nonzero(bins[i])[0]:
                total += int(bins[i, t]) << int(t)   # exact: weight 2^(t + _EXP_LO)
            out[i] = math.ldexp(float(total), _EXP_LO) if total else 0.0
    return out.reshape(B, H, D)


def k_mean_of(k_chunks) -> np.ndarray:
    """Global virtual K-centring mean over the real keys of every chunk ([UR] Summary:
    the key mean is taken on real, unpadded tokens, the same for every ring step).

    The exact sum rounded once to fp64 (exact_sum_f64), one fp64 division by N, one
    round-to-nearest-even to fp32.  The pages do not fix a summation order; taking the sum
    exactly makes the mean independent of the order of chunks, keys and any partial sums
    (a running fp64 sum of fp32 keys over tens of thousands of keys is not exact)."""
    chunks = [np.asarray(c, dtype=np.float64) for c in k_chunks]
    n = sum(c.shape[1] for c in chunks)
    return (exact_sum_f64(chunks) / n).astype(np.float32)


def _rowsum_sq_in_order(x: np.ndarray) -> np.ndarray:
    """sum_d x[..., d]^2 accumulated in index order d = 0, 1, ..., D-1 (fp64)."""
    acc = np.zeros(x.shape[:-1], dtype=np.float64)
    for d in range(x.shape[-1]):
        acc += x[..., d] * x[..., d]
    return acc


def _shift_of(u: np.ndarray, C: int) -> np.ndarray:
    """m = ceil(u) - C as int64; INT32_MAX where u is not finite or m leaves int32."""
    finite = np.isfinite(u)
    m = np.full(u.shape, INT32_MAX, dtype=np.int64)
    m[finite] = np.ceil(u[finite]).astype(np.int64) - C
    return np.where((m > INT32_MAX) | (m < -INT32_MAX - 1), INT32_MAX, m)


def bounds(q, k_chunks, v_chunks, *, scale: float, q_block: int, center: str = "none",
           k_mean=None, dtype: str = "bf16", shift: str = "block") -> Bounds:
    """Per-(b, h, q-block) shift and eligibility ([FM] Summary equations).

    center: "none" (k_mean = 0), "supplied" (the given fp32 [B,H,D] mean) or "compute"
    (k_mean_of over all chunks).  Centred norms are used exactly when centring is on:
    the bound and the centring form a matched pair ([FM] "This PR is additive").

      U  = alpha * sqrt(Q2 * K2)            (Cauchy-Schwarz on the base-2 logit)
      m  = ceil(U) - C(N)
      elig = v_ok and dtype in {bf16, fp32} and U <= gate and U finite
    with v_ok = (max |v| <= 256), taken over the whole V ([FM] review thread on the
    V check; commit message, contract 2) and dtype safety from the same commit message.

    shift="row" adds the per-query-row bound of [CM] "Picking a max that is safe without
    measuring it" (the row's own norm times the largest key norm; Best practices, "Give each
    query row its own bound") in the same base-2, integer-shift form:
      U_i = alpha * sqrt(Q2_i * K2) with Q2_i = sum_d q_id^2,   m_i = ceil(U_i) - C(N).
    Row i's shifted exponents then lie in [C - U_i - ceil(U_i), C], so the gate condition is
    the same per row; the body is chosen per q-block, so eligibility stays the block's.
    """
    if shift not in ("block", "row"):
        raise ValueError(f"unknown shift granularity {shift!r}")
    q = np.asarray(q, dtype=np.float64)
    kc = [np.asarray(c, dtype=np.float64) for c in k_chunks]
    vc = [np.asarray(c, dtype=np.float64) for c in v_chunks]
    B, Sq, H, D = q.shape
    n = sum(c.shape[1] for c in kc)
    L, C, W, gate = constants(n)
    if center == "none":
        kbar = np.zeros((B, H, D), dtype=np.float32)
    elif center == "supplied":
        kbar = np.asarray(k_mean, dtype=np.float32).reshape(B, H, D)
    elif center == "compute":
        kbar = k_mean_of(kc)
    else:
        raise ValueError(f"unknown centring mode {center!r}")
    kbar64 = kbar.astype(np.float64)

    # K2[b,h] = max_j sum_d (k_jd - kbar_d)^2 over every real key of every chunk.
    k2 = np.zeros((B, H), dtype=np.float64)
    for c in kc:
        if c.shape[1] == 0:                              # an empty chunk has no keys
            continue
        diff = c - kbar64[:, None, :, :]                 # [B, Sc, H, D]
        k2 = np.maximum(k2, _rowsum_sq_in_order(diff).max(axis=1))

    # Q2[b,h,beta] = max over the real rows i of block beta of sum_d q_id^2.
    nqb = -(-Sq // q_block)
    qn = _rowsum_sq_in_order(q)                          # [B, Sq, H]
    q2 = np.zeros((B, H, nqb), dtype=np.float64)
    for beta in range(nqb):
        lo, hi = beta * q_block, min((beta + 1) * q_block, Sq)
        q2[:, :, beta] = qn[:, lo:hi, :].max(axis=1)

    alpha = alpha_of(scale)
    u = alpha * np.sqrt(q2 * k2[:, :, None])

    vabs = 0.0
    v_ok = True
    for c in vc:
        a = np.abs(c)
        if np.isnan(a).any():
            v_ok = False
            vabs = float("nan")
        elif a.size:
            vabs = max(vabs, float(a.max()))
    v_ok = v_ok and (vabs <= VMAX)
    dtype_ok = dtype in ("bf16", "fp32")

    finite = np.isfinite(u)
    m = _shift_of(u, C)
    elig = finite & (u <= gate) & v_ok & dtype_ok
    bnd = Bounds(L, C, W, gate, n, kbar, q2, k2, u, m, elig, bool(v_ok), vabs, shift)
    if shift == "row":
        bnd.q2_row = np.ascontiguousarray(qn.transpose(0, 2, 1))          # [B, H, Sq]
        bnd.u_row = alpha * np.sqrt(bnd.q2_row * k2[:, :, None])
        bnd.m_row = _shift_of(bnd.u_row, C)
    return bnd


# --------------------------------------------------------------------------------------
# The plain definition of the result: softmax attention over all N keys
# ([CM] "What you should know": the max exists for range only)
# --------------------------------------------------------------------------------------
def _attn_one_head(q, k, v, scale):
    """q [Sq, D], k/v [N, D] (fp64).  Returns O [Sq, D], lse [Sq] (natural log)."""
    s = float(np.float32(scale)) * (q @ k.T)
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    return o, mx[:, 0] + np.log(l)


def attention(q, k, v, scale: float, row_block: int = 512):
    """Exact non-causal softmax attention in fp64.

    q [B, Sq, H, D]; k, v [B, N, H, D] (all chunks concatenated).  Returns
    O [B, Sq, H, D] and lse [B, H, Sq] with lse_i = ln sum_j exp(scale * q_i . k_j)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.zeros((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = np.ascontiguousarray(k[b, :, h, :])
            vh = np.ascontiguousarray(v[b, :, h, :])
            for lo in range(0, Sq, row_block):
                hi = min(lo + row_block, Sq)
                o, ls = _attn_one_head(q[b, lo:hi, h, :], kh, vh, scale)
                out[b, lo:hi, h, :] = o
                lse[b, h, lo:hi] = ls
    return out, lse


def attention_rows(q, k, v, scale: float, rows):
    """Exact attention for a subset of query rows: returns O [B, len(rows), H, D] and
    lse [B, H, len(rows)].  Used for sampled checks at sizes too large to do in full."""
    q = np.asarray(q)[:, np.asarray(rows)]
    return attention(q, k, v, scale)


def attention_bruteforce(q, k, v, scale: float):
    """Textbook softmax attention with pure-Python loops and math.exp, for tiny inputs.
    Independent of numpy's linear algebra; nested lists or arrays accepted."""
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    B, Sq, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    N = len(k[0])
    s32 = float(np.float32(scale))
    out = [[[[0.0] * D for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for i in range(Sq):
            for h in range(H):
                logits = []
                for j in range(N):
                    dot = 0.0
                    for d in range(D):
                        dot += q[b][i][h][d] * k[b][j][h][d]
                    logits.append(s32 * dot)
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                tot = sum(w)
                for d in range(D):
                    out[b][i][h][d] = sum(w[j] * v[b][j][h][d] for j in range(N)) / tot
    return np.array(out)


def softmax_mass(q, k, scale: float, lse):
    """mass_i = sum_j exp(scale * q_i . k_j - lse_i) for one head: q [Sq, D], k [N, D],
    lse [Sq].  Equals 1 for every row when lse is the row's log-sum-exp."""
    s = float(np.float32(scale)) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    return np.exp(s - np.asarray(lse, np.float64)[:, None]).sum(axis=1)


# --------------------------------------------------------------------------------------
# Emulations of the two accumulation bodies (self-checks of the method)
# --------------------------------------------------------------------------------------
def fixed_m_emulate(q, k_chunks, v_chunks, *, scale: float, k_mean, m, C: int,
                    check_window: bool = True):
    """The eligible body for one (b, h, q-block) on one head ([FM] Summary; [CM] "A static
    bound makes the ring reduction pure addition", "Accumulate, then normalize once").

    q [R, D]; chunks [Sc, D] in visit order; k_mean [D]; integer shift m: one for the block,
    or an array of R per-row shifts.
    Per key j: e_ij = alpha * q_i . (k_j - k_mean) - m;  p = 2^e;  acc += p v_j;  l += p.
    The chunks merge by pure addition (the first visit initialises), then O = acc / l.
    Returns (O, lse, e_min, e_max) with lse = ln2 * (m + alpha q_i.k_mean + log2 l)."""
    alpha = alpha_of(scale)
    qa = alpha * np.asarray(q, dtype=np.float64)
    kbar = np.asarray(k_mean, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    m_col = m[:, None] if m.ndim == 1 else m
    acc = None
    l = None
    e_min, e_max = math.inf, -math.inf
    for kc, vc in zip(k_chunks, v_chunks):
        kc = np.asarray(kc, dtype=np.float64)
        vc = np.asarray(vc, dtype=np.float64)
        e = qa @ (kc - kbar).T - m_col
        if e.size:
            e_min = min(e_min, float(e.min()))
            e_max = max(e_max, float(e.max()))
        p = np.exp2(e)
        part_o = p @ vc
        part_l = p.sum(axis=1)
        if acc is None:           # first ring step initialises
            acc, l = part_o, part_l
        else:                     # later steps add, no rescaling
            acc = acc + part_o
            l = l + part_l
    if check_window:
        assert e_min >= -125.0, f"shifted exponent {e_min} below -125"
        assert e_max <= C, f"shifted exponent {e_max} above C={C}"
        assert np.all(np.abs(acc) < 2.0**127) and np.all(l < 2.0**127)
    o = acc / l[:, None]
    lse = math.log(2.0) * (m + qa @ kbar + np.log2(l))
    return o, lse, e_min, e_max


def online_softmax_emulate(q, k_chunks, v_chunks, *, scale: float, block: int = 64):
    """The fallback body: base-2 online softmax over KV blocks, state carried across the
    chunks ([UR] Summary "Cross-Ring Safety Fallback"; [CM] "Dropping the online max").

    Per block: r' = max(r, max_j z_ij); acc = acc 2^(r-r') + sum_j 2^(z_ij - r') v_j;
    l = l 2^(r-r') + sum_j 2^(z_ij - r'); r = r'.  Returns (O, lse)."""
    alpha = alpha_of(scale)
    qa = alpha * np.asarray(q, dtype=np.float64)
    R, D = qa.shape
    r = np.full(R, -np.inf)
    acc = np.zeros((R, D))
    l = np.zeros(R)
    for kc, vc in zip(k_chunks, v_chunks):
        kc = np.asarray(kc, dtype=np.float64)
        vc = np.asarray(vc, dtype=np.float64)
        for lo in range(0, kc.shape[0], block):
            z = qa @ kc[lo:lo + block].T
            r_new = np.maximum(r, z.max(axis=1))
            f = np.exp2(r - r_new)
            p = np.exp2(z - r_new[:, None])
            acc = acc * f[:, None] + p @ vc[lo:lo + block]
            l = l * f + p.sum(axis=1)
            r = r_new
    return acc / l[:, None], math.log(2.0) * (r + np.log2(l))


def method_forward(q, k_chunks, v_chunks, bnd: Bounds, *, scale: float, q_block: int,
                   block: int = 64):
    """The whole method on every (b, h, q-block): fixed-m body where eligible, the
    online-softmax body elsewhere, one final O / l.  Returns O [B,Sq,H,D], lse [B,H,Sq]
    and the list of (b, h, beta, e_min, e_max) for the eligible blocks."""
    q = np.asarray(q, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    windows = []
    for b in range(B):
        for h in range(H):
            kh = [np.asarray(c, np.float64)[b, :, h, :] for c in k_chunks]
            vh = [np.asarray(c, np.float64)[b, :, h, :] for c in v_chunks]
            for beta in range(-(-Sq // q_block)):
                lo, hi = beta * q_block, min((beta + 1) * q_block, Sq)
                qb = q[b, lo:hi, h, :]
                if bnd.elig[b, h, beta]:
                    shift = (bnd.m_row[b, h, lo:hi] if bnd.m_row is not None
                             else int(bnd.m[b, h, beta]))
                    o, ls, e0, e1 = fixed_m_emulate(qb, kh, vh, scale=scale,
                                                    k_mean=bnd.k_mean[b, h],
                                                    m=shift, C=bnd.C)
                    windows.append((b, h, beta, e0, e1))
                else:
                    o, ls = online_softmax_emulate(qb, kh, vh, scale=scale, block=block)
                out[b, lo:hi, h, :] = o
                lse[b, h, lo:hi] = ls
    return out, lse, windows


# --------------------------------------------------------------------------------------
# Soundness checks ([FM] Summary inequality; "This PR is additive"; "Why the gate is halved")
# --------------------------------------------------------------------------------------
def window_lower_edge(u: float, C: int) -> float:
    """Worst-case shifted exponent C - (U + ceil(U)) for a bound U ([FM] Summary)."""
    return C - (u + math.ceil(u))


def max_shifted_exponent(qa, keys_for_logits, u_bound: float, C: int):
    """Shift m = ceil(u_bound) - C is applied to the logits the kernel would really
    exponentiate, qa . key (qa already includes alpha).  Returns (max e, min e, verdict):
    'rejected' when some exponent exceeds C (2^e then no longer fits the accumulator's
    headroom; above 128 it overflows fp32 by itself) or falls below -125 (flush-risk)."""
    m = math.ceil(u_bound) - C
    e = np.asarray(qa, np.float64) @ np.asarray(keys_for_logits, np.float64).T - m
    emax, emin = float(e.max()), float(e.min())
    verdict = "accepted" if (emax <= C and emin >= -125.0) else "rejected"
    return emax, emin, verdict


def raw_key_unsound_case(n_keys: int = 4096, key_norm: float = 100.0):
    """The raw-key-bound counterexample of [FM] "This PR is additive": every key has norm
    100, so the raw bound is 100 (below the N=4096 gate of 116), but after centring one
    key's logit is about 200 and the raw-bound shift lets its exponent pass 2^128.

    Construction (along one unit direction u, base-2 units, ||alpha q|| = 1):
      n-1 keys = +key_norm*u, one key = -key_norm*u, alpha*q = -u.
    Returns a dict of the quantities the page states."""
    L, C, W, gate = constants(n_keys)
    u_dir = np.zeros(4)
    u_dir[0] = 1.0
    keys = np.tile(key_norm * u_dir, (n_keys, 1))
    keys[-1] = -key_norm * u_dir
    qa = (-u_dir)[None, :]
    kbar = keys.mean(axis=0)
    raw_u = 1.0 * np.linalg.norm(keys, axis=1).max()
    centred = keys - kbar
    centred_u = 1.0 * np.linalg.norm(centred, axis=1).max()
    emax, emin, verdict = max_shifted_exponent(qa, centred, raw_u, C)
    return {
        "C": C, "gate": gate, "raw_u": raw_u, "raw_passes_gate": raw_u <= gate,
        "centred_max_logit": float((qa @ centred.T).max()), "raw_shift": math.ceil(raw_u) - C,
        "max_exponent": emax, "verdict": verdict, "centred_u": centred_u,
        "centred_passes_gate": centred_u <= gate,
    }
