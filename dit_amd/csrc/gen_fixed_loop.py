"""Generates fixed_loop.inc: the steady-state fixed-m attention loop for gfx950 as one inline
assembly block with every value in a named register.

    python dit_amd/csrc/gen_fixed_loop.py      # run by dit_amd.build before compiling

Why assembly: one wave per SIMD must overlap the matrix cores with the vector ALUs.  The
exp2/convert/row-sum work of a 32-key tile is four to five VALU instructions per MFMA, and a
wave only hides them if they sit between its MFMAs; the compiler keeps the output
accumulator in VGPRs, runs out of registers for prefetched fragments, and bunches the VALU
work behind one half of the MFMAs.  Here the register classes and the instruction order
are fixed by hand:

  AGPR  a[0:127]    O^T accumulators o[n][m]      (n: 32-query tile, m: 32-dim tile)
        a[128:191]  resident query fragments q[n][kk] (pre-scaled by alpha, see below)
        a[192:223]  K fragments of the next tile
        a[224:255]  V^T fragments of even tiles
  VGPR  v[0:63]     S^T scores, double buffered by tile parity (v[32:63] holds the odd tiles)
        v[64:95]    packed bf16 probabilities P, double buffered (v[64:79] even tiles)
        v[96:127]   16 copies each of -(m + c_i) for the two query tiles: the initial
                    accumulator of the S MFMAs, so S arrives as the fixed-m exponent
        v[128:159]  V^T fragments of odd tiles
        v160-161    row sums l[n] (low bf16 halves);  v162-163  -(m + c_i) per query column
        v164-171    K fragment LDS addresses;  v172-175  V^T fragment LDS addresses
        v176-179    DMA lane offsets (K row 0/1, V row 0/1)
        v186-187    row sums of the high keys of each pair (folded into v160-161 when the
                    block ends)
  SGPR  s[60:61] next K tile address, s[62:63] next V tile address, s[64:65] / s[66:67]
        bytes between tiles, s68 this wave's LDS DMA base, s70 group count

The query fragments hold bf16(alpha q) (alpha = softmax scale x log2 e, applied in fp32 and
rounded once: the base-2 logit rescale of Q that the TPU path folds into Q's producer, in
"feat(attention): fixed-m splash attention kernel with dynamic bounds and safety
fallbacks", Summary, "Relayout optimization"), and c_i = (alpha q_i) . k_mean, so the exponent of the fixed-m body is
K (alpha Q)^T - (m + c_i): the MFMA chain starts from -(m + c_i) and the VALU work per score
is one exp2.

One step handles tile t (its stage in the 8-deep LDS ring is static inside the unrolled
group of 8 steps):
  wait for this wave's part of tile t+1, barrier; then 16 MFMAs O += V(t-1) P(t-1) and 16
  MFMAs S(t+1) = K(t+1) Q^T - (m + c), with the 80 VALU instructions that turn S(t) into
  P(t) and the row sums placed slot by slot (softmax_plan), the K(t+1) fragment reads and the DMA of tile
  t+6 (into the stage tile t-2 used) between the first PV MFMAs, and the 16 LDS transpose
  reads of V(t) (used next step) in the first half of the S MFMAs.

Measured choices (shader-clock cycles per step, s_memtime-instrumented builds on gfx950):
issuing the K reads and the DMA as a block after the barrier left the matrix cores idle
(-7.5% when spread between the MFMAs); summing the bf16 pairs with v_dot2c_f32_bf16 costs
~9 cycles of matrix-core time per instruction; adding the fp32 probabilities to the row sums
(two plain ops a pair) beats unpacking the bf16 pairs (four) only when every reader of an exp
sits two or more MFMA slots after it (a transcendental result arrives late: one slot behind
measured 1.6% slower than the unpacking, two slots behind 1.5% faster); the per-score
v_fma_f32 that applied alpha and the shift cost ~3 cycles each (-6.5% without it); one exp
per MFMA slot with the plain ops a slot or more behind (softmax_plan) instead of groups of
eight exps: -7.3% (1,485 -> 1,377 cycles a step).  Work-removal builds put the rest: without
any VALU work a step takes ~1,220 cycles, without the exps ~1,310; moving the transpose reads
next to the PV MFMAs or doubling up exps after the barrier costs 2-3%.

Hazards the assembler does not resolve are covered by construction and checked here:
  * a VALU read of an MFMA result (S) waits >= 12 wait states after the producing MFMA
    (16 enforced);
  * M0 written by SALU is followed by one wait state before the LDS DMA that reads it;
  * every register an LDS read or VALU op overwrites was last read by an MFMA at least one
    whole step earlier (double buffers), and every LDS read is waited for (lgkmcnt) before
    its value is used or the block ends;
  * the block starts and ends with 16 wait states so compiler code on either side sees no
    MFMA or VALU hazard across the boundary.
"""
from __future__ import annotations

import os
import sys

STAGES = 8
AHEAD = 6
TILE_BYTES = 8192
V_RING = STAGES * TILE_BYTES          # the V ring starts 64 KB into the shared buffer
# DMA instructions allowed in flight at a barrier: tile t+1 must have landed (one barrier per two
# steps, waiting for tiles t+1 and t+2 and loading t+6 and t+7 at even steps, measured 0.6% slower)
DMA_WAIT = (AHEAD - 2) * 4

O_BASE, Q_BASE, K_BASE, V0_ABASE = 0, 128, 192, 224
S_BASE, P_BASE, SHIFT_BASE, V1_VBASE = 0, 64, 96, 128
LSUM, NSHIFT, KOFF, VOFF, DMA = 160, 162, 164, 172, 176
# The DMA cursor, s[64:79], is loaded whole from a piece descriptor (one s_load_dwordx16):
S_D = 64
S_KT, S_VT, S_KTILE, S_VTILE, S_KLAST, S_VLAST = 64, 66, 68, 70, 72, 74
S_DREM, S_KSS, S_VSS, S_RSH = 76, 77, 78, 79
# The mask cursor, s[80:83], from the descriptor's mask fields (one s_load_dwordx4):
S_M = 80
S_MREM, S_LOLAST, S_LOBASE = 80, 81, 82
S_DPTR, S_MPTR, S_TMP = 84, 86, 88    # descriptor addresses of the two cursors; temporaries
S_TCNT, S_CNT, S_LO, S_LOPREV, S_FLAG, S_LDS = 90, 91, 92, 93, 94, 95
PIECE_BYTES = 128                     # one piece descriptor (32 dwords)
MASK_OFF = 64                         # byte offset of its mask fields
KB4, NEG_INF, MASK_X = 188, 189, 190      # 4 (lane / 32); -inf; mask / lane-offset temporary
ALPHA = 180                           # v180: alpha (fp32), the logit factor of the fp32a variant
LSUM_HI = 186                         # v186-v187: row sums of the high halves
ROW, CK, CV = 181, 183, (185, 191)    # this lane's tile rows (DMA instructions 0, 1) and the
                                      # byte offsets of its K and V chunks in those rows
# online variant: per query tile n a row-max / rescale-factor register A and a scratch B,
# the two tiles' growth masks (s96:97) and the accumulator-rescale flag (s98)
OA, OB = (192, 194), (193, 195)
S_GROW, S_RESC = 96, 98
S_SLACK = S_M + 3                     # s83, descriptor word 19: the running reference is raised
                                      # when a row max exceeds it by more than this (fp32, base 2)


def areg(base, n=1):
    return f"a{base}" if n == 1 else f"a[{base}:{base + n - 1}]"


def vreg(base, n=1):
    return f"v{base}" if n == 1 else f"v[{base}:{base + n - 1}]"


def o_reg(n, m):
    return areg(O_BASE + 16 * (4 * n + m), 16)


def q_reg(n, kk):
    return areg(Q_BASE + 32 * n + 4 * kk, 4)


def k_reg(buf, kk):
    # single buffer: K(t+1) is read after step t's barrier, when the S MFMAs of step t-1
    # (the last readers of K(t)) have long been issued
    return areg(K_BASE + 4 * kk, 4)


def s_first(buf, n):
    return S_BASE + 32 * buf + 16 * n


def p_first(buf, n):
    return P_BASE + 16 * buf + 8 * n


def v_frag(buf, st, m, half=None):
    """V^T fragment (st, m) of the tile parity `buf`: even tiles in AGPRs a[224:255], odd
    tiles in VGPRs v[128:159]; `half` selects the 2-register half one transpose read fills."""
    first = (V0_ABASE if buf == 0 else V1_VBASE) + 4 * (4 * st + m)
    mk = areg if buf == 0 else vreg
    return mk(first, 4) if half is None else mk(first + 2 * half, 2)


def shift_reg(n):
    """16 copies of -(m + c_i) for query tile n: the initial accumulator of the S MFMAs."""
    return vreg(SHIFT_BASE + 16 * n, 16)


# VALU slot plan of a step (one list entry per MFMA slot, 16 PV then 16 S slots):
#  * exps: one per slot, two in S slot 4 and none in the last slot, so the last pair's
#    convert and row-sum work still fits in the step;
#  * budget of plain VALU ops beside the exp: small in the slots that also carry the DMA /
#    K reads (PV slots 0-9) or the transpose reads (S slots 0-7), none beside two exps,
#    larger elsewhere; the last slot takes what is left.
EXP_QUOTA = [1] * 20 + [2] + [1] * 10 + [0]
SIMPLE_CAP = [1, 1, 1, 1, 3, 3, 3, 3, 3, 3, 4, 4, 4, 4, 4, 4, 2, 2, 2, 2, 0, 2, 2, 2, 4, 4, 4, 4, 4, 4, 4, 4]
# online variant: the first ONLINE_PRE slots hold the row maxima and the rescale test, so the 32
# exps go to the slots after them (two in five of those slots)
ONLINE_PRE = 4
ONLINE_EXP_QUOTA = [0] * ONLINE_PRE + [2 if s in (10, 14, 20, 25, 29) else 1 for s in range(ONLINE_PRE, 31)] + [0]
ONLINE_SIMPLE_CAP = [0] * ONLINE_PRE + [1, 1, 1, 1, 1, 1, 3, 3, 3, 3, 0, 3, 3, 3, 0, 3, 2, 2, 2, 2, 0, 2, 2,
                                         2, 2, 0, 4, 4]
DEP_DIST = 2                          # a plain VALU op sits >= 2 instructions after its producer
EXP_GAP = 2                           # ... and >= 2 MFMA slots after an exp it reads
BARRIER_AFTER = 2                     # PV MFMAs issued before a step's vmcnt wait and barrier
DMA_WITH_KREAD = True                 # a K fragment read between each M0 write and its DMA
                                      # (DMAs first with s_nop 0, K reads after: same speed)
V_TR_PER_SLOT, V_TR_FIRST = 2, 0      # V^T transpose reads per S MFMA slot, from this slot on
                                      # (one per slot over all 16, or two per slot in the second
                                      # half, measured 0.5-0.6% slower)


def softmax_plan(buf, online=False):
    """The 80 VALU instructions that turn S(t) (scores buffer `buf`) into P(t) and the row
    sums, placed into the 32 MFMA slots of a step.  Returns 32 lists of (text, whether the
    instruction reads the scores buffer).

    A v_exp_f32 holds the vector ALU for about half an MFMA, so at most one goes between two
    MFMAs (bunching them starves the matrix cores: -7% cycles a step for this plan against
    groups of exps).  Each bf16 pair (word) w of P takes 2 exps, then v_cvt_pk_bf16_f32 and
    two row-sum adds of the fp32 exps.  A consumer of an exp goes EXP_GAP or more slots later
    (the last slot takes what is left, one slot behind); other consumers go >= DEP_DIST
    instructions after their producer, and the low and high keys of a pair add into separate
    accumulators so that the adds of one slot do not depend on each other."""
    ops = []          # dicts: text, reads (scores buffer), deps, war, acc

    def add(text, reads, deps=(), war=(), acc=None):
        ops.append(dict(text=text, reads=reads, deps=list(deps), war=list(war), acc=acc))
        return len(ops) - 1

    exps, word_exps = [], []
    for w in range(16):
        n, i = w % 2, w // 2                     # word w: tile n, S registers 2i, 2i+1
        x = s_first(buf, n) + 2 * i
        pair = [add(f"v_exp_f32 v{r}, v{r}", True) for r in (x, x + 1)]
        exps += pair
        word_exps.append(pair)
    plain = []
    for w in range(16):
        n, i = w % 2, w // 2
        x = s_first(buf, n) + 2 * i
        pw = p_first(buf, n) + i
        cvt = add(f"v_cvt_pk_bf16_f32 v{pw}, v{x}, v{x + 1}", True, word_exps[w])
        a_lo = add(f"v_add_f32 v{LSUM + n}, v{LSUM + n}, v{x}", True, [word_exps[w][0]], acc=LSUM + n)
        a_hi = add(f"v_add_f32 v{LSUM_HI + n}, v{LSUM_HI + n}, v{x + 1}", True, [word_exps[w][1]],
                   acc=LSUM_HI + n)
        plain += [cvt, a_lo, a_hi]

    pos = {}                                      # op -> (slot, index in the slot)
    last_acc = {}
    plan = [[] for _ in range(32)]
    ei, pending = 0, list(plain)
    quota, caps = (ONLINE_EXP_QUOTA, ONLINE_SIMPLE_CAP) if online else (EXP_QUOTA, SIMPLE_CAP)
    assert len(quota) == 32 and len(caps) == 32 and sum(quota) == 32
    for s in range(32):
        for _ in range(quota[s]):
            pos[exps[ei]] = (s, len(plan[s]))
            plan[s].append(exps[ei])
            ei += 1
        cap = caps[s] if s < 31 else len(pending)
        dist = DEP_DIST if s < 31 else 1
        took = 0
        while took < cap:
            pick = None
            for k in pending:
                o = ops[k]
                ok = True
                for d in o["deps"] + o["war"]:
                    if d not in pos:
                        ok = False
                        break
                    ds, di = pos[d]
                    if ops[d]["text"].startswith("v_exp") and s - ds < (EXP_GAP if s < 31 else 1):
                        ok = False
                        break
                    if ds == s and len(plan[s]) - di < dist:
                        ok = False
                        break
                if ok and o["acc"] in last_acc:
                    ls, li = last_acc[o["acc"]]
                    ok = not (ls == s and len(plan[s]) - li < dist)
                if ok:
                    pick = k
                    break
            if pick is None:
                break
            pos[pick] = (s, len(plan[s]))
            plan[s].append(pick)
            pending.remove(pick)
            took += 1
            if ops[pick]["acc"] is not None:
                last_acc[ops[pick]["acc"]] = pos[pick]
    assert ei == 32 and not pending, "VALU plan does not fit the step"
    return [[(ops[k]["text"], ops[k]["reads"]) for k in sl] for sl in plan]


class Emitter:
    """Collects the instruction lines and pads VALU reads of MFMA-written score registers.

    Forward branches (branch() to a label placed later with label()) merge the hazard state:
    at the label each score buffer counts as written as recently as on any path that reaches
    it.  A loop head (loop_head()) is reached by a back edge, so the tracking restarts there
    as if an MFMA had just written both buffers."""

    MIN_WAIT = 16

    def __init__(self):
        self.lines = []
        self.count = 0                          # instructions emitted (each >= 1 wait state)
        self.s_written = {0: -10**9, 1: -10**9}  # index of the last MFMA writing each S buffer
        self.pending = {}                       # forward label -> wait-state distances at branches
        self.n_labels = 0
        self.deferred = []                      # out-of-line blocks, emitted after the epilogue

    def emit(self, text, reads_sbuf=None, writes_sbuf=None):
        if reads_sbuf is not None:
            gap = self.count - self.s_written[reads_sbuf] - 1
            if gap < self.MIN_WAIT:
                self.lines.append(f"s_nop {self.MIN_WAIT - gap - 1}")
                self.count += self.MIN_WAIT - gap
        self.lines.append(text)
        if writes_sbuf is not None:
            self.s_written[writes_sbuf] = self.count
        self.count += 1

    def new_label(self):
        self.n_labels += 1
        return f"L_fixedm_f{self.n_labels}_%="

    def branch(self, op, label):
        self.emit(f"{op} {label}")
        self.pending.setdefault(label, []).append({b: self.count - w for b, w in self.s_written.items()})

    def label(self, label):
        for dist in self.pending.pop(label, []):
            for b in (0, 1):
                self.s_written[b] = max(self.s_written[b], self.count - dist[b])
        self.lines.append(f"{label}:")

    def loop_head(self, label):
        self.lines.append(f"{label}:")
        self.s_written = {0: self.count - 1, 1: self.count - 1}

    def seq(self, items):
        """Emits a list of instructions, ("branch", op, label) and ("label", label) items."""
        for it in items:
            if isinstance(it, tuple):
                if it[0] == "branch":
                    self.branch(it[1], it[2])
                else:
                    self.label(it[1])
            else:
                self.emit(it)


def lane_offsets():
    """The DMA lane offsets of the DMA cursor's piece: row = max(row_i - rshift, 0) (rshift > 0
    only for a chunk shorter than a tile, whose keys then fill the tile's last rows), offset
    = row x row stride + this lane's 16-byte chunk in the row."""
    out = []
    for i in range(2):
        out += [f"v_subrev_u32 v{MASK_X}, s{S_RSH}, v{ROW + i}",
                f"v_max_i32 v{MASK_X}, 0, v{MASK_X}",
                f"v_mul_lo_u32 v{DMA + i}, v{MASK_X}, s{S_KSS}",
                f"v_add_u32 v{DMA + i}, v{DMA + i}, v{CK + i}",
                f"v_mul_lo_u32 v{DMA + 2 + i}, v{MASK_X}, s{S_VSS}",
                f"v_add_u32 v{DMA + 2 + i}, v{DMA + 2 + i}, v{CV[i]}"]
    return out


def stale_offsets(e):
    """Recomputes the lane offsets if the DMA cursor has moved to another piece since they
    were formed (s[S_FLAG] set; the descriptor load has been waited for)."""
    lab = e.new_label()
    return ([f"s_cmp_eq_u32 s{S_FLAG}, 0", ("branch", "s_cbranch_scc1", lab)] + lane_offsets()
            + [f"s_mov_b32 s{S_FLAG}, 0", ("label", lab)])


def dma_issue(stage):
    """The four DMA instructions of this wave's share of a tile into LDS stage `stage`, each
    after its M0 write (an instruction goes between them: the wait state M0 needs)."""
    out = []
    for i in range(2):
        for base, vreg_i, sreg in ((stage * TILE_BYTES, DMA + i, S_KT),
                                    (V_RING + stage * TILE_BYTES, DMA + 2 + i, S_VT)):
            out.append([f"s_add_u32 m0, s{S_LDS}, {base + 1024 * i}", None,
                        f"global_load_lds_dwordx4 v{vreg_i}, s[{sreg}:{sreg + 1}]"])
    return out


ADVANCE = [[f"s_add_u32 s{S_KT}, s{S_KT}, s{S_KTILE}", f"s_addc_u32 s{S_KT + 1}, s{S_KT + 1}, s{S_KTILE + 1}"],
           [f"s_add_u32 s{S_VT}, s{S_VT}, s{S_VTILE}", f"s_addc_u32 s{S_VT + 1}, s{S_VT + 1}, s{S_VTILE + 1}"]]
LAST_WINDOW = [f"s_cselect_b64 s[{S_KT}:{S_KT + 1}], s[{S_KLAST}:{S_KLAST + 1}], s[{S_KT}:{S_KT + 1}]",
               f"s_cselect_b64 s[{S_VT}:{S_VT + 1}], s[{S_VLAST}:{S_VLAST + 1}], s[{S_VT}:{S_VT + 1}]"]


def dma_advance(e):
    """After a DMA in a step that may reach a piece's end: the next tile's addresses, the
    piece's last window for its last tile, and at the piece's end the next descriptor (its
    values are used from the next step on, after that step's lgkmcnt wait)."""
    lab = e.new_label()
    return [list(ADVANCE[0]), list(ADVANCE[1]),
            [f"s_sub_u32 s{S_DREM}, s{S_DREM}, 1", f"s_cmp_eq_u32 s{S_DREM}, 1"] + LAST_WINDOW,
            [f"s_cmp_lg_u32 s{S_DREM}, 0", ("branch", "s_cbranch_scc1", lab),
             f"s_add_u32 s{S_DPTR}, s{S_DPTR}, {PIECE_BYTES}", f"s_addc_u32 s{S_DPTR + 1}, s{S_DPTR + 1}, 0",
             f"s_load_dwordx16 s[{S_D}:{S_D + 15}], s[{S_DPTR}:{S_DPTR + 1}], 0x0",
             f"s_mov_b32 s{S_FLAG}, 1", ("label", lab)]]


def mask_step(e: Emitter, fp32a: bool):
    # fp32a: the S chain starts from 0 (the fp32-factor and online variants)
    """The initial accumulator of the next S tile: -(m + c_i) (0 in fp32a) for its real keys and
    -inf for the rest.  Real keys sit in rows >= lo: lo = the piece's lo_last for its last tile
    (32 - rem for a partial last tile), lo_base for the others (0; 32 past the last piece).  The
    32 initial-value registers are rewritten only when lo changes."""
    l_next, l_same = e.new_label(), e.new_label()
    e.emit(f"s_cmp_eq_u32 s{S_MREM}, 1")
    e.emit(f"s_cselect_b32 s{S_LO}, s{S_LOLAST}, s{S_LOBASE}")
    e.emit(f"s_sub_u32 s{S_MREM}, s{S_MREM}, 1")
    e.emit(f"s_cmp_lg_u32 s{S_MREM}, 0")
    e.branch("s_cbranch_scc1", l_next)
    e.emit(f"s_add_u32 s{S_MPTR}, s{S_MPTR}, {PIECE_BYTES}")
    e.emit(f"s_addc_u32 s{S_MPTR + 1}, s{S_MPTR + 1}, 0")
    e.emit(f"s_load_dwordx4 s[{S_M}:{S_M + 3}], s[{S_MPTR}:{S_MPTR + 1}], {MASK_OFF}")
    e.label(l_next)
    e.emit(f"s_cmp_eq_u32 s{S_LO}, s{S_LOPREV}")
    e.branch("s_cbranch_scc1", l_same)
    e.emit(f"s_mov_b32 s{S_LOPREV}, s{S_LO}")
    e.emit(f"v_sub_u32 v{MASK_X}, s{S_LO}, v{KB4}")         # lo - 4 (lane / 32)
    for r in range(16):
        key = 8 * (r >> 2) + (r & 3)                          # row of register r, lane half 0
        e.emit(f"v_cmp_lt_i32_e32 vcc, {key}, v{MASK_X}")
        for n in range(2):
            init = "0" if fp32a else f"v{NSHIFT + n}"
            e.emit(f"v_cndmask_b32_e32 v{SHIFT_BASE + 16 * n + r}, {init}, v{NEG_INF}, vcc")
    e.emit("s_nop 1")
    e.label(l_same)


def online_pre(cur):
    """Online variant, per query tile n: the row maximum of S(t) over the tile's 32 keys (16 in
    this lane, 16 in lane ^ 32, exchanged by v_permlane32_swap), scaled by alpha, and the test
    alpha max > r + slack (r = -NSHIFT, the running reference; slack in s[S_SLACK]); the two tiles' tests
    are or-ed into s[S_GROW].  Four lists, one per leading MFMA slot; each entry is (text,
    whether it reads the scores buffer)."""
    groups = []
    for n in range(2):
        x, a, b = s_first(cur, n), OA[n], OB[n]
        chain = [(f"v_max3_f32 v{a}, v{x}, v{x + 1}, v{x + 2}", True)]
        for i in range(3, 15, 2):
            chain.append((f"v_max3_f32 v{a}, v{a}, v{x + i}, v{x + i + 1}", True))
        chain.append((f"v_max_f32 v{a}, v{a}, v{x + 15}", True))
        tail = [(f"v_mov_b32 v{b}, v{a}", False), ("s_nop 1", False),
                (f"v_permlane32_swap_b32 v{a}, v{b}", False), ("s_nop 1", False),
                (f"v_max_f32 v{a}, v{a}, v{b}", False),
                (f"v_mul_f32 v{a}, v{a}, v{ALPHA}", False),
                (f"v_add_f32 v{b}, v{a}, v{NSHIFT + n}", False),
                (f"v_cmp_lt_f32_e32 vcc, s{S_SLACK}, v{b}", False)]
        tail.append((f"s_mov_b64 s[{S_GROW}:{S_GROW + 1}], vcc", False) if n == 0 else
                    (f"s_or_b64 s[{S_GROW}:{S_GROW + 1}], s[{S_GROW}:{S_GROW + 1}], vcc", False))
        groups += [chain, tail]
    return groups


def online_raise(e: Emitter):
    """Online variant, after the tests: if some row grew, raise every row's reference to
    max(r, alpha max), rescale its row sums by f = 2^(r_old - r_new) now and, through s[S_RESC],
    its accumulators at the end of the step (after this step's PV products, made with the old
    reference).  OA[n] keeps f until then.  With r = -inf (NSHIFT = +inf) f is 0."""
    lab = e.new_label()
    e.branch("s_cbranch_scc0", lab)
    for n in range(2):
        a, b = OA[n], OB[n]
        e.emit(f"v_min_f32 v{b}, v{NSHIFT + n}, -v{a}")
        e.emit(f"v_sub_f32 v{a}, v{b}, v{NSHIFT + n}")
        e.emit(f"v_exp_f32 v{a}, v{a}")
        e.emit(f"v_mov_b32 v{NSHIFT + n}, v{b}")
        e.emit("s_nop 1")
        e.emit(f"v_mul_f32 v{LSUM + n}, v{LSUM + n}, v{a}")
        e.emit(f"v_mul_f32 v{LSUM_HI + n}, v{LSUM_HI + n}, v{a}")
    e.emit(f"s_mov_b32 s{S_RESC}, 1")
    e.label(lab)


def online_rescale_acc(e: Emitter):
    """Online variant, end of a step: when s[S_RESC] is set, multiplies the accumulators of
    query tile n by OA[n] (the PV MFMAs of this step have long completed: the 16 score MFMAs
    came after them).  The rare block is out of line, after the epilogue, so the loop's code
    stays contiguous; it branches back to the step's end.  It touches no score register, so
    the hazard state after it is the state at the branch."""
    block, back = e.new_label(), e.new_label()
    e.emit(f"s_cmp_lg_u32 s{S_RESC}, 0")
    e.emit(f"s_cbranch_scc1 {block}")
    e.lines.append(f"{back}:")
    body = ["s_nop 7", "s_nop 7"]
    tmp = (MASK_X, OB[0])
    k = 0
    for n in range(2):
        for i in range(64):
            reg = O_BASE + 64 * n + i
            t = tmp[k % 2]
            body += [f"v_accvgpr_read_b32 v{t}, a{reg}", f"v_mul_f32 v{t}, v{t}, v{OA[n]}",
                     f"v_accvgpr_write_b32 a{reg}, v{t}"]
            k += 1
    body += [f"s_mov_b32 s{S_RESC}, 0", "s_nop 2", f"s_branch {back}"]
    e.deferred.append((block, body))


def step(e: Emitter, jj: int, mode: str, fp32a: bool = False, online: bool = False):
    """Step jj of an unrolled group: tile t with t = 1 + jj (mod 8).

    mode "fast": every tile the step loads and scores lies inside one piece, not its last
    tile, so the DMA address just advances and the keys are all real (the group's entry check
    ensures it).  "slow": the DMA cursor may reach a piece's end (last window, next
    descriptor) and the S tile's mask is formed.  "first": the priming step t = 0 (S(0)
    already issued): no PV product (there is no tile -1), otherwise slow.  online: the
    online-softmax variant (fp32a arithmetic with a running reference, see online_pre)."""
    first = mode == "first"
    slow = mode != "fast"
    t_mod = 0 if first else 1 + jj
    cur = t_mod % 2            # parity of t: S(t), P(t), V(t) buffers
    prv = 1 - cur              # parity of t-1 (= parity of t+1)
    stage_t = t_mod % STAGES
    stage_next = (t_mod + 1) % STAGES
    stage_dma = (t_mod + AHEAD) % STAGES

    early = 0 if first else BARRIER_AFTER
    if early == 0:
        e.emit(f"s_waitcnt vmcnt({DMA_WAIT})")
        e.emit("s_barrier")
    e.emit("s_waitcnt lgkmcnt(0)")
    # The first BARRIER_AFTER PV MFMAs need only registers (V(t-1) fragments, waited for just
    # above, and P(t-1)), so they go before the wait for tile t+1 and the barrier: a wave that
    # reaches the barrier early keeps the matrix cores busy meanwhile (2 measured 0.5% faster
    # than 0 in same-box A/B runs, 1 slower, 3-4 in between).  Nothing before the barrier
    # touches the LDS ring.
    # The matrix cores start right after the barrier; the K(t+1) fragment reads and the DMA
    # of tile t+6 into the stage of tile t-2 (K rows then V rows of this wave) ride between
    # the first PV MFMAs (issued back to back after the barrier they left the matrix cores
    # idle for ~180 cycles a step).  Each M0 write is separated from the DMA that reads it
    # by at least one instruction, the wait state that hazard needs.
    kreads = [f"ds_read_b128 {k_reg(prv, kk)}, v{KOFF + kk} offset:{stage_next * TILE_BYTES}" for kk in range(8)]
    extra = []
    if first:
        # the S(0) MFMAs issued just before read the K fragment registers the K(1) reads
        # overwrite: let them take their operands first
        e.emit("s_nop 7")
        e.emit("s_nop 7")
    if slow:
        extra.append(stale_offsets(e))
    for grp in dma_issue(stage_dma):
        grp[1] = kreads.pop(0) if DMA_WITH_KREAD and kreads else "s_nop 0"
        extra.append(grp)
    extra += [[kr] for kr in kreads]
    extra += dma_advance(e) if slow else [list(a) for a in ADVANCE]

    plan = softmax_plan(cur, online=online)
    pre = online_pre(cur) if online else []
    slot = 0

    def valu_slot():
        nonlocal slot
        if slot < len(pre):
            for text, reads in pre[slot]:
                e.emit(text, reads_sbuf=cur if reads else None)
            if slot == len(pre) - 1:
                online_raise(e)
        for text, reads in plan[slot]:
            if (fp32a or online) and text.startswith("v_exp_f32"):
                # fp32a: the exponent is alpha S - (m + c_i), one FMA right before the exp
                r = int(text.split()[1].rstrip(",")[1:])
                n = (r - s_first(cur, 0)) // 16
                e.emit(f"v_fma_f32 v{r}, v{r}, v{ALPHA}, v{NSHIFT + n}", reads_sbuf=cur)
            e.emit(text, reads_sbuf=cur if reads else None)
        slot += 1

    # O^T += V(t-1)^T P(t-1)^T, with the K reads and the DMA after the first MFMAs (the
    # priming step has no PV product: its slots hold only the other work)
    i_mfma = 0
    for st in range(2):
        for m in range(4):
            for n in range(2):
                vf = v_frag(prv, st, m)
                p = vreg(p_first(prv, n) + 4 * st, 4)
                if not first:
                    e.emit(f"v_mfma_f32_32x32x16_bf16 {o_reg(n, m)}, {vf}, {p}, {o_reg(n, m)}")
                if i_mfma == early - 1:
                    e.emit(f"s_waitcnt vmcnt({DMA_WAIT})")
                    e.emit("s_barrier")
                if extra and i_mfma >= early:
                    e.seq(extra.pop(0))
                valu_slot()
                i_mfma += 1
    assert not extra
    if slow:
        mask_step(e, fp32a or online)
    # S(t+1) = K(t+1) Q^T - (m + c), with the V(t) transpose reads in the first half
    e.emit("s_waitcnt lgkmcnt(0)")
    tr = [(st, m, h) for st in range(2) for m in range(4) for h in range(2)]
    ti = 0
    for kk in range(8):
        for n in range(2):
            s0 = s_first(prv, n)
            src_c = shift_reg(n) if kk == 0 else vreg(s0, 16)
            e.emit(f"v_mfma_f32_32x32x16_bf16 {vreg(s0, 16)}, {k_reg(prv, kk)}, {q_reg(n, kk)}, {src_c}",
                   writes_sbuf=prv)
            if ti < len(tr) and 2 * kk + n >= V_TR_FIRST:
                for _ in range(V_TR_PER_SLOT):
                    st, m, h = tr[ti]
                    dst = v_frag(cur, st, m, h)
                    off = stage_t * TILE_BYTES + 4096 * st + 2048 * h
                    e.emit(f"ds_read_b64_tr_b16 {dst}, v{VOFF + m} offset:{off}")
                    ti += 1
            valu_slot()
    assert slot == 32 and ti == 16
    if online:
        online_rescale_acc(e)


def fast_check(e: Emitter):
    """At a group boundary: the number of fast groups that can follow (the DMA cursor and the
    mask cursor each keep >= 1 tile of their piece beyond them, the mask registers hold an
    all-real tile and the cursors are not past the last piece), then into the fast loop if
    any.  Lane offsets left stale by a descriptor switch are formed first."""
    e.emit("s_waitcnt lgkmcnt(0)")
    e.seq(stale_offsets(e))
    e.emit(f"s_sub_u32 s{S_TMP}, s{S_DREM}, 1")
    e.emit(f"s_sub_u32 s{S_TMP + 1}, s{S_MREM}, 1")
    e.emit(f"s_min_u32 s{S_TMP}, s{S_TMP}, s{S_TMP + 1}")
    e.emit(f"s_lshr_b32 s{S_CNT}, s{S_TMP}, 3")
    e.emit(f"s_or_b32 s{S_TMP + 1}, s{S_LOPREV}, s{S_LOBASE}")
    e.emit(f"s_cmp_eq_u32 s{S_TMP + 1}, 0")
    e.emit(f"s_cselect_b32 s{S_CNT}, s{S_CNT}, 0")
    e.emit(f"s_cmp_lg_u32 s{S_CNT}, 0")
    e.emit("s_cbranch_scc1 L_fixedm_fast_%=")


def init_acc(e: Emitter):
    """O's start value: zero when %[accp] is 0, else the state a previous call saved (the
    workspace's register order: o[n][m] part j at accp + 16 lane + (16 n + 4 m + j) KB, with
    %[accv] = 16 lane), loaded straight into O's registers.  The loads are not waited for
    here: they precede the prologue's tile loads, whose first wait (for tile 0) covers them
    (vector loads complete in order), and O is first read by the PV products of step 1.
    v0-v7 (score registers, free until S(0)) hold the eight (n, m) address offsets."""
    zero, done = e.new_label(), e.new_label()
    e.emit("s_cmp_eq_u64 %[accp], 0")
    e.branch("s_cbranch_scc1", zero)
    for n in range(2):
        for m in range(4):
            e.emit(f"v_add_u32 v{4 * n + m}, {4096 * (4 * n + m)}, %[accv]")
    for n in range(2):
        for m in range(4):
            for j in range(4):
                e.emit(f"global_load_dwordx4 {areg(O_BASE + 16 * (4 * n + m) + 4 * j, 4)}, v{4 * n + m}, "
                       f"%[accp] offset:{1024 * j}")
    e.branch("s_branch", done)
    e.label(zero)
    for r in range(128):
        e.emit(f"v_accvgpr_write_b32 a{O_BASE + r}, 0")
    e.label(done)


def generate_variant(variant: str) -> str:
    """One assembly function: "r17", the fixed-m loop on bf16(alpha q); "fp32a", the fixed-m
    loop that applies alpha in fp32 with an FMA per score; "online", the online-softmax loop
    (fp32a arithmetic against a running reference raised lazily, see online_pre)."""
    fp32a = variant == "fp32a"
    online = variant == "online"
    e = Emitter()
    init_acc(e)
    for n in range(2):
        for i in range(16):
            e.emit(f"v_mov_b32 v{SHIFT_BASE + 16 * n + i}, {'0' if fp32a or online else f'v{NSHIFT + n}'}")
    e.emit(f"v_mov_b32 v{NEG_INF}, 0xff800000")
    e.emit(f"v_mov_b32 v{LSUM_HI}, 0")
    e.emit(f"v_mov_b32 v{LSUM_HI + 1}, 0")
    e.emit(f"s_load_dwordx16 s[{S_D}:{S_D + 15}], s[{S_DPTR}:{S_DPTR + 1}], 0x0")
    e.emit(f"s_load_dwordx4 s[{S_M}:{S_M + 3}], s[{S_DPTR}:{S_DPTR + 1}], {MASK_OFF}")
    e.emit(f"s_mov_b64 s[{S_MPTR}:{S_MPTR + 1}], s[{S_DPTR}:{S_DPTR + 1}]")
    e.emit(f"s_mov_b32 s{S_LOPREV}, 0")
    e.emit(f"s_mov_b32 s{S_FLAG}, 1")
    if online:
        e.emit(f"s_mov_b32 s{S_RESC}, 0")
    e.emit("s_nop 7")
    e.emit("s_nop 7")
    # Prologue: tiles 0 .. 5 into stages 0 .. 5, then tile 0 waited for and met at a barrier.
    for tile in range(AHEAD):
        e.emit("s_waitcnt lgkmcnt(0)")
        e.seq(stale_offsets(e))
        for grp in dma_issue(tile):
            grp[1] = "s_nop 0"
            e.seq(grp)
        for grp in dma_advance(e):
            e.seq(grp)
    e.emit(f"s_waitcnt vmcnt({(AHEAD - 1) * 4})")
    e.emit("s_barrier")
    # S(0) from stage 0 with tile 0's mask, then the priming step t = 0 (P(0), the row sums of
    # tile 0, S(1), V(0)'s fragments, the DMA of tile 6).
    mask_step(e, fp32a or online)
    for kk in range(8):
        e.emit(f"ds_read_b128 {k_reg(0, kk)}, v{KOFF + kk} offset:0")
    e.emit("s_waitcnt lgkmcnt(0)")
    for kk in range(8):
        for n in range(2):
            s0 = s_first(0, n)
            src_c = shift_reg(n) if kk == 0 else vreg(s0, 16)
            e.emit(f"v_mfma_f32_32x32x16_bf16 {vreg(s0, 16)}, {k_reg(0, kk)}, {q_reg(n, kk)}, {src_c}",
                   writes_sbuf=0)
    step(e, 0, "first", fp32a=fp32a, online=online)
    fast_check(e)
    # slow groups: steps t = 1 .. n_tiles, one at a time, leaving after step t = n_tiles (the PV
    # product of the last tile); at each group boundary the fast check
    e.loop_head("L_fixedm_slow_%=")
    for jj in range(STAGES):
        step(e, jj, "slow", fp32a=fp32a, online=online)
        e.emit(f"s_sub_u32 s{S_TCNT}, s{S_TCNT}, 1")
        e.emit(f"s_cmp_eq_u32 s{S_TCNT}, 0")
        e.emit("s_cbranch_scc1 L_fixedm_end_%=")
    fast_check(e)
    e.emit("s_branch L_fixedm_slow_%=")
    # fast groups of 8 steps
    e.loop_head("L_fixedm_fast_%=")
    for jj in range(STAGES):
        step(e, jj, "fast", fp32a=fp32a, online=online)
    e.emit(f"s_sub_u32 s{S_DREM}, s{S_DREM}, 8")
    e.emit(f"s_sub_u32 s{S_MREM}, s{S_MREM}, 8")
    e.emit(f"s_sub_u32 s{S_TCNT}, s{S_TCNT}, 8")
    e.emit(f"s_sub_u32 s{S_CNT}, s{S_CNT}, 1")
    e.emit(f"s_cmp_lg_u32 s{S_CNT}, 0")
    e.emit("s_cbranch_scc1 L_fixedm_fast_%=")
    e.emit(f"s_cmp_eq_u32 s{S_DREM}, 1")
    for ins in LAST_WINDOW:
        e.emit(ins)
    e.emit("s_branch L_fixedm_slow_%=")
    e.loop_head("L_fixedm_end_%=")
    assert not e.pending
    e.emit(f"v_add_f32 v{LSUM}, v{LSUM}, v{LSUM_HI}")
    e.emit(f"v_add_f32 v{LSUM + 1}, v{LSUM + 1}, v{LSUM_HI + 1}")
    e.emit("s_waitcnt lgkmcnt(0)")
    e.emit("s_nop 7")
    e.emit("s_nop 7")
    if e.deferred:
        e.emit("s_branch L_fixedm_done_%=")
        for block, body in e.deferred:
            e.lines.append(f"{block}:")
            for ins in body:
                e.emit(ins)
        e.lines.append("L_fixedm_done_%=:")
    body = "\n".join(f'      "{l}\\n"' for l in e.lines)

    outs = []
    for n in range(2):
        for m in range(4):
            outs.append(f'"={{{o_reg(n, m)}}}"(o[{n}][{m}])')
    outs += [f'"+{{v{LSUM}}}"(lsum[0])', f'"+{{v{LSUM + 1}}}"(lsum[1])',
             f'"+{{s[{S_DPTR}:{S_DPTR + 1}]}}"(pieces)', f'"+{{s{S_TCNT}}}"(n_tiles)']
    if online:
        outs += [f'"+{{v{NSHIFT}}}"(nshift[0])', f'"+{{v{NSHIFT + 1}}}"(nshift[1])']
    ins = []
    for n in range(2):
        for kk in range(8):
            ins.append(f'"{{{q_reg(n, kk)}}}"(qf[{n}][{kk}])')
    if not online:
        ins += [f'"{{v{NSHIFT}}}"(nshift[0])', f'"{{v{NSHIFT + 1}}}"(nshift[1])']
    ins += [f'"{{v{KOFF + kk}}}"(koff[{kk}])' for kk in range(8)]
    ins += [f'"{{v{VOFF + m}}}"(voff[{m}])' for m in range(4)]
    ins += [f'"{{v{ROW + i}}}"(lane[{i}])' for i in range(2)]
    ins += [f'"{{v{CK + i}}}"(lane[{2 + i}])' for i in range(2)]
    ins += [f'"{{v{CV[i]}}}"(lane[{4 + i}])' for i in range(2)]
    ins += [f'"{{v{KB4}}}"(kb4)']
    if fp32a or online:
        ins += [f'"{{v{ALPHA}}}"(alpha)']
    ins += [f'"{{s{S_LDS}}}"(lds_wave)', '[accp] "s"(accp)', '[accv] "v"(accv)']
    clob = ([f"v{i}" for i in range(S_BASE, S_BASE + 64)] + [f"v{i}" for i in range(P_BASE, P_BASE + 32)]
            + [f"v{i}" for i in range(SHIFT_BASE, SHIFT_BASE + 32)] + [f"v{i}" for i in range(V1_VBASE, V1_VBASE + 32)]
            + [f"v{DMA + i}" for i in range(4)] + [f"v{LSUM_HI}", f"v{LSUM_HI + 1}"]
            + [f"v{NEG_INF}", f"v{MASK_X}"]
            + [f"a{i}" for i in range(K_BASE, K_BASE + 64)]
            + [f"s{i}" for i in range(S_D, S_M + 4)] + [f"s{i}" for i in range(S_MPTR, S_TMP + 2)]
            + [f"s{i}" for i in (S_CNT, S_LO, S_LOPREV, S_FLAG)]
            + ([f"v{r}" for r in OA + OB] + [f"s{i}" for i in (S_GROW, S_GROW + 1, S_RESC)] if online else [])
            + ["vcc", "scc", "memory"])
    clob_text = ",\n        ".join(", ".join(f'"{c}"' for c in clob[i:i + 12]) for i in range(0, len(clob), 12))

    def join(items):
        return ",\n        ".join(items)

    name = {"r17": "fixed_loop_asm", "fp32a": "fixed_loop_fp32a_asm", "online": "online_loop_asm"}[variant]
    what = {"fp32a": "the query fragments are bf16(q) and each exponent is alpha S - (m + c_i) (one FMA "
                     "before its exp; the S chain starts from 0)",
            "r17": "the query fragments are bf16(alpha q) and the S chain starts from -(m + c_i), so S is "
                   "the exponent",
            "online": "online softmax: the query fragments are bf16(q) and each exponent is alpha S - r_i, "
                      "with r_i = -nshift[n] the running reference of query row i, raised to the row's "
                      "maximum only when that exceeds it by more than the slack s of the piece "
                      "descriptors (base 2; the row sums and accumulators then rescaled, so every "
                      "probability is at most 2^s); on entry r_i = -inf (nshift = +inf), on exit "
                      "nshift = -r_i"}[variant]
    return f"""// {what}.
// The whole fixed-m pass of one work item over its n_tiles (>= 1) tiles of 32 keys, the
// tiles of its chunk pieces in order (the piece descriptor list at `pieces`, ended by a
// terminator): O set to zero (accp = 0) or loaded from the state a previous call saved at
// accp (accv = 16 x lane), the prologue (tiles 0 .. 5 loaded, tile 0 waited for and met at a barrier),
// S(0), the priming step t = 0, then steps t = 1 .. n_tiles in groups of 8, each turning S(t)
// into P(t), adding V(t-1) P(t-1) to O and computing S(t+1); the last step completes the PV
// product of the last tile.  Keys past the last tile are masked (p = 0).  The LDS ring and
// its barriers continue across piece boundaries.  On exit every LDS read has completed;
// DMAs of tiles past the end may still be in flight.
__device__ __attribute__((always_inline)) inline void {name}(
    f32x16 (&o)[2][4], const bf16x8 (&qf)[2][8], float (&lsum)[2], {"float" if online else "const float"} (&nshift)[2],
    const uint32_t (&koff)[8], const uint32_t (&voff)[4], const uint32_t (&lane)[6], uint32_t kb4,
    uint64_t pieces, uint32_t n_tiles, uint32_t lds_wave{", float alpha" if fp32a or online else ""}, uint64_t accp,
    uint32_t accv) {{
  asm volatile(
{body}
      : {join(outs)}
      : {join(ins)}
      : {clob_text});
}}
"""


def generate() -> str:
    head = ("// Generated by gen_fixed_loop.py; do not edit by hand.\n\n"
            f"static_assert(kStages == {STAGES} && kAhead == {AHEAD} && kTileBytes == {TILE_BYTES},\n"
            "              \"the generated loop assumes this LDS ring geometry\");\n\n")
    return head + generate_variant("r17") + "\n" + generate_variant("fp32a") + "\n" + generate_variant("online")


def main(out_path=None):
    out_path = out_path or os.path.join(os.path.dirname(os.path.abspath(__file__)), "fixed_loop.inc")
    text = generate()
    old = None
    if os.path.exists(out_path):
        with open(out_path) as f:
            old = f.read()
    if old != text:
        with open(out_path, "w") as f:
            f.write(text)
    return out_path


if __name__ == "__main__":
    print(main(sys.argv[1] if len(sys.argv) > 1 else None))
