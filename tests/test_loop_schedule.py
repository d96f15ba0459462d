"""The generated assembly loop's scalar and control code, run on the CPU by a small interpreter
against piece descriptor lists built by the kernel's own list builder (dit_amd/csrc/pieces.h,
compiled for the host).  For chunk sequences with ragged tails, chunks shorter than a tile,
differing strides and split tile ranges it checks, for every lane: each tile load reads the
keys that tile holds (and stays inside a chunk past the last tile), lands in the right LDS
stage, each score tile's mask marks exactly the keys that are not real, the loop meets
n_tiles + 2 barriers (as many as the compiled body), and no descriptor load is read or
overwritten before it is waited for.  CPU only."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dit_amd", "csrc")
M32 = 0xffffffff
TBL = 0x7000_0000_0000
KT = 32
SLACK_BITS = 0x40e00000                # 7.0f: the descriptors' word 19 in these cases


@pytest.fixture(scope="module")
def gen():
    sys.path.insert(0, CSRC)
    try:
        import gen_fixed_loop
    finally:
        sys.path.remove(CSRC)
    return gen_fixed_loop


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("pieces") / "libpieces.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC,
                    os.path.join(ROOT, "tests", "pieces_host.cpp"), "-o", str(out)], check=True)
    L = ctypes.CDLL(str(out))
    L.build_piece_list_host.restype = ctypes.c_int
    return L


def build_list(lib, chunks, v0, v1):
    n = len(chunks)
    out = np.zeros((n + 1) * 32, dtype=np.uint32)
    arr = lambda key, t: np.ascontiguousarray([c[key] for c in chunks], dtype=t)
    kb, vb = arr("kb", np.uint64), arr("vb", np.uint64)
    kss, vss, ln = arr("k_ss", np.int64), arr("v_ss", np.int64), arr("len", np.int64)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    np_ = lib.build_piece_list_host(p(out), p(kb), p(vb), p(kss), p(vss), p(ln), n, ctypes.c_int64(v0),
                                    ctypes.c_int64(v1), ctypes.c_uint32(SLACK_BITS))
    return np_, out


def _body(text):
    return re.findall(r'^\s*"([^"\\]*)\\n"', text, flags=re.M)


class Fault(AssertionError):
    pass


class Machine:
    """Executes the scalar, branch, lane-offset, mask and load instructions of the loop; the
    matrix, LDS-read and exp work is skipped (it does not steer the control flow)."""

    def __init__(self, lines, mem, wave, n_tiles, lds0=0, seed=0, accp=0):
        self.lines = lines
        self.accp = accp                                 # %[accp]: the saved state's address, or 0
        self.acc_loads = []                              # (first AGPR, per-lane address)
        self.acc_zeroed = []                             # AGPRs written with 0
        self.rng = np.random.default_rng(seed)
        self.vcc_bit = 0                                 # the online growth test (data dependent)
        self.rescales = 0
        self.labels = {l[:-1]: i for i, l in enumerate(lines) if l.endswith(":")}
        self.mem = mem
        self.s = {}
        self.poison = set()
        self.pending = {}
        self.scc = 0
        self.m0 = None
        lane = np.arange(64, dtype=np.int64)
        self.v = {}
        for i in range(2):
            row = 4 * (2 * wave + i) + lane // 16
            self.v[181 + i] = row
            self.v[183 + i] = 16 * ((lane & 15) ^ (row & 15))
            self.v[(185, 191)[i]] = 16 * ((lane & 15) ^ ((row & 3) << 2))
        self.v[188] = 4 * (lane >> 5)
        self.accv = 16 * lane                            # %[accv]
        self.mask = np.zeros((64, 32), dtype=bool)     # v96..v127: True where -inf
        self.vcc = np.zeros(64, dtype=bool)
        self.s[84], self.s[85] = TBL & M32, TBL >> 32
        self.s[90] = n_tiles
        self.s[95] = lds0 + 2048 * wave
        self.dmas = []                                   # (m0, per-lane address)
        self.s_tiles = []                                # (n, mask of the 16 registers)
        self.barriers = 0

    def sreg(self, tok):
        m = re.fullmatch(r"s(\d+)", tok)
        if m:
            r = int(m.group(1))
            if r in self.poison:
                raise Fault(f"s{r} read before its load was waited for")
            if r not in self.s:
                raise Fault(f"s{r} read before it was written")
            return self.s[r]
        if tok == "m0":
            return self.m0
        return int(tok, 0)

    def spair(self, tok):
        a, b = map(int, re.fullmatch(r"s\[(\d+):(\d+)\]", tok).groups())
        assert b == a + 1
        return self.sreg(f"s{a}") | (self.sreg(f"s{b}") << 32)

    def wset(self, r, val):
        if r in self.poison:
            raise Fault(f"s{r} written while a load into it is in flight")
        self.s[r] = val & M32

    def wpair(self, tok, val):
        a = int(re.fullmatch(r"s\[(\d+):\d+\]", tok).group(1))
        self.wset(a, val)
        self.wset(a + 1, val >> 32)

    def vreg(self, tok):
        return self.v[int(tok[1:])]

    def run(self, limit=10**7):
        pc = 0
        steps = 0
        while pc < len(self.lines):
            steps += 1
            if steps > limit:
                raise Fault("did not finish")
            ln = self.lines[pc]
            pc += 1
            if ln.endswith(":"):
                continue
            op, _, rest = ln.partition(" ")
            ops = [o.strip() for o in rest.split(",")] if rest else []
            if op in ("s_cbranch_scc1", "s_cbranch_scc0", "s_branch"):
                take = op == "s_branch" or (self.scc == 1) == (op == "s_cbranch_scc1")
                if take:
                    pc = self.labels[ops[0]]
                continue
            self.exec(op, ops, ln)

    def exec(self, op, ops, ln):
        if op == "s_waitcnt":
            if "lgkmcnt(0)" in ln:
                for r, val in self.pending.items():
                    self.s[r] = val
                self.pending.clear()
                self.poison.clear()
            return
        if op in ("s_nop",):
            return
        if op == "s_barrier":
            self.barriers += 1
            return
        if op.startswith("s_load_dword"):
            n = int(op[len("s_load_dwordx"):])
            lo, hi = map(int, re.fullmatch(r"s\[(\d+):(\d+)\]", ops[0]).groups())
            assert hi - lo + 1 == n and lo % 4 == 0
            addr = self.spair(ops[1]) + int(ops[2], 0)
            for i in range(n):
                if lo + i in self.poison:
                    raise Fault("two loads in flight into one register")
                if addr + 4 * i not in self.mem:
                    raise Fault(f"descriptor load outside the table at {addr + 4 * i:#x}")
                self.pending[lo + i] = self.mem[addr + 4 * i]
                self.poison.add(lo + i)
            return
        if op == "global_load_dwordx4":             # O's saved state: a[lo:lo+3], vX, %[accp] offset:K
            lo, hi = map(int, re.fullmatch(r"a\[(\d+):(\d+)\]", ops[0]).groups())
            assert hi == lo + 3 and ops[2].startswith("%[accp] offset:")
            self.acc_loads.append((lo, self.accp + self.vreg(ops[1]) + int(ops[2].split(":")[1])))
            return
        if op.startswith("s_"):
            # the reads come first, so a pending destination register is caught by wset
            if op == "s_cmp_eq_u64":
                assert ops == ["%[accp]", "0"]
                self.scc = int(self.accp == 0)
            elif op == "s_mov_b64" and ops[1] == "vcc":
                self.wpair(ops[0], self.vcc_bit)
            elif op == "s_or_b64" and ops[2] == "vcc":
                r = self.spair(ops[1]) | self.vcc_bit
                self.scc = int(r != 0)
                self.wpair(ops[0], r)
            elif op in ("s_add_u32", "s_addc_u32", "s_sub_u32"):
                a, b = self.sreg(ops[1]), self.sreg(ops[2])
                if op == "s_add_u32":
                    r = a + b
                    self.scc = r >> 32
                elif op == "s_addc_u32":
                    r = a + b + self.scc
                    self.scc = r >> 32
                else:
                    r = a - b
                    self.scc = 1 if a < b else 0
                if ops[0] == "m0":
                    self.m0 = r & M32
                else:
                    self.wset(int(ops[0][1:]), r)
            elif op in ("s_cmp_eq_u32", "s_cmp_lg_u32"):
                a, b = self.sreg(ops[0]), self.sreg(ops[1])
                self.scc = int((a == b) == (op == "s_cmp_eq_u32"))
                if op == "s_cmp_lg_u32" and ops[0] == "s98" and self.scc:
                    self.rescales += 1
            elif op == "s_cselect_b32":
                self.wset(int(ops[0][1:]), self.sreg(ops[1]) if self.scc else self.sreg(ops[2]))
            elif op == "s_cselect_b64":
                self.wpair(ops[0], self.spair(ops[1]) if self.scc else self.spair(ops[2]))
            elif op == "s_mov_b32":
                self.wset(int(ops[0][1:]), self.sreg(ops[1]))
            elif op == "s_mov_b64":
                self.wpair(ops[0], self.spair(ops[1]))
            elif op == "s_min_u32":
                a, b = self.sreg(ops[1]), self.sreg(ops[2])
                self.scc = int(a < b)
                self.wset(int(ops[0][1:]), min(a, b))
            elif op == "s_lshr_b32":
                r = self.sreg(ops[1]) >> self.sreg(ops[2])
                self.scc = int(r != 0)
                self.wset(int(ops[0][1:]), r)
            elif op == "s_or_b32":
                r = self.sreg(ops[1]) | self.sreg(ops[2])
                self.scc = int(r != 0)
                self.wset(int(ops[0][1:]), r)
            else:
                raise Fault(f"unmodelled scalar instruction: {ln}")
            return
        # vector and memory instructions: every scalar operand must be readable
        for tok in re.findall(r"s\[\d+:\d+\]|\bs\d+\b", ln):
            if tok.startswith("s["):
                self.spair(tok)
            else:
                self.sreg(tok)
        if op == "global_load_lds_dwordx4":
            self.dmas.append((self.m0, self.spair(ops[1]) + self.vreg(ops[0])))
        elif op == "v_subrev_u32":
            self.v[int(ops[0][1:])] = (self.vreg(ops[2]) - self.sreg(ops[1])) & M32
        elif op == "v_max_i32":
            x = self.vreg(ops[2]).astype(np.uint32).astype(np.int32).astype(np.int64)
            self.v[int(ops[0][1:])] = np.maximum(int(ops[1]), x) & M32
        elif op == "v_mul_lo_u32":
            self.v[int(ops[0][1:])] = (self.vreg(ops[1]) * self.sreg(ops[2])) & M32
        elif op == "v_add_u32" and ops[2] == "%[accv]":
            self.v[int(ops[0][1:])] = (int(ops[1]) + self.accv) & M32
        elif op == "v_add_u32":
            self.v[int(ops[0][1:])] = (self.vreg(ops[1]) + self.vreg(ops[2])) & M32
        elif op == "v_accvgpr_write_b32" and ops[1] == "0":    # O's zero start (the online
            self.acc_zeroed.append(int(ops[0][1:]))             # rescale writes registers back)
        elif op == "v_sub_u32":
            self.v[int(ops[0][1:])] = (self.sreg(ops[1]) - self.vreg(ops[2])) & M32
        elif op == "v_cmp_lt_f32_e32":       # the online growth test: either outcome
            if self.sreg(ops[1]) != SLACK_BITS:
                raise Fault(f"growth test against {ops[1]}, not the descriptors' slack word")
            self.vcc_bit = int(self.rng.integers(0, 2))
        elif op == "v_cmp_lt_i32_e32":
            x = self.vreg(ops[2]).astype(np.uint32).astype(np.int32)
            self.vcc = int(ops[1]) < x
        elif op == "v_cndmask_b32_e32":
            d = int(ops[0][1:])
            assert 96 <= d < 128 and ops[2] == "v189" and ops[3] == "vcc"
            self.mask[:, d - 96] = self.vcc
        elif op == "v_mov_b32":
            d = int(ops[0][1:])
            if 96 <= d < 128:
                self.mask[:, d - 96] = False
        elif op.startswith("v_mfma"):
            src_c = ops[-1]
            if src_c in ("v[96:111]", "v[112:127]"):
                n = 0 if src_c == "v[96:111]" else 1
                self.s_tiles.append((n, self.mask[:, 16 * n:16 * n + 16].copy()))
        elif op.startswith(("v_", "ds_")):
            m = re.match(r"v(\d+)$", ops[0]) if ops else None
            if m and int(m.group(1)) in (176, 177, 178, 179, 181, 182, 183, 184, 185, 188, 191):
                raise Fault(f"unmodelled write of a tracked register: {ln}")
        else:
            raise Fault(f"unmodelled instruction: {ln}")


ACC_BASE = 0x5000_0000_0000


def check_acc_init(m, accp):
    """O's start: all 128 accumulation registers zeroed, or each 4-register group of o[n][m]
    loaded once from its 16 bytes per lane of the saved state."""
    lane = np.arange(64)
    if accp == 0:
        assert sorted(m.acc_zeroed) == list(range(128)) and not m.acc_loads
        return
    assert not m.acc_zeroed and len(m.acc_loads) == 32
    for lo, addr in m.acc_loads:
        n, m_, j = lo // 64, (lo // 16) % 4, (lo // 4) % 4
        assert np.array_equal(addr, accp + 16 * lane + 1024 * (16 * n + 4 * m_ + j)), (lo,)
    assert sorted(lo for lo, _ in m.acc_loads) == list(range(0, 128, 4))


def _tiles(chunks):
    """(chunk index, tile j) of the launch's tile sequence."""
    return [(c, j) for c, ch in enumerate(chunks) for j in range((ch["len"] + KT - 1) // KT)]


def _expected_rows(ch, j, row):
    """Key row of chunk `ch` that tile j's row `row` holds, and the tile's first real row."""
    L = ch["len"]
    if L < KT:
        return np.maximum(row - (KT - L), 0), KT - L
    n_full, rem = L // KT, L % KT
    start = min(KT * j, L - KT)
    lo = KT - rem if (j == n_full and rem > 0) else 0
    return start + row, lo


def _chunks(lens, strides):
    out = []
    for c, (L, (ks, vs)) in enumerate(zip(lens, strides)):
        out.append(dict(kb=(c + 1) << 36, vb=((c + 1) << 36) + (1 << 35), k_ss=ks, v_ss=vs, len=L))
    return out


def run_case(gen, lib, lens, strides, parts=1, part=None, waves=(0, 3), variants=("r17", "fp32a", "online")):
    chunks = _chunks(lens, strides)
    seq = _tiles(chunks)
    T = len(seq)
    v0, v1 = (0, T) if part is None else (T * part // parts, T * (part + 1) // parts)
    n_pieces, table = build_list(lib, chunks, v0, v1)
    n_tiles = v1 - v0
    if n_tiles == 0:
        assert n_pieces == 0
        return
    mem = {TBL + 4 * i: int(w) for i, w in enumerate(table[:(n_pieces + 1) * 32])}
    items = seq[v0:v1]
    for variant in variants:
        lines = _body(gen.generate_variant(variant))
        for wave in waves:
            accp = ACC_BASE if (wave + n_tiles) % 2 else 0   # both ways O starts
            m = Machine(lines, mem, wave, n_tiles, seed=wave + 7 * n_tiles, accp=accp)
            m.run()
            check_acc_init(m, accp)
            if variant == "online" and n_tiles >= 4:
                assert m.rescales > 0       # the out-of-line accumulator rescale ran
            assert m.barriers == n_tiles + 2
            # loads: tiles 0 .. n_tiles + 6, four instructions each, in the ring's stages
            assert len(m.dmas) == 4 * (n_tiles + 7), (len(m.dmas), n_tiles)
            lane = np.arange(64)
            for k, (m0, addr) in enumerate(m.dmas):
                tile = k // 4
                off = m0 - 2048 * wave
                is_v = off >= 65536
                i = (off % 8192) // 1024
                assert (off % 65536) // 8192 == tile % 8 and off % 1024 == 0 and i in (0, 1), (k, off)
                row = 4 * (2 * wave + i) + lane // 16
                chunk16 = 16 * (((lane & 15) ^ ((row & 3) << 2)) if is_v else ((lane & 15) ^ (row & 15)))
                key = "vb" if is_v else "kb"
                sk = "v_ss" if is_v else "k_ss"
                if tile < n_tiles:
                    c, j = items[tile]
                    ch = chunks[c]
                    krow, _ = _expected_rows(ch, j, row)
                    want = ch[key] + krow * 2 * ch[sk] + chunk16
                    assert np.array_equal(addr, want), (tile, k, lens)
                else:   # past the end: inside some chunk, this lane's chunk of a whole row
                    ok = np.zeros(64, dtype=bool)
                    for ch in chunks:
                        rel = addr - ch[key]
                        ok |= (rel >= 0) & (rel < ch["len"] * 2 * ch[sk]) & (rel % (2 * ch[sk]) == chunk16)
                    assert ok.all(), (tile, lens)
            # score tiles 0 .. n_tiles + 1 (the last is never used), two query tiles each
            assert len(m.s_tiles) == 2 * (n_tiles + 2)
            hh = lane >> 5
            for tile in range(n_tiles + 1):
                lo = KT if tile == n_tiles else _expected_rows(chunks[items[tile][0]], items[tile][1], 0)[1]
                for n in range(2):
                    nn, mk = m.s_tiles[2 * tile + n]
                    assert nn == n
                    for r in range(16):
                        keyrow = 8 * (r >> 2) + 4 * hh + (r & 3)
                        assert np.array_equal(mk[:, r], keyrow < lo), (tile, r, lens)


def test_single_long_chunk(gen, lib):
    run_case(gen, lib, [1000], [(128, 128)])


def test_ring_chunks_of_whole_tiles(gen, lib):
    run_case(gen, lib, [1024, 1024, 1024, 1024], [(5120, 5120)] * 4)


def test_ragged_and_short_chunks(gen, lib):
    run_case(gen, lib, [300, 5, 33, 64, 1, 31, 32, 97], [(128, 256), (40, 40), (5120, 128), (128, 128),
                                                          (128, 5000), (128, 128), (2048, 2048), (128, 128)])


def test_partial_tile_before_a_fast_run(gen, lib):
    """A partial last tile scored just before a group boundary, followed by a long chunk: the
    fast groups may start only once the mask registers hold an all-real tile again."""
    run_case(gen, lib, [300, 610], [(128, 128), (256, 256)])
    run_case(gen, lib, [44, 1000], [(128, 128), (128, 128)])


def test_tiny_items(gen, lib):
    for lens in ([1], [31], [32], [33], [64], [65], [1, 1], [20, 40]):
        run_case(gen, lib, lens, [(128, 128)] * len(lens), waves=(1,))


@pytest.mark.parametrize("parts", [2, 3, 4])
def test_split_parts(gen, lib, parts):
    lens = [290, 7, 610, 64, 33]
    for part in range(parts):
        run_case(gen, lib, lens, [(128, 128), (128, 256), (5120, 5120), (128, 128), (256, 128)], parts, part,
                 waves=(2,), variants=("r17",))


def test_random_sequences(gen, lib):
    rng = np.random.default_rng(11)
    for _ in range(6):
        n = int(rng.integers(1, 9))
        lens = [int(x) for x in rng.choice([1, 3, 17, 31, 32, 33, 63, 64, 65, 100, 256, 257, 400], size=n)]
        strides = [(int(rng.choice([128, 640, 5120])), int(rng.choice([128, 640, 5120]))) for _ in range(n)]
        parts = int(rng.integers(1, 5))
        part = None if parts == 1 else int(rng.integers(0, parts))
        run_case(gen, lib, lens, strides, parts, part, waves=(int(rng.integers(0, 4)),),
                 variants=(("r17", "fp32a", "online")[int(rng.integers(0, 3))],))


def test_empty_part_writes_no_list(gen, lib):
    chunks = _chunks([40], [(128, 128)])   # 2 tiles: part 0 of 4 is empty
    n, _ = build_list(lib, chunks, 0, 0)
    assert n == 0
