"""The generated assembly loop of the bf16 kernel: the committed fixed_loop.inc is exactly
what gen_fixed_loop.py writes, and the structural rules its docstring states hold (CPU only)."""
import os
import re
import sys

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "dit_amd", "csrc")


@pytest.fixture(scope="module")
def gen():
    sys.path.insert(0, CSRC)
    try:
        import gen_fixed_loop
    finally:
        sys.path.remove(CSRC)
    return gen_fixed_loop


def _body(text):
    return re.findall(r'^\s*"([^"\\]*)\\n"', text, flags=re.M)


def test_committed_loop_matches_generator(gen):
    with open(os.path.join(CSRC, "fixed_loop.inc")) as f:
        assert f.read() == gen.generate()


@pytest.mark.parametrize("online", [False, True])
def test_every_step_places_all_exps_and_row_sums(gen, online):
    for buf in (0, 1):
        plan = gen.softmax_plan(buf, online=online)
        assert len(plan) == 32
        texts = [t for slot in plan for t, _ in slot]
        assert sum(t.startswith("v_exp_f32") for t in texts) == 32
        assert sum(t.startswith("v_cvt_pk_bf16_f32") for t in texts) == 16
        assert sum(t.startswith("v_add_f32") for t in texts) == 32
        # every score register is exponentiated exactly once
        regs = sorted(int(re.match(r"v_exp_f32 v(\d+)", t).group(1)) for t in texts if t.startswith("v_exp"))
        first = gen.s_first(buf, 0)
        assert regs == list(range(first, first + 32))


def test_exp_readers_sit_behind_their_exp(gen):
    """A reader of an exp result sits EXP_GAP or more MFMA slots after it (one slot in the
    step's last slot), never in the same slot."""
    for buf in (0, 1):
        plan = gen.softmax_plan(buf)
        exp_slot = {}
        for s, slot in enumerate(plan):
            for t, _ in slot:
                m = re.match(r"v_exp_f32 v(\d+)", t)
                if m:
                    exp_slot[int(m.group(1))] = s
        for s, slot in enumerate(plan):
            for t, _ in slot:
                if t.startswith("v_exp"):
                    continue
                for r in (int(x) for x in re.findall(r"v(\d+)", t.split(" ", 1)[1])[1:]):
                    if r in exp_slot:
                        gap = s - exp_slot[r]
                        assert gap >= (gen.EXP_GAP if s < 31 else 1), (t, gap)


def test_mfma_results_are_waited_for(gen):
    """Every VALU read of a score register comes >= 16 wait states (an instruction is one, s_nop N is N+1)
    after the MFMA that last wrote that score buffer.  A forward-branch target (L_fixedm_fN) takes the
    closest write over the paths that reach it; at any other label (a loop head) the tracking restarts
    as if an MFMA had just written both buffers, as the generator assumes.  The online variant's
    out-of-line accumulator-rescale blocks read no score register and branch back to the step's end."""
    lines = _body(gen.generate())
    written = {}
    count = 0
    pending = {}
    seen = set()
    s_regs = {0: set(range(gen.s_first(0, 0), gen.s_first(0, 0) + 32)),
              1: set(range(gen.s_first(1, 0), gen.s_first(1, 0) + 32))}
    for ln in lines:
        if ln.endswith(":"):
            lab = ln[:-1]
            seen.add(lab)
            if re.match(r"L_fixedm_f\d+_%=$", lab):
                for dist in pending.pop(lab, []):
                    for b, d in dist.items():
                        written[b] = max(written.get(b, -10**9), count - d)
            else:
                written = {b: count - 1 for b in (0, 1)}
            continue
        m = re.match(r"s_c?branch\S* (L_fixedm_f\d+_%=)$", ln)
        if m:
            count += 1
            if m.group(1) not in seen:    # a forward branch (a backward one returns from an
                pending.setdefault(m.group(1), []).append({b: count - w for b, w in written.items()})
            continue                      # out-of-line block that reads no score register)
        if ln.startswith("v_mfma") and re.match(r"v_mfma\S* v\[(\d+):", ln):
            lo = int(re.match(r"v_mfma\S* v\[(\d+):", ln).group(1))
            for b, regs in s_regs.items():
                if lo in regs:
                    written[b] = count
        elif ln.startswith(("v_exp", "v_cvt_pk", "v_add_f32", "v_fma_f32", "v_max3_f32", "v_max_f32")):
            for r in (int(x) for x in re.findall(r"v(\d+)", ln)[1:]):
                for b, regs in s_regs.items():
                    if r in regs and b in written:
                        assert count - written[b] - 1 >= 16, ln
        count += int(ln.split()[1]) + 1 if ln.startswith("s_nop") else 1
    assert not pending


def test_online_row_max_covers_every_score(gen):
    """The online variant's row maximum of query tile n reads each of its 16 score registers
    (the other 16 keys come from lane ^ 32 through the swap), and no exp precedes the test that
    may raise the reference."""
    for buf in (0, 1):
        pre = gen.online_pre(buf)
        assert len(pre) == gen.ONLINE_PRE
        for n in range(2):
            texts = [t for t, _ in pre[2 * n] + pre[2 * n + 1]]
            read = set()
            for t in texts:
                if t.startswith(("v_max3_f32", "v_max_f32")):
                    read |= {int(x) for x in re.findall(r"v(\d+)", t)[1:]}
            first = gen.s_first(buf, n)
            assert set(range(first, first + 16)) <= read
            assert any(t.startswith("v_permlane32_swap_b32") for t in texts)
        plan = gen.softmax_plan(buf, online=True)
        assert all(not plan[s] for s in range(gen.ONLINE_PRE))
