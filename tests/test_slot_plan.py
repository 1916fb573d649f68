"""Host check of the pipelined attention kernel's issue-slot plan.

The kernel places its softmax work between MFMAs according to a constexpr
planner (PipeSlotPlan in csrc/attention.hip); the kernel itself only asserts
that a plan exists.  This test compiles the planner's own source with the host
compiler, prints the plans for the built widths, and checks every scheduling
rule here, stated independently of the planner's procedure:

- a step has NQ score MFMA slots (0..NQ-1), then NV value MFMAs of key half 0
  and NV of half 1; row block nb's first value MFMA of half u is slot
  NQ + u*NV + nb;
- an fp16 pack follows its two exponentials and precedes the first value MFMA
  that reads it;
- the copies of the next block's scores follow its last score MFMA (NQ - 1) by
  at least one slot; a block max follows its eight copies; a row's rescale test
  follows both of its maxes;
- each slot's work stays within the plan's budget of plain-VALU units (a
  v_exp_f32 counts two) and within eight items;
- items issue in order: each half's exponentials interleaved with the packs they
  complete, then copies, maxes and tests.
"""
import pathlib
import shutil
import subprocess

import pytest

SRC = pathlib.Path(__file__).resolve().parents[1] / "mla_latent_kv_vmla_amd" / "csrc" / "attention.hip"

# (NQ, NV) per built pipelined width: NQ = 2 row blocks x (d_c + d_r) / 16 k-steps,
# NV = 2 x d_c / 32 value fragments.  d_c 192 is dispatched; d_c 96 is the
# measured-and-rejected variant whose budget the notes quote.
WIDTHS = {192: (28, 12), 96: (16, 6)}
BUDGET = {192: 4, 96: 6}

N_ITEMS = 86
EXP0, PACK0, EXP1, PACK1, COPY, MAX, CMP = 0, 16, 24, 40, 48, 80, 84


def _cost(i):
    if EXP0 <= i < PACK0 or EXP1 <= i < PACK1:
        return 2  # v_exp_f32
    if PACK0 <= i < EXP1 or PACK1 <= i < COPY:
        return 2  # v_cvt_pk_f16_f32 + v_dot2
    if COPY <= i < MAX:
        return 1  # v_accvgpr_read
    return 4      # max over 8 scores (v_maximum3 chain) / pair max + test


def _issue_order():
    order = []
    for base_e, base_p in ((EXP0, PACK0), (EXP1, PACK1)):
        for q in range(8):
            order += [base_e + 2 * q, base_e + 2 * q + 1, base_p + q]
    return order + list(range(COPY, N_ITEMS))


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    s = SRC.read_text()
    a = s.index("struct PipeSlotPlan {")
    e = s.index("\n", s.index("inline constexpr PipeSlotPlan kPipeSlotPlan = pipe_slot_plan(NQ, NV);")) + 1
    dumps = "".join(f"  dump<{nq}, {nv}>();\n" for nq, nv in WIDTHS.values())
    prog = ("#include <cstdio>\n" + s[a:e] + """
template <int NQ, int NV> void dump() {
  constexpr PipeSlotPlan p = kPipeSlotPlan<NQ, NV>;
  std::printf("%d %d %d %d\\n", NQ, NV, (int)p.ok, p.budget);
  for (int i = 0; i < PipeSlotPlan::NITEM; ++i) std::printf("%d ", p.slot_of[i]);
  std::printf("\\n");
}
int main() {
""" + dumps + "  return 0;\n}\n")
    d = tmp_path_factory.mktemp("slot_plan")
    (d / "plan.cpp").write_text(prog)
    subprocess.run([gxx, "-std=c++17", "-O1", str(d / "plan.cpp"), "-o", str(d / "plan")], check=True)
    lines = subprocess.run([str(d / "plan")], check=True, capture_output=True, text=True).stdout.splitlines()
    out = {}
    for k in range(0, len(lines), 2):
        nq, nv, ok, budget = map(int, lines[k].split())
        out[(nq, nv)] = (bool(ok), budget, list(map(int, lines[k + 1].split())))
    return out


@pytest.mark.parametrize("dc", sorted(WIDTHS))
def test_plan_meets_every_rule(plans, dc):
    nq, nv = WIDTHS[dc]
    ok, budget, slot = plans[(nq, nv)]
    ns = nq + 2 * nv
    assert ok and len(slot) == N_ITEMS
    assert budget == BUDGET[dc]
    assert all(0 <= x < ns for x in slot)
    for u, (base_e, base_p) in enumerate(((EXP0, PACK0), (EXP1, PACK1))):
        for q in range(8):
            nb = q // 4
            p = slot[base_p + q]
            assert p > slot[base_e + 2 * q] and p > slot[base_e + 2 * q + 1], (u, q)
            assert p < nq + u * nv + nb, (u, q)  # before the value MFMA that reads it
    assert min(slot[COPY:MAX]) >= nq + 1
    for k in range(4):
        nb, half = k // 2, k % 2
        copies = [slot[COPY + 16 * nb + 8 * half + j] for j in range(8)]
        assert slot[MAX + k] > max(copies), k
    for nb in range(2):
        assert slot[CMP + nb] > max(slot[MAX + 2 * nb], slot[MAX + 2 * nb + 1]), nb
    load, count = [0] * ns, [0] * ns
    for i, x in enumerate(slot):
        load[x] += _cost(i)
        count[x] += 1
    assert max(load) <= budget and max(count) <= 8
    order = [slot[i] for i in _issue_order()]
    assert order == sorted(order)

