"""Host check of the pipelined attention kernel's issue-slot plan.

The kernel places its softmax work between MFMAs according to a constexpr
planner (PipeSlotPlan in csrc/attention.hip); the kernel itself only asserts
that a plan exists.  This test compiles the planner's own source with the host
compiler, prints the plans for the built widths, and checks every scheduling
rule here, stated independently of the planner's procedure:

- a step with NB 32-row blocks per wave has NQ score MFMA slots (0..NQ-1),
  then NB*NV/2 value MFMAs of key half 0 and NB*NV/2 of half 1; row block
  nb's first value MFMA of half u is slot NQ + u*NB*NV/2 + nb;
- the items are those of row blocks 0..NB-1: per half 8*NB exponentials and
  4*NB packs, 16*NB copies (AGPR accumulators only), 2*NB maxes, NB tests;
- an fp16 pack follows its two exponentials and precedes the first value MFMA
  that reads it;
- with AGPR score accumulators (d_c 192) the copies of the next block's scores
  follow its last score MFMA (NQ - 1) by at least one slot and a block max
  follows its eight copies; with VGPR accumulators (d_c 96 and 448) there are
  no copies and every max follows the last score MFMA by at least one slot; a
  row's rescale test follows both of its maxes;
- each slot's work stays within the plan's budget of plain-VALU units (a
  v_exp_f32 counts two, a pack two with its v_dot2 row sum, one where the
  row sums come from a ones block of value MFMAs; an item alone in its slot
  may exceed it) and within eight items;
- items issue in order: each half's exponentials interleaved with the packs they
  complete (a pack right after its pair's second exponential, or, with one-unit
  packs, after the next pair's), then copies (if any), maxes and tests.
"""
import pathlib
import shutil
import subprocess

import pytest

SRC = pathlib.Path(__file__).resolve().parents[1] / "mla_latent_kv_vmla_amd" / "csrc" / "attention.hip"

# (NQ, NV, copies, pack cost, lagged packs, NB) per built pipelined width:
# NQ = NB row blocks x (d_c + d_r) / 16 k-steps, NV = 2 x (d_c / 32 value
# fragments, plus the ones block at d_c 96); copies: AGPR score accumulators.
WIDTHS = {192: (28, 12, True, 2, False, 2), 96: (16, 8, False, 1, True, 2), 448: (30, 28, False, 2, False, 1)}
BUDGET = {192: 4, 96: 4, 448: 3}

N_ITEMS = 86
EXP0, PACK0, EXP1, PACK1, COPY, MAX, CMP = 0, 16, 24, 40, 48, 80, 84


def _cost(i, pack_cost):
    if EXP0 <= i < PACK0 or EXP1 <= i < PACK1:
        return 2  # v_exp_f32
    if PACK0 <= i < EXP1 or PACK1 <= i < COPY:
        return pack_cost  # v_cvt_pk_f16_f32 (+ v_dot2)
    if COPY <= i < MAX:
        return 1  # v_accvgpr_read
    return 4      # max over 8 scores (v_maximum3 chain) / pair max + test


def _issue_order(copies, lag, nb):
    order = []
    for base_e, base_p in ((EXP0, PACK0), (EXP1, PACK1)):
        for q in range(4 * nb):
            order += [base_e + 2 * q, base_e + 2 * q + 1]
            if not lag:
                order.append(base_p + q)
            elif q > 0:
                order.append(base_p + q - 1)
        if lag:
            order.append(base_p + 4 * nb - 1)
    if copies:
        order += list(range(COPY, COPY + 16 * nb))
    return order + list(range(MAX, MAX + 2 * nb)) + list(range(CMP, CMP + nb))


@pytest.fixture(scope="module")
def plans(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    s = SRC.read_text()
    a = s.index("struct PipeSlotPlan {")
    e = s.index("\n", s.index("inline constexpr PipeSlotPlan kPipeSlotPlan = pipe_slot_plan(NQ, NV, COPIES, PACKC, LAG, NB);")) + 1
    b = lambda v: "true" if v else "false"
    dumps = "".join(f"  dump<{nq}, {nv}, {b(c)}, {pc}, {b(lag)}, {nb}>();\n" for nq, nv, c, pc, lag, nb in WIDTHS.values())
    prog = ("#include <cstdio>\n" + s[a:e] + """
template <int NQ, int NV, bool C, int PC, bool L, int NB> void dump() {
  constexpr PipeSlotPlan p = kPipeSlotPlan<NQ, NV, C, PC, L, NB>;
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
    nq, nv, copies, pack_cost, lag, nbk = WIDTHS[dc]
    ok, budget, slot = plans[(nq, nv)]
    ns = nq + nbk * nv
    assert ok and len(slot) == N_ITEMS
    assert budget == BUDGET[dc]
    placed = _issue_order(copies, lag, nbk)
    assert all(0 <= slot[i] < ns for i in placed)
    assert all(slot[i] == -1 for i in range(N_ITEMS) if i not in placed)
    for u, (base_e, base_p) in enumerate(((EXP0, PACK0), (EXP1, PACK1))):
        for q in range(4 * nbk):
            nb = q // 4
            p = slot[base_p + q]
            assert p > slot[base_e + 2 * q] and p > slot[base_e + 2 * q + 1], (u, q)
            assert p < nq + u * nbk * nv // 2 + nb, (u, q)  # before the value MFMA that reads it
    if copies:
        assert min(slot[COPY:COPY + 16 * nbk]) >= nq + 1
        for k in range(2 * nbk):
            nb, half = k // 2, k % 2
            cps = [slot[COPY + 16 * nb + 8 * half + j] for j in range(8)]
            assert slot[MAX + k] > max(cps), k
    else:
        assert min(slot[MAX:MAX + 2 * nbk]) >= nq + 1
    for nb in range(nbk):
        assert slot[CMP + nb] > max(slot[MAX + 2 * nb], slot[MAX + 2 * nb + 1]), nb
    load, count = [0] * ns, [0] * ns
    for i in placed:
        load[slot[i]] += _cost(i, pack_cost)
        count[slot[i]] += 1
    assert all(ld <= budget or c == 1 for ld, c in zip(load, count)) and max(count) <= 8
    order = [slot[i] for i in placed]
    assert order == sorted(order)
