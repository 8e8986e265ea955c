"""CPU models of the fused GEMM kernels' work assignment and flags, run under
random schedules: the progress arguments and the data each wait protects.

GEMM + reduce-scatter (the work items of the fused kernel): items (phase,
position, rank) are numbered phase by phase, position by position, the ranks
of a position adjacent; G resident workgroups each take items g, g + G, ...
in order.  An item of phase f > 0 waits for the left rank's item at the same
position of phase f - 1 and adds that item's partial tile to its own product
("全归约 3：Ring——每步大小恒定", Walkthrough: in round s rank q adds its chunk
(q - s - 2) mod P to what its left neighbour sends).  The model checks that
every schedule finishes and that every rank ends with the sum of its chunk.

All-gather + GEMM: a tile of phase f reads its panel of chunk (q - f) mod P
(from an input block in phases 0 and 1, else from the left rank's gathered
buffer once the left rank's phase-(f - 1) tiles of the panel have flagged)
and copies its column tile's K range of the panel into rank q's gathered
buffer.  The model checks that every schedule finishes, that every tile
reads its whole panel after it was written, and that every gathered buffer
ends complete.

Each model plants a mistake that the checks must catch.
"""
import numpy as np
import pytest


# ------------------------------------------------------- GEMM + reduce-scatter
def _chunk(q, phase, P):
    """Chunk of rank q's phase (the kernel's schedule)."""
    if P == 1:
        return 0
    return (q - 1) % P if phase == 0 else (q - phase - 1) % P


def _gemm_rs_sim(P, tpc, G, rng, numbering="phase_major", wait_phase_offset=1):
    """Returns (finished, out) where out[q][pos] is rank q's final sum at
    tile position pos of its own chunk.  Products are random integers per
    (rank, chunk, position)."""
    prod = {(q, c, pos): int(rng.integers(-1000, 1000)) for q in range(P) for c in range(P)
            for pos in range(tpc)}
    items = P * P * tpc

    def decode(it):
        if numbering == "phase_major":
            return it // (P * tpc), (it // P) % tpc, it % P
        # planted: rank-major numbering, where a wait can point at a larger number
        q = it // (P * tpc)
        rem = it % (P * tpc)
        return rem // tpc, rem % tpc, q

    partial = {}        # (phase, q, pos) -> value published for the right neighbour
    out = {}
    nxt = [g for g in range(G)]   # each workgroup's current item
    while True:
        ready = []
        for g in range(G):
            it = nxt[g]
            if it >= items:
                continue
            f, pos, q = decode(it)
            dep = (f - wait_phase_offset, (q - 1) % P, pos)
            if f == 0 or dep in partial:
                ready.append(g)
        if not ready:
            break
        g = ready[int(rng.integers(len(ready)))]
        f, pos, q = decode(nxt[g])
        c = _chunk(q, f, P)
        v = prod[(q, c, pos)]
        if f > 0:
            v += partial[(f - wait_phase_offset, (q - 1) % P, pos)]
        if f == P - 1:
            out[(q, pos)] = v
        else:
            partial[(f, q, pos)] = v
        nxt[g] += G
    finished = all(n >= items for n in nxt)
    want = {(q, pos): sum(prod[(r, q, pos)] for r in range(P)) for q in range(P) for pos in range(tpc)}
    return finished, out == want


@pytest.mark.parametrize("P,tpc", [(1, 3), (2, 1), (2, 5), (3, 4), (4, 16), (8, 2)])
def test_gemm_rs_items_always_finish_with_the_sums(P, tpc):
    rng = np.random.default_rng(900 + P * 31 + tpc)
    items = P * P * tpc
    for G in sorted({1, 2, P, P + 1, items // 2 or 1, items}):
        for _ in range(20):
            finished, right = _gemm_rs_sim(P, tpc, G, rng)
            assert finished, (P, tpc, G)
            assert right, (P, tpc, G)


def test_gemm_rs_rank_major_numbering_can_deadlock():
    """Numbering the items rank by rank puts a rank's later phases before
    the left rank's earlier ones: with few workgroups the schedule stalls."""
    rng = np.random.default_rng(910)
    stalls = 0
    for _ in range(20):
        finished, _ = _gemm_rs_sim(4, 4, 4, rng, numbering="rank_major")
        stalls += not finished
    assert stalls > 0


def test_gemm_rs_wrong_wait_is_caught():
    """Waiting for the phase before the previous one (a wrong flag row) adds
    the wrong partial: the sums come out wrong."""
    rng = np.random.default_rng(911)
    bad = 0
    for _ in range(10):
        finished, right = _gemm_rs_sim(4, 4, 64, rng, wait_phase_offset=2)
        bad += (not finished) or (not right)
    assert bad == 10


# ------------------------------------------------------------ all-gather + GEMM
def _ag_gemm_sim(P, tm_chunk, tn, groups, rng, skip_wait=False, flag_first=False):
    """Returns (finished, tiles_ok, gathered_ok).  Workgroup (group g, rank
    q) takes tile positions pos = g, g + groups, ... (pos = pr * tn + t: panel
    pr, column tile t) in every phase f, phases in order.  A tile of phase f
    reads the whole panel pr of chunk c = (q - f) mod P -- from rank q's own
    block (f = 0), the left rank's own block (f = 1) or the left rank's
    gathered buffer (f >= 2), waiting for the left rank's tn phase-(f - 1)
    tiles of that panel -- and copies K range t of it into its own gathered
    buffer, then flags (f, q, pos).  A token (c, pr, t) names a piece of the
    data.  Planted: skip_wait reads without waiting; flag_first sets the flag
    before the copy lands."""
    tpc = tm_chunk * tn
    gathered = [[[[None] * tn for _ in range(tm_chunk)] for _ in range(P)] for _ in range(P)]
    flags = set()       # (phase, rank, pos)
    tiles_ok = True

    def program(q, grp):
        left = (q - 1) % P
        steps = []
        for f in range(P):
            for pos in range(grp, tpc, groups):
                pr = pos // tn
                waits = [] if (f < 2 or skip_wait) else [(f - 1, left, pr * tn + t) for t in range(tn)]
                if flag_first:
                    steps.append((waits, ("flag", q, f, pos)))
                    steps.append(([], ("tile", q, f, pos)))
                else:
                    steps.append((waits, ("tile", q, f, pos)))
                    steps.append(([], ("flag", q, f, pos)))
        return steps

    progs = {(q, g): program(q, g) for q in range(P) for g in range(groups)}
    pc = {k: 0 for k in progs}
    while True:
        ready = [k for k in progs if pc[k] < len(progs[k])
                 and all(w in flags for w in progs[k][pc[k]][0])]
        if not ready:
            break
        k = ready[int(rng.integers(len(ready)))]
        _, act = progs[k][pc[k]]
        pc[k] += 1
        _, q, f, pos = act
        if act[0] == "flag":
            if 1 <= f <= P - 2:
                flags.add((f, q, pos))
            continue
        left = (q - 1) % P
        c = (q - f) % P
        pr, t = pos // tn, pos % tn
        if f < 2:
            panel = [(c, pr, u) for u in range(tn)]            # an input block: always whole
        else:
            panel = list(gathered[left][c][pr])
        tiles_ok &= panel == [(c, pr, u) for u in range(tn)]
        gathered[q][c][pr][t] = panel[t]
    finished = all(pc[k] == len(progs[k]) for k in progs)
    gathered_ok = all(gathered[q][c][pr][t] == (c, pr, t) for q in range(P) for c in range(P)
                      for pr in range(tm_chunk) for t in range(tn))
    return finished, tiles_ok, gathered_ok


@pytest.mark.parametrize("P,tm_chunk,tn,groups", [(1, 2, 2, 2), (2, 1, 2, 2), (3, 2, 2, 1), (4, 2, 4, 3),
                                                  (4, 1, 16, 16), (8, 1, 2, 1), (5, 2, 3, 4)])
def test_ag_gemm_every_schedule_finishes_with_whole_panels(P, tm_chunk, tn, groups):
    rng = np.random.default_rng(920 + P + tn + groups)
    for _ in range(15):
        finished, tiles_ok, gathered_ok = _ag_gemm_sim(P, tm_chunk, tn, groups, rng)
        assert finished and tiles_ok and gathered_ok, (P, tm_chunk, tn, groups)


@pytest.mark.parametrize("mistake", ["skip_wait", "flag_first"])
def test_ag_gemm_planted_mistakes_are_caught(mistake):
    """A tile that reads the left rank's gathered panel without waiting, or a
    flag set before its tile's copy, lets some schedule read a hole."""
    rng = np.random.default_rng(930)
    caught = 0
    for _ in range(30):
        finished, tiles_ok, gathered_ok = _ag_gemm_sim(4, 2, 4, 2, rng, **{mistake: True})
        caught += not (finished and tiles_ok and gathered_ok)
    assert caught > 0
