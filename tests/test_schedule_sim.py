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

All-gather + GEMM: workgroup (group g, rank q) forwards its slices of phase
f + 1 (waiting for the left rank's slice of phase f) and then computes its
tiles of phase f (waiting for every slice of the tile's panel).  The model
checks that every schedule finishes, that every tile reads its whole panel
after it was written, and that every gathered buffer ends complete.

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
def _ag_gemm_sim(P, tm_chunk, tn, groups, rng, ahead=True, skip_forward_wait=False):
    """Returns (finished, tiles_ok, gathered_ok).  Slices are the kernel's:
    tile position pos = pr * tn + t forwards rows 256 t / tn .. of panel pr;
    here a slice is one token that names (source chunk, panel, slice)."""
    tpc = tm_chunk * tn
    # gathered[q][c][pos] holds the token of chunk c's slice pos, or None
    gathered = [[[None] * tpc for _ in range(P)] for _ in range(P)]
    flags = set()       # (phase, rank, pos)
    tiles_ok = True

    def token(c, pos):
        return (c, pos)

    # each workgroup's program as a list of steps; a step is (wait_keys, action)
    def program(q, grp):
        left = (q - 1) % P
        mine = list(range(grp, tpc, groups))
        steps = []
        for pos in mine:                                # place the local block
            steps.append(([], ("place", q, pos)))

        def forward(g_):
            for pos in mine:
                waits = [] if (g_ < 2 or skip_forward_wait) else [(g_ - 1, left, pos)]
                steps.append((waits, ("fwd", q, g_, pos)))

        for f in range(P):
            if ahead and f + 1 < P:
                forward(f + 1)
            if not ahead and f >= 1:
                forward(f)
            for pos in mine:
                pr = pos // tn
                waits = [] if f == 0 else [(f, q, pr * tn + t) for t in range(tn)]
                steps.append((waits, ("tile", q, f, pos)))
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
        if act[0] == "place":
            _, q, pos = act
            gathered[q][q][pos] = token(q, pos)
        elif act[0] == "fwd":
            _, q, g_, pos = act
            left = (q - 1) % P
            c = (q - g_) % P
            # phase 1 copies the left rank's own shard; later phases its gathered buffer
            src = token(c, pos) if g_ == 1 else gathered[left][c][pos]
            gathered[q][c][pos] = src
            flags.add((g_, q, pos))
        else:
            _, q, f, pos = act
            c = (q - f) % P
            pr = pos // tn
            if f > 0:
                panel = [gathered[q][c][pr * tn + t] for t in range(tn)]
                tiles_ok &= panel == [token(c, pr * tn + t) for t in range(tn)]
    finished = all(pc[k] == len(progs[k]) for k in progs)
    gathered_ok = all(gathered[q][c][pos] == token(c, pos) for q in range(P) for c in range(P)
                      for pos in range(tpc))
    return finished, tiles_ok, gathered_ok


@pytest.mark.parametrize("P,tm_chunk,tn,groups", [(1, 2, 2, 2), (2, 1, 2, 2), (3, 2, 2, 1), (4, 2, 4, 3),
                                                  (4, 1, 16, 16), (8, 1, 2, 1)])
@pytest.mark.parametrize("ahead", [True, False])
def test_ag_gemm_every_schedule_finishes_with_whole_panels(P, tm_chunk, tn, groups, ahead):
    rng = np.random.default_rng(920 + P + tn + groups)
    for _ in range(15):
        finished, tiles_ok, gathered_ok = _ag_gemm_sim(P, tm_chunk, tn, groups, rng, ahead=ahead)
        assert finished and tiles_ok and gathered_ok, (P, tm_chunk, tn, groups, ahead)


def test_ag_gemm_forward_without_wait_is_caught():
    """Forwarding a slice before the left rank has it copies a hole: some
    schedule gives a tile a panel with a missing slice or leaves a gathered
    buffer incomplete."""
    rng = np.random.default_rng(930)
    caught = 0
    for _ in range(30):
        finished, tiles_ok, gathered_ok = _ag_gemm_sim(4, 2, 4, 2, rng, skip_forward_wait=True)
        caught += not (finished and tiles_ok and gathered_ok)
    assert caught > 0
