"""CPU model of the chunk-step kernel's flag protocol, run under random
schedules -- a race detector for the protocol itself.

The model mirrors what one wave of the kernel does for tile j of rank r in
round k ("全归约 3：Ring——每步大小恒定", Walkthrough; tiles as in
"Triton-distributed 语义", producer/consumer):
  * reduce-scatter round s = k (k < P-1): chunk c = (r - s - 2) mod P,
    read own src[r][c] and the left neighbour's src[left][c] (s = 0) or
    dst[left][c] (s > 0), write dst[r][c] = own + recv;
  * all-gather round t = k - (P-1): chunk c = (r - t - 1) mod P,
    read dst[left][c], write dst[r][c];
  * the read may start once flag (k, left, j) is set (the left rank wrote
    tile j in round k-1) and this wave finished its own round k-1; the
    flag (k+1, r, j) is set only after the write completed.
Each task is split into a read action and a write action, and the scheduler
interleaves all ready actions at random, so any write-after-read or stale
read the flags do not prevent would change the result.  Runs in place
(dst == src, the harshest aliasing) and out of place, and is compared with
the oracle bit for bit.  A planted protocol bug (one wait dropped) must be
caught.
"""
import random

import numpy as np
import pytest

import oracle


def _simulate(x, T, rng, in_place, rounds=None, drop_wait=None):
    """Run the all-reduce protocol on (P, n) fp32 data with T tiles per chunk
    under one random schedule; returns dst."""
    P, n = x.shape
    C = n // P
    k_end = 2 * (P - 1) if rounds is None else rounds
    src = x.copy()
    dst = src if in_place else np.full_like(src, np.nan)
    bounds = [(j * C // T, (j + 1) * C // T) for j in range(T)]

    def left(r):
        return (r - 1 + P) % P

    def action(k, r, j):
        lo, hi = bounds[j]
        if k < P - 1:
            c = (r - k - 2 + 2 * P) % P
            own = src[r, c * C + lo:c * C + hi].copy()
            recv_buf = src if k == 0 else dst
            recv = recv_buf[left(r), c * C + lo:c * C + hi].copy()
            return c, (own + recv).astype(np.float32)
        t = k - (P - 1)
        c = (r - t - 1 + P) % P
        return c, dst[left(r), c * C + lo:c * C + hi].copy()

    done_write = set()                 # (k, r, j) whose write completed
    read_result = {}                   # (k, r, j) -> (c, values) read, not yet written
    next_round = {(r, j): 0 for r in range(P) for j in range(T)}

    def ready_reads():
        out = []
        for (r, j), k in next_round.items():
            if k >= k_end or (k, r, j) in read_result:
                continue
            if k > 0 and (k - 1, r, j) not in done_write:
                continue                             # this wave's own previous round
            needs_flag = k > 0 and drop_wait != (k, r)
            if needs_flag and (k - 1, left(r), j) not in done_write:
                continue                             # flag (k, left, j) not yet set
            out.append((k, r, j))
        return out

    while True:
        reads = ready_reads()
        writes = list(read_result)
        if not reads and not writes:
            break
        pick = rng.choice(reads + writes)
        if pick in read_result:
            k, r, j = pick
            c, vals = read_result.pop(pick)
            lo, hi = bounds[j]
            dst[r, c * C + lo:c * C + hi] = vals
            done_write.add(pick)
            next_round[(r, j)] = k + 1
        else:
            read_result[pick] = action(*pick)
    return dst


@pytest.mark.parametrize("P", [2, 3, 4, 5])
@pytest.mark.parametrize("in_place", [True, False])
def test_random_schedules_match_oracle(P, in_place):
    rng = random.Random(1000 + 10 * P + in_place)
    T = 3
    x = np.random.default_rng(P).standard_normal((P, P * T * 2)).astype(np.float32)
    want = oracle.all_reduce(x)
    for _ in range(150):
        got = _simulate(x, T, rng, in_place)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_random_schedules_p8():
    rng = random.Random(7)
    P, T = 8, 2
    x = np.random.default_rng(8).standard_normal((P, P * T)).astype(np.float32)
    want = oracle.all_reduce(x)
    for _ in range(60):
        got = _simulate(x, T, rng, in_place=True)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_reduce_scatter_only_rounds():
    """Stopping after the P-1 reduce-scatter rounds leaves each owner chunk
    complete, whatever the schedule."""
    rng = random.Random(3)
    P, T = 4, 2
    x = np.random.default_rng(4).integers(-100, 100, size=(P, P * T * 3)).astype(np.float32)
    want = oracle.reduce_scatter(x)
    C = x.shape[1] // P
    for _ in range(100):
        got = _simulate(x, T, rng, in_place=False, rounds=P - 1)
        for r in range(P):
            np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C])


@pytest.mark.parametrize("drop", [(1, 0), (2, 2), (4, 1)])
def test_planted_missing_wait_is_caught(drop):
    """Remove one wait (rank drop[1] ignores flag row drop[0]): some random
    schedule must then read a tile before its neighbour wrote it."""
    rng = random.Random(11)
    P, T = 4, 2
    x = np.random.default_rng(5).standard_normal((P, P * T * 2)).astype(np.float32)
    want = oracle.all_reduce(x)
    caught = False
    for _ in range(300):
        got = _simulate(x, T, rng, in_place=True, drop_wait=drop)
        if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
            caught = True
            break
    assert caught


# ---------------------------------------------------------------------------
# The low-latency rounds: the value a rank passes right travels in a word
# with a ready mark instead of behind a flag.  A wave's round k reads its own
# input and (k > 0) the words (k - 1, left, j), clearing them as it takes
# them; its write action stores the result into dst and sets the words
# (k, r, j).  Nothing else orders the ranks: the in-place hazards (rank r's
# all-gather overwriting the input chunk rank r+1 reads in round 0) must be
# ordered by the chain of words alone.
def _simulate_ll(x, T, rng, in_place, words, drop_wait=None):
    P, n = x.shape
    C = n // P
    k_end = 2 * (P - 1)
    src = x.copy()
    dst = src if in_place else np.full_like(src, np.nan)
    bounds = [(j * C // T, (j + 1) * C // T) for j in range(T)]

    def left(r):
        return (r - 1 + P) % P

    def read(k, r, j):
        lo, hi = bounds[j]
        if k > 0:
            got = words.pop((k - 1, left(r), j), None)
            recv = got if got is not None else np.zeros(hi - lo, np.float32)
        if k < P - 1:
            c = (r - k - 2 + 2 * P) % P
            own = src[r, c * C + lo:c * C + hi].copy()
            if k == 0:
                recv = src[left(r), c * C + lo:c * C + hi].copy()
            return c, (own + recv).astype(np.float32)
        t = k - (P - 1)
        return (r - t - 1 + P) % P, recv

    pending = {}
    next_round = {(r, j): 0 for r in range(P) for j in range(T)}
    while True:
        reads = []
        for (r, j), k in next_round.items():
            if k >= k_end or (k, r, j) in pending:
                continue
            if k > 0 and drop_wait != (k, r) and (k - 1, left(r), j) not in words:
                continue                             # the marks are not set yet
            reads.append((k, r, j))
        writes = list(pending)
        if not reads and not writes:
            break
        pick = rng.choice(reads + writes)
        if pick in pending:
            k, r, j = pick
            c, vals = pending.pop(pick)
            lo, hi = bounds[j]
            dst[r, c * C + lo:c * C + hi] = vals
            if k + 1 < k_end:
                words[(k, r, j)] = vals.copy()
            next_round[(r, j)] = k + 1
        else:
            pending[pick] = read(*pick)
    return dst


@pytest.mark.parametrize("P", [2, 3, 4, 5])
@pytest.mark.parametrize("in_place", [True, False])
def test_ll_random_schedules_match_oracle(P, in_place):
    """Two launches in a row on one set of words: each gives the oracle's
    bits, and each leaves every word taken (cleared)."""
    rng = random.Random(2000 + 10 * P + in_place)
    T = 3
    x = np.random.default_rng(20 + P).standard_normal((P, P * T * 2)).astype(np.float32)
    want = oracle.all_reduce(x)
    for _ in range(100):
        words = {}
        for launch in range(2):
            got = _simulate_ll(x, T, rng, in_place, words)
            np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32), err_msg="launch %d" % launch)
            assert not words


@pytest.mark.parametrize("drop", [(1, 0), (3, 2), (5, 1)])
def test_ll_planted_missing_wait_is_caught(drop):
    """Rank drop[1] takes round drop[0]'s words without waiting for their
    marks: some schedule must then take a word before it was written."""
    rng = random.Random(13)
    P, T = 4, 2
    x = np.random.default_rng(6).standard_normal((P, P * T * 2)).astype(np.float32)
    want = oracle.all_reduce(x)
    caught = False
    for _ in range(300):
        got = _simulate_ll(x, T, rng, True, {}, drop_wait=drop)
        if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
            caught = True
            break
    assert caught
