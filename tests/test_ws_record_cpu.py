"""CPU checks of the workspace's record of data left behind, with no GPU:
the library's workspace sizes against the layout the record relies on
(status block, flags, low-latency words, then the bf16 partial sums), and
the claims the GPU tests build on:
  * the status block is the first 256 bytes, and every flag table, word
    region and data region lies past it;
  * for one shape and operation, the span a call leaves data in lies above
    the span it checks (from the end of the status block through its flags
    or words), in either kind of rounds, so calls of one shape never trip
    the check;
  * the scenario of the GPU test (a bf16 all-reduce at P = 4, 1 Mi per rank,
    then an fp32 all-reduce at P = 8, 1 Mi per rank, on the same workspace)
    really puts the second call's flags over the first one's partial sums.
The layout below is the one ring_collectives.h and the design notes state:
[status 256 B | flags, one per 64 B, (2(P-1)) x P x T with T = ceil(C /
tile) + 1 and tile the smallest one (1024 elements) | words, 8 B per
element and round, for chunks of at most 256 KiB whose words take at most
64 MiB | bf16 only: P n fp32 partial sums], each part 256-byte aligned."""
import pytest

from ring_collectives_amd import _native as N

F32, BF16, I32 = N.RING_F32, N.RING_BF16, N.RING_I32
ESZ = {F32: 4, BF16: 2, I32: 4}


def _up(x):
    return (x + 255) // 256 * 256


def layout(P, n, dt, with_ll=True):
    C = n // P
    T = -(-C // 1024) + 1
    rows = 2 * (P - 1) if P > 1 else 1
    flags = (256, 256 + _up(rows * P * T * 64))
    ll_ok = P > 1 and C * ESZ[dt] <= 256 << 10 and 2 * (P - 1) * n * 8 <= 64 << 20
    words = (flags[1], flags[1] + (_up(rows * n * 8) if with_ll and ll_ok else 0))
    carry = (words[1], words[1] + (_up(P * n * 4) if dt == BF16 else 0))
    return {"flags": flags, "words": words, "carry": carry}


def overlaps(a, b):
    return a[1] > a[0] and b[1] > b[0] and a[0] < b[1] and b[0] < a[1]


SHAPES = [(P, n, dt) for P in (2, 3, 4, 8, 16) for n in (P * 256, P * 4096, P * 65536, P * (1 << 18), P * (1 << 20))
          for dt in (F32, BF16, I32)]


@pytest.mark.parametrize("P,n,dt", SHAPES)
def test_layout_matches_the_library(P, n, dt):
    L = layout(P, n, dt)
    assert N.lib().ring_workspace_bytes(N.OP_ALL_REDUCE, P, n, dt) == L["carry"][1]
    assert N.lib().ring_workspace_bytes(N.OP_ALL_GATHER, P, n, dt) == L["words"][1]


@pytest.mark.parametrize("P,n,dt", SHAPES)
def test_one_shape_never_trips(P, n, dt):
    L = layout(P, n, dt)
    for part in ("flags", "words", "carry"):
        assert L[part][0] >= 256
    # the span a launch checks runs from the end of the status block through
    # its flags (flag rounds) or its words (low-latency rounds); the carry of
    # the flag rounds is what stays behind, above it
    for zero in ((256, L["flags"][1]), (256, L["words"][1])):
        assert not overlaps(zero, L["carry"]) and L["carry"][0] >= zero[1]


def test_gpu_scenario_overlaps():
    a = layout(4, 1 << 20, BF16)
    b = layout(8, 1 << 20, F32)
    assert a["words"][1] == a["words"][0]            # 512 KiB chunks: the flag rounds
    assert b["words"][1] == b["words"][0]
    assert overlaps(b["flags"], a["carry"])
    assert b["flags"][1] <= a["carry"][1]             # and the second call fits the first's workspace
