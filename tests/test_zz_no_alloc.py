"""GPU test of ring_all_reduce_noalloc, the all-reduce for callers that
cannot allocate: its flags, words and partial sums live in the library's
static device array.  Through the C ABI, every case runs two calls in a row,
the second on a smaller input, and each output must equal ring_all_reduce's
(the entry point with a caller-owned workspace) bit for bit -- and the
oracle's.  Sizes the array cannot hold are rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc
from ring_collectives_amd import inputs

from _gpu_helpers import bits, empty_ranks, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()
    yield


def _data(kind, P, n, seed):
    if kind == "f32":
        return inputs.normal_f32(P, n, seed=seed)
    if kind == "bf16":
        return inputs.normal_bf16(P, n, seed=seed, std=1.0)
    rng = np.random.default_rng(seed)
    return rng.integers(-1000, 1000, size=(P, n), endpoint=True, dtype=np.int32)


def _want(kind, x):
    return oracle.all_reduce_bf16(x) if kind == "bf16" else oracle.all_reduce(x)


# (dtype, (P, n) of the first call, (P, n) of the second, smaller call)
CASES = [
    ("f32", (8, 64 << 20), (8, 1 << 20)),        # the headline size, then a flag-round call
    ("f32", (4, 4 * 4096), (2, 2 * 1024)),       # low-latency rounds, both
    ("bf16", (4, 655360), (4, 1 << 16)),         # flag rounds with the fp32 partial sums, then low-latency
    ("bf16", (4, 4 * 4096), (3, 3 * 256)),       # low-latency rounds
    ("i32", (8, 8 * 1024), (4, 4 * 128)),
    ("f32", (6, 6 * 100003), (5, 5 * 7)),        # ragged chunks
]


@pytest.mark.parametrize("kind,first,second", CASES)
def test_two_calls_match_the_workspace_entry_point(kind, first, second):
    for call, (P, n) in enumerate((first, second)):
        note("noalloc %s P=%d n=%d call %d" % (kind, P, n, call))
        x = _data(kind, P, n, seed=960 + call)
        src = to_dev(x, kind)
        got = empty_ranks(P, n, kind)
        rc.all_reduce_noalloc(src, got)
        ref = empty_ranks(P, n, kind)
        ws = rc.all_reduce(src, ref)
        assert rc.last_error(ws)[0] == 0
        g, r = to_host(got, kind), to_host(ref, kind)
        np.testing.assert_array_equal(bits(g), bits(r), err_msg="call %d" % call)
        np.testing.assert_array_equal(bits(g), bits(_want(kind, x)), err_msg="call %d" % call)


def test_in_place_and_one_rank():
    P, n = 4, 4 << 16
    x = _data("f32", P, n, 970)
    buf = to_dev(x, "f32")
    note("noalloc in place")
    rc.all_reduce_noalloc(buf, buf)
    np.testing.assert_array_equal(bits(to_host(buf, "f32")), bits(oracle.all_reduce(x)))
    one = to_dev(x[:1], "f32")
    out = empty_ranks(1, n, "f32")
    rc.all_reduce_noalloc(one, out)
    np.testing.assert_array_equal(bits(to_host(out, "f32")), bits(x[:1]))


@pytest.mark.parametrize("kind,P,n", [("f32", 4, 4 * (3 * 4096 + 96)), ("f32", 4, 4 * 4096), ("bf16", 4, 655360)])
def test_captured_in_a_graph(kind, P, n):
    """The case the entry point is for: captured in a HIP graph (it records
    no allocation and no memset; the static array's flags are cleared by a
    fill kernel) and replayed three times, with an eager call of the same
    entry point on another, smaller input between replays (the one static
    array serves both, in stream order); every replay bit for bit against
    the oracle."""
    note("noalloc graph %s P=%d n=%d" % (kind, P, n))
    x = _data(kind, P, n, 972)
    src, dst = to_dev(x, kind), empty_ranks(P, n, kind)
    other = _data(kind, 3, 3 * 1000, 973)
    other_src, other_dst = to_dev(other, kind), empty_ranks(3, 3 * 1000, kind)
    rc.all_reduce_noalloc(src, dst)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc.all_reduce_noalloc(src, dst)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in src:
            t.neg_()                                              # eager input change (exact)
        for t in dst:
            t.view(torch.int16 if kind == "bf16" else torch.int32).fill_(-1)
        rc.all_reduce_noalloc(other_src, other_dst)               # eager call, same static array
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(_want(kind, to_host(src, kind))),
                                      err_msg="replay %d" % rep)
        np.testing.assert_array_equal(bits(to_host(other_dst, kind)), bits(_want(kind, other)))


def test_too_large_is_rejected_before_any_launch():
    """P = 8 with 128 Mi fp32 per rank needs a flag table larger than the
    static array: RING_EWORKSPACE, synchronously; a normal call follows."""
    P, n = 8, 128 << 20
    src = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(P)]
    with pytest.raises(N.RingError) as e:
        rc.all_reduce_noalloc(src, src)
    assert e.value.code == N.RING_EWORKSPACE
    del src
    x = _data("f32", 4, 4096, 971)
    out = empty_ranks(4, 4096, "f32")
    rc.all_reduce_noalloc(to_dev(x, "f32"), out)
    np.testing.assert_array_equal(bits(to_host(out, "f32")), bits(oracle.all_reduce(x)))
