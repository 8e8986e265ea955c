"""GPU tests of the ring collectives on rank buffers larger than 4 GiB, and of
the fused GEMMs with outputs (and partial tiles) larger than 4 GiB.

P = 2 and n = 5 * 2^28 + 4098 elements per rank (about 5 GiB of int32 per
rank; chunks of 671,090,689 elements, so the second chunk starts past 2^31
bytes and a rank buffer ends past 2^32 bytes; the chunks end in a partial
tile).  Every offset into a rank buffer, the flag table, the bf16 carry
and the psum slots must be 64-bit.  The inputs are a fixed pattern of
small integers, made on the device; the checks:
  * windows around the first element, the 2^31- and 2^32-byte offsets, the
    chunk boundary and the last element, against the oracle on the same
    windows (sums of small integers are exact in any order);
  * at every element, properties that hold at any size: ppermute's output
    is the left rank's input, the all-gather's every chunk is its piece,
    the all-reduce and the psum leave the same sum on every rank.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc

from _gpu_helpers import note

pytestmark = pytest.mark.gpu

P = 2
n = 5 * (1 << 28) + 4098
C = n // P
WIN = 4096
STARTS = sorted({0, (1 << 29) - WIN // 2, (1 << 30) - WIN // 2, C - WIN // 2, n - WIN})


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()
    yield


def _pattern_host(r, a, b, lo, hi):
    i = np.arange(a, b, dtype=np.int64)
    return ((i * 7919 + r * 104729) % (hi - lo + 1) + lo)


def _pattern_dev(r, dtype, lo, hi):
    out = torch.empty(n, dtype=dtype, device="cuda")
    step = 1 << 27
    for a in range(0, n, step):
        b = min(n, a + step)
        i = torch.arange(a, b, dtype=torch.int64, device="cuda")
        out[a:b] = ((i * 7919 + r * 104729) % (hi - lo + 1) + lo).to(dtype)
    return out


def _windows(ts, r):
    return np.concatenate([ts[r][a:a + WIN].float().cpu().numpy() for a in STARTS])


def _host_windows(lo, hi):
    """(P, windows) of the inputs, as the oracle takes them."""
    return np.stack([np.concatenate([_pattern_host(r, a, a + WIN, lo, hi) for a in STARTS])
                     for r in range(P)]).astype(np.int32)


def _sum_windows(lo, hi):
    x = _host_windows(lo, hi)
    return oracle.all_reduce(x)[0].astype(np.float64)


def _in_chunk(r):
    """Mask of the window elements that lie in chunk r."""
    idx = np.concatenate([np.arange(a, a + WIN) for a in STARTS])
    return (idx >= r * C) & (idx < (r + 1) * C)


def test_ppermute_and_all_gather_over_4_gib():
    note("max size: ppermute and all-gather, P=2 n=%d int32" % n)
    src = [_pattern_dev(r, torch.int32, -1001, 1001) for r in range(P)]
    dst = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for _ in range(P)]
    rc.ppermute(src, dst)
    torch.cuda.synchronize()
    for r in range(P):
        assert torch.equal(dst[r], src[(r - 1) % P]), "ppermute rank %d" % r
    pieces = [s[r * C:(r + 1) * C].clone() for r, s in enumerate(src)]
    for t in dst:
        t.fill_(-7)
    ws = rc.all_gather(dst, src=pieces)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    for r in range(P):
        for c in range(P):
            assert torch.equal(dst[r][c * C:(c + 1) * C], pieces[c]), "all-gather rank %d chunk %d" % (r, c)


@pytest.mark.parametrize("kind", ["i32", "bf16"])
def test_all_reduce_over_4_gib(kind):
    """int32 in [-1001, 1001]; bf16 in [-64, 64] (sums exact in bf16), which
    also puts the fp32 carry (P n floats) past 4 GiB."""
    note("max size: all-reduce %s" % kind)
    dt, lo, hi = (torch.int32, -1001, 1001) if kind == "i32" else (torch.bfloat16, -64, 64)
    src = [_pattern_dev(r, dt, lo, hi) for r in range(P)]
    dst = [torch.empty(n, dtype=dt, device="cuda") for _ in range(P)]
    ws = rc.all_reduce(src, dst)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    assert torch.equal(dst[0], dst[1])
    want = _sum_windows(lo, hi)
    np.testing.assert_array_equal(_windows(dst, 0), want)


@pytest.mark.parametrize("op", ["reduce_scatter", "bidir", "psum"])
def test_reduce_scatter_forms_over_4_gib(op):
    note("max size: %s" % op)
    src = [_pattern_dev(r, torch.int32, -1001, 1001) for r in range(P)]
    dst = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for _ in range(P)]
    fn = {"reduce_scatter": rc.reduce_scatter, "bidir": rc.reduce_scatter_bidir,
          "psum": rc.psum_circulating}[op]
    ws = fn(src, dst)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    want = _sum_windows(-1001, 1001)
    for r in range(P):
        got = _windows(dst, r)
        mask = np.ones_like(want, dtype=bool) if op == "psum" else _in_chunk(r)
        np.testing.assert_array_equal(got[mask], want[mask], err_msg="%s rank %d" % (op, r))
    if op == "psum":
        assert torch.equal(dst[0], dst[1])


# ------------------------------------------------------------ fused GEMMs
def _dev_bf16(x):
    return [torch.from_numpy(np.ascontiguousarray(x[q]).view(np.int16)).cuda().view(torch.bfloat16)
            for q in range(x.shape[0])]


def test_all_gather_gemm_output_over_4_gib():
    """P = 2, M = 40960, N = 32768, K = 64 on integer-valued operands (every
    product exact): C is 5 GiB of fp32 per rank.  Rows around the 2^31- and
    2^32-byte offsets of C and the last rows, bit for bit against the
    oracle's fp64 rows; the gathered A everywhere."""
    from ring_collectives_amd import inputs
    Pg, M, Nn, K = 2, 40960, 32768, 64
    note("max size: all_gather_gemm P=%d M=%d N=%d K=%d" % (Pg, M, Nn, K))
    rng = np.random.default_rng(1400)
    As = inputs.small_int_bf16(rng, (Pg, M // Pg, K))
    B = inputs.small_int_bf16(rng, (Pg, K, Nn))
    a, b = _dev_bf16(As), _dev_bf16(B)
    full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(Pg)]
    Cs = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(Pg)]
    ws = rc.all_gather_gemm(a, b, full, Cs)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    want_full = As.reshape(M, K)
    rows = np.array([0, 1, 16383, 16384, 20479, 20480, 32767, 32768, M - 2, M - 1])
    for q in range(Pg):
        np.testing.assert_array_equal(full[q].view(torch.int16).cpu().numpy().view(np.uint16), want_full)
        want, _ = oracle.all_gather_gemm_rows_f64(As, B, q, rows)
        got = Cs[q][torch.from_numpy(rows).cuda()].cpu().numpy()
        np.testing.assert_array_equal(got, want.astype(np.float32), err_msg="rank %d" % q)


def test_gemm_reduce_scatter_output_over_4_gib():
    """P = 2, M = 81920, N = 32768, K = 64 on integer-valued operands: each
    output is 5 GiB of fp32 and the partial tiles take 20 GiB of workspace.
    Rows around the 2^31- and 2^32-byte offsets and the last rows of each
    output, bit for bit against the oracle's fp64 rows."""
    from ring_collectives_amd import inputs
    Pg, M, Nn, K = 2, 81920, 32768, 64
    note("max size: gemm_reduce_scatter P=%d M=%d N=%d K=%d" % (Pg, M, Nn, K))
    rng = np.random.default_rng(1410)
    A = inputs.small_int_bf16(rng, (Pg, M, K))
    B = inputs.small_int_bf16(rng, (Pg, K, Nn))
    a, b = _dev_bf16(A), _dev_bf16(B)
    out = [torch.empty((M // Pg, Nn), dtype=torch.float32, device="cuda") for _ in range(Pg)]
    ws = rc.gemm_reduce_scatter(a, b, out)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    rows = np.array([0, 1, 16383, 16384, 32767, 32768, M // Pg - 2, M // Pg - 1])
    for r in range(Pg):
        want, _ = oracle.gemm_reduce_scatter_rows_f64(A, B, r, rows)
        got = out[r][torch.from_numpy(rows).cuda()].cpu().numpy()
        np.testing.assert_array_equal(got, want.astype(np.float32), err_msg="rank %d" % r)
