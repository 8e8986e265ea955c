"""GPU parity of the circulating-input psum ("Pallas TPU Distributed
Collectives 复习文档", section 3) against the CPU oracle, through the C ABI:
every rank's result bit for bit (each rank adds in its own order, x_{r-1}
first and its own input last, exactly as the oracle does)."""
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


@pytest.fixture(autouse=True)
def _default_tuning():
    old = N.get_tuning()
    yield
    N.set_tuning(**old)


def _run(x, kind, in_place=False, ws=None):
    src = to_dev(x, kind)
    dst = src if in_place else empty_ranks(x.shape[0], x.shape[1], kind)
    ws = rc.psum_circulating(src, dst, ws=ws)
    got = to_host(dst, kind)
    assert rc.last_error(ws)[0] == 0
    return got


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("n", [1, 7, 4096, (1 << 20) + 12, 1 << 20])
def test_psum_f32(P, n):
    note("psum f32 P=%d n=%d" % (P, n))
    x = inputs.normal_f32(P, n, seed=70 + n % 97) if n > 1 else np.ones((P, 1), np.float32)
    want, _ = oracle.psum_circulating(x)
    np.testing.assert_array_equal(bits(_run(x, "f32")), bits(want))


@pytest.mark.parametrize("P", [2, 4, 8])
def test_psum_int32(P):
    note("psum int32 P=%d" % P)
    x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    got = _run(x, "i32")
    want, _ = oracle.psum_circulating(x)
    np.testing.assert_array_equal(got, want)
    total = x.astype(np.int64).sum(axis=0)
    for r in range(P):
        np.testing.assert_array_equal(got[r].astype(np.int64), total)


@pytest.mark.parametrize("P", [2, 4, 16])
@pytest.mark.parametrize("n", [8, 4096 * 3 + 8, 1001])
def test_psum_bf16(P, n):
    note("psum bf16 P=%d n=%d" % (P, n))
    x = inputs.normal_bf16(P, n, seed=71 + P)
    np.testing.assert_array_equal(_run(x, "bf16"), oracle.psum_circulating_bf16(x))


def test_psum_page_order_wide_range():
    """Data whose fp32 sums depend on the order: each rank's own order."""
    P, n = 4, 8192
    rng = np.random.default_rng(72)
    x = (rng.standard_normal((P, n)) * np.exp2(rng.integers(-20, 20, size=(P, n)))).astype(np.float32)
    note("psum wide range")
    got = _run(x, "f32")
    want, _ = oracle.psum_circulating(x)
    np.testing.assert_array_equal(bits(got), bits(want))
    assert any(np.any(bits(got[r]) != bits(got[0])) for r in range(1, P))


def test_psum_in_place_tuning_repeated():
    P, n = 8, 300000
    x = inputs.normal_f32(P, n, seed=73)
    want, _ = oracle.psum_circulating(x)
    note("psum in place")
    np.testing.assert_array_equal(bits(_run(x, "f32", in_place=True)), bits(want))
    ws = rc.workspace(N.OP_PSUM_CIRCULATING, P, n, torch.float32)
    for tv in (4, 16, 8):
        note("psum tile_vecs=%d" % tv)
        N.set_tuning(tile_vecs=tv)
        np.testing.assert_array_equal(bits(_run(x, "f32", ws=ws)), bits(want))


def test_psum_errors_and_watchdog():
    P, n = 4, 4096 * 4
    x = inputs.normal_f32(P, n, seed=74)
    src = to_dev(x, "f32")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.psum_circulating(src, src, ws=small)
    assert e.value.code == N.RING_EWORKSPACE
    dst = empty_ranks(P, n, "f32")
    ws = rc.workspace(N.OP_PSUM_CIRCULATING, P, n, torch.float32)
    note("psum watchdog drop_round=2")
    N.set_tuning(drop_round=2, timeout_s=0.05)
    rc.psum_circulating(src, dst, ws=ws)
    code, info = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    rc.psum_circulating(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    want, _ = oracle.psum_circulating(x)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(want))


def test_psum_full_size_fp32_p8_64Mi():
    """P = 8, 64 Mi fp32 per rank (the bandwidth workload's inputs): the sum
    is elementwise, so the oracle on a sample of columns gives exactly those
    elements of every rank's result."""
    P, n = 8, 64 << 20
    note("psum full size generate")
    x = inputs.normal_f32(P, n, seed=inputs.SEED_F32_BW)
    note("psum full size run")
    got = _run(x, "f32")
    idx = np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(2).integers(0, n, size=1 << 16)]))
    want, _ = oracle.psum_circulating(np.ascontiguousarray(x[:, idx]))
    np.testing.assert_array_equal(bits(np.ascontiguousarray(got[:, idx])), bits(want))
