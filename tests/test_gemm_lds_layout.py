"""The fused GEMMs' LDS layout, on the CPU: where the direct global->LDS
loads put each operand element, where the fragment reads look for it, and
which banks the reads touch.

The address maps restate those of the MFMA tile (16-byte chunks of a row
XOR-ed with a function of the row).  The checks are properties, not a
second copy of the formulas: every element a fragment read asks for is the
element the loads stored there, every stored row is a permutation of its
chunks, and the 32 lanes of an 8-byte transposed read (or 16 of a 16-byte
read) of one cycle touch 256 distinct bytes of the 64 four-byte banks.
"""
import pytest


def swz_b(bn, k):
    return 4 * ((k >> 1) & 1) if bn == 64 else 4 * (k & 3)


def swz_a(m):
    return (m >> 1) & 7


@pytest.mark.parametrize("bn", [64, 128, 256])
def test_b_loads_and_transposed_reads_agree(bn):
    row_bytes = bn * 2
    bc = bn // 8                      # 16-byte chunks per row
    rows_per_load = 1024 // row_bytes
    bkb = 64 if bn == 256 else 32
    # loads: instruction i of the stage covers rows rows_per_load * i ..; lane
    # l stores at the next 16 bytes and fetches logical chunk (l % bc) ^ swz
    stored = {}
    for i in range(bkb // rows_per_load):
        for lane in range(64):
            k = i * rows_per_load + lane // bc
            logical = (lane % bc) ^ swz_b(bn, k)
            at = i * 1024 + lane * 16
            assert at == k * row_bytes + (lane % bc) * 16
            for e in range(8):
                stored[at + 2 * e] = (k, logical * 8 + e)
    assert len(stored) == bkb * bn
    # reads: lane l of a ds_read_b64_tr_b16 points at row krow, columns n .. n+3
    nwaves_across = {64: 2, 128: 2, 256: 4}[bn]
    wn = bn // nwaves_across
    for wc in range(nwaves_across):
        for ni in range(wn // 32):
            for kk in range(bkb // 16):
                for half in (0, 4):
                    banks = [set(), set()]
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        krow = 8 * (g >> 1) + (i >> 2) + half + 16 * kk
                        n = wc * wn + ni * 32 + 16 * (g & 1) + 4 * (i & 3)
                        chunk = (n >> 3) ^ swz_b(bn, krow)
                        at = krow * row_bytes + chunk * 16 + (n & 7) * 2
                        for e in range(4):
                            assert stored[at + 2 * e] == (krow, n + e), (bn, lane)
                        for b in range(8):
                            banks[lane // 32].add((at + b) % 256)
                    assert all(len(s) == 256 for s in banks), (bn, wc, ni, kk, half)


def test_a_loads_and_fragment_reads_agree():
    bka, row_bytes, chunks = 64, 128, 8
    stored = {}
    for i in range(256 // 8):         # 8 rows of 128 bytes per 1-KiB load
        for lane in range(64):
            m = i * 8 + lane // chunks
            logical = (lane % chunks) ^ swz_a(m)
            at = i * 1024 + lane * 16
            for e in range(8):
                stored[at + 2 * e] = (m, logical * 8 + e)
    assert len(stored) == 256 * bka
    for wr in range(2):
        for mi in range(4):
            for ka in range(bka // 16):
                banks = [set() for _ in range(4)]
                for lane in range(64):
                    m = wr * 128 + mi * 32 + (lane & 31)
                    chunk = (2 * ka + (lane >> 5)) ^ swz_a(lane & 31)
                    at = m * row_bytes + chunk * 16
                    for e in range(8):
                        assert stored[at + 2 * e] == (m, 16 * ka + 8 * (lane >> 5) + e)
                    for b in range(16):
                        banks[lane // 16].add((at + b) % 256)
                assert all(len(s) == 256 for s in banks), (wr, mi, ka)


def _transposed_read_distinct_bytes(row_bytes, swz):
    """Fewest distinct bytes over the 32-lane halves of one transposed read."""
    worst = 256
    for half in (0, 4):
        for h32 in range(2):
            seen = set()
            for lane in range(32 * h32, 32 * h32 + 32):
                g, i = lane >> 4, lane & 15
                krow = 8 * (g >> 1) + (i >> 2) + half
                n = 16 * (g & 1) + 4 * (i & 3)
                at = krow * row_bytes + ((n >> 3) ^ swz(krow)) * 16 + (n & 7) * 2
                seen.update((at + b) % 256 for b in range(8))
            worst = min(worst, len(seen))
    return worst


def test_planted_swizzle_mistakes_are_caught():
    """The 256-byte-row swizzle on the 64-wide tile's 128-byte rows leaves
    the row (chunks 8.. do not exist); no B swizzle there, or no A swizzle,
    gives 2-way bank conflicts.  The checks above would see each."""
    assert any(c ^ (4 * (k & 3)) >= 8 for k in range(4) for c in range(8))
    assert _transposed_read_distinct_bytes(128, lambda k: 0) < 256
    assert _transposed_read_distinct_bytes(128, lambda k: swz_b(64, k)) == 256
    seen = set()
    for lane in range(16):
        seen.update(((lane & 31) * 128 + b) % 256 for b in range(16))
    assert len(seen) < 256
