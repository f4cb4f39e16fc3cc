"""LDS bank model of the fine kernel's two operand reads (CPU).

The fine kernel (video_dit_block_amd/csrc/fwd.hip) stores every 16-byte chunk
c of LDS row r at slot c ^ swz(r) and reads
  K:   ds_read_b128, lane l reading chunk (2 st + l / 32) of row l % 32 (the A
       operand of the 32x32x16 MFMA, one read per k-step st);
  V^T: ds_read_b64_tr_b16, lane l in 16-lane group G = l / 16, s = l % 16,
       reading 8 bytes of row 16 kk + h + 4 (G / 2) + s / 4 (h in {0, 8}) at
       column 32 db + 16 (G % 2) + 4 (s % 4).
The swizzles below restate swz_k / swz_v of that file. Model: 4-byte banks
(32 or 64 of them); a read is served in groups of as many lanes as the banks
can feed at once (banks * 4 / bytes per lane), and a group is conflict-free
when no two distinct dwords it touches share a bank. The profiler's bank
conflict counter reads 0 for this kernel; this test shows the swizzles are
conflict-free by construction under either bank count, and that the model
does see conflicts (the unswizzled layout has them).
"""
import pytest


def swz_k(D, r):
    if D == 128:
        return r & 15
    return (1 if r & 1 else 0) ^ (4 if r & 2 else 0) ^ (2 if r & 4 else 0) ^ (1 if r & 8 else 0)


def swz_v(D, r):
    if D == 128:
        return (10 if r & 1 else 0) ^ (4 if r & 2 else 0)
    return (2 if r & 1 else 0) ^ (4 if r & 2 else 0)


def worst_degree(addrs, width, banks):
    """Largest number of distinct dwords on one bank within a lane group."""
    group = banks * 4 // width
    worst = 0
    for g0 in range(0, len(addrs), group):
        per_bank = {}
        for a in addrs[g0:g0 + group]:
            for w in range(width // 4):
                dw = a // 4 + w
                per_bank.setdefault(dw % banks, set()).add(dw)
        worst = max(worst, max(len(v) for v in per_bank.values()))
    return worst


def addr(D, row, chunk, swz, off=0):
    return row * 2 * D + 16 * (chunk ^ swz(D, row)) + off


def k_reads(D, swz):
    for st in range(D // 16):
        yield [addr(D, l % 32, 2 * st + l // 32, swz) for l in range(64)]


def vt_reads(D, swz):
    for db in range(D // 32):
        for kk in range(2):
            for h in (0, 8):
                a = []
                for l in range(64):
                    G, s = l // 16, l % 16
                    row = 16 * kk + h + 4 * (G // 2) + s // 4
                    d0 = 32 * db + 16 * (G % 2) + 4 * (s % 4)
                    a.append(addr(D, row, d0 // 8, swz, (d0 % 8) * 2))
                yield a


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("banks", [32, 64])
def test_operand_reads_are_conflict_free(D, banks):
    for a in k_reads(D, swz_k):
        assert worst_degree(a, 16, banks) == 1
    for a in vt_reads(D, swz_v):
        assert worst_degree(a, 8, banks) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_model_sees_conflicts_without_the_swizzle(D):
    none = lambda D, r: 0
    assert max(worst_degree(a, 16, 64) for a in k_reads(D, none)) > 1
    assert max(worst_degree(a, 8, 64) for a in vt_reads(D, none)) > 1


def test_swizzles_permute_the_chunks_of_a_row():
    for D in (64, 128):
        for r in range(32):
            for swz in (swz_k, swz_v):
                assert sorted(c ^ swz(D, r) for c in range(D // 8)) == list(range(D // 8))
