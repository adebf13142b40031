"""CPU model of the one-copy tile swizzle of the bf16 backward kernels
(swz_b in kernel_born_bf16_d64_bwd.hip).

A 64-row stage of one bf16 plane is 64 rows of 128 bytes, eight 16-byte
chunks each; the LDS-direct copy puts logical chunk c of row r at slot
c ^ swz(r).  The tile is read two ways:
  * as a row-major operand: lane (l32, h) reads 16 bytes, logical chunk
    2 j + h of row l32 (+ 32 per block);
  * through the transposing read, two 8-byte reads per lane: lane
    16 G + 4 r + c4 (h = G >> 1) addresses row 4 h + r (+ 8 for the second
    read, + 16 m + 32 per block), logical chunk 4 cc + 2 (G & 1) + (c4 >> 1),
    its first or second 8 bytes by c4 & 1.
The kernel's per-lane offsets are restated here.  The model checks that
every read finds the logical bytes it asks for (so an offset that ignores a
bit of the row the swizzle depends on fails), and that under 64 banks
(16-byte reads 16 lanes at a time, 8-byte reads 32 at a time) and 32 banks
(8 and 16 lanes) no read touches a bank at two addresses in one step.  A
swizzle that is a function of the low two row bits only (the value tiles'
swizzle) fails the row-major reads, and the key tiles' swizzle fails the
transposing reads (the forward's two swizzles, which a tile read both ways
would need twice over).
"""
import pytest

ROWB = 128


def swz_b(row):
    i = (row >> 1) & 7
    return (((i & 1) << 2) | (i >> 1)) ^ ((row & 1) << 1)


def swz_k(row):
    return ((row >> 1) & 7) ^ ((row & 1) << 2)


def swz_v(row):
    return (row & 3) << 1


def placement(swz):
    """byte address -> (row, logical byte within the row) after the copy."""
    where = {}
    for row in range(64):
        for slot in range(8):
            lc = slot ^ swz(row)
            for b in range(16):
                where[row * ROWB + 16 * slot + b] = (row, 16 * lc + b)
    return where


def row_reads(swz, sb):
    """per k-step j: lane -> (address, [(row, logical byte)] expected)."""
    out = []
    for j in range(4):
        lanes = []
        for lane in range(64):
            l32, h = lane & 31, lane >> 5
            row = 32 * sb + l32
            off = l32 * ROWB + (((2 * j + h) ^ swz(l32)) << 4)   # the kernel's koff
            addr = 32 * sb * ROWB + off
            lanes.append((addr, 16, [(row, 16 * (2 * j + h) + b) for b in range(16)]))
        out.append(lanes)
    return out


def tr_reads(swz, sb, m, cc, second):
    lanes = []
    for lane in range(64):
        G, r, c4 = lane >> 4, (lane >> 2) & 3, lane & 3
        h = G >> 1
        lc = 4 * cc + 2 * (G & 1) + (c4 >> 1)
        rr = 4 * h + r + (8 if second else 0)
        off = rr * ROWB + ((lc ^ swz(rr)) << 4) + ((c4 & 1) << 3)   # the kernel's voff / voffh
        addr = (32 * sb + 16 * m) * ROWB + off
        row = 32 * sb + 16 * m + rr
        lanes.append((addr, 8, [(row, 16 * lc + 8 * (c4 & 1) + b) for b in range(8)]))
    return lanes


def all_reads(swz):
    reads = []
    for sb in range(2):
        reads += row_reads(swz, sb)
        for m in range(2):
            for cc in range(2):
                for second in (False, True):
                    reads.append(tr_reads(swz, sb, m, cc, second))
    return reads


def worst_degree(lanes, lanes_per_step, nbanks):
    worst = 0
    for g0 in range(0, 64, lanes_per_step):
        banks = {}
        for addr, size, _ in lanes[g0:g0 + lanes_per_step]:
            for w in range(size // 4):
                a = addr // 4 + w
                banks.setdefault(a % nbanks, set()).add(a)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


def test_reads_find_their_data():
    where = placement(swz_b)
    for lanes in all_reads(swz_b):
        for addr, size, want in lanes:
            assert [where[addr + b] for b in range(size)] == want


def test_second_transposing_read_needs_its_own_offset():
    # planted mistake: the second read taken 8 rows past the first with the
    # first's swizzle (what a swizzle of the low row bits allows) misreads
    where = placement(swz_b)
    bad = 0
    for lanes in [tr_reads(swz_b, 0, 0, 0, False)]:
        for addr, size, want in lanes:
            got = [where[addr + 8 * ROWB + b] for b in range(size)]
            want8 = [(row + 8, byte) for row, byte in want]
            bad += got != want8
    assert bad > 0


@pytest.mark.parametrize("nbanks,row_lanes,tr_lanes", [(64, 16, 32), (32, 8, 16)])
def test_swz_b_conflict_free(nbanks, row_lanes, tr_lanes):
    for sb in range(2):
        for lanes in row_reads(swz_b, sb):
            assert worst_degree(lanes, row_lanes, nbanks) == 1
        for m in range(2):
            for cc in range(2):
                for second in (False, True):
                    assert worst_degree(tr_reads(swz_b, sb, m, cc, second), tr_lanes, nbanks) == 1


def test_single_purpose_swizzles_conflict_one_way():
    assert max(worst_degree(l, 16, 64) for l in row_reads(swz_v, 0)) > 1
    assert max(worst_degree(tr_reads(swz_k, 0, 0, cc, s), 32, 64) for cc in range(2) for s in (False, True)) > 1
    assert max(worst_degree(l, 16, 64) for l in row_reads(swz_k, 0)) == 1
    assert max(worst_degree(tr_reads(swz_v, 0, 0, cc, s), 32, 64) for cc in range(2) for s in (False, True)) == 1
