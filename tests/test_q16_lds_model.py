"""CPU model of the LDS addressing of the width-128 bf16 Born forward kernel
(kernel_born_bf16_q16.hip: 16 x 16 x 32 products, tiles of 16 queries).

Restated for one 64-key stage of two 32-key blocks: the LDS-direct staging
(load h of lane (j16, g) of wave w covers row 8 w + 4 h + g of each region,
physical slot j16, and fetches logical chunk j16 ^ swz(row)), the K' operand
reads, and the two transposing V reads per output tile and block (lane
4 r + c4 of group g points at row 32 sb + 4 g + r, channels
16 m + 4 c4 .. + 3; the hardware hands lane i of the 16-lane group column i of
the 4 addressed rows).  The model checks that every read finds the logical
data the products need, that the V^T operand and the packed weights agree on
the key behind every contraction index, that the stores cover every output
channel once, and that every access touches each LDS bank at most once per
service step under both bank models; planted mistakes (no K swizzle, no V
swizzle, the second V read at the first's rows) fail.
"""
import pytest

ROWB = 256          # bytes per row of one plane region (128 bf16 channels)
NCR = ROWB // 16    # 16-byte chunks per row
BN = 64             # keys per stage
BLKB = 32 * ROWB    # bytes of a 32-key block
NW = 8


def swz_k(row):
    return row & 15


def swz_v(row):
    return (row & 7) << 1


def staging(swz):
    """physical LDS byte offset (within a region) -> (row, logical chunk)"""
    where = {}
    for w in range(NW):
        for h in range(2):
            for lane in range(64):
                j16, g = lane & 15, lane >> 4
                row = 8 * w + 4 * h + g
                phys = w * 2048 + h * 1024 + 16 * lane
                assert phys == row * ROWB + 16 * j16
                where[phys] = (row, j16 ^ swz(row))
    return where


def worst_degree(addrs, lanes_per_step, nbanks, width):
    worst = 0
    for g0 in range(0, len(addrs), lanes_per_step):
        banks = {}
        for a0 in addrs[g0:g0 + lanes_per_step]:
            for wd in range(width):
                a = a0 // 4 + wd
                banks.setdefault(a % nbanks, set()).add(a)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


MODELS_B128 = [(16, 64), (8, 32)]    # 16-byte reads: lanes per step, banks
MODELS_B64 = [(32, 64), (16, 32)]    # 8-byte reads


def k_read(lane, sb, kt, ks, swz=swz_k):
    j16, g = lane & 15, lane >> 4
    return sb * BLKB + kt * 16 * ROWB + j16 * ROWB + 16 * ((4 * (ks & 3) + g) ^ swz(j16))


def v_read(lane, sb, m, second, swz=swz_v, second_rows=16):
    g, r, c4 = lane >> 4, (lane >> 2) & 3, lane & 3
    row = 4 * g + r
    off = sb * BLKB + row * ROWB + 16 * ((2 * m + (c4 >> 1)) ^ swz(row)) + 8 * (c4 & 1)
    return off + (second_rows * ROWB if second else 0)


def test_staging_is_a_bijection():
    for swz in (swz_k, swz_v):
        where = staging(swz)
        assert sorted(where.values()) == [(r, c) for r in range(BN) for c in range(NCR)]


def test_k_reads_find_their_rows_and_chunks_without_conflicts():
    where = staging(swz_k)
    for sb in range(2):
        for kt in range(2):
            for ks in range(8):
                addrs = []
                for lane in range(64):
                    j16, g = lane & 15, lane >> 4
                    a = k_read(lane, sb, kt, ks)
                    # region (Re K for ks < 4, Im K after) chosen by ks; inside it:
                    assert where[a] == (32 * sb + 16 * kt + j16, 4 * (ks & 3) + g)
                    addrs.append(a)
                for lanes, nb in MODELS_B128:
                    assert worst_degree(addrs, lanes, nb, 4) == 1


def v_operand(lane, sb, m):
    """(key, channel) of each of the 8 A-operand elements of lane `lane` for tile m of block sb"""
    where = staging(swz_v)
    out = []
    for second in (False, True):
        # group of the lane; the 16 lanes of the group address the 4 x 16 block
        g = lane >> 4
        i = lane & 15
        rows = []
        for rr in range(4):
            src = 16 * g + 4 * rr + i // 4      # the lane holding row rr, column quad i // 4
            a = v_read(src, sb, m, second)
            row, chunk = where[a - a % 16]
            half = (a % 16) // 8
            chan = 8 * chunk + 4 * half + i % 4
            rows.append((row, chan))
        out.extend(rows)
    return out


def test_v_reads_and_weights_agree_on_every_key():
    for sb in range(2):
        for m in range(8):
            for lane in range(64):
                j, g = lane & 15, lane >> 4
                ops = v_operand(lane, sb, m)
                for jj in range(8):
                    key_v, chan = ops[jj]
                    # the packed weights: element jj of lane (query j, group g) is score
                    # register jj % 4 of tile jj // 4 of the block, i.e. key 16 (jj // 4) + 4 g + jj % 4
                    key_w = 32 * sb + 16 * (jj // 4) + 4 * g + jj % 4
                    assert key_v == key_w
                    assert chan == 16 * m + j       # A row i = lane % 16 is the tile's channel i


def test_v_reads_have_no_bank_conflicts():
    for sb, m in [(sb, m) for sb in range(2) for m in range(8)]:
        for second in (False, True):
            addrs = [v_read(lane, sb, m, second) for lane in range(64)]
            for lanes, nb in MODELS_B64:
                assert worst_degree(addrs, lanes, nb, 2) == 1


def test_stores_cover_each_channel_once():
    seen = []
    for c in range(16):
        for g in range(4):
            for r in range(4):
                seen.append((c // 8, 16 * (c & 7) + 4 * g + r))
    assert sorted(seen) == [(pl, ch) for pl in range(2) for ch in range(128)]


def test_lds_budget_two_waves_per_simd():
    stage = 4 * BN * ROWB
    assert 2 * stage + 128 * 8 <= 160 * 1024


def test_planted_mistakes_fail():
    # no K swizzle: the 16 rows of one read share banks
    addrs = [k_read(lane, 0, 0, 0, swz=lambda r: 0) for lane in range(64)]
    assert worst_degree(addrs, 16, 64, 4) > 1
    # no V swizzle: two groups' rows share banks
    addrs = [v_read(lane, 0, 0, False, swz=lambda r: 0) for lane in range(64)]
    assert worst_degree(addrs, 32, 64, 2) > 1
    # the second V read at the first's rows: keys 16 + 4 g .. never reach the operand
    where = staging(swz_v)
    lane = 5
    a = v_read(lane, 1, 0, True, second_rows=0)
    assert where[a - a % 16][0] < 32 + 16
