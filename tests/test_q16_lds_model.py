"""CPU model of the LDS addressing of the 16-query bf16 Born forward kernel
(born_bf16_q16_impl.h: 16 x 16 x 32 products) at head widths 128 and 32.

Restated for one 64-key stage of two 32-key blocks: the LDS-direct staging
(width 32: wave-wide load i of wave w is load L = 8 i + w of the stage: region
L / LPR, rows RPL (L mod LPR) .., lane l on row RPL (L mod LPR) + l / NCR and
physical slot l mod NCR; width 128: load h of lane (j16, g) of wave w on row
8 w + 4 h + g, slot j16; each lane fetching logical chunk slot ^ swz(row)), the K' operand reads
(block sb, k-step ks, tile kt: row 32 sb + 16 kt + j16, logical chunk
4 (ks mod KH) + g), and the two transposing V reads per output tile and block
(lane 4 r + c4 of group g points at row 32 sb + 4 g + r, channels
16 m + 4 c4 .. + 3; the hardware hands lane i of the 16-lane group column i of
the 4 addressed rows; the second read is 16 rows further).  The model checks
that every read finds the logical data the products need, that the V^T
operand and the packed weights agree on the key behind every contraction
index, that the stores cover every output channel once, and that every access
touches each LDS bank at most once per service step under both bank models;
planted mistakes (no K swizzle, no V swizzle, width 128's swizzles at width
32, the second V read at the first's rows) fail.
"""
import pytest

BN, NW = 64, 8
MODELS_B128 = [(16, 64), (8, 32)]    # 16-byte reads: lanes per step, banks
MODELS_B64 = [(32, 64), (16, 32)]    # 8-byte reads


def swz_k(D, row):
    if D == 128:
        return row & 15
    return ((row >> 1) ^ (row >> 2)) & 3


def swz_v(D, row):
    if D == 128:
        return (row & 7) << 1
    return (((row >> 1) ^ (row >> 2)) & 1) << 1


def geom(D):
    rowb = 2 * D
    g = dict(D=D, ROWB=rowb, NCR=rowb // 16, REGION=BN * rowb, KH=D // 32, CH=D // 16,
             RPL=1024 // rowb, LPR=BN * rowb // 1024)
    g["LPW"] = 4 * g["LPR"] // NW
    g["NP"] = g["LPR"] // NW if g["LPR"] > NW else 1
    return g


def staging(D, swz):
    """physical byte offset within the stage -> (region, row, logical chunk)"""
    c = geom(D)
    where = {}
    if D == 128:
        # width 128 keeps its own mapping: load h of wave w covers row 8 w + 4 h + g
        for r in range(4):
            for w in range(NW):
                for h in range(2):
                    for lane in range(64):
                        j16, g = lane & 15, lane >> 4
                        row = 8 * w + 4 * h + g
                        phys = r * c["REGION"] + w * 2048 + h * 1024 + 16 * lane
                        assert phys == r * c["REGION"] + row * c["ROWB"] + 16 * j16
                        where[phys] = (r, row, j16 ^ swz(D, row))
        return where
    for w in range(NW):
        for i in range(c["LPW"]):
            L = NW * i + w
            r, li = L // c["LPR"], L % c["LPR"]
            # the kernel keeps one offset per residue of i mod NP: the rows must repeat so
            assert li == (NW * (i % c["NP"]) + w) % c["LPR"]
            for lane in range(64):
                row = c["RPL"] * li + lane // c["NCR"]
                slot = lane % c["NCR"]
                phys = r * c["REGION"] + li * 1024 + 16 * lane
                assert phys == r * c["REGION"] + row * c["ROWB"] + 16 * slot
                where[phys] = (r, row, slot ^ swz(D, row))
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


def k_read(D, lane, sb, kt, ks, swz=swz_k):
    c = geom(D)
    j16, g = lane & 15, lane >> 4
    row = 32 * sb + 16 * kt + j16
    return (ks // c["KH"]) * c["REGION"] + row * c["ROWB"] + 16 * ((4 * (ks % c["KH"]) + g) ^ swz(D, j16))


def v_read(D, lane, sb, tile, second, swz=swz_v, second_rows=16):
    c = geom(D)
    g, r, c4 = lane >> 4, (lane >> 2) & 3, lane & 3
    m = tile % c["CH"]
    row = 4 * g + r
    off = ((2 + tile // c["CH"]) * c["REGION"] + (32 * sb + row) * c["ROWB"]
           + 16 * ((2 * m + (c4 >> 1)) ^ swz(D, row)) + 8 * (c4 & 1))
    return off + (second_rows * c["ROWB"] if second else 0)


WIDTHS = [128, 32]


@pytest.mark.parametrize("D", WIDTHS)
def test_staging_is_a_bijection(D):
    c = geom(D)
    for swz in (swz_k, swz_v):
        where = staging(D, swz)
        assert sorted(where.values()) == [(r, row, ch) for r in range(4) for row in range(BN) for ch in range(c["NCR"])]


@pytest.mark.parametrize("D", WIDTHS)
def test_k_reads_find_their_rows_and_chunks_without_conflicts(D):
    c = geom(D)
    where = staging(D, swz_k)
    for sb in range(2):
        for kt in range(2):
            for ks in range(2 * c["KH"]):
                addrs = []
                for lane in range(64):
                    j16, g = lane & 15, lane >> 4
                    a = k_read(D, lane, sb, kt, ks)
                    assert where[a] == (ks // c["KH"], 32 * sb + 16 * kt + j16, 4 * (ks % c["KH"]) + g)
                    addrs.append(a)
                for lanes, nb in MODELS_B128:
                    assert worst_degree(addrs, lanes, nb, 4) == 1


def v_operand(D, lane, sb, tile):
    """(plane, key, channel) of each of the 8 A-operand elements of lane `lane`"""
    where = staging(D, swz_v)
    out = []
    g, i = lane >> 4, lane & 15
    for second in (False, True):
        for rr in range(4):
            src = 16 * g + 4 * rr + i // 4      # the lane that addressed row rr, column quad i // 4
            a = v_read(D, src, sb, tile, second)
            r, row, chunk = where[a - a % 16]
            half = (a % 16) // 8
            out.append((r - 2, row, 8 * chunk + 4 * half + i % 4))
    return out


@pytest.mark.parametrize("D", WIDTHS)
def test_v_reads_and_weights_agree_on_every_key(D):
    c = geom(D)
    for sb in range(2):
        for tile in range(2 * c["CH"]):
            for lane in range(64):
                j, g = lane & 15, lane >> 4
                ops = v_operand(D, lane, sb, tile)
                for jj in range(8):
                    plane, key_v, chan = ops[jj]
                    # the packed weights: element jj of lane (query j, group g) is score
                    # register jj % 4 of tile jj // 4 of the block, i.e. key 16 (jj // 4) + 4 g + jj % 4
                    assert key_v == 32 * sb + 16 * (jj // 4) + 4 * g + jj % 4
                    # A row i = lane % 16 is channel i of the tile, in the tile's plane
                    assert (plane, chan) == (tile // c["CH"], 16 * (tile % c["CH"]) + j)


@pytest.mark.parametrize("D", WIDTHS)
def test_v_reads_have_no_bank_conflicts(D):
    c = geom(D)
    for sb in range(2):
        for tile in range(2 * c["CH"]):
            for second in (False, True):
                addrs = [v_read(D, lane, sb, tile, second) for lane in range(64)]
                for lanes, nb in MODELS_B64:
                    assert worst_degree(addrs, lanes, nb, 2) == 1


@pytest.mark.parametrize("D", WIDTHS)
def test_stores_cover_each_channel_once(D):
    c = geom(D)
    seen = []
    for tile in range(2 * c["CH"]):
        for g in range(4):
            for r in range(4):
                seen.append((tile // c["CH"], 16 * (tile % c["CH"]) + 4 * g + r))
    assert sorted(seen) == [(pl, ch) for pl in range(2) for ch in range(D)]


@pytest.mark.parametrize("D,waves_per_simd", [(128, 2), (32, 4)])
def test_lds_budget(D, waves_per_simd):
    c = geom(D)
    per_wg = 2 * 4 * c["REGION"] + 8 * D
    assert per_wg * (waves_per_simd * 4 // NW) <= 160 * 1024


def test_planted_mistakes_fail():
    # no K swizzle: the 16 rows of one read share banks
    addrs = [k_read(128, lane, 0, 0, 0, swz=lambda D, r: 0) for lane in range(64)]
    assert worst_degree(addrs, 16, 64, 4) > 1
    # no V swizzle: two groups' rows share banks
    addrs = [v_read(128, lane, 0, 0, False, swz=lambda D, r: 0) for lane in range(64)]
    assert worst_degree(addrs, 32, 64, 2) > 1
    # width 128's K swizzle at width 32: four rows to a bank window collide
    addrs = [k_read(32, lane, 0, 0, 0, swz=lambda D, r: swz_k(128, r) & 3) for lane in range(64)]
    assert worst_degree(addrs, 16, 64, 4) > 1
    # the second V read at the first's rows: keys 16 + 4 g .. never reach the operand
    where = staging(128, swz_v)
    a = v_read(128, 5, 1, 0, True, second_rows=0)
    assert where[a - a % 16][1] < 32 + 16
