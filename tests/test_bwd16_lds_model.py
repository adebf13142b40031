"""CPU model of the LDS addressing of the 16 x 16 fp32 backward kernels
(kernel_bwd_f32_mfma16.hip) at head widths 32, 64 and 128.

The kernels' addresses are restated for one workgroup: the staging writes
(thread t stages row t / LPK, 16-byte chunks t % LPK + LPK i rotated by 7 on
odd rows), the score operand reads (lane (j16, g) reads row j16 at the lane
group's quarter of the wave's channel group) and the gradient operand reads
(lane (j16, g) reads the NC floats NC j16 .. of row 4 g + t of its channel
group, in 16-byte pieces whose order is rotated by
rho(i) = (i / (8 / NCK) + i / 8) mod NCK, NCK = NC / 4).  The model checks
that each access finds the floats it stands for, that the gradient tiles'
channels, the stored channels and the owned operand's floats agree (and pair
c with c ^ 1 as real and imaginary parts), that every access touches each
bank at most once per service step (16 lanes over 64 banks, or 8 over 32),
and the LDS budget.  Planted mistakes (no rotation of the gradient reads, a
rotation by i / (16 / NCK) alone, no rotation of the staging rows) show bank
conflicts.
"""
import pytest

NW, NT, TR = 4, 256, 16


def cfg(D, CH):
    KD = 2 * D
    KDC = KD // CH
    c = dict(D=D, CH=CH, KD=KD, KDC=KDC, KQ=KDC // 4, NC=KDC // 16, ROW=KD + 4, NCH=KD // 4,
             BN=16 if CH > 1 else 32)
    c["NCK"] = c["NC"] // 4
    c["RDIV"] = 8 // c["NCK"]
    c["LPK"] = NT // c["BN"]
    c["CPT"] = c["NCH"] // c["LPK"]
    c["STAGE"] = 2 * c["BN"] * c["ROW"] + 2 * c["BN"]
    c["XCH"] = NW * 12 * 64 if CH > 1 else 0
    return c


# (width, channel groups): 32 and 64 whole rows; 128 split for Born, whole for PCT
CONFIGS = [(32, 1), (64, 1), (128, 2), (128, 1)]
MODELS = [(16, 64), (8, 32)]


def worst_degree(addrs, lanes_per_step, nbanks, width=4):
    worst = 0
    for g0 in range(0, len(addrs), lanes_per_step):
        banks = {}
        for a0 in addrs[g0:g0 + lanes_per_step]:
            for w in range(width):
                banks.setdefault((a0 + w) % nbanks, set()).add(a0 + w)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


def stage_chunk(c, t, i, rotate=True):
    row, sc = t // c["LPK"], t % c["LPK"]
    rot = 7 * (row & 1) if rotate else 0
    return row, (sc + c["LPK"] * i + rot) % c["NCH"]


def rho(c, i, rotate="both"):
    if rotate == "both":
        return (i // c["RDIV"] + i // 8) % c["NCK"]
    if rotate == "64 banks":
        return (i // (16 // c["NCK"])) % c["NCK"]
    return 0


def run_read(c, j16, p, hc, rotate="both"):
    """float offset within a row of read p of lane j16's run (channel group hc)"""
    return c["KDC"] * hc + c["NC"] * j16 + 4 * ((p + rho(c, j16, rotate)) % c["NCK"])


def tile_channel(c, tile, i, hc):
    """real channel that gradient tile `tile`, row i stands for"""
    return c["KDC"] * hc + c["NC"] * i + 4 * ((tile // 4 + rho(c, i)) % c["NCK"]) + tile % 4


def store_channel(c, g, r, tile, hc):
    """channel a lane (group g) stores for tile `tile`, register r"""
    q, e = tile // 4, tile % 4
    rot = rho(c, 4 * g + r)
    return c["KDC"] * hc + g * c["KQ"] + c["NC"] * r + 4 * ((q + rot) % c["NCK"]) + e


def own_index(c, g, r, tile):
    """index into the owned operand's quarter (own_of)"""
    m = ((tile >> 2) + rho(c, 4 * g + r)) % c["NCK"]
    return c["NC"] * r + 4 * m + (tile & 3)


@pytest.mark.parametrize("D,CH", CONFIGS)
def test_staging_covers_every_chunk_once_without_conflicts(D, CH):
    c = cfg(D, CH)
    assert c["CPT"] * c["LPK"] == c["NCH"]
    seen = {}
    for t in range(NT):
        for i in range(c["CPT"]):
            row, ch = stage_chunk(c, t, i)
            assert row < c["BN"]
            seen.setdefault(row, []).append(ch)
    for row in range(c["BN"]):
        assert sorted(seen[row]) == list(range(c["NCH"]))
    for w in range(NW):
        for i in range(c["CPT"]):
            addrs = []
            for t in range(64 * w, 64 * w + 64):
                row, ch = stage_chunk(c, t, i)
                addrs.append(row * c["ROW"] + 4 * ch)
            for lanes, nbanks in MODELS:
                assert worst_degree(addrs, lanes, nbanks) == 1


@pytest.mark.parametrize("D,CH", CONFIGS)
def test_score_reads_cover_the_group_without_conflicts(D, CH):
    c = cfg(D, CH)
    for hc in range(CH):
        got = set()
        for g in range(4):
            for s in range(c["KQ"]):
                got.add(c["KDC"] * hc + g * c["KQ"] + s)
        assert got == set(range(c["KDC"] * hc, c["KDC"] * (hc + 1)))
        for p0 in range(0, c["KQ"], 4):
            addrs = [(l & 15) * c["ROW"] + c["KDC"] * hc + (l >> 4) * c["KQ"] + p0 for l in range(64)]
            for lanes, nbanks in MODELS:
                assert worst_degree(addrs, lanes, nbanks) == 1


@pytest.mark.parametrize("D,CH", CONFIGS)
def test_gradient_runs_find_their_channels_without_conflicts(D, CH):
    c = cfg(D, CH)
    for hc in range(CH):
        for j16 in range(16):
            out = {}
            for p in range(c["NCK"]):
                for e in range(4):
                    out[4 * p + e] = run_read(c, j16, p, hc) + e
            for tile in range(c["NC"]):
                assert out[tile] == tile_channel(c, tile, j16, hc)
                # the Born imaginary part takes the partner channel
                assert tile_channel(c, tile ^ 1, j16, hc) == tile_channel(c, tile, j16, hc) ^ 1
        for t in range(4):
            for p in range(c["NCK"]):
                addrs = [(4 * (l >> 4) + t) * c["ROW"] + run_read(c, l & 15, p, hc) for l in range(64)]
                for lanes, nbanks in MODELS:
                    assert worst_degree(addrs, lanes, nbanks) == 1


@pytest.mark.parametrize("D,CH", CONFIGS)
def test_stores_and_owned_floats_match_the_tiles(D, CH):
    c = cfg(D, CH)
    for hc in range(CH):
        stored = []
        for g in range(4):
            for r in range(4):
                for tile in range(c["NC"]):
                    ch = store_channel(c, g, r, tile, hc)
                    assert ch == tile_channel(c, tile, 4 * g + r, hc)
                    assert ch == c["KDC"] * hc + g * c["KQ"] + own_index(c, g, r, tile)
                    stored.append(ch)
        assert sorted(stored) == list(range(c["KDC"] * hc, c["KDC"] * (hc + 1)))


@pytest.mark.parametrize("D,CH", CONFIGS)
def test_lds_budget(D, CH):
    c = cfg(D, CH)
    total = (2 * c["STAGE"] + c["XCH"]) * 4
    wpe = 1 if (D >= 128 and CH == 1) else 2
    per_cu = total * (1 if wpe == 1 else 2)   # workgroups of 4 waves per compute unit
    assert per_cu <= 160 * 1024


def test_planted_mistakes_conflict():
    c = cfg(64, 1)
    # gradient runs read in the same order on every lane: two lanes per bank
    addrs = [(4 * (l >> 4)) * c["ROW"] + run_read(c, l & 15, 0, 0, rotate=None) for l in range(64)]
    assert worst_degree(addrs, 16, 64) > 1
    assert worst_degree([(4 * (l >> 4)) * c["ROW"] + run_read(c, l & 15, 0, 0) for l in range(64)], 16, 64) == 1
    # a rotation that only separates the lanes of a 64-bank step
    for D, CH in [(64, 1), (128, 1), (128, 2)]:
        cc = cfg(D, CH)
        addrs = [(4 * (l >> 4)) * cc["ROW"] + run_read(cc, l & 15, 0, 0, rotate="64 banks") for l in range(64)]
        assert worst_degree(addrs, 16, 64) == 1
        assert worst_degree(addrs, 8, 32) == 2
    # staging rows without the odd-row rotation: two rows share banks
    addrs = []
    for t in range(64):
        row, ch = stage_chunk(c, t, 0, rotate=False)
        addrs.append(row * c["ROW"] + 4 * ch)
    assert worst_degree(addrs, 16, 64) > 1
