"""CPU model of the LDS bank mapping of the complex64 forward kernel (16 x 16
fp32 matrix tiles).

The kernel's addresses are restated for one wave: the K' operand reads, the
value-operand reads (two 16-byte halves per lane at head width 64, swapped on
rows i with ((i >> 2) ^ (i >> 3)) odd) and the staging writes (16-byte chunk
c + 8 i of a key row, rotated by 7 chunks on odd rows).  LDS has banks of 4
bytes; a 16-byte access is taken to be served either 16 lanes at a time over
64 banks or 8 lanes at a time over 32 banks.  Under both, every access must
touch each bank at most once per service step.
"""
import pytest


def worst_degree(addrs, lanes_per_step, nbanks, width=4):
    worst = 0
    for g0 in range(0, 64, lanes_per_step):
        banks = {}
        for lane in range(g0, g0 + lanes_per_step):
            for w in range(width):
                a = addrs[lane] + w
                banks.setdefault(a % nbanks, set()).add(a)
        worst = max(worst, max(len(s) for s in banks.values()))
    return worst


MODELS = [(16, 64), (8, 32)]


def k_reads(D):
    KD, ROW = 2 * D, 2 * D + 4
    KQ = KD // 4
    return [[(l & 15) * ROW + (l >> 4) * KQ + 4 * i for l in range(64)] for i in range(KQ // 4)]


def v_reads(D, swap=True):
    KD, ROW = 2 * D, 2 * D + 4
    CPL = KD // 16
    out = []
    for t in range(4):
        for half in range(CPL // 4):
            addrs = []
            for l in range(64):
                j, g = l & 15, l >> 4
                s = 4 * (((j >> 2) ^ (j >> 3)) & 1) if (swap and CPL == 8) else 0
                addrs.append((4 * g + t) * ROW + CPL * j + ((4 * half) ^ s))
            out.append(addrs)
    return out


def stage_writes(D, rot):
    KD, ROW = 2 * D, 2 * D + 4
    nch = KD // 4
    cpt = nch // 8
    return [[(l // 8) * ROW + 4 * ((l % 8 + 8 * i + rot * ((l // 8) & 1)) % nch) for l in range(64)]
            for i in range(cpt)]


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("lanes,nbanks", MODELS)
def test_kernel_lds_accesses_are_conflict_free(D, lanes, nbanks):
    for acc in k_reads(D) + v_reads(D) + stage_writes(D, 7):
        assert worst_degree(acc, lanes, nbanks) == 1


def test_unswapped_value_reads_conflict():
    # the plain layout is two-way at width 64, which is what the swap removes
    assert max(worst_degree(a, 16, 64) for a in v_reads(64, swap=False)) == 2


def test_swapped_output_rows_match_swapped_reads():
    # a value row i is read swapped iff ((i >> 2) ^ (i >> 3)) is odd; output
    # row i = 4 g + r of lane group g is stored swapped iff (g ^ (g >> 1)) is odd
    for g in range(4):
        for r in range(4):
            i = 4 * g + r
            assert (((i >> 2) ^ (i >> 3)) & 1) == ((g ^ (g >> 1)) & 1)
