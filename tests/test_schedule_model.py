"""CPU model of how the complex64 forward kernel (16 x 16 fp32 matrix tiles)
splits a head's work among the eight waves of a workgroup.

The kernel's own decisions are replayed for a range of lengths: which row
blocks a workgroup pairs, when a wave of the short causal block switches to
its SIMD partner's long tile, which 16-key block of a stage each wave then
takes, and who writes each tile.  Every (16-query tile, 16-key block) pair
that the mask keeps must be computed exactly once, and every tile written
exactly once.  The GPU parity tests check the numbers; this checks the
schedule on lengths no GPU test reaches.
"""
from collections import Counter

import pytest

BM, TQ, BN = 64, 16, 32   # queries per row block, per wave tile; keys per stage


def replay(T: int, causal: bool):
    nrb = (T + BM - 1) // BM
    nwork = (nrb + 1) // 2
    done, writes = Counter(), Counter()
    for item in range(nwork):
        for wave in range(8):
            half, tq = wave >> 2, wave & 3
            if causal:
                rb = nrb - 1 - item if half == 0 else (item if item != nrb - 1 - item else -1)
            else:
                rb = 2 * item + half if 2 * item + half < nrb else -1
            qt0 = rb * BM + TQ * tq
            live = rb >= 0 and qt0 < T
            rbl = nrb - 1 - item
            qtl = rbl * BM + TQ * tq
            live_l = causal and qtl < T
            st_switch = 1 << 31
            if causal:
                st_switch = (item * BM + TQ * tq) // BN + 1 if item != rbl else 0
            kend = min(T, rbl * BM + BM) if causal else T
            nstages = (kend + BN - 1) // BN
            qt_cur, live_cur, helping = qt0, live, False
            for st in range(nstages):
                if half == 1 and st == st_switch:
                    if live:
                        writes[qt0] += 1
                    helping, qt_cur, live_cur = True, qtl, live_l
                split = st >= st_switch
                for sb in range(BN // 16):
                    if split and sb != half:
                        continue
                    kb0 = st * BN + 16 * sb
                    if not live_cur or kb0 >= T or (causal and kb0 > qt_cur):
                        continue
                    done[(qt_cur, kb0)] += 1
            if not helping and live_cur:
                writes[qt_cur] += 1
    return done, writes


LENGTHS = list(range(1, 200)) + [255, 256, 257, 1000, 1024, 2048, 4097]


@pytest.mark.parametrize("causal", [True, False])
def test_every_pair_once_every_tile_written_once(causal):
    for T in LENGTHS:
        done, writes = replay(T, causal)
        for qt in range(0, T, TQ):
            assert writes[qt] == 1, (T, qt, writes[qt])
            for kb in range(0, T, 16):
                need = kb <= qt if causal else True
                assert done[(qt, kb)] == int(need), (T, qt, kb, done[(qt, kb)])
        assert all(q < T and k < T for q, k in done), T


# ---------------------------------------------------------------------------
# The bf16 width-64 backward's key-side kernel: a workgroup owns 128 keys (32
# per wave) and streams 64-query stages.  Stages [s_lo, s_hi) run with no mask
# or skip branch; the replay checks that every such stage holds only queries
# inside T that every key of the tile may see, and that the general stages
# before and after it cover the rest of the stream.
BT_KEYS, BS_QUERIES = 128, 64


def key_tile_stages(T: int, causal: bool, kt: int):
    k0 = kt * BT_KEYS
    qs = k0 if causal else 0
    nstages = (T - qs + BS_QUERIES - 1) // BS_QUERIES if qs < T else 0
    s_lo = min((BT_KEYS - 1 + BS_QUERIES - 1) // BS_QUERIES if causal else 0, nstages)
    s_hi = max(s_lo, (T - qs) // BS_QUERIES if nstages > 0 else 0)
    return k0, qs, nstages, s_lo, s_hi


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_key_tile_branch_free_stages(causal):
    for T in list(range(1, 700)) + [4095, 4096, 4097, 16384]:
        for kt in range((T + BT_KEYS - 1) // BT_KEYS):
            k0, qs, nstages, s_lo, s_hi = key_tile_stages(T, causal, kt)
            assert 0 <= s_lo <= s_hi <= nstages, (T, kt)
            # every query the stream must visit: causal, those at or after the tile's first key
            assert qs + nstages * BS_QUERIES >= T and (nstages == 0 or qs + (nstages - 1) * BS_QUERIES < T)
            for s in range(s_lo, s_hi):
                q_first, q_last = qs + s * BS_QUERIES, qs + s * BS_QUERIES + BS_QUERIES - 1
                assert q_last < T, (T, kt, s)   # staged rows are real queries, not clamped copies
                if causal:
                    assert q_first >= k0 + BT_KEYS - 1, (T, kt, s)   # past every key of the tile
