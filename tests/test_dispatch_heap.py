"""The decode dispatch plan equals the one a per-workgroup greedy simulation
gives (a heap of compute-unit finish times, one workgroup at a time), for
shapes from one record per workgroup to three. The library simulates the
same dispatch with (time, count) groups of units."""
import heapq
import os

import pytest

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "kv_cache_compression_encode_amd", "libcg.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcg.so not built")

# measured workgroup times per chains per wavefront (3 chains = 1000), as the
# library plans with them; 16 wavefronts, at most 3 records, chains run three
# at a time (more than three: further rounds)
WG_COST = [0, 380, 710, 1000]
CUS = 256


def wg_cost(c):
    return (c // 3) * WG_COST[3] + WG_COST[c % 3]


def heap_plan(n_rec, sets, lg_max, last):
    chains = lambda r: -(-r * lg_max // 16)  # noqa: E731
    max_r = 1
    while max_r < 3 and chains(max_r + 1) <= 3:
        max_r += 1

    def cost(r, lst):
        rest = wg_cost(chains(r - 1)) if r > 1 else 0
        return wg_cost(chains(r)) * lst // 1024 + rest * (1024 - lst) // 1024 + 5

    best = None
    for r1 in range(1, min(max_r, n_rec) + 1):
        for r2 in range(1, r1 + 1):
            for split in range(0, n_rec + 1, r1):
                if split == n_rec and r2 != 1:
                    continue
                n1, n2, rem = split // r1, -(-(n_rec - split) // r2), (n_rec - split) % r2
                h = [0] * CUS

                def run(jobs, t):
                    for _ in range(jobs):
                        heapq.heapreplace(h, h[0] + t)

                if n2 == 0:
                    run((n1 - 1) * sets, cost(r1, 1024))
                    run(sets, cost(r1, last))
                else:
                    run(n1 * sets, cost(r1, 1024))
                    run((n2 - 1) * sets, cost(r2, 1024))
                    run(sets, cost(rem if rem else r2, last))
                span = max(h)
                if best is None or span < best[0]:
                    best = (span, r1, split, r2)
    return best[1:]


CASES = [
    # L, H, D, T, C (one layer group)
    (16, 1, 64, 1024, 256), (16, 64, 64, 35, 3), (16, 64, 64, 26, 2), (16, 32, 64, 181, 16),
    (16, 8, 128, 32768, 1536), (11, 32, 128, 8192, 1536), (16, 48, 128, 5000, 300),
    (8, 64, 64, 700, 50), (33, 16, 64, 900, 64), (5, 128, 128, 3000, 200), (16, 96, 64, 97, 7),
    (64, 8, 128, 4096, 512), (100, 2, 64, 333, 33),
]


@pytest.mark.parametrize("L,H,D,T,Cc", CASES)
def test_plan_matches_per_workgroup_simulation(L, H, D, T, Cc):
    from kv_cache_compression_encode_amd import cg as C
    lv = C.Level(2, [0] * L, [0.7])
    n = -(-T // Cc)
    last = (T - (n - 1) * Cc) * 1024 // Cc
    assert C.cg_decode_plan(C.shape(L, H, D, T, Cc), [lv], n, CUS) == heap_plan(n, 2 * H * (D // 64), L, last)
