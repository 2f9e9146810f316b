"""The split schedule that include/kvq.h documents (tests/_schedule.py), on
the CPU: every block taken once, in order, with distinct partial slots;
splits that line up with the units stay lined up; a workgroup that crosses
into a further unit takes about the switch cost fewer blocks; short
problems use ranges of at least one block per wave.  The GPU side
(test_partials_follow_the_documented_schedule) checks that the kernel
follows this description."""

import os
import re

import numpy as np
import pytest

import _schedule as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NWG = 512  # one round of two workgroups on each of 256 CUs


def check_cover(block_counts, nwg, c=S.SEG_COST):
    r = S.ranges(block_counts, nwg, c)
    seen = [np.zeros(nb, dtype=np.int32) for nb in block_counts]
    prev = (-1, -1)
    slots = set()
    for w, segs in enumerate(r):
        for u, i, n in segs:
            assert n > 0
            assert (u, i) > prev, "ranges run in (unit, block) order"
            prev = (u, i + n - 1)
            seen[u][i:i + n] += 1
            assert u + w not in slots, "slot u + w is unique"
            slots.add(u + w)
        for (u0, i0, n0), (u1, i1, n1) in zip(segs, segs[1:]):
            # contiguous: the next segment starts the next unit that has blocks
            assert i1 == 0 and i0 + n0 == block_counts[u0], "a range is contiguous"
            assert u1 > u0 and all(block_counts[u] == 0 for u in range(u0 + 1, u1)), "a range is contiguous"
    assert all(np.all(s == 1) for s in seen), "every block is taken exactly once"
    return r


@pytest.mark.parametrize("block_counts,nwg", [
    ([1], 1), ([5, 0, 7], 3), ([0, 0], 4), ([64, 64], NWG), ([300] * 12, 7), ([16384] * 4, NWG),
    ([4096] * 32, NWG), ([256] * 8192, NWG), (list(range(0, 400, 7)), 333),
])
def test_cover_order_and_slots(block_counts, nwg):
    check_cover(block_counts, nwg)


def test_random_mixes():
    rng = np.random.default_rng(3)
    for _ in range(200):
        units = int(rng.integers(1, 60))
        counts = [int(x) for x in rng.choice([0, 1, 3, 16, int(rng.integers(0, 3000))], size=units)]
        check_cover(counts, int(rng.choice([1, 2, 5, 64, 333, NWG])), int(rng.choice([0, 1, 24])))


@pytest.mark.parametrize("units,blocks,per_wg_units", [
    (4, 16384, None),   # 1 x 262144 tokens, 4 kv heads
    (32, 4096, None),   # 8 x 65536 tokens
    (8192, 256, 16),    # MTP: 256 x 4096 tokens, 32 kv heads
])
def test_aligned_splits_stay_aligned(units, blocks, per_wg_units):
    r = check_cover([blocks] * units, NWG)
    if per_wg_units is None:  # every workgroup inside one unit
        assert all(len(segs) == 1 for segs in r)
    else:  # whole units, the same number each
        assert all(len(segs) == per_wg_units and all(n == blocks for _, _, n in segs) for segs in r)


def test_switch_cost_on_a_batched_mix():
    rng = np.random.default_rng(11)
    lens = rng.integers(8192, 32769, size=32)
    counts = [int((L + 15) // 16) for L in lens for _ in range(4)]  # 4 kv heads per sequence
    r = check_cover(counts, NWG)
    one = [sum(n for _, _, n in s) for s in r if len(s) == 1]
    two = [sum(n for _, _, n in s) for s in r if len(s) == 2]
    assert len(two) > 50 and len(one) > 300
    assert abs((np.mean(one) - np.mean(two)) - S.SEG_COST) < 2.0
    # without the cost, both kinds take the same share
    r0 = check_cover(counts, NWG, c=0)
    one0 = [sum(n for _, _, n in s) for s in r0 if len(s) == 1]
    two0 = [sum(n for _, _, n in s) for s in r0 if len(s) == 2]
    assert abs(np.mean(one0) - np.mean(two0)) < 1.0


def test_short_problems_take_one_block_per_wave():
    counts = [64, 64]  # 1 x 1024 tokens, 2 kv heads
    r = check_cover(counts, NWG)
    busy = [sum(n for _, _, n in s) for s in r if s]
    assert len(busy) <= 256
    assert min(busy) >= 1 and max(busy) <= 4 + 1  # about one 16-token block per wave
    C = S.cost_line([16] * 200)
    assert S.ways(C, NWG) <= 256  # at most about one workgroup per CU below 256 x 128 positions


def test_the_library_and_the_header_state_the_same_cost():
    api = open(os.path.join(ROOT, "decode_attention_quant_amd", "csrc", "kvq_api.hip")).read()
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    m = re.search(r"constexpr int32_t SEG_COST = (\d+);", api)
    assert m and int(m.group(1)) == S.SEG_COST
    assert "with %d positions between one unit" % S.SEG_COST in hdr
    assert "C = T + %d (units - 1)" % S.SEG_COST in hdr
