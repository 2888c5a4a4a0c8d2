"""The live repin decision of the HBM / host expert tier (moe_tier_plan),
host logic only: hand-worked cases, then seeded random cases held to the
policy's invariants and to a plain statement of the policy.

The policy (wpnews.pro feature list, "Live tier adaptation (--repin N)"):
a decaying heat map replaces cold pinned experts by hot streamed ones, with
25% hysteresis and at most four swaps per repin.  Free slots are filled
first with the hottest streamed experts that were used at all."""
import random

import pytest

from quantized_moe_noaux_amd import moe
from quantized_moe_noaux_amd.moe import MoeError


def test_fill_free_slots_hottest_first():
    # nothing pinned yet: the two hottest used experts, lowest slot first
    assert moe.moe_tier_plan([5, 0, 9, 1, 7, 3], 2, [-1] * 6) == (2, [-1, -1, 0, -1, 1, -1])
    # experts never used are not pinned even when slots are free
    assert moe.moe_tier_plan([0, 2, 0, 0], 3, [-1] * 4) == (1, [-1, 0, -1, -1])


def test_swaps_need_more_than_25_percent():
    # pinned e0 (5) and e5 (3); streamed e2 (9) beats e5, then e4 (7) beats e0 (7*4 > 5*5)
    assert moe.moe_tier_plan([5, 0, 9, 1, 7, 3], 2, [0, -1, -1, -1, -1, 1]) == (2, [-1, -1, 1, -1, 0, -1])
    # e4 (7) against pinned e0 (6): 28 > 30 fails, nothing moves
    assert moe.moe_tier_plan([6, 0, 9, 1, 7, 3], 2, [0, -1, 1, -1, -1, -1]) == (0, [0, -1, 1, -1, -1, -1])
    # exactly 25% hotter is not enough (5 vs 4: 20 > 20 fails)
    assert moe.moe_tier_plan([4, 5], 1, [0, -1]) == (0, [0, -1])
    assert moe.moe_tier_plan([4, 6], 1, [0, -1]) == (1, [-1, 0])


def test_four_swaps_at_most():
    E, C = 12, 6
    heat = [1] * C + [100] * (E - C)      # six cold pinned, six hot streamed
    slot_in = list(range(C)) + [-1] * (E - C)
    n, out = moe.moe_tier_plan(heat, C, slot_in)
    assert n == 4 and sum(s >= 0 for s in out) == C
    assert moe.moe_tier_plan(heat, C, slot_in, max_swaps=6)[0] == 6
    assert moe.moe_tier_plan(heat, C, slot_in, max_swaps=0)[0] == 0


def test_ties_go_to_the_lower_index():
    # equal heat: e1 is streamed before e3; the coldest pinned tie goes to the higher index first
    n, out = moe.moe_tier_plan([1, 8, 1, 8], 2, [0, -1, 1, -1], max_swaps=1)
    assert n == 1 and out == [0, 1, -1, -1]


def test_bad_arguments():
    with pytest.raises(MoeError):
        moe.moe_tier_plan([1, 2, 3], 2, [0, 0, -1])     # two experts in one slot
    with pytest.raises(MoeError):
        moe.moe_tier_plan([1, 2, 3], 2, [0, 2, -1])     # slot out of range
    with pytest.raises(MoeError):
        moe.moe_tier_plan([1, 2, 3], 4, [-1, -1, -1])   # more slots than experts


def policy(heat, C, slot_in, max_swaps):
    """The repin decision, stated step by step."""
    E = len(heat)
    out = list(slot_in)
    used = {s for s in slot_in if s >= 0}
    streamed = sorted((e for e in range(E) if slot_in[e] < 0 and heat[e] > 0), key=lambda e: (-heat[e], e))
    i = 0
    for s in range(C):
        if s not in used and i < len(streamed):
            out[streamed[i]] = s
            i += 1
    pinned = sorted((e for e in range(E) if slot_in[e] >= 0), key=lambda e: (heat[e], -e))
    swaps = 0
    for cold in pinned:
        if swaps == max_swaps or i == len(streamed) or not 4 * heat[streamed[i]] > 5 * heat[cold]:
            break
        out[streamed[i]] = out[cold]
        out[cold] = -1
        i += 1
        swaps += 1
    return sum(1 for e in range(E) if out[e] >= 0 and slot_in[e] < 0), out


@pytest.mark.parametrize("seed", range(40))
def test_random_against_policy_and_invariants(seed):
    r = random.Random(seed)
    E = r.choice([8, 16, 64, 256])
    C = r.randint(0, E)
    heat = [r.choice([0, 0, 1, 2, 3, r.randint(0, 1000)]) for _ in range(E)]
    slots = r.sample(range(C), r.randint(0, C)) if C else []
    slot_in = [-1] * E
    for s, e in zip(slots, r.sample(range(E), len(slots))):
        slot_in[e] = s
    max_swaps = r.choice([0, 1, 4, 4, 8])
    n, out = moe.moe_tier_plan(heat, C, slot_in, max_swaps)
    assert (n, out) == policy(heat, C, slot_in, max_swaps)
    # invariants: each slot holds one expert; residents leave only by a swap
    taken = [s for s in out if s >= 0]
    assert len(taken) == len(set(taken)) and all(0 <= s < C for s in taken)
    free_before = C - sum(s >= 0 for s in slot_in)
    entered = [e for e in range(E) if out[e] >= 0 and slot_in[e] < 0]
    left = [e for e in range(E) if slot_in[e] >= 0 and out[e] < 0]
    assert n == len(entered) and len(left) <= max_swaps
    assert len(entered) == len(left) + min(free_before, len(entered))
    # each displaced expert's slot went to one more than 25% hotter; only used experts enter
    for e in left:
        (x,) = [i for i in entered if out[i] == slot_in[e]]
        assert 4 * heat[x] > 5 * heat[e]
    assert all(heat[e] > 0 for e in entered)
