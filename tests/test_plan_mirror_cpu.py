"""CPU pins of the paged split-plan mirror (tests/plan_mirror.py): whatever the batch and
range count, its segments cover every visible tile of every request exactly once and in
order, slots are unique and inside the workspace, the per-request first / last ranges
bracket the request's segments, and the layout matches mla_paged_workspace_bytes.  A
mirror with an off-by-one in the tile mapping or the cost axis fails these."""

import numpy as np
import pytest

import mla_split_kv_02_amd as mla
import plan_mirror as pm


def _check_partition(lens, ns, q_len=1, window=0, max_len=1 << 20, tile=32):
    segs, first, last, W = pm.plan(lens, max_len, ns, q_len, window, tile)
    n = [min(max(x, 0), max_len) for x in lens]
    cover = {b: [] for b in range(len(lens))}
    slots = set()
    for s in segs:
        assert 0 <= s.w < ns and s.slot == s.w + s.b and s.slot < ns + len(lens) - 1
        assert s.slot not in slots
        slots.add(s.slot)
        assert 0 <= s.t0 < s.t1 <= n[s.b]
        cover[s.b].append((s.t0, s.t1, s.w))
    for b, parts in cover.items():
        if n[b] == 0:
            assert not parts and first[b] == -1 and last[b] == -1
            continue
        lo = (max(n[b] - q_len - window + 1, 0) // tile) * tile if window > 0 else 0
        parts.sort()
        assert parts[0][0] == lo and parts[-1][1] == n[b]
        for a, c in zip(parts, parts[1:]):
            assert a[1] == c[0] and a[2] < c[2]          # contiguous, ranges increasing
            assert a[1] % tile == 0                      # cuts fall on tile boundaries
        assert first[b] == parts[0][2] and last[b] == parts[-1][2]
    tiles = [-(-x // tile) - ((max(x - q_len - window + 1, 0) // tile) if window > 0 else 0) if x > 0 else 0
             for x in n]
    assert W == sum(t + pm.segment_cost(tile) for t in tiles if t > 0)
    return segs


@pytest.mark.parametrize("seed", range(12))
def test_mirror_partitions_random_batches(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.2] = 0
    for tile in (32, 64):
        for ns in (1, 2, 3, 7, 64, 256, 1000):
            _check_partition(lens.tolist(), ns, tile=tile)
            _check_partition(lens.tolist(), ns, q_len=2, window=int(rng.integers(1, 500)), tile=tile)


def test_mirror_one_range_is_one_segment_per_request():
    lens = [5, 0, 64, 33, 1]
    segs = _check_partition(lens, 1)
    assert [(s.b, s.slot, s.t0, s.t1) for s in segs] == [(0, 0, 0, 5), (2, 2, 0, 64), (3, 3, 0, 33), (4, 4, 0, 1)]


def test_mirror_balances_cost():
    """Ranges take equal shares of the cost axis: with one request of 1000 tiles and 4
    ranges, the cost cuts fall at 252, 505 and 757 of the 1010 units (the first 10 are
    the overhead part), i.e. at tiles 242, 495 and 747."""
    segs = _check_partition([32000], 4)
    assert [(s.t0 // 32, s.t1 // 32) for s in segs] == [(0, 242), (242, 495), (495, 747), (747, 1000)]


def test_mirror_balances_cost_64_token_tiles():
    """The same request in 64-token tiles (500 tiles + 8 overhead units = 508): the cost
    cuts fall at 127, 254 and 381, i.e. at tiles 119, 246 and 373."""
    segs = _check_partition([32000], 4, tile=64)
    assert [(s.t0 // 64, s.t1 // 64) for s in segs] == [(0, 119), (119, 246), (246, 373), (373, 500)]


def test_layout_matches_library_size():
    for B, q_len, H, ns in ((64, 1, 128, 256), (1, 1, 16, 1), (128, 2, 128, 128), (7, 8, 64, 33)):
        L = pm.workspace_layout(B, q_len, H, ns)
        assert L["total"] == mla.paged_workspace_bytes(B, q_len, H, ns)
