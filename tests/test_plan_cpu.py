"""The length-aware split plan (mla_plan_decode_splits) on the host: no GPU.

For seeded length mixes (the paged V3 workload's U[1024, 16384], uniform
lengths, short and empty sequences, one long sequence among short ones) the
plan must cover every sequence's 32-token tiles exactly once, give every
sequence at least one item, keep a sequence's item sizes within one tile of
each other, number the partial rows 0 .. n-1 with a sequence's items on
consecutive rows in token order (the merge map), list the items longest
first (the launch order), stay within the capacity, have no item longer than
the one-round budget (the fewest tiles per item such that every item has a
resident workgroup slot), and predict a launch no longer than the one-round
plan's under the planner's own dispatch model (workgroup i on XCD i % 8, each
XCD starting its next item on its first free slot, an item costing its tiles
plus 4)."""
import heapq

import numpy as np
import pytest

from mla_absorbed_latent_absorb_amd import binding

ITEM_COST = 4  # fixed cost of an item in the planner's model, in tiles


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def _slots(H, cus):
    # resident workgroups per CU of the bf16 decode kernels (LDS-bound):
    # 128 heads 1, 64 heads 2, 32 heads 4, 16 heads 1
    per_cu = 1 if H >= 128 else (2 if H >= 64 else (4 if H >= 32 else 1))
    return cus * per_cu


def _min_tiles(max_len):
    return -(-max(32, min(256, max_len // 32)) // 32)


def _one_round_budget(tiles, slots, min_tiles):
    """Smallest per-item tile budget (>= min_tiles) whose cut fits `slots`."""
    top = max([min_tiles] + list(tiles))
    for per in range(min_tiles, top + 1):
        if sum(max(1, -(-t // per)) for t in tiles) <= max(slots, len(tiles)):
            return per
    return top


def _cut(tiles, per):
    """Near-equal consecutive items of at most `per` tiles, in launch order."""
    its = []
    for b, t in enumerate(tiles):
        n = max(1, -(-t // per))
        for i in range(n):
            its.append(t // n + (1 if i < t % n else 0))
    return sorted(its, reverse=True)


def _predicted(counts, slots):
    groups = 8 if slots % 8 == 0 else 1
    worst = 0
    for x in range(groups):
        h = [0] * (slots // groups)
        for c in counts[x::groups]:
            heapq.heappush(h, heapq.heappop(h) + ITEM_COST + c)
        worst = max(worst, max(h))
    return worst


def _check_plan(lens, max_len, H, cus):
    B = len(lens)
    d = binding.dims(B, H, 0.07)
    items, first = binding.mla_plan_decode_splits(d, lens, max_len, cus)
    items, first = items.numpy(), first.numpy()
    n = items.shape[0]
    assert items.shape[1] == 4
    tiles = [-(-min(max(int(t), 0), max_len) // 32) for t in lens]
    assert n <= B + 12 * cus
    # partial rows: a permutation of 0 .. n-1
    assert sorted(items[:, 3].tolist()) == list(range(n))
    # launch order: longest first
    assert np.all(np.diff(items[:, 2]) <= 0)
    by_row = items[np.argsort(items[:, 3])]
    assert first[0] == 0 and first[B] == n
    for b in range(B):
        its = by_row[first[b]:first[b + 1]]
        assert len(its) >= 1, b
        assert np.all(its[:, 0] == b)
        # consecutive rows, in token order, covering [0, tiles_b)
        pos = 0
        for _, f, c, _ in its:
            assert f == pos
            pos += c
        assert pos == tiles[b], (b, pos, tiles[b])
        if tiles[b] > 0:
            assert its[:, 2].min() >= 1
            assert its[:, 2].max() - its[:, 2].min() <= 1
    slots = _slots(H, cus)
    best = _one_round_budget(tiles, slots, _min_tiles(max_len))
    assert items[:, 2].max() <= max(best, 0)
    assert _predicted(items[:, 2].tolist(), slots) <= _predicted(_cut(tiles, best), slots)
    return items, first


def test_plan_paged_v3_lengths(lib):
    """The paged V3 mix: more, shorter items than slots, dispatched longest
    first, predict a shorter launch than one item per slot."""
    rng = np.random.default_rng(20264)
    lens = rng.integers(1024, 16385, 128)
    items, _ = _check_plan(lens, int(lens.max()), 128, 256)
    uniform_chunk_tiles = 256  # ceil(16384 / 2) tokens at the recommended 2 splits
    assert items[:, 2].max() < uniform_chunk_tiles
    tiles = [-(-int(t) // 32) for t in lens]
    one_round = _cut(tiles, _one_round_budget(tiles, 256, _min_tiles(int(lens.max()))))
    assert len(one_round) <= 256 < items.shape[0]
    assert _predicted(items[:, 2].tolist(), 256) < 0.9 * _predicted(one_round, 256)


@pytest.mark.parametrize("seed,B,lo,hi,H,cus", [(1, 32, 4096, 4096, 128, 256), (2, 64, 4096, 4096, 16, 256),
                                                 (3, 7, 0, 50, 64, 80), (4, 300, 1, 9000, 128, 256),
                                                 (5, 1, 26, 26, 16, 256), (6, 16, 0, 0, 32, 256),
                                                 (7, 33, 100, 70000, 128, 304)])
def test_plan_invariants(lib, seed, B, lo, hi, H, cus):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, B)
    _check_plan(lens, max(int(lens.max()), 1), H, cus)


def test_plan_one_long_sequence_among_short(lib):
    lens = [32768] + [64] * 63
    items, first = _check_plan(lens, 32768, 128, 256)
    # the long one takes the spare slots down to the shortest split (256 tokens)
    assert first[1] - first[0] == 1024 // 8 and items[:, 2].max() == 8


def test_plan_uniform_lengths_match_uniform_splits(lib):
    """Equal lengths: the plan is the uniform split rule at the recommended
    split count (V3, B=32, 4096 tokens: 8 items of 16 tiles per sequence)."""
    d = binding.dims(32, 128, 0.07)
    items, first = binding.mla_plan_decode_splits(d, [4096] * 32, 4096, 256)
    assert items.shape[0] == 256
    assert set(items[:, 2].tolist()) == {16}
    assert binding.mla_recommended_splits(d, 4096, 256) == 8


def test_plan_lengths_clamped_and_empty(lib):
    d = binding.dims(4, 16, 0.07)
    items, first = binding.mla_plan_decode_splits(d, [0, -5, 100, 10 ** 6], 100, 256)
    items = items.numpy()
    # empty sequences: one item without tiles (launched last); the others 4
    # tiles each, cut down to the shortest split (32 tokens at this context)
    assert list(first.numpy()) == [0, 1, 2, 6, 10]
    assert items[:4].tolist() == [[2, i, 1, 2 + i] for i in range(4)]
    assert items[4:8].tolist() == [[3, i, 1, 6 + i] for i in range(4)]
    assert items[8:].tolist() == [[0, 0, 0, 0], [1, 0, 0, 1]]


def test_plan_errors_name_the_field(lib):
    import ctypes
    d = binding.dims(3, 128, 0.07)
    lens = (ctypes.c_int32 * 3)(10, 20, 30)
    items = (ctypes.c_int32 * 12)()
    first = (ctypes.c_int32 * 4)()
    n = ctypes.c_int32(0)
    st = lib.mla_plan_decode_splits(ctypes.byref(d), ctypes.cast(lens, ctypes.c_void_p), 30, 256, 1,
                                    ctypes.cast(items, ctypes.c_void_p), ctypes.cast(first, ctypes.c_void_p),
                                    ctypes.byref(n))
    assert st == 5 and "capacity" in binding.mla_last_error()
    st = lib.mla_plan_decode_splits(ctypes.byref(d), None, 30, 256, 1, ctypes.cast(items, ctypes.c_void_p),
                                    ctypes.cast(first, ctypes.c_void_p), ctypes.byref(n))
    assert st == 1 and "host_seq_lens" in binding.mla_last_error()
    d0 = binding.dims(3, 128, 0.07, kv_lora_rank=0)
    st = lib.mla_plan_decode_splits(ctypes.byref(d0), ctypes.cast(lens, ctypes.c_void_p), 30, 256, 3,
                                    ctypes.cast(items, ctypes.c_void_p), ctypes.cast(first, ctypes.c_void_p),
                                    ctypes.byref(n))
    assert st == 2 and "kv_lora_rank" in binding.mla_last_error()
