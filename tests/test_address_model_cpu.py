"""Every cache read, LDS access and output store of the decode kernels (and
of the absorb_q / expand_v projections) stays in bounds
(tests/address_model.py: the kernels' address arithmetic on the host), for
the shapes the GPU tests use and the five benchmark
workloads at full size -- including the copies issued past the last tile,
the clamped rows of ragged tiles, split boundaries, planned items, paged
caches with 32-, 64- and 256-token blocks, E4M3 tiles (64-row tiles in two
32-row halves for 128 heads) and prefill query groups.  No GPU is used."""
import numpy as np
import pytest

from mla_absorbed_latent_absorb_amd import binding
from tests.address_model import (Launch, Violation, check_absorb_q, check_expand_v, check_fp8, check_latent16,
                                 check_narrow, check_wide)


def _paged(lens, bs, seed):
    rng = np.random.default_rng(seed)
    nblk = [-(-int(t) // bs) for t in lens]
    perm = rng.permutation(sum(nblk))
    table = np.zeros((len(lens), max(max(nblk), 1)), dtype=np.int64)
    off = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, sum(nblk) * bs


def _check(L, max_items=None):
    if L.H == 128:
        return (check_fp8 if L.fp8 else check_wide)(L, max_items)
    if L.H == 16 and not L.fp8:
        return check_latent16(L, max_items)
    return check_narrow(L, max_items)


def _recommended(B, H, S, cus=256):
    return binding.mla_recommended_splits(binding.dims(B, H, 0.07), S, cus)


@pytest.mark.parametrize("name,H,B,S,fp8,P", [
    ("v2lite_b1_s26", 16, 1, 26, False, 1),
    ("v2lite_b64_s4096", 16, 64, 4096, False, None),
    ("v3_b32_s4096", 128, 32, 4096, False, None),
    ("v3_b64_s32768_fp8", 128, 64, 32768, True, None),
])
def test_benchmark_workloads_contiguous(name, H, B, S, fp8, P):
    P = P or _recommended(B, H, S)
    L = Launch(H, [S] * B, S, num_splits=P, fp8=fp8, seq_stride=S, num_slots=B * S)
    c = _check(L, max_items=None if B * P <= 256 else 96)
    assert c["copies"] > 0 and c["stores"] > 0


@pytest.mark.parametrize("planned", [False, True])
@pytest.mark.parametrize("fp8", [False, True])
def test_paged_v3_workload(planned, fp8):
    rng = np.random.default_rng(20264)
    lens = rng.integers(1024, 16385, 128)
    S = int(lens.max())
    table, slots = _paged(lens, 64, 1)
    items = None
    if planned:
        it, _ = binding.mla_plan_decode_splits(binding.dims(128, 128, 0.07), lens, S, 256)
        items = it.numpy()
    L = Launch(128, lens, S, num_splits=_recommended(128, 128, S), fp8=fp8, block_table=table, block_size=64,
               num_slots=slots, items=items)
    c = _check(L, max_items=64)
    assert c["workgroups"] == 64


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("P", [1, 3, 16])
def test_ragged_lengths_and_splits(H, fp8, P):
    lens = [0, 1, 31, 32, 33, 95, 700, 1000]
    S = 1000
    L = Launch(H, lens, S, num_splits=P, fp8=fp8, seq_stride=S, num_slots=len(lens) * S)
    _check(L)


@pytest.mark.parametrize("bs", [32, 64, 256])
@pytest.mark.parametrize("H,fp8", [(128, False), (16, False), (128, True), (32, True)])
def test_paged_block_sizes(bs, H, fp8):
    lens = [700, 1, 257, 64]
    table, slots = _paged(lens, bs, bs)
    L = Launch(H, lens, 700, num_splits=4, fp8=fp8, block_table=table, block_size=bs, num_slots=slots)
    _check(L)


def test_planned_items_including_malformed():
    lens = [200, 200, 200]
    items = [[0, 0, 7, 0], [-1, 0, 3, 1], [3, 0, 3, 2], [1, -3, 2, 3], [1, 0, 0, 4], [2, 100, 1, 5], [2, 0, 7, 6],
             [1, 2, 10 ** 6, 7], [0, 0, 7, -1], [2, 0, 7, 9]]
    for H in (128, 32):
        _check(Launch(H, lens, 200, seq_stride=200, num_slots=600, items=items))


@pytest.mark.parametrize("H,L_,starts,P,qg", [(128, 37, [100, 0], 1, 1), (16, 21, [0, 250], 1, 8),
                                              (32, 6, [100, 0, 254], 1, 4), (64, 9, [650, 200], 3, 1)])
def test_prefill_rows(H, L_, starts, P, qg):
    S = 700
    lens = [S] * len(starts)
    L = Launch(H, lens, S, num_splits=P, seq_stride=S, num_slots=len(starts) * S, q_start=starts, q_per_seq=L_,
               q_group=qg)
    # grouped queries (q_group > 1) run on the 128-row kernel
    (check_wide if qg > 1 or H == 128 else _check)(L)


def test_checker_catches_a_cache_too_small_for_the_lengths():
    """The model is live: lengths beyond the allocation are reported."""
    L = Launch(128, [100, 100], 100, seq_stride=100, num_slots=150)
    with pytest.raises(Violation):
        check_wide(L)
    L = Launch(16, [100, 100], 100, seq_stride=100, num_slots=150)
    with pytest.raises(Violation):
        check_latent16(L)
    L = Launch(32, [100, 100], 100, seq_stride=100, num_slots=150)
    with pytest.raises(Violation):
        check_narrow(L)
    L = Launch(128, [100, 100], 100, fp8=True, seq_stride=100, num_slots=150)
    with pytest.raises(Violation):
        check_fp8(L)


def test_fp8_checker_catches_a_half_tile_across_blocks():
    """A 64-row tile is copied as two 32-row halves, each from its own block:
    with 16-token blocks a half would span two blocks, which the model reports
    (the host accepts block sizes that are multiples of 32 only)."""
    lens = [100]
    table, slots = _paged(lens, 16, 3)
    with pytest.raises(Violation):
        check_fp8(Launch(128, lens, 100, fp8=True, block_table=table, block_size=16, num_slots=slots))


def test_checker_catches_unclamped_ragged_rows(monkeypatch):
    """Without the clamp of a ragged tile's rows the 128-row kernel would read
    rows past the end of its range; the model reports it."""
    import tests.address_model as am
    L = Launch(128, [33, 700], 700, num_splits=3, seq_stride=700, num_slots=1400)
    check_wide(L)
    monkeypatch.setattr(am, "CLAMP_RAGGED_ROWS", False)
    with pytest.raises(Violation):
        check_wide(L)


# The projection kernels (absorb_q_kernel<NW>, expand_v_kernel<NW>): the GPU
# tests' shapes and the five workloads' (batch, heads).
@pytest.mark.parametrize("B,H", [(1, 16), (5, 16), (64, 16), (3, 32), (17, 64), (130, 64), (200, 16), (32, 128),
                                 (64, 128), (128, 128)])
def test_projection_kernels_in_bounds(B, H):
    a = check_absorb_q(B, H)
    e = check_expand_v(B, H)
    # one 16-byte q_lat store per 8 columns, one 8-byte out store per 4 columns
    assert a["stores"] == B * H * 512 // 8
    assert e["stores"] == B * H * 128 // 4
    assert a["copies"] == e["copies"] == H * 8 * 16
