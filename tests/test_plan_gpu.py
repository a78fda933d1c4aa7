"""Planned split-KV decode (mla_plan_decode_splits -> mla_decode_latent_planned
-> mla_combine_splits_planned / mla_combine_expand_v_planned) through the C
ABI, against the oracle: every item's partial (o_i, lse_i) against the
oracle's latent attention over that item's token range, every merged row
against the oracle's decode, and the paged V3 workload (B=128, lengths
U[1024, 16384]) at full size end to end, every sequence.  Equal lengths give
the uniform rule's items, bit for bit.  Malformed items and merge ranges
produce zero-weight results and touch nothing outside the outputs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import (TOL_BF16, TOL_FP8, assert_guards, cache_args, f64, guarded, rel_err,
                               split_bounds)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FP8_PAGED = dataclasses.replace(datagen.WORKLOADS["v3_b128_paged"], name="v3_b128_paged_fp8", dtype="fp8_e4m3",
                                seed=20266)


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(workload, **kw):
    wl = FP8_PAGED if workload == FP8_PAGED.name else datagen.WORKLOADS[workload]
    return datagen.make_inputs(wl, device=DEV, **kw)


def _cache(x):
    return binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                              block_size=x.block_size, token_scale=x.token_scale)


def _ncu():
    return torch.cuda.get_device_properties(DEV).multi_processor_count


@pytest.mark.parametrize("workload,H,B,T,cus", [("v3_b128_paged", 128, 6, 3000, 16), ("v3_b128_paged", 16, 5, 2000, 8),
                                                ("v3_b128_paged_fp8", 128, 4, 2500, 12),
                                                ("v3_b32_s4096", 64, 3, 777, 256)])
def test_planned_partials_and_merge_vs_oracle(workload, H, B, T, cus):
    announce(f"planned decode + merge {workload} H={H} B={B} T<={T} cus={cus}")
    x = _inputs(workload, batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, 41, device=DEV)
    d = binding.dims(B, H, x.scale)
    lens = x.seq_lens.cpu().numpy()
    plan = binding.mla_plan_decode_splits(d, lens, x.max_seq_len, cus, device=DEV)
    n = plan.num_items
    assert n > B  # some sequences are cut
    gp, glp, go, gl = guarded(DEV, ((n, H, 512), torch.bfloat16), ((n, H), torch.float32),
                              ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    binding.mla_decode_latent_planned(d, _cache(x), q_lat, x.q_pe, x.seq_lens, x.max_seq_len, plan, o_part=gp.tensor,
                                      lse_part=glp.tensor)
    binding.mla_combine_splits_planned(d, gp.tensor, glp.tensor, plan, o_lat=go.tensor, lse=gl.tensor)
    torch.cuda.synchronize()
    assert_guards(gp, glp, go, gl)
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    args = cache_args(x)
    q64, qpe64 = f64(q_lat), f64(x.q_pe)
    op, lp = f64(gp.tensor), glp.tensor.cpu().numpy()
    items, first = plan.items_host.numpy(), plan.seq_first_host.numpy()
    by_row = items[np.argsort(items[:, 3])]  # items in partial-row order
    for b in range(B):
        T_b = int(lens[b])
        slots = oracle.token_slots(b, T_b, args["seq_stride"], args["block_table"], args["block_size"])
        c, k_r = oracle.load_rows(args["kv_codes"], args["pe_codes"], slots, args["dtype"], args["token_scale"])
        its = by_row[first[b]:first[b + 1]]
        bounds = [min(32 * int(f), T_b) for _, f, _, _ in its] + [T_b]
        ro, rl = oracle.latent_attention_ranges(q64[b], qpe64[b], c, k_r, x.scale, bounds)
        for i, row in enumerate(range(first[b], first[b + 1])):
            assert rel_err(op[row], ro[i]) <= tol, (b, i)
            assert np.max(np.abs(lp[row] - rl[i])) <= tol, (b, i)
    ref_o, ref_l = oracle.latent_decode(q64, qpe64, seq_lens=lens, scale=x.scale, **args)
    e_o, e_l = rel_err(f64(go.tensor), ref_o), float(np.max(np.abs(gl.tensor.cpu().numpy() - ref_l)))
    print(f"  {n} items: o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= tol and e_l <= tol
    # the partial row comes from the item, not from its launch position: the
    # same items launched in a shuffled order give the same bits
    perm = torch.from_numpy(np.random.default_rng(7).permutation(n))
    shuffled = binding.SplitPlan(plan.items_host[perm].contiguous(), plan.seq_first_host, DEV)
    op2, lp2 = binding.mla_decode_latent_planned(d, _cache(x), q_lat, x.q_pe, x.seq_lens, x.max_seq_len, shuffled)
    o2, l2 = binding.mla_combine_splits_planned(d, op2, lp2, shuffled)
    torch.cuda.synchronize()
    assert torch.equal(op2, gp.tensor) and torch.equal(lp2, glp.tensor)
    assert torch.equal(o2, go.tensor) and torch.equal(l2, gl.tensor)


def test_planned_equal_lengths_equal_uniform_splits_bitwise():
    """Equal lengths: the plan's items are the uniform rule's splits, so the
    partials and the merge are bit-identical to mla_decode_latent with that
    split count."""
    announce("planned == uniform bitwise, V3 B=4 T=1024 P=8")
    B, H, T = 4, 128, 1024
    x = _inputs("v3_b32_s4096", batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, 42, device=DEV)
    d = binding.dims(B, H, x.scale)
    plan = binding.mla_plan_decode_splits(d, [T] * B, T, 32, device=DEV)
    assert plan.num_items == 32 and set(plan.items_host[:, 2].tolist()) == {4}
    cache = _cache(x)
    op, lp = binding.mla_decode_latent_planned(d, cache, q_lat, x.q_pe, x.seq_lens, T, plan)
    ou, lu = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, T, 8)
    o1, l1 = binding.mla_combine_splits_planned(d, op, lp, plan)
    o2, l2 = binding.mla_combine_splits(d, ou, lu)
    torch.cuda.synchronize()
    assert torch.equal(op, ou.view(32, H, 512)) and torch.equal(lp, lu.view(32, H))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_planned_full_size_paged_v3_every_sequence():
    """The paged V3 workload (B=128, lengths U[1024, 16384]) through the
    planned step absorb_q -> decode_latent_planned -> combine_expand_v_planned,
    every sequence against the oracle's absorbed decode."""
    announce("planned full step v3_b128_paged, all 128 sequences")
    x = _inputs("v3_b128_paged")
    d = binding.dims(x.batch, x.heads, x.scale)
    lens = x.seq_lens.cpu().numpy()
    plan = binding.mla_plan_decode_splits(d, lens, x.max_seq_len, _ncu(), device=DEV)
    q_lat = binding.mla_absorb_q(d, x.q_nope, x.w_uk)
    op, lp = binding.mla_decode_latent_planned(d, _cache(x), q_lat, x.q_pe, x.seq_lens, x.max_seq_len, plan)
    o_lat = torch.empty((x.batch, x.heads, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((x.batch, x.heads), dtype=torch.float32, device=DEV)
    out = binding.mla_combine_expand_v_planned(d, op, lp, plan, x.w_uv, o_lat=o_lat, lse=lse)
    o2, l2 = binding.mla_combine_splits_planned(d, op, lp, plan)
    torch.cuda.synchronize()
    assert torch.equal(o_lat, o2) and torch.equal(lse, l2)
    ref = oracle.absorbed_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv), seq_lens=lens, scale=x.scale,
                                 batch_indices=list(range(x.batch)), **cache_args(x))
    e_out, e_lat = rel_err(f64(out), ref["out"]), rel_err(f64(o_lat), ref["o_lat"])
    e_lse = float(np.max(np.abs(lse.cpu().numpy() - ref["lse"])))
    print(f"  {plan.num_items} items, longest {int(plan.items_host[:, 2].max())} tiles: out {e_out:.2e} "
          f"o_lat {e_lat:.2e} lse {e_lse:.2e}")
    assert max(e_out, e_lat, e_lse) <= TOL_BF16


@pytest.mark.parametrize("H", [128, 32])
def test_planned_malformed_items_and_ranges(H):
    """Items naming a sequence outside the batch, a negative or too-large
    first tile, or no tiles write o = 0, lse = -inf into their own rows; items
    whose partial row is outside [0, n) write nothing; merge ranges that are
    empty or leave the partials give o = 0, lse = -inf, out = 0; nothing is
    written outside the outputs."""
    announce(f"planned malformed items / ranges H={H}")
    B, T = 3, 200
    x = _inputs("v3_b32_s4096", batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, 43, device=DEV)
    d = binding.dims(B, H, x.scale)
    items = torch.tensor([[0, 0, 7, 0], [-1, 0, 3, 1], [B, 0, 3, 2], [1, -3, 2, 3], [1, 0, 0, 4], [2, 100, 1, 5],
                          [2, 0, 7, 6], [0, 0, 7, -1], [2, 0, 7, 9]], dtype=torch.int32)
    first = torch.tensor([0, 1, 5, 99], dtype=torch.int32)
    plan = binding.SplitPlan(items, first, DEV)
    n = plan.num_items
    gp, glp, go, gl, gout = guarded(DEV, ((n, H, 512), torch.bfloat16), ((n, H), torch.float32),
                                    ((B, H, 512), torch.bfloat16), ((B, H), torch.float32),
                                    ((B, H, 128), torch.bfloat16))
    binding.mla_decode_latent_planned(d, _cache(x), q_lat, x.q_pe, x.seq_lens, T, plan, o_part=gp.tensor,
                                      lse_part=glp.tensor)
    binding.mla_combine_splits_planned(d, gp.tensor, glp.tensor, plan, o_lat=go.tensor, lse=gl.tensor)
    torch.cuda.synchronize()
    op, lp = gp.tensor, glp.tensor
    for i in (1, 2, 3, 4, 5):
        assert torch.all(op[i] == 0) and torch.all(torch.isneginf(lp[i])), i
    # rows 7 and 8 belong to no valid item: still the initial NaN fill
    for i in (7, 8):
        assert torch.all(torch.isnan(op[i].float())) and torch.all(torch.isnan(lp[i])), i
    args = cache_args(x)
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=np.array([T] * B), scale=x.scale, **args)
    # sequence 0: item 0 covers all 200 tokens
    assert rel_err(f64(op[0]), ref_o[0]) <= TOL_BF16
    assert rel_err(f64(go.tensor[0]), ref_o[0]) <= TOL_BF16
    # sequence 1: items 1..4 are all empty -> zero weight; sequence 2: range ends past the partials
    for b in (1, 2):
        assert torch.all(go.tensor[b] == 0) and torch.all(torch.isneginf(gl.tensor[b])), b
    w_uv = x.w_uv
    binding.mla_combine_expand_v_planned(d, gp.tensor, glp.tensor, plan, w_uv, out=gout.tensor)
    torch.cuda.synchronize()
    assert torch.all(gout.tensor[1] == 0) and torch.all(gout.tensor[2] == 0)
    assert_guards(gp, glp, go, gl, gout)
