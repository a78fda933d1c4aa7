"""Parity of the HIP library (through its C ABI) with the float64 oracle.

Every case draws seeded inputs with the generator module, runs the GPU path,
and compares element by element with the oracle on the same stored bytes:
max |gpu - oracle| / max |oracle| <= 2e-2 for bf16 outputs (fp32
accumulation), lse within 2e-2 absolute.  Full-size workloads are checked on
every sequence (all heads, all 512 latent columns).  Outputs of the per-call
cases are guarded: they sit between sentinel regions that must stay intact,
and start as NaN patterns that fail the comparison if left unwritten.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import (TOL_BF16, TOL_FP8, assert_guards, bits8, bits16, cache_args, f64, guarded,
                               mismatch_report, rel_err, tol_for,
                               split_bounds)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


# E4M3 variant of the paged workload (same structure, fp8 cache): the ABI
# accepts every layout with either dtype.
FP8_PAGED = dataclasses.replace(datagen.WORKLOADS["v3_b128_paged"], name="v3_b128_paged_fp8", dtype="fp8_e4m3",
                                seed=20266)


def _inputs(workload, **kw):
    if workload == FP8_PAGED.name:
        workload = FP8_PAGED
    return datagen.make_inputs(workload, device=DEV, **kw)


def _cache(x):
    return binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                              block_size=x.block_size, token_scale=x.token_scale)


# ---------------------------------------------------------------------------
# mla_absorb_q / mla_expand_v
# ---------------------------------------------------------------------------

PROJ_CASES = [(1, 16), (5, 16), (64, 16), (3, 32), (17, 64), (32, 128), (128, 128), (130, 64), (200, 16)]


@pytest.mark.parametrize("B,H", PROJ_CASES)
def test_absorb_q(B, H):
    announce(f"absorb_q B={B} H={H}")
    x = _inputs("v3_b32_s4096", batch=B, seq_len=32, heads=H)
    d = binding.dims(B, H, x.scale)
    (g,) = guarded(DEV, ((B, H, 512), torch.bfloat16))
    q_lat = binding.mla_absorb_q(d, x.q_nope, x.w_uk, q_lat=g.tensor)
    torch.cuda.synchronize()
    assert_guards(g)
    ref = oracle.absorb_q(f64(x.q_nope), f64(x.w_uk))
    err = rel_err(f64(q_lat), ref)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("B,H", PROJ_CASES)
def test_expand_v(B, H):
    announce(f"expand_v B={B} H={H}")
    x = _inputs("v3_b32_s4096", batch=B, seq_len=32, heads=H)
    o_lat = datagen.random_latent_queries(B, H, seed=77 + B, device=DEV)
    d = binding.dims(B, H, x.scale)
    (g,) = guarded(DEV, ((B, H, 128), torch.bfloat16))
    out = binding.mla_expand_v(d, o_lat, x.w_uv, out=g.tensor)
    torch.cuda.synchronize()
    assert_guards(g)
    ref = oracle.expand_v(f64(o_lat), f64(x.w_uv))
    err = rel_err(f64(out), ref)
    assert err <= TOL_BF16, err


# ---------------------------------------------------------------------------
# mla_decode_latent, one split
# ---------------------------------------------------------------------------

DECODE_CASES = [
    # (workload for layout, H, B, T)  T covers one row, ragged tails, exact tiles, many tiles
    ("v2lite_b1_s26", 16, 1, 26),
    ("v2lite_b1_s26", 16, 2, 1),
    ("v3_b32_s4096", 16, 3, 31),
    ("v3_b32_s4096", 32, 2, 32),
    ("v3_b32_s4096", 64, 2, 33),
    ("v3_b32_s4096", 128, 2, 100),
    ("v3_b32_s4096", 128, 3, 257),
    ("v3_b32_s4096", 128, 1, 1000),
    ("v3_b32_s4096", 64, 3, 777),
    ("v3_b128_paged", 128, 3, 300),
    ("v3_b128_paged", 16, 4, 200),
    # E4M3 cache (decoded in-kernel), every head count, ragged tails
    ("v3_b64_s32768_fp8", 128, 2, 100),
    ("v3_b64_s32768_fp8", 128, 1, 1000),
    ("v3_b64_s32768_fp8", 64, 2, 257),
    ("v3_b64_s32768_fp8", 32, 2, 33),
    ("v3_b64_s32768_fp8", 16, 3, 31),
    ("v3_b128_paged_fp8", 128, 3, 300),
]


def _latent_case(workload, H, B, T, seed):
    x = _inputs(workload, batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, seed=seed, device=DEV)
    return x, q_lat


@pytest.mark.parametrize("workload,H,B,T", DECODE_CASES)
def test_decode_latent_single_split(workload, H, B, T):
    announce(f"decode_latent P=1 {workload} H={H} B={B} T={T}")
    x, q_lat = _latent_case(workload, H, B, T, seed=1000 + T)
    d = binding.dims(B, H, x.scale)
    cache = _cache(x)
    go, gl = guarded(DEV, ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    o_lat, lse = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, 1, o_lat=go.tensor,
                                           lse=gl.tensor)
    torch.cuda.synchronize()
    assert_guards(go, gl)
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=x.seq_lens.cpu().numpy(),
                                        scale=x.scale, **cache_args(x))
    err = rel_err(f64(o_lat), ref_o)
    lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
    assert err <= tol_for(x) and lerr <= tol_for(x), (err, lerr)


# ---------------------------------------------------------------------------
# split-KV partials and their merge
# ---------------------------------------------------------------------------

SPLIT_CASES = [
    ("v3_b32_s4096", 128, 2, 1000, 3),
    ("v3_b32_s4096", 128, 2, 257, 8),    # later splits empty for short sequences? (all equal lengths here)
    ("v3_b128_paged", 128, 5, 2000, 8),  # varied lengths: some splits empty
    ("v3_b32_s4096", 16, 3, 4096, 16),
    ("v3_b32_s4096", 64, 2, 95, 2),
    ("v3_b64_s32768_fp8", 128, 2, 1000, 4),
    ("v3_b128_paged_fp8", 128, 4, 1500, 8),
]


@pytest.mark.parametrize("workload,H,B,T,P", SPLIT_CASES)
def test_decode_latent_splits_and_combine(workload, H, B, T, P):
    announce(f"decode_latent P={P} + combine {workload} H={H} B={B} T={T}")
    x, q_lat = _latent_case(workload, H, B, T, seed=2000 + P)
    d = binding.dims(B, H, x.scale)
    cache = _cache(x)
    gp, glp, go, gl = guarded(DEV, ((B, P, H, 512), torch.bfloat16), ((B, P, H), torch.float32),
                              ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    o_part, lse_part = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P,
                                                 o_part=gp.tensor, lse_part=glp.tensor)
    o_lat, lse = binding.mla_combine_splits(d, o_part, lse_part, o_lat=go.tensor, lse=gl.tensor)
    torch.cuda.synchronize()
    assert_guards(gp, glp, go, gl)
    args = cache_args(x)
    lens = x.seq_lens.cpu().numpy()
    q64, qpe64 = f64(q_lat), f64(x.q_pe)
    o_part_h, lse_part_h = f64(o_part), lse_part.cpu().numpy()
    for b in range(B):
        slots = oracle.token_slots(b, int(lens[b]), args["seq_stride"], args["block_table"], args["block_size"])
        c, k_r = oracle.load_rows(args["kv_codes"], args["pe_codes"], slots, args["dtype"], args["token_scale"])
        bounds = split_bounds(int(lens[b]), x.max_seq_len, P)
        ro, rl = oracle.latent_attention_ranges(q64[b], qpe64[b], c, k_r, x.scale, bounds)
        for i in range(P):
            if np.isneginf(rl[i]).all():
                assert np.isneginf(lse_part_h[b, i]).all() and np.all(o_part_h[b, i] == 0), (b, i)
            else:
                assert rel_err(o_part_h[b, i], ro[i]) <= tol_for(x), (b, i)
                assert np.max(np.abs(lse_part_h[b, i] - rl[i])) <= tol_for(x), (b, i)
    ref_o, ref_l = oracle.latent_decode(q64, qpe64, seq_lens=lens, scale=x.scale, **args)
    assert rel_err(f64(o_lat), ref_o) <= TOL_BF16
    assert np.max(np.abs(lse.cpu().numpy() - ref_l)) <= TOL_BF16


@pytest.mark.parametrize("B,P,H", [(2, 3, 16), (4, 8, 128), (1, 1, 64), (3, 16, 32), (2, 9, 16), (2, 70, 16), (1, 130, 32)])
def test_combine_random_partials(B, P, H):
    announce(f"combine random partials B={B} P={P} H={H}")
    o_part, lse_part = datagen.random_partials(B, P, H, seed=31 + P, device=DEV)
    d = binding.dims(B, H, 0.07)
    go, gl = guarded(DEV, ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    o_lat, lse = binding.mla_combine_splits(d, o_part, lse_part, o_lat=go.tensor, lse=gl.tensor)
    torch.cuda.synchronize()
    assert_guards(go, gl)
    op, lp = o_part.cpu().double().numpy(), lse_part.cpu().double().numpy()
    for b in range(B):
        ro, rl = oracle.combine_splits(op[b], lp[b])
        assert rel_err(f64(o_lat[b]), ro) <= TOL_BF16
        assert np.max(np.abs(lse[b].cpu().numpy() - rl)) <= 1e-4


# ---------------------------------------------------------------------------
# properties that hold at any size
# ---------------------------------------------------------------------------

def _paged_copy(x, B, T, bs, seed):
    """The contiguous rows (and token scales) of x behind a block table of
    bs-token blocks in a permuted pool."""
    nblk = -(-T // bs)
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(B * nblk, generator=g)
    fp8 = x.token_scale is not None
    pool = torch.zeros((B * nblk * bs, 576), dtype=x.storage.dtype, device=DEV)
    pscale = torch.zeros((B * nblk * bs,), dtype=torch.float32, device=DEV) if fp8 else None
    table = torch.empty((B, nblk), dtype=torch.int32)
    rows = x.storage.view(B, x.seq_stride, 576)
    for b in range(B):
        for j in range(nblk):
            blk = int(perm[b * nblk + j])
            table[b, j] = blk
            n = min(bs, T - j * bs)
            pool[blk * bs: blk * bs + n] = rows[b, j * bs: j * bs + n]
            if fp8:
                pscale[blk * bs: blk * bs + n] = x.token_scale.view(B, x.seq_stride)[b, j * bs: j * bs + n]
    table = table.to(DEV)
    return binding.make_cache(pool[:, :512], pool[:, 512:], block_table=table, block_size=bs, token_scale=pscale), \
        dict(kv_codes=(bits8 if fp8 else bits16)(pool[:, :512]), pe_codes=(bits8 if fp8 else bits16)(pool[:, 512:]),
             dtype="fp8_e4m3" if fp8 else "bf16", seq_stride=None, block_table=table.cpu().numpy(), block_size=bs,
             token_scale=None if not fp8 else pscale.cpu().numpy())


@pytest.mark.parametrize("bs,H,workload", [(32, 128, "v3_b32_s4096"), (64, 128, "v3_b32_s4096"),
                                           (256, 128, "v3_b32_s4096"), (32, 16, "v3_b32_s4096"),
                                           (256, 64, "v3_b32_s4096"), (32, 128, "v3_b64_s32768_fp8"),
                                           (256, 32, "v3_b64_s32768_fp8")])
def test_paged_block_sizes(bs, H, workload):
    """The same token rows behind a permuted table of bs-token blocks give
    bit-identical outputs to the contiguous cache (the kernels read the same
    values in the same order), and match the oracle through the paged
    addressing."""
    announce(f"paged bs={bs} == contiguous bitwise and vs oracle, {workload} H={H} B=3 T=700")
    B, T = 3, 700
    x = _inputs(workload, batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, seed=5, device=DEV)
    d = binding.dims(B, H, x.scale)
    contig = _cache(x)
    paged, pargs = _paged_copy(x, B, T, bs, 9 + bs)
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    for P in (1, 4):
        a = binding.mla_decode_latent(d, contig, q_lat, x.q_pe, x.seq_lens, T, P)
        c = binding.mla_decode_latent(d, paged, q_lat, x.q_pe, x.seq_lens, T, P)
        torch.cuda.synchronize()
        if not (torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])):
            names = ("b", "split", "head", "col") if P > 1 else ("b", "head", "col")
            print(f"P={P} o: {mismatch_report(a[0], c[0], names)}", flush=True)
            print(f"P={P} lse: {mismatch_report(a[1], c[1], names[:-1])}", flush=True)
        assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1]), P
        if P == 1:
            ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=x.seq_lens.cpu().numpy(),
                                                scale=x.scale, **pargs)
            assert rel_err(f64(c[0]), ref_o) <= tol
            assert np.max(np.abs(c[1].cpu().numpy() - ref_l)) <= tol


def test_single_token_returns_that_row():
    """With one cached token the softmax weight is exactly 1, so o_lat is that
    token's latent row, bit for bit."""
    announce("T=1 -> o_lat == c_0")
    B, H = 4, 128
    x = _inputs("v3_b32_s4096", batch=B, seq_len=1, heads=H)
    q_lat = datagen.random_latent_queries(B, H, seed=6, device=DEV)
    d = binding.dims(B, H, x.scale)
    cache = _cache(x)
    o_lat, lse = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, 1, 1)
    torch.cuda.synchronize()
    for b in range(B):
        row = x.kv_rows[b * x.seq_stride]
        assert torch.equal(o_lat[b], row.unsqueeze(0).expand(H, 512)), b


def test_zero_query_averages_rows():
    """q = 0 gives a uniform softmax: o_lat is the mean latent row and
    lse = ln T."""
    announce("q=0 -> mean row, lse = ln T")
    B, H, T = 2, 64, 500
    x = _inputs("v3_b32_s4096", batch=B, seq_len=T, heads=H)
    zq = torch.zeros((B, H, 512), dtype=torch.bfloat16, device=DEV)
    zpe = torch.zeros((B, H, 64), dtype=torch.bfloat16, device=DEV)
    d = binding.dims(B, H, x.scale)
    cache = _cache(x)
    o_lat, lse = binding.mla_decode_latent(d, cache, zq, zpe, x.seq_lens, T, 1)
    torch.cuda.synchronize()
    c = f64(x.kv_rows).reshape(B, x.seq_stride, 512)[:, :T]
    mean = c.mean(axis=1)
    for b in range(B):
        assert rel_err(f64(o_lat[b]), np.repeat(mean[b][None], H, 0)) <= TOL_BF16
    assert np.max(np.abs(lse.cpu().numpy() - math.log(T))) <= 1e-5


def test_deterministic_rerun():
    """Two runs of the full step give byte-identical outputs."""
    announce("determinism v3 B=32 S=4096")
    x = _inputs("v3_b32_s4096")
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = _cache(x)
    P = binding.mla_recommended_splits(d, x.max_seq_len, torch.cuda.get_device_properties(DEV).multi_processor_count)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, P, DEV)
    a = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv).clone()
    la = step.lse.clone()
    b = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, step.lse)


# ---------------------------------------------------------------------------
# the full 4-call step on the workloads, at full size, in the bench launch
# configuration (recommended number of splits)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("workload", ["v2lite_b1_s26", "v2lite_b64_s4096", "v3_b32_s4096", "v3_b128_paged",
                                      "v3_b64_s32768_fp8"])
def test_full_step_against_oracle(workload):
    announce(f"full step {workload}")
    x = _inputs(workload)
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = _cache(x)
    ncu = torch.cuda.get_device_properties(DEV).multi_processor_count
    P = binding.mla_recommended_splits(d, x.max_seq_len, ncu)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, P, DEV)
    out = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv)
    torch.cuda.synchronize()
    idx = list(range(x.batch))
    ref = oracle.absorbed_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                                 seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale, batch_indices=idx,
                                 **cache_args(x))
    got_out = f64(out)[idx]
    e_out = rel_err(got_out, ref["out"])
    e_lat = rel_err(f64(step.o_lat)[idx], ref["o_lat"])
    e_q = rel_err(f64(step.q_lat)[idx], ref["q_lat"])
    e_lse = float(np.max(np.abs(step.lse.cpu().numpy()[idx] - ref["lse"])))
    print(f"  {workload} P={P} all {x.batch} sequences: out {e_out:.2e} o_lat {e_lat:.2e} q_lat {e_q:.2e} lse {e_lse:.2e}")
    assert np.isfinite(got_out).all()
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    assert max(e_out, e_lat, e_q, e_lse) <= tol


def test_v2lite_s26_against_naive_oracle():
    """The 26-token V2-Lite-shaped step also matches the expanded (naive)
    form of the oracle."""
    announce("v2lite_b1_s26 vs naive oracle")
    x = _inputs("v2lite_b1_s26")
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = _cache(x)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, 1, DEV)
    out = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv)
    torch.cuda.synchronize()
    ref = oracle.naive_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                              seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale, **cache_args(x))
    assert rel_err(f64(out), ref) <= TOL_BF16


def test_fp8_decode_matches_bf16_decode_of_the_decoded_cache():
    """An E4M3 cache and the bf16 cache holding the same decoded values
    (e4m3 * scale, rounded to bf16) give the same result up to the rounding
    of the P.V weights (E4M3 with a block scale per 32 tokens for 128 heads)
    and of the bf16 copy: a property check that needs no oracle; lse, which
    keeps the exact sum, agrees closely."""
    announce("fp8 vs bf16 of the decoded values, H=128 B=2 T=700")
    x = _inputs("v3_b64_s32768_fp8", batch=2, seq_len=700, heads=128)
    d = binding.dims(2, 128, x.scale)
    q_lat = datagen.random_latent_queries(2, 128, seed=77, device=DEV)
    o8, l8 = binding.mla_decode_latent(d, _cache(x), q_lat, x.q_pe, x.seq_lens, x.max_seq_len, 1)
    # decode on the host with the oracle's E4M3 table, round to bf16 on the device
    args = cache_args(x)
    vals = oracle.e4m3fn_to_f64(args["kv_codes"]) * args["token_scale"][:, None]
    pes = oracle.e4m3fn_to_f64(args["pe_codes"]) * args["token_scale"][:, None]
    kv16 = torch.from_numpy(vals).to(device=DEV, dtype=torch.float32).to(torch.bfloat16).contiguous()
    pe16 = torch.from_numpy(pes).to(device=DEV, dtype=torch.float32).to(torch.bfloat16).contiguous()
    c16 = binding.make_cache(kv16, pe16, seq_stride=x.seq_stride)
    o16, l16 = binding.mla_decode_latent(d, c16, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, 1)
    torch.cuda.synchronize()
    assert rel_err(f64(o8), f64(o16)) <= TOL_FP8
    assert float(torch.max(torch.abs(l8 - l16))) <= 1e-2


# lengths 0 (o = 0, lse = -inf), 1, a ragged 33 and one above max_seq_len
# (clamped to it) in one batch; with 3 splits some splits are empty
EDGE_CASES = [("v3_b32_s4096", 128, 1), ("v3_b32_s4096", 128, 3), ("v3_b64_s32768_fp8", 128, 1),
              ("v3_b64_s32768_fp8", 128, 3), ("v3_b32_s4096", 16, 2), ("v3_b64_s32768_fp8", 32, 1)]


@pytest.mark.parametrize("workload,H,P", EDGE_CASES)
def test_decode_lengths_zero_one_ragged_and_clamped(workload, H, P):
    S = 100
    announce(f"decode lengths 0/1/33/clamped {workload} H={H} P={P}")
    x = _inputs(workload, batch=4, seq_len=S, heads=H)
    lens = torch.tensor([0, 1, 33, S + 100], dtype=torch.int32, device=DEV)
    d = binding.dims(4, H, x.scale)
    q_lat = datagen.random_latent_queries(4, H, seed=7, device=DEV)
    cache = _cache(x)
    if P == 1:
        o_lat, lse = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, lens, S, 1)
    else:
        o_part, lse_part = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, lens, S, P)
        o_lat, lse = binding.mla_combine_splits(d, o_part, lse_part)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=np.array([0, 1, 33, S]), scale=x.scale,
                                        **cache_args(x))
    got, gl = f64(o_lat), lse.cpu().numpy()
    assert np.all(got[0] == 0) and np.isneginf(gl[0]).all()
    for b in (1, 2, 3):
        assert rel_err(got[b], ref_o[b]) <= tol_for(x), b
        assert np.max(np.abs(gl[b] - ref_l[b])) <= tol_for(x), b
