"""Parity of mla_prefill_latent (absorbed chunked prefill: each query of a
chunk attends causally to the cached rows up to its own position) with the
oracle, element by element: for every query row, the oracle's
latent_attention over that query's causal prefix; max |gpu - oracle| /
max |oracle| <= 2e-2 (6e-2 with an E4M3 cache), lse within the same bound.
An end-to-end case runs append (key RoPE), absorb, prefill and expand on a
fresh sequence and compares with the oracle's one-shot causal forward."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, TOL_FP8, assert_guards, bits16, cache_args, f64, guarded, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _cache(x):
    return binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                              block_size=x.block_size, token_scale=x.token_scale)


def _queries(B, L, H, seed):
    q_lat = datagen.random_latent_queries(B * L, H, seed, device=DEV).view(B, L, H, 512)
    q_pe = datagen.random_latent_queries(B * L, H, seed + 1, device=DEV)[..., :64].contiguous().view(B, L, H, 64)
    return q_lat, q_pe


def _oracle_rows(x, q_lat, q_pe, q_start, max_len, rows):
    """Oracle o_lat / lse for the query rows (b, i) listed."""
    args = cache_args(x)
    ql, qp = f64(q_lat), f64(q_pe)
    os_, ls_ = [], []
    for b, i in rows:
        T = min(int(q_start[b]) + i + 1, max_len)
        slots = oracle.token_slots(b, T, args["seq_stride"], args["block_table"], args["block_size"])
        c, k_r = oracle.load_rows(args["kv_codes"], args["pe_codes"], slots, args["dtype"], args["token_scale"])
        o, l = oracle.latent_attention(ql[b, i], qp[b, i], c, k_r, x.scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


@pytest.mark.parametrize("workload,B,S,H,L,starts,P", [
    ("v3_b32_s4096", 2, 300, 128, 37, [100, 0], 1),          # two chunks, one at the start of its sequence
    ("v2lite_b64_s4096", 3, 200, 16, 50, [150, 7, 64], 1),    # H=16, ragged
    ("v3_b128_paged", 2, 400, 32, 33, [300, 360], 1),         # paged cache
    ("v3_b64_s32768_fp8", 2, 160, 128, 20, [140, 31], 1),     # E4M3 cache
    ("v3_b32_s4096", 2, 700, 64, 9, [650, 200], 3),           # split-KV + merge over B*L rows
    ("v2lite_b64_s4096", 2, 300, 16, 21, [0, 250], 1),        # 8-query groups with a 5-query tail
    ("v3_b32_s4096", 3, 260, 32, 6, [100, 0, 254], 1),        # 4-query groups with a 2-query tail
    ("v3_b32_s4096", 2, 200, 64, 3, [190, 5], 1),             # 2-query groups with a 1-query tail
])
def test_prefill_against_oracle(workload, B, S, H, L, starts, P):
    announce(f"prefill {workload} B={B} S={S} H={H} L={L} starts={starts} P={P}")
    x = datagen.make_inputs(datagen.WORKLOADS[workload], device=DEV, batch=B, seq_len=S, heads=H)
    d = binding.dims(B, H, x.scale)
    q_lat, q_pe = _queries(B, L, H, 11)
    q_start = torch.tensor(starts, dtype=torch.int32, device=DEV)
    max_len = x.max_seq_len
    cache = _cache(x)
    if P == 1:
        go, gl = guarded(DEV, ((B, L, H, 512), torch.bfloat16), ((B, L, H), torch.float32))
        o_lat, lse = binding.mla_prefill_latent(d, cache, q_lat, q_pe, q_start, max_len, o_lat=go.tensor,
                                                lse=gl.tensor)
        gs = (go, gl)
    else:
        gp, glp = guarded(DEV, ((B * L, P, H, 512), torch.bfloat16), ((B * L, P, H), torch.float32))
        o_part, lse_part = binding.mla_prefill_latent(d, cache, q_lat, q_pe, q_start, max_len, num_splits=P,
                                                      o_part=gp.tensor, lse_part=glp.tensor)
        dr = binding.dims(B * L, H, x.scale)
        o_lat, lse = binding.mla_combine_splits(dr, o_part, lse_part)
        o_lat, lse = o_lat.view(B, L, H, 512), lse.view(B, L, H)
        gs = (gp, glp)
    torch.cuda.synchronize()
    assert_guards(*gs)
    rows = [(b, i) for b in range(B) for i in range(L)]
    ro, rl = _oracle_rows(x, q_lat, q_pe, starts, max_len, rows)
    got_o = f64(o_lat).reshape(B * L, H, 512)
    got_l = lse.cpu().numpy().reshape(B * L, H)
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    e_o, e_l = rel_err(got_o, ro), float(np.max(np.abs(got_l - rl)))
    print(f"  o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= tol and e_l <= tol


def test_prefill_last_row_equals_decode():
    """The chunk's last query attends exactly the prefix a decode step at
    length q_start + L attends: both launches give bit-identical rows."""
    announce("prefill last row == decode, H=128")
    B, S, H, L = 3, 500, 128, 16
    x = datagen.make_inputs(datagen.WORKLOADS["v3_b32_s4096"], device=DEV, batch=B, seq_len=S, heads=H)
    d = binding.dims(B, H, x.scale)
    q_lat, q_pe = _queries(B, L, H, 21)
    starts = torch.tensor([400, 0, 484], dtype=torch.int32, device=DEV)
    cache = _cache(x)
    o_lat, lse = binding.mla_prefill_latent(d, cache, q_lat, q_pe, starts, S)
    lens = (starts + L).to(torch.int32)
    o_dec, l_dec = binding.mla_decode_latent(d, cache, q_lat[:, L - 1].contiguous(), q_pe[:, L - 1].contiguous(),
                                             lens, S, 1)
    torch.cuda.synchronize()
    assert torch.equal(o_lat[:, L - 1], o_dec) and torch.equal(lse[:, L - 1], l_dec)


def _rotate_queries(q_pe_raw, positions, base):
    """Rotate q_pe rows [L, H, 64] at their token's position with the library's
    own RoPE (mla_cache_append on a scratch cache: one sequence per (i, h),
    its single new row at position positions[i])."""
    L, H, _ = q_pe_raw.shape
    rows = torch.zeros((L * H, 1, 576), dtype=torch.bfloat16, device=DEV)
    rows[:, 0, 512:] = q_pe_raw.reshape(L * H, 64)
    S = int(max(positions)) + 1
    store = torch.zeros((L * H * S, 576), dtype=torch.bfloat16, device=DEV)
    c = binding.make_cache(store[:, :512], store[:, 512:], seq_stride=S)
    pos = torch.tensor(np.repeat(np.asarray(positions), H), dtype=torch.int32, device=DEV)
    binding.mla_cache_append(binding.dims(L * H, 16, 0.07), c, rows, pos, rope_base=base)
    slots = torch.arange(L * H, device=DEV) * S + pos.to(torch.int64)
    return store[slots, 512:].reshape(L, H, 64).contiguous()


def test_prefill_end_to_end_vs_causal_forward():
    """A fresh 48-token sequence at the V2-Lite shape: append (keys rotated at
    their positions), absorb the chunk's queries, causal prefill, expand.
    Equals the oracle's one-shot causal forward with decoupled RoPE."""
    announce("prefill end to end vs causal forward, L=48 H=16")
    L, H, base = 48, 16, 10000.0
    x = datagen.make_inputs(datagen.WORKLOADS["v2lite_b1_s26"], device=DEV)
    rows = datagen.random_projection_rows(1, L, 71, device=DEV)          # c_t | k_R,t before rotation
    qn = datagen.random_latent_queries(L, H, 72, device=DEV)[..., :128].contiguous()
    qr_raw = datagen.random_latent_queries(L, H, 73, device=DEV)[..., :64].contiguous()
    store = torch.zeros((64, 576), dtype=torch.bfloat16, device=DEV)
    cache = binding.make_cache(store[:, :512], store[:, 512:], seq_stride=64)
    d1 = binding.dims(1, H, x.scale)
    binding.mla_cache_append(d1, cache, rows, torch.zeros(1, dtype=torch.int32, device=DEV), rope_base=base)
    qr = _rotate_queries(qr_raw, list(range(L)), base)
    dL = binding.dims(L, H, x.scale)
    q_lat = binding.mla_absorb_q(dL, qn, x.w_uk)
    o_lat, lse = binding.mla_prefill_latent(d1, cache, q_lat.view(1, L, H, 512), qr.view(1, L, H, 64),
                                            torch.zeros(1, dtype=torch.int32, device=DEV), 64)
    out = binding.mla_expand_v(dL, o_lat.view(L, H, 512).contiguous(), x.w_uv)
    torch.cuda.synchronize()
    r = f64(rows)[0]
    ref = oracle.causal_naive_forward(f64(qn), f64(qr_raw), r[:, :512], r[:, 512:], f64(x.w_uk), f64(x.w_uv),
                                      x.scale, rope_base=base)
    e = rel_err(f64(out), ref)
    print(f"  out {e:.2e}")
    assert e <= TOL_BF16


def test_prefill_full_size_sampled():
    """The last 256-query chunk of a 4096-token V3 sequence (B=2), in the
    launch configuration the bench times; sampled query rows vs the oracle."""
    announce("prefill full size, V3 B=2 S=4096 chunk 256")
    B, S, H, L = 2, 4096, 128, 256
    x = datagen.make_inputs(datagen.WORKLOADS["v3_b32_s4096"], device=DEV, batch=B, seq_len=S, heads=H)
    d = binding.dims(B, H, x.scale)
    q_lat, q_pe = _queries(B, L, H, 31)
    starts = [S - L, S - L]
    o_lat, lse = binding.mla_prefill_latent(d, _cache(x), q_lat, q_pe, torch.tensor(starts, dtype=torch.int32,
                                                                                      device=DEV), S)
    torch.cuda.synchronize()
    rows = [(0, 0), (0, 1), (0, 127), (0, 255), (1, 0), (1, 200), (1, 255)]
    ro, rl = _oracle_rows(x, q_lat, q_pe, starts, S, rows)
    got_o = np.stack([f64(o_lat[b, i]) for b, i in rows])
    got_l = np.stack([lse[b, i].cpu().numpy() for b, i in rows])
    assert rel_err(got_o, ro) <= TOL_BF16 and float(np.max(np.abs(got_l - rl))) <= TOL_BF16
