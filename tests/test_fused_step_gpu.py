"""Parity of mla_decode_step_fused (the three decode stages in one launch)
with the float64 oracle, element by element on the same seeded inputs:
max |gpu - oracle| / max |oracle| <= 2e-2 for out and o_lat (6e-2 with an
E4M3 cache), lse within the same bound in natural-log units."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, TOL_FP8, assert_guards, cache_args, f64, guarded, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _run(x, check_all=True):
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                               block_size=x.block_size, token_scale=x.token_scale)
    B, H = x.batch, x.heads
    gout, go, gl = guarded(DEV, ((B, H, 128), torch.bfloat16), ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    out, o_lat, lse = binding.mla_decode_step_fused(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens,
                                                    x.max_seq_len, out=gout.tensor, o_lat=go.tensor, lse=gl.tensor,
                                                    want_latent=True)
    torch.cuda.synchronize()
    assert_guards(gout, go, gl)
    ref = oracle.absorbed_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                                 seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale, **cache_args(x))
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    e_out = rel_err(f64(out), ref["out"])
    e_lat = rel_err(f64(o_lat), ref["o_lat"])
    e_lse = float(np.max(np.abs(lse.cpu().numpy() - ref["lse"])))
    print(f"  out {e_out:.2e} o_lat {e_lat:.2e} lse {e_lse:.2e}")
    assert np.isfinite(f64(out)).all()
    assert max(e_out, e_lat, e_lse) <= tol
    return out


@pytest.mark.parametrize("workload,B,T,H", [
    ("v2lite_b1_s26", None, None, None),      # the 26-token V2-Lite step, as drawn
    ("v2lite_b64_s4096", 3, 37, None),        # ragged: 37 tokens, not a multiple of 16
    ("v3_b32_s4096", 2, 300, 128),
    ("v3_b128_paged", 2, None, 32),           # paged, lengths drawn from the workload
    ("v3_b64_s32768_fp8", 2, 150, 64),        # E4M3 cache
])
def test_fused_step_against_oracle(workload, B, T, H):
    announce(f"fused step {workload} B={B} T={T} H={H}")
    kw = {}
    if B is not None:
        kw["batch"] = B
    if T is not None:
        kw["seq_len"] = T
    if H is not None:
        kw["heads"] = H
    if workload == "v3_b128_paged" and T is None:
        kw["seq_len"] = 200  # upper end of the drawn lengths, kept short for this path
    _run(datagen.make_inputs(datagen.WORKLOADS[workload], device=DEV, **kw))


def test_fused_step_matches_four_call_path():
    """The fused step and the four-call step agree to bf16 rounding of their
    intermediates on the 26-token workload."""
    announce("fused vs four calls, v2lite_b1_s26")
    x = datagen.make_inputs(datagen.WORKLOADS["v2lite_b1_s26"], device=DEV)
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, 1, DEV)
    four = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv).clone()
    fused = binding.mla_decode_step_fused(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, x.max_seq_len)
    torch.cuda.synchronize()
    assert rel_err(f64(fused), f64(four)) <= 1e-2


def test_fused_step_special_lengths():
    """Length 1 (o_lat is that row), length 0 (o = 0, lse = -inf, out = 0) and
    lengths above max_seq_len (clamped) in one batch."""
    announce("fused step lengths 1 / 0 / clamped")
    x = datagen.make_inputs(datagen.WORKLOADS["v3_b32_s4096"], device=DEV, batch=3, seq_len=40, heads=16)
    lens = torch.tensor([1, 0, 40], dtype=torch.int32, device=DEV)
    d = binding.dims(3, 16, x.scale)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride)
    out, o_lat, lse = binding.mla_decode_step_fused(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, lens, 33,
                                                    want_latent=True)
    torch.cuda.synchronize()
    row0 = f64(x.kv_rows[0])
    assert np.array_equal(f64(o_lat[0]), np.broadcast_to(row0, (16, 512)))
    assert torch.all(o_lat[1] == 0) and torch.all(out[1] == 0) and torch.all(torch.isinf(lse[1]))
    ref = oracle.absorbed_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                                 seq_lens=np.array([1, 0, 33]), scale=x.scale, batch_indices=[0, 2],
                                 **cache_args(x))
    assert rel_err(f64(out)[[0, 2]], ref["out"]) <= TOL_BF16
    assert rel_err(f64(o_lat)[[2]], ref["o_lat"][1:]) <= TOL_BF16
