"""mla_combine_expand_v (split merge + W_UV in one launch) through the C ABI:
bit for bit the result of mla_combine_splits followed by mla_expand_v, and
within the bf16 bar of the float64 oracle's combine_splits + expand_v."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, assert_guards, f64, guarded, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _weights(H, seed):
    x = datagen.make_inputs("v3_b32_s4096", device=DEV, batch=1, seq_len=32, heads=H)
    return x.w_uv


# batch sizes around the 16- and 32-sequence workgroups (ragged groups; 32
# sequences per workgroup once batch x heads >= 8,192: the last three), split
# counts up to past 64 (the lse re-read path), 16 .. 128 heads
CASES = [(2, 3, 16), (32, 8, 128), (17, 8, 64), (1, 1, 64), (3, 16, 32), (5, 70, 16), (1, 130, 32), (40, 9, 128),
         (64, 4, 128), (70, 5, 128), (100, 3, 128)]


@pytest.mark.parametrize("B,P,H", CASES)
def test_combine_expand_matches_two_calls_and_oracle(B, P, H):
    announce(f"combine_expand random partials B={B} P={P} H={H}")
    o_part, lse_part = datagen.random_partials(B, P, H, seed=71 + P + B, device=DEV)
    w_uv = _weights(H, seed=5)
    d = binding.dims(B, H, 0.07)
    o_ref, l_ref = binding.mla_combine_splits(d, o_part, lse_part)
    out_ref = binding.mla_expand_v(d, o_ref, w_uv)
    gout, go, gl, gout2 = guarded(DEV, ((B, H, 128), torch.bfloat16), ((B, H, 512), torch.bfloat16),
                                  ((B, H), torch.float32), ((B, H, 128), torch.bfloat16))
    o_lat, lse = go.tensor, gl.tensor
    out = binding.mla_combine_expand_v(d, o_part, lse_part, w_uv, out=gout.tensor, o_lat=o_lat, lse=lse)
    out_nolat = binding.mla_combine_expand_v(d, o_part, lse_part, w_uv, out=gout2.tensor)
    torch.cuda.synchronize()
    assert_guards(gout, go, gl, gout2)
    assert torch.equal(out, out_ref) and torch.equal(out_nolat, out_ref)
    assert torch.equal(o_lat, o_ref)
    assert torch.equal(lse, l_ref)
    # the oracle: merge every (b, h) row from the stored partials, then W_UV
    op, lp = o_part.cpu().double().numpy(), lse_part.cpu().double().numpy()
    ro = np.stack([oracle.combine_splits(op[b], lp[b])[0] for b in range(B)])
    ref_out = oracle.expand_v(ro, f64(w_uv))
    assert rel_err(f64(out), ref_out) <= TOL_BF16
    assert rel_err(f64(o_lat), ro) <= TOL_BF16


def test_combine_expand_empty_rows():
    """A (sequence, head) row whose splits are all empty has zero weight
    everywhere: o_lat = 0, lse = -inf, out = 0 (no NaN)."""
    B, P, H = 18, 4, 32
    announce(f"combine_expand empty rows B={B} P={P} H={H}")
    o_part, lse_part = datagen.random_partials(B, P, H, seed=5, device=DEV)
    lse_part[3] = -float("inf")
    o_part[3] = 0
    lse_part[17, :, 5] = -float("inf")
    o_part[17, :, 5] = 0
    w_uv = _weights(H, seed=6)
    d = binding.dims(B, H, 0.07)
    o_lat = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    out = binding.mla_combine_expand_v(d, o_part, lse_part, w_uv, o_lat=o_lat, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(o_lat).all()
    assert (out[3] == 0).all() and (o_lat[3] == 0).all() and torch.isneginf(lse[3]).all()
    assert (out[17, 5] == 0).all() and (o_lat[17, 5] == 0).all() and torch.isneginf(lse[17, 5])
    assert torch.isfinite(lse[17, :5]).all() and torch.isfinite(lse[16]).all()


def test_decode_step_split_matches_four_calls():
    """The V3 decode step with 8 splits (absorb_q, decode_latent,
    combine_expand_v) equals the four-call step bit for bit."""
    announce("decode step v3_b32_s4096 P=8: fused merge vs four calls")
    x = datagen.make_inputs("v3_b32_s4096", device=DEV)
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, 8, DEV)
    out = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv).clone()
    o_lat, lse = step.o_lat.clone(), step.lse.clone()
    q_lat = binding.mla_absorb_q(d, x.q_nope, x.w_uk)
    o_part, lse_part = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, 8)
    o2, l2 = binding.mla_combine_splits(d, o_part, lse_part)
    out2 = binding.mla_expand_v(d, o2, x.w_uv)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(o_lat, o2) and torch.equal(lse, l2)
