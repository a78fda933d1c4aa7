"""Parity of mla_naive_decode (expand every step, then multi-head attention)
with the oracle's expanded form (naive_decode), element by element:
max |gpu - oracle| / max |oracle| <= 2e-2 (6e-2 with an E4M3 cache); and
agreement with the absorbed four-call path on the same inputs."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, TOL_FP8, cache_args, f64, rel_err, sample_batch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _cache(x):
    return binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                              block_size=x.block_size, token_scale=x.token_scale)


@pytest.mark.parametrize("workload,B,T,H", [
    ("v2lite_b1_s26", None, None, None),      # 26 tokens: one partial 128-token tile
    ("v2lite_b64_s4096", 3, 300, None),       # several tiles and a ragged tail
    ("v3_b32_s4096", 2, 257, 128),
    ("v3_b128_paged", 3, 400, 32),            # paged, varying lengths
    ("v3_b64_s32768_fp8", 2, 200, 16),        # E4M3 cache
])
def test_naive_decode_against_oracle(workload, B, T, H):
    announce(f"naive decode {workload} B={B} T={T} H={H}")
    kw = {k: v for k, v in (("batch", B), ("seq_len", T), ("heads", H)) if v is not None}
    x = datagen.make_inputs(datagen.WORKLOADS[workload], device=DEV, **kw)
    d = binding.dims(x.batch, x.heads, x.scale)
    out = binding.mla_naive_decode(d, _cache(x), x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, x.max_seq_len)
    torch.cuda.synchronize()
    ref = oracle.naive_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                              seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale, **cache_args(x))
    tol = TOL_FP8 if x.workload.dtype == "fp8_e4m3" else TOL_BF16
    e = rel_err(f64(out), ref)
    print(f"  out {e:.2e}")
    assert np.isfinite(f64(out)).all() and e <= tol


def test_naive_matches_absorbed_full_size_sampled():
    """At the V2-Lite B=64 S=4096 workload (the expansion writes 2.1 GB), the
    naive and absorbed paths agree; sampled sequences also match the oracle."""
    announce("naive vs absorbed, v2lite_b64_s4096 full size")
    x = datagen.make_inputs(datagen.WORKLOADS["v2lite_b64_s4096"], device=DEV)
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = _cache(x)
    naive = binding.mla_naive_decode(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, x.max_seq_len)
    P = binding.mla_recommended_splits(d, x.max_seq_len, torch.cuda.get_device_properties(DEV).multi_processor_count)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, P, DEV)
    absorbed = step(x.q_nope, x.q_pe, x.w_uk, x.w_uv)
    torch.cuda.synchronize()
    assert rel_err(f64(naive), f64(absorbed)) <= TOL_BF16
    idx = sample_batch(x.batch, 3)
    ref = oracle.naive_decode(f64(x.q_nope), f64(x.q_pe), f64(x.w_uk), f64(x.w_uv),
                              seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale, batch_indices=idx, **cache_args(x))
    assert rel_err(f64(naive)[idx], ref) <= TOL_BF16


def test_naive_single_token():
    """One cached token: softmax weight 1, out = W_UV c_0 (up to bf16 rounding
    of the expanded row and of out)."""
    announce("naive T=1")
    x = datagen.make_inputs(datagen.WORKLOADS["v3_b32_s4096"], device=DEV, batch=2, seq_len=1, heads=16)
    d = binding.dims(2, 16, x.scale)
    out = binding.mla_naive_decode(d, _cache(x), x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, 1)
    torch.cuda.synchronize()
    for b in range(2):
        want = np.einsum("hjc,c->hj", f64(x.w_uv), f64(x.kv_rows[b * x.seq_stride]))
        assert rel_err(f64(out[b]), want) <= 1e-2
