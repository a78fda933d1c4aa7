"""The E4M3 decode paths through the C ABI: the codes are widened to bf16
exactly, the per-token scale multiplies the fp32 score, and the probability
that multiplies the codes in P.V carries the scale.  With power-of-two token
scales every one of these products is exact, so an E4M3 cache must give
bit-identical o_lat / lse (or partials) to a bf16 cache holding code * scale
(exact in bf16) -- for the 128-head kernel and the 16/32/64-head kernel, with
and without splits, contiguous and paged, and in prefill.  Parity of the E4M3
path with the float64 oracle at general scales is covered by the E4M3 cases
of test_parity_gpu.py, test_rescale_gpu.py and test_prefill_gpu.py."""
import dataclasses

import pytest
import torch

from mla_absorbed_latent_absorb_amd import binding, datagen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FP8_PAGED = dataclasses.replace(datagen.WORKLOADS["v3_b128_paged"], name="v3_b128_paged_fp8", dtype="fp8_e4m3",
                                seed=20266)


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _inputs(workload, **kw):
    wl = FP8_PAGED if workload == FP8_PAGED.name else workload
    x = datagen.make_inputs(wl, device=DEV, **kw)
    # power-of-two token scales (the codes are unchanged)
    x.token_scale.copy_(torch.exp2(torch.round(torch.log2(x.token_scale))))
    return x


def _caches(x):
    """(E4M3 cache, bf16 cache of code * scale, exact) over the same slots."""
    c8 = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                            block_size=x.block_size, token_scale=x.token_scale)
    sc = x.token_scale[:, None]
    kv16 = (x.kv_rows.view(torch.float8_e4m3fn).float() * sc).to(torch.bfloat16).contiguous()
    pe16 = (x.pe_rows.view(torch.float8_e4m3fn).float() * sc).to(torch.bfloat16).contiguous()
    assert torch.equal(kv16.float(), x.kv_rows.view(torch.float8_e4m3fn).float() * sc)
    c16 = binding.make_cache(kv16, pe16, seq_stride=x.seq_stride, block_table=x.block_table,
                             block_size=x.block_size)
    return c8, c16, (kv16, pe16)


# (workload, H, B, T, P): ragged tails, one and two tiles per split, empty
# splits of short sequences in the paged pool, every head count
CASES = [
    ("v3_b64_s32768_fp8", 128, 3, 700, 1),
    ("v3_b64_s32768_fp8", 128, 3, 1000, 4),
    ("v3_b64_s32768_fp8", 128, 2, 33, 1),
    ("v3_b64_s32768_fp8", 128, 2, 5, 1),
    ("v3_b64_s32768_fp8", 128, 2, 2048, 8),
    ("v3_b128_paged_fp8", 128, 4, 1500, 8),
    ("v3_b128_paged_fp8", 128, 3, 300, 1),
    ("v3_b64_s32768_fp8", 64, 3, 700, 1),
    ("v3_b64_s32768_fp8", 32, 3, 333, 3),
    ("v3_b64_s32768_fp8", 16, 2, 97, 1),
    ("v3_b128_paged_fp8", 16, 3, 900, 4),
]


@pytest.mark.parametrize("workload,H,B,T,P", CASES)
def test_fp8_pow2_scales_equal_bf16_cache(workload, H, B, T, P):
    announce(f"E4M3 (power-of-two scales) vs bf16 of code*scale {workload} H={H} B={B} T={T} P={P}")
    x = _inputs(workload, batch=B, seq_len=T, heads=H)
    d = binding.dims(B, H, x.scale)
    q_lat = datagen.random_latent_queries(B, H, seed=90 + P, device=DEV)
    c8, c16, keep = _caches(x)
    r8 = binding.mla_decode_latent(d, c8, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
    r16 = binding.mla_decode_latent(d, c16, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
    torch.cuda.synchronize()
    assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1])
    assert torch.isfinite(r8[0].float()).all()


# (H, P): with fewer than 128 heads and one split, a bf16 prefill groups
# 128 / H queries per workgroup of the 128-row kernel while an E4M3 prefill
# runs one query per workgroup, so the two sum in different orders; with
# splits both take the same kernel
@pytest.mark.parametrize("H,P", [(128, 1), (128, 3), (32, 3)])
def test_fp8_pow2_prefill_equals_bf16_cache(H, P):
    B, L, T = 2, 5, 300
    announce(f"E4M3 prefill (power-of-two scales) vs bf16 of code*scale H={H} P={P} B={B} L={L} T={T}")
    x = _inputs("v3_b64_s32768_fp8", batch=B, seq_len=T, heads=H)
    d = binding.dims(B, H, x.scale)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    q_lat = torch.randn((B, L, H, 512), generator=gen, device=DEV).to(torch.bfloat16)
    q_pe = torch.randn((B, L, H, 64), generator=gen, device=DEV).to(torch.bfloat16)
    q_start = torch.tensor([T - L, T - L - 40], dtype=torch.int32, device=DEV)
    c8, c16, keep = _caches(x)
    r8 = binding.mla_prefill_latent(d, c8, q_lat, q_pe, q_start, T, num_splits=P)
    r16 = binding.mla_prefill_latent(d, c16, q_lat, q_pe, q_start, T, num_splits=P)
    torch.cuda.synchronize()
    assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1])
