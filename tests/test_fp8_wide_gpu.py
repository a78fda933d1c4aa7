"""The 128-head E4M3 decode (each wave decodes its rows of every raw tile,
code times token scale in fp32 rounded to bf16, into the bf16 tile ring)
through the C ABI: bit for bit the result of the same kernel on a bf16 cache
that holds those decoded values, computed here by torch with the same fp32
arithmetic.  Parity of the E4M3 path with the float64 oracle is covered by
the E4M3 workloads of test_parity_gpu.py and test_prefill_gpu.py."""
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
    return datagen.make_inputs(wl, device=DEV, **kw)


def _caches(x):
    """(E4M3 cache, bf16 cache of the decoded values) over the same slots."""
    c8 = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                            block_size=x.block_size, token_scale=x.token_scale)
    sc = x.token_scale[:, None]
    kv16 = (x.kv_rows.view(torch.float8_e4m3fn).float() * sc).to(torch.bfloat16).contiguous()
    pe16 = (x.pe_rows.view(torch.float8_e4m3fn).float() * sc).to(torch.bfloat16).contiguous()
    c16 = binding.make_cache(kv16, pe16, seq_stride=x.seq_stride, block_table=x.block_table,
                             block_size=x.block_size)
    return c8, c16, (kv16, pe16)


# (workload, B, T, P): ragged tails, one and two tiles per split, empty
# splits of short sequences in the paged pool
CASES = [
    ("v3_b64_s32768_fp8", 3, 700, 1),
    ("v3_b64_s32768_fp8", 3, 1000, 4),
    ("v3_b64_s32768_fp8", 2, 33, 1),
    ("v3_b64_s32768_fp8", 2, 5, 1),
    ("v3_b64_s32768_fp8", 2, 2048, 8),
    ("v3_b128_paged_fp8", 4, 1500, 8),
    ("v3_b128_paged_fp8", 3, 300, 1),
]


@pytest.mark.parametrize("workload,B,T,P", CASES)
def test_fp8_decode_equals_bf16_decode_of_decoded_cache(workload, B, T, P):
    announce(f"wide E4M3 decode vs bf16 of decoded values {workload} B={B} T={T} P={P}")
    x = _inputs(workload, batch=B, seq_len=T, heads=128)
    d = binding.dims(B, 128, x.scale)
    q_lat = datagen.random_latent_queries(B, 128, seed=90 + P, device=DEV)
    c8, c16, keep = _caches(x)
    r8 = binding.mla_decode_latent(d, c8, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
    r16 = binding.mla_decode_latent(d, c16, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
    torch.cuda.synchronize()
    assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1])
    assert torch.isfinite(r8[0].float()).all()


def test_fp8_prefill_equals_bf16_prefill_of_decoded_cache():
    B, L, T = 2, 5, 300
    announce(f"wide E4M3 prefill vs bf16 of decoded values B={B} L={L} T={T}")
    x = _inputs("v3_b64_s32768_fp8", batch=B, seq_len=T, heads=128)
    d = binding.dims(B, 128, x.scale)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    q_lat = torch.randn((B, L, 128, 512), generator=gen, device=DEV).to(torch.bfloat16)
    q_pe = torch.randn((B, L, 128, 64), generator=gen, device=DEV).to(torch.bfloat16)
    q_start = torch.tensor([T - L, T - L - 40], dtype=torch.int32, device=DEV)
    c8, c16, keep = _caches(x)
    for P in (1, 3):
        r8 = binding.mla_prefill_latent(d, c8, q_lat, q_pe, q_start, T, num_splits=P)
        r16 = binding.mla_prefill_latent(d, c16, q_lat, q_pe, q_start, T, num_splits=P)
        torch.cuda.synchronize()
        assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1]), P
