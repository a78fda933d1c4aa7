"""The E4M3 decode paths through the C ABI against a bf16 cache holding the
same values (code * scale, exact in bf16 when the token scales are powers of
two).

32 and 64 heads: the codes are widened to bf16 exactly, the token scale
multiplies the fp32 score, and the probability that multiplies the codes in
P.V carries the scale; with power-of-two scales every one of these products
is exact, so the E4M3 cache gives bit-identical o_lat / lse (or partials) to
the bf16 cache, with and without splits, contiguous and paged, and in
prefill.

16 heads: the same holds for the E4M3 path, but a bf16 cache runs the
kernel whose two computing waves split each tile by tokens (another
summation order), so both results are checked against the oracle at the
bf16 bar and against each other.

128 heads: the stored codes go to fp8 MFMAs and the P.V weights are E4M3
with a power-of-two scale per (head, 32 tokens), so o differs from the bf16
cache's by that rounding: checked against the oracle and against the bf16
cache's result at the E4M3 bar (6e-2); lse keeps the exact sum (within 1e-3
of the bf16 cache's).
Parity of every E4M3 path with the float64 oracle at general scales is
covered by the E4M3 cases of test_parity_gpu.py, test_rescale_gpu.py and
test_prefill_gpu.py."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, TOL_FP8, cache_args, f64, rel_err

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
    assert torch.isfinite(r8[0].float()).all()
    if H == 16:
        _check_two_orders(x, d, q_lat, r8, r16, P)
        return
    if H < 128:
        assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1])
        return
    _check_fp8_mfma(x, d, q_lat, r8, r16, P)


def _check_two_orders(x, d, q_lat, r8, r16, P):
    """16 heads: E4M3 (codes widened exactly) and bf16 (token-split kernel)
    both at the bf16 bar of the oracle, and within it of each other."""
    if P > 1:
        o8, l8 = binding.mla_combine_splits(d, *r8)
        o16, l16 = binding.mla_combine_splits(d, *r16)
    else:
        (o8, l8), (o16, l16) = r8, r16
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale,
                                        **cache_args(x))
    e8, e16 = rel_err(f64(o8), ref_o), rel_err(f64(o16), ref_o)
    el8 = float(np.max(np.abs(l8.cpu().numpy() - ref_l)))
    el16 = float(np.max(np.abs(l16.cpu().numpy() - ref_l)))
    e_b = rel_err(f64(o8), f64(o16))
    print(f"  vs oracle: E4M3 o_lat {e8:.2e} lse {el8:.2e}, bf16 o_lat {e16:.2e} lse {el16:.2e}; "
          f"between them {e_b:.2e}")
    assert max(e8, e16, e_b) <= TOL_BF16 and max(el8, el16) <= 1e-4


def _check_fp8_mfma(x, d, q_lat, r8, r16, P):
    """128 heads: oracle parity at the E4M3 bar, and close to the bf16 cache."""
    if P > 1:
        o8, l8 = binding.mla_combine_splits(d, *r8)
        o16, l16 = binding.mla_combine_splits(d, *r16)
    else:
        (o8, l8), (o16, l16) = r8, r16
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale,
                                        **cache_args(x))
    e_o, e_l = rel_err(f64(o8), ref_o), float(np.max(np.abs(l8.cpu().numpy() - ref_l)))
    e_b = rel_err(f64(o8), f64(o16))
    e_bl = float(torch.max(torch.abs(l8 - l16)))
    print(f"  vs oracle: o_lat {e_o:.2e} lse {e_l:.2e}; vs bf16 cache: o_lat {e_b:.2e} lse {e_bl:.2e}")
    assert e_o <= TOL_FP8 and e_l <= TOL_FP8
    assert e_b <= TOL_FP8 and e_bl <= 1e-3


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
    if H < 128:
        assert torch.equal(r8[0], r16[0]) and torch.equal(r8[1], r16[1])
    else:
        # empty split ranges are o = 0, lse = -inf in both
        l8, l16 = r8[1].cpu().numpy(), r16[1].cpu().numpy()
        assert np.array_equal(np.isneginf(l8), np.isneginf(l16))
        fin = np.isfinite(l16)
        assert rel_err(f64(r8[0]), f64(r16[0])) <= TOL_FP8
        assert float(np.max(np.abs(l8[fin] - l16[fin]))) <= 1e-3
