"""The 128-head E4M3 decode with token scales that are zero, tiny, or far
below their neighbours', against the float64 oracle.

Such a token's stored values (code * scale) are zero or nearly so, but its
score is not, so its probability p belongs in the softmax sum while its row
adds (almost) nothing to o.  The kernel normalises o by the sum of the E4M3
weights as stored, each over its token scale; a token whose scale is 0 or
below 2^-6 of the largest of its 32 counts at its exact p instead (its weight
may round to zero).  Dropping these tokens from the sum would scale o up by
the share of their probability mass (here ~1/4), far outside the E4M3 bar,
so these cases pin that rule.  Scales at 2^-5 of the largest stay on the
stored-weight side of it."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_FP8, cache_args, f64, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _plant_scales(x):
    """Zero, tiny and reduced token scales at a fixed pattern of slots (the
    codes stay as generated).  Returns the number of planted slots."""
    sc = x.token_scale
    n = sc.numel()
    idx = torch.arange(n, device=DEV)
    zero = idx % 7 == 3
    tiny = idx % 11 == 5
    low = (idx % 13 == 1) & ~zero & ~tiny          # below 2^-6 of the others
    mid = (idx % 17 == 2) & ~zero & ~tiny & ~low   # 2^-5: above the threshold
    sc[zero] = 0.0
    sc[tiny] = 1e-30
    sc[low] = sc[low] * 2.0 ** -9
    sc[mid] = sc[mid] * 2.0 ** -5
    return int((zero | tiny | low | mid).sum())


# (workload, B, T, P)
CASES = [
    ("v3_b64_s32768_fp8", 2, 700, 1),
    ("v3_b64_s32768_fp8", 3, 1000, 3),
    ("v3_b128_paged", 3, 900, 4),
]


@pytest.mark.parametrize("workload,B,T,P", CASES)
def test_fp8_zero_and_tiny_token_scales(workload, B, T, P):
    announce(f"E4M3 128 heads, zero / tiny / reduced token scales {workload} B={B} T={T} P={P}")
    wl = datagen.WORKLOADS[workload]
    if wl.dtype != "fp8_e4m3":
        import dataclasses
        wl = dataclasses.replace(wl, name=wl.name + "_fp8", dtype="fp8_e4m3", seed=wl.seed + 11)
    x = datagen.make_inputs(wl, batch=B, seq_len=T, heads=128, device=DEV)
    planted = _plant_scales(x)
    assert planted > 0
    d = binding.dims(B, 128, x.scale)
    q_lat = datagen.random_latent_queries(B, 128, seed=31 + P, device=DEV)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                               block_size=x.block_size, token_scale=x.token_scale)
    r = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
    o, lse = binding.mla_combine_splits(d, *r) if P > 1 else r
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.latent_decode(f64(q_lat), f64(x.q_pe), seq_lens=x.seq_lens.cpu().numpy(), scale=x.scale,
                                        **cache_args(x))
    e_o = rel_err(f64(o), ref_o)
    e_l = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
    print(f"  planted {planted} slots; vs oracle: o_lat {e_o:.2e} lse {e_l:.2e}")
    assert e_o <= TOL_FP8 and e_l <= 1e-3
