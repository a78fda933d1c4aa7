"""mla_decode_latent_noalloc, the entry point for callers that cannot
allocate (split partials in the library's per-GPU device array), through the
C ABI: bit for bit the result of mla_decode_latent with caller-provided
partials followed by mla_combine_splits, on two calls in a row (the second
with a smaller batch, fewer splits and shorter contexts, so the array holds
the first call's larger contents when it starts), and on the E4M3 and paged
layouts.  Sizes beyond the array are rejected before anything is launched."""
import numpy as np
import pytest
import torch

import oracle
from mla_absorbed_latent_absorb_amd import binding, datagen
from tests.gpu_helpers import TOL_BF16, assert_guards, cache_args, f64, guarded, rel_err

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _cache(x):
    return binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                              block_size=x.block_size, token_scale=x.token_scale)


def _both(workload, B, T, H, P, seed):
    x = datagen.make_inputs(datagen.WORKLOADS[workload], device=DEV, batch=B, seq_len=T, heads=H)
    q_lat = datagen.random_latent_queries(B, H, seed, device=DEV)
    d = binding.dims(B, H, x.scale)
    cache = _cache(x)
    go, gl = guarded(DEV, ((B, H, 512), torch.bfloat16), ((B, H), torch.float32))
    binding.mla_decode_latent_noalloc(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P, go.tensor, gl.tensor)
    if P > 1:
        o_part, lse_part = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, P)
        ref_o, ref_l = binding.mla_combine_splits(d, o_part, lse_part)
    else:
        ref_o, ref_l = binding.mla_decode_latent(d, cache, q_lat, x.q_pe, x.seq_lens, x.max_seq_len, 1)
    torch.cuda.synchronize()
    assert_guards(go, gl)
    return x, q_lat, go.tensor, gl.tensor, ref_o, ref_l


def test_noalloc_two_calls_second_smaller():
    announce("noalloc: V3 B=32 T=4096 P=8, then B=3 T=700 P=3")
    x, q_lat, o1, l1, r1, rl1 = _both("v3_b32_s4096", 32, 4096, 128, 8, 11)
    assert torch.equal(o1, r1) and torch.equal(l1, rl1)
    x2, q2, o2, l2, r2, rl2 = _both("v3_b32_s4096", 3, 700, 128, 3, 12)
    assert torch.equal(o2, r2) and torch.equal(l2, rl2)
    # and within the parity bar of the oracle
    ref_o, ref_l = oracle.latent_decode(f64(q2), f64(x2.q_pe), seq_lens=x2.seq_lens.cpu().numpy(), scale=x2.scale,
                                        **cache_args(x2))
    assert rel_err(f64(o2), ref_o) <= TOL_BF16
    assert np.max(np.abs(l2.cpu().numpy() - ref_l)) <= TOL_BF16


@pytest.mark.parametrize("workload,B,T,H,P", [("v3_b64_s32768_fp8", 4, 1000, 128, 4), ("v3_b128_paged", 5, 2000, 128, 2),
                                              ("v2lite_b64_s4096", 6, 900, 16, 16), ("v3_b32_s4096", 2, 300, 64, 1)])
def test_noalloc_layouts(workload, B, T, H, P):
    announce(f"noalloc: {workload} B={B} T={T} H={H} P={P}")
    *_, o, l, r, rl = _both(workload, B, T, H, P, 13)
    assert torch.equal(o, r) and torch.equal(l, rl)


def test_noalloc_rejects_more_partials_than_the_scratch_holds():
    announce("noalloc: oversize request rejected on the host")
    B, H, T = 256, 128, 64
    x = datagen.make_inputs(datagen.WORKLOADS["v3_b32_s4096"], device=DEV, batch=B, seq_len=T, heads=H)
    d = binding.dims(B, H, x.scale)
    o = torch.empty((B, H, 512), dtype=torch.bfloat16, device=DEV)
    l = torch.empty((B, H), dtype=torch.float32, device=DEV)
    q_lat = datagen.random_latent_queries(B, H, 3, device=DEV)
    with pytest.raises(binding.MlaError) as e:
        binding.mla_decode_latent_noalloc(d, _cache(x), q_lat, x.q_pe, x.seq_lens, T, 2, o, l)
    assert e.value.status == 5 and "scratch" in e.value.message
