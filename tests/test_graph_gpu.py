"""The library's calls captured in a HIP graph: every replay (with eager work
and synchronisations in between) reproduces the eager results bit for bit.
The kernels record no memset or allocation, so a captured step is safe to
replay; this checks it."""
import pytest
import torch

from mla_absorbed_latent_absorb_amd import binding, datagen

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("workload,B,T,H,P", [("v3_b32_s4096", 3, 700, 128, 4), ("v2lite_b1_s26", None, None, None, 1),
                                              ("v3_b64_s32768_fp8", 2, 300, 128, 2)])
def test_graph_replays_match_eager(workload, B, T, H, P):
    announce(f"graph replay {workload} P={P}")
    kw = {k: v for k, v in (("batch", B), ("seq_len", T), ("heads", H)) if v is not None}
    x = datagen.make_inputs(datagen.WORKLOADS[workload], device=DEV, **kw)
    d = binding.dims(x.batch, x.heads, x.scale)
    cache = binding.make_cache(x.kv_rows, x.pe_rows, seq_stride=x.seq_stride, block_table=x.block_table,
                               block_size=x.block_size, token_scale=x.token_scale)
    step = binding.DecodeStep(d, cache, x.seq_lens, x.max_seq_len, P, DEV)
    fused_out = torch.empty_like(step.out)
    new_rows = datagen.random_projection_rows(x.batch, 1, 5, device=DEV)
    pos = (x.seq_lens - 1).to(torch.int32)

    def work():
        step(x.q_nope, x.q_pe, x.w_uk, x.w_uv)
        binding.mla_decode_step_fused(d, cache, x.q_nope, x.q_pe, x.w_uk, x.w_uv, x.seq_lens, x.max_seq_len,
                                      out=fused_out)
        binding.mla_cache_append(d, cache, new_rows, pos)

    work()
    work()  # the append rewrote the last row; a second pass sees the final cache
    torch.cuda.synchronize()
    eager = [t.clone() for t in (step.q_lat, step.o_lat, step.lse, step.out, fused_out, x.kv_rows, x.pe_rows)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for r in range(3):
        for t in (step.q_lat, step.o_lat, step.out, fused_out):
            t.fill_(0)
        step.lse.fill_(0.0)
        # unrelated eager work between replays
        torch.randn(1 << 20, device=DEV).sum().item()
        g.replay()
        torch.cuda.synchronize()
        got = (step.q_lat, step.o_lat, step.lse, step.out, fused_out, x.kv_rows, x.pe_rows)
        for i, (a, b) in enumerate(zip(eager, got)):
            assert torch.equal(a, b), (r, i)
