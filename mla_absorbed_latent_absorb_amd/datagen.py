"""Seeded synthetic inputs for absorbed-MLA decode.

This module only draws random numbers and stores them in the cache formats
(bfloat16, or OCP E4M3 with one float32 scale per token) and layouts
(contiguous or paged) the decode path reads.  It holds none of the attention
arithmetic, and both the HIP path and the float64 oracle consume its output:
the oracle decodes the stored bytes itself.

The source pages measured real DeepSeek-V2-Lite activations and weights,
which are not available here; these draws stand in for them with the shapes of
the DeepSeek-V2-Lite (H=16) and DeepSeek-V3 (H=128) attention layers:
kv_lora_rank 512, qk_rope_head_dim 64, qk_nope_head_dim 128, v_head_dim 128.

Recipe (per workload): one ``torch.Generator`` on the target device, seeded
with the workload's seed, draws in this order: sequence lengths (if they
vary), the physical block permutation (if paged), q_nope, q_pe, W_UK, W_UV,
then the cache rows: contiguous caches one [T_b, 576] draw per sequence,
paged caches one [num_blocks, block_size, 576] draw in physical block
order.  Draws are float32 N(0,1) scaled by the stated std, then rounded to
bfloat16 (round to nearest even).  For an E4M3 cache each token's 576 values
x_t get the scale s_t = max|x_t| / 448 (float32) and are stored as the E4M3
code of x_t / s_t (round to nearest even, clamped to +-448).
"""

from dataclasses import dataclass, field
import math
from typing import Optional

import torch

D_C = 512      # kv_lora_rank
D_R = 64       # qk_rope_head_dim
D_N = 128      # qk_nope_head_dim
D_V = 128      # v_head_dim
D_K = D_C + D_R

E4M3_MAX = 448.0


@dataclass
class Workload:
    """Shape and structure of one synthetic decode workload."""
    name: str
    batch: int
    heads: int
    seed: int
    dtype: str = "bf16"              # cache element type: "bf16" or "fp8_e4m3"
    seq_len: Optional[int] = None    # uniform context length
    len_range: Optional[tuple] = None  # (lo, hi) inclusive uniform lengths
    seq_capacity: Optional[int] = None  # token slots per sequence (contiguous)
    layout: str = "fused"            # "fused" [.,576], "separate" kv/pe, "paged"
    block_size: int = 64
    description: str = ""


WORKLOADS = {
    "v2lite_b1_s26": Workload(
        "v2lite_b1_s26", batch=1, heads=16, seed=20261, seq_len=26, seq_capacity=32,
        layout="separate",
        description="V2-Lite shape, 25-token prefill + 1-token decode (26 cached tokens) in a "
                    "32-slot buffer; W ~ N(0, 1/512); scale 1/sqrt(192)"),
    "v2lite_b64_s4096": Workload(
        "v2lite_b64_s4096", batch=64, heads=16, seed=20262, seq_len=4096, layout="fused",
        description="V2-Lite shape H=16, B=64, uniform context 4096, fused [64,4096,576] bf16 cache"),
    "v3_b32_s4096": Workload(
        "v3_b32_s4096", batch=32, heads=128, seed=20263, seq_len=4096, layout="fused",
        description="DeepSeek-V3 shape H=128, B=32, context 4096, bf16 cache"),
    "v3_b128_paged": Workload(
        "v3_b128_paged", batch=128, heads=128, seed=20264, len_range=(1024, 16384), layout="paged",
        block_size=64,
        description="V3 shape H=128, B=128, lengths ~ U[1024,16384], paged bf16 cache, 64-token "
                    "blocks, random permuted block table"),
    "v3_b64_s32768_fp8": Workload(
        "v3_b64_s32768_fp8", batch=64, heads=128, seed=20265, seq_len=32768, layout="fused",
        dtype="fp8_e4m3",
        description="V3 shape H=128, B=64, context 32768, E4M3 cache with a float32 scale per token"),
}


@dataclass
class DecodeInputs:
    """Device tensors of one decode step plus the layout description.

    Cache addressing: the latent row of token t of sequence b is row
    ``slot`` of ``kv_rows`` ([num_slots, 512] view) and its rope row is row
    ``slot`` of ``pe_rows`` ([num_slots, 64] view), where slot =
    b * seq_stride + t (contiguous) or
    block_table[b, t // block_size] * block_size + t % block_size (paged).
    """
    workload: Workload
    scale: float
    q_nope: torch.Tensor          # [B, H, 128] bf16
    q_pe: torch.Tensor            # [B, H, 64] bf16
    w_uk: torch.Tensor            # [H, 128, 512] bf16
    w_uv: torch.Tensor            # [H, 128, 512] bf16
    storage: torch.Tensor         # the cache allocation (bf16 or uint8)
    kv_rows: torch.Tensor         # [num_slots, 512] view into storage
    pe_rows: torch.Tensor         # [num_slots, 64] view into storage
    seq_lens: torch.Tensor        # [B] int32
    seq_stride: int               # token slots per sequence (contiguous), else 0
    block_table: Optional[torch.Tensor] = None   # [B, max_blocks] int32
    block_size: int = 0
    token_scale: Optional[torch.Tensor] = None   # [num_slots] float32 (E4M3 cache)
    max_seq_len: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return self.q_nope.shape[0]

    @property
    def heads(self):
        return self.q_nope.shape[1]

    def cache_bytes(self):
        """Bytes of cache rows the decode step reads (active tokens only)."""
        per_tok = D_K * (2 if self.workload.dtype == "bf16" else 1)
        if self.workload.dtype == "fp8_e4m3":
            per_tok += 4
        return int(self.seq_lens.to(torch.int64).sum().item()) * per_tok


def _normal(gen, shape, std, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _to_e4m3(x):
    """Per-token E4M3 encoding of x [..., 576] float32 -> (codes uint8, scale float32)."""
    amax = x.abs().amax(dim=-1)
    scale = (amax / E4M3_MAX).clamp_min(torch.finfo(torch.float32).tiny)
    q = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), scale


def make_inputs(workload, device="cpu", batch=None, seq_len=None, heads=None):
    """Draw one workload's inputs on `device`.

    `batch`, `seq_len` and `heads` override the workload's sizes (used for
    reduced-size cases in tests); the recipe is otherwise unchanged.
    """
    if isinstance(workload, str):
        workload = WORKLOADS[workload]
    B = batch if batch is not None else workload.batch
    H = heads if heads is not None else workload.heads
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(workload.seed)

    if workload.len_range is not None:
        lo, hi = workload.len_range
        if seq_len is not None:
            lo, hi = max(1, lo * seq_len // workload.len_range[1]), seq_len
        lens = torch.randint(lo, hi + 1, (B,), generator=gen, device=dev, dtype=torch.int64)
    else:
        S = seq_len if seq_len is not None else workload.seq_len
        lens = torch.full((B,), S, dtype=torch.int64, device=dev)
    lens_host = lens.cpu()
    max_len = int(lens_host.max().item())

    block_table = None
    perm = None
    if workload.layout == "paged":
        bs = workload.block_size
        nblk = [(int(t) + bs - 1) // bs for t in lens_host]
        total_blocks = sum(nblk)
        perm = torch.randperm(total_blocks, generator=gen, device=dev).to(torch.int32)
        max_blocks = max(nblk)
        bt = torch.zeros((B, max_blocks), dtype=torch.int32, device=dev)
        off = 0
        for b in range(B):
            bt[b, :nblk[b]] = perm[off:off + nblk[b]]
            off += nblk[b]
        block_table = bt

    wstd = 1.0 / math.sqrt(D_C)
    q_nope = _normal(gen, (B, H, D_N), 1.0, dev).to(torch.bfloat16)
    q_pe = _normal(gen, (B, H, D_R), 1.0, dev).to(torch.bfloat16)
    w_uk = _normal(gen, (H, D_N, D_C), wstd, dev).to(torch.bfloat16)
    w_uv = _normal(gen, (H, D_V, D_C), wstd, dev).to(torch.bfloat16)

    fp8 = workload.dtype == "fp8_e4m3"
    elem = torch.uint8 if fp8 else torch.bfloat16
    token_scale = None
    if workload.layout == "paged":
        bs = workload.block_size
        total_blocks = int(perm.numel())
        x = _normal(gen, (total_blocks, bs, D_K), 1.0, dev)
        if fp8:
            storage, token_scale = _to_e4m3(x)
        else:
            storage = x.to(torch.bfloat16)
        del x
        seq_stride = 0
        rows = storage.view(total_blocks * bs, D_K)
        kv_rows, pe_rows = rows[:, :D_C], rows[:, D_C:]
    else:
        cap = workload.seq_capacity if (workload.seq_capacity and seq_len is None) else max_len
        cap = max(cap, max_len)
        if workload.layout == "separate":
            kv = torch.zeros((B, cap, D_C), dtype=elem, device=dev)
            pe = torch.zeros((B, cap, D_R), dtype=elem, device=dev)
        else:
            storage = torch.zeros((B, cap, D_K), dtype=elem, device=dev)
        if fp8:
            token_scale = torch.zeros((B, cap), dtype=torch.float32, device=dev)
        for b in range(B):
            T = int(lens_host[b])
            x = _normal(gen, (T, D_K), 1.0, dev)
            if fp8:
                codes, sc = _to_e4m3(x)
                token_scale[b, :T] = sc
                vals = codes
            else:
                vals = x.to(torch.bfloat16)
            if workload.layout == "separate":
                kv[b, :T] = vals[:, :D_C]
                pe[b, :T] = vals[:, D_C:]
            else:
                storage[b, :T] = vals
        seq_stride = cap
        if workload.layout == "separate":
            storage = kv
            kv_rows = kv.view(B * cap, D_C)
            pe_rows = pe.view(B * cap, D_R)
        else:
            rows = storage.view(B * cap, D_K)
            kv_rows, pe_rows = rows[:, :D_C], rows[:, D_C:]
        if token_scale is not None:
            token_scale = token_scale.view(B * cap)

    if token_scale is not None and workload.layout == "paged":
        token_scale = token_scale.view(-1)

    extra = {}
    if workload.layout == "separate":
        extra["pe_storage"] = pe

    return DecodeInputs(
        workload=workload, scale=1.0 / math.sqrt(D_N + D_R), q_nope=q_nope, q_pe=q_pe,
        w_uk=w_uk, w_uv=w_uv, storage=storage, kv_rows=kv_rows, pe_rows=pe_rows,
        seq_lens=lens.to(torch.int32), seq_stride=seq_stride, block_table=block_table,
        block_size=workload.block_size if workload.layout == "paged" else 0,
        token_scale=token_scale, max_seq_len=max_len, extra=extra)


def random_latent_queries(batch, heads, seed, device="cpu"):
    """Stand-alone latent queries q_lat [B, H, 512] bf16 ~ N(0, 1), for testing
    the latent decode step in isolation (a wider score range than the absorbed
    queries of the workloads, whose std is about 0.5)."""
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(seed)
    return _normal(gen, (batch, heads, D_C), 1.0, torch.device(device)).to(torch.bfloat16)


def random_partials(batch, splits, heads, seed, device="cpu", empty_fraction=0.25):
    """Split-KV partial results for testing the combine step in isolation:
    o_part [B, P, H, 512] bfloat16 ~ N(0,1), lse_part [B, P, H] float32
    ~ N(0, 4) with about `empty_fraction` of the (b, p) slots set to -inf
    (an empty token range); slot p = 0 is never empty."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    o = _normal(gen, (batch, splits, heads, D_C), 1.0, dev)
    lse = _normal(gen, (batch, splits, heads), 2.0, dev)
    u = torch.rand((batch, splits), generator=gen, device=dev)
    empty = u < empty_fraction
    empty[:, 0] = False
    lse = torch.where(empty.unsqueeze(-1), torch.full_like(lse, -math.inf), lse)
    o = torch.where(empty.unsqueeze(-1).unsqueeze(-1), torch.zeros_like(o), o)
    return o.to(torch.bfloat16), lse


def random_projection_rows(batch, num_new, seed, device="cpu", width=D_K):
    """New tokens for the cache-append step: [B, n, width] bfloat16 ~ N(0, 1),
    each row standing for a token's fused down-projection output (512 latent
    values, then the 64-wide RoPE key before rotation; the cache rows of the
    workloads have the same distribution)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    return _normal(gen, (batch, num_new, width), 1.0, dev).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# Dominant ("sink" / outlier) tokens.  Real attention often has a few cached
# tokens whose scores stand far above the rest for every head; an online
# softmax that meets one late must move its running max and rescale what it
# has accumulated.  These draws plant such tokens: the RoPE query of every head
# shares one unit direction u, and a planted token's RoPE key points along u
# with a chosen length, so its score rises by a chosen amount for every head.
# ---------------------------------------------------------------------------

def sink_direction(seed, device="cpu"):
    """A unit vector u in the 64-wide RoPE space (float32)."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    u = _normal(gen, (D_R,), 1.0, dev)
    return u / u.norm()


def aligned_rope_queries(shape, u, seed, device="cpu"):
    """RoPE queries [*shape, 64] bfloat16 of the form r u + n: weight
    r ~ U[0.5, 1.5] along the shared direction u, plus n ~ N(0, 1) with its
    component along u removed.  A planted token whose key has length g along u
    adds about r * g * scale to this query's score."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    u = u.to(device=dev, dtype=torch.float32)
    r = torch.rand(tuple(shape) + (1,), generator=gen, device=dev) + 0.5
    n = _normal(gen, tuple(shape) + (D_R,), 1.0, dev)
    n = n - (n @ u).unsqueeze(-1) * u
    return (r * u + n).to(torch.bfloat16)


def plant_sink_tokens(x, sinks, u, seed):
    """Overwrite cached tokens of DecodeInputs x with dominant tokens, in place.

    sinks: iterable of (b, t, jump): sequence b, position t, and jump in
    natural-log units.  Token (b, t) gets a fresh row: 512 latent values and a
    64-wide RoPE key ~ N(0, 1), then the key's component along u is set to
    jump / x.scale, so for a query r u + n (aligned_rope_queries) its score
    gains about r * jump.  The row is stored like every other row of x (bf16,
    or E4M3 codes with a fresh per-token scale) at the slot of (b, t) in x's
    layout (contiguous slot b * seq_stride + t, or through the block table).
    """
    dev = x.kv_rows.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    u = u.to(device=dev, dtype=torch.float32)
    fp8 = x.workload.dtype == "fp8_e4m3"
    for b, t, jump in sinks:
        if x.block_table is not None:
            slot = int(x.block_table[b, t // x.block_size].item()) * x.block_size + t % x.block_size
        else:
            slot = b * x.seq_stride + t
        row = _normal(gen, (1, D_K), 1.0, dev)
        k = row[0, D_C:]
        k -= (k @ u) * u
        k += (float(jump) / x.scale) * u
        if fp8:
            codes, sc = _to_e4m3(row)
            x.kv_rows[slot] = codes[0, :D_C]
            x.pe_rows[slot] = codes[0, D_C:]
            x.token_scale[slot] = sc[0]
        else:
            vals = row.to(torch.bfloat16)
            x.kv_rows[slot] = vals[0, :D_C]
            x.pe_rows[slot] = vals[0, D_C:]
