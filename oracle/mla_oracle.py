"""Plain float64 CPU oracle for DeepSeek Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it: the two share no kernels, helpers, tables or
constants.  Inputs reach both sides from the seeded generators only.

Everything here is NumPy in float64, written for a reader to check against the
source pages by eye, not for speed.  Library primitives (matmul, exp, sum) are
used as single steps; there is no blocking, fusion or reordering beyond what
the plain definitions state.

Source pages cited below (by title; sections as titled on each page):

* [AUDIT]  "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
           (llm-atlas research note on running V2-Lite layer-1 through the
           official naive and absorb attention paths).
* [MLA80]  "80 行 PyTorch 从零写 DeepSeek 的 MLA：量一遍 KV cache、踩一遍
           absorption …" (blog post with a minimal PyTorch MLA).
* [TRACE]  "DeepSeek-V2-Lite 真实权重执行审计" (real-weight trace of V2-Lite).
* [G5SPEC] "G5 MLA KV 访存建模设计规格" (design spec for modelling MLA decode
           KV reads; equations eq:gmkv-cache, eq:gmkv-read, eq:gmkv-ratio).

Pins: every function below is checked in ``tests/test_oracle_*.py`` against
something other than itself (numbers printed on the pages, closed forms,
brute force on tiny inputs, special cases that reduce to a library routine,
algebraic identities).  No function here is "parity unpinned".

Readings where the pages leave a step open (listed again in the design doc):

* softmax scale is an explicit argument; the synthetic workloads use
  1/sqrt(qk_nope + qk_rope) = 1/sqrt(192) (the SDPA default for a 192-wide
  query, [MLA80] §2 code), with no YaRN factor;
* the decode query attends to every cached token, itself included ([MLA80]
  §2: the causal mask is only used when there is no past);
* the RoPE half of the cache holds keys that are already rotated;
* lse is the natural log of sum_t exp(s_t) with s already scaled; an empty
  token range has lse = -inf and contributes weight 0;
* W_UK is stored [H, qk_nope, kv_lora_rank] and W_UV [H, v_head, kv_lora_rank].
"""

import math

import numpy as np

# ---------------------------------------------------------------------------
# Decoding of stored element codes into float64
# ---------------------------------------------------------------------------


def bf16_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64, exactly.

    A bfloat16 number is the upper half of an IEEE binary32 word, so shifting
    the 16 stored bits into the high half of a 32-bit word gives the same
    number as a float32, which widens to float64 without rounding.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes):
    """OCP FP8 E4M3 ("FN": no infinities) codes (uint8) -> float64, exactly.

    Layout s.eeee.mmm with exponent bias 7.  Exponent field 0 is subnormal,
    m/8 * 2**-6; otherwise (1 + m/8) * 2**(e-7).  The pattern with all
    exponent and mantissa bits set (0x7f, 0xff) is NaN; the largest finite
    magnitude is 1.75 * 2**8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)


# ---------------------------------------------------------------------------
# Cache-size closed forms ([G5SPEC] eq:gmkv-cache / eq:gmkv-read / eq:gmkv-ratio,
# [AUDIT] §2.1 and §4, [MLA80] §1, [TRACE] §3.2)
# ---------------------------------------------------------------------------


def _require(name, value, source):
    """MLA dimensions have no defaults: a missing one is an error that names
    the field and where it was expected ([G5SPEC] constraints section and
    Appendix C interface contract)."""
    if value is None:
        raise ValueError(f"required MLA field '{name}' is missing (source: {source})")
    return value


def latent_cache_bytes_per_token(kv_lora_rank, qk_rope_head_dim, elem_bytes, source="mla config"):
    """Bytes one token occupies in one layer's latent cache:
    (d_c + d_rope) * e  ([G5SPEC] eq:gmkv-cache; [MLA80] §1 table, MLA row)."""
    d_c = _require("kv_lora_rank", kv_lora_rank, source)
    d_r = _require("qk_rope_head_dim", qk_rope_head_dim, source)
    return (d_c + d_r) * elem_bytes


def decode_kv_read_bytes(batch, s_ctx, kv_lora_rank, qk_rope_head_dim, elem_bytes, source="mla config"):
    """Bytes one decode step reads from the latent cache of one layer:
    B * s_ctx * (d_c + d_rope) * e, with no head-count term
    ([G5SPEC] eq:gmkv-read and use case 1)."""
    return batch * s_ctx * latent_cache_bytes_per_token(kv_lora_rank, qk_rope_head_dim, elem_bytes, source)


def mha_equivalent_ratio(kv_lora_rank, qk_rope_head_dim, num_heads, head_dim, source="mla config"):
    """Latent cache size over an MHA cache with the same heads:
    (d_c + d_rope) / (2 * n_h * d_h)  ([G5SPEC] eq:gmkv-ratio)."""
    d_c = _require("kv_lora_rank", kv_lora_rank, source)
    d_r = _require("qk_rope_head_dim", qk_rope_head_dim, source)
    return (d_c + d_r) / (2.0 * num_heads * head_dim)


def equivalent_gqa_groups(kv_lora_rank, qk_rope_head_dim, head_dim):
    """Number of GQA key/value groups whose cache equals the latent cache:
    (d_c + d_rope) / (2 * d_h)  ([G5SPEC] background and Appendix A)."""
    return (kv_lora_rank + qk_rope_head_dim) / (2.0 * head_dim)


def naive_cache_bytes_per_token(num_heads, qk_nope_head_dim, qk_rope_head_dim, v_head_dim, elem_bytes):
    """Bytes per token per layer when the expanded per-head keys
    (nope + rope) and values are cached: H * (d_n + d_r + d_v) * e
    ([AUDIT] §2.1 and §4.1; [TRACE] §3.2)."""
    return num_heads * (qk_nope_head_dim + qk_rope_head_dim + v_head_dim) * elem_bytes


def mha_cache_bytes_per_token(num_heads, head_dim, elem_bytes):
    """MHA cache: n_h keys and n_h values of d_h each, 2 * n_h * d_h * e
    ([MLA80] §1 table)."""
    return 2 * num_heads * head_dim * elem_bytes


def gqa_cache_bytes_per_token(num_kv_heads, head_dim, elem_bytes):
    """GQA cache: n_kv shared key/value heads, 2 * n_kv * d_h * e
    ([MLA80] §1 table)."""
    return 2 * num_kv_heads * head_dim * elem_bytes


# ---------------------------------------------------------------------------
# Decode steps, each in float64
# ---------------------------------------------------------------------------


def absorb_q(q_nope, w_uk):
    """Key absorption: move W_UK from every cached token onto the query.

    q_lat[b, h, c] = sum_d q_nope[b, h, d] * W_UK[h, d, c]

    because q^T (W_K c_t) = (W_K^T q)^T c_t ([AUDIT] §2.2; [MLA80] §4 and §5).
    q_nope [B, H, d_n], w_uk [H, d_n, d_c] -> q_lat [B, H, d_c].
    """
    B, H, _ = q_nope.shape
    q_lat = np.empty((B, H, w_uk.shape[2]))
    for h in range(H):
        q_lat[:, h, :] = q_nope[:, h, :] @ w_uk[h]
    return q_lat


def latent_attention(q_lat, q_pe, c, k_r, scale):
    """Scores of every head against the shared latent cache of one sequence,
    softmax over the cached tokens, and the probability-weighted sum of the
    latent rows (aggregation in latent space).

    s[h, t] = scale * (q_lat[h] . c_t + q_pe[h] . k_R,t)   ([AUDIT] §2.2, §2.4;
                                                            [MLA80] §5)
    p[h, :] = softmax_t(s[h, :])
    o_lat[h] = sum_t p[h, t] * c_t                           ([AUDIT] §2.3)
    lse[h]   = log sum_t exp(s[h, t])

    q_lat [H, d_c], q_pe [H, d_r], c [T, d_c], k_r [T, d_r].  With T = 0 the
    result is o_lat = 0 and lse = -inf (an empty range carries no weight).
    """
    H = q_lat.shape[0]
    T = c.shape[0]
    if T == 0:
        return np.zeros((H, c.shape[1])), np.full(H, -np.inf)
    s = scale * (q_lat @ c.T + q_pe @ k_r.T)
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1, keepdims=True)
    p = w / l
    o_lat = p @ c
    lse = m[:, 0] + np.log(l[:, 0])
    return o_lat, lse


def expand_v(o_lat, w_uv):
    """Value absorption, second half: expand the latent aggregate per head.

    out[b, h, j] = sum_c W_UV[h, j, c] * o_lat[b, h, c]

    because sum_t p_t (W_V c_t) = W_V (sum_t p_t c_t) ([AUDIT] §2.3).
    o_lat [B, H, d_c], w_uv [H, d_v, d_c] -> out [B, H, d_v].
    """
    B, H, _ = o_lat.shape
    out = np.empty((B, H, w_uv.shape[1]))
    for h in range(H):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h].T
    return out


def combine_splits(o_parts, lse_parts):
    """Merge attention results computed over disjoint token ranges.

    Range i gives (o_i, lse_i) with o_i its own softmax-weighted latent sum.
    The whole-range result is LSE = log sum_i exp(lse_i) and
    o = sum_i exp(lse_i - LSE) * o_i.  A range with lse = -inf gets weight 0.
    The pages name flash-decoding only in passing ([G5SPEC] Appendix B: the
    cache read runs concurrently with the attention); this is the plain
    log-sum-exp identity of a softmax over a union of disjoint sets.

    o_parts [P, H, d_c], lse_parts [P, H] -> (o [H, d_c], lse [H]).
    """
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    mx = lse_parts.max(axis=0)
    finite = np.isfinite(mx)
    safe_mx = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_mx[None, :]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, safe_mx + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o = np.einsum("ph,phc->hc", w, o_parts) / np.where(tot > 0, tot, 1.0)[:, None]
    return o, lse


def latent_attention_ranges(q_lat, q_pe, c, k_r, scale, bounds):
    """latent_attention applied separately to each token range
    [bounds[i], bounds[i+1]) of one sequence.  Returns o [P, H, d_c] and
    lse [P, H] (each range normalised by its own softmax sum)."""
    os_, ls_ = [], []
    for i in range(len(bounds) - 1):
        a, z = bounds[i], bounds[i + 1]
        o, l = latent_attention(q_lat, q_pe, c[a:z], k_r[a:z], scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def naive_attention(q_nope, q_pe, c, k_r, w_uk, w_uv, scale):
    """The expanded ("naive"/"standard") form for one sequence: every cached
    latent row is projected to a per-head key and value, then ordinary
    softmax attention runs per head ([AUDIT] §2.1; [MLA80] §2 code).

    key_t  = [W_UK[h] c_t ; k_R,t]  (d_n + d_r)   the RoPE key is shared by
                                                 all heads ([AUDIT] §2.4)
    val_t  = W_UV[h] c_t            (d_v)
    out[h] = sum_t softmax_t(scale * key_t . [q_nope[h]; q_pe[h]]) * val_t

    q_nope [H, d_n], q_pe [H, d_r], c [T, d_c], k_r [T, d_r] -> out [H, d_v].
    """
    H = q_nope.shape[0]
    out = np.empty((H, w_uv.shape[1]))
    for h in range(H):
        keys = np.concatenate([c @ w_uk[h].T, k_r], axis=1)
        vals = c @ w_uv[h].T
        q = np.concatenate([q_nope[h], q_pe[h]])
        s = scale * (keys @ q)
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ vals
    return out


# ---------------------------------------------------------------------------
# Encoding into the stored formats (used by the cache append)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x):
    """float32 values -> bfloat16 bit patterns, rounded to nearest, ties to
    the even pattern (finite inputs).

    The bfloat16 values are the float32 values whose low 16 bits are zero; x
    lies between the two bracketing ones, lo = x with the low bits cleared and
    lo + one bf16 step, and the nearer one is taken (the even one on a tie).
    """
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lo = u & np.uint64(0xFFFF0000)
    rem = u & np.uint64(0xFFFF)
    half = np.uint64(0x8000)
    up = (rem > half) | ((rem == half) & (((lo >> np.uint64(16)) & np.uint64(1)) == np.uint64(1)))
    return ((lo >> np.uint64(16)) + up.astype(np.uint64)).astype(np.uint16)


def e4m3fn_encode(x):
    """Values within [-448, 448] -> OCP E4M3 codes: the nearest finite E4M3
    value, ties to the even code (even mantissa), sign from the sign bit.

    Written as a search over the 127 non-negative finite codes, which are
    increasing in value (e4m3fn_to_f64 gives the grid).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 448.0) or np.any(np.isnan(x)):
        raise ValueError("e4m3fn_encode expects finite values within [-448, 448]")
    grid = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))  # codes 0 .. 126
    a = np.abs(x)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)  # first grid value >= a
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def e4m3_quantize_token(v32):
    """One token's float32 values [..., n] -> (codes uint8, scale float32) with
    one scale per token: scale = max|v| / 448 in float32 (at least the
    smallest normal float32), code = E4M3(v / scale), the division in float32.

    This is the per-token reading of the fp8 cache record: all 576 values of
    a token share one fp32 scale ([G5SPEC] use case 1, 576 bytes per token).
    """
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.max(np.abs(v32), axis=-1)
    scale = np.maximum(amax / np.float32(448.0), np.finfo(np.float32).tiny).astype(np.float32)
    q = np.clip((v32 / scale[..., None]).astype(np.float32), np.float32(-448.0), np.float32(448.0))
    return e4m3fn_encode(q), scale


def cache_append_rows(kv_in_bits, positions, dtype, rope_base=10000.0, d_c=512, d_r=64):
    """Expected cache contents for appending new tokens.

    kv_in_bits [B, n, >= d_c + d_r] bfloat16 bits: each row is a token's
    fused projection output, d_c latent values then d_r RoPE-key values
    before rotation ([TRACE] §3, the fused kv_a_proj output; [AUDIT] §2.4,
    the rope key is cached separately).  Token j of sequence b sits at
    position positions[b] + j; its key half is rotated there
    (rope_interleaved, float64) before it is stored ([MLA80] §2: the key is
    rotated at its own position before it enters the cache).

    Returns (pos [B, n] int64, kv [B, n, d_c], pe [B, n, d_r], scale [B, n] or
    None): bf16 caches hold the latent bits unchanged and the rotated key
    rounded float64 -> float32 -> bfloat16 (nearest-even at each step); E4M3
    caches hold e4m3_quantize_token of the token's float32 values (latent
    exact, rotated key rounded to float32).
    """
    bits = np.asarray(kv_in_bits, dtype=np.uint16)
    B, n = bits.shape[0], bits.shape[1]
    pos = np.asarray(positions, dtype=np.int64)[:, None] + np.arange(n, dtype=np.int64)[None, :]
    k_r = bf16_to_f64(bits[..., d_c:d_c + d_r])
    rot = np.stack([rope_interleaved(k_r[b], pos[b], base=rope_base) for b in range(B)])
    if dtype == "bf16":
        return pos, bits[..., :d_c].copy(), f32_to_bf16_bits(rot.astype(np.float32)), None
    if dtype == "fp8_e4m3":
        v32 = np.concatenate([bf16_to_f64(bits[..., :d_c]).astype(np.float32), rot.astype(np.float32)], axis=-1)
        codes, scale = e4m3_quantize_token(v32)
        return pos, codes[..., :d_c], codes[..., d_c:], scale
    raise ValueError(f"unknown cache dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Cache addressing (contiguous slots or a block table) and batched decode
# ---------------------------------------------------------------------------


def token_slots(b, length, seq_stride=None, block_table=None, block_size=None):
    """Storage slot of tokens 0..length-1 of sequence b.

    Contiguous cache: slot = b * seq_stride + t.  Paged cache: token t lives
    in the physical block block_table[b, t // block_size] at offset
    t % block_size.  (The pages only name a paged cache as a production
    prerequisite, [AUDIT] §7; this is the plain reading of a block table.)
    """
    t = np.arange(length, dtype=np.int64)
    if block_table is None:
        return b * int(seq_stride) + t
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[b, t // block_size] * block_size + t % block_size


def load_rows(kv_codes, pe_codes, slots, dtype, token_scale=None):
    """Read the cached rows at `slots` and decode them to float64.

    kv_codes [num_slots, d_c] and pe_codes [num_slots, d_r] hold bfloat16 bit
    patterns (uint16) or E4M3 codes (uint8).  For E4M3 every element of a
    token is multiplied by that token's float32 scale.
    """
    if dtype == "bf16":
        return bf16_to_f64(kv_codes[slots]), bf16_to_f64(pe_codes[slots])
    if dtype == "fp8_e4m3":
        sc = np.asarray(token_scale, dtype=np.float32)[slots].astype(np.float64)[:, None]
        return e4m3fn_to_f64(kv_codes[slots]) * sc, e4m3fn_to_f64(pe_codes[slots]) * sc
    raise ValueError(f"unknown cache dtype {dtype!r}")


def latent_decode(q_lat, q_pe, kv_codes, pe_codes, seq_lens, scale, dtype="bf16",
                  seq_stride=None, block_table=None, block_size=None, token_scale=None,
                  batch_indices=None):
    """latent_attention for each sequence of a batch against its cached rows.

    q_lat [B, H, d_c], q_pe [B, H, d_r] float64.  Returns o_lat [n, H, d_c]
    and lse [n, H] for the sequences in `batch_indices` (default: all).
    """
    idx = range(q_lat.shape[0]) if batch_indices is None else batch_indices
    os_, ls_ = [], []
    for b in idx:
        slots = token_slots(b, int(seq_lens[b]), seq_stride, block_table, block_size)
        c, k_r = load_rows(kv_codes, pe_codes, slots, dtype, token_scale)
        o, l = latent_attention(q_lat[b], q_pe[b], c, k_r, scale)
        os_.append(o)
        ls_.append(l)
    return np.stack(os_), np.stack(ls_)


def absorbed_decode(q_nope, q_pe, w_uk, w_uv, kv_codes, pe_codes, seq_lens, scale, dtype="bf16",
                    seq_stride=None, block_table=None, block_size=None, token_scale=None,
                    batch_indices=None):
    """Absorbed-mode decode of one layer: absorb_q, latent_decode, expand_v.

    Returns a dict with q_lat, o_lat, lse and out for the selected sequences.
    """
    idx = list(range(q_nope.shape[0])) if batch_indices is None else list(batch_indices)
    q_lat = absorb_q(q_nope[idx], w_uk)
    sub_lens = np.asarray(seq_lens)[idx]
    os_, ls_ = [], []
    for j, b in enumerate(idx):
        slots = token_slots(b, int(sub_lens[j]), seq_stride, block_table, block_size)
        c, k_r = load_rows(kv_codes, pe_codes, slots, dtype, token_scale)
        o, l = latent_attention(q_lat[j], q_pe[b], c, k_r, scale)
        os_.append(o)
        ls_.append(l)
    o_lat = np.stack(os_)
    return {"q_lat": q_lat, "o_lat": o_lat, "lse": np.stack(ls_), "out": expand_v(o_lat, w_uv)}


def naive_decode(q_nope, q_pe, w_uk, w_uv, kv_codes, pe_codes, seq_lens, scale, dtype="bf16",
                 seq_stride=None, block_table=None, block_size=None, token_scale=None,
                 batch_indices=None):
    """Expanded-form decode of one layer (naive_attention per sequence)."""
    idx = range(q_nope.shape[0]) if batch_indices is None else batch_indices
    outs = []
    for b in idx:
        slots = token_slots(b, int(seq_lens[b]), seq_stride, block_table, block_size)
        c, k_r = load_rows(kv_codes, pe_codes, slots, dtype, token_scale)
        outs.append(naive_attention(q_nope[b], q_pe[b], c, k_r, w_uk, w_uv, scale))
    return np.stack(outs)


# ---------------------------------------------------------------------------
# RoPE, one-shot causal forward, and the decoupled-RoPE negative control
# ---------------------------------------------------------------------------


def rope_interleaved(x, positions, base=10000.0):
    """Rotary embedding on interleaved pairs ([MLA80] Appendix A).

    For a d-wide vector at position p, the pair (x[2i], x[2i+1]) is rotated by
    the angle p * base**(-2i/d):
        y[2i]   = x[2i]   * cos - x[2i+1] * sin
        y[2i+1] = x[2i+1] * cos + x[2i]   * sin
    x is [L, ..., d]: axis 0 is the position axis, matching `positions`
    (length L); any middle axes (e.g. heads) share the token's angle.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.outer(np.asarray(positions, dtype=np.float64), inv)  # [L, d/2]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    cos = np.cos(ang).reshape(shape)
    sin = np.sin(ang).reshape(shape)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * cos - x1 * sin
    y[..., 1::2] = x1 * cos + x0 * sin
    return y


def causal_naive_forward(q_nope, q_pe_raw, c, k_r_raw, w_uk, w_uv, scale, rope_base=10000.0):
    """One-shot forward of L tokens in expanded form with a causal mask and
    decoupled RoPE applied at each token's position ([MLA80] §2 code: RoPE on
    the per-head rope query and the shared rope key; causal mask when there is
    no past).

    q_nope [L, H, d_n], q_pe_raw [L, H, d_r] (not yet rotated),
    c [L, d_c], k_r_raw [L, d_r] (not yet rotated) -> out [L, H, d_v].
    """
    L, H, _ = q_nope.shape
    pos = np.arange(L)
    q_pe = rope_interleaved(q_pe_raw, pos, rope_base)
    k_r = rope_interleaved(k_r_raw, pos, rope_base)
    out = np.empty((L, H, w_uv.shape[1]))
    for h in range(H):
        keys = np.concatenate([c @ w_uk[h].T, k_r], axis=1)        # [L, d_n+d_r]
        vals = c @ w_uv[h].T                                         # [L, d_v]
        q = np.concatenate([q_nope[:, h, :], q_pe[:, h, :]], axis=1)  # [L, d_n+d_r]
        s = scale * (q @ keys.T)                                      # [L, L]
        s = np.where(np.tril(np.ones((L, L), dtype=bool)), s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ vals
    return out


def content_scores(q_nope, c, w_uk, absorbed, rope_on_content=False, positions_q=None,
                   positions_k=None, rope_base=10000.0):
    """Content half of the attention score for one head, two ways
    ([MLA80] §4).

    absorbed=False: expand K_C = c W_UK^T per token, then q_nope . K_C.
    absorbed=True:  q_lat = W_UK^T q_nope, then q_lat . c.
    rope_on_content=True rotates the expanded K_C (and q_nope) by position,
    the design that decoupled RoPE avoids; the absorbed form cannot express
    the rotation, so the two forms then disagree.

    q_nope [Lq, d_n], c [Lk, d_c], w_uk [d_n, d_c] -> [Lq, Lk].
    """
    if absorbed:
        return (q_nope @ w_uk) @ c.T
    k_c = c @ w_uk.T
    q = q_nope
    if rope_on_content:
        k_c = rope_interleaved(k_c, positions_k, rope_base)
        q = rope_interleaved(q_nope, positions_q, rope_base)
    return q @ k_c.T


def softmax_scale_default(qk_nope_head_dim, qk_rope_head_dim):
    """1/sqrt(query width), the SDPA default for a (d_n + d_r)-wide query
    ([MLA80] §2 code calls SDPA without an explicit scale)."""
    return 1.0 / math.sqrt(qk_nope_head_dim + qk_rope_head_dim)
