"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that at least one pin in oracle_pins.py fails for each: a dropped term, a
wrong sign, scale or index, a transposed or shifted operand."""
import importlib.util
import math
import os

import numpy as np
import pytest

from tests import oracle_pins as pins

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "mla_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("mla_oracle_mutant", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _latent_attention_factory(variant):
    def latent_attention(q_lat, q_pe, c, k_r, scale):
        H, T = q_lat.shape[0], c.shape[0]
        if T == 0:
            return np.zeros((H, c.shape[1])), np.full(H, -np.inf)
        if variant == "drop_rope":
            s = scale * (q_lat @ c.T)
        elif variant == "no_scale":
            s = q_lat @ c.T + q_pe @ k_r.T
        elif variant == "rope_sign":
            s = scale * (q_lat @ c.T - q_pe @ k_r.T)
        else:
            s = scale * (q_lat @ c.T + q_pe @ k_r.T)
        axis = 0 if variant == "softmax_over_heads" else 1
        m = s.max(axis=axis, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=axis, keepdims=True)
        p = w if variant == "unnormalised" else w / l
        o = p @ c
        if axis == 0:
            lse = (m + np.log(l)).max(axis=0) * np.ones(H)
        else:
            lse = m[:, 0] + np.log(l[:, 0])
        if variant == "lse_log2":
            lse = m[:, 0] + np.log2(l[:, 0])
        return o, lse
    return latent_attention


def _absorb_q_shifted(q_nope, w_uk):
    B, H, _ = q_nope.shape
    out = np.empty((B, H, w_uk.shape[2]))
    for h in range(H):
        out[:, h, :] = q_nope[:, h, ::-1] @ w_uk[h]
    return out


def _expand_v_wrong_head(o_lat, w_uv):
    B, H, _ = o_lat.shape
    out = np.empty((B, H, w_uv.shape[1]))
    for h in range(H):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[(h + 1) % H].T
    return out


def _combine_no_norm(o_parts, lse_parts):
    w = np.exp(lse_parts)
    return np.einsum("ph,phc->hc", w, o_parts), np.log(w.sum(0))


def _combine_plain_mean(o_parts, lse_parts):
    ok = np.isfinite(lse_parts)
    return o_parts.sum(0) / np.maximum(ok.sum(0), 1)[:, None], np.log(np.exp(lse_parts).sum(0))


def _rope_sign(x, positions, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.outer(np.asarray(positions, dtype=np.float64), inv)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    cos, sin = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * cos + x[..., 1::2] * sin
    y[..., 1::2] = x[..., 1::2] * cos - x[..., 0::2] * sin
    return y


def _rope_half_split(x, positions, base=10000.0):
    # rotates (x[i], x[i + d/2]) instead of the interleaved pairs
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.outer(np.asarray(positions, dtype=np.float64), inv)
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    cos, sin = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def _e4m3_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 8.0))
    return np.where((e == 15) & ((c & 7) == 7), np.nan, sign * mag)


def _bf16_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _slots_wrong_offset(b, length, seq_stride=None, block_table=None, block_size=None):
    t = np.arange(length, dtype=np.int64)
    if block_table is None:
        return b * int(seq_stride) + t
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[b, t // block_size] * block_size + t // block_size


def _latent_bytes_no_rope(kv_lora_rank, qk_rope_head_dim, elem_bytes, source="mla config"):
    if kv_lora_rank is None or qk_rope_head_dim is None:
        raise ValueError(f"kv_lora_rank / qk_rope_head_dim missing ({source})")
    return kv_lora_rank * elem_bytes


def _latent_bytes_default(kv_lora_rank, qk_rope_head_dim, elem_bytes, source="mla config"):
    return ((kv_lora_rank or 512) + (qk_rope_head_dim or 64)) * elem_bytes


def _naive_attention_no_rope_key(q_nope, q_pe, c, k_r, w_uk, w_uv, scale):
    H = q_nope.shape[0]
    out = np.empty((H, w_uv.shape[1]))
    for h in range(H):
        s = scale * ((c @ w_uk[h].T) @ q_nope[h])
        w = np.exp(s - s.max())
        out[h] = (w / w.sum()) @ (c @ w_uv[h].T)
    return out


def _causal_no_mask(q_nope, q_pe_raw, c, k_r_raw, w_uk, w_uv, scale, rope_base=10000.0):
    L, H, _ = q_nope.shape
    pos = np.arange(L)
    mod = fresh_oracle()
    q_pe = mod.rope_interleaved(q_pe_raw, pos, rope_base)
    k_r = mod.rope_interleaved(k_r_raw, pos, rope_base)
    out = np.empty((L, H, w_uv.shape[1]))
    for h in range(H):
        keys = np.concatenate([c @ w_uk[h].T, k_r], axis=1)
        q = np.concatenate([q_nope[:, h, :], q_pe[:, h, :]], axis=1)
        s = scale * (q @ keys.T)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (w / w.sum(axis=1, keepdims=True)) @ (c @ w_uv[h].T)
    return out


def _bf16_truncate(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _bf16_ties_odd(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lo, rem = u >> np.uint64(16), u & np.uint64(0xFFFF)
    up = (rem > 0x8000) | ((rem == 0x8000) & ((lo & np.uint64(1)) == np.uint64(0)))
    return (lo + up.astype(np.uint64)).astype(np.uint16)


def _e4m3_encode_factory(variant):
    def e4m3fn_encode(x):
        mod = fresh_oracle()
        x = np.asarray(x, dtype=np.float64)
        grid = mod.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
        a = np.abs(x)
        hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)
        lo = np.clip(hi - 1, 0, len(grid) - 1)
        d_lo, d_hi = a - grid[lo], grid[hi] - a
        tie_hi = (hi % 2 == 1) if variant == "ties_odd" else (hi % 2 == 0)
        code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & tie_hi), hi, lo).astype(np.uint8)
        if variant == "drop_sign":
            return code
        return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return e4m3fn_encode


def _quantize_amax_240(v32):
    mod = fresh_oracle()
    v32 = np.asarray(v32, dtype=np.float32)
    scale = np.maximum(np.max(np.abs(v32), axis=-1) / np.float32(240.0), np.finfo(np.float32).tiny).astype(np.float32)
    q = np.clip((v32 / scale[..., None]).astype(np.float32), -448, 448)
    return mod.e4m3fn_encode(q), scale


def _append_factory(variant):
    def cache_append_rows(kv_in_bits, positions, dtype, rope_base=10000.0, d_c=512, d_r=64):
        mod = fresh_oracle()
        bits = np.asarray(kv_in_bits, dtype=np.uint16)
        B, n = bits.shape[0], bits.shape[1]
        step = np.zeros(n, dtype=np.int64) if variant == "no_offset" else np.arange(n, dtype=np.int64)
        pos = np.asarray(positions, dtype=np.int64)[:, None] + step[None, :]
        shift = 1 if variant == "rope_plus_one" else 0
        k_r = mod.bf16_to_f64(bits[..., d_c:d_c + d_r])
        rot = np.stack([mod.rope_interleaved(k_r[b], pos[b] + shift, base=rope_base) for b in range(B)])
        if variant == "fp8_unrotated" and dtype == "fp8_e4m3":
            rot = k_r
        if dtype == "bf16":
            return pos, bits[..., :d_c].copy(), mod.f32_to_bf16_bits(rot.astype(np.float32)), None
        v32 = np.concatenate([mod.bf16_to_f64(bits[..., :d_c]).astype(np.float32), rot.astype(np.float32)], axis=-1)
        codes, scale = mod.e4m3_quantize_token(v32)
        return pos, codes[..., :d_c], codes[..., d_c:], scale
    return cache_append_rows


MUTANTS = {
    "latent_attention/drop_rope_term": ("latent_attention", _latent_attention_factory("drop_rope")),
    "latent_attention/no_scale": ("latent_attention", _latent_attention_factory("no_scale")),
    "latent_attention/rope_term_sign": ("latent_attention", _latent_attention_factory("rope_sign")),
    "latent_attention/softmax_over_heads": ("latent_attention", _latent_attention_factory("softmax_over_heads")),
    "latent_attention/unnormalised": ("latent_attention", _latent_attention_factory("unnormalised")),
    "latent_attention/lse_in_log2": ("latent_attention", _latent_attention_factory("lse_log2")),
    "absorb_q/reversed_nope_index": ("absorb_q", _absorb_q_shifted),
    "expand_v/wrong_head": ("expand_v", _expand_v_wrong_head),
    "combine_splits/unnormalised": ("combine_splits", _combine_no_norm),
    "combine_splits/plain_mean": ("combine_splits", _combine_plain_mean),
    "rope/sign_flipped": ("rope_interleaved", _rope_sign),
    "rope/half_split_pairs": ("rope_interleaved", _rope_half_split),
    "e4m3/bias_8": ("e4m3fn_to_f64", _e4m3_bias8),
    "bf16/shift_15": ("bf16_to_f64", _bf16_shift15),
    "token_slots/paged_offset": ("token_slots", _slots_wrong_offset),
    "cache_bytes/no_rope_term": ("latent_cache_bytes_per_token", _latent_bytes_no_rope),
    "cache_bytes/silent_defaults": ("latent_cache_bytes_per_token", _latent_bytes_default),
    "naive_attention/no_rope_key": ("naive_attention", _naive_attention_no_rope_key),
    "causal_forward/no_mask": ("causal_naive_forward", _causal_no_mask),
    "bf16_encode/truncate": ("f32_to_bf16_bits", _bf16_truncate),
    "bf16_encode/ties_to_odd": ("f32_to_bf16_bits", _bf16_ties_odd),
    "e4m3_encode/ties_to_odd": ("e4m3fn_encode", _e4m3_encode_factory("ties_odd")),
    "e4m3_encode/drop_sign": ("e4m3fn_encode", _e4m3_encode_factory("drop_sign")),
    "e4m3_quantize/max_240": ("e4m3_quantize_token", _quantize_amax_240),
    "cache_append/no_position_offset": ("cache_append_rows", _append_factory("no_offset")),
    "cache_append/rope_position_plus_one": ("cache_append_rows", _append_factory("rope_plus_one")),
    "cache_append/fp8_key_unrotated": ("cache_append_rows", _append_factory("fp8_unrotated")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    attr, fn = MUTANTS[name]
    mod = fresh_oracle()
    assert hasattr(mod, attr)
    setattr(mod, attr, fn)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # any failure of the pin counts as catching the mutant
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
