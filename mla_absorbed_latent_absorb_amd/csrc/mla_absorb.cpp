// Host side of the C ABI declared in include/mla_absorb.h: argument checks,
// split planning and kernel launches on the caller's stream.  Nothing here
// allocates, frees or synchronises.
#include "../../include/mla_absorb.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

mla_status fail(mla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mla_status ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p, name, where)                                                              \
  do {                                                                                           \
    if ((p) == nullptr) return fail(MLA_ERR_NULL, "%s is NULL (%s)", name, where);               \
    if (!aligned16(p)) return fail(MLA_ERR_ALIGN, "%s is not 16-byte aligned (%s)", name, where); \
  } while (0)

// Required-dimension checks: zero means missing, and nothing is defaulted.
mla_status check_latent_dims(const mla_dims* d, const char* where) {
  if (d == nullptr) return fail(MLA_ERR_NULL, "dims is NULL (%s)", where);
  if (d->kv_lora_rank <= 0) return fail(MLA_ERR_MISSING_DIM, "kv_lora_rank missing (mla_dims, %s)", where);
  if (d->qk_rope_head_dim <= 0)
    return fail(MLA_ERR_MISSING_DIM, "qk_rope_head_dim missing (mla_dims, %s)", where);
  return MLA_OK;
}

mla_status check_dims(const mla_dims* d, const char* where) {
  mla_status st = check_latent_dims(d, where);
  if (st != MLA_OK) return st;
  if (d->batch <= 0) return fail(MLA_ERR_MISSING_DIM, "batch missing (mla_dims, %s)", where);
  if (d->num_heads <= 0) return fail(MLA_ERR_MISSING_DIM, "num_heads missing (mla_dims, %s)", where);
  if (d->qk_nope_head_dim <= 0)
    return fail(MLA_ERR_MISSING_DIM, "qk_nope_head_dim missing (mla_dims, %s)", where);
  if (d->v_head_dim <= 0) return fail(MLA_ERR_MISSING_DIM, "v_head_dim missing (mla_dims, %s)", where);
  if (d->softmax_scale == 0.0f) return fail(MLA_ERR_MISSING_DIM, "softmax_scale missing (mla_dims, %s)", where);
  if (!(d->softmax_scale > 0.0f) || !std::isfinite(d->softmax_scale))
    return fail(MLA_ERR_UNSUPPORTED, "softmax_scale must be positive and finite (mla_dims, %s)", where);
  if (d->kv_lora_rank != 512)
    return fail(MLA_ERR_UNSUPPORTED, "kv_lora_rank %d not supported, built for 512 (%s)", d->kv_lora_rank, where);
  if (d->qk_rope_head_dim != 64)
    return fail(MLA_ERR_UNSUPPORTED, "qk_rope_head_dim %d not supported, built for 64 (%s)", d->qk_rope_head_dim,
                where);
  if (d->qk_nope_head_dim != 128)
    return fail(MLA_ERR_UNSUPPORTED, "qk_nope_head_dim %d not supported, built for 128 (%s)", d->qk_nope_head_dim,
                where);
  if (d->v_head_dim != 128)
    return fail(MLA_ERR_UNSUPPORTED, "v_head_dim %d not supported, built for 128 (%s)", d->v_head_dim, where);
  const int H = d->num_heads;
  if (H != 16 && H != 32 && H != 64 && H != 128)
    return fail(MLA_ERR_UNSUPPORTED, "num_heads %d not supported (16, 32, 64 or 128) (%s)", H, where);
  return MLA_OK;
}

size_t bytes_per_token(const mla_dims* d, int32_t dtype) {
  const size_t e = dtype == MLA_DTYPE_FP8_E4M3 ? 1 : 2;
  return (size_t)(d->kv_lora_rank + d->qk_rope_head_dim) * e + (dtype == MLA_DTYPE_FP8_E4M3 ? 4 : 0);
}

mla_status launch_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int32_t split_chunk(int32_t max_seq_len, int32_t num_splits) {
  const int64_t per = ((int64_t)max_seq_len + num_splits - 1) / num_splits;
  return (int32_t)(((per + 31) / 32) * 32);
}

// Checks of a cache description read by decode (shared by mla_decode_latent and
// mla_decode_step_fused).
mla_status check_read_cache(const mla_dims* dims, const mla_cache* cache, int32_t max_seq_len, const char* where) {
  if (cache->dtype != MLA_DTYPE_BF16 && cache->dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "mla_cache.dtype %d unknown (%s)", cache->dtype, where);
  const bool fp8 = cache->dtype == MLA_DTYPE_FP8_E4M3;
  // 16-byte copies: row strides must be multiples of 16 bytes
  const int64_t stride_align = fp8 ? 16 : 8;
  REQUIRE_PTR(cache->kv, "mla_cache.kv", where);
  REQUIRE_PTR(cache->pe, "mla_cache.pe", where);
  if (cache->kv_stride < dims->kv_lora_rank || cache->kv_stride % stride_align != 0)
    return fail(MLA_ERR_BUFFER, "mla_cache.kv_stride %lld must be >= %d and a multiple of %lld elements (%s)",
                (long long)cache->kv_stride, dims->kv_lora_rank, (long long)stride_align, where);
  if (cache->pe_stride < dims->qk_rope_head_dim || cache->pe_stride % stride_align != 0)
    return fail(MLA_ERR_BUFFER, "mla_cache.pe_stride %lld must be >= %d and a multiple of %lld elements (%s)",
                (long long)cache->pe_stride, dims->qk_rope_head_dim, (long long)stride_align, where);
  // the kernels address the rows of one 32-token tile with 32-bit offsets
  if (cache->kv_stride > (int64_t)1 << 23 || cache->pe_stride > (int64_t)1 << 23)
    return fail(MLA_ERR_BUFFER, "mla_cache.kv_stride %lld / pe_stride %lld above %lld elements (%s)",
                (long long)cache->kv_stride, (long long)cache->pe_stride, (long long)1 << 23, where);
  if (fp8) {
    if (cache->token_scale == nullptr)
      return fail(MLA_ERR_NULL, "mla_cache.token_scale is NULL (E4M3 cache needs one fp32 scale per slot, %s)", where);
    if (reinterpret_cast<uintptr_t>(cache->token_scale) % 4 != 0)
      return fail(MLA_ERR_ALIGN, "mla_cache.token_scale is not 4-byte aligned (%s)", where);
  } else if (cache->token_scale != nullptr) {
    return fail(MLA_ERR_BUFFER, "mla_cache.token_scale must be NULL for a bf16 cache (%s)", where);
  }
  if (max_seq_len < 1) return fail(MLA_ERR_BAD_LENGTH, "max_seq_len %d < 1 (%s)", max_seq_len, where);
  if (cache->block_table != nullptr) {
    if (cache->block_size <= 0 || cache->block_size % 32 != 0)
      return fail(MLA_ERR_BAD_LENGTH, "mla_cache.block_size %d must be a positive multiple of 32 (%s)",
                  cache->block_size, where);
    const int64_t need = ((int64_t)max_seq_len + cache->block_size - 1) / cache->block_size;
    if (cache->max_blocks_per_seq < need)
      return fail(MLA_ERR_BUFFER, "mla_cache.max_blocks_per_seq %d < %lld blocks for max_seq_len %d (%s)",
                  cache->max_blocks_per_seq, (long long)need, max_seq_len, where);
  } else {
    if (cache->seq_stride < max_seq_len)
      return fail(MLA_ERR_BUFFER, "mla_cache.seq_stride %lld < max_seq_len %d (contiguous cache, %s)",
                  (long long)cache->seq_stride, max_seq_len, where);
  }
  return MLA_OK;
}

// Latent attention for decode (one query row per sequence, lengths from
// seq_lens) or a prefill chunk (q_per_seq query rows per sequence, causal
// lengths from q_start); the caller has checked the mode-specific arguments.
mla_status latent_attention_rows(const char* where, const mla_dims* dims, const mla_cache* cache, const void* q_lat,
                                 const void* q_pe, const int32_t* seq_lens, const int32_t* q_start,
                                 int32_t q_per_seq, int32_t max_seq_len, int32_t num_splits, void* o_part,
                                 float* lse_part, void* o_lat, float* lse, void* stream,
                                 const int32_t* items = nullptr, int32_t num_items = 0) {
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (cache == nullptr) return fail(MLA_ERR_NULL, "cache is NULL (%s)", where);
  st = check_read_cache(dims, cache, max_seq_len, where);
  if (st != MLA_OK) return st;
  const bool fp8 = cache->dtype == MLA_DTYPE_FP8_E4M3;
  REQUIRE_PTR(q_lat, "q_lat", where);
  REQUIRE_PTR(q_pe, "q_pe", where);
  if (q_start == nullptr && seq_lens == nullptr) return fail(MLA_ERR_NULL, "seq_lens is NULL (%s)", where);
  if (num_splits < 1) return fail(MLA_ERR_BAD_LENGTH, "num_splits %d < 1 (%s)", num_splits, where);
  const int64_t rows = (int64_t)dims->batch * q_per_seq;
  if (rows * num_splits > (int64_t)1 << 30)
    return fail(MLA_ERR_BAD_LENGTH, "query rows * num_splits too large (%s)", where);
  if (num_splits == 1) {
    REQUIRE_PTR(o_lat, "o_lat", where);
    if (lse == nullptr) return fail(MLA_ERR_NULL, "lse is NULL (%s)", where);
    if (o_part != nullptr || lse_part != nullptr)
      return fail(MLA_ERR_BUFFER, "o_part/lse_part must be NULL when num_splits == 1 (%s)", where);
  } else {
    REQUIRE_PTR(o_part, "o_part", where);
    if (lse_part == nullptr) return fail(MLA_ERR_NULL, "lse_part is NULL (%s)", where);
    if (o_lat != nullptr || lse != nullptr)
      return fail(MLA_ERR_BUFFER, "o_lat/lse must be NULL when num_splits > 1; merge with mla_combine_splits (%s)",
                  where);
  }

  mla::DecodeArgs a{};
  a.q_lat = static_cast<const uint16_t*>(q_lat);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.kv = static_cast<const char*>(cache->kv);
  a.pe = static_cast<const char*>(cache->pe);
  a.kv_sb = cache->kv_stride * (fp8 ? 1 : 2);
  a.pe_sb = cache->pe_stride * (fp8 ? 1 : 2);
  a.token_scale = cache->token_scale;
  a.fp8 = fp8 ? 1 : 0;
  a.seq_stride = cache->seq_stride;
  a.block_table = cache->block_table;
  a.block_size = cache->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.q_per_seq = q_per_seq;
  a.q_start = q_start;
  // prefill chunks with fewer than 128 heads: 128 / H queries share a workgroup
  a.q_group = (q_start != nullptr && !fp8 && num_splits == 1 && dims->num_heads < 128) ? 128 / dims->num_heads : 1;
  a.batch = (int32_t)rows;
  a.num_heads = dims->num_heads;
  a.num_splits = num_splits;
  a.chunk = split_chunk(max_seq_len, num_splits);
  a.max_seq_len = max_seq_len;
  a.scale = dims->softmax_scale;
  a.scale_log2 = dims->softmax_scale * 1.4426950408889634f;
  a.o_part = static_cast<uint16_t*>(o_part);
  a.lse_part = lse_part;
  a.o_lat = static_cast<uint16_t*>(o_lat);
  a.lse = lse;
  a.items = items;
  a.num_items = num_items;
  return launch_result(mla::launch_decode_latent(a, static_cast<hipStream_t>(stream)), where);
}

// Workgroups of the bf16 decode kernel resident per CU, as its LDS allows:
// 16 heads, a ring of four 36 KiB tiles: 1; 32 heads, two waves with one
// buffer: 4; 64 heads, four waves with two buffers: 2; the 128-head kernel
// holds a whole CU.
int wg_per_cu(int num_heads) {
  return num_heads >= 128 ? 1 : (num_heads >= 64 ? 2 : (num_heads >= 32 ? 4 : 1));
}

// Shortest split: 1/32 of the context, within [32, 256] tokens (each split
// pays a fixed prologue and epilogue and one more partial to merge).
int64_t min_split_tokens(int32_t max_seq_len) {
  int64_t m = max_seq_len / 32;
  return m < 32 ? 32 : (m > 256 ? 256 : m);
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_err; }

const char* mla_version(void) { return "mla_absorb gfx950 0.1"; }

mla_status mla_kv_cache_bytes(const mla_dims* dims, int32_t dtype, size_t* bytes) {
  mla_status st = check_latent_dims(dims, "mla_kv_cache_bytes");
  if (st != MLA_OK) return st;
  if (bytes == nullptr) return fail(MLA_ERR_NULL, "bytes_per_token is NULL (mla_kv_cache_bytes)");
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d unknown (mla_kv_cache_bytes)", dtype);
  *bytes = bytes_per_token(dims, dtype);
  return ok();
}

mla_status mla_decode_kv_read_bytes(const mla_dims* dims, int32_t dtype, const int32_t* host_seq_lens,
                                    size_t* bytes) {
  mla_status st = check_latent_dims(dims, "mla_decode_kv_read_bytes");
  if (st != MLA_OK) return st;
  if (dims->batch <= 0) return fail(MLA_ERR_MISSING_DIM, "batch missing (mla_dims, mla_decode_kv_read_bytes)");
  if (host_seq_lens == nullptr) return fail(MLA_ERR_NULL, "host_seq_lens is NULL (mla_decode_kv_read_bytes)");
  if (bytes == nullptr) return fail(MLA_ERR_NULL, "bytes is NULL (mla_decode_kv_read_bytes)");
  if (dtype != MLA_DTYPE_BF16 && dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "dtype %d unknown (mla_decode_kv_read_bytes)", dtype);
  size_t tokens = 0;
  for (int32_t b = 0; b < dims->batch; ++b) {
    if (host_seq_lens[b] < 0)
      return fail(MLA_ERR_BAD_LENGTH, "host_seq_lens[%d] = %d is negative (mla_decode_kv_read_bytes)", b,
                  host_seq_lens[b]);
    tokens += (size_t)host_seq_lens[b];
  }
  *bytes = tokens * bytes_per_token(dims, dtype);
  return ok();
}

mla_status mla_absorb_q(const mla_dims* dims, const void* q_nope, const void* w_uk, void* q_lat, void* stream) {
  const char* where = "mla_absorb_q";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  REQUIRE_PTR(q_nope, "q_nope", where);
  REQUIRE_PTR(w_uk, "w_uk", where);
  REQUIRE_PTR(q_lat, "q_lat", where);
  mla::ProjArgs a{static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(w_uk),
                  static_cast<uint16_t*>(q_lat), dims->batch, dims->num_heads};
  return launch_result(mla::launch_absorb_q(a, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_expand_v(const mla_dims* dims, const void* o_lat, const void* w_uv, void* out, void* stream) {
  const char* where = "mla_expand_v";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  REQUIRE_PTR(o_lat, "o_lat", where);
  REQUIRE_PTR(w_uv, "w_uv", where);
  REQUIRE_PTR(out, "out", where);
  mla::ProjArgs a{static_cast<const uint16_t*>(o_lat), static_cast<const uint16_t*>(w_uv),
                  static_cast<uint16_t*>(out), dims->batch, dims->num_heads};
  return launch_result(mla::launch_expand_v(a, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_combine_splits(const mla_dims* dims, const void* o_part, const float* lse_part, int32_t num_splits,
                              void* o_lat, float* lse, void* stream) {
  const char* where = "mla_combine_splits";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_BAD_LENGTH, "num_splits %d < 1 (%s)", num_splits, where);
  REQUIRE_PTR(o_part, "o_part", where);
  if (lse_part == nullptr) return fail(MLA_ERR_NULL, "lse_part is NULL (%s)", where);
  REQUIRE_PTR(o_lat, "o_lat", where);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  mla::CombineArgs a{static_cast<const uint16_t*>(o_part), lse_part, static_cast<uint16_t*>(o_lat), lse, dims->batch, dims->num_heads,
                     num_splits};
  return launch_result(mla::launch_combine(a, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_combine_expand_v(const mla_dims* dims, const void* o_part, const float* lse_part, int32_t num_splits,
                                const void* w_uv, void* out, void* o_lat, float* lse, void* stream) {
  const char* where = "mla_combine_expand_v";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_BAD_LENGTH, "num_splits %d < 1 (%s)", num_splits, where);
  REQUIRE_PTR(o_part, "o_part", where);
  if (lse_part == nullptr) return fail(MLA_ERR_NULL, "lse_part is NULL (%s)", where);
  REQUIRE_PTR(w_uv, "w_uv", where);
  REQUIRE_PTR(out, "out", where);
  if (o_lat != nullptr && (reinterpret_cast<uintptr_t>(o_lat) & 15u))
    return fail(MLA_ERR_ALIGN, "o_lat is not 16-byte aligned (%s)", where);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  mla::CombineExpandArgs a{static_cast<const uint16_t*>(o_part), lse_part, static_cast<const uint16_t*>(w_uv),
                           static_cast<uint16_t*>(out), static_cast<uint16_t*>(o_lat), lse, dims->batch,
                           dims->num_heads, num_splits};
  return launch_result(mla::launch_combine_expand(a, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_decode_latent(const mla_dims* dims, const mla_cache* cache, const void* q_lat, const void* q_pe,
                             const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, void* o_part,
                             float* lse_part, void* o_lat, float* lse, void* stream) {
  const char* where = "mla_decode_latent";
  return latent_attention_rows(where, dims, cache, q_lat, q_pe, seq_lens, nullptr, 1, max_seq_len, num_splits, o_part,
                               lse_part, o_lat, lse, stream);
}

mla_status mla_decode_latent_noalloc(const mla_dims* dims, const mla_cache* cache, const void* q_lat, const void* q_pe,
                                     const int32_t* seq_lens, int32_t max_seq_len, int32_t num_splits, void* o_lat,
                                     float* lse, void* stream) {
  const char* where = "mla_decode_latent_noalloc";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (num_splits < 1) return fail(MLA_ERR_BAD_LENGTH, "num_splits %d < 1 (%s)", num_splits, where);
  REQUIRE_PTR(o_lat, "o_lat", where);
  if (lse == nullptr) return fail(MLA_ERR_NULL, "lse is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  if (num_splits == 1)  // no partials: straight to o_lat / lse
    return latent_attention_rows(where, dims, cache, q_lat, q_pe, seq_lens, nullptr, 1, max_seq_len, 1, nullptr,
                                 nullptr, o_lat, lse, stream);
  // partials [B, P, H, 512] bf16, then lse [B, P, H] fp32 (256-byte aligned)
  const size_t rows = (size_t)dims->batch * (size_t)num_splits * (size_t)dims->num_heads;
  const size_t part_bytes = ((rows * dims->kv_lora_rank * 2 + 255) / 256) * 256;
  const size_t need = part_bytes + rows * 4;
  if (need > mla::kScratchBytes)
    return fail(MLA_ERR_BUFFER,
                "batch * num_splits * num_heads = %zu needs %zu bytes of split partials, above the %zu-byte "
                "device scratch of %s (use fewer splits, or mla_decode_latent with caller buffers)",
                rows, need, mla::kScratchBytes, where);
  void* base = nullptr;
  const hipError_t e = mla::scratch_region(&base);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "device scratch lookup failed: %s (%s)", hipGetErrorString(e), where);
  void* o_part = base;
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(base) + part_bytes);
  st = latent_attention_rows(where, dims, cache, q_lat, q_pe, seq_lens, nullptr, 1, max_seq_len, num_splits, o_part,
                             lse_part, nullptr, nullptr, stream);
  if (st != MLA_OK) return st;
  mla::CombineArgs c{static_cast<const uint16_t*>(o_part), lse_part, static_cast<uint16_t*>(o_lat), lse, dims->batch,
                     dims->num_heads, num_splits};
  return launch_result(mla::launch_combine(c, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_prefill_latent(const mla_dims* dims, const mla_cache* cache, const void* q_lat, const void* q_pe,
                              const int32_t* q_start, int32_t num_q, int32_t max_seq_len, int32_t num_splits,
                              void* o_part, float* lse_part, void* o_lat, float* lse, void* stream) {
  const char* where = "mla_prefill_latent";
  if (num_q < 1) return fail(MLA_ERR_BAD_LENGTH, "num_q %d < 1 (%s)", num_q, where);
  if (q_start == nullptr) return fail(MLA_ERR_NULL, "q_start is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(q_start) % 4 != 0)
    return fail(MLA_ERR_ALIGN, "q_start is not 4-byte aligned (%s)", where);
  return latent_attention_rows(where, dims, cache, q_lat, q_pe, nullptr, q_start, num_q, max_seq_len, num_splits,
                               o_part, lse_part, o_lat, lse, stream);
}

mla_status mla_decode_step_fused(const mla_dims* dims, const mla_cache* cache, const void* q_nope, const void* q_pe,
                                 const void* w_uk, const void* w_uv, const int32_t* seq_lens, int32_t max_seq_len,
                                 void* out, void* o_lat, float* lse, void* stream) {
  const char* where = "mla_decode_step_fused";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (cache == nullptr) return fail(MLA_ERR_NULL, "cache is NULL (%s)", where);
  st = check_read_cache(dims, cache, max_seq_len, where);
  if (st != MLA_OK) return st;
  REQUIRE_PTR(q_nope, "q_nope", where);
  REQUIRE_PTR(q_pe, "q_pe", where);
  REQUIRE_PTR(w_uk, "w_uk", where);
  REQUIRE_PTR(w_uv, "w_uv", where);
  if (seq_lens == nullptr) return fail(MLA_ERR_NULL, "seq_lens is NULL (%s)", where);
  REQUIRE_PTR(out, "out", where);
  if (o_lat != nullptr && !aligned16(o_lat)) return fail(MLA_ERR_ALIGN, "o_lat is not 16-byte aligned (%s)", where);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  if ((int64_t)dims->batch * dims->num_heads > (int64_t)1 << 30)
    return fail(MLA_ERR_BAD_LENGTH, "batch * num_heads too large (%s)", where);
  const bool fp8 = cache->dtype == MLA_DTYPE_FP8_E4M3;
  mla::FusedStepArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.kv = static_cast<const char*>(cache->kv);
  a.pe = static_cast<const char*>(cache->pe);
  a.kv_sb = cache->kv_stride * (fp8 ? 1 : 2);
  a.pe_sb = cache->pe_stride * (fp8 ? 1 : 2);
  a.seq_stride = cache->seq_stride;
  a.block_table = cache->block_table;
  a.block_size = cache->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  a.token_scale = cache->token_scale;
  a.seq_lens = seq_lens;
  a.batch = dims->batch;
  a.num_heads = dims->num_heads;
  a.max_seq_len = max_seq_len;
  a.scale_log2 = dims->softmax_scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.o_lat = static_cast<uint16_t*>(o_lat);
  a.lse = lse;
  return launch_result(mla::launch_decode_step_fused(a, fp8, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_naive_workspace_bytes(const mla_dims* dims, int32_t max_seq_len, size_t* bytes) {
  const char* where = "mla_naive_workspace_bytes";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (bytes == nullptr) return fail(MLA_ERR_NULL, "bytes is NULL (%s)", where);
  if (max_seq_len < 1) return fail(MLA_ERR_BAD_LENGTH, "max_seq_len %d < 1 (%s)", max_seq_len, where);
  *bytes = (size_t)dims->batch * (size_t)max_seq_len * (size_t)dims->num_heads * (dims->qk_nope_head_dim + dims->v_head_dim) * 2;
  return ok();
}

mla_status mla_naive_decode(const mla_dims* dims, const mla_cache* cache, const void* q_nope, const void* q_pe,
                            const void* w_uk, const void* w_uv, const int32_t* seq_lens, int32_t max_seq_len,
                            void* workspace, size_t workspace_bytes, void* out, void* stream) {
  const char* where = "mla_naive_decode";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (cache == nullptr) return fail(MLA_ERR_NULL, "cache is NULL (%s)", where);
  st = check_read_cache(dims, cache, max_seq_len, where);
  if (st != MLA_OK) return st;
  REQUIRE_PTR(q_nope, "q_nope", where);
  REQUIRE_PTR(q_pe, "q_pe", where);
  REQUIRE_PTR(w_uk, "w_uk", where);
  REQUIRE_PTR(w_uv, "w_uv", where);
  if (seq_lens == nullptr) return fail(MLA_ERR_NULL, "seq_lens is NULL (%s)", where);
  REQUIRE_PTR(workspace, "workspace", where);
  REQUIRE_PTR(out, "out", where);
  const size_t need = (size_t)dims->batch * (size_t)max_seq_len * (size_t)dims->num_heads * 256 * 2;
  if (workspace_bytes < need)
    return fail(MLA_ERR_BUFFER, "workspace_bytes %zu < %zu needed (B * max_seq_len * H * 256 bf16, %s)",
                workspace_bytes, need, where);
  if (dims->batch > 65535) return fail(MLA_ERR_BAD_LENGTH, "batch %d above 65535 (%s)", dims->batch, where);
  const bool fp8 = cache->dtype == MLA_DTYPE_FP8_E4M3;
  mla::NaiveArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.kv = static_cast<const char*>(cache->kv);
  a.pe = static_cast<const char*>(cache->pe);
  a.kv_sb = cache->kv_stride * (fp8 ? 1 : 2);
  a.pe_sb = cache->pe_stride * (fp8 ? 1 : 2);
  a.seq_stride = cache->seq_stride;
  a.block_table = cache->block_table;
  a.block_size = cache->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  a.token_scale = cache->token_scale;
  a.seq_lens = seq_lens;
  a.batch = dims->batch;
  a.num_heads = dims->num_heads;
  a.max_seq_len = max_seq_len;
  a.scale_log2 = dims->softmax_scale * 1.4426950408889634f;
  a.ws = static_cast<uint16_t*>(workspace);
  a.out = static_cast<uint16_t*>(out);
  return launch_result(mla::launch_naive_decode(a, fp8, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_cache_append(const mla_dims* dims, const mla_cache* cache, const void* kv_in, int64_t in_stride,
                            const int32_t* positions, int32_t num_new, float rope_base, void* stream) {
  const char* where = "mla_cache_append";
  mla_status st = check_latent_dims(dims, where);
  if (st != MLA_OK) return st;
  if (dims->batch <= 0) return fail(MLA_ERR_MISSING_DIM, "batch missing (mla_dims, %s)", where);
  if (dims->kv_lora_rank != 512)
    return fail(MLA_ERR_UNSUPPORTED, "kv_lora_rank %d not supported, built for 512 (%s)", dims->kv_lora_rank, where);
  if (dims->qk_rope_head_dim != 64)
    return fail(MLA_ERR_UNSUPPORTED, "qk_rope_head_dim %d not supported, built for 64 (%s)", dims->qk_rope_head_dim,
                where);
  if (rope_base == 0.0f) return fail(MLA_ERR_MISSING_DIM, "rope_base missing (%s)", where);
  if (!(rope_base > 0.0f) || !std::isfinite(rope_base))
    return fail(MLA_ERR_UNSUPPORTED, "rope_base must be positive and finite (%s)", where);
  if (cache == nullptr) return fail(MLA_ERR_NULL, "cache is NULL (%s)", where);
  if (cache->dtype != MLA_DTYPE_BF16 && cache->dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "mla_cache.dtype %d unknown (%s)", cache->dtype, where);
  const bool fp8 = cache->dtype == MLA_DTYPE_FP8_E4M3;
  const int64_t stride_align = fp8 ? 16 : 8;
  REQUIRE_PTR(cache->kv, "mla_cache.kv", where);
  REQUIRE_PTR(cache->pe, "mla_cache.pe", where);
  if (cache->kv_stride < dims->kv_lora_rank || cache->kv_stride % stride_align != 0)
    return fail(MLA_ERR_BUFFER, "mla_cache.kv_stride %lld must be >= %d and a multiple of %lld elements (%s)",
                (long long)cache->kv_stride, dims->kv_lora_rank, (long long)stride_align, where);
  if (cache->pe_stride < dims->qk_rope_head_dim || cache->pe_stride % stride_align != 0)
    return fail(MLA_ERR_BUFFER, "mla_cache.pe_stride %lld must be >= %d and a multiple of %lld elements (%s)",
                (long long)cache->pe_stride, dims->qk_rope_head_dim, (long long)stride_align, where);
  if (fp8) {
    if (cache->token_scale == nullptr)
      return fail(MLA_ERR_NULL, "mla_cache.token_scale is NULL (E4M3 cache needs one fp32 scale per slot, %s)", where);
    if (reinterpret_cast<uintptr_t>(cache->token_scale) % 4 != 0)
      return fail(MLA_ERR_ALIGN, "mla_cache.token_scale is not 4-byte aligned (%s)", where);
  } else if (cache->token_scale != nullptr) {
    return fail(MLA_ERR_BUFFER, "mla_cache.token_scale must be NULL for a bf16 cache (%s)", where);
  }
  if (cache->block_table != nullptr) {
    if (reinterpret_cast<uintptr_t>(cache->block_table) % 4 != 0)
      return fail(MLA_ERR_ALIGN, "mla_cache.block_table is not 4-byte aligned (%s)", where);
    if (cache->block_size <= 0)
      return fail(MLA_ERR_BAD_LENGTH, "mla_cache.block_size %d must be positive (%s)", cache->block_size, where);
    if (cache->max_blocks_per_seq <= 0)
      return fail(MLA_ERR_BUFFER, "mla_cache.max_blocks_per_seq %d must be positive (%s)", cache->max_blocks_per_seq,
                  where);
  } else if (cache->seq_stride <= 0) {
    return fail(MLA_ERR_BUFFER, "mla_cache.seq_stride %lld must be positive (contiguous cache, %s)",
                (long long)cache->seq_stride, where);
  }
  if (num_new < 0) return fail(MLA_ERR_BAD_LENGTH, "num_new %d < 0 (%s)", num_new, where);
  if ((int64_t)dims->batch * num_new > (int64_t)1 << 31)
    return fail(MLA_ERR_BAD_LENGTH, "batch * num_new above 2^31 rows (%s)", where);
  REQUIRE_PTR(kv_in, "kv_in", where);
  const int64_t row_width = dims->kv_lora_rank + dims->qk_rope_head_dim;
  if (in_stride < row_width || in_stride % 8 != 0)
    return fail(MLA_ERR_BUFFER, "in_stride %lld must be >= %lld and a multiple of 8 elements (%s)",
                (long long)in_stride, (long long)row_width, where);
  if (positions == nullptr) return fail(MLA_ERR_NULL, "positions is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(positions) % 4 != 0)
    return fail(MLA_ERR_ALIGN, "positions is not 4-byte aligned (%s)", where);
  if (num_new == 0) return ok();

  mla::AppendArgs a{};
  a.kv_in = static_cast<const uint16_t*>(kv_in);
  a.in_stride = in_stride;
  a.positions = positions;
  a.batch = dims->batch;
  a.num_new = num_new;
  // the cache description is shared with decode, which only reads it
  a.kv = const_cast<char*>(static_cast<const char*>(cache->kv));
  a.pe = const_cast<char*>(static_cast<const char*>(cache->pe));
  a.kv_sb = cache->kv_stride * (fp8 ? 1 : 2);
  a.pe_sb = cache->pe_stride * (fp8 ? 1 : 2);
  a.token_scale = const_cast<float*>(cache->token_scale);
  a.seq_stride = cache->seq_stride;
  a.block_table = cache->block_table;
  a.block_size = cache->block_size;
  a.max_blocks = cache->max_blocks_per_seq;
  // pair i turns by position * base^(-2i/64); the exponent -2i/64 is exact
  for (int i = 0; i < 32; ++i) a.inv_freq[i] = std::pow((double)rope_base, -(double)(2 * i) / 64.0);
  return launch_result(mla::launch_cache_append(a, fp8, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_plan_decode_splits(const mla_dims* dims, const int32_t* host_seq_lens, int32_t max_seq_len,
                                  int32_t num_cus, int32_t capacity, int32_t* items, int32_t* seq_first,
                                  int32_t* num_items) {
  const char* where = "mla_plan_decode_splits";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (host_seq_lens == nullptr) return fail(MLA_ERR_NULL, "host_seq_lens is NULL (%s)", where);
  if (items == nullptr || seq_first == nullptr || num_items == nullptr)
    return fail(MLA_ERR_NULL, "items / seq_first / num_items is NULL (%s)", where);
  if (max_seq_len < 1) return fail(MLA_ERR_BAD_LENGTH, "max_seq_len %d < 1 (%s)", max_seq_len, where);
  if (num_cus < 1) return fail(MLA_ERR_BAD_LENGTH, "num_cus %d < 1 (%s)", num_cus, where);
  const int B = dims->batch;
  // 32-token tiles per sequence (lengths clamped to [0, max_seq_len] as the kernels do)
  auto tiles_of = [&](int b) -> int64_t {
    const int64_t t = host_seq_lens[b] < 0 ? 0 : (host_seq_lens[b] > max_seq_len ? max_seq_len : host_seq_lens[b]);
    return (t + 31) / 32;
  };
  int64_t max_tiles = 0, total_tiles = 0;
  for (int b = 0; b < B; ++b) {
    max_tiles = std::max<int64_t>(max_tiles, tiles_of(b));
    total_tiles += tiles_of(b);
  }
  auto items_for = [&](int64_t per) -> int64_t {  // items when no item exceeds `per` tiles
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += std::max<int64_t>(1, (tiles_of(b) + per - 1) / per);
    return n;
  };
  // Resident workgroup slots; a budget below the shortest useful split is never used.
  const int64_t slots = std::max<int64_t>((int64_t)num_cus * wg_per_cu(dims->num_heads), 1);
  const int64_t lo = std::max<int64_t>(1, (min_split_tokens(max_seq_len) + 31) / 32);
  // One round: the fewest tiles per item such that every item has a slot.
  int64_t one_round;
  {
    int64_t l = lo, h = std::max<int64_t>(lo, max_tiles);
    const int64_t cap = std::max<int64_t>(slots, B);
    while (l < h) {
      const int64_t mid = l + (h - l) / 2;
      if (items_for(mid) <= cap) h = mid;
      else l = mid + 1;
    }
    one_round = l;
  }
  // Items of a budget: each sequence's tiles in near-equal consecutive items
  // (sizes differ by at most one tile), partial rows in sequence order.
  struct Item {
    int32_t seq, first, count, slot;
  };
  std::vector<Item> cand, best;
  auto build = [&](int64_t per, std::vector<Item>& out) {
    out.clear();
    int32_t k = 0;
    for (int b = 0; b < B; ++b) {
      const int64_t tiles = tiles_of(b);
      const int64_t n = std::max<int64_t>(1, (tiles + per - 1) / per);
      int64_t first = 0;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t cnt = tiles / n + (i < tiles % n ? 1 : 0);
        out.push_back({b, (int32_t)first, (int32_t)cnt, k++});
        first += cnt;
      }
    }
    // launch order: longest first (ties in sequence order)
    std::stable_sort(out.begin(), out.end(), [](const Item& x, const Item& y) { return x.count > y.count; });
  };
  // Predicted launch time of an item order, in tiles: workgroup i goes to XCD
  // i % 8, and each XCD starts its next item on the first of its slots to
  // free up; an item costs its tiles plus a fixed kItemCost (prologue,
  // epilogue, partial row).
  constexpr int64_t kItemCost = 4;
  std::vector<int64_t> heap;
  auto makespan = [&](const std::vector<Item>& order) -> int64_t {
    const int64_t groups = slots % 8 == 0 ? 8 : 1;
    const int64_t per_group = slots / groups;
    int64_t worst = 0;
    for (int64_t x = 0; x < groups; ++x) {
      heap.assign((size_t)per_group, 0);  // all zero: a valid min-heap
      for (size_t i = (size_t)x; i < order.size(); i += (size_t)groups) {
        std::pop_heap(heap.begin(), heap.end(), std::greater<int64_t>());
        heap.back() += kItemCost + order[i].count;
        std::push_heap(heap.begin(), heap.end(), std::greater<int64_t>());
      }
      worst = std::max(worst, *std::max_element(heap.begin(), heap.end()));
    }
    return worst;
  };
  // Candidate budgets: the one-round budget and ~m items per slot on average
  // for m = 1.1 .. 3.0; the lowest predicted time wins (ties: fewer items).
  int64_t best_time = -1;
  auto consider = [&](int64_t per) {
    per = std::max(lo, std::min(per, std::max<int64_t>(lo, max_tiles)));
    if (items_for(per) > capacity) return;
    build(per, cand);
    const int64_t t = makespan(cand);
    if (best_time < 0 || t < best_time || (t == best_time && cand.size() < best.size())) {
      best_time = t;
      best.swap(cand);
    }
  };
  consider(one_round);
  for (int m10 = 11; m10 <= 30; ++m10) consider((10 * total_tiles + slots * m10 - 1) / (slots * m10));
  if (best_time < 0)
    return fail(MLA_ERR_BUFFER, "the plan has %lld items, above capacity %d (%s)", (long long)items_for(one_round),
                capacity, where);
  // merge map: sequence b's partial rows are seq_first[b] .. seq_first[b + 1] - 1
  std::vector<int32_t> count_of(B, 0);
  for (const Item& it : best) ++count_of[it.seq];
  seq_first[0] = 0;
  for (int b = 0; b < B; ++b) seq_first[b + 1] = seq_first[b] + count_of[b];
  for (size_t i = 0; i < best.size(); ++i) {
    items[4 * i] = best[i].seq;
    items[4 * i + 1] = best[i].first;
    items[4 * i + 2] = best[i].count;
    items[4 * i + 3] = best[i].slot;
  }
  *num_items = (int32_t)best.size();
  return ok();
}

mla_status mla_decode_latent_planned(const mla_dims* dims, const mla_cache* cache, const void* q_lat, const void* q_pe,
                                     const int32_t* seq_lens, int32_t max_seq_len, const int32_t* items,
                                     int32_t num_items, void* o_part, float* lse_part, void* stream) {
  const char* where = "mla_decode_latent_planned";
  if (items == nullptr) return fail(MLA_ERR_NULL, "items is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(items) & 3u) return fail(MLA_ERR_ALIGN, "items is not 4-byte aligned (%s)", where);
  if (num_items < 1 || num_items > (1 << 30))
    return fail(MLA_ERR_BAD_LENGTH, "num_items %d outside [1, 2^30] (%s)", num_items, where);
  // num_splits > 1 selects the partial outputs in the shared checks
  return latent_attention_rows(where, dims, cache, q_lat, q_pe, seq_lens, nullptr, 1, max_seq_len, 2, o_part,
                               lse_part, nullptr, nullptr, stream, items, num_items);
}

mla_status mla_combine_splits_planned(const mla_dims* dims, const void* o_part, const float* lse_part,
                                      const int32_t* seq_first, int32_t num_items, void* o_lat, float* lse,
                                      void* stream) {
  const char* where = "mla_combine_splits_planned";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (num_items < 1) return fail(MLA_ERR_BAD_LENGTH, "num_items %d < 1 (%s)", num_items, where);
  REQUIRE_PTR(o_part, "o_part", where);
  if (lse_part == nullptr) return fail(MLA_ERR_NULL, "lse_part is NULL (%s)", where);
  if (seq_first == nullptr) return fail(MLA_ERR_NULL, "seq_first is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(seq_first) & 3u)
    return fail(MLA_ERR_ALIGN, "seq_first is not 4-byte aligned (%s)", where);
  REQUIRE_PTR(o_lat, "o_lat", where);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  mla::CombineArgs a{static_cast<const uint16_t*>(o_part), lse_part, static_cast<uint16_t*>(o_lat), lse, dims->batch,
                     dims->num_heads, num_items, seq_first};
  return launch_result(mla::launch_combine(a, static_cast<hipStream_t>(stream)), where);
}

mla_status mla_combine_expand_v_planned(const mla_dims* dims, const void* o_part, const float* lse_part,
                                        const int32_t* seq_first, int32_t num_items, const void* w_uv, void* out,
                                        void* o_lat, float* lse, void* stream) {
  const char* where = "mla_combine_expand_v_planned";
  mla_status st = check_dims(dims, where);
  if (st != MLA_OK) return st;
  if (num_items < 1) return fail(MLA_ERR_BAD_LENGTH, "num_items %d < 1 (%s)", num_items, where);
  REQUIRE_PTR(o_part, "o_part", where);
  if (lse_part == nullptr) return fail(MLA_ERR_NULL, "lse_part is NULL (%s)", where);
  if (seq_first == nullptr) return fail(MLA_ERR_NULL, "seq_first is NULL (%s)", where);
  if (reinterpret_cast<uintptr_t>(seq_first) & 3u)
    return fail(MLA_ERR_ALIGN, "seq_first is not 4-byte aligned (%s)", where);
  REQUIRE_PTR(w_uv, "w_uv", where);
  REQUIRE_PTR(out, "out", where);
  if (o_lat != nullptr && (reinterpret_cast<uintptr_t>(o_lat) & 15u))
    return fail(MLA_ERR_ALIGN, "o_lat is not 16-byte aligned (%s)", where);
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(MLA_ERR_ALIGN, "lse is not 4-byte aligned (%s)", where);
  mla::CombineExpandArgs a{static_cast<const uint16_t*>(o_part), lse_part, static_cast<const uint16_t*>(w_uv),
                           static_cast<uint16_t*>(out), static_cast<uint16_t*>(o_lat), lse, dims->batch,
                           dims->num_heads, num_items, 0, seq_first};
  return launch_result(mla::launch_combine_expand(a, static_cast<hipStream_t>(stream)), where);
}

int32_t mla_recommended_splits(const mla_dims* dims, int32_t max_seq_len, int32_t num_cus) {
  if (dims == nullptr || dims->batch <= 0 || dims->num_heads <= 0 || max_seq_len <= 0 || num_cus <= 0) return 1;
  const int64_t want = (int64_t)num_cus * wg_per_cu(dims->num_heads);
  int64_t p = (want + dims->batch - 1) / dims->batch;
  // short splits keep few sequences busy, but each pays a fixed cost
  const int64_t min_tokens = min_split_tokens(max_seq_len);
  const int64_t max_p = (max_seq_len + min_tokens - 1) / min_tokens;
  if (p > max_p) p = max_p;
  if (p < 1) p = 1;
  return (int32_t)p;
}

}  // extern "C"
