// Kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
  const uint16_t* q_lat;      // [B, H, 512] bf16
  const uint16_t* q_pe;       // [B, H, 64] bf16
  const char* kv;             // latent element 0 of slot 0
  const char* pe;             // rope element 0 of slot 0
  int64_t kv_sb;              // bytes between consecutive slots (kv)
  int64_t pe_sb;              // bytes between consecutive slots (pe)
  int64_t seq_stride;         // contiguous: slots per sequence
  const int32_t* block_table; // paged: [B, max_blocks]; null = contiguous
  int32_t block_size;
  int32_t max_blocks;
  const float* token_scale;   // E4M3 cache: one fp32 scale per slot (else null)
  int32_t fp8;                // cache holds OCP E4M3 codes
  const int32_t* seq_lens;    // [B]
  int32_t q_per_seq;          // query rows per cached sequence: 1 (decode) or L (prefill chunk)
  const int32_t* q_start;     // prefill: [B] position of each sequence's first query; null: decode
  int32_t q_group;            // prefill with H < 128 heads (wide kernel, one split): consecutive
                              // queries per workgroup, 128 / H (128 rows); else 1
  int32_t batch;              // query rows (decode: sequences; prefill: sequences * L)
  int32_t num_heads;
  int32_t num_splits;
  const int32_t* items;       // planned decode: [num_items, 4] (sequence, first 32-token tile,
                              // tile count, partial row), item i on workgroup i; null: uniform splits
  int32_t num_items;
  int32_t chunk;              // tokens per split, multiple of 32
  int32_t max_seq_len;
  float scale;                // softmax scale
  float scale_log2;           // softmax scale * log2(e)
  uint16_t* o_part;           // [B, P, H, 512] bf16 (P > 1)
  float* lse_part;            // [B, P, H] fp32 (P > 1)
  uint16_t* o_lat;            // [B, H, 512] bf16 (P == 1)
  float* lse;                 // [B, H] fp32 (P == 1)
};

struct ProjArgs {
  const uint16_t* x;     // absorb: q_nope [B, H, 128]; expand: o_lat [B, H, 512]
  const uint16_t* w;     // absorb: W_UK [H, 128, 512]; expand: W_UV [H, 128, 512]
  uint16_t* y;           // absorb: q_lat [B, H, 512]; expand: out [B, H, 128]
  int32_t batch;
  int32_t num_heads;
};

struct CombineArgs {
  const uint16_t* o_part; // [B, P, H, 512] bf16 (planned: [num_items, H, 512])
  const float* lse_part; // [B, P, H] (planned: [num_items, H])
  uint16_t* o_lat;       // [B, H, 512]
  float* lse;            // [B, H] or null
  int32_t batch;
  int32_t num_heads;
  int32_t num_splits;    // uniform splits per sequence (planned: num_items)
  const int32_t* seq_first;  // planned: [B + 1] first item of each sequence; null: uniform
};

struct CombineExpandArgs {
  const uint16_t* o_part; // [B, P, H, 512] bf16
  const float* lse_part; // [B, P, H]
  const uint16_t* w_uv;  // [H, 128, 512] bf16
  uint16_t* out;         // [B, H, 128] bf16
  uint16_t* o_lat;       // [B, H, 512] bf16 or null
  float* lse;            // [B, H] or null
  int32_t batch;
  int32_t num_heads;
  int32_t num_splits;    // uniform splits per sequence (planned: num_items)
  int32_t rows;          // sequences per workgroup: 4, 8 or 16 (set by the launcher)
  const int32_t* seq_first;  // planned: [B + 1] first item of each sequence; null: uniform
};

struct AppendArgs {
  const uint16_t* kv_in;      // [B, num_new, in_stride] bf16: 512 latent, then 64 unrotated key
  int64_t in_stride;          // elements between consecutive input rows
  const int32_t* positions;   // [B]: position of each sequence's first new token
  int32_t batch;
  int32_t num_new;
  char* kv;                   // latent element 0 of slot 0
  char* pe;                   // rope element 0 of slot 0
  int64_t kv_sb;              // bytes between consecutive slots (kv)
  int64_t pe_sb;              // bytes between consecutive slots (pe)
  float* token_scale;         // E4M3 cache: one fp32 scale per slot (else null)
  int64_t seq_stride;         // contiguous: slots per sequence
  const int32_t* block_table; // paged: [B, max_blocks]; null = contiguous
  int32_t block_size;
  int32_t max_blocks;
  double inv_freq[32];        // rotation frequency of key pair i: base^(-2i/64)
};

struct FusedStepArgs {
  const uint16_t* q_nope;     // [B, H, 128] bf16
  const uint16_t* q_pe;       // [B, H, 64] bf16
  const uint16_t* w_uk;       // [H, 128, 512] bf16
  const uint16_t* w_uv;       // [H, 128, 512] bf16
  const char* kv;             // cache addressing as in DecodeArgs
  const char* pe;
  int64_t kv_sb;
  int64_t pe_sb;
  int64_t seq_stride;
  const int32_t* block_table;
  int32_t block_size;
  int32_t max_blocks;
  const float* token_scale;
  const int32_t* seq_lens;    // [B]
  int32_t batch;
  int32_t num_heads;
  int32_t max_seq_len;
  float scale_log2;           // softmax scale * log2(e)
  uint16_t* out;              // [B, H, 128] bf16
  uint16_t* o_lat;            // [B, H, 512] bf16 or null
  float* lse;                 // [B, H] fp32 or null
};

struct NaiveArgs {
  const uint16_t* q_nope;     // [B, H, 128] bf16
  const uint16_t* q_pe;       // [B, H, 64] bf16
  const uint16_t* w_uk;       // [H, 128, 512] bf16
  const uint16_t* w_uv;       // [H, 128, 512] bf16
  const char* kv;             // cache addressing as in DecodeArgs
  const char* pe;
  int64_t kv_sb;
  int64_t pe_sb;
  int64_t seq_stride;
  const int32_t* block_table;
  int32_t block_size;
  int32_t max_blocks;
  const float* token_scale;
  const int32_t* seq_lens;    // [B]
  int32_t batch;
  int32_t num_heads;
  int32_t max_seq_len;
  float scale_log2;           // softmax scale * log2(e)
  uint16_t* ws;               // [B, max_seq_len, H, 256] bf16: expanded k_nope | v per token and head
  uint16_t* out;              // [B, H, 128] bf16
};

// Device scratch of mla_decode_latent_noalloc (split partials), per GPU.
constexpr size_t kScratchBytes = (size_t)48 << 20;
// Device address of this GPU's scratch array (looked up once per device).
hipError_t scratch_region(void** ptr);

hipError_t launch_decode_latent(const DecodeArgs& a, hipStream_t stream);
// 128 heads, bf16 cache: 32-head waves with P.V woven into the next tile's scores.
hipError_t launch_decode_latent_wide(const DecodeArgs& a, hipStream_t stream);
// 16 heads, bf16 cache: two computing waves split each tile by tokens
hipError_t launch_decode_latent16(const DecodeArgs& a, hipStream_t stream);
// 128 heads, E4M3 cache: the stored codes on fp8 MFMAs.
hipError_t launch_decode_latent_fp8(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_absorb_q(const ProjArgs& a, hipStream_t stream);
hipError_t launch_expand_v(const ProjArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// combine + expand_v in one launch
hipError_t launch_combine_expand(const CombineExpandArgs& a, hipStream_t stream);
hipError_t launch_decode_step_fused(const FusedStepArgs& a, bool fp8, hipStream_t stream);
// Naive decode: expansion GEMM into a.ws, then attention over the expanded rows.
hipError_t launch_naive_decode(const NaiveArgs& a, bool fp8, hipStream_t stream);
// fp8 selects the E4M3 cache encoding.
hipError_t launch_cache_append(const AppendArgs& a, bool fp8, hipStream_t stream);

}  // namespace mla
