// Latent attention of absorbed-MLA decode for 128 heads over an E4M3 latent
// cache, on gfx950's fp8 matrix cores.
//
// Same computation as the bf16 kernels ("DeepSeek MLA 吸收式缓存：真实权重执行与
// FlashMLA 架构边界" §2.2-§2.4, §6.1: every head scores the shared 576-wide
// cache rows, online softmax, o[h] = sum_t p_t c_t over the 512 latent
// columns) for a cache stored as OCP E4M3 codes with one fp32 scale per token
// ("G5 MLA KV 访存建模设计规格" use case 1): c_t = token_scale_t * code_t.
// The stored codes are multiplied as they are, on v_mfma_scale_f32_32x32x64
// (fp8 x fp8, per-32-element power-of-two block scales):
//   - scores: the bf16 query q of a head is split into two E4M3 parts,
//     q = 2^k (hi + lo / 16) with hi = E4M3(q 2^-k), lo = E4M3((q 2^-k - hi) 16),
//     2^k chosen so max |q 2^-k| of the head lies in [128, 256); the block
//     scales carry 2^k and 2^(k-4), so s = q . code is as close to the bf16
//     query's as a bf16 product; the token scale then multiplies s in fp32;
//   - P.V: the probability that multiplies code_t is p_t * token_scale_t,
//     stored as E4M3 with a power-of-two scale per (head, 32 tokens) taken
//     from a bound (the block's largest p times its largest token scale) so
//     that its largest value is below 256.  The 3-bit mantissa of these
//     weights is the one rounding that bf16 products would not make; the
//     normaliser is therefore the sum of the weights as stored (each divided
//     by its token scale), so that o is a convex combination of the cached
//     rows with the stored weights, while lse keeps the exact sum.  A token
//     whose scale is 0 or below 2^-6 of the block's largest counts at its
//     exact p in the normaliser (its row is (nearly) zero but its p is not);
//     any other weight that rounds to zero has p below 2^-11 of the block's
//     largest and leaves both sums alike.
// No code is widened to bf16: tiles stay in LDS as the stored bytes.
//
// One workgroup per (sequence, split) or planned item, 4 waves, one per SIMD;
// wave w owns heads 32w .. 32w+31 from the query to the output.
//   - Tiles of 64 cached rows: the latent codes (64 x 512 B) go to a ring of 4
//     buffers, the RoPE codes (64 x 64 B) to a ring of 3 and the token scales
//     to a ring of 4.  16-byte direct-to-LDS copies; chunk c of row r lands in
//     slot c ^ (r % 16) (latent) or c ^ ((r / 4) % 4) (RoPE), so both the
//     score reads (16 rows, one chunk) and the transposing P.V reads (8 rows x
//     16 bytes) hit distinct banks.
//   - Scores: per 64-wide slice of the 576 dims and 32-token half, (hi, lo):
//     S^T[token][head] on 32x32x64 MFMAs with the split query block (144
//     VGPRs) as the B operand.
//   - Softmax per 32-token half.  The reference max m is an integer in the
//     exp2 domain and moves only when a half's max exceeds it by more than
//     2^kRescaleLog2, to the ceiling of that max, so every correction of
//     earlier sums is an exact power of two.
//   - P.V: O^T[column][head] for all 512 columns of the wave's 32 heads (256
//     AGPRs); V^T through ds_read_b64_tr_b8.  The probabilities of a half are
//     already in the B-operand layout where the score MFMA left them (a lane
//     holds one head and 16 tokens of each half; a half is one 32-element
//     scale block), so they never leave registers, and a later max of the
//     same tile corrects the first half's block scale.
//   - Per tile k, three stages: the score MFMAs of half 0 of tile k with the
//     softmax of half 1 of tile k-1 between them; the P.V MFMAs of tile k-1
//     with the first part of the softmax of half 0 of tile k; the score MFMAs
//     of half 1 of tile k with the rest of that softmax and the copies of
//     tile k+2.  A wave's vector work issues while its own MFMA runs, so the
//     softmax is cut into steps of about one MFMA's time, one after each
//     MFMA: the matrix core then waits on neither.
#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_layout.hpp"

namespace mla {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int kT8 = 64;                 // cached rows per tile
constexpr int kLat8 = kT8 * kDc;        // 32768: latent codes of a tile
constexpr int kPe8 = kT8 * kDr;         // 4096: RoPE codes of a tile
constexpr int kSc8 = 2 * 256;           // token scales of a tile: two halves of 32 (plus copies)
constexpr uint32_t kE8m0One = 0x7F7F7F7Fu;  // block scale 1.0 in every byte
// Smallest exponent of a weight bound: the scaled p (at most 2^(142 - eb))
// of 32 tokens then sum below 2^128.
constexpr int kEbMin = 20;

// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 A and B.  Lanes l and l+32 hold
// row (A) / column (B) l % 32; byte p of lane l + 32 g is contraction element
// (g, p): A and B pair equal (g, p).  The block scale of elements p < 16 (of
// both lanes) comes from lane l % 32, of p >= 16 from lane l % 32 + 32; byte
// BSEL of the B scale register is used (checked on gfx950 with in-bounds
// probes).  D[8 (j/4) + 4 (l/32) + j%4][l%32] = accumulator j of lane l.
// Issued as inline asm so the score accumulators live in VGPRs and the P.V
// accumulators in AGPRs.
template <int BSEL>
__device__ __forceinline__ void mfma8_v(i32x8 a, i32x8 b, uint32_t sa, uint32_t sb, f32x16& c) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
      : "+v"(c)
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(BSEL & 1), "n"(BSEL >> 1));
}
template <int BSEL>
__device__ __forceinline__ void mfma8_v_first(i32x8 a, i32x8 b, uint32_t sa, uint32_t sb, f32x16& c) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
      : "=&v"(c)
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(BSEL & 1), "n"(BSEL >> 1));
}
template <int BSEL>
__device__ __forceinline__ void mfma8_a(i32x8 a, i32x8 b, uint32_t sa, uint32_t sb, f32x16& c) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[0,%5,0] op_sel_hi:[0,%6,0]"
      : "+a"(c)
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(BSEL & 1), "n"(BSEL >> 1));
}
// VALU reads of an MFMA result wait for it (the first of a run carries the
// wait states); VALU writes of an accumulator precede its next MFMA.
__device__ __forceinline__ void drain8_v(f32x16& c, bool first) {
  if (first) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
  else asm volatile("" : "+v"(c));
}
__device__ __forceinline__ void acc8_fence_read(f32x16& c, bool first) {
  if (first) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(c));
  else asm volatile("" : "+a"(c));
}
__device__ __forceinline__ void acc8_fence_write(f32x16& c, bool last) {
  if (last) asm volatile("s_nop 7" : "+a"(c));
  else asm volatile("" : "+a"(c));
}

// Transposing 8-bit LDS read (ds_read_b64_tr_b8): within each group of 16
// lanes, lanes 2m and 2m+1 point at bytes 0..7 and 8..15 of row m of an
// 8 x 16-byte block; lane j receives byte j of the 8 rows, row 0 first.
__device__ __forceinline__ i32x2 lds_read_tr8(uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(uintptr_t)byte_off);
}

__device__ __forceinline__ i32x8 lds_read_i32x8(uint32_t byte_off) {
  const u32x4 lo = lds_read_u32x4(byte_off), hi = lds_read_u32x4(byte_off + 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four fp32 values -> four E4M3 codes (nearest even) in one dword, first in
// the low byte.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// Latent copy c (0..7) of a full tile: 1 KiB from sbase + voff to LDS
// lds + 1024 c (the offset as an immediate of the M0 add); NT sets the
// non-temporal bit.
template <bool NT>
__device__ __forceinline__ void lat_copy_full(int c, const char* sbase, uint32_t voff, uint32_t lds) {
  switch (c) {
    case 0: dma16_off<0, 0, NT>(sbase, voff, lds); break;
    case 1: dma16_off<0, 1024, NT>(sbase, voff, lds); break;
    case 2: dma16_off<0, 2048, NT>(sbase, voff, lds); break;
    case 3: dma16_off<0, 3072, NT>(sbase, voff, lds); break;
    case 4: dma16_off<0, 4096, NT>(sbase, voff, lds); break;
    case 5: dma16_off<0, 5120, NT>(sbase, voff, lds); break;
    case 6: dma16_off<0, 6144, NT>(sbase, voff, lds); break;
    default: dma16_off<0, 7168, NT>(sbase, voff, lds); break;
  }
}

// Biased fp32 exponent of x (0 for zero).
__device__ __forceinline__ int f32_exp(float x) { return (int)((__float_as_uint(x) >> 23) & 0xFFu); }

// Maximum over the 32 lanes of each wave half (DPP within rows of 16, then
// the row swap): lanes 0..31 get the max of lanes 0..31, lanes 32..63 of 32..63.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  return vmax(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float max_lanes32(float x) {
  x = dpp_max<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x141>(x);  // row_half_mirror
  x = dpp_max<0x140>(x);  // row_mirror
  return vmax_xor16(x);
}

}  // namespace

template <bool PAGED, bool STREAM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_latent_fp8_kernel(DecodeArgs a) {
  constexpr int NW = 4;                   // waves: one per SIMD
  constexpr int H = NW * 32;              // heads
  constexpr int CT = kDc / 32;            // 32-column tiles of V^T / O^T
  constexpr int NLAT = 4, NPE = 3, NSC = 4;  // ring lengths
  constexpr int kLatRing = 0;
  constexpr int kPeRing = kLatRing + NLAT * kLat8;     // 131072
  constexpr int kScRing = kPeRing + NPE * kPe8;        // 143360
  constexpr int kRtsOff = kScRing + NSC * kSc8;        // 145408: [wave][2][64 tokens] 1 / token scale
  constexpr int kSmem = kRtsOff + NW * 2 * 256;        // 147456
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  static_assert(NW * 32 * kDc * 2 <= kPeRing, "epilogue staging must fit in the latent ring");
  static_assert(kLat8 % 1024 == 0 && kPeRing % 1024 == 0 && kScRing % 256 == 0, "buffer alignment");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int li = lane & 31;   // head 32w + li
  const int lg = lane >> 5;   // lane half
  // uniform splits: a sequence's splits share an XCD (and its L2 copy of the
  // queries); planned decode: workgroup i runs item i, in the order the plan
  // gives; prefill rows go round-robin over the XCDs, longest first
  const bool planned = a.items != nullptr;
  const int item = planned || a.q_start != nullptr ? (int)blockIdx.x : xcd_grouped_index(blockIdx.x, gridDim.x);
  const PlanItem pl = planned ? plan_item(a.items, item, a.batch, a.max_seq_len, a.num_items) : PlanItem{0, 0, 0, 0};
  if (pl.slot < 0) return;  // no partial row to write
  const int qrow = planned ? pl.seq : item / a.num_splits;
  const int split = planned ? item : item - qrow * a.num_splits;
  const int b = a.q_start == nullptr ? qrow : a.batch - 1 - qrow;  // query row
  const int cb = b / a.q_per_seq;                                   // the sequence it reads
  int T = a.q_start == nullptr ? a.seq_lens[b] : max(a.q_start[cb], 0) + (b - cb * a.q_per_seq) + 1;
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
  const int t_begin = planned ? pl.t_begin : split * a.chunk;
  const int t_end = min(T, planned ? pl.t_end : t_begin + a.chunk);
  const bool final_out = !planned && a.num_splits == 1;
  const size_t part = planned ? (size_t)pl.slot : (size_t)b * a.num_splits + split;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  uint16_t* const out_rows = final_out ? a.o_lat + (size_t)b * H * kDc : a.o_part + part * H * kDc;
  float* const lse_out = final_out ? a.lse + (size_t)b * H : a.lse_part + part * H;

  if (t_begin >= t_end) {
    // No tokens in this range: zero weight (o = 0, lse = -inf).
    for (int r = 0; r < 32; ++r)
      *reinterpret_cast<u32x4*>(out_rows + (size_t)(32 * w + r) * kDc + lane * 8) = u32x4{0u, 0u, 0u, 0u};
    if (lg == 0) lse_out[32 * w + li] = -INFINITY;
    return;
  }

  const int n_tiles = (t_end - t_begin + kT8 - 1) / kT8;
  const char* kv_base = uniform_ptr(a.kv);
  const char* pe_base = uniform_ptr(a.pe);
  const uint32_t kv_sb = (uint32_t)a.kv_sb, pe_sb = (uint32_t)a.pe_sb;

  // ---- tile copies (HBM -> LDS, the stored bytes) ----
  // Wave w copies rows 16w .. 16w+15 of a tile: 8 latent copies of two rows
  // (1 KiB) and one RoPE copy of 16 rows; waves 0 and 1 also copy the token
  // scales of rows 0..31 / 32..63.  A tile's two 32-row halves are addressed
  // separately (a paged block holds a multiple of 32 rows).  Rows past the end
  // re-read the last row.
  struct Half {
    const char* kv;   // latent row of the half's first token
    const char* pe;   // its RoPE row
    const char* sc;   // its token scale
  };
  auto half_src = [&](int t0) -> Half {
    Half h;
    int64_t slot;
    if (PAGED) {
      const int blk = scalar_load(a.block_table, (size_t)cb * a.max_blocks + t0 / a.block_size);
      slot = (int64_t)blk * a.block_size + (t0 % a.block_size);
    } else {
      slot = (int64_t)cb * a.seq_stride + t0;
    }
    h.kv = uniform_ptr(kv_base + slot * a.kv_sb);
    h.pe = uniform_ptr(pe_base + slot * a.pe_sb);
    h.sc = uniform_ptr(reinterpret_cast<const char*>(a.token_scale + slot));
    return h;
  };
  auto lat_buf = [&](int tile) -> uint32_t { return lds0 + kLatRing + (uint32_t)(tile % NLAT) * kLat8; };
  auto pe_buf = [&](int tile) -> uint32_t { return lds0 + kPeRing + (uint32_t)(tile % NPE) * kPe8; };
  auto sc_buf = [&](int tile) -> uint32_t { return lds0 + kScRing + (uint32_t)(tile % NSC) * kSc8; };
  auto rts_buf = [&](int tile) -> uint32_t { return lds0 + kRtsOff + (uint32_t)w * 512u + (uint32_t)(tile & 1) * 256u; };
  // A tile's copies are issued one at a time between MFMAs (a copy can hold
  // the wave's issue while the memory pipeline is busy): tile_src() gathers
  // the tile's source rows and buffers, copy(c) issues copy c of this wave
  // (c < 10: 8 latent, 1 RoPE, and for waves 0 and 1 the scales).
  struct TileSrc {
    Half h0, h1;
    int last;        // last valid row of the tile
    uint32_t lat, pe, sc;
  };
  auto tile_src = [&](int tile) -> TileSrc {
    TileSrc t;
    const int t0 = t_begin + tile * kT8;
    t.last = min(kT8, t_end - t0) - 1;
    t.h0 = half_src(t0);
    t.h1 = t.last >= 32 ? half_src(t0 + 32) : t.h0;
    t.lat = lat_buf(tile);
    t.pe = pe_buf(tile);
    t.sc = sc_buf(tile);
    return t;
  };
  // A full tile (64 valid rows) needs no clamping: copy c's rows lie in half
  // w / 2, and its latent offsets follow from two lane constants: the chunk
  // part XOR 2c (the lane chunk XOR (2c + lg) is (lane chunk ^ lg) ^ 2c) plus
  // the row part plus 2c rows.  copy_refresh() hides their values from the
  // compiler once per tile, so that it does not hoist the eight per-copy
  // offsets out of the loop (they would not fit the registers).
  uint32_t cp_lat_chunk = (((uint32_t)lane & 31u) ^ ((uint32_t)lane >> 5)) << 4;
  uint32_t cp_lat_row = (16u * (uint32_t)(w & 1) + ((uint32_t)lane >> 5)) * kv_sb;
  auto copy_refresh = [&]() { asm volatile("" : "+v"(cp_lat_chunk), "+v"(cp_lat_row)); };
  auto copy = [&](const TileSrc& t, int c) {
    if (t.last == kT8 - 1) {
      const Half& hs = w >= 2 ? t.h1 : t.h0;
      if (c < 8) {
        const uint32_t voff = (cp_lat_chunk ^ ((uint32_t)c << 5)) + (cp_lat_row + (uint32_t)(2 * c) * kv_sb);
        lat_copy_full<STREAM>(c, hs.kv, voff, t.lat + (uint32_t)(16 * w) * kDc);
      } else if (c == 8) {
        const uint32_t ln = lane_id();
        const uint32_t voff = (16u * (uint32_t)(w & 1) + (ln >> 2)) * pe_sb + (((ln & 3u) ^ ((ln >> 4) & 3u)) << 4);
        dma16<STREAM>(hs.pe, voff, t.pe + (uint32_t)(16 * w) * kDr);
      } else if (c == 9 && w < 2) {
        dma4(w ? t.h1.sc : t.h0.sc, (lane_id() & 31u) * 4u, t.sc + 256u * (uint32_t)w);
      }
      return;
    }
    const uint32_t ln = lane_id();
    if (c < 8) {
      // latent rows 16w + 2c + (ln / 32): slot ln % 32 holds chunk slot ^ (row % 16)
      const int r0 = 16 * w + 2 * c;
      const int rb = min(r0, t.last);                      // the copy's rows all lie in rb's half
      const int hf = rb >> 5;
      const uint32_t r = (uint32_t)r0 + (ln >> 5);
      const uint32_t rc = (uint32_t)min((int)r, t.last) - 32u * (uint32_t)hf;
      const uint32_t voff = rc * kv_sb + (((ln & 31u) ^ (r & 15u)) << 4);
      dma16<STREAM>(hf ? t.h1.kv : t.h0.kv, voff, t.lat + (uint32_t)r0 * kDc);
    } else if (c == 8) {
      // RoPE rows 16w + ln / 4: slot ln % 4 holds chunk slot ^ ((row / 4) % 4)
      const int r0 = 16 * w;
      const int rb = min(r0, t.last);
      const int hf = rb >> 5;
      const uint32_t r = (uint32_t)r0 + (ln >> 2);
      const uint32_t rc = (uint32_t)min((int)r, t.last) - 32u * (uint32_t)hf;
      const uint32_t voff = rc * pe_sb + (((ln & 3u) ^ ((r >> 2) & 3u)) << 4);
      dma16<STREAM>(hf ? t.h1.pe : t.h0.pe, voff, t.pe + (uint32_t)r0 * kDr);
    } else if (c == 9 && w < 2) {
      // token scales of rows 32w .. 32w+31 (lane ln: row 32w + ln % 32) at
      // 256 w + 4 (ln % 32), and again at + 128
      const int rb = min(32 * w, t.last);
      const int hf = rb >> 5;
      const uint32_t r = 32u * (uint32_t)w + (ln & 31u);
      const uint32_t rc = (uint32_t)min((int)r, t.last) - 32u * (uint32_t)hf;
      dma4(hf ? t.h1.sc : t.h0.sc, rc * 4u, t.sc + 256u * (uint32_t)w);
    }
  };
  auto issue_tile = [&](int tile) {
    const TileSrc t = tile_src(tile);
#pragma unroll
    for (int c = 0; c < 10; ++c) copy(t, c);
  };
  // this wave's copies of the oldest tile in flight have landed (the next
  // tile's, if requested, may still be in flight)
  auto wait_tile = [&](bool next_in_flight) {
    if (!next_in_flight) wait_vmcnt<0>();
    else if (w < 2) wait_vmcnt<10>();
    else wait_vmcnt<9>();
  };

  // ---- query block: two E4M3 parts per head, in the B-operand layout ----
  // Lane li + 32 lg of wave w holds, for slice s (dims 64 s .. 64 s + 63;
  // s = 8 is the RoPE part), head 32w + li's dims 64 s + 32 lg + p in byte p
  // of qh[s] (hi) and ql[s] (lo); qs holds the E8M0 scales of hi (byte 0) and
  // lo (byte 1).
  i32x8 qh[9], ql[9];
  uint32_t qs;
  {
    const int head = 32 * w + li;
    const u32x4* qlat = reinterpret_cast<const u32x4*>(a.q_lat + ((size_t)b * H + head) * kDc);
    const u32x4* qpe = reinterpret_cast<const u32x4*>(a.q_pe + ((size_t)b * H + head) * kDr);
    auto qload = [&](int s, int k) -> u32x4 {  // 8 bf16: dims 64 s + 32 lg + 8 k .. +7
      return s < 8 ? qlat[8 * s + 4 * lg + k] : qpe[4 * lg + k];
    };
    // pass 1: largest magnitude of the head (both lane halves)
    float mx = 0.f;
#pragma unroll
    for (int s = 0; s < 9; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = qload(s, k);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mx = vmax3(mx, fabsf(__uint_as_float(v[e] << 16)), fabsf(__uint_as_float(v[e] & 0xffff0000u)));
      }
    mx = vmax_xor32(mx);
    // 2^k with max |q| 2^-k in [128, 256): k = e - 134 (e: biased exponent)
    const int e = max(f32_exp(mx), 12);
    const float mult = __uint_as_float((uint32_t)(261 - e) << 23);
    qs = (uint32_t)(e - 7) | ((uint32_t)(e - 11) << 8);
    issue_tile(0);
    // pass 2: hi = E4M3(q 2^-k), lo = E4M3((q 2^-k - hi) 16)
#pragma unroll
    for (int s = 0; s < 9; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const u32x4 v = qload(s, k);
        float x[8];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          x[2 * e2] = __uint_as_float(v[e2] << 16) * mult;
          x[2 * e2 + 1] = __uint_as_float(v[e2] & 0xffff0000u) * mult;
        }
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const uint32_t hv = pack_e4m3x4(x[4 * d], x[4 * d + 1], x[4 * d + 2], x[4 * d + 3]);
          const f32x2 h01 = e4m3x2_to_f32<false>(hv), h23 = e4m3x2_to_f32<true>(hv);
          const uint32_t lv = pack_e4m3x4((x[4 * d] - h01[0]) * 16.f, (x[4 * d + 1] - h01[1]) * 16.f,
                                          (x[4 * d + 2] - h23[0]) * 16.f, (x[4 * d + 3] - h23[1]) * 16.f);
          qh[s][2 * k + d] = (int)hv;
          ql[s][2 * k + d] = (int)lv;
        }
      }
    // tile 1 after the query (whose loads the compiler waits for in issue
    // order, so they would otherwise wait for these copies too)
    if (n_tiles > 1) issue_tile(1);
  }

  // ---- per-lane LDS addresses inside a tile ----
  // Score A operand (K): lane li + 32 lg, token row R = 32 tb + li, bytes p ->
  // dims 64 s + 32 lg + p: latent chunks 4 s + 2 lg + q (q = 0, 1) at slot
  // chunk ^ (R % 16), i.e. the lane's base for q XORed with (s % 4) << 6, plus
  // 256 (s / 4) + 16384 tb.  RoPE: chunks 2 lg + q at slot chunk ^ ((R / 4) % 4).
  // Probabilities (B operand of P.V): lane li + 32 g, byte p is token
  // tok(g, p) = 32 (p / 16) + 8 ((p % 16) / 4) + 4 g + p % 4 of head li: bytes
  // 0..15 are the lane's score accumulators 0..15 of half 0, bytes 16..31 those
  // of half 1, and the block scale of bytes p < 16 (half 0) comes from lane li,
  // of p >= 16 (half 1) from lane li + 32.
  // V^T A operand of column tile ct: lane c + 32 g, byte p holds
  // V[tok(g, p)][32 ct + c].  Read q gives bytes 8q .. 8q+7: in the 16-lane
  // group G = lane / 16 (c = 16 (G % 2) + i, g = G / 2), lanes 2m and 2m+1
  // point at bytes 0..7 / 8..15 of column chunk 2 ct + G % 2 of row
  // 16 q + 8 (m / 4) + 4 g + m % 4, whose low four bits r0 do not depend on q:
  // the chunk's slot is (2 ct + G % 2) ^ r0 = 16 (ct / 8) + (2 (ct % 8) ^ kap)
  // with kap = (G % 2) ^ r0, i.e. the lane's base XORed with 32 (ct % 8), plus
  // 256 (ct / 8) + 8192 q.  (Tile buffers are 1 KiB aligned, so the XORs act
  // on the lane's part alone.)
  const uint32_t ln0 = (uint32_t)lane;
  const uint32_t ki = ln0 & 31u, kg = ln0 >> 5;
  const uint32_t kbl0 = ki * (uint32_t)kDc + (((2u * kg) ^ (ki & 15u)) << 4);
  const uint32_t kbl1 = ki * (uint32_t)kDc + (((2u * kg + 1u) ^ (ki & 15u)) << 4);
  const uint32_t pbl = ki * (uint32_t)kDr + (((2u * kg) ^ ((ki >> 2) & 3u)) << 4);
  const uint32_t vG = ln0 >> 4, vi = ln0 & 15u;
  const uint32_t vr0 = 8u * (vi >> 3) + 4u * (vG >> 1) + ((vi >> 1) & 3u);
  const uint32_t vbl = vr0 * (uint32_t)kDc + (((vG & 1u) ^ vr0) << 4) + 8u * (vi & 1u);
  const uint32_t lgo = 16u * kg;   // per-token values: the lane half's 4-token groups
  struct KAddr {
    uint32_t k0, k1, pe;
  };
  auto k_addr = [&](uint32_t lat, uint32_t pe) { return KAddr{lat + kbl0, lat + kbl1, pe + pbl}; };
  auto k_read = [&](const KAddr& ka, int tb, int s) -> i32x8 {
    u32x4 lo, hi;
    if (s < 8) {
      const uint32_t x = (uint32_t)(s & 3) << 6, m = 256u * (uint32_t)(s >> 2) + 32u * (uint32_t)kDc * (uint32_t)tb;
      lo = lds_read_u32x4((ka.k0 ^ x) + m);
      hi = lds_read_u32x4((ka.k1 ^ x) + m);
    } else {
      const uint32_t m = 32u * (uint32_t)kDr * (uint32_t)tb;
      lo = lds_read_u32x4(ka.pe + m);
      hi = lds_read_u32x4((ka.pe ^ 16u) + m);
    }
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto v_read = [&](uint32_t vb, int ct) -> i32x8 {  // vb: tile buffer + vbl
    const uint32_t base = (vb ^ ((uint32_t)(ct & 7) << 5)) + 256u * (uint32_t)(ct >> 3);
    i32x8 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const i32x2 r = lds_read_tr8(base + 8192u * (uint32_t)q);
      v[2 * q] = r[0];
      v[2 * q + 1] = r[1];
    }
    return v;
  };

  f32x16 o[CT];  // o[ct][j] = O^T[32 ct + 8 (j/4) + 4 lg + j%4][head 32w + li]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int j = 0; j < 16; ++j) o[ct][j] = 0.f;
    acc8_fence_write(o[ct], ct == CT - 1);
  }
  // softmax state of head 32w + li (lanes li and li + 32 agree on m)
  const float c2 = a.scale_log2;
  float m = -INFINITY;   // reference max, an integer, of x = (q . k) * scale * log2(e)
  float l = 0.f;         // this lane's share of sum_t exp2(x_t - m)
  float lh = 0.f;        // the same with each weight as stored for P.V
  int dpend = 0;         // O still to be multiplied by 2^-dpend
  uint32_t pscale = 0x7Fu;  // block scale byte of the probabilities: half 0 in lanes 0..31, half 1 in 32..63
  i32x8 pcur = {0, 0, 0, 0, 0, 0, 0, 0};
  f32x16 sc[2];          // score accumulators of the two token halves, then their softmax

  // Keeps a step's results where the step is placed: without it the compiler
  // sinks their computation to the next use (a later stage), which keeps the
  // inputs live across the MFMAs in between.
  auto pin = [](auto& x) { asm volatile("" : "+v"(x)); };

  // ---- softmax of half h of a tile, in 18 steps ----
  // A step follows an MFMA and runs while it does (a wave's vector work
  // issues under its own MFMA), so each step holds at most ~12 vector
  // instructions (about one MFMA's time) and short dependent chains.  Step 0
  // only requests the token scales; the others:
  //    1-2  q . code -> q . k (token scales in fp32), ragged tail at -inf
  //    3    the half's max;  4  the reference max (and the rescale it implies)
  //    5    the weight bound's exponent eb, exponentials 0-1
  //    6-9  exponentials (p 2^(134 - eb)) and the first partial sum
  //    10   the sums l (exact) and lh
  //    11-12 weights p * token scale (scaled);  13  their E4M3 codes
  //    14-17 the stored-weight normaliser lh, the block scale
  // scb / rtsb: the tile's token scales and reciprocal scales (16-byte reads
  // of 4 tokens, issued a step or two ahead); nvalid: the tile's rows.  Lane
  // li + 32 lg holds tokens 32 h + 8 (j/4) + 4 lg + j%4 of head li in sc[h][j].
  // fresh: the half's last score MFMA was just issued.
  f32x4 t0 = {0.f, 0.f, 0.f, 0.f}, t1 = {0.f, 0.f, 0.f, 0.f};
  float hm = 0.f, xmh = 0.f, bias = 0.f, psa = 0.f, cs0 = 0.f, cs1 = 0.f;
  int eb = kEbMin;       // biased exponent of the half's weight bound
  float tsm0 = 0.f, tsm1 = 0.f;  // largest token scale of each half of the newest tile
  auto step = [&](int h, int i, uint32_t scb, uint32_t rtsb, int nvalid, bool fresh) {
    f32x16& s = sc[h];
    const uint32_t sp = scb + 256u * (uint32_t)h + lgo;    // token scales, + 32 a4
    const uint32_t rp = rtsb + 128u * (uint32_t)h + lgo;   // their reciprocals
    // the inverse of the weights' scale 2^(134 - eb) (the E8M0 block scale)
    auto inv_mult = [&]() { return __uint_as_float((uint32_t)(eb - 7) << 23); };
    if (i == 0) {
      t0 = lds_read_f32x4(sp);
      t1 = lds_read_f32x4(sp + 32u);
    } else if (i == 1 || i == 2) {
      if (i == 1) drain8_v(s, fresh);
      const int j0 = 8 * (i - 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s[j0 + k] *= t0[k];
        s[j0 + 4 + k] *= t1[k];
      }
      if (i == 1) {
        t0 = lds_read_f32x4(sp + 64u);
        t1 = lds_read_f32x4(sp + 96u);
      } else if (nvalid < 32 * (h + 1)) {
        const int tl = 4 * (int)kg;
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (32 * h + 8 * (j >> 2) + tl + (j & 3) >= nvalid) s[j] = -INFINITY;
      }
    } else if (i == 3) {
      const float h0 = vmax3(vmax3(s[0], s[1], s[2]), vmax3(s[3], s[4], s[5]), vmax3(s[6], s[7], s[8]));
      const float h1 = vmax3(vmax3(s[9], s[10], s[11]), vmax3(s[12], s[13], s[14]), s[15]);
      hm = vmax_xor32(vmax(h0, h1));
    } else if (i == 4) {
      // a new reference max when the half's max grows past the threshold
      xmh = hm * c2;
      const bool up = xmh > m + kRescaleLog2;
      const float mn = up ? ceilf(xmh) : m;
      const int d = (up && m != -INFINITY) ? (int)fminf(mn - m, 255.f) : 0;
      m = mn;
      const float f = d >= 127 ? 0.f : __uint_as_float((uint32_t)(127 - d) << 23);  // 2^-d
      l *= f;
      lh *= f;
      dpend += d;
      // half 0 of this tile is already stored against the old max
      if (h == 1 && lg == 0) pscale = (uint32_t)max((int)pscale - d, 0);
      pin(m);
      pin(l);
      pin(lh);
      pin(dpend);
      pin(pscale);
    } else if (i >= 5 && i <= 9) {
      if (i == 5) {
        // the weights p * token scale are at most (largest p) x (largest
        // token scale) of the half: they are scaled by 2^(134 - eb) with eb
        // the bound's exponent, so that the largest is below 256 (E4M3 holds
        // 448); p 2^(134 - eb) = exp2(x - m + 134 - eb)
        eb = max(f32_exp(fast_exp2(xmh - m) * (h ? tsm1 : tsm0)), kEbMin);
        bias = (float)(134 - eb) - m;
        pin(eb);
      }
      const int j0 = i == 5 ? 0 : 4 * (i - 6) + 2;
      const int j1 = i == 9 ? 16 : (i == 5 ? 2 : j0 + 4);
#pragma unroll
      for (int j = j0; j < j1; ++j) s[j] = fast_exp2(fmaf(s[j], c2, bias));
      if (i == 9) psa = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
    } else if (i == 10) {
      const float ps = psa + (((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15])));
      l = fmaf(ps, inv_mult(), l);
      lh = fmaf(ps, inv_mult(), lh);
      pin(l);
      pin(lh);
      t0 = lds_read_f32x4(sp);
      t1 = lds_read_f32x4(sp + 32u);
    } else if (i == 11 || i == 12) {
      const int j0 = 8 * (i - 11);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s[j0 + k] *= t0[k];
        s[j0 + 4 + k] *= t1[k];
      }
      if (i == 11) {
        t0 = lds_read_f32x4(sp + 64u);
        t1 = lds_read_f32x4(sp + 96u);
      } else {
        t0 = lds_read_f32x4(rp);
        t1 = lds_read_f32x4(rp + 32u);
        pin(s);
      }
    } else if (i == 13) {
      // E4M3 codes (this half's previous codes were last read by the P.V of
      // the tile before)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        pcur[4 * h + a4] = (int)pack_e4m3x4(s[4 * a4], s[4 * a4 + 1], s[4 * a4 + 2], s[4 * a4 + 3]);
      pin(pcur);
    } else if (i >= 14 && i <= 17) {
      // normaliser: each exact p replaced by (stored weight) / (token scale);
      // a token whose reciprocal scale was set to 0 (a zero scale, or one far
      // below the half's largest) keeps its exact p
      const int a4 = i - 14;
      const f32x4 rt = (a4 & 1) ? t1 : t0;
      const f32x2 d01 = e4m3x2_to_f32<false>((uint32_t)pcur[4 * h + a4]);
      const f32x2 d23 = e4m3x2_to_f32<true>((uint32_t)pcur[4 * h + a4]);
      const float c0 = a4 == 0 ? 0.f : cs0, c1 = a4 == 0 ? 0.f : cs1;
      cs0 = fmaf(d01[0] - s[4 * a4], rt[0], fmaf(d23[0] - s[4 * a4 + 2], rt[2], c0));
      cs1 = fmaf(d01[1] - s[4 * a4 + 1], rt[1], fmaf(d23[1] - s[4 * a4 + 3], rt[3], c1));
      if (a4 == 0) t0 = lds_read_f32x4(rp + 64u);
      if (a4 == 1) t1 = lds_read_f32x4(rp + 96u);
      if (a4 == 3) {
        lh = fmaf(cs0 + cs1, inv_mult(), lh);
        if (lg == h) pscale = (uint32_t)(eb - 7);
        pin(lh);
        pin(pscale);
      }
    }
  };

  // Per tile, once its scales have landed: the largest token scale of each
  // half (tsm0 / tsm1, for the weight bounds) and the reciprocal scales in a
  // per-wave region, 0 where the scale is 0 or below 2^-6 of its half's
  // largest (such a token's weight may round to zero while its p matters).
  float rts_v = 0.f;
  auto rts_load = [&](int tile) {
    const uint32_t ln = lane_id();  // (formed here: a lane constant held across the loop would spill)
    rts_v = lds_read_f32(sc_buf(tile) + 256u * (ln >> 5) + 4u * (ln & 31u));
  };
  auto rts_store = [&](int tile) {
    const float mx = max_lanes32(rts_v);
    tsm0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 0));
    tsm1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 32));
    const bool keep = rts_v > 0.f && rts_v * 64.f >= mx;
    lds_write_f32(rts_buf(tile) + 4u * lane_id(), keep ? __builtin_amdgcn_rcpf(rts_v) : 0.f);
  };

  // score MFMAs of half h of a tile, chunk(j) after the j-th (j = 0..17); two
  // K fragments in registers, each requested two slices ahead
  auto scores = [&](const KAddr& ka, int h, auto chunk) {
    i32x8 kb[2];
    kb[0] = k_read(ka, h, 0);
    kb[1] = k_read(ka, h, 1);
#pragma unroll
    for (int s = 0; s < 9; ++s) {
      if (s == 0) mfma8_v_first<0>(kb[0], qh[0], kE8m0One, qs, sc[h]);
      else mfma8_v<0>(kb[s & 1], qh[s], kE8m0One, qs, sc[h]);
      __builtin_amdgcn_sched_barrier(0);
      chunk(2 * s);
      __builtin_amdgcn_sched_barrier(0);
      mfma8_v<1>(kb[s & 1], ql[s], kE8m0One, qs, sc[h]);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 2 < 9) kb[s & 1] = k_read(ka, h, s + 2);
      __builtin_amdgcn_sched_barrier(0);
      chunk(2 * s + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // P.V MFMAs of a tile (probabilities in pcur / pscale); after column tile ct, chunk(ct)
  auto pv = [&](uint32_t lat, auto chunk) {
    asm volatile("s_nop 4" : "+v"(pcur), "+v"(pscale));  // VALU writes before the MFMA reads
    const uint32_t vb = lat + vbl;
    i32x8 va[2];
    va[0] = v_read(vb, 0);
    va[1] = v_read(vb, 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      mfma8_a<0>(va[ct & 1], pcur, kE8m0One, pscale, o[ct]);
      __builtin_amdgcn_sched_barrier(0);
      if (ct + 2 < CT) va[ct & 1] = v_read(vb, ct + 2);
      __builtin_amdgcn_sched_barrier(0);
      chunk(ct);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto rescale_o = [&]() {  // O *= 2^-dpend (rare after the first tiles)
    if (__ballot(dpend != 0) != 0) {
      const float f = dpend >= 127 ? 0.f : __uint_as_float((uint32_t)(127 - dpend) << 23);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        acc8_fence_read(o[ct], ct == 0);
        o[ct] *= f;
        acc8_fence_write(o[ct], ct == CT - 1);
      }
      dpend = 0;
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto tile_rows = [&](int tile) { return min(kT8, t_end - (t_begin + tile * kT8)); };

  // ---- pipeline ----
  // Iteration k < n_tiles, after the barrier (tile k landed; tile k+1's copies
  // may be in flight; every wave is done with iteration k-1):
  //   A. scores of half 0 of tile k | softmax steps 1..17 of half 1 of tile
  //      k-1; the scale maxima and reciprocal scales of tile k
  //   B. O rescale; P.V of tile k-1 | softmax steps 0..12 of half 0 of tile k
  //   C. scores of half 1 of tile k | softmax steps 13..17 of half 0 of tile
  //      k, this wave's copies of tile k+2 (into the buffers of tile k-2 --
  //      latent and scales, last read in iteration k-1 -- and of tile k-1 for
  //      the RoPE rows, scored in iteration k-1), step 0 of half 1 of tile k
  // (step 13 rewrites half 0's probability registers, which the P.V of stage
  // B has read by then).  A last part finishes tile n_tiles-1: the softmax of
  // its half 1 and its P.V.
  auto begin_tile = [&](int k) {
    copy_refresh();
    wait_tile(k + 1 < n_tiles);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // stage C of iteration k (after score MFMA j of half 1)
  auto stage_c = [&](int k, const TileSrc& t2, int j, uint32_t sc_k, uint32_t rts_k, int nv_k) {
    if (j < 5) step(0, 13 + j, sc_k, rts_k, nv_k, false);
    else if (j < 15 && k + 2 < n_tiles) copy(t2, j - 5);
    else if (j == 17) step(1, 0, sc_k, rts_k, nv_k, false);
  };
  {
    begin_tile(0);
    const TileSrc t2 = tile_src(min(2, n_tiles - 1));  // (a tile past the end is not copied)
    const KAddr ka = k_addr(lat_buf(0), pe_buf(0));
    const uint32_t sc_k = sc_buf(0), rts_k = rts_buf(0);
    const int nv_k = tile_rows(0);
    scores(ka, 0, [&](int j) {
      if (j == 16) rts_load(0);
      if (j == 17) rts_store(0);
    });
#pragma unroll
    for (int i = 0; i < 13; ++i) step(0, i, sc_k, rts_k, nv_k, i == 1);
    scores(ka, 1, [&](int j) { stage_c(0, t2, j, sc_k, rts_k, nv_k); });
  }
  for (int k = 1; k < n_tiles; ++k) {
    begin_tile(k);
    const TileSrc t2 = tile_src(min(k + 2, n_tiles - 1));
    const KAddr ka = k_addr(lat_buf(k), pe_buf(k));
    const uint32_t sc_k = sc_buf(k), rts_k = rts_buf(k);
    const int nv_k = tile_rows(k);
    const uint32_t sc_p = sc_buf(k - 1), rts_p = rts_buf(k - 1);
    const int nv_p = tile_rows(k - 1);
    scores(ka, 0, [&](int j) {
      if (j < 17) step(1, j + 1, sc_p, rts_p, nv_p, false);
      if (j == 16) rts_load(k);
      if (j == 17) rts_store(k);
    });
    rescale_o();
    pv(lat_buf(k - 1), [&](int ct) {
      if (ct < 13) step(0, ct, sc_k, rts_k, nv_k, false);
    });
    scores(ka, 1, [&](int j) { stage_c(k, t2, j, sc_k, rts_k, nv_k); });
  }
  {
    const int k = n_tiles - 1;
    const uint32_t sc_p = sc_buf(k), rts_p = rts_buf(k);
    const int nv_p = tile_rows(k);
#pragma unroll
    for (int i = 1; i < 18; ++i) step(1, i, sc_p, rts_p, nv_p, i == 1);
    rescale_o();
    pv(lat_buf(k), [&](int) {});
  }

  // ---- finalize: o = O / (stored-weight sum), lse from the exact sum ----
  const float l_tot = sum_xor32(l);
  const float inv = 1.0f / sum_xor32(lh);
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();  // every wave is done with the latent ring: it stages the output
  if (lg == 0) lse_out[32 * w + li] = m * 0.69314718055994531f + __logf(l_tot);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc8_fence_read(o[ct], ct == 0);
  // Stage the wave's 32 rows (1 KiB each, 16-byte chunk slots XOR-swizzled by
  // row) and store whole rows.
  const uint32_t stage = lds0 + (uint32_t)w * (uint32_t)(32 * kDc * 2);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x2 v = {pack_bf16x2(o[ct][4 * jj + 0] * inv, o[ct][4 * jj + 1] * inv),
                       pack_bf16x2(o[ct][4 * jj + 2] * inv, o[ct][4 * jj + 3] * inv)};
      const uint32_t chunk = ((uint32_t)(4 * ct + jj)) ^ ((uint32_t)li & 15u);
      lds_write_b64(stage + (uint32_t)li * (uint32_t)(2 * kDc) + (chunk << 4) + ((uint32_t)lg << 3), v);
    }
  }
#pragma unroll
  for (int r8 = 0; r8 < 32; r8 += 8) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = lds_read_u32x4(stage + (uint32_t)(r8 + k) * (uint32_t)(2 * kDc) +
                            (((uint32_t)lane ^ (uint32_t)((r8 + k) & 15)) << 4));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(out_rows + (size_t)(32 * w + r8 + k) * kDc + lane * 8));
  }
}

hipError_t launch_decode_latent_fp8(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_heads != 128 || !a.fp8 || a.q_group != 1) return hipErrorInvalidValue;
  const int grid = a.items != nullptr ? a.num_items : a.batch * a.num_splits;
  // Decode reads every cache row once: non-temporal copies (E4M3 V3 64 x
  // 32,768: decode 429.6-430.1 us against 431.0-432.8 us with plain copies,
  // same box, alternated).  Prefill rows re-read their sequence's prefix,
  // which plain copies find in L2 or the Infinity Cache.
  const bool stream_copies = a.q_start == nullptr;
  if (a.block_table != nullptr) {
    if (stream_copies)
      hipLaunchKernelGGL((decode_latent_fp8_kernel<true, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_latent_fp8_kernel<true, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (stream_copies)
      hipLaunchKernelGGL((decode_latent_fp8_kernel<false, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_latent_fp8_kernel<false, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
