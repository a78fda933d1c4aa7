// Latent attention of absorbed-MLA decode on gfx950.
//
// For one sequence b and one split of its cached tokens, every head h scores
// the shared 576-wide cache rows (512 latent c_t + 64 RoPE key kR_t):
//   s[h,t] = scale * (q_lat[b,h] . c_t + q_pe[b,h] . kR_t)
// then an online softmax over t and the latent aggregate o[h] = sum_t p c_t
// ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2-§2.4 and
// §6.1: absorbed decode is MQA with a 576-wide key whose first 512 elements
// are also the value).
//
// This kernel runs 32 and 64 heads with a bf16 cache and 16, 32 and 64 heads
// with an E4M3 cache (16 heads with a bf16 cache: decode_latent16.hip).
//
// Work decomposition: one workgroup per (sequence, split), NW = H/16 waves.
//   - The workgroup streams its token range in tiles of 32 cache rows
//     (36,864 bytes) from HBM into LDS with 16-byte direct-to-LDS loads; each
//     row is read from HBM exactly once, through a ring of NBUF tile buffers
//     (prefetch distance NBUF - 1 tiles).
//   - Scores: wave w owns heads 16w .. 16w+15.  Its 16 x 576 query block stays
//     in registers as the B operand of S^T[token][head] = K . Q^T
//     (16x16x32 bf16 MFMA), so a lane holds scores of one head and the
//     softmax row reductions stay within a lane plus two cross-lane steps.
//   - P.V: the waves split the 512 latent columns instead of the heads: wave
//     w accumulates O^T[c][head] for columns [w*512/NW, (w+1)*512/NW) and all
//     H heads.  The bf16 probability fragments (already in the MFMA operand
//     layout) are exchanged through LDS, so every V^T element of a tile is
//     fetched with the (slow) transposing LDS read exactly once, and each V^T
//     fragment feeds NW MFMAs.
//   - The running max of a head moves (and O is rescaled by exp2 of the
//     difference) only when it grows by more than 2^8 in the exp2 domain; the
//     owner wave publishes the factor through LDS, so rescales are rare after
//     the first tile.
#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_layout.hpp"

namespace mla {

// Waves per SIMD: the bf16 rings (one tile at 32 heads, two at 64) leave room
// for two workgroups per CU, so a wave is held to half the registers; an E4M3
// ring (four raw tiles and the bf16 tile) takes one workgroup per CU.
template <int NW, int NBUF, bool FP8>
constexpr int narrow_waves_per_simd() { return FP8 ? 1 : 2; }

template <int NW, int NBUF, bool PAGED, bool FP8>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(narrow_waves_per_simd<NW, NBUF, FP8>(), narrow_waves_per_simd<NW, NBUF, FP8>())))
void decode_latent_kernel(DecodeArgs a) {
  constexpr int H = NW * 16;
  // bf16 tile copies: each wave copies KV_PW latent rows; the 4 RoPE copies
  // (8 rows each) go to waves 0..3 (or are shared evenly among fewer).
  constexpr int KV_PW = kTile / NW;       // latent rows per wave
  constexpr int PE_W = NW < 4 ? NW : 4;   // waves that copy RoPE rows
  constexpr int PE_PW = 4 / PE_W;         // RoPE copies per such wave
  constexpr int CB = 32 / NW;             // 16-column blocks of O owned by a wave
  constexpr int C = 512 / NW;             // latent columns owned by a wave
  static_assert(kTile % NW == 0 && 4 % PE_W == 0, "tile copies must split evenly");
  // E4M3 tiles (FP8): the raw tile (latent rows, RoPE rows, per-token scales)
  // streams into a ring of raw buffers and its codes are widened once per
  // tile into a single bf16 tile in the layout the bf16 path reads (exact:
  // every E4M3 value is a bf16 value).  The token scale s_t enters in fp32:
  // score = s_t (q . code_t), and P.V multiplies code_t by p_t s_t, rounded
  // to bf16 as p_t alone would be.  Copies per wave and
  // tile: KV8 latent copies (2 rows each) plus E8 extras (RoPE halves, the
  // scales, or a dummy copy so that every wave issues the same number).
  constexpr int KV8 = 16 / NW;
  constexpr int E8 = (3 + NW - 1) / NW;
  constexpr int kCopies8 = KV8 + E8;
  static_assert(!FP8 || NBUF > 1, "the E4M3 path uses a ring of raw tiles");
  // LDS: tile ring (bf16 tiles, or raw tiles plus one bf16 tile), then the
  // probability exchange (one 1 KiB fragment per wave), the per-head rescale
  // factors / reciprocal sums, and the flags.
  constexpr int kBf16Off = FP8 ? ((NBUF * kRawTileBytes + 1023) / 1024) * 1024 : 0;
  constexpr int kRing = kBf16Off + (FP8 ? kTileBytes : NBUF * kTileBytes);
  constexpr int kPOff = kRing;
  constexpr int kAlphaOff = kPOff + NW * 1024;
  constexpr int kFlagOff = kAlphaOff + H * 4;
  constexpr int kSmem = kFlagOff + 64;
  static_assert(NW * C * 32 <= kRing, "epilogue staging (16 rows x C bf16 per wave) must fit in the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hl = lane & 15;   // row/column within a 16-block
  const int g4 = lane >> 4;   // 16-lane group
  // uniform splits: a sequence's splits share an XCD (and its L2 copy of the
  // queries); planned decode: workgroup i runs item i, in the order the plan
  // gives; prefill rows go round-robin over the XCDs, longest first
  const bool planned = a.items != nullptr;
  const int item = planned || a.q_start != nullptr ? (int)blockIdx.x : xcd_grouped_index(blockIdx.x, gridDim.x);
  // query row: its queries and outputs.  Prefill rows run last query first:
  // the longest causal prefixes start earliest, so the launch ends balanced.
  // A planned decode reads its sequence, token range and partial row from
  // the plan.
  const PlanItem pl = planned ? plan_item(a.items, item, a.batch, a.max_seq_len, a.num_items) : PlanItem{0, 0, 0, 0};
  if (pl.slot < 0) return;  // no partial row to write
  const int qrow = planned ? pl.seq : item / a.num_splits;
  const int split = planned ? item : item - qrow * a.num_splits;
  const int b = a.q_start == nullptr ? qrow : a.batch - 1 - qrow;
  const int cb = b / a.q_per_seq;      // the sequence whose cached rows it reads
  const int h = w * 16 + hl;  // head whose scores this lane computes

  // decode: the sequence's length; prefill: causal, tokens up to the query's own position
  int T = a.q_start == nullptr ? a.seq_lens[b] : max(a.q_start[cb], 0) + (b - cb * a.q_per_seq) + 1;
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
  const int t_begin = planned ? pl.t_begin : split * a.chunk;
  const int t_end = min(T, planned ? pl.t_end : t_begin + a.chunk);
  const bool final_out = !planned && a.num_splits == 1;
  const size_t part = planned ? (size_t)pl.slot : (size_t)b * a.num_splits + split;  // partial slot
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int col0 = w * C;     // first latent column of this wave's P.V share

  if (t_begin >= t_end) {
    // No tokens in this range: zero weight (o = 0, lse = -inf).
    for (int r = 0; r < 16; ++r) {
      const size_t row = (size_t)(w * 16 + r);
      uint16_t* dst = final_out ? a.o_lat + ((size_t)b * a.num_heads + row) * kDc
                                : a.o_part + (part * a.num_heads + row) * kDc;
      *reinterpret_cast<u32x4*>(dst + lane * 8) = u32x4{0u, 0u, 0u, 0u};
    }
    if (g4 == 0) {
      if (final_out) a.lse[(size_t)b * a.num_heads + h] = -INFINITY;
      else a.lse_part[part * a.num_heads + h] = -INFINITY;
    }
    return;
  }

  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const char* kv_base = uniform_ptr(a.kv);
  const char* pe_base = uniform_ptr(a.pe);

  // Source of one tile (all wave-uniform): first cache slot, last valid row,
  // LDS destination.  Rows past the end re-read the last valid row.
  struct TileSrc {
    int64_t slot0;
    int last;
    uint32_t dst;
  };
  auto tile_src = [&](int tile, int buf) -> TileSrc {
    const int t0 = t_begin + tile * kTile;
    TileSrc ts;
    ts.last = min(kTile, t_end - t0) - 1;
    if (PAGED) {
      // Scalar load (constant address space): a vector load here would make
      // the compiler wait for every tile copy in flight before using it.
      const auto* table = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
          reinterpret_cast<uintptr_t>(a.block_table));
      const int blk = table[(size_t)cb * a.max_blocks + t0 / a.block_size];
      ts.slot0 = (int64_t)blk * a.block_size + (t0 % a.block_size);
    } else {
      ts.slot0 = (int64_t)cb * a.seq_stride + t0;
    }
    ts.dst = lds0 + buf * (FP8 ? kRawTileBytes : kTileBytes);
    return ts;
  };
  // Per-lane offsets come from the lane id (mbcnt) of the current iteration
  // rather than being kept live across the loop: a spilled value's scratch
  // reload would wait for every tile copy in flight (vmcnt counts in issue
  // order).  ln16 = 16 * lane.
  auto copy_kv = [&](const TileSrc& ts, int r, uint32_t ln16) {  // latent row r
    const int64_t slot = ts.slot0 + min(r, ts.last);
    const uint32_t voff = ln16 ^ (kv_swizzle(r) << 4);
    dma16(uniform_ptr(kv_base + slot * a.kv_sb), voff, ts.dst + r * kKvRow);
  };
  auto copy_pe = [&](const TileSrc& ts, int i, uint32_t ln16) {  // RoPE rows 8i .. 8i+7
    const uint32_t r = 8 * i + (ln16 >> 7);
    const uint32_t c = ((ln16 >> 4) & 7u) ^ pe_swizzle(r);
    const uint32_t voff = (uint32_t)min((int)r, ts.last) * (uint32_t)a.pe_sb + (c << 4);
    dma16(uniform_ptr(pe_base + ts.slot0 * a.pe_sb), voff, ts.dst + kPeRegion + i * 1024);
  };
  // Copy k of this wave: latent row w*KV_PW + k, then (waves < PE_W) RoPE
  // copy w*PE_PW + k - KV_PW.
  const bool pe_wave = w < PE_W;
  const int n_copy = KV_PW + (pe_wave ? PE_PW : 0);
  auto issue_copy = [&](const TileSrc& ts, int k, uint32_t ln16) {
    if (k < KV_PW) copy_kv(ts, w * KV_PW + k, ln16);
    else copy_pe(ts, w * PE_PW + (k - KV_PW), ln16);
  };

  // E4M3 raw tile: latent row r at r*512, RoPE row r at kRawPeOff + r*64,
  // scale of row r at kRawScaleOff + 4r.  Rows past the end re-read the last
  // valid row (also for the scales, so no read leaves the sequence).
  // ln = lane id.
  auto copy8_kv = [&](const TileSrc& ts, int k, uint32_t ln) {  // latent rows 2k, 2k+1
    const uint32_t r = (uint32_t)min(2 * k + (int)(ln >> 5), ts.last);
    const uint32_t voff = r * (uint32_t)a.kv_sb + ((ln & 31u) << 4);
    dma16(uniform_ptr(kv_base + ts.slot0 * a.kv_sb), voff, ts.dst + k * 1024);
  };
  auto copy8_pe = [&](const TileSrc& ts, int k, uint32_t ln) {  // RoPE rows 16k .. 16k+15
    const uint32_t r = (uint32_t)min(16 * k + (int)(ln >> 2), ts.last);
    const uint32_t voff = r * (uint32_t)a.pe_sb + ((ln & 3u) << 4);
    dma16(uniform_ptr(pe_base + ts.slot0 * a.pe_sb), voff, ts.dst + kRawPeOff + k * 1024);
  };
  auto copy8_scale = [&](const TileSrc& ts, uint32_t ln, uint32_t dst_off) {  // 4 B per lane, row (l%32)
    const uint32_t r = (uint32_t)min((int)(ln & 31u), ts.last);
    dma4(uniform_ptr(reinterpret_cast<const char*>(a.token_scale + ts.slot0)), r * 4u, ts.dst + dst_off);
  };
  auto issue_copy8 = [&](const TileSrc& ts, int k, uint32_t ln) {
    if (k < KV8) {
      copy8_kv(ts, w * KV8 + k, ln);
    } else {
      const int e = w * E8 + (k - KV8);
      if (e < 2) copy8_pe(ts, e, ln);
      else copy8_scale(ts, ln, e == 2 ? kRawScaleOff : kRawDummyOff);
    }
  };

  auto issue_tile = [&](int tile, int buf) {
    const TileSrc ts = tile_src(tile, buf);
    if (FP8) {
      const uint32_t ln = lane_id();
#pragma unroll
      for (int k = 0; k < kCopies8; ++k) issue_copy8(ts, k, ln);
      return;
    }
    const uint32_t ln16 = lane_id() << 4;
#pragma unroll
    for (int k = 0; k < KV_PW; ++k) copy_kv(ts, w * KV_PW + k, ln16);
    if (pe_wave) {
#pragma unroll
      for (int k = 0; k < PE_PW; ++k) copy_pe(ts, w * PE_PW + k, ln16);
    }
  };

  // ---- query block of this wave (B operand of the score MFMA) ----
  // lane (hl, g4) holds q[h][32 s + 8 g4 .. +7] for s = 0..17 (16 latent + 2 rope)
  bf16x8 q[18];
  {
    const bf16x8* ql = reinterpret_cast<const bf16x8*>(a.q_lat + ((size_t)b * a.num_heads + h) * kDc);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * a.num_heads + h) * kDr);
#pragma unroll
    for (int s = 0; s < 16; ++s) q[s] = ql[s * 4 + g4];
#pragma unroll
    for (int s = 0; s < 2; ++s) q[16 + s] = qr[s * 4 + g4];
    // make the query loads complete before any tile copy is in flight, so the
    // compiler's own wait for them cannot drain the tile pipeline
#pragma unroll
    for (int s = 0; s < 18; ++s) asm volatile("" : : "v"(q[s]));
  }

  // Expand raw tile `buf` into the bf16 tile: 32 rows x 72 chunks of 8
  // elements (64 latent + 8 RoPE), each code decoded (OCP E4M3) to bf16 into
  // the swizzled bf16 layout.
  auto expand_tile = [&](int buf) {
    const uint32_t raw = lds0 + buf * kRawTileBytes;
    const uint32_t bt = lds0 + kBf16Off;
    const uint32_t ln = lane_id();
#pragma unroll
    for (int k0 = 0; k0 < 32 * 72; k0 += 64 * NW) {
      const uint32_t k = (uint32_t)(k0 + 64 * w) + ln;
      if (k < 32 * 72) {
        const uint32_t r = k / 72u, c = k - r * 72u;
        uint32_t src, dst;
        if (c < 64u) {
          src = raw + r * 512u + c * 8u;
          dst = bt + r * kKvRow + ((c ^ kv_swizzle(r)) << 4);
        } else {
          src = raw + kRawPeOff + r * 64u + (c - 64u) * 8u;
          dst = bt + kPeRegion + r * kPeRow + (((c - 64u) ^ pe_swizzle(r)) << 4);
        }
        const u32x2 v = lds_read_u32x2(src);
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 f = (e & 1) ? e4m3x2_to_f32<true>(v[e >> 1]) : e4m3x2_to_f32<false>(v[e >> 1]);
          out[e] = pack_bf16x2(f[0], f[1]);
        }
        lds_write_u32x4(dst, out);
      }
    }
  };

  // ---- per-lane LDS addresses inside a tile (swizzled) ----
  // The swizzles XOR only the 16-byte chunk index and tile buffers are 1 KiB
  // aligned, so every fragment address is a per-lane base XOR a step constant
  // plus an immediate offset: one VALU op per read instead of recomputing the
  // swizzle.
  //   score K fragment of step s: token row l%16 (and 16 + l%16), elements
  //   32 s + 8 (l/16) .. +7, i.e. chunk 4 s + l/16 of the latent row (s < 16)
  //   or chunk 4 (s-16) + l/16 of the RoPE row.  With s = 4 m + s4 the latent
  //   chunk is 16 m + ((l/16 ^ swz) ^ 4 s4).
  auto k_base = [&](uint32_t l) -> uint32_t {
    const uint32_t r = l & 15u;
    return r * kKvRow + (((l >> 4) ^ kv_swizzle(r)) << 4);
  };
  auto pe_lane_base = [&](uint32_t l) -> uint32_t {
    const uint32_t r = l & 15u;
    return kPeRegion + r * kPeRow + (((l >> 4) ^ pe_swizzle(r)) << 4);
  };
  //   V^T fragment of column block cb of the wave: rows 4 (l/16) + (l%16)/4
  //   (and +16), columns col0 + 16 cb + 4 (l%4) .. +3 (transposing read: lane
  //   l%16 receives column col0 + 16 cb + l%16).  col0 / 16 is a multiple of
  //   CB, so the chunk 2 (col0/16 + cb) + (l%4)/2 is (2 col0/16 + (l%4)/2) XOR 2 cb.
  auto v_base = [&](uint32_t l) -> uint32_t {
    const uint32_t r = 4 * (l >> 4) + ((l & 15u) >> 2);
    return r * kKvRow + ((((uint32_t)(2 * (col0 >> 4)) | ((l & 3u) >> 1)) ^ kv_swizzle(r)) << 4) + ((l & 1u) << 3);
  };
  static_assert(kTileBytes % 1024 == 0, "tile buffers must stay 1 KiB aligned");

  f32x4 o[CB][NW];   // o[cb][n][j] = O^T[col0 + 16 cb + 4 g4 + j][16 n + hl]
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int n = 0; n < NW; ++n) o[cb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of raw scores q.k of head h (owner)
  float l_sum = 0.f;        // this lane's share of sum_t exp2((s - m_ref) * c) (owner)
  const float c2 = a.scale_log2;

  if (w == 0 && lane == 0) lds_write_u32x2(lds0 + kFlagOff, u32x2{0u, 0u});  // published by the first barrier

  // ---- prologue: tiles 0 .. NBUF-2 in flight ----
  if (NBUF == 1) {
    issue_tile(0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (i < n_tiles) issue_tile(i, i);
  }

  // Copies a wave has in flight per tile: KV_PW, plus PE_PW for waves < PE_W.
  // With a ring of several tiles the next tile's copies are spread over the
  // score loop (one every kCopyStride steps) so the address unit drains them
  // while the MFMAs run instead of stalling the waves at the issue.
  constexpr int kCompCopies = KV_PW + PE_PW;
  constexpr int kCopyStride = kCompCopies > 0 && 18 / kCompCopies > 0 ? 18 / kCompCopies : 1;
  constexpr int kCopiesPerStep = (kCompCopies + 17) / 18;
  static_assert(FP8 || NBUF == 1 || (KV_PW + PE_PW) * kCopyStride <= 18 * kCopiesPerStep,
                "copies must fit in the score loop");
  static_assert(kCopiesPerStep == 1 || kCopyStride == 1, "several copies per step only at stride 1");
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = NBUF == 1 ? 0 : it % NBUF;
    {
      // wait for this wave's copies of tile it (later tiles may stay in flight)
      const int later = NBUF > 1 ? min(NBUF - 2, n_tiles - 1 - it) : 0;
      if constexpr (FP8) {
        if (later <= 0) wait_vmcnt<0>();
        else if (later == 1) wait_vmcnt<kCopies8>();
        else wait_vmcnt<(NBUF > 3 ? 2 * kCopies8 : 0)>();
      } else {
        if (later <= 0) {
          wait_vmcnt<0>();
        } else if (later == 1) {
          if (pe_wave) wait_vmcnt<KV_PW + PE_PW>(); else wait_vmcnt<KV_PW>();
        } else {
          if (pe_wave) wait_vmcnt<(NBUF > 3 ? 2 * (KV_PW + PE_PW) : 0)>(); else wait_vmcnt<(NBUF > 3 ? 2 * KV_PW : 0)>();
        }
      }
    }
    // Tile it is visible to all waves, and every wave has finished iteration
    // it-1, so the buffer of tile it-1 can be refilled.
    barrier();
    const int nxt = it + NBUF - 1;
    const bool copy_next = NBUF > 1 && nxt < n_tiles;
    const TileSrc nts = tile_src(copy_next ? nxt : it, NBUF > 1 ? nxt % NBUF : 0);
    __builtin_amdgcn_sched_barrier(0);
    if (FP8) {
      // the raw tile of iteration it-1 was expanded then: refill its buffer,
      // and expand tile it into the bf16 tile (free: every wave has finished
      // iteration it-1)
      if (copy_next) {
        const uint32_t ln = lane_id();
#pragma unroll
        for (int k = 0; k < kCopies8; ++k) issue_copy8(nts, k, ln);
      }
      expand_tile(buf);
      barrier();  // the bf16 tile is complete
      __builtin_amdgcn_sched_barrier(0);
    }

    const uint32_t tb = lds0 + (FP8 ? kBf16Off : buf * kTileBytes);
    const uint32_t ln = lane_id();
    const uint32_t ln16 = ln << 4;
    const uint32_t kb0 = tb + k_base(ln);
    const uint32_t pb0 = tb + pe_lane_base(ln);

    // ---- scores: S^T[token][head] for tokens 0..15 (s0) and 16..31 (s1) ----
    auto k_addr = [&](int s) -> uint32_t {
      if (s < 16) return (kb0 ^ ((uint32_t)(s & 3) << 6)) + 256u * (uint32_t)(s >> 2);
      return pb0 ^ ((uint32_t)(s - 16) << 6);
    };
    auto k_hi = [&](int s) -> uint32_t { return s < 16 ? 16u * kKvRow : 16u * kPeRow; };
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    bf16x8 ka[3], kb[3];
    ka[0] = lds_read_b128(k_addr(0));
    kb[0] = lds_read_b128(k_addr(0) + k_hi(0));
    ka[1] = lds_read_b128(k_addr(1));
    kb[1] = lds_read_b128(k_addr(1) + k_hi(1));
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      if (s + 2 < 18) {
        const uint32_t ad = k_addr(s + 2);
        ka[(s + 2) % 3] = lds_read_b128(ad);
        kb[(s + 2) % 3] = lds_read_b128(ad + k_hi(s + 2));
      }
      if (!FP8 && NBUF > 1 && s % kCopyStride == 0) {
#pragma unroll
        for (int c = 0; c < kCopiesPerStep; ++c) {
          const int idx = (s / kCopyStride) * kCopiesPerStep + c;
          if (idx < KV_PW + PE_PW && copy_next && idx < n_copy) issue_copy(nts, idx, ln16);
        }
      }
      s0 = mfma16(ka[s % 3], q[s], s0);
      s1 = mfma16(kb[s % 3], q[s], s1);
      __builtin_amdgcn_sched_barrier(0);
    }

    // V^T fragment of the wave's column block cb (independent of the scores,
    // so the first reads are issued before the softmax to hide their latency)
    const uint32_t vb0 = tb + v_base(ln);
    auto va_load = [&](int cb) -> bf16x8 {
      const uint32_t off = vb0 ^ ((uint32_t)cb << 5);
      const bf16x4 lo = lds_read_tr16(off);                // tokens 4 g4 + 0..3
      const bf16x4 hi = lds_read_tr16(off + 16 * kKvRow);  // tokens 16 + 4 g4 + 0..3
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // Many heads (NW > CB): all CB fragments stay in registers and the NW
    // probability fragments stream.  Few heads: the other way round.
    constexpr bool kKeepV = NW > CB;
    constexpr int kVPre = kKeepV ? CB : (CB < 2 ? CB : 2);
    bf16x8 va[kKeepV ? CB : 3];
#pragma unroll
    for (int cb = 0; cb < kVPre; ++cb) va[cb] = va_load(cb);

    // E4M3: q . code_t -> q . k_t with the scales of this lane's tokens
    // 4 g4 + j and 16 + 4 g4 + j (raw tile `buf` holds tile it until the next
    // iteration refills it)
    f32x4 tsA = {}, tsB = {};
    if constexpr (FP8) {
      const uint32_t sr = lds0 + buf * kRawTileBytes + kRawScaleOff + (uint32_t)g4 * 16u;
      tsA = lds_read_f32x4(sr);
      tsB = lds_read_f32x4(sr + 64u);
      s0 *= tsA;
      s1 *= tsB;
    }

    // ---- mask the ragged tail ----
    const int t0 = t_begin + it * kTile;
    const int nvalid = min(kTile, t_end - t0);
    if (nvalid < kTile) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * g4 + j >= nvalid) s0[j] = -INFINITY;
        if (16 + 4 * g4 + j >= nvalid) s1[j] = -INFINITY;
      }
    }

    // ---- online softmax of the wave's own heads ----
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_ref, mx);
    const bool grow = (m_new - m_ref) * c2 > kRescaleLog2;
    const bool any_grow = __ballot(grow) != 0;
    float alpha = 1.0f;
    if (any_grow) {
      alpha = fast_exp2((m_ref - m_new) * c2);
      l_sum *= alpha;
      m_ref = m_new;
    }
    const float mb = m_ref * c2;
    float p[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(fmaf(s0[j], c2, -mb));
      p[4 + j] = fast_exp2(fmaf(s1[j], c2, -mb));
    }
    l_sum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    // B operand of P.V for head 16 w + hl: element i <-> token
    // i<4 ? 4 g4 + i : 16 + 4 g4 + (i-4)
    // E4M3: P.V multiplies the codes, so the probability carries the token scale
    float pv[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pv[j] = FP8 ? p[j] * tsA[j] : p[j];
      pv[4 + j] = FP8 ? p[4 + j] * tsB[j] : p[4 + j];
    }
    const u32x4 pk = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                      pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
    lds_write_u32x4(lds0 + kPOff + w * 1024 + lane * 16, pk);
    if (g4 == 0) lds_write_f32(lds0 + kAlphaOff + h * 4, alpha);
    if (lane == 0) lds_write_u8(lds0 + kFlagOff + w, any_grow ? 1u : 0u);
    barrier();  // probabilities and rescale factors of every head are published
    __builtin_amdgcn_sched_barrier(0);

    // ---- rescale (rare after the first tile) ----
    const u32x2 fl = lds_read_u32x2(lds0 + kFlagOff);  // one byte per wave
    if ((fl[0] | fl[1]) != 0) {
#pragma unroll
      for (int n = 0; n < NW; ++n) {
        const float al = lds_read_f32(lds0 + kAlphaOff + (16 * n + hl) * 4);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][n] *= al;
      }
    }

    // ---- O^T[c][head] += V^T . P^T for the wave's columns, all heads ----
    auto p_load = [&](int n) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, lds_read_u32x4(lds0 + kPOff + n * 1024 + lane * 16));
    };
    if constexpr (kKeepV) {
      bf16x8 pf[2];
      pf[0] = p_load(0);
#pragma unroll
      for (int n = 0; n < NW; ++n) {
        if (n + 1 < NW) pf[(n + 1) & 1] = p_load(n + 1);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) o[cb][n] = mfma16(va[cb], pf[n & 1], o[cb][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      bf16x8 pf[NW];
#pragma unroll
      for (int n = 0; n < NW; ++n) pf[n] = p_load(n);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        if (cb + 2 < CB) va[(cb + 2) % 3] = va_load(cb + 2);
#pragma unroll
        for (int n = 0; n < NW; ++n) o[cb][n] = mfma16(va[cb % 3], pf[n], o[cb][n]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    if (NBUF == 1) {
      barrier();  // the single buffer is free
      if (it + 1 < n_tiles) issue_tile(it + 1, 0);
    }
  }

  // ---- finalize ----
  const float l_tot = sum_xor32(sum_xor16(l_sum));
  const float lse_val = m_ref * a.scale + __logf(l_tot);
  if (g4 == 0) {
    lds_write_f32(lds0 + kAlphaOff + h * 4, 1.0f / l_tot);
    if (final_out) a.lse[(size_t)b * a.num_heads + h] = lse_val;
    else a.lse_part[part * a.num_heads + h] = lse_val;
  }
  barrier();
  float inv[NW];
#pragma unroll
  for (int n = 0; n < NW; ++n) inv[n] = lds_read_f32(lds0 + kAlphaOff + (16 * n + hl) * 4);

  // Each wave holds its C columns for all H heads.  Per 16-head block, stage
  // the bf16 rows in a private LDS region of the (idle) tile ring, chunk slots
  // XOR-swizzled by row, and store whole row segments of C columns: to o_lat
  // (one split) or to the split's bf16 partial rows.
  uint16_t* const out_rows = final_out ? a.o_lat + (size_t)b * a.num_heads * kDc
                                       : a.o_part + part * a.num_heads * kDc;
  const uint32_t stage = lds0 + (uint32_t)w * (uint32_t)(C * 32);
  constexpr int RC = C / 8;                  // 16-byte chunks per bf16 row
  constexpr uint32_t SWZ = RC >= 16 ? 15u : (uint32_t)(RC - 1);
#pragma unroll
  for (int n = 0; n < NW; ++n) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      // columns 16 cb + 4 g4 .. +3 -> 8 bytes at chunk 2 cb + g4/2, half g4 % 2
      const u32x2 v = {pack_bf16x2(o[cb][n][0] * inv[n], o[cb][n][1] * inv[n]),
                       pack_bf16x2(o[cb][n][2] * inv[n], o[cb][n][3] * inv[n])};
      const uint32_t chunk = ((uint32_t)(2 * cb + (g4 >> 1))) ^ ((uint32_t)hl & SWZ);
      lds_write_b64(stage + hl * (uint32_t)(2 * C) + (chunk << 4) + ((g4 & 1) << 3), v);
    }
#pragma unroll
    for (int k = 0; k < (16 * RC) / 64; ++k) {
      const uint32_t L = (uint32_t)(64 * k + lane);
      const uint32_t row = L / RC, ch = L % RC;
      const u32x4 v = lds_read_u32x4(stage + row * (uint32_t)(2 * C) + ((ch ^ (row & SWZ)) << 4));
      // non-temporal: nothing in the kernel reads the rows again (measured
      // 5% faster than plain stores at 16 heads, 64 x 4096 tokens)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out_rows + (size_t)(16 * n + row) * kDc + col0 + ch * 8));
    }
  }
}

template <int NW, int NBUF, bool FP8>
static hipError_t launch_nw(const DecodeArgs& a, int grid, hipStream_t stream) {
  const int threads = NW * 64;
  if (a.block_table != nullptr) {
    hipLaunchKernelGGL((decode_latent_kernel<NW, NBUF, true, FP8>), dim3(grid), dim3(threads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_latent_kernel<NW, NBUF, false, FP8>), dim3(grid), dim3(threads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_latent(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.items != nullptr ? a.num_items : a.batch * a.num_splits;
  if (a.fp8) {
    switch (a.num_heads) {
      case 16: return launch_nw<1, 4, true>(a, grid, stream);
      case 32: return launch_nw<2, 4, true>(a, grid, stream);
      case 64: return launch_nw<4, 4, true>(a, grid, stream);
      case 128: return launch_decode_latent_fp8(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  // prefill with fewer heads: 128 / H queries per workgroup of the wide kernel
  if (a.q_group > 1) return launch_decode_latent_wide(a, stream);
  switch (a.num_heads) {
    case 128: return launch_decode_latent_wide(a, stream);
    case 16: return launch_decode_latent16(a, stream);
    case 32: return launch_nw<2, 1, false>(a, grid, stream);
    case 64: return launch_nw<4, 2, false>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
