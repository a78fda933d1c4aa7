// Latent attention of absorbed-MLA decode with 16 heads and a bf16 cache on
// gfx950 (DeepSeek-V2-Lite: 16 heads).
//
// The same operation as the other decode kernels ("DeepSeek MLA 吸收式缓存：
// 真实权重执行与 FlashMLA 架构边界" §2.2-§2.4, §6.1): every head scores the
// shared 576-wide cache rows, s[h,t] = scale * (q_lat[h] . c_t + q_pe[h] . kR_t),
// and o[h] = sum_t softmax_t(s[h,.]) c_t over one split of the sequence.
//
// Work decomposition: one workgroup per (sequence, split) and one per CU (the
// ring of tiles takes most of the LDS); six waves:
//   - four copy waves issue all 36 wave-wide 1 KiB copies of every tile of 32
//     cache rows into a ring of NBUF LDS tiles, NBUF - 1 tiles ahead (a 64-lane
//     load that misses the cache holds its wave for ~155 cycles, so the waves
//     that compute do not copy, and two copy waves would spend most of a
//     tile's streaming time issuing);
//   - two computing waves split each tile by tokens: wave u scores tokens
//     16u .. 16u+15 against all 16 heads (S^T[token][head] = K . Q^T, 16x16x32
//     bf16 MFMA over the 576 elements), and keeps its own running max, sum and
//     O^T[512 columns][16 heads] for its tokens.  The score fragment of a lane
//     (tokens 4 (l/16) .. +3 of head l%16) is the B-operand layout of the
//     16x16x16 MFMA, so P.V takes the probabilities straight from registers
//     and the V^T operand with one transposing LDS read per 16 columns: the
//     two waves exchange nothing while streaming and meet at one barrier per
//     tile (the tile landed, and the buffer of the tile before can be
//     refilled).
// After the last tile the two states merge (log-sum-exp of the two halves)
// through LDS; each computing wave normalises and stores 256 of the columns.
// Six waves on four SIMDs leave a wave at most 256 registers: the 128 O
// accumulators live in ordinary VGPRs (the library compiles this file with
// VGPR-form MFMAs), next to the 72 of the query block.
// The running max moves (O and the sum are rescaled by exp2 of the
// difference) only when it grows by more than 2^8 in the exp2 domain.
#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_layout.hpp"

namespace mla {

namespace {

// 16x16x16 bf16 MFMA: D[16x16] += A[16x16] * B[16x16] in fp32.  Lane l holds
// A[l%16][4*(l/16) .. +3], B[4*(l/16) .. +3][l%16] and D[4*(l/16) + j][l%16].
__device__ __forceinline__ f32x4 mfma16k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                  0, 0, 0);
}

constexpr int kComp = 2;   // computing waves (token halves of a tile)
constexpr int kVDist = 6;  // V^T fragments read ahead of their MFMA

}  // namespace

template <int NCW, int NBUF, bool PAGED>
__global__ __launch_bounds__((kComp + NCW) * 64)
void decode_latent16_kernel(DecodeArgs a) {
  constexpr int H = 16;
  constexpr int kCopies = kTileDma / NCW;  // copies per copy wave and tile
  static_assert(kTileDma % NCW == 0, "the copies of a tile split evenly over the copy waves");
  static_assert(NBUF == 3 || NBUF == 4, "prefetch distance 2 or 3 tiles");
  static_assert(2 * kCopies < 64, "vmcnt range");
  // LDS: the tile ring.  After the last tile it holds the halves of O the
  // computing waves exchange (16 KiB each), their bf16 output staging (8 KiB
  // each) and the (max, sum) of every head of both waves.
  constexpr int kRing = NBUF * kTileBytes;
  constexpr int kXchg = 0;
  constexpr int kStage = 2 * 16384;
  constexpr int kStat = kStage + 2 * 8192;
  static_assert(kStat + 2 * H * 8 <= kRing, "the merge fits in the ring");
  __shared__ __attribute__((aligned(1024))) char smem[kRing];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hl = lane & 15;   // head of this lane's scores and of its O columns
  const int g4 = lane >> 4;   // 16-lane group
  // uniform splits: a sequence's splits share an XCD (and its L2 copy of the
  // queries); planned decode: workgroup i runs item i, in the order the plan
  // gives; prefill rows go round-robin over the XCDs, longest first
  const bool planned = a.items != nullptr;
  const int item = planned || a.q_start != nullptr ? (int)blockIdx.x : xcd_grouped_index(blockIdx.x, gridDim.x);
  const PlanItem pl = planned ? plan_item(a.items, item, a.batch, a.max_seq_len, a.num_items) : PlanItem{0, 0, 0, 0};
  if (pl.slot < 0) return;  // no partial row to write
  const int qrow = planned ? pl.seq : item / a.num_splits;
  const int split = planned ? item : item - qrow * a.num_splits;
  const int b = a.q_start == nullptr ? qrow : a.batch - 1 - qrow;
  const int cseq = b / a.q_per_seq;    // the sequence whose cached rows it reads
  // decode: the sequence's length; prefill: causal, tokens up to the query's own position
  int T = a.q_start == nullptr ? a.seq_lens[b] : max(a.q_start[cseq], 0) + (b - cseq * a.q_per_seq) + 1;
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
  const int t_begin = planned ? pl.t_begin : split * a.chunk;
  const int t_end = min(T, planned ? pl.t_end : t_begin + a.chunk);
  const bool final_out = !planned && a.num_splits == 1;
  const size_t part = planned ? (size_t)pl.slot : (size_t)b * a.num_splits + split;  // partial slot
  uint16_t* const out_rows = final_out ? a.o_lat + (size_t)b * H * kDc : a.o_part + part * H * kDc;
  float* const lse_out = final_out ? a.lse + (size_t)b * H : a.lse_part + part * H;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  if (t_begin >= t_end) {
    // No tokens in this range: zero weight (o = 0, lse = -inf).
    if (w >= kComp) return;
    for (int r = 8 * w; r < 8 * w + 8; ++r)
      *reinterpret_cast<u32x4*>(out_rows + (size_t)r * kDc + lane * 8) = u32x4{0u, 0u, 0u, 0u};
    if (w == 0 && g4 == 0) lse_out[hl] = -INFINITY;
    return;
  }
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;

  // ---- copy waves: copy i of a tile (i = 0..35) is latent row i (i < 32) or
  // RoPE rows 8 (i-32) .. +7; copy wave j issues copies j, j + NCW, ... ----
  if (w >= kComp) {
    const int j = w - kComp;
    const char* kv_base = uniform_ptr(a.kv);
    const char* pe_base = uniform_ptr(a.pe);
    // Decode reads every cache row once: non-temporal copies (V2-Lite 64 x
    // 4096: decode 49.3 us against 55.0 us with plain copies).  Query rows of
    // a prefill re-read their sequence's prefix, which plain copies find in
    // L2 or the Infinity Cache.
    const bool nt = a.q_start == nullptr;
    auto copy16 = [&](const char* src, uint32_t voff, uint32_t dst) {
      if (nt) dma16<true>(src, voff, dst);
      else dma16<false>(src, voff, dst);
    };
    auto copy_tile = [&](int tile, int buf) {
      const int t0 = t_begin + tile * kTile;
      const int last = min(kTile, t_end - t0) - 1;   // rows past the end re-read the last valid row
      int64_t slot0;
      if (PAGED) {
        // scalar load: a vector load would wait for every copy in flight
        const int blk = scalar_load(a.block_table, (size_t)cseq * a.max_blocks + t0 / a.block_size);
        slot0 = (int64_t)blk * a.block_size + (t0 % a.block_size);
      } else {
        slot0 = (int64_t)cseq * a.seq_stride + t0;
      }
      const uint32_t dst = lds0 + (uint32_t)(buf * kTileBytes);
      // the lane id is recomputed per tile: a value kept live across the loop
      // could be spilled, and its reload would wait for every copy in flight
      const uint32_t ln16 = lane_id() << 4;
#pragma unroll
      for (int k = 0; k < kCopies; ++k) {
        const int i = j + NCW * k;
        if (i < kTile) {
          const uint32_t voff = ln16 ^ (kv_swizzle((uint32_t)i) << 4);
          copy16(uniform_ptr(kv_base + (slot0 + min(i, last)) * a.kv_sb), voff, dst + (uint32_t)(i * kKvRow));
        } else {
          const int pi = i - kTile;
          const uint32_t r = (uint32_t)(8 * pi) + (ln16 >> 7);
          const uint32_t c = ((ln16 >> 4) & 7u) ^ pe_swizzle(r);
          const uint32_t voff = (uint32_t)min((int)r, last) * (uint32_t)a.pe_sb + (c << 4);
          copy16(uniform_ptr(pe_base + slot0 * a.pe_sb), voff, dst + (uint32_t)(kPeRegion + pi * 1024));
        }
      }
    };
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (i < n_tiles) copy_tile(i, i);
    for (int it = 0; it < n_tiles; ++it) {
      // this wave's copies of tile it have landed (later tiles may stay in flight)
      const int later = min(NBUF - 2, n_tiles - 1 - it);
      if (later <= 0) wait_vmcnt<0>();
      else if (later == 1) wait_vmcnt<kCopies>();
      else wait_vmcnt<2 * kCopies>();
      barrier();  // tile it is visible; the computing waves are done with tile it-1
      if (it + NBUF - 1 < n_tiles) copy_tile(it + NBUF - 1, (it + NBUF - 1) % NBUF);
    }
    return;  // a wave that has ended no longer counts at the barriers
  }

  // ---- computing wave u = w: tokens 16u .. 16u+15 of every tile ----
  const int u = w;
  // query block (B operand of the score MFMA): lane (hl, g4) holds
  // q[hl][32 s + 8 g4 .. +7] for s = 0..17 (16 latent steps, then 2 RoPE steps)
  bf16x8 q[18];
  {
    const bf16x8* ql = reinterpret_cast<const bf16x8*>(a.q_lat + ((size_t)b * H + hl) * kDc);
    const bf16x8* qr = reinterpret_cast<const bf16x8*>(a.q_pe + ((size_t)b * H + hl) * kDr);
#pragma unroll
    for (int s = 0; s < 16; ++s) q[s] = ql[s * 4 + g4];
#pragma unroll
    for (int s = 0; s < 2; ++s) q[16 + s] = qr[s * 4 + g4];
  }

  // Per-lane LDS offsets inside a tile (relative to the first row of this
  // wave's half; the swizzles of rows r and 16 + r are equal).  The swizzles
  // XOR only the 16-byte chunk index inside a row, and tiles are 1 KiB
  // aligned, so each fragment address is a base XOR a step constant.
  //   K fragment of step s: token row l%16, elements 32 s + 8 (l/16) .. +7:
  //   latent chunk 4 s + l/16 (s < 16), RoPE chunk 4 (s-16) + l/16.  With
  //   s = 4 m + s4 the latent slot is 16 m + ((l/16 ^ swz) ^ 4 s4).
  //   V^T fragment of column block cb: token rows 4 (l/16) + (l%16)/4,
  //   columns 16 cb + 4 (l%4) .. +3, read transposed so that lane l receives
  //   column 16 cb + l%16 of tokens 4 (l/16) .. +3: chunk 2 cb + (l%4)/2.
  auto k_lane = [](uint32_t l) -> uint32_t {
    const uint32_t r = l & 15u;
    return r * kKvRow + (((l >> 4) ^ kv_swizzle(r)) << 4);
  };
  auto pe_lane = [](uint32_t l) -> uint32_t {
    const uint32_t r = l & 15u;
    return kPeRegion + r * kPeRow + (((l >> 4) ^ pe_swizzle(r)) << 4);
  };
  auto v_lane = [](uint32_t l) -> uint32_t {
    const uint32_t r = 4 * (l >> 4) + ((l & 15u) >> 2);
    return r * kKvRow + ((((l & 3u) >> 1) ^ kv_swizzle(r)) << 4) + ((l & 1u) << 3);
  };

  f32x4 o[32];  // o[cb][j] = O^T[16 cb + 4 g4 + j][head hl] over this wave's tokens
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of the raw scores q.k of head hl (this wave's tokens)
  float l_sum = 0.f;        // this lane's share of sum_t exp2((s - m_ref) * c2)
  const float c2 = a.scale_log2;

  for (int it = 0; it < n_tiles; ++it) {
    barrier();  // tile it landed; both computing waves are done with tile it-1
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t half = lds0 + (uint32_t)((it % NBUF) * kTileBytes);
    const uint32_t ln = lane_id();
    const uint32_t kb0 = half + (uint32_t)(u * 16 * kKvRow) + k_lane(ln);
    const uint32_t pb0 = half + (uint32_t)(u * 16 * kPeRow) + pe_lane(ln);
    auto k_addr = [&](int s) -> uint32_t {
      if (s < 16) return (kb0 ^ ((uint32_t)(s & 3) << 6)) + 256u * (uint32_t)(s >> 2);
      return pb0 ^ ((uint32_t)(s - 16) << 6);
    };

    // ---- scores S^T[token 16u + 4 g4 + j][head hl] ----
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    bf16x8 ka[3];
    ka[0] = lds_read_b128(k_addr(0));
    ka[1] = lds_read_b128(k_addr(1));
#pragma unroll
    for (int s = 0; s < 18; ++s) {
      if (s + 2 < 18) ka[(s + 2) % 3] = lds_read_b128(k_addr(s + 2));
      sc = mfma16(ka[s % 3], q[s], sc);
      __builtin_amdgcn_sched_barrier(0);
    }

    // V^T fragments do not depend on the scores: the first reads go out
    // before the softmax
    const uint32_t vb0 = half + (uint32_t)(u * 16 * kKvRow) + v_lane(ln);
    auto va_load = [&](int cb) -> bf16x4 { return lds_read_tr16(vb0 ^ ((uint32_t)cb << 5)); };
    bf16x4 va[kVDist + 1];
#pragma unroll
    for (int cb = 0; cb < kVDist; ++cb) va[cb] = va_load(cb);

    // ---- mask the ragged tail ----
    const int nvalid = min(kTile, t_end - (t_begin + it * kTile));
    if (nvalid < kTile) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (16 * u + 4 * g4 + j >= nvalid) sc[j] = -INFINITY;
    }

    // ---- online softmax of this wave's tokens ----
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(m_ref, mx);
    // m_ref = -inf only while every token of this wave so far was masked
    // (then no head grows: all its scores are -inf)
    const bool grow = (m_new - m_ref) * c2 > kRescaleLog2;
    if (__ballot(grow) != 0) {
      const float alpha = grow ? fast_exp2((m_ref - m_new) * c2) : 1.0f;
      l_sum *= alpha;
      m_ref = grow ? m_new : m_ref;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) o[cb] *= alpha;
    }
    const float mb = m_ref == -INFINITY ? 0.f : m_ref * c2;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(fmaf(sc[j], c2, -mb));
    l_sum += (p[0] + p[1]) + (p[2] + p[3]);
    const bf16x4 pb = __builtin_bit_cast(bf16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});

    // ---- O^T[c][head] += V^T[c][tokens] . P^T[tokens][head] ----
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      if (cb + kVDist < 32) va[(cb + kVDist) % (kVDist + 1)] = va_load(cb + kVDist);
      o[cb] = mfma16k16(va[cb % (kVDist + 1)], pb, o[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- merge the two token halves and store ----
  // Wave u keeps columns [256 u, 256 u + 256) (blocks 16 u .. 16 u + 15) and
  // hands the other half of its O to the other wave.
  barrier();  // both computing waves are done with the ring
  const float l_tot = sum_xor32(sum_xor16(l_sum));
  const uint32_t stat = lds0 + kStat;
  if (g4 == 0) lds_write_u32x2(stat + (uint32_t)((u * H + hl) * 8), u32x2{__float_as_uint(m_ref), __float_as_uint(l_tot)});
  const uint32_t x_mine = lds0 + kXchg + (uint32_t)(u * 16384) + (uint32_t)lane * 16u;   // written by the other wave
  const uint32_t x_other = lds0 + kXchg + (uint32_t)((1 - u) * 16384) + (uint32_t)lane * 16u;
  if (u == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) lds_write_f32x4(x_other + k * 1024, o[16 + k]);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) lds_write_f32x4(x_other + k * 1024, o[k]);
  }
  barrier();  // both halves and both states are published
  const u32x2 st = lds_read_u32x2(stat + (uint32_t)(((1 - u) * H + hl) * 8));
  const float m_oth = __uint_as_float(st[0]), l_oth = __uint_as_float(st[1]);
  // wave 0 always has a valid token (the first of the range), so m is finite
  const float m = fmaxf(m_ref, m_oth);
  const float f_me = fast_exp2((m_ref - m) * c2), f_oth = fast_exp2((m_oth - m) * c2);
  const float l_all = fmaf(f_me, l_tot, f_oth * l_oth);
  const float inv = 1.0f / l_all;
  const float g_me = f_me * inv, g_oth = f_oth * inv;
  if (u == 0 && g4 == 0) lse_out[hl] = m * a.scale + __logf(l_all);

  // Stage the bf16 rows (16 heads x 256 columns, chunk slots XOR-swizzled by
  // row) and store whole 512-byte row segments.
  const uint32_t stage = lds0 + kStage + (uint32_t)(u * 8192);
  auto put = [&](int k, f32x4 mine) {
    const f32x4 oth = lds_read_f32x4(x_mine + k * 1024);
    const f32x4 v = mine * g_me + oth * g_oth;
    // columns 16 k + 4 g4 .. +3 -> 8 bytes at chunk 2 k + g4/2, half g4 % 2
    const uint32_t chunk = ((uint32_t)(2 * k + (g4 >> 1))) ^ (uint32_t)hl;
    lds_write_b64(stage + (uint32_t)hl * 512u + (chunk << 4) + ((uint32_t)(g4 & 1) << 3),
                  u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
  };
  if (u == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) put(k, o[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) put(k, o[16 + k]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t L = (uint32_t)(64 * k + lane);
    const uint32_t row = L >> 5, ch = L & 31u;
    const u32x4 v = lds_read_u32x4(stage + row * 512u + ((ch ^ (row & 15u)) << 4));
    // non-temporal: nothing in the kernel reads the rows again
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out_rows + (size_t)row * kDc + 256 * u + ch * 8));
  }
}

// Four copy waves (nine copies each per tile) and a ring of three tiles (two
// in flight ahead of the one being computed).  Measured at 64 sequences x
// 4096 tokens: streaming alone (the computing waves skipping their work) runs
// at the same rate with two tiles ahead as with three, and the whole kernel
// ran ~1 us faster with the smaller ring; four copy waves 50.3 us, three
// 51.2 us, six 50.5 us (same box, alternated).
hipError_t launch_decode_latent16(const DecodeArgs& a, hipStream_t stream) {
  constexpr int kNcw = 4, kNbuf = 3;
  const int grid = a.items != nullptr ? a.num_items : a.batch * a.num_splits;
  const int threads = (kComp + kNcw) * 64;
  if (a.block_table != nullptr) {
    hipLaunchKernelGGL((decode_latent16_kernel<kNcw, kNbuf, true>), dim3(grid), dim3(threads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_latent16_kernel<kNcw, kNbuf, false>), dim3(grid), dim3(threads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
