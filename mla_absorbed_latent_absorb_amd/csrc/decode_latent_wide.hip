// Latent attention of absorbed-MLA decode on gfx950 for 128 heads: 32-head
// waves, one wave per SIMD, with the P.V product of one cache tile woven into
// the score MFMAs of the next.
//
// Same computation as decode_latent.hip ("DeepSeek MLA 吸收式缓存：真实权重执行与
// FlashMLA 架构边界" §2.2-§2.4, §6.1: every head scores the shared 576-wide
// cache rows, online softmax, o[h] = sum_t p c_t over the 512 latent
// columns), with a different work split and schedule.
//
// One workgroup per (sequence, split), 4 waves, one per SIMD, each with the
// SIMD's whole register file (256 VGPRs + 256 AGPRs).
//   - Tiles of 32 cache rows stream from HBM into LDS with 16-byte
//     direct-to-LDS copies: the 32 latent rows (32 KiB) into a ring of NBUF
//     buffers, the 32 RoPE rows (4 KiB) into a ring of NBUF - 1 buffers (a
//     tile's RoPE rows are dead once it is scored, one step before its latent
//     rows, which P.V still reads).
//   - The query block reaches the registers through LDS: whole 1 KiB rows are
//     copied direct-to-LDS (coalesced), then read back in the MFMA operand
//     layout.  Loaded straight into that layout, every load instruction would
//     touch 16 rows, which the address path serves at a fraction of the rate.
//   - Scores: wave w owns heads 32w .. 32w+31.  Per 32-wide k-step it runs
//     four independent 16x16x32 MFMAs (2 token halves x 2 head halves) with
//     its 32 x 576 query block in VGPRs as the B operand: every K fragment
//     read from LDS feeds 32 heads, half the LDS traffic of 16-head waves.
//   - P.V: wave w accumulates O^T[c][head] for latent columns [128w, 128w+128)
//     and all 128 heads in 32x32x16 tiles: 256 accumulators in AGPRs.  The
//     bf16 probabilities of every head go through LDS in the B-operand layout.
//   - Schedule: iteration k runs, in one instruction stream, the 72 score
//     MFMAs of tile k+1 and the 32 P.V MFMAs of tile k (independent work, so
//     the LDS latency of either is covered by the other's matrix work), then
//     the online softmax of tile k+1, whose probabilities, rescale factors and
//     flags go to the other half of double-buffered LDS slots.  One workgroup
//     barrier per tile.
//   - The running max of a head moves only when it grows by more than
//     2^kRescaleLog2 in the exp2 domain, so O is rarely rescaled.
// (A bf16 cache; an E4M3 cache with 128 heads runs decode_latent_fp8.hip.)
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_layout.hpp"

namespace mla {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Both MFMA kinds are issued as inline asm so the register classes are ours:
// the P.V accumulators live in AGPRs ("a"), the query block, score
// accumulators and fragments in VGPRs.  (With builtins the compiler gives
// every MFMA accumulator of the function the same class and runs out of
// registers.)  The hazards the compiler would cover are then ours:
//   - a chain's first MFMA takes a literal 0 accumulator, later ones
//     accumulate into exactly the same registers (forwarded by the matrix
//     core);
//   - MFMA inputs come from LDS reads, covered by the compiler's lgkmcnt waits
//     on asm operands, and are overwritten only by later LDS reads, which
//     return after the MFMA has read them;
//   - VALU reads of a result wait 24 cycles after the last MFMA (drain_v /
//     acc_fence_read); VALU writes of an accumulator precede its next MFMA by
//     8 cycles (acc_fence_write).

// 16x16x32 bf16, accumulator in VGPRs.  Lane l holds A[l%16][8*(l/16) .. +7],
// B[8*(l/16) .. +7][l%16], D[4*(l/16) + j][l%16].
__device__ __forceinline__ f32x4 mfma16_v_first(bf16x8 a, bf16x8 b) {
  f32x4 d;
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ f32x4 mfma16_v(bf16x8 a, bf16x8 b, f32x4 c) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
  return c;
}
// 32x32x16 bf16, accumulator in AGPRs.  Lane l holds A[l%32][8*(l/32) .. +7],
// B[8*(l/32) .. +7][l%32], D[8*(j/4) + 4*(l/32) + j%4][l%32] for j = 0..15.
__device__ __forceinline__ void mfma32_a(bf16x8 a, bf16x8 b, f32x16& c) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Ordering points (volatile asm keeps its order; each names one value so the
// compiler's own reads / copies of it stay after / before).  The first of a
// run carries the wait states.
__device__ __forceinline__ void drain_v(f32x4& c, bool first) {
  if (first) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(c));
  else asm volatile("" : "+v"(c));
}
__device__ __forceinline__ void acc_fence_read(f32x16& c, bool first) {
  if (first) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(c));
  else asm volatile("" : "+a"(c));
}
__device__ __forceinline__ void acc_fence_write(f32x16& c, bool last) {
  if (last) asm volatile("s_nop 7" : "+a"(c));
  else asm volatile("" : "+a"(c));
}

// Latent rows of a tile in LDS: 32 blocks of 1 KiB, block 8 (r / 8) + c / 8
// holding 16-byte chunks c .. c+7 (c a multiple of 8) of rows r .. r+7 (r a
// multiple of 8) as eight 128-byte rows, chunk c of row r at 16-byte slot
// (c % 8) ^ lat_swz(r).  A direct-to-LDS copy fills one block (eight rows x
// 128 bytes, whole cache lines) from a per-lane source offset that stays the
// same for every block of a wave; the K fragment read (16 rows, one chunk)
// and the transposing V^T read (4 rows x 4 adjacent chunks) become a per-lane
// base plus an immediate.  The swizzle was chosen by measurement (LDS read
// rate of both patterns over 264 candidates): both reads run at the best
// rate seen for them (~210 and ~160 B/clk per CU with 8 waves).
__device__ __forceinline__ uint32_t lat_swz(uint32_t r) {
  return (((r >> 1) & 1u) * 6u) ^ (((r >> 2) & 1u) * 4u) ^ (((r >> 3) & 1u) * 3u);
}

}  // namespace

// STREAM: tile copies with the non-temporal bit (planned decode: every cache
// row is read exactly once; paged V3 with lengths U[1024, 16384]: decode 1.5%
// faster, same box).  Uniform splits keep plain copies (the 32 x 4096 decode
// measured the same or slower with them) and prefill re-reads its prefixes.
template <int NBUF, bool PAGED, bool STREAM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_latent_wide_kernel(DecodeArgs a) {
  static_assert(NBUF >= 3, "a tile's latent rows stay live for two iterations");
  constexpr int NW = 4;                   // waves: one per SIMD
  constexpr int H = NW * 32;              // heads
  constexpr int NT = NW;                  // 32-head tiles (all heads)
  constexpr int C = 512 / NW;             // latent columns owned by a wave in P.V
  constexpr int CT = C / 32;              // their 32-column tiles
  constexpr int KV_PW = kTile / NW;       // latent rows copied per wave and tile
  constexpr int PE_PW = 4 / NW;           // RoPE copies (8 rows each) per wave
  constexpr int kCopies = KV_PW + PE_PW;  // copies per wave and tile
  constexpr int NLAT = NBUF;              // latent ring length
  constexpr int NPE = NBUF - 1;           // RoPE ring length
  constexpr int kLatBytes = kTile * kKvRow;
  constexpr int kPeBytes = kTile * kPeRow;
  constexpr int kPeRing = 0;                    // RoPE ring, then the latent ring
  constexpr int kLatRing = kPeRing + NPE * kPeBytes;
  constexpr int kPBuf = NW * 2048;              // one tile's probabilities, [head tile][k-step] 1 KiB
  constexpr int kPOff = kLatRing + NLAT * kLatBytes;
  constexpr int kAlphaOff = kPOff + 2 * kPBuf;  // [2][H] rescale factors, then 1/l
  constexpr int kFlagOff = kAlphaOff + 2 * H * 4;  // [2][8] byte per wave: its softmax rescaled
  constexpr int kSmem = kFlagOff + 64;
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  // query staging (prologue only): per wave 16 latent rows (16 KiB) + 16
  // RoPE rows (2 KiB), from latent buffer 2 on (latent buffers 2 .. 3 and the
  // probability slots, all unused until tile 2 is issued)
  constexpr int kQStage = kLatRing + 2 * kLatBytes;
  constexpr int kQWave = 16 * 1024 + 2048;
  static_assert(NBUF == 4 && kQStage + NW * kQWave <= kAlphaOff, "query staging must fit before the factors");
  static_assert(NW * 32 * C * 2 <= kPOff, "epilogue staging must fit in the rings");
  static_assert(kLatBytes % 1024 == 0 && kPeBytes % 1024 == 0 && kLatRing % 1024 == 0 && kPOff % 1024 == 0,
                "buffers must stay 1 KiB aligned");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  // score / softmax layout (16x16 tiles): head 32w + 16 hh + h16, tokens
  // 16 th + 4 q4 + j
  const int h16 = lane & 15;
  const int q4 = lane >> 4;
  // P.V / output layout (32x32 tiles): head 32 n + h32, columns 8 (j/4) + 4 g2 + j%4
  const int h32 = lane & 31;
  const int g2 = lane >> 5;
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
  // Workgroup rows: decode, one sequence (128 heads); prefill, one query (128
  // heads), or with fewer heads a group of QG = 128 / H consecutive queries of
  // one sequence (row r = query r / H, head r % H; one split).
  const int QG = a.q_group;
  const int groups = (a.q_per_seq + QG - 1) / QG;                     // workgroups per sequence
  const int n_wg = QG > 1 ? (a.batch / a.q_per_seq) * groups : a.batch;
  const int b = a.q_start == nullptr ? qrow : n_wg - 1 - qrow;
  const int cb = b / groups;                // the sequence whose cached rows it reads
  const int i0 = (b - cb * groups) * QG;    // its first query
  const int nq = min(QG, a.q_per_seq - i0);  // queries in this workgroup
  const size_t row0 = (size_t)cb * a.q_per_seq + i0;  // first query row (decode: the sequence)
  const int Hq = a.num_heads;              // heads per query
  const int n_rows = nq * Hq;               // rows that are stored (the rest repeat the last query)
  const int col0 = w * C;  // first latent column of the wave's P.V share

  // decode: the sequence's length; prefill: causal, tokens up to the query's own position
  auto length_of = [&](int qi) {
    int t = a.q_start == nullptr ? a.seq_lens[b] : max(a.q_start[cb], 0) + qi + 1;
    return t < 0 ? 0 : (t > a.max_seq_len ? a.max_seq_len : t);
  };
  const int T = length_of(i0 + nq - 1);
  const int t_begin = planned ? pl.t_begin : split * a.chunk;
  const int t_end = min(T, planned ? pl.t_end : t_begin + a.chunk);
  // query of each 16-row half of this wave (rows 32w + 16hh .. +15) and its tokens
  int qo[2], t_end_h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    qo[hh] = min((32 * w + 16 * hh) / Hq, nq - 1);
    t_end_h[hh] = QG > 1 ? min(length_of(i0 + qo[hh]), t_begin + a.chunk) : t_end;
  }
  const bool final_out = !planned && a.num_splits == 1;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const size_t part = planned ? (size_t)pl.slot : (size_t)b * a.num_splits + split;  // partial slot
  uint16_t* const out_rows = final_out ? a.o_lat + row0 * Hq * kDc : a.o_part + part * Hq * kDc;
  float* const lse_out = final_out ? a.lse + row0 * Hq : a.lse_part + part * Hq;

  if (t_begin >= t_end) {
    // No tokens in this range: zero weight (o = 0, lse = -inf).
    for (int r = 0; r < 32; ++r)
      if (32 * w + r < n_rows)
        *reinterpret_cast<u32x4*>(out_rows + (size_t)(32 * w + r) * kDc + lane * 8) = u32x4{0u, 0u, 0u, 0u};
    if (g2 == 0 && 32 * w + h32 < n_rows) lse_out[32 * w + h32] = -INFINITY;
    return;
  }

  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const char* kv_base = uniform_ptr(a.kv);
  const char* pe_base = uniform_ptr(a.pe);

  // ---- tile copies (HBM -> LDS, 16 B per lane) ----
  // Wave w copies latent blocks (w, k), k = 0..7 (rows 8w .. 8w+7, chunks
  // 8k .. 8k+7) and RoPE rows 8w .. 8w+7 of each tile.  Every iteration
  // issues one tile's copies, also past the last tile: those re-read the last
  // tile's rows into ring buffers that nobody reads, or, for the RoPE buffer
  // that the last iteration scores again, that tile's own bytes.  So the
  // number of copies in flight never depends on the tile count.
  static_assert(KV_PW == 8 && PE_PW == 1, "one latent block row and one RoPE copy per wave");
  struct TileSrc {
    const char* kv0;  // latent row of the source tile's first token (rows of a tile share a page)
    const char* pe0;  // its RoPE row
    uint32_t kvoff;   // per-lane source offset of the wave's latent copies (rows past the end re-read the last)
    uint32_t peoff;   // per-lane source offset of the wave's RoPE copy
    uint32_t lat;     // LDS latent buffer
    uint32_t pe;      // LDS RoPE buffer
  };
  auto lat_buf = [&](int tile) -> uint32_t { return lds0 + kLatRing + (uint32_t)(tile % NLAT) * kLatBytes; };
  auto pe_buf = [&](int tile) -> uint32_t { return lds0 + kPeRing + (uint32_t)(tile % NPE) * kPeBytes; };
  // Row offsets inside a tile fit 32 bits (token strides are below 2^24 bytes).
  const uint32_t kv_sb32 = (uint32_t)a.kv_sb, pe_sb32 = (uint32_t)a.pe_sb;
  // source offsets of the lane's row r = 8w + l/8 in a whole tile
  uint32_t kvoff_full, peoff_full;
  {
    const uint32_t ln = lane_id();
    const uint32_t r = 8u * (uint32_t)w + (ln >> 3);
    kvoff_full = r * kv_sb32 + (((ln & 7u) ^ lat_swz(r)) << 4);
    peoff_full = r * pe_sb32 + (((ln & 7u) ^ pe_swizzle(r)) << 4);
  }
  // Contiguous cache: the source rows of the next tile to copy, advanced by
  // one tile per call of tile_src (tiles are requested in order) and held at
  // the last tile.
  const char* kv_next = kv_base + ((int64_t)cb * a.seq_stride + t_begin) * a.kv_sb;
  const char* pe_next = pe_base + ((int64_t)cb * a.seq_stride + t_begin) * a.pe_sb;
  const uint32_t kv_step = kTile * kv_sb32, pe_step = kTile * pe_sb32;
  auto tile_src = [&](int tile) -> TileSrc {
    const int src = min(tile, n_tiles - 1);
    const int t0 = t_begin + src * kTile;
    const int last = min(kTile, t_end - t0) - 1;
    TileSrc ts;
    if (PAGED) {
      // scalar load: a vector load would make the compiler wait for every
      // tile copy in flight before using it
      const auto* table = reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
          reinterpret_cast<uintptr_t>(a.block_table));
      const int blk = table[(size_t)cb * a.max_blocks + t0 / a.block_size];
      const int64_t slot0 = (int64_t)blk * a.block_size + (t0 % a.block_size);
      ts.kv0 = uniform_ptr(kv_base + slot0 * a.kv_sb);
      ts.pe0 = uniform_ptr(pe_base + slot0 * a.pe_sb);
    } else {
      ts.kv0 = uniform_ptr(kv_next);
      ts.pe0 = uniform_ptr(pe_next);
      if (tile < n_tiles - 1) {
        kv_next += kv_step;
        pe_next += pe_step;
      }
    }
    ts.kvoff = kvoff_full;
    ts.peoff = peoff_full;
    if (last < kTile - 1) {  // ragged tile: rows past the end re-read the last
      const uint32_t ln = lane_id();
      const uint32_t r = 8u * (uint32_t)w + (ln >> 3);
      const uint32_t rc = (uint32_t)min((int)r, last);
      ts.kvoff = rc * kv_sb32 + (((ln & 7u) ^ lat_swz(r)) << 4);
      ts.peoff = rc * pe_sb32 + (((ln & 7u) ^ pe_swizzle(r)) << 4);
    }
    ts.lat = lat_buf(tile);
    ts.pe = pe_buf(tile);
    return ts;
  };
  // Copy k < 8: latent block (w, k) (the immediate offset 128 k moves the
  // source to chunk 8k and the destination by the same amount, hence M0 =
  // block - 128 k); copy 8: the RoPE rows.
  auto issue_copy = [&](const TileSrc& ts, int k) {
    const uint32_t blk0 = ts.lat + (uint32_t)w * 8192u;
    switch (k) {
      case 0: dma16_off<0, 0, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 1: dma16_off<128, 896, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 2: dma16_off<256, 1792, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 3: dma16_off<384, 2688, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 4: dma16_off<512, 3584, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 5: dma16_off<640, 4480, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 6: dma16_off<768, 5376, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      case 7: dma16_off<896, 6272, STREAM>(ts.kv0, ts.kvoff, blk0); break;
      default: dma16<STREAM>(ts.pe0, ts.peoff, ts.pe + (uint32_t)w * 1024u); break;
    }
  };
  auto issue_tile = [&](int tile) {
    const TileSrc ts = tile_src(tile);
#pragma unroll
    for (int k = 0; k < kCopies; ++k) issue_copy(ts, k);
  };

  // ---- prologue ----
  // Copies in issue order: query half 0 (heads 32w .. 32w+15), tile 0, query
  // half 1, tile 1; each query half is read back as soon as it has landed (the
  // query is on the critical path: every split of a sequence fetches the same
  // 147 KB while the whole grid starts at once), and tile 2 goes into the
  // staging area once every wave is done with it.  The splits of a sequence
  // start their query rows at different heads, so they do not all ask for the
  // same lines at the same moment (both orders measured faster).
  const uint32_t qstage = lds0 + kQStage + (uint32_t)w * kQWave;
  // Query half hh: latent row of head j (0..15) at qstage + 1024 j with
  // chunk c at slot c ^ j; RoPE rows of heads 8i .. 8i+7 at qstage + 16 KiB +
  // 1024 i, head j's chunk k at slot 8 (j % 8) + (k ^ ((j / 2) % 8)).  Both
  // make the 16 rows that one fragment read touches land in 16 bank slots.
  auto stage_q = [&](int hh) {
    const size_t head0 = (row0 + (size_t)qo[hh]) * Hq + (size_t)((32 * w + 16 * hh) % Hq);
    const uint32_t ln = lane_id();
    const char* ql = uniform_ptr(reinterpret_cast<const char*>(a.q_lat + head0 * kDc));
    const char* qr = uniform_ptr(reinterpret_cast<const char*>(a.q_pe + head0 * kDr));
    const uint32_t rot = (uint32_t)(split * 2) & 15u;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const uint32_t j = ((uint32_t)jj + rot) & 15u;
      dma16(ql + j * (kDc * 2), (ln ^ j) << 4, qstage + j * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t j = 8 * i + (ln >> 3);
      dma16(qr, j * (kDr * 2) + (((ln & 7u) ^ ((j >> 1) & 7u)) << 4), qstage + 16384 + i * 1024);
    }
  };
  // q[s][hh]: head 32w + 16 hh + h16, elements 32 s + 8 q4 .. +7 (s < 16
  // latent, s = 16, 17 RoPE): the B operand of the score MFMAs
  bf16x8 q[18][2];
  auto read_q = [&](int hh) {
    const uint32_t ln = lane_id();
    const uint32_t j = ln & 15u, qq = ln >> 4;
#pragma unroll
    for (int s = 0; s < 16; ++s) q[s][hh] = lds_read_b128(qstage + j * 1024 + (((4 * s + qq) ^ j) << 4));
#pragma unroll
    for (int s = 0; s < 2; ++s)
      q[16 + s][hh] = lds_read_b128(qstage + 16384 + (j >> 3) * 1024 + ((j & 7u) * 8 + ((4 * s + qq) ^ ((j >> 1) & 7u))) * 16);
    // the reads are complete before the staging area is overwritten
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  stage_q(0);
  issue_tile(0);
  wait_vmcnt<kCopies>();
  read_q(0);
  stage_q(1);
  issue_tile(1);
  wait_vmcnt<kCopies>();
  read_q(1);
  // every wave has read its query block (the staging area is free) and its
  // copies of tile 0 have landed; tile 1 may still be in flight
  barrier();
  issue_tile(2);

  // ---- per-lane LDS addresses inside a tile ----
  //   K fragment of score step s < 16, token half th: row 16 th + l%16, latent
  //   chunk 4 s + l/16, at kb[s % 2] + 16 KiB th + 1 KiB (s / 2), where kb[1]
  //   = kb[0] ^ 64 (the chunk's bit 2 is the step's parity, XORed into a slot
  //   whose bit 2 also depends on the row).  Steps 16, 17: RoPE chunk
  //   4 (s-16) + l/16 at pb0 ^ 64 (s-16) (+ 2 KiB th).
  // Per-lane parts of the fragment addresses, the same for every tile
  // (buffers are 1 KiB aligned, so the ring offset adds and the ^ 64 of the
  // odd bases acts on the lane part alone).
  uint32_t kb_lane, pb_lane, vb_lane, p_lane;
  {
    const uint32_t ln = lane_id();
    const uint32_t r16 = ln & 15u;
    kb_lane = ((r16 >> 3) << 13) + ((r16 & 7u) << 7) + (((ln >> 4) ^ lat_swz(r16)) << 4);
    pb_lane = r16 * kPeRow + (((ln >> 4) ^ pe_swizzle(r16)) << 4);
    const uint32_t g = ln >> 5, i = (ln & 15u) >> 2, cb2 = (ln >> 3) & 2u, a2 = (ln & 3u) >> 1;
    vb_lane = (g << 13) + ((uint32_t)w << 11) + (i << 7) + (((cb2 | a2) ^ (6u * (i >> 1)) ^ (3u * g)) << 4) +
              ((ln & 1u) << 3);
    p_lane = ln << 4;
  }
  auto k_addr_fn = [&](uint32_t kbe, uint32_t kbo, uint32_t pb0, int s) -> uint32_t {
    if (s < 16) return ((s & 1) ? kbo : kbe) + 1024u * (uint32_t)(s >> 1);
    return pb0 ^ ((uint32_t)(s - 16) << 6);
  };
  auto k_hi = [&](int s) -> uint32_t { return s < 16 ? 16u * kKvRow : 16u * kPeRow; };
  //   V^T fragment (column tile ct, k-step kk): the 16-lane group l/16 reads
  //   rows 16 kk + 8 (l/32) + (l%16)/4 (and + 4), columns col0 + 32 ct +
  //   16 ((l/16) % 2) + 4 (l%4) .. +3; lane l receives column col0 + 32 ct +
  //   l%32 of those 4 rows (transposing read).  Row bit 2 (the + 4) and
  //   column-tile bit 0 both land in bit 2 of the slot, so the read is
  //   vb[(ct % 2) ^ (row part / 4)] + 16 KiB kk + 1 KiB (ct / 2) (+ 512 for
  //   the + 4 rows) with vb[1] = vb[0] ^ 64.

  f32x16 o[CT][NT];  // o[ct][n][j] = O^T[col0 + 32 ct + 8 (j/4) + 4 g2 + j%4][32 n + h32]
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int j = 0; j < 16; ++j) o[ct][n][j] = 0.f;
      acc_fence_write(o[ct][n], ct == CT - 1 && n == NT - 1);
    }
  // softmax state of the lane's two heads 32w + 16 hh + h16 (the four lanes
  // with the same h16 hold the same reference max)
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference max of the raw scores q.k
  float l_sum[2] = {0.f, 0.f};              // this lane's share of sum_t exp2((s - m_ref) c2)
  const float c2 = a.scale_log2;

  static_assert(kCopies <= 9, "one copy every other score step");

  typedef f32x4 Scores[2][2];  // [token half th][head half hh]

  // P.V operands, kept across iterations (see `iteration`): probability
  // fragments of the four head tiles, V^T fragments of three column tiles.
  bf16x8 pf[NT], va[3];
#pragma unroll
  for (int n = 0; n < NT; ++n) pf[n] = bf16x8{};
#pragma unroll
  for (int i = 0; i < 3; ++i) va[i] = bf16x8{};
  // P.V MFMA m: k-step m / 16, column tile (m / 4) % 4, head tile m % 4
  auto pv_mfma = [&](int m) {
    const int vi = m >> 2, ct = vi & 3, n = m & 3;
    mfma32_a(va[vi % 3], pf[n], o[ct][n]);
  };

  // One iteration of the pipeline as a single instruction stream.  A wave
  // issues in order and an MFMA holds the issue until the matrix core takes
  // it, so other work overlaps the matrix core only when it sits between two
  // MFMAs: the stream alternates single MFMAs with single other operations
  // (sched_barrier keeps the source order).
  //   - Score phase, 18 steps: the four score MFMAs of k-step s of tile tq
  //     (into sc), separated by the two K reads of step s + 2 and two more
  //     slots: on odd steps one of this wave's copies of tile `nts`; in the
  //     first steps the operand reads of the first P.V MFMAs of tile tv.
  //   - P.V phase: P.V MFMAs m = 0 .. 27 of tile tv with the probabilities of
  //     slot pb, each followed by the operand reads it makes due and one chunk
  //     of the online softmax of the scores just computed.  The softmax writes
  //     the probabilities, rescale factors and flags of slot ps; the running
  //     max and sum change only if commit.
  //   - P.V MFMAs 28 .. 31 are issued at the start of the next iteration (or
  //     after the loop), where they cover the latency of its first LDS reads.
  //     Their operands stay in pf / va, which live across iterations and start
  //     as zeros, so the deferred MFMAs of the first iteration add zeros.
  //   P.V MFMA m: k-step kk = m / 16 (tokens 16 kk .. +15), column tile
  //   ct = (m / 4) % 4, head tile n = m % 4.  The V^T fragment of (kk, ct) is
  //   read two column tiles ahead; the four probability fragments of k-step 0
  //   are replaced by those of k-step 1 right after their last use.
  //   After the deferred MFMAs of tile tv - 1 (DO_PV and rescale_check):
  //   O *= alpha of slot pb if any wave's softmax of tile tv moved its
  //   reference max.
  auto iteration = [&](auto pv_tag, int tq, Scores& sc, int tv, int pb, int ps, bool rescale_check,
                       bool commit, const TileSrc& nts) {
    constexpr bool DO_PV = decltype(pv_tag)::value;
    // one byte per wave; read now, tested after the deferred MFMAs
    const uint32_t flags = DO_PV ? lds_read_u32(lds0 + kFlagOff + pb * 8) : 0u;
    const uint32_t kbe = lat_buf(tq) + kb_lane;
    const uint32_t kbo = kbe ^ 64u;
    const uint32_t pb0 = pe_buf(tq) + pb_lane;
    uint32_t vb0 = 0, vb1 = 0;
    const uint32_t pbase = lds0 + kPOff + (uint32_t)pb * kPBuf + p_lane;
    if (DO_PV) {
      vb0 = lat_buf(tv) + vb_lane;
      vb1 = vb0 ^ 64u;
    }
    auto va_load = [&](int vi) -> bf16x8 {  // vi = 4 kk + ct
      const int ct = vi & 3, kk = vi >> 2;
      const uint32_t imm = (uint32_t)kk * 16u * kKvRow + (uint32_t)(ct >> 1) * 1024u;
      const bf16x4 lo = lds_read_tr16(((ct & 1) ? vb1 : vb0) + imm);
      const bf16x4 hi = lds_read_tr16(((ct & 1) ? vb0 : vb1) + imm + 512u);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto pf_load = [&](int n, int kk) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, lds_read_u32x4(pbase + (uint32_t)(n * 2 + kk) * 1024u));
    };
    constexpr int D = 2;  // score steps of K fragments in flight
    bf16x8 kf[D + 1][2];
#pragma unroll
    for (int st = 0; st < D; ++st) {
      const uint32_t ad = k_addr_fn(kbe, kbo, pb0, st);
      kf[st][0] = lds_read_b128(ad);
      kf[st][1] = lds_read_b128(ad + k_hi(st));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (DO_PV) {
#pragma unroll
      for (int m = 28; m < 32; ++m) {  // deferred from the previous tile
        pv_mfma(m);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (rescale_check && flags != 0u) {  // rare after the first tile
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const float al = lds_read_f32(lds0 + kAlphaOff + (uint32_t)pb * (H * 4) + (32 * n + h32) * 4);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            acc_fence_read(o[ct][n], n == 0 && ct == 0);
            o[ct][n] *= al;
            acc_fence_write(o[ct][n], n == NT - 1 && ct == CT - 1);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- score phase ----
    // slot work of step st (two slots per step): this wave's copy i in the
    // first slot of step 2i + 1, P.V operand preloads in steps 0 .. 3
    auto slot = [&](int st, int k) {
      if (DO_PV && (st & 1) == 1 && k == 0 && (st >> 1) < kCopies) issue_copy(nts, st >> 1);
      if (DO_PV) {
        if (k == 0 && st < 2) pf[2 * st] = pf_load(2 * st, 0);
        else if (k == 1 && st < 2) pf[2 * st + 1] = pf_load(2 * st + 1, 0);
        else if (k == 1 && st == 2) va[0] = va_load(0);
        else if (k == 1 && st == 3) va[1] = va_load(1);
      }
    };
#pragma unroll
    for (int st = 0; st < 18; ++st) {
      const uint32_t ad = st + D < 18 ? k_addr_fn(kbe, kbo, pb0, st + D) : 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int th = e >> 1, hh = e & 1;
        sc[th][hh] = st == 0 ? mfma16_v_first(kf[0][th], q[0][hh])
                             : mfma16_v(kf[st % (D + 1)][th], q[st][hh], sc[th][hh]);
        __builtin_amdgcn_sched_barrier(0);
        if (e < 2) {
          if (st + D < 18) kf[(st + D) % (D + 1)][e] = lds_read_b128(ad + (e ? k_hi(st + D) : 0u));
        } else {
          slot(st, e - 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- P.V phase with the online softmax of tile tq ----
    Scores& sp = sc;
    const int t0q = t_begin + tq * kTile;
    const int nvalid_h[2] = {min(kTile, t_end_h[0] - t0q), min(kTile, t_end_h[1] - t0q)};
    float mx[2], alpha[2], mb[2];
    bool any_grow = false;
    auto softmax_chunk = [&](int c) {
      if (c == 0) {
        drain_v(sp[0][0], true);
        drain_v(sp[0][1], false);
        drain_v(sp[1][0], false);
        drain_v(sp[1][1], false);
        // ragged tail (and, in a query group, tokens past each half's own
        // query): tokens 16 th + 4 q4 + j at or past the half's count
        if (min(nvalid_h[0], nvalid_h[1]) < kTile) {
#pragma unroll
          for (int th = 0; th < 2; ++th)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (16 * th + 4 * q4 + j >= nvalid_h[hh]) sp[th][hh][j] = -INFINITY;
        }
      } else if (c == 1 || c == 2) {
        const int hh = c - 1;
        mx[hh] = vmax(vmax3(vmax3(sp[0][hh][0], sp[0][hh][1], sp[0][hh][2]), sp[0][hh][3], sp[1][hh][0]),
                      vmax3(sp[1][hh][1], sp[1][hh][2], sp[1][hh][3]));
      } else if (c == 3) {
        mx[0] = vmax_xor16(mx[0]);
        mx[1] = vmax_xor16(mx[1]);
      } else if (c == 4) {
        mx[0] = vmax_xor32(mx[0]);
        mx[1] = vmax_xor32(mx[1]);
      } else if (c == 5) {
        bool grow = false;
        float m_new[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          m_new[hh] = vmax(m_ref[hh], mx[hh]);
          grow = grow || (m_new[hh] - m_ref[hh]) * c2 > kRescaleLog2;
        }
        any_grow = __ballot(grow) != 0;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float ex = fast_exp2((m_ref[hh] - m_new[hh]) * c2);
          alpha[hh] = any_grow ? ex : 1.0f;
          const float m_use = any_grow ? m_new[hh] : m_ref[hh];
          mb[hh] = m_use * c2;
          if (commit) m_ref[hh] = m_use;
        }
      } else if (c >= 6 && c < 22) {
        // one of the lane's 16 probabilities per chunk
        const int e = c - 6, th = e >> 3, hh = (e >> 2) & 1, j = e & 3;
        sp[th][hh][j] = fast_exp2(fmaf(sp[th][hh][j], c2, -mb[hh]));
      } else if (c == 22 || c == 23) {
        // B operand of P.V (k-step th of head tile w): lane h' + 32 g' holds
        // tokens 16 th + 8 g' + i; this lane's 4 tokens 16 th + 4 q4 + j are
        // elements 4 (q4 % 2) + j of lane (16 hh + h16) + 32 (q4 / 2)
        const int th = c - 22;
        const uint32_t pw = lds0 + kPOff + (uint32_t)ps * kPBuf + (uint32_t)w * 2048u + (uint32_t)th * 1024u;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x2 pk = {pack_bf16x2(sp[th][hh][0], sp[th][hh][1]), pack_bf16x2(sp[th][hh][2], sp[th][hh][3])};
          const uint32_t dl = (uint32_t)(16 * hh + h16 + 32 * (q4 >> 1));
          lds_write_b64(pw + dl * 16u + (uint32_t)(q4 & 1) * 8u, pk);
        }
      } else if (c == 24 || c == 25) {
        const int hh = c - 24;
        const float psum = ((sp[0][hh][0] + sp[0][hh][1]) + (sp[0][hh][2] + sp[0][hh][3])) +
                           ((sp[1][hh][0] + sp[1][hh][1]) + (sp[1][hh][2] + sp[1][hh][3]));
        const float nl = fmaf(l_sum[hh], alpha[hh], psum);
        if (commit) l_sum[hh] = nl;
      } else if (c == 26) {
        if (q4 == 0) {
          const uint32_t ab = lds0 + kAlphaOff + (uint32_t)ps * (H * 4);
          lds_write_f32(ab + (32 * w + h16) * 4, alpha[0]);
          lds_write_f32(ab + (32 * w + 16 + h16) * 4, alpha[1]);
        }
        if (lane == 0) lds_write_u8(lds0 + kFlagOff + ps * 8 + w, any_grow ? 1u : 0u);
      }
    };
#pragma unroll
    for (int m = 0; m < 28; ++m) {
      if (DO_PV) {
        pv_mfma(m);
        __builtin_amdgcn_sched_barrier(0);
        const int vi = m >> 2, n = m & 3;
        if ((m & 3) == 0 && vi + 2 < 8) va[(vi + 2) % 3] = va_load(vi + 2);
        if (m >= 12 && m < 16) pf[n] = pf_load(n, 1);
      }
      softmax_chunk(m);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Pipeline.  Before the loop: scores and softmax of tile 0 (slot 0).
  // Iteration k, after barrier A (tile k+1 landed: only tile k+2's copies
  // may still be in flight; every wave's probabilities of tile k are in slot
  // k%2; every wave is done with iteration k-1, so the latent buffer of tile
  // k-1 and the RoPE buffer of tile k are free and the copies of tile
  // k + NBUF - 1 go there): the P.V of tile k woven with the scores and
  // softmax of tile k+1 into slot (k+1)%2 (whose previous contents, tile
  // k-1's, were consumed in iteration k-1).  The last tile has no successor:
  // its own rows are scored again and that softmax is not committed (one
  // code path keeps the registers allocated once).
  static_assert(NBUF == 4, "the waits count one tile of copies in flight");
  Scores sc;
  __builtin_amdgcn_sched_barrier(0);
  iteration(std::false_type(), 0, sc, 0, 0, 0, false, true, TileSrc{});
  for (int it = 0; it < n_tiles; ++it) {
    const bool has_next = it + 1 < n_tiles;
    wait_vmcnt<kCopies>();
    barrier();  // barrier A
    __builtin_amdgcn_sched_barrier(0);
    const TileSrc nts = tile_src(it + 3);
    iteration(std::true_type(), has_next ? it + 1 : it, sc, it, it & 1, (it + 1) & 1, it > 0, has_next, nts);
  }
#pragma unroll
  for (int m = 28; m < 32; ++m) pv_mfma(m);  // deferred from the last tile

  // ---- finalize: normalise by the per-head sum and store ----
  float l_tot[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) l_tot[hh] = sum_xor32(sum_xor16(l_sum[hh]));
  // every wave is done with the tiles and the rescale factors, and its last
  // copies (past the last tile) have landed before the rings are reused
  wait_vmcnt<0>();
  barrier();
  if (q4 == 0) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int hd = 32 * w + 16 * hh + h16;
      lds_write_f32(lds0 + kAlphaOff + hd * 4, 1.0f / l_tot[hh]);
      if (hd < n_rows) lse_out[hd] = m_ref[hh] * a.scale + __logf(l_tot[hh]);
    }
  }
  barrier();
  float inv[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) inv[n] = lds_read_f32(lds0 + kAlphaOff + (32 * n + h32) * 4);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc_fence_read(o[ct][n], ct == 0 && n == 0);

  // Per 32-head tile, stage the wave's C columns of the 32 rows in a private
  // region of the latent ring (16-byte chunk slots XOR-swizzled by row) and
  // store whole row segments.
  constexpr int RC = C / 8;                 // 16-byte chunks per bf16 row segment
  constexpr uint32_t SWZ = RC >= 16 ? 15u : (uint32_t)(RC - 1);
  const uint32_t stage = lds0 + (uint32_t)w * (uint32_t)(32 * C * 2);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        // columns 32 ct + 8 jj + 4 g2 .. +3 of head row h32: 8 bytes at chunk
        // 4 ct + jj, half g2
        const u32x2 v = {pack_bf16x2(o[ct][n][4 * jj + 0] * inv[n], o[ct][n][4 * jj + 1] * inv[n]),
                         pack_bf16x2(o[ct][n][4 * jj + 2] * inv[n], o[ct][n][4 * jj + 3] * inv[n])};
        const uint32_t chunk = ((uint32_t)(4 * ct + jj)) ^ ((uint32_t)h32 & SWZ);
        lds_write_b64(stage + (uint32_t)h32 * (uint32_t)(2 * C) + (chunk << 4) + ((uint32_t)g2 << 3), v);
      }
    }
    // all reads first, then the stores: one LDS round trip per head tile
    constexpr int KR = (32 * RC) / 64;
    u32x4 v[KR];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const uint32_t L = (uint32_t)(64 * k + lane);
      const uint32_t row = L / RC, ch = L % RC;
      v[k] = lds_read_u32x4(stage + row * (uint32_t)(2 * C) + ((ch ^ (row & SWZ)) << 4));
    }
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const uint32_t L = (uint32_t)(64 * k + lane);
      const uint32_t row = L / RC, ch = L % RC;
      // Non-temporal stores: every workgroup writes its 128 KiB of partials at
      // the same moment and nothing here reads them again; streaming them
      // past the caches measured 4.5 us faster per V3 launch than plain stores.
      if ((int)(32 * n + row) < n_rows)
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4*>(out_rows + (size_t)(32 * n + row) * kDc + col0 + ch * 8));
    }
  }
}

hipError_t launch_decode_latent_wide(const DecodeArgs& a, hipStream_t stream) {
  if (a.fp8 || a.num_heads * a.q_group != 128 || (a.q_group > 1 && (a.q_start == nullptr || a.num_splits != 1)))
    return hipErrorInvalidValue;
  const int groups = (a.q_per_seq + a.q_group - 1) / a.q_group;
  const int grid = a.items != nullptr ? a.num_items
                                      : (a.q_group > 1 ? (a.batch / a.q_per_seq) * groups : a.batch) * a.num_splits;
  const bool planned = a.items != nullptr;
  if (a.block_table != nullptr) {
    if (planned)
      hipLaunchKernelGGL((decode_latent_wide_kernel<4, true, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_latent_wide_kernel<4, true, false>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    if (planned)
      hipLaunchKernelGGL((decode_latent_wide_kernel<4, false, true>), dim3(grid), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_latent_wide_kernel<4, false, false>), dim3(grid), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
