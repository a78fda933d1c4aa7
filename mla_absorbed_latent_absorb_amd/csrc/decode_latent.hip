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
// Work decomposition (one workgroup per (sequence, split)):
//   - the workgroup streams its token range in tiles of 32 cache rows
//     (36,864 bytes) from HBM into LDS with 16-byte direct-to-LDS loads,
//     each row read exactly once, through a ring of NBUF tile buffers
//     (prefetch distance NBUF - 1 tiles);
//   - each wave owns 16 heads.  Its 16 x 576 query block stays in registers
//     as the B operand of the score product S^T[token][head] = K . Q^T
//     (16x16x32 bf16 MFMA), so a lane holds the scores of one head and the
//     softmax row reductions stay within a lane and across 4 lanes;
//   - the probabilities go straight from the score accumulators to the B
//     operand of O^T[c][head] += V^T . P^T, with V^T read from the same LDS
//     tile by transposing LDS reads: both products run on MFMA and every
//     head shares the one LDS copy of each tile;
//   - the running max is only moved (and O rescaled) when it grows by more
//     than 2^8 in the exp2 domain, so the rescale of the 128 accumulator
//     registers is rare after the first tile.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {

constexpr int kTile = 32;                      // cache rows per tile
constexpr int kKvRow = kDc * 2;                // 1024-byte latent row in LDS
constexpr int kPeRow = kDr * 2;                // 128-byte RoPE row in LDS
constexpr int kPeRegion = kTile * kKvRow;      // RoPE rows follow the 32 latent rows
constexpr int kTileBytes = kTile * (kKvRow + kPeRow);  // 36864
constexpr int kTileDma = kTile + kTile * kPeRow / 1024;  // 36 wave-wide 1 KiB copies per tile
constexpr float kRescaleLog2 = 8.0f;           // lazy-rescale threshold (exp2 domain)

// LDS tile (per ring buffer):
//   [0, 32 KiB)      latent rows: row r holds chunk c (16 bytes = 8 elements)
//                    of token r at chunk slot c ^ kv_swizzle(r)
//   [32, 36 KiB)     RoPE rows: row r holds chunk c of token r at slot
//                    c ^ pe_swizzle(r)
// A wave-wide 1 KiB copy fills one latent row (one token: scalar base
// address) or eight RoPE rows.

template <int NW, int NBUF, bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_latent_kernel(DecodeArgs a) {
  constexpr int LW = NW < 4 ? NW : 4;     // waves that issue the tile copies
  constexpr int LPW = kTileDma / LW;      // copies per loading wave per tile
  constexpr int KV_PW = kTile / LW;       // latent rows per loading wave
  constexpr int PE_PW = (kTile / 8) / LW; // RoPE copies (8 rows each) per loading wave
  static_assert(kTileDma % LW == 0 && kTile % LW == 0 && (kTile / 8) % LW == 0, "tile copies must split evenly");
  __shared__ __attribute__((aligned(1024))) char smem[NBUF * kTileBytes];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hl = lane & 15;   // head within the wave's 16
  const int g4 = lane >> 4;   // 16-lane group
  const int b = blockIdx.x / a.num_splits;
  const int split = blockIdx.x - b * a.num_splits;
  const int h = w * 16 + hl;

  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
  const int t_begin = split * a.chunk;
  const int t_end = min(T, t_begin + a.chunk);
  const bool final_out = a.num_splits == 1;

  float* part_row = nullptr;
  uint16_t* final_row = nullptr;
  if (final_out) {
    final_row = a.o_lat + ((size_t)b * a.num_heads + h) * kDc;
  } else {
    part_row = a.o_part + (((size_t)b * a.num_splits + split) * a.num_heads + h) * kDc;
  }

  if (t_begin >= t_end) {
    // No tokens in this range: zero weight (o = 0, lse = -inf).
    for (int cb = 0; cb < 32; ++cb) {
      if (final_out) {
        *reinterpret_cast<u32x2*>(final_row + cb * 16 + g4 * 4) = u32x2{0u, 0u};
      } else {
        *reinterpret_cast<f32x4*>(part_row + cb * 16 + g4 * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (g4 == 0) {
      if (final_out) a.lse[(size_t)b * a.num_heads + h] = -INFINITY;
      else a.lse_part[((size_t)b * a.num_splits + split) * a.num_heads + h] = -INFINITY;
    }
    return;
  }

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

  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;
  const char* kv_base = uniform_ptr(a.kv);
  const char* pe_base = uniform_ptr(a.pe);

  auto issue_tile = [&](int tile, int buf) {
    if (w >= LW) return;
    const int t0 = t_begin + tile * kTile;
    const int last = min(kTile, t_end - t0) - 1;  // rows past the end re-read the last row
    int64_t slot0;
    if (PAGED) {
      const int blk = a.block_table[(size_t)b * a.max_blocks + t0 / a.block_size];
      slot0 = (int64_t)blk * a.block_size + (t0 % a.block_size);
    } else {
      slot0 = (int64_t)b * a.seq_stride + t0;
    }
    const uint32_t dst = lds0 + buf * kTileBytes;
#pragma unroll
    for (int k = 0; k < KV_PW; ++k) {
      const int r = w * KV_PW + k;
      const int64_t slot = slot0 + min(r, last);
      const uint32_t voff = ((uint32_t)lane ^ kv_swizzle(r)) << 4;
      dma16(uniform_ptr(kv_base + slot * a.kv_sb), voff, dst + r * kKvRow);
    }
#pragma unroll
    for (int k = 0; k < PE_PW; ++k) {
      const int i = w * PE_PW + k;
      const uint32_t r = 8 * i + (lane >> 3);
      const uint32_t c = ((uint32_t)lane & 7u) ^ pe_swizzle(r);
      const uint32_t voff = (uint32_t)min((int)r, last) * (uint32_t)a.pe_sb + (c << 4);
      dma16(uniform_ptr(pe_base + slot0 * a.pe_sb), voff, dst + kPeRegion + i * 1024);
    }
  };

  // ---- per-lane LDS offsets (swizzled) ----
  // score K fragment: token row hl (and 16 + hl), element block d = 32 s + 8 g4
  const uint32_t kx = kv_swizzle(hl);
  uint32_t k_off[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) k_off[m] = hl * kKvRow + (((4u * m + g4) ^ kx) << 4);
  const uint32_t p_off0 = kPeRegion + hl * kPeRow + (((uint32_t)g4 ^ pe_swizzle(hl)) << 4);
  const uint32_t p_off1 = kPeRegion + hl * kPeRow + (((uint32_t)(4 + g4) ^ pe_swizzle(hl)) << 4);
  // P.V fragment: rows 4 g4 + hl/4 (and +16), columns 16 cb + 4 (hl%4) .. +3
  const uint32_t vr = 4 * g4 + (hl >> 2);
  const uint32_t vx = kv_swizzle(vr);
  const uint32_t vsel = (hl & 3) >> 1;
  uint32_t v_off[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) v_off[m] = vr * kKvRow + (((2u * m + vsel) ^ vx) << 4) + ((hl & 1) << 3);

  f32x4 o[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of raw scores q.k (unscaled)
  float l_sum = 0.f;        // this lane's share of sum_t exp2((s - m_ref) * c)
  const float c2 = a.scale_log2;

  // ---- prologue ----
  if (NBUF == 1) {
    issue_tile(0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
      if (i < n_tiles) issue_tile(i, i);
  }

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = NBUF == 1 ? 0 : it % NBUF;
    if (NBUF > 1) {
      const int nxt = it + NBUF - 1;
      if (nxt < n_tiles) issue_tile(nxt, nxt % NBUF);
    }
    if (w < LW) {
      // copies of later tiles still allowed in flight
      const int later = NBUF > 1 ? min(NBUF - 1, n_tiles - 1 - it) : 0;
      if (later <= 0) wait_vmcnt<0>();
      else if (later == 1) wait_vmcnt<(NBUF > 1 ? LPW : 0)>();
      else if (later == 2) wait_vmcnt<(NBUF > 2 ? 2 * LPW : 0)>();
      else wait_vmcnt<(NBUF > 3 ? 3 * LPW : 0)>();
    }
    barrier();
    __builtin_amdgcn_sched_barrier(0);

    const uint32_t tb = lds0 + buf * kTileBytes;

    // ---- scores: S^T[token][head] for tokens 0..15 (s0) and 16..31 (s1) ----
    // K fragments are read two steps ahead of their MFMAs.
    auto k_addr = [&](int s) -> uint32_t {
      if (s < 16) return tb + k_off[s & 3] + (uint32_t)(s >> 2) * 256u;
      return tb + (s == 16 ? p_off0 : p_off1);
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
        ka[(s + 2) % 3] = lds_read_b128(k_addr(s + 2));
        kb[(s + 2) % 3] = lds_read_b128(k_addr(s + 2) + k_hi(s + 2));
      }
      s0 = mfma16(ka[s % 3], q[s], s0);
      s1 = mfma16(kb[s % 3], q[s], s1);
      __builtin_amdgcn_sched_barrier(0);
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

    // ---- online softmax (one head per lane; 4 lanes share a head) ----
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_ref, mx);
    const bool grow = (m_new - m_ref) * c2 > kRescaleLog2;
    if (__ballot(grow) != 0) {
      const float alpha = fast_exp2((m_ref - m_new) * c2);
      l_sum *= alpha;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) o[cb] *= alpha;
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
    // B operand of P.V: element i <-> token i<4 ? 4 g4 + i : 16 + 4 g4 + (i-4)
    const u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
    __builtin_amdgcn_sched_barrier(0);

    // ---- O^T[c][head] += V^T . P^T over the 32 tokens ----
    auto v_addr = [&](int cb) -> uint32_t { return tb + v_off[cb & 7] + (uint32_t)(cb >> 3) * 256u; };
    bf16x4 vl[3], vh[3];
    vl[0] = lds_read_tr16(v_addr(0));
    vh[0] = lds_read_tr16(v_addr(0) + 16 * kKvRow);
    vl[1] = lds_read_tr16(v_addr(1));
    vh[1] = lds_read_tr16(v_addr(1) + 16 * kKvRow);
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      if (cb + 2 < 32) {
        vl[(cb + 2) % 3] = lds_read_tr16(v_addr(cb + 2));                // tokens 4 g4 + 0..3
        vh[(cb + 2) % 3] = lds_read_tr16(v_addr(cb + 2) + 16 * kKvRow);  // tokens 16 + 4 g4 + 0..3
      }
      const bf16x8 va = __builtin_shufflevector(vl[cb % 3], vh[cb % 3], 0, 1, 2, 3, 4, 5, 6, 7);
      o[cb] = mfma16(va, pb, o[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }

    barrier();  // every wave is done with this buffer
    if (NBUF == 1 && it + 1 < n_tiles) issue_tile(it + 1, 0);
  }

  // ---- finalize ----
  float l_tot = l_sum + __shfl_xor(l_sum, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = 1.0f / l_tot;
  const float lse_val = m_ref * a.scale + __logf(l_tot);
  if (final_out) {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      const u32x2 v = {pack_bf16x2(o[cb][0] * inv, o[cb][1] * inv), pack_bf16x2(o[cb][2] * inv, o[cb][3] * inv)};
      *reinterpret_cast<u32x2*>(final_row + cb * 16 + g4 * 4) = v;
    }
    if (g4 == 0) a.lse[(size_t)b * a.num_heads + h] = lse_val;
  } else {
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) *reinterpret_cast<f32x4*>(part_row + cb * 16 + g4 * 4) = o[cb] * inv;
    if (g4 == 0) a.lse_part[((size_t)b * a.num_splits + split) * a.num_heads + h] = lse_val;
  }
}

template <int NW, int NBUF>
static hipError_t launch_nw(const DecodeArgs& a, int grid, hipStream_t stream) {
  if (a.block_table != nullptr) {
    hipLaunchKernelGGL((decode_latent_kernel<NW, NBUF, true>), dim3(grid), dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_latent_kernel<NW, NBUF, false>), dim3(grid), dim3(NW * 64), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_latent(const DecodeArgs& a, hipStream_t stream) {
  const int grid = a.batch * a.num_splits;
  switch (a.num_heads) {
    case 16: return launch_nw<1, 1>(a, grid, stream);
    case 32: return launch_nw<2, 1>(a, grid, stream);
    case 64: return launch_nw<4, 2>(a, grid, stream);
    case 128: return launch_nw<8, 4>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mla
