// One whole decode step in one launch, for short contexts where launch
// latency dominates: key absorption, latent attention with a single split, and
// value absorption ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界"
// §2.2-§2.4: q_lat = q_nope W_UK[h], scores of q_lat and the rotated q_pe
// against the shared 576-wide cache rows, o_lat = softmax-weighted sum of
// latent rows, out = W_UV[h] o_lat; "80 行 PyTorch 从零写 DeepSeek 的 MLA" §4-§5).
//
// One workgroup of 4 waves per (sequence, head).  All first loads go out
// together before any arithmetic (one memory round trip): W_UV[h] straight
// into LDS (16-byte direct-to-LDS copies, read back only at the end), W_UK[h]
// rows, the first 32 cache rows and the queries into registers.
//   a1  wave w multiplies q_nope rows 32w..32w+31 into W_UK[h] rows of 1 KiB
//       (lane l: latent columns 8l..8l+7); the four partial q_lat vectors meet
//       in LDS.  q_lat stays fp32.
//   a2-a4  wave w takes tokens 32k + 8w + i of each 32-token group: the dot
//       products with q_lat are per-lane partial sums reduced across the wave,
//       the online softmax runs in the exp2 domain, and o accumulates the
//       lane's 8 latent columns in fp32.  The four waves' (max, sum, o) merge
//       in LDS.
//   a6  wave w owns output rows 32w..32w+31 of W_UV[h], read from LDS.
//       Per-lane partial dot products are summed by a reduce-scatter over the
//       wave: two permlane swaps halve the rows a lane holds twice (no
//       selects), then DPP row sums finish 8 rows per 16-lane row.
// The work of a workgroup grows with the context (every head streams its
// sequence's rows itself), so this path is meant for short contexts; the
// four-call path splits long contexts over many workgroups instead.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

constexpr int kStepWaves = 4;
constexpr int kRowsPerWave = 8;  // cache rows a wave loads before using them

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }

// Sum over the 16 lanes of a DPP row (quad_perm swaps of neighbours and pairs,
// then rotations by 4 and 8 within the row): every lane gets the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x128>(v);  // row_ror:8
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return sum_xor32(sum_xor16(row_sum(v))); }

// One reduce-scatter step over lane bit 5 (permlane32 swap) or 4 (permlane16
// swap): with a = this lane's rows k and b = its rows k + n/2, the swap leaves
// (own a, partner's a) in lanes whose bit is 0 and (partner's b, own b) in the
// others, so their sum is the pair-reduced row the lane keeps.
__device__ __forceinline__ float scatter32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float scatter16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint16_t to_bf16(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

template <bool PAGED>
__device__ __forceinline__ int64_t step_slot(const FusedStepArgs& a, int b, int t) {
  if (PAGED) {
    const int32_t blk = a.block_table[(int64_t)b * a.max_blocks + t / a.block_size];
    return (int64_t)blk * a.block_size + t % a.block_size;
  }
  return (int64_t)b * a.seq_stride + t;
}

// One cached row as this lane loads it: latent columns 8l..8l+7 and, in
// lanes 0..7, RoPE-key columns 8l..8l+7 (bf16 pairs, or E4M3 codes + scale).
template <bool FP8>
struct RawRow {
  u32x4 c;
  u32x4 r;
  float s;
};

template <bool FP8, bool PAGED>
__device__ __forceinline__ void load_row(const FusedStepArgs& a, int b, int t, int lane, RawRow<FP8>& row) {
  const int64_t slot = step_slot<PAGED>(a, b, t);
  row.r = u32x4{0u, 0u, 0u, 0u};
  if (!FP8) {
    row.c = *reinterpret_cast<const u32x4*>(a.kv + slot * a.kv_sb + 16 * lane);
    if (lane < 8) row.r = *reinterpret_cast<const u32x4*>(a.pe + slot * a.pe_sb + 16 * lane);
    row.s = 1.0f;
  } else {
    const u32x2 c = *reinterpret_cast<const u32x2*>(a.kv + slot * a.kv_sb + 8 * lane);
    row.c = u32x4{c[0], c[1], 0u, 0u};
    if (lane < 8) {
      const u32x2 r = *reinterpret_cast<const u32x2*>(a.pe + slot * a.pe_sb + 8 * lane);
      row.r = u32x4{r[0], r[1], 0u, 0u};
    }
    row.s = a.token_scale[slot];
  }
}

// The lane's 8 latent and 8 RoPE-key values of a row in fp32 (E4M3: code
// times the token scale).
template <bool FP8>
__device__ __forceinline__ void unpack_row(const RawRow<FP8>& row, float (&c)[8], float (&r)[8]) {
  if (!FP8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c[2 * k] = lo16(row.c[k]);
      c[2 * k + 1] = hi16(row.c[k]);
      r[2 * k] = lo16(row.r[k]);
      r[2 * k + 1] = hi16(row.r[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const f32x2 c0 = e4m3x2_to_f32<false>(row.c[k]), c1 = e4m3x2_to_f32<true>(row.c[k]);
      const f32x2 r0 = e4m3x2_to_f32<false>(row.r[k]), r1 = e4m3x2_to_f32<true>(row.r[k]);
      c[4 * k] = c0[0] * row.s;
      c[4 * k + 1] = c0[1] * row.s;
      c[4 * k + 2] = c1[0] * row.s;
      c[4 * k + 3] = c1[1] * row.s;
      r[4 * k] = r0[0] * row.s;
      r[4 * k + 1] = r0[1] * row.s;
      r[4 * k + 2] = r1[0] * row.s;
      r[4 * k + 3] = r1[1] * row.s;
    }
  }
}

// Online-softmax update of one wave with a group of kRowsPerWave rows
// (tokens base .. base + kRowsPerWave - 1, those >= T ignored), exp2 domain.
template <bool FP8>
__device__ __forceinline__ void attend_rows(const RawRow<FP8> (&rows)[kRowsPerWave], int base, int T,
                                            const float (&ql)[8], const float (&qr)[8], float scale_log2,
                                            float& m, float& l, float (&o)[8]) {
  float s[kRowsPerWave];
  float m_new = m;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    float c[8], r[8];
    unpack_row<FP8>(rows[i], c, r);
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) d += ql[k] * c[k] + qr[k] * r[k];
    d = wave_sum(d) * scale_log2;
    s[i] = base + i < T ? d : -INFINITY;
    m_new = fmaxf(m_new, s[i]);
  }
  const float alpha = fast_exp2(m - m_new);  // m = -inf before the first group: alpha = 0
  l *= alpha;
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] *= alpha;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    if (base + i < T) {
      float c[8], r[8];
      unpack_row<FP8>(rows[i], c, r);
      const float p = fast_exp2(s[i] - m_new);
      l += p;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] += p * c[k];
    }
  }
  m = m_new;
}

template <bool PAGED, bool FP8>
__global__ __launch_bounds__(64 * kStepWaves) void decode_step_fused_kernel(FusedStepArgs a) {
  __shared__ __attribute__((aligned(1024))) char wuv_s[kDv * kDc * 2];  // W_UV[h]: 128 rows of 1 KiB
  __shared__ float part[kStepWaves][kDc];                                 // a1 partial q_lat, then each wave's o
  __shared__ float qlat[kDc];
  __shared__ float wave_ml[kStepWaves][2];
  const int H = a.num_heads;
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);  // one head's workgroups share an XCD
  const int h = item / a.batch, b = item % a.batch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);

  // Every load of the first memory round trip goes out before any compute:
  // this wave's 32 W_UV rows straight into LDS, its 32 W_UK rows and its first
  // group of cache rows into registers, and the RoPE query.
  const uint32_t wuv_lds = (uint32_t)(uintptr_t)wuv_s;
  {
    const char* wp = reinterpret_cast<const char*>(a.w_uv + ((int64_t)h * kDv + 32 * w) * kDc);
#pragma unroll
    for (int i = 0; i < 32; ++i) dma16(uniform_ptr(wp + i * 1024), 16u * lane, wuv_lds + (32 * w + i) * 1024);
  }
  u32x4 wk[32];
  {
    const uint16_t* wp = a.w_uk + ((int64_t)h * kDn + 32 * w) * kDc + 8 * lane;
#pragma unroll
    for (int i = 0; i < 32; ++i) wk[i] = *reinterpret_cast<const u32x4*>(wp + (int64_t)i * kDc);
  }
  RawRow<FP8> rows[kRowsPerWave] = {};
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
    if (kRowsPerWave * w + i < T) load_row<FP8, PAGED>(a, b, kRowsPerWave * w + i, lane, rows[i]);
  u32x4 qp = {0u, 0u, 0u, 0u};
  if (lane < 8) qp = *reinterpret_cast<const u32x4*>(a.q_pe + ((int64_t)b * H + h) * kDr + 8 * lane);
  __builtin_amdgcn_sched_barrier(0);

  // ---- a1: q_lat[c] = sum_d q_nope[d] W_UK[h][d][c], wave w: rows d = 32w .. 32w+31
  {
    const uint16_t* qn = a.q_nope + ((int64_t)b * H + h) * kDn + 32 * w;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float q = bf16_at(qn + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += q * lo16(wk[i][k]);
        acc[2 * k + 1] += q * hi16(wk[i][k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) part[w][8 * lane + k] = acc[k];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < kDc; c += 64 * kStepWaves)
    qlat[c] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
  __syncthreads();

  // ---- a2-a4: online softmax over this wave's tokens 32k + 8w + i
  float ql[8], qr[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ql[2 * k] = qlat[8 * lane + 2 * k];
    ql[2 * k + 1] = qlat[8 * lane + 2 * k + 1];
    qr[2 * k] = lo16(qp[k]);
    qr[2 * k + 1] = hi16(qp[k]);
  }
  float m = -INFINITY, l = 0.0f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int kGroup = kRowsPerWave * kStepWaves;
  if (kRowsPerWave * w < T) attend_rows<FP8>(rows, kRowsPerWave * w, T, ql, qr, a.scale_log2, m, l, o);
  for (int base = kGroup + kRowsPerWave * w; base < T; base += kGroup) {
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      if (base + i < T) load_row<FP8, PAGED>(a, b, base + i, lane, rows[i]);
    attend_rows<FP8>(rows, base, T, ql, qr, a.scale_log2, m, l, o);
  }

  // merge the four waves: o = sum_w 2^(m_w - M) o_w / L
#pragma unroll
  for (int k = 0; k < 8; ++k) part[w][8 * lane + k] = o[k];
  if (lane == 0) {
    wave_ml[w][0] = m;
    wave_ml[w][1] = l;
  }
  wait_vmcnt<0>();  // this wave's W_UV copies have landed; the barrier publishes all four
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kStepWaves; ++v) M = fmaxf(M, wave_ml[v][0]);
  float e[kStepWaves], L = 0.0f;
#pragma unroll
  for (int v = 0; v < kStepWaves; ++v) {
    e[v] = wave_ml[v][0] == -INFINITY ? 0.0f : fast_exp2(wave_ml[v][0] - M);
    L += e[v] * wave_ml[v][1];
  }
  const float inv_l = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float x = 0.0f;
#pragma unroll
    for (int v = 0; v < kStepWaves; ++v) x += e[v] * part[v][8 * lane + k];
    o[k] = x * inv_l;
  }
  if (w == 0) {
    if (a.o_lat != nullptr) {
      u32x4 ov;
#pragma unroll
      for (int k = 0; k < 4; ++k) ov[k] = (uint32_t)to_bf16(o[2 * k]) | ((uint32_t)to_bf16(o[2 * k + 1]) << 16);
      *reinterpret_cast<u32x4*>(a.o_lat + ((int64_t)b * H + h) * kDc + 8 * lane) = ov;
    }
    if (a.lse != nullptr && lane == 0)
      a.lse[(int64_t)b * H + h] = L > 0.0f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
  }

  // ---- a6: out[j] = sum_c W_UV[h][j][c] o[c], rows j = 32w .. 32w+31 (from LDS)
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const u32x4 wr = lds_read_u32x4(wuv_lds + (32 * w + i) * 1024 + 16 * lane);
    float d = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) d += lo16(wr[k]) * o[2 * k] + hi16(wr[k]) * o[2 * k + 1];
    v[i] = d;
  }
  // reduce-scatter over lane bits 5 and 4: a lane keeps 8 rows,
  // 16 * bit5 + 8 * bit4 + k, summed over its 4-lane group; then row sums
  // over the 16 lanes of the DPP row
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = scatter32(v[k], v[k + 16]);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = scatter16(v[k], v[k + 8]);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = row_sum(v[k]);
  if ((lane & 15) == 0) {
    u32x4 ov;
#pragma unroll
    for (int k = 0; k < 4; ++k) ov[k] = (uint32_t)to_bf16(v[2 * k]) | ((uint32_t)to_bf16(v[2 * k + 1]) << 16);
    *reinterpret_cast<u32x4*>(a.out + ((int64_t)b * H + h) * kDv + 32 * w + ((lane >> 4) << 3)) = ov;
  }
}

}  // namespace

hipError_t launch_decode_step_fused(const FusedStepArgs& a, bool fp8, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)a.batch * a.num_heads));
  const dim3 block(64 * kStepWaves);
  const bool paged = a.block_table != nullptr;
  if (fp8) {
    if (paged) hipLaunchKernelGGL((decode_step_fused_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_step_fused_kernel<false, true>), grid, block, 0, stream, a);
  } else {
    if (paged) hipLaunchKernelGGL((decode_step_fused_kernel<true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_step_fused_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
