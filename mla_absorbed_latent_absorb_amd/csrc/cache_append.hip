// Cache append: writes new tokens into the latent cache.  Each new token is
// one row of the fused down-projection output (512 latent values, then the
// 64-wide decoupled RoPE key before rotation).  The latent half is stored as
// it is; the key is rotated at the token's absolute position and stored
// beside it ("DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.4: the
// RoPE key is cached separately, already rotated; "80 行 PyTorch 从零写
// DeepSeek 的 MLA" §2 and Appendix A: interleaved pairs, angle
// position * base^(-2i/64)).
//
// bf16 cache: key rotated in fp64, rounded to fp32 and then to bf16 (nearest
// even at each step).  E4M3 cache: the token's 576 values in fp32 (latent
// exact, rotated key rounded to fp32) share one scale max|x| / 448 (at least
// the smallest normal fp32); each value / scale (IEEE division, clamped to
// +-448) is encoded as OCP E4M3 with nearest-even rounding
// ("G5 MLA KV 访存建模设计规格" use case 1: 576 one-byte elements per token
// plus an fp32 scale).
//
// One wave per two tokens (A, B).  Lane l moves latent elements 8l .. 8l+7
// of both (16 bytes in, 16 bytes or 8 codes out each); lanes 0..31 rotate
// key pair l of A and lanes 32..63 key pair l-32 of B, so every lane does
// one fp64 rotation.  The kernel is a stream of 1152-byte rows: HBM-bound for
// prefill-sized appends, launch-bound for a decode step's one token per
// sequence.
#include "device_common.hpp"
#include "kernels.hpp"

#include <float.h>

namespace mla {
namespace {

constexpr int kAppendWaves = 4;  // waves per workgroup (two tokens each)

// fp32 -> bf16 bit pattern, nearest, ties to the even pattern (finite x).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// x / s for a token scale s >= FLT_MIN with y = RN(1/s), clamped to +-448.
// The quotient |x| / s is correctly rounded by one reciprocal multiply and
// two FMA corrections (Markstein's theorem: y within half an ulp of 1/s and
// a faithful q0 make RN(q0 + (|x| - s q0) y) the correctly rounded quotient;
// the remainder is exact in one FMA).  Quotients below 2^-10, where the
// theorem's no-underflow condition may fail, all encode to a zero code
// anyway.  The sign is x's own, as for an IEEE division by a positive number
// (-0 keeps its sign).
__device__ __forceinline__ float div_by_scale(float x, float s, float y) {
  const float a = fabsf(x);
  const float q0 = __fmul_rn(a, y);
  const float r = __builtin_fmaf(-q0, s, a);
  return __builtin_copysignf(fminf(__builtin_fmaf(r, y, q0), 448.0f), x);
}

// Two fp32 values -> two OCP E4M3 codes in bytes 2*HI, 2*HI+1 of `old`
// (v_cvt_pk_fp8_f32: nearest even in the default rounding mode, subnormal
// codes included; inputs are within +-448 so nothing saturates).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2(float lo, float hi, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, (int)old, HI);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Key pair (x0, x1) rotated by angle pos * inv_freq, in fp64, rounded to fp32.
// No contraction into FMAs: the products and the sum are rounded separately,
// as the definition writes them.
__device__ __forceinline__ void rotate_pair(float x0f, float x1f, double pos, double inv_freq, float& y0,
                                            float& y1) {
#pragma clang fp contract(off)
  const double x0 = x0f, x1 = x1f;
  double s, c;
  sincos(pos * inv_freq, &s, &c);
  const double p0 = x0 * c, p1 = x1 * s, p2 = x1 * c, p3 = x0 * s;
  y0 = (float)(p0 - p1);
  y1 = (float)(p2 + p3);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = max_xor16(v);
  v = max_xor32(v);
  return v;
}

// Slot of input row `row` (token j of sequence b at position positions[b]+j),
// or -1 when the row does not exist or its position has no slot.
template <bool PAGED>
__device__ __forceinline__ int64_t slot_of(const AppendArgs& a, int64_t row, int64_t rows, int64_t& pos) {
  pos = 0;
  if (row >= rows) return -1;
  const int b = (int)(row / a.num_new);
  const int j = (int)(row - (int64_t)b * a.num_new);
  pos = (int64_t)a.positions[b] + j;
  if (pos < 0) return -1;
  if (PAGED) {
    const int64_t blk = pos / a.block_size;
    if (blk >= a.max_blocks) return -1;
    const int32_t phys = a.block_table[(int64_t)b * a.max_blocks + blk];
    if (phys < 0) return -1;
    return (int64_t)phys * a.block_size + (pos - blk * a.block_size);
  }
  if (pos >= a.seq_stride) return -1;
  return (int64_t)b * a.seq_stride + pos;
}

__device__ __forceinline__ float amax8(u32x4 w) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}

__device__ __forceinline__ u32x2 encode8(u32x4 w, float s, float y) {
  u32x2 c;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t lo = e4m3x2<false>(div_by_scale(bf16_lo(w[2 * h]), s, y), div_by_scale(bf16_hi(w[2 * h]), s, y), 0u);
    c[h] = e4m3x2<true>(div_by_scale(bf16_lo(w[2 * h + 1]), s, y), div_by_scale(bf16_hi(w[2 * h + 1]), s, y), lo);
  }
  return c;
}

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int pair = lane & 31;
  const int64_t rows = (int64_t)a.batch * a.num_new;
  const int64_t row_a = ((int64_t)blockIdx.x * kAppendWaves + (threadIdx.x >> 6)) * 2;
  if (row_a >= rows) return;  // whole wave
  int64_t pos_a, pos_b;
  const int64_t slot_a = slot_of<PAGED>(a, row_a, rows, pos_a);
  const int64_t slot_b = slot_of<PAGED>(a, row_a + 1, rows, pos_b);
  if (slot_a < 0 && slot_b < 0) return;  // whole wave

  const uint16_t* src_a = a.kv_in + row_a * a.in_stride;
  const uint16_t* src_b = src_a + a.in_stride;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  const u32x4 lat_a = slot_a >= 0 ? *reinterpret_cast<const u32x4*>(src_a + 8 * lane) : zero4;
  const u32x4 lat_b = slot_b >= 0 ? *reinterpret_cast<const u32x4*>(src_b + 8 * lane) : zero4;
  // this lane's key pair: token A in lanes 0..31, token B in lanes 32..63
  const int64_t my_slot = half ? slot_b : slot_a;
  float y0 = 0.0f, y1 = 0.0f;
  if (my_slot >= 0) {
    const uint32_t kp = *reinterpret_cast<const uint32_t*>((half ? src_b : src_a) + kDc + 2 * pair);
    rotate_pair(bf16_lo(kp), bf16_hi(kp), (double)(half ? pos_b : pos_a), a.inv_freq[pair], y0, y1);
  }

  if (!FP8) {
    if (slot_a >= 0) *reinterpret_cast<u32x4*>(a.kv + slot_a * a.kv_sb + 16 * lane) = lat_a;
    if (slot_b >= 0) *reinterpret_cast<u32x4*>(a.kv + slot_b * a.kv_sb + 16 * lane) = lat_b;
    if (my_slot >= 0)
      *reinterpret_cast<uint32_t*>(a.pe + my_slot * a.pe_sb + 4 * pair) = bf16_bits_rne(y0) | (bf16_bits_rne(y1) << 16);
    return;
  }

  // per-token scale: max |x| over the token's 512 latent and 64 rotated values
  const float key_max = fmaxf(fabsf(y0), fabsf(y1));
  float m_a = amax8(lat_a), m_b = amax8(lat_b);
  if (half) m_b = fmaxf(m_b, key_max);
  else m_a = fmaxf(m_a, key_max);
  m_a = wave_max(m_a);
  m_b = wave_max(m_b);
  const float s_a = fmaxf(__fdiv_rn(m_a, 448.0f), FLT_MIN);
  const float s_b = fmaxf(__fdiv_rn(m_b, 448.0f), FLT_MIN);
  const float r_a = __fdiv_rn(1.0f, s_a);
  const float r_b = __fdiv_rn(1.0f, s_b);
  if (slot_a >= 0) *reinterpret_cast<u32x2*>(a.kv + slot_a * a.kv_sb + 8 * lane) = encode8(lat_a, s_a, r_a);
  if (slot_b >= 0) *reinterpret_cast<u32x2*>(a.kv + slot_b * a.kv_sb + 8 * lane) = encode8(lat_b, s_b, r_b);
  if (my_slot >= 0) {
    const float s = half ? s_b : s_a, y = half ? r_b : r_a;
    *reinterpret_cast<uint16_t*>(a.pe + my_slot * a.pe_sb + 2 * pair) =
        (uint16_t)e4m3x2<false>(div_by_scale(y0, s, y), div_by_scale(y1, s, y), 0u);
    if (pair == 0) a.token_scale[my_slot] = s;
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendArgs& a, bool fp8, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.num_new;
  const int64_t waves = (rows + 1) / 2;
  const dim3 grid((unsigned)((waves + kAppendWaves - 1) / kAppendWaves));
  const dim3 block(64 * kAppendWaves);
  const bool paged = a.block_table != nullptr;
  if (fp8) {
    if (paged) hipLaunchKernelGGL((cache_append_kernel<true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((cache_append_kernel<true, false>), grid, block, 0, stream, a);
  } else {
    if (paged) hipLaunchKernelGGL((cache_append_kernel<false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((cache_append_kernel<false, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mla
