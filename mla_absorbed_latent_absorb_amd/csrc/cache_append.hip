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
// One wave per token.  Lane l moves latent elements 8l .. 8l+7 (16 bytes in,
// 16 bytes or 8 codes out); lanes 0..31 rotate key pair l.  The kernel is a
// stream of 1152-byte rows: HBM-bound for prefill-sized appends, launch-bound
// for a decode step's one token per sequence.
#include "device_common.hpp"
#include "kernels.hpp"

#include <float.h>

namespace mla {
namespace {

constexpr int kAppendWaves = 4;  // tokens per workgroup

// fp32 -> bf16 bit pattern, nearest, ties to the even pattern (finite x).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// |x| <= 448, finite -> OCP E4M3 code, nearest, ties to the even code.
// Below the smallest normal (2^-6) E4M3 steps are 2^-9, so the code is
// x * 2^9 rounded to an integer (8 is the smallest normal itself).  Above it,
// the code is the fp32 pattern with 20 mantissa bits rounded off (nearest
// even) and the exponent rebased from bias 127 to bias 7 (120 << 3 = 960).
__device__ __forceinline__ uint32_t e4m3_code_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const uint32_t r = __float_as_uint(a);
    code = ((r + 0x7FFFFu + ((r >> 20) & 1u)) >> 20) - 960u;
  }
  return sign | code;
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

template <bool FP8, bool PAGED>
__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (row >= (int64_t)a.batch * a.num_new) return;
  const int b = (int)(row / a.num_new);
  const int j = (int)(row - (int64_t)b * a.num_new);
  const int64_t pos = (int64_t)a.positions[b] + j;
  // rows outside the cache are not written (the whole wave leaves together)
  int64_t slot;
  if (pos < 0) return;
  if (PAGED) {
    const int64_t blk = pos / a.block_size;
    if (blk >= a.max_blocks) return;
    const int32_t phys = a.block_table[(int64_t)b * a.max_blocks + blk];
    if (phys < 0) return;
    slot = (int64_t)phys * a.block_size + (pos - blk * a.block_size);
  } else {
    if (pos >= a.seq_stride) return;
    slot = (int64_t)b * a.seq_stride + pos;
  }

  const uint16_t* src = a.kv_in + row * a.in_stride;
  const u32x4 lat = *reinterpret_cast<const u32x4*>(src + 8 * lane);
  float y0 = 0.0f, y1 = 0.0f;
  if (lane < 32) {
    const uint32_t kp = *reinterpret_cast<const uint32_t*>(src + kDc + 2 * lane);
    rotate_pair(bf16_lo(kp), bf16_hi(kp), (double)pos, a.inv_freq[lane], y0, y1);
  }

  char* dkv = a.kv + slot * a.kv_sb;
  char* dpe = a.pe + slot * a.pe_sb;
  if (!FP8) {
    *reinterpret_cast<u32x4*>(dkv + 16 * lane) = lat;
    if (lane < 32)
      *reinterpret_cast<uint32_t*>(dpe + 4 * lane) = bf16_bits_rne(y0) | (bf16_bits_rne(y1) << 16);
    return;
  }

  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(lat[i]);
    v[2 * i + 1] = bf16_hi(lat[i]);
  }
  float amax = fmaxf(fabsf(y0), fabsf(y1));
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max(amax);
  const float scale = fmaxf(__fdiv_rn(amax, 448.0f), FLT_MIN);
  auto enc = [&](float x) {
    const float q = fminf(fmaxf(__fdiv_rn(x, scale), -448.0f), 448.0f);
    return e4m3_code_rne(q);
  };
  u32x2 codes;
#pragma unroll
  for (int w = 0; w < 2; ++w)
    codes[w] = enc(v[4 * w]) | (enc(v[4 * w + 1]) << 8) | (enc(v[4 * w + 2]) << 16) | (enc(v[4 * w + 3]) << 24);
  *reinterpret_cast<u32x2*>(dkv + 8 * lane) = codes;
  if (lane < 32) *reinterpret_cast<uint16_t*>(dpe + 2 * lane) = (uint16_t)(enc(y0) | (enc(y1) << 8));
  if (lane == 0) a.token_scale[slot] = scale;
}

}  // namespace

hipError_t launch_cache_append(const AppendArgs& a, bool fp8, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.num_new;
  const dim3 grid((unsigned)((rows + kAppendWaves - 1) / kAppendWaves));
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
