// The per-head projections around latent attention and the split-KV merge.
//
// absorb_q: q_lat[b,h,c] = sum_d q_nope[b,h,d] W_UK[h,d,c]   (key absorption,
//   "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2)
// expand_v: out[b,h,j] = sum_c W_UV[h,j,c] o_lat[b,h,c]       (value absorption, §2.3)
// combine : LSE = ln sum_i exp(lse_i); o = sum_i exp(lse_i - LSE) o_i
//
// Both projections are per-head batched GEMMs with the batch as the M
// dimension (16x16x32 bf16 MFMA, fp32 accumulation).  At decode batch sizes
// they are bound by reading the weights once (2 MiB per 16 heads).
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// absorb_q: workgroup = (head h, 64 output columns); wave w owns 16 columns.
// The W_UK[h] slab [128 d][64 c] is staged in LDS row-major and read back
// transposed (column-major fragments) with ds_read_b64_tr_b16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_q_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kDn * 64];  // 16 KiB
  const int h = blockIdx.x >> 3;
  const int cblk = blockIdx.x & 7;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nl = lane & 15, g = lane >> 4;

  const uint16_t* wsrc = a.w + (size_t)h * kDn * kDc + cblk * 64;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * 256 + t;  // 16-byte piece: row idx/8, chunk idx%8
    const int row = idx >> 3, ch = idx & 7;
    *reinterpret_cast<u32x4*>(wt + row * 64 + ch * 8) =
        *reinterpret_cast<const u32x4*>(wsrc + (size_t)row * kDc + ch * 8);
  }
  __syncthreads();

  // B fragments for the 4 k-steps of 32 (d = 32 s + 8 g + i), column 16 w + nl
  const uint32_t wbase = (uint32_t)(uintptr_t)wt;
  bf16x8 bfrag[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t row = 32 * s + 8 * g + (nl >> 2);
    const uint32_t off = wbase + row * 128 + (16 * w + 4 * (nl & 3)) * 2;
    const bf16x4 lo = lds_read_tr16(off);
    const bf16x4 hi = lds_read_tr16(off + 4 * 128);
    bfrag[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  const int c = cblk * 64 + 16 * w + nl;
  for (int mb = 0; mb * 16 < a.batch; ++mb) {
    const int brow = mb * 16 + nl;  // A row held by this lane
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 af;
      if (brow < a.batch) {
        af = *reinterpret_cast<const bf16x8*>(a.x + ((size_t)brow * a.num_heads + h) * kDn + 32 * s + 8 * g);
      } else {
        af = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
      acc = mfma16(af, bfrag[s], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bo = mb * 16 + 4 * g + j;
      if (bo < a.batch) {
        const __bf16 v = (__bf16)acc[j];
        a.y[((size_t)bo * a.num_heads + h) * kDc + c] = __builtin_bit_cast(uint16_t, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// expand_v: workgroup = (head h, 64 output columns j); wave w owns 16 columns.
// The B operand W_UV[h][j][c .. c+7] is contiguous in memory, so each lane
// keeps its 16 fragments (one 128-column quarter of row j) in registers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void expand_v_kernel(ProjArgs a) {
  const int h = blockIdx.x >> 1;
  const int jblk = blockIdx.x & 1;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int j = jblk * 64 + 16 * w + nl;

  bf16x8 bfrag[16];
  const uint16_t* wrow = a.w + ((size_t)h * kDv + j) * kDc;
#pragma unroll
  for (int s = 0; s < 16; ++s) bfrag[s] = *reinterpret_cast<const bf16x8*>(wrow + 32 * s + 8 * g);

  for (int mb = 0; mb * 16 < a.batch; ++mb) {
    const int brow = mb * 16 + nl;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow = a.x + ((size_t)brow * a.num_heads + h) * kDc;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      bf16x8 af;
      if (brow < a.batch) af = *reinterpret_cast<const bf16x8*>(xrow + 32 * s + 8 * g);
      else af = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      acc = mfma16(af, bfrag[s], acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int bo = mb * 16 + 4 * g + r;
      if (bo < a.batch) {
        const __bf16 v = (__bf16)acc[r];
        a.y[((size_t)bo * a.num_heads + h) * kDv + j] = __builtin_bit_cast(uint16_t, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: one wave per (sequence, head); lane handles 8 latent columns.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.batch * a.num_heads) return;
  const int b = wid / a.num_heads;
  const int h = wid - b * a.num_heads;
  const int lane = threadIdx.x & 63;
  const int P = a.num_splits;

  float m = -INFINITY;
  for (int i = 0; i < P; ++i) m = fmaxf(m, a.lse_part[((size_t)b * P + i) * a.num_heads + h]);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int i = 0; i < P; ++i) {
      const float li = a.lse_part[((size_t)b * P + i) * a.num_heads + h];
      if (li == -INFINITY) continue;
      const float wi = __expf(li - m);
      tot += wi;
      const f32x4* src = reinterpret_cast<const f32x4*>(
          a.o_part + (((size_t)b * P + i) * a.num_heads + h) * kDc + lane * 8);
      acc0 += wi * src[0];
      acc1 += wi * src[1];
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  const u32x4 v = {pack_bf16x2(acc0[0] * inv, acc0[1] * inv), pack_bf16x2(acc0[2] * inv, acc0[3] * inv),
                   pack_bf16x2(acc1[0] * inv, acc1[1] * inv), pack_bf16x2(acc1[2] * inv, acc1[3] * inv)};
  *reinterpret_cast<u32x4*>(a.o_lat + ((size_t)b * a.num_heads + h) * kDc + lane * 8) = v;
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)b * a.num_heads + h] = tot > 0.f ? m + __logf(tot) : -INFINITY;
}

hipError_t launch_absorb_q(const ProjArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(absorb_q_kernel, dim3(a.num_heads * 8), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_expand_v(const ProjArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(expand_v_kernel, dim3(a.num_heads * 2), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int waves = a.batch * a.num_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
