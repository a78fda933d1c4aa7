// The per-head projections around latent attention and the split-KV merge.
//
// absorb_q: q_lat[b,h,c] = sum_d q_nope[b,h,d] W_UK[h,d,c]   (key absorption,
//   "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2)
// expand_v: out[b,h,j] = sum_c W_UV[h,j,c] o_lat[b,h,c]       (value absorption, §2.3)
// combine : LSE = ln sum_i exp(lse_i); o = sum_i exp(lse_i - LSE) o_i
//
// Both projections are per-head batched GEMMs that are bound by reading the
// weights once (16 MiB each for 128 heads).  They are computed transposed,
// D^T[column][batch] = W^T . X^T with 16x16x32 bf16 MFMAs, so a lane ends up
// with four consecutive output columns of one batch row (one 8-byte store),
// and every load a workgroup needs is issued before its first use.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// absorb_q: workgroup = (head h, 64 output columns c); wave w owns columns
// 16 w .. 16 w + 15 of the block (the 16 rows of its D^T tiles).
//   A[c][d] = W_UK[h][d][c]: the [128 d][64 c] slab is staged in LDS and read
//             transposed with ds_read_b64_tr_b16 (lane l: column l%16, 8 rows).
//   B[d][b] = q_nope[b][h][d]: 16-byte contiguous loads from global.
// ---------------------------------------------------------------------------
constexpr int kAbsorbBatchBlocks = 4;  // batch blocks of 16 whose query fragments are loaded together

__global__ __launch_bounds__(256) void absorb_q_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t wt[kDn * 64];  // 16 KiB
  // the 8 column blocks of a head run on one XCD (shared L2 for its rows)
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);
  const int h = item >> 3;
  const int cblk = item & 7;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int nl = lane & 15, g = lane >> 4;

  // slab rows: thread t copies 16-byte pieces k*256 + t (row piece/8, chunk piece%8)
  const uint16_t* wsrc = a.w + (size_t)h * kDn * kDc + cblk * 64;
  u32x4 wreg[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * 256 + t;
    wreg[k] = *reinterpret_cast<const u32x4*>(wsrc + (size_t)(idx >> 3) * kDc + (idx & 7) * 8);
  }
  // query fragments of the first batch blocks, in flight with the slab
  auto load_q = [&](int mb, bf16x8 (&qf)[4]) {
    const int brow = mb * 16 + nl;
    if (brow < a.batch) {
      const bf16x8* src = reinterpret_cast<const bf16x8*>(a.x + ((size_t)brow * a.num_heads + h) * kDn + 8 * g);
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[s] = src[4 * s];
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  };
  const int nblk = (a.batch + 15) / 16;
  bf16x8 qf[kAbsorbBatchBlocks][4];
#pragma unroll
  for (int i = 0; i < kAbsorbBatchBlocks; ++i)
    if (i < nblk) load_q(i, qf[i]);

#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * 256 + t;
    *reinterpret_cast<u32x4*>(wt + (idx >> 3) * 64 + (idx & 7) * 8) = wreg[k];
  }
  __syncthreads();

  // A fragments for the 4 k-steps of 32 (d = 32 s + 8 g + i), column 16 w + nl
  const uint32_t wbase = (uint32_t)(uintptr_t)wt;
  bf16x8 af[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t row = 32 * s + 8 * g + (nl >> 2);
    const uint32_t off = wbase + row * 128 + (16 * w + 4 * (nl & 3)) * 2;
    const bf16x4 lo = lds_read_tr16(off);
    const bf16x4 hi = lds_read_tr16(off + 4 * 128);
    af[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  // D^T[c = 16 w + 4 g + j][b = 16 mb + nl]: four consecutive columns per lane
  const int c0 = cblk * 64 + 16 * w + 4 * g;
  auto emit = [&](int mb, const bf16x8 (&q)[4]) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16(af[s], q[s], acc);
    const int bo = mb * 16 + nl;
    if (bo < a.batch) {
      const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(a.y + ((size_t)bo * a.num_heads + h) * kDc + c0) = v;
    }
  };
#pragma unroll
  for (int i = 0; i < kAbsorbBatchBlocks; ++i)
    if (i < nblk) emit(i, qf[i]);
  for (int mb = kAbsorbBatchBlocks; mb < nblk; ++mb) {
    bf16x8 q[4];
    load_q(mb, q);
    emit(mb, q);
  }
}

// ---------------------------------------------------------------------------
// expand_v: workgroup = (head h, 16 output columns j); wave w reduces the
// latent range c in [128 w, 128 w + 128) for every batch block, and the four
// partial D^T tiles are summed through LDS.
//   A[j][c] = W_UV[h][j][c], B[c][b] = o_lat[b][h][c]: both contiguous rows.
// ---------------------------------------------------------------------------
// NB = batch blocks per pass (at most 8: partials in LDS 32 KiB); sized to the
// batch so small batches do not reserve registers for unused blocks.
template <int NB>
__global__ __launch_bounds__(256) void expand_v_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) f32x4 red[4][NB][64];
  // the 8 row blocks of a head run on one XCD, which then fetches the head's
  // o_lat rows into its L2 once
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);
  const int h = item >> 3;
  const int jblk = item & 7;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int cbase = 128 * w + 8 * g;

  bf16x8 af[4];
  {
    const bf16x8* wrow = reinterpret_cast<const bf16x8*>(a.w + ((size_t)h * kDv + jblk * 16 + nl) * kDc + cbase);
#pragma unroll
    for (int s = 0; s < 4; ++s) af[s] = wrow[4 * s];
  }
  const int nblk = (a.batch + 15) / 16;
  for (int mb0 = 0; mb0 < nblk; mb0 += NB) {
    bf16x8 bq[NB][4];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int brow = (mb0 + i) * 16 + nl;
      if (mb0 + i < nblk && brow < a.batch) {
        const bf16x8* src = reinterpret_cast<const bf16x8*>(a.x + ((size_t)brow * a.num_heads + h) * kDc + cbase);
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[i][s] = src[4 * s];
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[i][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (mb0 + i < nblk) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(af[s], bq[i][s], acc);
        red[w][i][lane] = acc;
      }
    }
    __syncthreads();
    // wave w finishes batch blocks i = w, w + 4: D^T[j = 4 g + r][b = 16 mb + nl]
    for (int i = w; i < NB && mb0 + i < nblk; i += 4) {
      const f32x4 acc = (red[0][i][lane] + red[1][i][lane]) + (red[2][i][lane] + red[3][i][lane]);
      const int bo = (mb0 + i) * 16 + nl;
      if (bo < a.batch) {
        const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *reinterpret_cast<u32x2*>(a.y + ((size_t)bo * a.num_heads + h) * kDv + jblk * 16 + 4 * g) = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// combine: one wave per (sequence, head); lane l handles latent columns
// 8 l .. 8 l + 7 of the bf16 partial rows.  The split weights are formed once
// per wave (lane i holds split i) and broadcast; all partial rows of a group
// of 8 splits are loaded before they are accumulated.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  // Sequences map to XCDs the way the decode kernel's splits do, so a
  // sequence's partial rows may still be in that XCD's L2.
  const int wid = xcd_grouped_index(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (wid >= a.batch * a.num_heads) return;
  const int b = wid / a.num_heads;
  const int h = wid - b * a.num_heads;
  const int lane = threadIdx.x & 63;
  const int P = a.num_splits;
  const float* lse_row = a.lse_part + (size_t)b * P * a.num_heads + h;

  float m = -INFINITY;
  for (int i = lane; i < P; i += 64) m = fmaxf(m, lse_row[(size_t)i * a.num_heads]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    const uint16_t* prow = a.o_part + ((size_t)b * P * a.num_heads + h) * kDc + lane * 8;
    for (int i0 = 0; i0 < P; i0 += 64) {
      // weight of split i0 + lane (0 for empty splits and lanes past P)
      const float li = i0 + lane < P ? lse_row[(size_t)(i0 + lane) * a.num_heads] : -INFINITY;
      const float wl = li == -INFINITY ? 0.f : __expf(li - m);
      float ws = wl;
#pragma unroll
      for (int k = 32; k >= 1; k >>= 1) ws += __shfl_xor(ws, k);
      tot += ws;
      const int n = min(64, P - i0);
      for (int j0 = 0; j0 < n; j0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j0 + j < n) v[j] = *reinterpret_cast<const u32x4*>(prow + (size_t)(i0 + j0 + j) * a.num_heads * kDc);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j0 + j < n) {
            const float wi = __shfl(wl, j0 + j);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              acc0[2 * e] += wi * __uint_as_float(v[j][e] << 16);
              acc0[2 * e + 1] += wi * __uint_as_float(v[j][e] & 0xffff0000u);
              acc1[2 * e] += wi * __uint_as_float(v[j][2 + e] << 16);
              acc1[2 * e + 1] += wi * __uint_as_float(v[j][2 + e] & 0xffff0000u);
            }
          }
        }
      }
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
  const int nblk = (a.batch + 15) / 16;
  const dim3 grid(a.num_heads * 8), block(256);
  if (nblk <= 1) hipLaunchKernelGGL(expand_v_kernel<1>, grid, block, 0, stream, a);
  else if (nblk <= 2) hipLaunchKernelGGL(expand_v_kernel<2>, grid, block, 0, stream, a);
  else if (nblk <= 4) hipLaunchKernelGGL(expand_v_kernel<4>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(expand_v_kernel<8>, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int waves = a.batch * a.num_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
