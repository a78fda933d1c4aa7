// Naive ("expand every step") decode: the baseline the absorbed path is
// measured against.  Each step re-expands every cached latent row into
// per-head keys and values, k_nope[t,h] = W_UK[h] c_t and v[t,h] = W_UV[h] c_t,
// and runs ordinary multi-head attention over [k_nope | kR_t] and v
// ("80 行 PyTorch 从零写 DeepSeek 的 MLA" §4 path A and §5: the base decode calls
// the up-projections on the whole latent cache every step; "DeepSeek MLA
// 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2: the expanded keys / values
// per head).  Mathematically the same result as the absorbed path.
//
// naive_expand_kernel: one GEMM per step, D[n][t] = W[n] . c_t over the 512
//   latent columns, W = the 2H heads of W_UK and W_UV stacked (n = 128 rows per
//   head), written as bf16 [B, S, H, 256] (k_nope in columns 0..127, v in
//   128..255).  Workgroup tile 128 W rows x 128 tokens, 4 waves of 64 x 64 on
//   32x32x16 bf16 MFMAs, the contraction in chunks of 128 staged through LDS
//   (256-byte rows, 16-byte chunks at slot chunk ^ (row % 16)), the next
//   chunk's loads in flight during the current chunk's MFMAs; the result is
//   staged through LDS and stored as whole rows.
// naive_attend_kernel: one workgroup per (sequence, head), 16 token streams
//   of 16 lanes (lane j: k_nope / v columns 8j..8j+7, RoPE-key columns
//   4j..4j+3); dot products summed over the 16 lanes with DPP, online softmax
//   per stream in the exp2 domain, streams merged in LDS.  HBM-bound on the
//   expanded rows (512 bytes per token and head).
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXM = 128;         // tokens per workgroup
constexpr int kXN = 128;         // W rows per workgroup (one head of W_UK or W_UV)
constexpr int kXK = 128;         // contraction chunk
constexpr int kXRow = kXK * 2;   // 256-byte LDS rows

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_len(const NaiveArgs& a, int b) {
  const int T = a.seq_lens[b];
  return T < 0 ? 0 : (T > a.max_seq_len ? a.max_seq_len : T);
}

template <bool PAGED>
__device__ __forceinline__ int64_t naive_slot(const NaiveArgs& a, int b, int t) {
  if (PAGED) {
    const int32_t blk = a.block_table[(int64_t)b * a.max_blocks + t / a.block_size];
    return (int64_t)blk * a.block_size + t % a.block_size;
  }
  return (int64_t)b * a.seq_stride + t;
}

__device__ __forceinline__ uint32_t xslot(uint32_t row, uint32_t chunk) { return row * kXRow + ((chunk ^ (row & 15u)) << 4); }

template <bool PAGED, bool FP8>
__global__ __launch_bounds__(256) void naive_expand_kernel(NaiveArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kXM * kXRow];  // W rows | token rows (64 KiB)
  const uint32_t wl = (uint32_t)(uintptr_t)smem, cl = wl + kXN * kXRow;
  const int H = a.num_heads;
  const int nt = blockIdx.x, mt = blockIdx.y, b = blockIdx.z;
  const int T = clamp_len(a, b);
  const int t0 = mt * kXM;
  if (t0 >= T) return;
  const bool is_v = nt >= H;
  const int head = is_v ? nt - H : nt;
  const uint16_t* wsrc = (is_v ? a.w_uv : a.w_uk) + (int64_t)head * kDn * kDc;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // thread slots: idx = tid + 256 j -> row idx / 16, chunk idx % 16 (8 per thread)
  int64_t row_off[8];  // byte offset of this slot's cache row (rows past T re-read row T-1)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (tid + 256 * j) >> 4;
    const int t = min(t0 + row, T - 1);
    row_off[j] = naive_slot<PAGED>(a, b, t) * a.kv_sb;
  }
  u32x4 wr[8], cr[8];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid + 256 * j, row = idx >> 4, chunk = idx & 15;
      const int col = kc * kXK + 8 * chunk;
      wr[j] = *reinterpret_cast<const u32x4*>(wsrc + (int64_t)row * kDc + col);
      if (!FP8) {
        cr[j] = *reinterpret_cast<const u32x4*>(a.kv + row_off[j] + 2 * col);
      } else {
        const int t = min(t0 + row, T - 1);
        const float s = a.token_scale[naive_slot<PAGED>(a, b, t)];
        const u32x2 c = *reinterpret_cast<const u32x2*>(a.kv + row_off[j] + col);
        u32x4 v;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const f32x2 lo = e4m3x2_to_f32<false>(c[k]), hi = e4m3x2_to_f32<true>(c[k]);
          v[2 * k] = pack_bf16x2(lo[0] * s, lo[1] * s);
          v[2 * k + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
        }
        cr[j] = v;
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  const uint32_t nbase = 64 * (w >> 1), tbase = 64 * (w & 1);
  const uint32_t lrow = lane & 31, lk = lane >> 5;

  load_chunk(0);
  for (int kc = 0; kc < kDc / kXK; ++kc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = tid + 256 * j, row = idx >> 4, chunk = idx & 15;
      lds_write_u32x4(wl + xslot(row, chunk), wr[j]);
      lds_write_u32x4(cl + xslot(row, chunk), cr[j]);
    }
    barrier();
    if (kc + 1 < kDc / kXK) load_chunk(kc + 1);
#pragma unroll
    for (int ks = 0; ks < kXK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_read_b128(wl + xslot(nbase + 32 * i + lrow, 2 * ks + lk));
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = lds_read_b128(cl + xslot(tbase + 32 * j + lrow, 2 * ks + lk));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    barrier();
  }

  // D[n][t]: lane holds n = nbase + 32 i + 8 (q/4) + 4 lk + q%4, t = tbase + 32 j + lrow.
  // Stage as [t][n] bf16 rows, then store whole 256-byte rows.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t n0 = nbase + 32 * i + 8 * q4 + 4 * lk;
        const uint32_t t = tbase + 32 * j + lrow;
        const u32x2 v = {pack_bf16x2(acc[i][j][4 * q4], acc[i][j][4 * q4 + 1]),
                         pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3])};
        lds_write_b64(wl + xslot(t, n0 >> 3) + (n0 & 7u) * 2, v);
      }
  barrier();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = tid + 256 * j, t = idx >> 4, chunk = idx & 15;
    if (t0 + t < T) {
      const u32x4 v = lds_read_u32x4(wl + xslot(t, chunk));
      *reinterpret_cast<u32x4*>(a.ws + (((int64_t)b * a.max_seq_len + t0 + t) * H + head) * 256 + (is_v ? 128 : 0) +
                                8 * chunk) = v;
    }
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a DPP row; every lane gets the row's sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x128>(v);  // row_ror:8
  return v;
}

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

constexpr int kStreams = 16;   // token streams per workgroup (16 lanes each)
constexpr int kUnroll = 4;     // tokens per stream and iteration

template <bool PAGED, bool FP8>
__global__ __launch_bounds__(256) void naive_attend_kernel(NaiveArgs a) {
  __shared__ float so[kStreams][kDv];
  __shared__ float sml[kStreams][2];
  const int H = a.num_heads;
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);  // a sequence's heads share an XCD
  const int b = item / H, h = item % H;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15;
  const int stream = (tid >> 6) * 4 + (lane >> 4);
  const int T = clamp_len(a, b);

  float qn[8], qr[4];
  {
    const u32x4 q = *reinterpret_cast<const u32x4*>(a.q_nope + ((int64_t)b * H + h) * kDn + 8 * j);
    const u32x2 p = *reinterpret_cast<const u32x2*>(a.q_pe + ((int64_t)b * H + h) * kDr + 4 * j);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      qn[2 * k] = lo16(q[k]);
      qn[2 * k + 1] = hi16(q[k]);
    }
    qr[0] = lo16(p[0]);
    qr[1] = hi16(p[0]);
    qr[2] = lo16(p[1]);
    qr[3] = hi16(p[1]);
  }
  float m = -INFINITY, l = 0.0f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* ws = a.ws + (((int64_t)b * a.max_seq_len) * H + h) * 256 + 8 * j;
  const int64_t ws_tok = (int64_t)H * 256;  // elements between tokens

  for (int base = stream; base < T; base += kStreams * kUnroll) {
    u32x4 kk[kUnroll], vv[kUnroll];
    float kr[kUnroll][4];
    float s[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = min(base + kStreams * u, T - 1);
      kk[u] = *reinterpret_cast<const u32x4*>(ws + t * ws_tok);
      vv[u] = *reinterpret_cast<const u32x4*>(ws + t * ws_tok + 128);
      const int64_t slot = naive_slot<PAGED>(a, b, t);
      if (!FP8) {
        const u32x2 p = *reinterpret_cast<const u32x2*>(a.pe + slot * a.pe_sb + 8 * j);
        kr[u][0] = lo16(p[0]);
        kr[u][1] = hi16(p[0]);
        kr[u][2] = lo16(p[1]);
        kr[u][3] = hi16(p[1]);
      } else {
        const float sc = a.token_scale[slot];
        const uint32_t p = *reinterpret_cast<const uint32_t*>(a.pe + slot * a.pe_sb + 4 * j);
        const f32x2 lo = e4m3x2_to_f32<false>(p), hi = e4m3x2_to_f32<true>(p);
        kr[u][0] = lo[0] * sc;
        kr[u][1] = lo[1] * sc;
        kr[u][2] = hi[0] * sc;
        kr[u][3] = hi[1] * sc;
      }
    }
    float m_new = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int k = 0; k < 4; ++k) d += qn[2 * k] * lo16(kk[u][k]) + qn[2 * k + 1] * hi16(kk[u][k]);
#pragma unroll
      for (int k = 0; k < 4; ++k) d += qr[k] * kr[u][k];
      d = row_sum16(d) * a.scale_log2;
      s[u] = base + kStreams * u < T ? d : -INFINITY;
      m_new = fmaxf(m_new, s[u]);
    }
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = base + kStreams * u < T ? fast_exp2(s[u] - m_new) : 0.0f;
      l += p;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        o[2 * k] += p * lo16(vv[u][k]);
        o[2 * k + 1] += p * hi16(vv[u][k]);
      }
    }
    m = m_new;
  }

#pragma unroll
  for (int k = 0; k < 8; ++k) so[stream][8 * j + k] = o[k];
  if (j == 0) {
    sml[stream][0] = m;
    sml[stream][1] = l;
  }
  __syncthreads();
  if (tid < kDv) {
    float M = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < kStreams; ++s2) M = fmaxf(M, sml[s2][0]);
    float L = 0.0f, x = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < kStreams; ++s2) {
      const float e = sml[s2][0] == -INFINITY ? 0.0f : fast_exp2(sml[s2][0] - M);
      L += e * sml[s2][1];
      x += e * so[s2][tid];
    }
    const float r = L > 0.0f ? x / L : 0.0f;
    a.out[((int64_t)b * H + h) * kDv + tid] = __builtin_bit_cast(uint16_t, (__bf16)r);
  }
}

template <bool PAGED, bool FP8>
hipError_t launch_naive_typed(const NaiveArgs& a, hipStream_t stream) {
  const dim3 gx((unsigned)(2 * a.num_heads), (unsigned)((a.max_seq_len + kXM - 1) / kXM), (unsigned)a.batch);
  hipLaunchKernelGGL((naive_expand_kernel<PAGED, FP8>), gx, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((naive_attend_kernel<PAGED, FP8>), dim3((unsigned)((int64_t)a.batch * a.num_heads)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_naive_decode(const NaiveArgs& a, bool fp8, hipStream_t stream) {
  const bool paged = a.block_table != nullptr;
  if (fp8) return paged ? launch_naive_typed<true, true>(a, stream) : launch_naive_typed<false, true>(a, stream);
  return paged ? launch_naive_typed<true, false>(a, stream) : launch_naive_typed<false, false>(a, stream);
}

}  // namespace mla
