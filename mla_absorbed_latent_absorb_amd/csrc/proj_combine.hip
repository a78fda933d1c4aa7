// The per-head projections around latent attention and the split-KV merge.
//
// absorb_q: q_lat[b,h,c] = sum_d q_nope[b,h,d] W_UK[h,d,c]   (key absorption,
//   "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界" §2.2)
// expand_v: out[b,h,j] = sum_c W_UV[h,j,c] o_lat[b,h,c]       (value absorption, §2.3)
// combine : LSE = ln sum_i exp(lse_i); o = sum_i exp(lse_i - LSE) o_i
// combine_expand: combine, then expand_v, in one launch
//
// Both projections are per-head batched GEMMs that are bound by reading the
// weights once (16 MiB each for 128 heads): one wave per 64 output columns
// (absorb_q) or 16 output rows (expand_v), in workgroups of one wave (fewer
// than 64 heads) or four, every operand copied into LDS as whole row
// segments, 16x16x32 bf16 MFMAs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace mla {

// ---------------------------------------------------------------------------
// Shared layout: every operand reaches LDS through 16-byte direct-to-LDS
// copies of whole rows (coalesced), the 16-byte chunks of row r stored at slot
// chunk ^ swz(r) so that the fragment reads (16 rows, one chunk each) spread
// over the banks.  Batch rows are processed in chunks of kProjRows; rows past
// the batch re-read the last row and are not stored.
// ---------------------------------------------------------------------------
constexpr int kProjRows = 32;  // batch rows per chunk

// ---------------------------------------------------------------------------
// absorb_q: wave = (head h, 64-column block cb): q_lat[b][h][64 cb + c];
// workgroup = NW waves on consecutive blocks of one head, sharing its query
// rows.
//   LDS per wave: W_UK[h][d][64 cb .. +64] as 128 rows of 128 B, 16-byte chunk
//        c of row d at slot c ^ 2 ((d / 8) % 4), and its output block as 32
//        rows of 128 B (chunk ^ b % 8) for row-wise stores; shared:
//        q_nope[b][h][:] as 32 rows of 256 B (chunk ^ b % 16).
//   D^T[c][b] = W^T . Q^T on 16x16x32 MFMAs: A[c][d] via transposing reads of
//   the W rows (one read covers 16 rows x 32 bytes; the four 8-row groups sit
//   on four different slot pairs, so the read hits every LDS bank twice, no
//   more), B[d][b] from the query rows.
// With few heads, one-wave workgroups (8 per head, 16 KiB of W_UK each) spread
// the launch over more CUs: at 16 heads the step is 0.5 us shorter than with
// two workgroups of 64 KiB per head; with 64 or more heads the launch already
// spans the chip and four-wave workgroups (2 per head) measured 0.5 us
// shorter per V3 step than one-wave ones.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 64;                       // output columns per wave
constexpr int kAbsBlocks = kDc / kAbsCols;         // waves per head
constexpr int kAbsW = kDn * kAbsCols * 2;          // 16 KiB W block per wave
constexpr int kAbsQ = kProjRows * kDn * 2;         // 8 KiB query rows
constexpr int kAbsOut = kProjRows * kAbsCols * 2;  // 4 KiB output staging per wave

template <int NW>
__global__ __launch_bounds__(64 * NW) void absorb_q_kernel(ProjArgs a) {
  static_assert(kAbsBlocks % NW == 0 && 8 % NW == 0, "blocks and query copies split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[NW * kAbsW + kAbsQ + NW * kAbsOut];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int w = wave_id();
  const uint32_t wl = lds0 + (uint32_t)w * kAbsW;
  const uint32_t ql = lds0 + NW * kAbsW;
  const uint32_t ol = ql + kAbsQ + (uint32_t)w * kAbsOut;
  // a head's workgroups run on one XCD (its query rows are fetched once)
  constexpr int kGroups = kAbsBlocks / NW;  // workgroups per head
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);
  const int h = item / kGroups, cb = (item - h * kGroups) * NW + w;
  const uint32_t ln = lane_id();
  const uint32_t nl = ln & 15u, g = ln >> 4;
  const size_t qrow_bytes = (size_t)a.num_heads * kDn * 2;  // stride of q_nope rows

  // W block of this wave: copy k (16) = rows 8k .. 8k+7 (lane l: row 8k +
  // l/8, slot l % 8, holding chunk slot ^ 2 (k % 4))
  {
    const char* wsrc = reinterpret_cast<const char*>(a.w + (size_t)h * kDn * kDc + cb * kAbsCols);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t src = (ln & 7u) ^ (2u * ((uint32_t)k & 3u));
      dma16(uniform_ptr(wsrc + (size_t)(8 * k) * (kDc * 2)), (ln >> 3) * (kDc * 2) + src * 16, wl + k * 1024);
    }
  }
  // query rows b0 .. b0+31: copy k (8 per workgroup, k % NW = w) = rows 4k ..
  // 4k+3 (lane l: row 4k + l/16, slot l % 16); rows past the batch re-read
  // the last one, and copies that hold no row of the batch are skipped (the
  // MFMA columns of those rows are not stored)
  auto stage_q = [&](int b0) {
    const char* qbase = reinterpret_cast<const char*>(a.x + (size_t)h * kDn);
#pragma unroll
    for (int i = 0; i < 8 / NW; ++i) {
      const int k = NW * i + w;
      if (b0 + 4 * k >= a.batch) continue;
      const int r0 = b0 + 4 * k;
      const uint32_t row = 4 * k + (ln >> 4);
      const int br = min(b0 + (int)row, a.batch - 1);
      const uint32_t src = (ln & 15u) ^ (row & 15u);
      dma16(uniform_ptr(qbase + (size_t)r0 * qrow_bytes), (uint32_t)(br - r0) * (uint32_t)qrow_bytes + src * 16,
            ql + k * 1024);
    }
  };
  stage_q(0);
  wait_vmcnt<0>();
  barrier();

  // A fragments (column tile ct = 16 ct .. +15 of the block, k-step s): lane
  // (nl, g) gets W[32 s + 8 g + i][c = 16 ct + nl], two transposing reads of 4 rows
  bf16x8 af[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const uint32_t colb = (uint32_t)(32 * ct) + (nl & 3u) * 8;  // byte in the 128 B row
      bf16x4 half[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t row = 32 * s + 8 * g + 4 * e + (nl >> 2);
        const uint32_t chunk = (colb >> 4) ^ (2u * ((row >> 3) & 3u));
        half[e] = lds_read_tr16(wl + row * 128 + (chunk << 4) + (colb & 15u));
      }
      af[ct][s] = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }

  for (int b0 = 0; b0 < a.batch; b0 += kProjRows) {
    if (b0 > 0) {
      stage_q(b0);
      wait_vmcnt<0>();
      barrier();
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      // B fragments: Q[b = 16 mb + nl][d = 32 s + 8 g .. +7]
      bf16x8 bq[4];
      const uint32_t brow = 16 * mb + nl;
#pragma unroll
      for (int s = 0; s < 4; ++s) bq[s] = lds_read_b128(ql + brow * 256 + (((uint32_t)(4 * s) + g) ^ (brow & 15u)) * 16);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma16(af[ct][s], bq[s], acc);
        // D^T[c = 16 ct + 4 g + j][b = 16 mb + nl] -> staging row b, 8 bytes
        const uint32_t c = 16 * ct + 4 * g;
        const uint32_t chunk = (c >> 3) ^ (brow & 7u);
        const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        lds_write_b64(ol + brow * 128 + (chunk << 4) + (c & 7u) * 2, v);
      }
    }
    barrier();
    // 32 rows x 8 chunks of 16 B -> q_lat row segments (128 contiguous bytes per row)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t idx = (uint32_t)(k * 64) + ln;
      const uint32_t row = idx >> 3, chunk = idx & 7u;
      const int b = b0 + (int)row;
      const u32x4 v = lds_read_u32x4(ol + row * 128 + ((chunk ^ (row & 7u)) << 4));
      if (b < a.batch)
        *reinterpret_cast<u32x4*>(a.y + ((size_t)b * a.num_heads + h) * kDc + cb * kAbsCols + chunk * 8) = v;
    }
    barrier();  // the query rows and the staging area are reused
  }
}

// ---------------------------------------------------------------------------
// expand_v: wave = (head h, 16 output rows jb): out[b][h][16 jb + j];
// workgroup = NW waves on consecutive row blocks of one head, sharing its
// o_lat rows.
//   LDS: W_UV[h][16 jb .. +16][:] as 16 rows of 1 KiB per wave (chunk ^ j % 16)
//        and o_lat[b][h][:] as 32 rows of 1 KiB (chunk ^ b % 16), shared.
//   D[j][b] = W . O^T on 16x16x32 MFMAs over the 512 latent columns.
// NW = 4 (two workgroups per head) from 64 heads; below, one wave per
// workgroup (8 per head) spreads the launch over more CUs.  o_lat rows past
// the batch are not copied: the MFMA columns they feed are not stored.
// ---------------------------------------------------------------------------
constexpr int kExpRows = 16;                       // output rows (j) per wave
constexpr int kExpBlocks = kDv / kExpRows;         // waves per head
constexpr int kExpW = kExpRows * kDc * 2;          // 16 KiB per wave
constexpr int kExpO = kProjRows * kDc * 2;         // 32 KiB

template <int NW>
__global__ __launch_bounds__(64 * NW) void expand_v_kernel(ProjArgs a) {
  static_assert(kExpBlocks % NW == 0 && kProjRows % NW == 0, "blocks and rows split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[NW * kExpW + kExpO];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int w = wave_id();
  const uint32_t wl = lds0 + (uint32_t)w * kExpW, ol = lds0 + NW * kExpW;
  constexpr int kGroups = kExpBlocks / NW;  // workgroups per head
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);
  const int h = item / kGroups, jb = (item - h * kGroups) * NW + w;
  const int nl = threadIdx.x & 15, g = (threadIdx.x & 63) >> 4;
  const size_t orow_bytes = (size_t)a.num_heads * kDc * 2;

  // W rows 16 jb .. +15 (contiguous 16 KiB): copy k (16) = row k
  {
    const uint32_t ln = lane_id();
    const char* wsrc = reinterpret_cast<const char*>(a.w + ((size_t)h * kDv + kExpRows * jb) * kDc);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      dma16(uniform_ptr(wsrc + (size_t)k * (kDc * 2)), (ln ^ (uint32_t)(k & 15)) * 16, wl + k * 1024);
  }
  // o_lat rows b0 .. b0+31 below the batch: copy k (k % NW = w) = row k
  auto stage_o = [&](int b0) {
    const uint32_t ln = lane_id();
    const char* obase = reinterpret_cast<const char*>(a.x + (size_t)h * kDc);
#pragma unroll
    for (int i = 0; i < kProjRows / NW; ++i) {
      const int k = NW * i + w;
      if (b0 + k < a.batch)
        dma16(uniform_ptr(obase + (size_t)(b0 + k) * orow_bytes), (ln ^ (uint32_t)(k & 15)) * 16, ol + k * 1024);
    }
  };
  stage_o(0);
  wait_vmcnt<0>();
  barrier();

  const uint32_t jrow = (uint32_t)nl;  // A row of this lane (within the wave's 16 rows)
  for (int b0 = 0; b0 < a.batch; b0 += kProjRows) {
    if (b0 > 0) {
      stage_o(b0);
      wait_vmcnt<0>();
      barrier();
    }
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t chunk = (uint32_t)(4 * s + g);
      const bf16x8 aw = lds_read_b128(wl + jrow * 1024 + ((chunk ^ (jrow & 15u)) << 4));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint32_t brow = 16 * mb + nl;
        const bf16x8 bo = lds_read_b128(ol + brow * 1024 + ((chunk ^ (brow & 15u)) << 4));
        acc[mb] = mfma16(aw, bo, acc[mb]);
      }
    }
    // D[j = 16 jb + 4 g + r][b = b0 + 16 mb + nl]: four consecutive output columns
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int b = b0 + 16 * mb + nl;
      if (b < a.batch) {
        const u32x2 v = {pack_bf16x2(acc[mb][0], acc[mb][1]), pack_bf16x2(acc[mb][2], acc[mb][3])};
        *reinterpret_cast<u32x2*>(a.y + ((size_t)b * a.num_heads + h) * kDv + kExpRows * jb + 4 * g) = v;
      }
    }
    barrier();  // the o_lat rows are reused
  }
}

// ---------------------------------------------------------------------------
// Split merge of one (sequence, head) row by one wave; lane l handles latent
// columns 8 l .. 8 l + 7 of the bf16 partial rows.  The rows of the first 8
// splits and the split lse values are all requested before any of them is
// used (one memory round trip); lane i holds split i's lse and weight, read
// by the other lanes with readlane; maxima and sums over the wave use DPP and
// permlane swaps.  Splits past the first 8 (P > 8) are read in
// further groups of 8.  combine_row_finish returns the lane's 8 merged
// columns as bf16 and the row's lse (every lane).  combine_kernel and
// combine_expand_kernel both merge through these functions, so their o_lat
// bits agree.
// ---------------------------------------------------------------------------
// Whole-wave reductions without LDS: DPP within rows of 16 lanes (pairs
// xor 1, xor 2, then the half-row and row mirrors), then the two permlane
// swaps.  Every lane ends with the same value (each step combines two
// operands with a commutative op).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm(1, 0, 3, 2)
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm(2, 3, 0, 1)
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  return sum_xor32(sum_xor16(x));
}

struct CombineRow {
  const float* lse_row;
  const uint16_t* prow;
  size_t split_stride;
  float li0;
  u32x4 v[8];
};

// Partial rows of one sequence: splits first .. first + P - 1 of the partial
// arrays (uniform splits: first = b * P).  A planned merge reads them from the
// per-sequence map seq_first; a malformed range (no splits, or outside the
// num_items partials) is reported as invalid and merges to o = 0, lse = -inf.
struct SplitRange {
  int first, P;
  bool valid;
};
__device__ __forceinline__ SplitRange split_range(const int32_t* seq_first, int num_splits, int b) {
  if (seq_first == nullptr) return SplitRange{b * num_splits, num_splits, true};
  const int f = scalar_load(seq_first, (size_t)b), e = scalar_load(seq_first, (size_t)b + 1);
  if (f < 0 || e <= f || e > num_splits) return SplitRange{0, 1, false};  // loads stay in bounds, result masked
  return SplitRange{f, e - f, true};
}

// Issue: lse of split `lane` (lanes < P, up to 64) and the first 8 rows.
__device__ __forceinline__ CombineRow combine_row_issue(const uint16_t* o_part, const float* lse_part, int num_heads,
                                                        int P, int first, int h, int lane) {
  CombineRow r;
  r.lse_row = lse_part + (size_t)first * num_heads + h;
  r.prow = o_part + ((size_t)first * num_heads + h) * kDc + lane * 8;
  r.split_stride = (size_t)num_heads * kDc;
  // Loads are unconditional (splits past P re-read the last one; those
  // values are never used): conditional loads make the compiler copy the
  // results, which waits for them before the next row's loads are issued.
  const float li = r.lse_row[(size_t)min(lane, P - 1) * num_heads];
  r.li0 = lane < P ? li : -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) r.v[j] = *reinterpret_cast<const u32x4*>(r.prow + (size_t)min(j, P - 1) * r.split_stride);
  return r;
}

__device__ __forceinline__ u32x4 combine_row_finish(CombineRow& r, int num_heads, int P, int lane, float& lse_out) {
  float m = r.li0;
  for (int i = 64 + lane; i < P; i += 64) m = fmaxf(m, r.lse_row[(size_t)i * num_heads]);
  m = wave_max(m);

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  auto accumulate = [&](float wl, int n) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < n) {
        const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          acc0[2 * e] += wi * __uint_as_float(r.v[j][e] << 16);
          acc0[2 * e + 1] += wi * __uint_as_float(r.v[j][e] & 0xffff0000u);
          acc1[2 * e] += wi * __uint_as_float(r.v[j][2 + e] << 16);
          acc1[2 * e + 1] += wi * __uint_as_float(r.v[j][2 + e] & 0xffff0000u);
        }
      }
    }
  };
  if (m != -INFINITY) {
    // weight of split lane (0 for empty splits and lanes past P)
    const float w0 = r.li0 == -INFINITY ? 0.f : __expf(r.li0 - m);
    tot = wave_sum(w0);
    accumulate(w0, min(P, 8));
    for (int i0 = 8; i0 < P; i0 += 8) {
      const int n = min(8, P - i0);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < n) r.v[j] = *reinterpret_cast<const u32x4*>(r.prow + (size_t)(i0 + j) * r.split_stride);
      // weights of splits i0 .. i0+7 on lanes 0..7 (the lse of splits >= 64 re-read here)
      const int si = i0 + (lane & 7);
      const float li = si < P ? r.lse_row[(size_t)si * num_heads] : -INFINITY;
      const float wl = li == -INFINITY ? 0.f : __expf(li - m);
      if (i0 >= 64) {
        // splits 64.. were not in the lane-wise total above
        tot += wave_sum(lane < 8 && si < P ? wl : 0.f);
      }
      accumulate(wl, n);
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  lse_out = tot > 0.f ? m + __logf(tot) : -INFINITY;
  return u32x4{pack_bf16x2(acc0[0] * inv, acc0[1] * inv), pack_bf16x2(acc0[2] * inv, acc0[3] * inv),
               pack_bf16x2(acc1[0] * inv, acc1[1] * inv), pack_bf16x2(acc1[2] * inv, acc1[3] * inv)};
}

// combine: one wave per (sequence, head).
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  // Sequences map to XCDs the way the decode kernel's splits do, so a
  // sequence's partial rows may still be in that XCD's L2.
  const int wid = xcd_grouped_index(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  if (wid >= a.batch * a.num_heads) return;
  const int b = wid / a.num_heads;
  const int h = wid - b * a.num_heads;
  const int lane = threadIdx.x & 63;
  float lse;
  const SplitRange sr = split_range(a.seq_first, a.num_splits, b);
  CombineRow r = combine_row_issue(a.o_part, a.lse_part, a.num_heads, sr.P, sr.first, h, lane);
  u32x4 o = combine_row_finish(r, a.num_heads, sr.P, lane, lse);
  if (!sr.valid) {
    o = u32x4{0u, 0u, 0u, 0u};
    lse = -INFINITY;
  }
  *reinterpret_cast<u32x4*>(a.o_lat + ((size_t)b * a.num_heads + h) * kDc + lane * 8) = o;
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)b * a.num_heads + h] = lse;
}

// ---------------------------------------------------------------------------
// combine_expand: the split merge and value absorption of one head for up to
// 32 sequences in one launch: out[b][h][:] = W_UV[h] . merge_i(o_part[b][i][h]).
// Workgroup = (head h, sequences R bg .. R bg + R - 1), R = 4, 8, 16 or 32
// (fewer when batch x heads is small, so the launch still spans the chip),
// 16 waves in two roles, so that no wave waits for loads it does not need:
//   - waves w < min(8, R / 2) merge sequences R bg + 16 p + 2 w, + 1 (pass p
//     < R / 16, at least one) with combine_row_issue / _finish (the same
//     arithmetic as combine_kernel; both rows' loads are issued first) into
//     rows of a bf16 tile of up to 32 rows in LDS (chunk ^ b % 16), also
//     stored as o_lat / lse if asked for (tile rows past R are not written:
//     the MFMA columns they feed are not stored);
//   - waves 8 .. 15 copy W_UV[h] (128 rows of 1 KiB) direct-to-LDS, 16 rows
//     each (chunk ^ j % 16).
//   Then D[j][b] = W . O^T as in expand_v_kernel (wave w < 8: rows 16 w ..
//   +15, the same MFMA order per 16 sequences), so out matches the two-launch
//   path bit for bit.
// The head's sequence groups are consecutive items on one XCD, which then
// fetches W_UV[h] once.  With 32 sequences per workgroup each copy of W_UV[h]
// into LDS serves twice as many sequences (at 128 x 128 rows the copies move
// 67 MB instead of 134 MB from L2).
// ---------------------------------------------------------------------------
constexpr int kCeRows = 32;                  // most sequences per workgroup
constexpr int kCeW = kDv * kDc * 2;          // 128 KiB

// RMAX: most sequences per workgroup of the instantiation (16 or 32); the
// 16-row form keeps its loops at one pass.
template <int RMAX>
__global__ __launch_bounds__(1024) void combine_expand_kernel(CombineExpandArgs a) {
  static_assert(RMAX == 16 || RMAX == 32, "one or two 16-row passes");
  constexpr int kCeO = RMAX * kDc * 2;  // the merged rows, 1 KiB each
  static_assert(kCeW + kCeO <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[kCeW + kCeO];
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t wl = lds0, ol = lds0 + kCeW;
  const int R = a.rows;
  const int groups = (a.batch + R - 1) / R;
  const int item = xcd_grouped_index(blockIdx.x, gridDim.x);
  const int h = item / groups, bg = item - h * groups;
  const int w = wave_id();
  const int lane = threadIdx.x & 63;
  const int nl = lane & 15, g = lane >> 4;

  if (2 * w < R && w < 8) {
    // rows 16 p + 2 w, + 1 (sequences past the batch repeat the last one and
    // are not stored)
    for (int p = 0; p < RMAX / 16 && 16 * p < R; ++p) {
      int b[2];
      SplitRange sr[2];
      CombineRow row[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        b[i] = min(R * bg + 16 * p + 2 * w + i, a.batch - 1);
        sr[i] = split_range(a.seq_first, a.num_splits, b[i]);
        row[i] = combine_row_issue(a.o_part, a.lse_part, a.num_heads, sr[i].P, sr[i].first, h, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 16 * p + 2 * w + i;
        const bool store = R * bg + r < a.batch;
        float lse;
        u32x4 o = combine_row_finish(row[i], a.num_heads, sr[i].P, lane, lse);
        if (!sr[i].valid) {
          o = u32x4{0u, 0u, 0u, 0u};
          lse = -INFINITY;
        }
        lds_write_u32x4(ol + (uint32_t)r * 1024u + (((uint32_t)lane ^ ((uint32_t)r & 15u)) << 4), o);
        if (store && a.o_lat != nullptr)
          *reinterpret_cast<u32x4*>(a.o_lat + ((size_t)b[i] * a.num_heads + h) * kDc + lane * 8) = o;
        if (store && a.lse != nullptr && lane == 0) a.lse[(size_t)b[i] * a.num_heads + h] = lse;
      }
    }
  } else if (w >= 8) {
    // W_UV[h] rows 16 (w - 8) .. +15: copy k = row k, chunk slot ^ (k % 16)
    const uint32_t ln = lane_id();
    const char* wsrc = reinterpret_cast<const char*>(a.w_uv + (size_t)h * kDv * kDc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = 16 * (w - 8) + i;
      dma16(uniform_ptr(wsrc + (size_t)k * (kDc * 2)), (ln ^ (uint32_t)(k & 15)) * 16, wl + k * 1024);
    }
  }
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  barrier();
  if (w >= kDv / 16) return;

  const uint32_t jrow = 16 * w + nl;  // A row of this lane
  for (int nb = 0; nb < RMAX / 16 && 16 * nb < R; ++nb) {
    const uint32_t brow = 16 * (uint32_t)nb + nl;  // B row (sequence) of this lane
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const uint32_t chunk = (uint32_t)(4 * s + g);
      const bf16x8 aw = lds_read_b128(wl + jrow * 1024 + ((chunk ^ (jrow & 15u)) << 4));
      const bf16x8 bo = lds_read_b128(ol + brow * 1024 + ((chunk ^ (brow & 15u)) << 4));
      acc = mfma16(aw, bo, acc);
    }
    // D[j = 16 w + 4 g + r][b = R bg + 16 nb + nl]: four consecutive output columns
    const int bo = R * bg + (int)brow;
    if ((int)brow < R && bo < a.batch) {
      const u32x2 v = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(a.out + ((size_t)bo * a.num_heads + h) * kDv + 16 * w + 4 * g) = v;
    }
  }
}

hipError_t launch_absorb_q(const ProjArgs& a, hipStream_t stream) {
  if (a.num_heads >= 64)
    hipLaunchKernelGGL(absorb_q_kernel<4>, dim3(a.num_heads * (kAbsBlocks / 4)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(absorb_q_kernel<1>, dim3(a.num_heads * kAbsBlocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_expand_v(const ProjArgs& a, hipStream_t stream) {
  if (a.num_heads >= 64)
    hipLaunchKernelGGL(expand_v_kernel<4>, dim3(a.num_heads * (kExpBlocks / 4)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(expand_v_kernel<1>, dim3(a.num_heads * kExpBlocks), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine_expand(const CombineExpandArgs& a_in, hipStream_t stream) {
  CombineExpandArgs a = a_in;
  // sequences per workgroup: the most (up to 32) that keeps the grid at >= 256
  // workgroups, at least 4
  const int64_t rows_total = (int64_t)a.batch * a.num_heads;
  a.rows = 4;
  while (a.rows < kCeRows && rows_total >= 256 * (int64_t)(2 * a.rows)) a.rows *= 2;
  const int groups = (a.batch + a.rows - 1) / a.rows;
  if (a.rows > 16)
    hipLaunchKernelGGL(combine_expand_kernel<32>, dim3(a.num_heads * groups), dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL(combine_expand_kernel<16>, dim3(a.num_heads * groups), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  const int waves = a.batch * a.num_heads;
  hipLaunchKernelGGL(combine_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
