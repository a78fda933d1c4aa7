// Device-side building blocks shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kDc = 512;            // kv_lora_rank
constexpr int kDr = 64;             // qk_rope_head_dim
constexpr int kDk = kDc + kDr;      // 576: width of one cached token
constexpr int kDn = 128;            // qk_nope_head_dim
constexpr int kDv = 128;            // v_head_dim

// 16x16x32 bf16 MFMA: D[16x16] += A[16x32] * B[32x16] in fp32.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) + j][l%16] for j = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte LDS read at a byte offset into the LDS window.
__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
      (uintptr_t)byte_off);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// if lane i points at row i/4, columns 4*(i%4) .. +3 of a 4 x 16 block of
// 16-bit elements, lane j receives column j of the four rows.
__device__ __forceinline__ bf16x4 lds_read_tr16(uint32_t byte_off) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)byte_off);
  return __builtin_bit_cast(bf16x4, v);
}

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4, scalar
// base + 32-bit per-lane offset).  Lane i reads sbase + voff and writes bytes
// [lds_base + 16*i, +16).  lds_base and sbase must be wave-uniform (lds_base is
// moved to a scalar register here even where the compiler cannot prove it).
// It is issued through inline asm so the compiler does not add a conservative
// vmcnt(0) before every later LDS read; completion is tracked explicitly with
// wait_vmcnt() followed by a workgroup barrier.  An SALU write of M0 needs one
// wait state before a load with LDS = 1 reads it (s_nop 0).
// NT sets the instruction's non-temporal bit, for data read exactly once
// (the cache tiles): streaming a V3-sized cache into LDS with it ran at 6.5
// TB/s against 5.75 TB/s without (copies alone, one workgroup per CU).
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  if (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase)
                 : "memory");
}
// The same with the instruction's immediate offset OFF, which the hardware
// adds to both addresses, and M0 = lds_base + MADD: lane i reads
// sbase + voff + OFF and writes bytes [lds_base + MADD + OFF + 16*i, +16)
// (checked on gfx950 with an in-bounds probe).
template <int OFF, int MADD, bool NT = false>
__device__ __forceinline__ void dma16_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  if (NT)
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3 nt"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase), "n"(OFF), "n"(MADD)
                 : "memory");
  else
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
                 :
                 : "s"(m0), "v"(voff), "s"(sbase), "n"(OFF), "n"(MADD)
                 : "memory");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane i writes
// [lds_base + 4*i, +4).
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(sbase)
               : "memory");
}

// The same with the immediate offset OFF (added to both addresses, as for
// dma16_off) and M0 = lds_base + MADD.
template <int OFF, int MADD>
__device__ __forceinline__ void dma4_off(const void* sbase, uint32_t voff, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 offset:%3"
               :
               : "s"(m0), "v"(voff), "s"(sbase), "n"(OFF), "n"(MADD)
               : "memory");
}

// Two OCP E4M3 (e4m3fn) codes, bytes 2*HI and 2*HI+1 of a 32-bit word, to
// fp32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
}

// Make a pointer that is uniform in value also uniform in register class.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS hand-offs between waves.  s_barrier does not
// wait for this wave's memory operations (the compiler adds no wait before
// it on gfx950), so LDS writes issued just before it could still be pending
// when another wave reads after it: the LDS (and scalar) operations of the
// wave are completed first (lgkmcnt(0)).  Vector-memory loads, the
// direct-to-LDS tile copies among them, stay in flight; their completion is
// awaited explicitly with wait_vmcnt.  The memory clobbers keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

// XOR swizzles of the 16-byte chunk index inside the rows of an LDS cache
// tile, as functions of the row.  gfx950's LDS has 64 four-byte banks, i.e.
// 16 sixteen-byte bank slots.
//
// Latent rows are 1024 bytes (every row starts in bank 0).  kv_swizzle keeps
// both read patterns of the decode kernel conflict-free:
//   - 16 consecutive rows, one chunk each (K fragment of the score MFMA):
//     the XOR value is a bijection of row % 16;
//   - 8 consecutive rows x 2 adjacent chunks {2m, 2m+1} (two transposing reads
//     of the V fragment of the P.V MFMA): the XOR value / 2 differs for the 8
//     rows, so the 16 chunk reads land in 16 different slots.
__device__ __forceinline__ uint32_t kv_swizzle(uint32_t row) {
  return ((row & 7u) << 1) | ((row >> 3) & 1u);
}
// RoPE rows are 128 bytes (8 chunks; odd rows start half a bank sweep after
// even rows): the XOR value is a bijection of (row / 2) % 8.
__device__ __forceinline__ uint32_t pe_swizzle(uint32_t row) { return (row >> 1) & 7u; }

__device__ __forceinline__ void lds_write_b64(uint32_t byte_off, u32x2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ void lds_write_f32x4(uint32_t byte_off, f32x4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) f32x4*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ void lds_write_u32x4(uint32_t byte_off, u32x4 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x4*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ void lds_write_f32(uint32_t byte_off, float v) {
  *reinterpret_cast<__attribute__((address_space(3))) float*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ void lds_write_u32(uint32_t byte_off, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ float lds_read_f32(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) float*>((uintptr_t)byte_off);
}
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)byte_off);
}
__device__ __forceinline__ u32x4 lds_read_u32x4(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>((uintptr_t)byte_off);
}
__device__ __forceinline__ f32x4 lds_read_f32x4(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>((uintptr_t)byte_off);
}

// Scalar (wave-uniform) load of an int32 through the constant address space:
// a vector load would make the compiler wait for every copy in flight.
__device__ __forceinline__ int32_t scalar_load(const int32_t* p, size_t i) {
  return reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(reinterpret_cast<uintptr_t>(p))[i];
}

// Work item of a planned decode: (sequence, first 32-token tile, tile count,
// partial row).  Workgroup i of the launch runs item i and writes partial row
// `slot`.  A malformed item (sequence outside [0, batch), negative tile index,
// no tiles) covers no tokens; ranges are clamped to max_tiles; an item whose
// partial row lies outside [0, num_items) writes nothing.
struct PlanItem {
  int seq;       // valid sequence (0 for a malformed item)
  int t_begin;   // first token
  int t_end;     // one past the last token (before clamping to the sequence length)
  int slot;      // partial row, or -1: write nothing
};
__device__ __forceinline__ PlanItem plan_item(const int32_t* items, int item, int batch, int max_seq_len,
                                              int num_items) {
  const int s = scalar_load(items, 4 * (size_t)item);
  const int f = scalar_load(items, 4 * (size_t)item + 1);
  const int n = scalar_load(items, 4 * (size_t)item + 2);
  const int slot = scalar_load(items, 4 * (size_t)item + 3);
  const int max_tiles = (max_seq_len + 31) / 32;
  PlanItem p{0, 0, 0, (slot >= 0 && slot < num_items) ? slot : -1};
  if (s >= 0 && s < batch && f >= 0 && f < max_tiles && n >= 1) {
    p.seq = s;
    p.t_begin = 32 * f;
    p.t_end = 32 * (f + min(n, max_tiles - f));
  }
  return p;
}

// Workgroups are handed to the 8 XCDs round-robin by id.  This maps the
// launch index so that consecutive work items (e.g. the splits of one
// sequence, which read the same query block) run on the same XCD and share
// its L2: XCD x receives the contiguous item range of its share of the grid.
__device__ __forceinline__ int xcd_grouped_index(int id, int grid) {
  constexpr int kXcd = 8;
  const int per = grid / kXcd, rem = grid % kXcd;
  const int x = id % kXcd, k = id / kXcd;
  const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + k;
}

// Cross-lane reductions between lanes l and l^16 / l^32 with the gfx950
// permlane swaps (VALU, no LDS round trip).  Each swap returns the pair
// {x[l], x[l^k]} in some order, so a commutative op of the two halves is the
// pairwise reduction.
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// IEEE maximum (NaN-propagating, +0 above -0): v_maximum3_f32 on gfx950.
// fmaxf's maxNum semantics make the compiler quiet every operand it cannot
// prove to be a non-signalling value (results of inline asm, lane swaps)
// with one extra instruction each; scores never hold NaN, where the two agree.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float vmax_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float vmax_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void lds_write_u8(uint32_t byte_off, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(3))) uint8_t*>((uintptr_t)byte_off) = (uint8_t)v;
}
__device__ __forceinline__ void lds_write_u32x2(uint32_t byte_off, u32x2 v) {
  *reinterpret_cast<__attribute__((address_space(3))) u32x2*>((uintptr_t)byte_off) = v;
}
__device__ __forceinline__ u32x2 lds_read_u32x2(uint32_t byte_off) {
  return *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>((uintptr_t)byte_off);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values -> bf16 pair (lo in bits 0..15), nearest even: one
// v_cvt_pk_bf16_f32 (two scalar casts compile to two converts, a shift and an
// OR).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Lane index recomputed at the point of use (v_mbcnt over a full mask).  It is
// opaque to the compiler on purpose: values derived from it are then computed
// where they are needed instead of being hoisted out of loops, kept live, and
// spilled under register pressure.
__device__ __forceinline__ uint32_t lane_id() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace mla
