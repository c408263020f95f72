// Device-side helpers shared by the gfx950 kernels of the DSA library.
// CDNA4 only: wave64, MFMA bf16/fp8 builtins, 160 KiB LDS per CU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming load: the data is read once, keep it out of the way of reused lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16x16x32 bf16 MFMA: A lane l holds row l%16, B lane l holds column l%16,
// each with 8 consecutive k-slots of group l/16; C lane l holds column l%16,
// rows 4*(l/16)+{0..3}.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// 32x32x16 bf16 MFMA: A lane l holds row l%32, B lane l holds column l%32,
// 8 k-slots of half l/32; C lane l holds column l%32,
// rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Round-to-nearest-even fp32 -> bf16 pair, packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

// Values of lanes l and l ^ 32 (v_permlane32_swap exchanges lanes 32..63 of
// its first operand with lanes 0..31 of its second; with both holding x,
// they end up as x[l] and x[l ^ 32] in some order).  Written as asm with two
// distinct in/out registers; the VALU writes of the copies need two wait
// states before the permute reads them.
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(v));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, v);
}

// Values of lanes l and l ^ 16 (v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second; with both
// holding x, one ends up with rows (0, 0, 2, 2) and the other with (1, 1, 3, 3)
// of x, so their sum is x[l] + x[l ^ 16]).  Same asm form and wait states as
// xor32_pair.
__device__ __forceinline__ void xor16_pair(float x, float& a, float& b) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(u), "+v"(v));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, v);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: expcnt and
// lgkmcnt fields left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)(p);
}

// 16-byte global -> LDS copy per lane: lane l's 16 bytes at gbase + voff go
// to LDS address lds_base + 16*l.  Written as asm so that the compiler's
// wait-count pass does not treat in-flight copies as hazards for unrelated
// LDS reads; callers await completion with wait_vmcnt<>() (and a barrier
// when other waves read the data).  An SALU write of M0 needs one wait state
// before an LDS-DMA reads it.  No memory clobber: callers order the copies
// against readers of the destination with their own waits and barriers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// NT: streaming (non-temporal) access for data read once.
template <bool NT = true>
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 ::"s"(lds_base), "v"(voff), "s"(gbase)
                 : "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 ::"s"(lds_base), "v"(voff), "s"(gbase)
                 : "m0");
}
// One byte per lane: lane l's byte at gbase + voff lands zero-extended in the
// LDS dword at lds_base + 4*l (same ordering rules as lds_dma16).
__device__ __forceinline__ void lds_dma_u8(const void* gbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ubyte %1, %2"
               ::"s"(lds_base), "v"(voff), "s"(gbase)
               : "m0");
}
#pragma clang diagnostic pop

// DPP source shift within rows of 16 lanes (lanes whose source is out of
// range read 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}

// Inclusive scan over the 64 lanes: shifts by 1, 2, 4, 8 within each row of
// 16 lanes, then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then lane 31's running total into rows 2 and 3
// (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<0x111, 0xf>(v);
  v += dpp<0x112, 0xf>(v);
  v += dpp<0x114, 0xf>(v);
  v += dpp<0x118, 0xf>(v);
  v += dpp<0x142, 0xa>(v);
  v += dpp<0x143, 0xc>(v);
  return v;
}

// Order-preserving 32-bit key of a score, as the top-k kernels rank them:
// larger score, larger key; -0.0 maps like +0.0.  Key 0 is reserved for
// "no element" (slots past a row's end): real scores map to >= 1 (only the
// all-ones NaN pattern would map to 0, and NaN scores have no defined place
// in the order).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (u == 0x80000000u) u = 0u;                 // -0.0 == +0.0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k > 1u ? k : 1u;
}

// ue8m0 exponent byte -> 2^(e-127) as fp32 (e = 0 gives 2^-127, a subnormal).
__device__ __forceinline__ float ue8m0_to_f32(uint32_t e) {
  return e == 0 ? __builtin_bit_cast(float, 0x00400000u) : __builtin_bit_cast(float, e << 23);
}

}  // namespace dsa
