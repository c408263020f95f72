// FP8 producer of the indexer's query / key vectors on gfx950.
//
// Per 128-element row x:  y = H x / sqrt(128)  (H: Sylvester Hadamard matrix,
// so H / sqrt(128) is orthonormal), then one power-of-two scale 2^e per row,
// the smallest with max|y| / 2^e <= 448, stored as the ue8m0 byte e + 127,
// and E4M3 ("fn") codes of y / 2^e, rounded to nearest with ties to even.
// HF model doc "DeepSeek-V3.2", section "DeepSeek Sparse Attention (DSA)",
// item 1 (the indexer runs in FP8 after an orthogonal Hadamard rotation, so
// rotated dot products equal the plain ones); "scale_fmt: ue8m0" in the
// released configuration excerpt of the atlas "DeepSeek-V3.2-Exp" token-ids
// page; F8_E4M3 on the drose page.
//
// 16 lanes per row, lane j holding elements 8j .. 8j+7 (one 16-byte load of
// bf16).  The rotation runs as butterflies in fp32 in a fixed order: stages
// h = 1, 2, 4 inside the lane, h = 8, 16, 32, 64 across lanes j ^ 1, 2, 4, 8,
// then one multiply by fp32(1/sqrt(128)).  The scale exponent comes from the
// bits of max|y|, and the codes from gfx950's fp32 -> E4M3 conversion
// (v_cvt_pk_fp8_f32: OCP "fn" format, round to nearest even; a sweep of
// every fp32 value of magnitude <= 448 matched that rule bit for bit), so
// the output is a pure function of the fp32 rotation.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;   // fp32(1/sqrt(128)) = 0x3db504f3

// Smallest e with amax / 2^e <= 448 = 1.75 * 2^8, from the bits of amax:
// amax = M * 2^E with M in [1, 2) gives e = E - 8 if M <= 1.75, else E - 7.
// 0 for amax == 0; clamped to [-127, 127].
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t u = __builtin_bit_cast(uint32_t, amax);
  if ((u >> 23) == 0u) return -127;               // subnormal maximum
  const int E = (int)(u >> 23) - 127;
  const int e = (u & 0x7fffffu) <= 0x600000u ? E - 8 : E - 7;
  return max(-127, min(127, e));
}

template <bool F32IN>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const void* x, int64_t rows, uint8_t* codes,
                                                           uint8_t* scales) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;                        // lane within the row
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4; r0 < rows; r0 += nwaves * 4) {
    const int64_t row = r0 + (lane >> 4);
    const bool live = row < rows;
    float v[8];
    if (live) {
      if constexpr (F32IN) {
        const float* p = static_cast<const float*>(x) + row * 128 + 8 * j;
        const f32x4 a = *reinterpret_cast<const f32x4*>(p);
        const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      } else {
        const u32x4 w = ld16(static_cast<const uint16_t*>(x) + row * 128 + 8 * j);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[2 * t] = bf16_lo(w[t]);
          v[2 * t + 1] = bf16_hi(w[t]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = 0.f;
    }
    // stages h = 1, 2, 4: pairs (t, t + h) inside the lane
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (!(t & h)) {
          const float a = v[t], b = v[t + h];
          v[t] = a + b;
          v[t + h] = a - b;
        }
    // stages h = 8, 16, 32, 64: element 8j + t pairs with lane j ^ (h / 8);
    // lanes j ^ 1 and j ^ 2 are read by DPP quad permutations (no LDS trip)
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) {
      const bool upper = (j & s) != 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float o;
        if (s == 1)
          o = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[t]), 0xB1, 0xf, 0xf, false));
        else if (s == 2)
          o = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[t]), 0x4E, 0xf, 0xf, false));
        else
          o = __shfl_xor(v[t], s, 64);
        v[t] = upper ? o - v[t] : v[t] + o;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      v[t] *= kInvSqrt128;
      amax = fmaxf(amax, fabsf(v[t]));
    }
#pragma unroll
    for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    const int e = scale_exp(amax);
    const float inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);   // 2^-e, exact
    // |v / 2^e| <= 448: every code is finite, no saturation involved
    uint32_t c[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q] * inv, v[4 * q + 1] * inv, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * q + 2] * inv, v[4 * q + 3] * inv, w, true);
      c[q] = (uint32_t)w;
    }
    if (live) {
      *reinterpret_cast<u32x2*>(codes + row * 128 + 8 * j) = u32x2{c[0], c[1]};
      if (j == 0) scales[row] = (uint8_t)(e + 127);
    }
  }
}

}  // namespace

hipError_t launch_rotate_quant(const void* x, int f32_in, int64_t rows, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
  const int64_t groups = (rows + 15) / 16;        // 16 rows per 256-thread block per pass
  const int grid = (int)(groups < 8192 ? groups : 8192);
  if (f32_in)
    hipLaunchKernelGGL(rotate_quant_kernel<true>, dim3(grid), dim3(256), 0, s, x, rows, codes, scales);
  else
    hipLaunchKernelGGL(rotate_quant_kernel<false>, dim3(grid), dim3(256), 0, s, x, rows, codes, scales);
  return hipGetLastError();
}

}  // namespace dsa
