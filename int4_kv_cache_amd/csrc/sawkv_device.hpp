// Device building blocks of the sawkv kernels (gfx950, wave64).
//
// Lane layout. One head vector has D = 128 channels and is held by a quad of
// 4 consecutive lanes; lane `lam` (0..3) of the quad holds the 32 channels
//     e = 32*i + 8*lam + j,   i = 0..3, j = 0..7,   in register x[8*i + j].
// So channel bits 0-2 (j) and 5-6 (i) are in-lane, bits 3-4 (lam) are the
// lane's position in its quad. A wave holds 16 vectors, a 256-thread block 64.
// Each lane's 8-channel chunk i is 16 contiguous bytes of fp16 input, so one
// quad reads 64 contiguous bytes per load instruction.
//
// Walsh-Hadamard butterflies. The stage of stride 2^b pairs channels that
// differ in bit b: in-lane for b in {0,1,2,5,6}, across lanes of the quad for
// b = 3 (partner lane lam^1) and b = 4 (partner lam^2). A cross-lane stage is
// one v_fmac_f32 with a DPP quad_perm operand per register:
//     x <- x + sg * x[partner],  sg = +1 on the lane holding the lower channel,
//                                sg = -1 on the other lane,
// which computes a + b on the lower lane and b - a = -(a - b) on the upper one.
// sg * x[partner] is exact, so every result is the float32-rounded a + b or
// a - b, up to a sign. The sign of every later value in a lane is the product
// of its lane's sg over the cross-lane stages done (in-lane stages keep it),
// and is removed exactly by multiplying with sign * c_h at the end. The only
// values whose sign can differ from the plain definition are exact zeros,
// which give the same INT4 code (0) either way.

#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace sawkv {

constexpr int kD = 128;
constexpr int kElems = 32;          // channels per lane
constexpr int kVecPerWave = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kVecPerBlock = kVecPerWave * kWaves;

// Keeps a value opaque to the optimiser (so fma(b, 1, a) stays one
// mixed-precision fma instead of being rewritten as convert + add).
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// float32(1/sqrt(h)): sqrt(2)'s float32 mantissa (0x3FB504F3) for odd
// log2(h), exact powers of two for even log2(h).
template <int HB>
__device__ __forceinline__ float c_h() {
  static_assert(HB == 16 || HB == 32 || HB == 64 || HB == 128, "block size");
  if constexpr (HB == 16) return 0.25f;
  if constexpr (HB == 32) return __builtin_bit_cast(float, 0x3E3504F3u);
  if constexpr (HB == 64) return 0.125f;
  return __builtin_bit_cast(float, 0x3DB504F3u);
}

// Cross-lane butterfly on 8 registers. The leading s_nop covers the
// "VALU writes a VGPR, DPP reads it" hazard (2 wait states) for the block's
// DPP reads, which the compiler cannot see inside the asm. Registers written
// by the block are DPP-read only by later blocks (which start with their own
// s_nop) or by compiler-visible code, never right after the block.
#define SAWKV_XBFLY8(NAME, PERM)                                                   \
  __device__ __forceinline__ void NAME(float& a0, float& a1, float& a2, float& a3, \
                                       float& a4, float& a5, float& a6, float& a7, \
                                       float sg) {                                 \
    asm volatile(                                                                  \
        "s_nop 1\n\t"                                                              \
        "v_fmac_f32_dpp %0, %0, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %1, %1, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %2, %2, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %3, %3, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %4, %4, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %5, %5, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %6, %6, %8 " PERM " row_mask:0xf bank_mask:0xf\n\t"        \
        "v_fmac_f32_dpp %7, %7, %8 " PERM " row_mask:0xf bank_mask:0xf"            \
        : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6),    \
          "+v"(a7)                                                                 \
        : "v"(sg));                                                                \
  }

SAWKV_XBFLY8(xbfly8_lane1, "quad_perm:[1,0,3,2]")
SAWKV_XBFLY8(xbfly8_lane2, "quad_perm:[2,3,0,1]")
#undef SAWKV_XBFLY8

// Value of the partner lane (lam ^ 1 or lam ^ 2) for reductions.
__device__ __forceinline__ float quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                            0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                            0x4E, 0xF, 0xF, true));
}

// 16-byte store marked nontemporal (streaming output that is not read back
// soon: it does not displace reusable lines from the caches).
__device__ __forceinline__ void store_stream(uint4 w, void* dst) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u4v*>(dst));
}

// In-lane butterfly stage over register-index bit (1 << RB).
template <int RB>
__device__ __forceinline__ void lane_stage(float (&x)[kElems]) {
#pragma unroll
  for (int k = 0; k < kElems; ++k) {
    if ((k & (1 << RB)) == 0) {
      const float a = x[k], b = x[k + (1 << RB)];
      x[k] = a + b;
      x[k + (1 << RB)] = a - b;
    }
  }
}

// Butterflies of F_HB, strides 2, 4, ..., HB/2 (the stride-1 stage is done by
// the caller), in increasing stride order. Returns the lane's sign.
template <int HB>
__device__ __forceinline__ float fwht_rest(float (&x)[kElems], int lam) {
  lane_stage<1>(x);                      // stride 2
  lane_stage<2>(x);                      // stride 4
  float sgn = 1.0f;
  if constexpr (HB > 8) {                // stride 8: lanes lam, lam ^ 1
    const float sg = (lam & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xbfly8_lane1(x[8 * q + 0], x[8 * q + 1], x[8 * q + 2], x[8 * q + 3],
                   x[8 * q + 4], x[8 * q + 5], x[8 * q + 6], x[8 * q + 7], sg);
    sgn *= sg;
  }
  if constexpr (HB > 16) {               // stride 16: lanes lam, lam ^ 2
    const float sg = (lam & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xbfly8_lane2(x[8 * q + 0], x[8 * q + 1], x[8 * q + 2], x[8 * q + 3],
                   x[8 * q + 4], x[8 * q + 5], x[8 * q + 6], x[8 * q + 7], sg);
    sgn *= sg;
  }
  if constexpr (HB > 32) lane_stage<3>(x);   // stride 32
  if constexpr (HB > 64) lane_stage<4>(x);   // stride 64
  return sgn;
}

}  // namespace sawkv
