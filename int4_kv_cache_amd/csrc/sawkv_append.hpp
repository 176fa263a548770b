// Input side of the append kernels, shared by the INT4 path and the INT8
// control: per-tensor and per-call parameters, the fetch of a wave's 16
// vectors and the rotation of the fetched fp16 values.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "sawkv_device.hpp"

namespace sawkv {

struct AppendTensor {
  const __half* src;     // [T][H][D], row stride `stride` elements
  int64_t stride;
  uint8_t* codes;        // [n_slots][H][D/2] (INT4) or [n_slots][H][D] (INT8 control)
  __half* scales;        // [n_slots][H]
};

struct AppendParams {
  AppendTensor t[2];     // blockIdx.y selects the tensor
  const int64_t* slots;  // [T]
  int64_t n_slots;       // N_pg * P
  int32_t T;
  int32_t TH;            // T * H vectors per tensor
  int32_t H;
  uint32_t h_magic;      // ceil(2^20 / H): n / H = (n * h_magic) >> 20 for n < 2^9
};

// u = float32 input (HB == 0, naive INT4), or F_h(x) up to the lane's sign;
// returns csg with y = f32(u * csg) the rotated vector f32(c_h * F_h(x))
// (csg = +-c_h, exact sign), or 1 for HB == 0.
template <int HB>
__device__ __forceinline__ float load_rotate(const uint4 (&raw)[4], float (&u)[kElems], int lam) {
  if constexpr (HB == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const __half2 hv = __builtin_bit_cast(__half2, w[m]);
        u[8 * i + 2 * m] = __low2float(hv);
        u[8 * i + 2 * m + 1] = __high2float(hv);
      }
    }
    return 1.0f;
  } else {
    // stride-1 butterflies straight from the fp16 pairs: fma(b, 1, a) = f32(a + b)
    // and fma(b, -1, a) = f32(a - b), one mixed-precision fma each
    const float one = opaque(1.0f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const __half2 hv = __builtin_bit_cast(__half2, w[m]);
        const float a = __low2float(hv), b = __high2float(hv);
        u[8 * i + 2 * m] = __builtin_fmaf(b, one, a);
        u[8 * i + 2 * m + 1] = __builtin_fmaf(b, -one, a);
      }
    }
    return c_h<HB>() * fwht_rest<HB>(u, lam);
  }
}

// y = float32 input, or f32(c_h * F_h(x)) with the lane's sign removed.
// HB == 0: no rotation (naive INT4).
template <int HB>
__device__ __forceinline__ void load_transform(const uint4 (&raw)[4], float (&y)[kElems],
                                               int lam) {
  const float csg = load_rotate<HB>(raw, y, lam);
  if constexpr (HB != 0) {
#pragma unroll
    for (int k = 0; k < kElems; ++k) y[k] = y[k] * csg;
  }
}

// (a << 4) | b as one instruction (kept from being re-associated)
__device__ __forceinline__ uint32_t shl4_or(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_lshl_or_b32 %0, %1, 4, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ uint32_t shl8_or(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_lshl_or_b32 %0, %1, 8, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// One wave's share of work: 16 consecutive (token, head) vectors, loaded.
struct Fetched {
  uint4 raw[4];
  int64_t slot;
  int32_t head;
  bool in_range;
};

// Wave-uniform position of the first vector of a batch: v0 = t0 * H + h0.
struct WavePos {
  uint32_t v0, t0, h0;
};

__device__ __forceinline__ Fetched fetch_batch(const AppendTensor& A, const AppendParams& p,
                                               WavePos w, int lam, int vq) {
  Fetched f;
  const uint32_t n = w.h0 + (uint32_t)vq;                 // < H + 16
  uint32_t dt = (n * p.h_magic) >> 20;                    // n / H, exact for n < 2^9
  f.head = (int32_t)(n - dt * (uint32_t)p.H);
  f.in_range = w.v0 + (uint32_t)vq < (uint32_t)p.TH;
  dt = min(dt, (uint32_t)p.T - 1u - w.t0);                // out-of-range lanes: a valid row
  const char* base = reinterpret_cast<const char*>(A.src) + (int64_t)w.t0 * A.stride * 2;
  const uint32_t off = dt * (uint32_t)A.stride * 2u + (uint32_t)f.head * (kD * 2) + 16u * lam;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    f.raw[i] = *reinterpret_cast<const uint4*>(base + off + 64 * i);
  f.slot = p.slots[w.t0 + dt];
  return f;
}

}  // namespace sawkv
