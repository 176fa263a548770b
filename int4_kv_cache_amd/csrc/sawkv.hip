// sawkv: fused block-diagonal Hadamard + token-wise INT4 paged-KV append and
// its read-back, for MI355X (gfx950). C ABI declared in include/sawkv.h.
//
// The method (youngju.dev reading of the SAW-INT4 preprint, fused-kernel
// diagram in "The System Is the Design - A Fused Kernel"; gist.science
// summary of SAW-INT4, §2 Metodologia, BDR items 1-3): each new token's fp16
// K/V head vector is rotated by a block-diagonal Hadamard transform,
// quantised to INT4 with one scale of its own, and written to its slot of a
// paged cache in one pass that reads the input once and touches nothing else.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off
//        -Xclang -target-feature -Xclang -packed-fp32-ops
// (-ffp-contract=off keeps every float32 operation separately rounded, as the
// definition requires; fused multiply-adds appear only where written).

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "sawkv.h"
#include "sawkv_append.hpp"
#include "sawkv_device.hpp"
#include "sawkv_host.hpp"

namespace sawkv {

// ---------------------------------------------------------------------------
// append: fp16 K/V -> rotate -> token-wise INT4 -> paged pool
// ---------------------------------------------------------------------------

// Packs 8 biased codes (q + 8 in the low 4 bits of each word, constant bits
// above bit 21) into one word of nibbles: byte b = q_{2b} | q_{2b+1} << 4.
__device__ __forceinline__ uint32_t pack_low(const uint32_t* w) {
  const uint32_t p01 = shl4_or(w[1], w[0]);   // byte 0 = nibbles 0,1; byte 1 = 0
  const uint32_t p23 = shl4_or(w[3], w[2]);
  const uint32_t p45 = shl4_or(w[5], w[4]);
  const uint32_t p67 = shl4_or(w[7], w[6]);
  const uint32_t lo = shl8_or(p23, p01);      // bytes 0-1 valid
  const uint32_t hi = shl8_or(p67, p45);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x88888888u;
}

// The same from codes held in byte 2 of each word (bits 16-19, bits 20-23 zero).
__device__ __forceinline__ uint32_t pack_byte2(const uint32_t* w) {
  const uint32_t e0 = __builtin_amdgcn_perm(w[4], w[0], 0x0C060C02u);   // c0, 0, c4, 0
  const uint32_t o0 = __builtin_amdgcn_perm(w[5], w[1], 0x0C060C02u);   // c1, 0, c5, 0
  const uint32_t e1 = __builtin_amdgcn_perm(w[6], w[2], 0x0C060C02u);   // c2, 0, c6, 0
  const uint32_t o1 = __builtin_amdgcn_perm(w[7], w[3], 0x0C060C02u);   // c3, 0, c7, 0
  const uint32_t y0 = shl4_or(o0, e0);   // c0|c1<<4, 0, c4|c5<<4, 0
  const uint32_t y1 = shl4_or(o1, e1);   // c2|c3<<4, 0, c6|c7<<4, 0
  return shl8_or(y1, y0) ^ 0x88888888u;
}

// min of the low 16 bits of three words
__device__ __forceinline__ uint32_t min3_lo16(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_min3_u16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

template <int HB>
__device__ __forceinline__ void quantize_store(const AppendTensor& A, const AppendParams& p,
                                               const Fetched& f, int lam) {
  float u[kElems];
  const float csg = load_rotate<HB>(f.raw, u, lam);   // y = f32(u * csg)

  // token-wise scale: amax over the 128 channels of the vector (4 lanes).
  // max |y| = f32(c_h * max |u|): rounding is monotonic and the sign exact.
  float mu = 0.0f;
#pragma unroll
  for (int k = 0; k < kElems; ++k) mu = fmaxf(mu, fabsf(u[k]));
  mu = fmaxf(mu, quad_xor1(mu));
  mu = fmaxf(mu, quad_xor2(mu));
  float m = mu;
  if constexpr (HB != 0) m = mu * c_h<HB>();
  // s32 = RN(amax / 7) by Markstein's correction with r7 = RN(1/7); the fma
  // residual is exact, so the corrected quotient is the IEEE one
  const float r7 = __builtin_bit_cast(float, 0x3E124925u);
  const float q7 = m * r7;
  const float s32 = __builtin_fmaf(__builtin_fmaf(-q7, 7.0f, m), r7, q7);
  const __half s16 = __float2half_rn(fminf(s32, 65504.0f));   // RNE, saturating
  const float sf = __half2float(s16);
  // r = RN(1/sf): the hardware reciprocal is within one ulp; one exact Newton
  // step (residual by fma) rounds to RN(1/sf), because sf has at most 11
  // significant bits and 1/sf is then never within 2^-35 (relative) of a
  // float32 midpoint, while the corrected value is within 2^-46 of 1/sf
  const float r0 = __builtin_amdgcn_rcpf(sf);
  const float r = sf > 0.0f ? __builtin_fmaf(r0, __builtin_fmaf(-sf, r0, 1.0f), r0) : 0.0f;
  // the clamp to [-8, 7] can bite only for a saturated or an f16-subnormal scale
  const bool need_clamp = (s32 > 65504.0f) || (sf > 0.0f && sf < 6.103515625e-05f);

  // Fast route, one fma per channel: t = u * RN(c_h r) + (136.5 + 2^-16),
  // rounded once to the 2^-16 grid of [128, 256), so byte 2 of t's bits is
  // floor(t - 128) = q + 8. u * RN(c_h r) is within 2^-19 of the exact
  // quotient f32(y / s) (|q| < 7.004, four float32 roundings), so the code is
  // rint(f32(y / s)) + 8 unless a half-integer lies within that distance;
  // then t lands on or one step above an integer, its low 16 bits are 0 or 1,
  // and the wave takes the exact route below. A zero scale gives r = 0, t =
  // 136.5 + 2^-16 and code 0.
  const float cr = HB != 0 ? r * csg : r;
  const float kT = __builtin_bit_cast(float, 0x43088001u);     // 136.5 + 2^-16
  uint32_t near = 0xFFFFu;
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t[j] = __builtin_bit_cast(uint32_t, __builtin_fmaf(u[8 * i + j], cr, kT));
#pragma unroll
    for (int j = 0; j < 8; j += 2) near = min3_lo16(near, t[j], t[j + 1]);
    d[i] = pack_byte2(t);
  }

  if (__any(need_clamp || (near & 0xFFFFu) <= 1u)) {
    uint32_t w[kElems];
    // Exact route: y = f32(u * csg); q = rint(f32(y / s)) from Markstein's
    // correction of y * RN(1/s) (residual by fma, exact), which is the
    // correctly rounded quotient; adding 1.5*2^23 + 8 rounds to an integer
    // half-to-even and leaves q + 8 in the low bits.
#pragma unroll
    for (int k = 0; k < kElems; ++k) {
      const float y = HB != 0 ? u[k] * csg : u[k];
      const float q0 = y * r;
      const float e = __builtin_fmaf(-q0, sf, y);
      const float q1 = __builtin_fmaf(e, r, q0);
      w[k] = __builtin_bit_cast(uint32_t, q1 + 12582920.0f);
    }
    if (__any(need_clamp)) {
#pragma unroll
      for (int k = 0; k < kElems; ++k) w[k] = min(max(w[k], 0x4B400000u), 0x4B40000Fu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = pack_low(w + 8 * i);
  }

  if (f.in_range && f.slot >= 0 && f.slot < p.n_slots) {
    const int64_t row = f.slot * p.H + f.head;
    uint8_t* dst = A.codes + row * (kD / 2) + 4 * lam;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 16 * i) = d[i];
    if (lam == 0) A.scales[row] = s16;
  }
}

// One wave: 16 consecutive (token, head) vectors of one tensor. (A persistent
// loop with next-batch prefetch measured slower on MI355X than this one-shot
// grid: the kernel is bound by HBM, and the one-shot grid keeps more waves
// resident.)
template <int HB>
__device__ __forceinline__ void append_tensor(const AppendTensor& A, const AppendParams& p,
                                              uint32_t bx) {
  const int lane = threadIdx.x & 63;
  const int lam = lane & 3;
  const int vq = lane >> 2;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WavePos w;
  w.v0 = (bx * kWaves + wave) * kVecPerWave;              // wave-uniform
  if (w.v0 >= (uint32_t)p.TH) return;
  w.t0 = w.v0 / (uint32_t)p.H;
  w.h0 = w.v0 - w.t0 * (uint32_t)p.H;
  quantize_store<HB>(A, p, fetch_batch(A, p, w, lam, vq), lam);
}

// Grid (blocks, tensors): every block of the first tensor is dispatched
// before any of the second. Grid (2 * blocks, 1) with two tensors: the
// tensors' blocks alternate in dispatch order (host side: only for inputs of
// at least kAlternateBytes, see append_impl).
template <int HB0, int HB1>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p) {
  if (gridDim.y == 1 && p.t[1].src != nullptr) {
    if ((blockIdx.x & 1u) == 0) append_tensor<HB0>(p.t[0], p, blockIdx.x >> 1);
    else append_tensor<HB1>(p.t[1], p, blockIdx.x >> 1);
  } else if (blockIdx.y == 0) {
    append_tensor<HB0>(p.t[0], p, blockIdx.x);
  } else {
    append_tensor<HB1>(p.t[1], p, blockIdx.x);
  }
}

// Several layers of one decode step in one launch: every layer shares the
// token count, heads, strides, slot mapping and pool geometry; blockIdx.y
// enumerates (layer, tensor). The per-layer pointers travel in the kernel
// arguments, so the call needs no device-side descriptor.
constexpr int kMaxLayers = 64;

struct LayerPtrs {
  const __half* k;
  const __half* v;
  uint8_t* k_codes;
  uint8_t* v_codes;
  __half* k_scales;
  __half* v_scales;
};

struct LayersParams {
  AppendParams common;   // its t[] are unused
  int64_t k_stride, v_stride;
  int32_t n_tensors;     // 1 or 2 per layer
  int32_t only_v;        // n_tensors == 1 and that tensor is V
  int32_t n_layers;
  LayerPtrs layer[kMaxLayers];
};

static_assert(sizeof(LayersParams) <= 4096, "kernel arguments must stay within 4 KB");

template <int HB0, int HB1>
__global__ __launch_bounds__(kThreads) void append_layers_kernel(LayersParams p) {
  // blockIdx.y = layer, blockIdx.z = tensor of the layer. Dispatch runs x,
  // then y, then z, so every layer's first tensor (K, the rotated one under
  // K-only rotation) is dispatched before any second tensor, and in a launch
  // of one round of waves the data that arrives last feeds the shorter
  // (unrotated) arithmetic. The layer's pointers are addressed by blockIdx.y
  // alone, so their argument loads go out with the first ones.
  const int slot_in_layer = (int)blockIdx.z;
  const LayerPtrs& L = p.layer[blockIdx.y];
  // every argument the wave needs, in one round of scalar loads
  asm volatile("" ::"s"(L.k), "s"(L.v), "s"(L.k_codes), "s"(L.v_codes), "s"(L.k_scales),
               "s"(L.v_scales), "s"(p.k_stride), "s"(p.v_stride), "s"(p.n_tensors),
               "s"(p.only_v), "s"(p.common.slots), "s"(p.common.n_slots), "s"(p.common.T),
               "s"(p.common.TH), "s"(p.common.H), "s"(p.common.h_magic));
  const bool is_v = p.n_tensors == 2 ? slot_in_layer == 1 : p.only_v != 0;
  const AppendTensor A = is_v ? AppendTensor{L.v, p.v_stride, L.v_codes, L.v_scales}
                              : AppendTensor{L.k, p.k_stride, L.k_codes, L.k_scales};
  if (slot_in_layer == 0) append_tensor<HB0>(A, p.common, blockIdx.x);
  else append_tensor<HB1>(A, p.common, blockIdx.x);
}

// ---------------------------------------------------------------------------
// gather: pool -> dequantise -> inverse rotation -> fp16
// ---------------------------------------------------------------------------

struct GatherTensor {
  const uint8_t* codes;  // [n_slots][H][D/2]
  const __half* scales;  // [n_slots][H]
  __half* out;           // [T][H][D]
};

struct GatherParams {
  GatherTensor t[2];
  const int64_t* slots;
  int64_t n_slots;
  int32_t T;
  int32_t TH;
  int32_t H;
  uint32_t h_magic;      // ceil(2^20 / H)
};

struct GatherFetched {
  uint32_t d[4];         // this lane's 32 codes (4 chunks of 8 nibbles)
  float sf;              // scale of the vector (0 for an invalid slot)
  int32_t v;             // vector index t * H + head (clamped into range)
  int32_t v0;            // first vector of the wave's batch
  int32_t TH;
  bool in_range;
};

__device__ __forceinline__ GatherFetched gather_fetch(const GatherTensor& G,
                                                      const GatherParams& p, uint32_t v0,
                                                      int lam, int vq) {
  GatherFetched f;
  const uint32_t H = (uint32_t)p.H;
  const uint32_t t0 = v0 / H, h0 = v0 - t0 * H;           // wave-uniform
  const uint32_t n = h0 + (uint32_t)vq;
  uint32_t dt = (n * p.h_magic) >> 20;                    // n / H, exact for n < 2^9
  const uint32_t head = n - dt * H;
  f.in_range = v0 + (uint32_t)vq < (uint32_t)p.TH;
  dt = min(dt, (uint32_t)p.T - 1u - t0);
  f.v = (int32_t)((t0 + dt) * H + head);
  f.v0 = (int32_t)v0;
  f.TH = p.TH;
  const int64_t slot = p.slots[t0 + dt];
  f.d[0] = f.d[1] = f.d[2] = f.d[3] = 0u;
  f.sf = 0.0f;
  if (slot >= 0 && slot < p.n_slots) {
    const int64_t row = slot * p.H + head;
    const uint8_t* src = G.codes + row * (kD / 2) + 4 * lam;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.d[i] = *reinterpret_cast<const uint32_t*>(src + 16 * i);
    f.sf = __half2float(G.scales[row]);
  }
  return f;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2v h2_of(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ uint32_t u_of(h2v v) { return __builtin_bit_cast(uint32_t, v); }

template <int HB>
__device__ __forceinline__ void gather_compute_store(const GatherTensor& G,
                                                     const GatherFetched& f, int lam) {
  float o[kElems];
  if constexpr (HB == 0) {
    float x[kElems];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[8 * i + j] = (float)(int)__builtin_amdgcn_sbfe(f.d[i], 4 * j, 4);
#pragma unroll
    for (int k = 0; k < kElems; ++k) o[k] = x[k] * f.sf;     // exact
  } else {
    // codes as fp16 pairs P[i][m] = (channel 8i+m, channel 8i+m+4); every
    // partial sum is an integer of magnitude <= 1024, exact in fp16
    h2v P[4][4];
    const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t x = f.d[i] ^ 0x88888888u;              // nibble + 8 in 0..15
#pragma unroll
      for (int m = 0; m < 4; ++m)
        P[i][m] = h2_of(((x >> (4 * m)) & 0x000F000Fu) | 0x64006400u) - off;   // 1024+n-1032
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int m = 0; m < 4; m += 2) {                       // stride 1
        const h2v a = P[i][m], b = P[i][m + 1];
        P[i][m] = a + b; P[i][m + 1] = a - b;
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {                          // stride 2
        const h2v a = P[i][m], b = P[i][m + 2];
        P[i][m] = a + b; P[i][m + 2] = a - b;
      }
      const h2v pm = {(_Float16)1.0f, (_Float16)-1.0f};
#pragma unroll
      for (int m = 0; m < 4; ++m)                            // stride 4 (lo, hi)
        P[i][m] = __builtin_elementwise_fma(P[i][m].yy, pm, P[i][m].xx);
    }
    float sgn = 1.0f;
    if constexpr (HB > 8) {                                  // stride 8
      const float sg = (lam & 1) ? -1.0f : 1.0f;
      const h2v s2 = {(_Float16)sg, (_Float16)sg};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          P[i][m] = __builtin_elementwise_fma(
              h2_of((uint32_t)__builtin_amdgcn_mov_dpp((int)u_of(P[i][m]), 0xB1, 0xF, 0xF, true)),
              s2, P[i][m]);
      sgn *= sg;
    }
    if constexpr (HB > 16) {                                 // stride 16
      const float sg = (lam & 2) ? -1.0f : 1.0f;
      const h2v s2 = {(_Float16)sg, (_Float16)sg};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          P[i][m] = __builtin_elementwise_fma(
              h2_of((uint32_t)__builtin_amdgcn_mov_dpp((int)u_of(P[i][m]), 0x4E, 0xF, 0xF, true)),
              s2, P[i][m]);
      sgn *= sg;
    }
    if constexpr (HB > 32) {                                 // stride 32
#pragma unroll
      for (int i = 0; i < 4; i += 2)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const h2v a = P[i][m], b = P[i + 1][m];
          P[i][m] = a + b; P[i + 1][m] = a - b;
        }
    }
    if constexpr (HB > 64) {                                 // stride 64
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const h2v a = P[i][m], b = P[i + 2][m];
          P[i][m] = a + b; P[i + 2][m] = a - b;
        }
    }
    const float csg = c_h<HB>() * sgn;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float t_lo = __builtin_fmaf((float)P[i][m].x, f.sf, 0.0f);   // exact
        const float t_hi = __builtin_fmaf((float)P[i][m].y, f.sf, 0.0f);
        o[8 * i + m] = opaque(__builtin_fmaf(t_lo, csg, 0.0f));
        o[8 * i + m + 4] = opaque(__builtin_fmaf(t_hi, csg, 0.0f));
      }
  }

  // stage the wave's 16 output rows (4 KB) through LDS, then store them as
  // four fully contiguous 1 KB wave stores, marked nontemporal; rows padded
  // to 272 bytes
  __shared__ uint4 stage[kWaves][kVecPerWave][17];
  const int wv = threadIdx.x >> 6, vq = (threadIdx.x & 63) >> 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 w;
    w.x = __builtin_bit_cast(uint32_t, __floats2half2_rn(o[8 * i + 0], o[8 * i + 1]));
    w.y = __builtin_bit_cast(uint32_t, __floats2half2_rn(o[8 * i + 2], o[8 * i + 3]));
    w.z = __builtin_bit_cast(uint32_t, __floats2half2_rn(o[8 * i + 4], o[8 * i + 5]));
    w.w = __builtin_bit_cast(uint32_t, __floats2half2_rn(o[8 * i + 6], o[8 * i + 7]));
    stage[wv][vq][4 * i + lam] = w;
  }
  __builtin_amdgcn_wave_barrier();
  const int lane = threadIdx.x & 63;
  const int32_t v_first = f.v0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4), c = lane & 15;
    const uint4 w = stage[wv][r][c];
    if (v_first + r < f.TH)
      store_stream(w, G.out + ((int64_t)v_first + r) * kD + 8 * c);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int HB>
__device__ __forceinline__ void gather_tensor(const GatherTensor& G, const GatherParams& p) {
  const int lane = threadIdx.x & 63;
  const int lam = lane & 3;
  const int vq = lane >> 2;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t v0 = (blockIdx.x * kWaves + wave) * kVecPerWave;
  if (v0 >= (uint32_t)p.TH) return;
  gather_compute_store<HB>(G, gather_fetch(G, p, v0, lam, vq), lam);
}

template <int HB0, int HB1>
__global__ __launch_bounds__(kThreads) void gather_kernel(GatherParams p) {
  if (blockIdx.y == 0) gather_tensor<HB0>(p.t[0], p);
  else gather_tensor<HB1>(p.t[1], p);
}

}  // namespace sawkv

// ---------------------------------------------------------------------------
// host side: validation, dispatch, C ABI
// ---------------------------------------------------------------------------

namespace sawkv {
namespace host {

thread_local char g_err[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return SAWKV_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_geometry(int64_t T, int32_t H, int32_t D, int64_t N_pg, int32_t P, int32_t h,
                   int32_t rot_mode, const int64_t* slots) {
  if (T < 0) return fail(SAWKV_EINVAL, "T = %lld is negative", (long long)T);
  if (H <= 0) return fail(SAWKV_EINVAL, "H = %d must be positive", H);
  if (D != sawkv::kD) return fail(SAWKV_EUNSUPPORTED, "D = %d unsupported (only 128)", D);
  if (P <= 0) return fail(SAWKV_EINVAL, "P = %d must be positive", P);
  if (N_pg <= 0) return fail(SAWKV_EINVAL, "N_pg = %lld must be positive", (long long)N_pg);
  if (N_pg > (INT64_C(1) << 40) / P || N_pg * P > (INT64_C(1) << 56) / ((int64_t)H * D))
    return fail(SAWKV_EINVAL, "pool of %lld pages x %d slots is too large", (long long)N_pg, P);
  if (h != 16 && h != 32 && h != 64 && h != 128)
    return fail(SAWKV_EUNSUPPORTED, "h = %d unsupported (16, 32, 64 or 128)", h);
  if (h > D) return fail(SAWKV_EUNSUPPORTED, "h = %d exceeds D = %d", h, D);
  if (rot_mode != SAWKV_ROT_NONE && rot_mode != SAWKV_ROT_K && rot_mode != SAWKV_ROT_KV)
    return fail(SAWKV_EINVAL, "rot_mode = %d invalid", rot_mode);
  if (H > 256) return fail(SAWKV_EUNSUPPORTED, "H = %d unsupported (at most 256)", H);
  if (T * (int64_t)H >= (INT64_C(1) << 31))
    return fail(SAWKV_EUNSUPPORTED, "T*H = %lld too large (< 2^31)", (long long)(T * H));
  if (slots == nullptr && T > 0) return fail(SAWKV_EINVAL, "slot_mapping is NULL");
  if (!aligned(slots, 8)) return fail(SAWKV_EALIGN, "slot_mapping not 8-byte aligned");
  return SAWKV_OK;
}

int check_tensor(const char* name, const void* x, int64_t stride, const void* codes,
                 const void* scales, int32_t H, int32_t D) {
  if (codes == nullptr || scales == nullptr)
    return fail(SAWKV_EINVAL, "%s pool pointer is NULL", name);
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 16))
    return fail(SAWKV_EALIGN, "%s tensor or pool pointer not 16-byte aligned", name);
  // a negative stride is below H*D too, so it is rejected here
  if (stride < (int64_t)H * D)
    return fail(SAWKV_EINVAL, "%s stride %lld < H*D = %d", name, (long long)stride, H * D);
  if (stride % 8 != 0)
    return fail(SAWKV_EALIGN, "%s stride %lld not a multiple of 8", name, (long long)stride);
  if (stride >= (INT64_C(1) << 26))
    return fail(SAWKV_EUNSUPPORTED, "%s stride %lld too large (< 2^26)", name, (long long)stride);
  return SAWKV_OK;
}

int check_output(const char* name, const void* out, const void* codes, const void* scales) {
  if (codes == nullptr || scales == nullptr)
    return fail(SAWKV_EINVAL, "%s pool pointer is NULL", name);
  if (!aligned(out, 16) || !aligned(codes, 16) || !aligned(scales, 16))
    return fail(SAWKV_EALIGN, "%s output or pool pointer not 16-byte aligned", name);
  return SAWKV_OK;
}

// K and V blocks alternate in dispatch order when the call reads at least
// kAlternateBytes of fp16 K and V, i.e. when the input streams from HBM at
// several times the 256 MB last-level cache. Measured on MI355X, alternating
// against every K block first (long-context batch of 2.1 M tokens, us per
// launch): 8 heads (8.6 GB) 2069 vs 2089, 4 heads 1037 vs 1041, 2 heads 517 vs
// 519, 1 head (1 GiB) 263.7 vs 264.2; below, prefill (0.54 GB) 127.0 vs 125.6
// and 0.27 GB 61.8 vs 60.2, where it is slower. The access-pattern control
// follows the same rule.
constexpr int64_t kAlternateBytes = INT64_C(1) << 30;

bool alternate_tensors(int64_t T, int32_t H, int32_t D) {
  return T * (int64_t)H * D * 2 * 2 >= kAlternateBytes;
}

// kernel index: 0 = naive, 1..4 = h 16/32/64/128
int hb_index(int32_t h, bool rot) {
  if (!rot) return 0;
  return h == 16 ? 1 : h == 32 ? 2 : h == 64 ? 3 : 4;
}

}  // namespace host
}  // namespace sawkv

namespace {

using sawkv::host::aligned;
using sawkv::host::alternate_tensors;
using sawkv::host::check_geometry;
using sawkv::host::check_output;
using sawkv::host::check_tensor;
using sawkv::host::fail;
using sawkv::host::g_err;
using sawkv::host::hb_index;
using sawkv::host::ok;

// Instantiated pairs (tensor 0, tensor 1): both naive, rotated + naive (keys
// only, or a single rotated tensor), both rotated with the same h.
#define SAWKV_TABLE(K)                                                              \
  {{(void*)&K<0, 0>, nullptr, nullptr, nullptr, nullptr},                           \
   {(void*)&K<16, 0>, (void*)&K<16, 16>, nullptr, nullptr, nullptr},                \
   {(void*)&K<32, 0>, nullptr, (void*)&K<32, 32>, nullptr, nullptr},                \
   {(void*)&K<64, 0>, nullptr, nullptr, (void*)&K<64, 64>, nullptr},                \
   {(void*)&K<128, 0>, nullptr, nullptr, nullptr, (void*)&K<128, 128>}}

const void* const kAppend[5][5] = SAWKV_TABLE(sawkv::append_kernel);
const void* const kAppendLayers[5][5] = SAWKV_TABLE(sawkv::append_layers_kernel);
const void* const kGather[5][5] = SAWKV_TABLE(sawkv::gather_kernel);

#undef SAWKV_TABLE

// One block = 4 waves = 64 vectors of one tensor.
unsigned append_blocks(int32_t TH) {
  return (unsigned)((TH + sawkv::kVecPerBlock - 1) / sawkv::kVecPerBlock);
}

// One gather block = 4 waves x 16 vectors = 64 vectors of one tensor.
unsigned gather_blocks(int32_t TH) {
  return (unsigned)((TH + sawkv::kVecPerBlock - 1) / sawkv::kVecPerBlock);
}

int launch(const void* fn, int grid_y, unsigned blocks, void* params, void* stream,
           int grid_z = 1) {
  if (fn == nullptr) return fail(SAWKV_EINVAL, "no kernel for this tensor/rotation combination");
  const dim3 grid(blocks, (unsigned)grid_y, (unsigned)grid_z);
  void* args[] = {params};
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(sawkv::kThreads), args, 0,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SAWKV_EHIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int append_impl(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                const int64_t* slots, int64_t T, int32_t H, int32_t D, void* k_codes,
                void* v_codes, void* k_scales, void* v_scales, int64_t N_pg, int32_t P,
                int32_t h, int32_t rot_mode, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, h, rot_mode, slots);
  if (st) return st;
  if (T == 0) return ok();              // nothing is read or written
  if (k == nullptr && v == nullptr) return fail(SAWKV_EINVAL, "both k and v are NULL");
  if (k && (st = check_tensor("k", k, k_stride, k_codes, k_scales, H, D))) return st;
  if (v && (st = check_tensor("v", v, v_stride, v_codes, v_scales, H, D))) return st;

  sawkv::AppendParams p{};
  int n = 0, hb[2] = {0, 0};
  if (k) {
    p.t[n] = {static_cast<const __half*>(k), k_stride, static_cast<uint8_t*>(k_codes),
              static_cast<__half*>(k_scales)};
    hb[n++] = hb_index(h, rot_mode != SAWKV_ROT_NONE);
  }
  if (v) {
    p.t[n] = {static_cast<const __half*>(v), v_stride, static_cast<uint8_t*>(v_codes),
              static_cast<__half*>(v_scales)};
    hb[n++] = hb_index(h, rot_mode == SAWKV_ROT_KV);
  }
  p.slots = slots;
  p.n_slots = N_pg * P;
  p.T = (int32_t)T;
  p.TH = (int32_t)(T * H);
  p.H = H;
  p.h_magic = (uint32_t)(((1u << 20) + (uint32_t)H - 1u) / (uint32_t)H);
  if (n == 2 && alternate_tensors(T, H, D))
    return launch(kAppend[hb[0]][hb[1]], 1, 2 * append_blocks(p.TH), &p, stream);
  return launch(kAppend[hb[0]][hb[1]], n, append_blocks(p.TH), &p, stream);
}

int append_layers_impl(const sawkv_layer_t* layers, int32_t n_layers, int64_t k_stride,
                       int64_t v_stride, const int64_t* slots, int64_t T, int32_t H, int32_t D,
                       int64_t N_pg, int32_t P, int32_t h, int32_t rot_mode, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, h, rot_mode, slots);
  if (st) return st;
  if (layers == nullptr) return fail(SAWKV_EINVAL, "layers is NULL");
  if (n_layers < 1 || n_layers > sawkv::kMaxLayers)
    return fail(SAWKV_EINVAL, "n_layers = %d outside [1, %d]", n_layers, sawkv::kMaxLayers);
  if (T == 0) return ok();
  const bool has_k = layers[0].k != nullptr, has_v = layers[0].v != nullptr;
  if (!has_k && !has_v) return fail(SAWKV_EINVAL, "layer 0 has neither k nor v");
  sawkv::LayersParams p{};
  for (int32_t l = 0; l < n_layers; ++l) {
    const sawkv_layer_t& L = layers[l];
    if ((L.k != nullptr) != has_k || (L.v != nullptr) != has_v)
      return fail(SAWKV_EINVAL, "layer %d: k/v presence differs from layer 0", l);
    for (int t = 0; t < 2; ++t) {
      const bool present = t == 0 ? has_k : has_v;
      if (!present) continue;
      st = t == 0 ? check_tensor("k", L.k, k_stride, L.k_codes, L.k_scales, H, D)
                  : check_tensor("v", L.v, v_stride, L.v_codes, L.v_scales, H, D);
      if (st) {
        char detail[sizeof g_err];
        snprintf(detail, sizeof detail, "%s", g_err);
        return fail(st, "layer %d: %s", l, detail);
      }
    }
    p.layer[l] = {static_cast<const __half*>(L.k), static_cast<const __half*>(L.v),
                  static_cast<uint8_t*>(L.k_codes), static_cast<uint8_t*>(L.v_codes),
                  static_cast<__half*>(L.k_scales), static_cast<__half*>(L.v_scales)};
  }
  int n = 0, hb[2] = {0, 0};
  if (has_k) hb[n++] = hb_index(h, rot_mode != SAWKV_ROT_NONE);
  if (has_v) hb[n++] = hb_index(h, rot_mode == SAWKV_ROT_KV);
  p.n_tensors = n;
  p.n_layers = n_layers;
  p.only_v = (!has_k && has_v) ? 1 : 0;
  p.k_stride = k_stride;
  p.v_stride = v_stride;
  p.common.slots = slots;
  p.common.n_slots = N_pg * P;
  p.common.T = (int32_t)T;
  p.common.TH = (int32_t)(T * H);
  p.common.H = H;
  p.common.h_magic = (uint32_t)(((1u << 20) + (uint32_t)H - 1u) / (uint32_t)H);
  // grid (blocks, layers, tensors per layer)
  return launch(kAppendLayers[hb[0]][hb[1]], n_layers, append_blocks(p.common.TH), &p, stream,
                n);
}

int gather_impl(const void* k_codes, const void* v_codes, const void* k_scales,
                const void* v_scales, int64_t N_pg, int32_t P, const int64_t* slots,
                int64_t T, int32_t H, int32_t D, void* k_out, void* v_out, int32_t h,
                int32_t rot_mode, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, h, rot_mode, slots);
  if (st) return st;
  if (T == 0) return ok();
  if (k_out == nullptr && v_out == nullptr) return fail(SAWKV_EINVAL, "both outputs are NULL");
  if (k_out && (st = check_output("k", k_out, k_codes, k_scales))) return st;
  if (v_out && (st = check_output("v", v_out, v_codes, v_scales))) return st;

  sawkv::GatherParams p{};
  int n = 0, hb[2] = {0, 0};
  if (k_out) {
    p.t[n] = {static_cast<const uint8_t*>(k_codes), static_cast<const __half*>(k_scales),
              static_cast<__half*>(k_out)};
    hb[n++] = hb_index(h, rot_mode != SAWKV_ROT_NONE);
  }
  if (v_out) {
    p.t[n] = {static_cast<const uint8_t*>(v_codes), static_cast<const __half*>(v_scales),
              static_cast<__half*>(v_out)};
    hb[n++] = hb_index(h, rot_mode == SAWKV_ROT_KV);
  }
  p.slots = slots;
  p.n_slots = N_pg * P;
  p.T = (int32_t)T;
  p.TH = (int32_t)(T * H);
  p.H = H;
  p.h_magic = (uint32_t)(((1u << 20) + (uint32_t)H - 1u) / (uint32_t)H);
  return launch(kGather[hb[0]][hb[1]], n, gather_blocks(p.TH), &p, stream);
}

}  // namespace

extern "C" {

int sawkv_quantize_append(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                          const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                          void* k_codes, void* v_codes, void* k_scales, void* v_scales,
                          int64_t N_pg, int32_t P, int32_t h, int32_t rot_mode,
                          void* stream) {
  return append_impl(k, v, k_stride, v_stride, slot_mapping, T, H, D, k_codes, v_codes,
                     k_scales, v_scales, N_pg, P, h, rot_mode, stream);
}

int sawkv_quantize_append_layers(const sawkv_layer_t* layers, int32_t n_layers,
                                 int64_t k_stride, int64_t v_stride,
                                 const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                                 int64_t N_pg, int32_t P, int32_t h, int32_t rot_mode,
                                 void* stream) {
  return append_layers_impl(layers, n_layers, k_stride, v_stride, slot_mapping, T, H, D, N_pg,
                            P, h, rot_mode, stream);
}

int sawkv_dequant_gather(const void* k_codes, const void* v_codes, const void* k_scales,
                         const void* v_scales, int64_t N_pg, int32_t P,
                         const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                         void* k_out, void* v_out, int32_t h, int32_t rot_mode,
                         void* stream) {
  return gather_impl(k_codes, v_codes, k_scales, v_scales, N_pg, P, slot_mapping, T, H, D,
                     k_out, v_out, h, rot_mode, stream);
}

int sawkv_naive_int4_append(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                            const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                            void* k_codes, void* v_codes, void* k_scales, void* v_scales,
                            int64_t N_pg, int32_t P, void* stream) {
  return append_impl(k, v, k_stride, v_stride, slot_mapping, T, H, D, k_codes, v_codes,
                     k_scales, v_scales, N_pg, P, 128, SAWKV_ROT_NONE, stream);
}

int sawkv_naive_int4_gather(const void* k_codes, const void* v_codes, const void* k_scales,
                            const void* v_scales, int64_t N_pg, int32_t P,
                            const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                            void* k_out, void* v_out, void* stream) {
  return gather_impl(k_codes, v_codes, k_scales, v_scales, N_pg, P, slot_mapping, T, H, D,
                     k_out, v_out, 128, SAWKV_ROT_NONE, stream);
}

const char* sawkv_status_string(int status) {
  switch (status) {
    case SAWKV_OK: return "ok";
    case SAWKV_EINVAL: return "invalid argument";
    case SAWKV_EUNSUPPORTED: return "unsupported size";
    case SAWKV_EALIGN: return "misaligned pointer or stride";
    case SAWKV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sawkv_last_error(void) { return g_err; }

int sawkv_version(void) { return SAWKV_VERSION; }

}  // extern "C"
