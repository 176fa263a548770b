// sawkv controls (gfx950): the uncompressed paged cache write and token-wise
// INT8, the baselines the INT4 cache is compared against, and an
// access-pattern control of the INT4 append (its loads and stores with no
// arithmetic of the method) that measures the bandwidth the append's pattern
// can reach at all (gist.science
// summary of SAW-INT4, §4 Risultati Sperimentali: accuracy and system
// throughput against a BF16 cache; ainews.cool, the comparison table under
// "技术深度解析": a uniform INT8 cache).
//
// INT8 follows the INT4 write path step for step (same fetch, same optional
// block-diagonal rotation, one fp16 scale per vector) with 256 levels:
//     s = f16(f32(amax / 127)),  q = clamp(rint(f32(y / s)), -128, 127),
// one signed byte per channel, codes [N_pg*P][H][D]. Its read-back transforms
// the integer codes (exact in float32: |partial sums| <= 2^14), then
// multiplies by s and by c_h, each rounded to float32, then rounds to fp16.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <stdint.h>

#include "sawkv.h"
#include "sawkv_append.hpp"
#include "sawkv_device.hpp"
#include "sawkv_host.hpp"

namespace sawkv {
namespace controls {

constexpr int kRow8 = kD;   // bytes of one INT8 code row

// Quantise the wave's 16 fetched vectors to INT8 and store them.
template <int HB>
__device__ __forceinline__ void quantize_store8(const AppendTensor& A, const AppendParams& p,
                                                const Fetched& f, int lam) {
  float y[kElems];
  load_transform<HB>(f.raw, y, lam);

  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kElems; ++k) m = fmaxf(m, fabsf(y[k]));
  m = fmaxf(m, quad_xor1(m));
  m = fmaxf(m, quad_xor2(m));
  // s32 = RN(amax / 127): Markstein's correction with r127 = RN(1/127)
  const float r127 = __builtin_bit_cast(float, 0x3C010204u);
  const float q127 = m * r127;
  const float s32 = __builtin_fmaf(__builtin_fmaf(-q127, 127.0f, m), r127, q127);
  const __half s16 = __float2half_rn(fminf(s32, 65504.0f));
  const float sf = __half2float(s16);
  // r = RN(1/sf) (hardware reciprocal + one exact Newton step, as for INT4)
  const float r0 = __builtin_amdgcn_rcpf(sf);
  const float r = sf > 0.0f ? __builtin_fmaf(r0, __builtin_fmaf(-sf, r0, 1.0f), r0) : 0.0f;
  // an fp16-subnormal scale can put a quotient past 127 (an fp16 K/V vector
  // cannot saturate an INT8 scale, but the test is kept for symmetry)
  const bool need_clamp = (s32 > 65504.0f) || (sf < 6.103515625e-05f);

  // q = rint(f32(y / s)) via Markstein's correction of y * r; adding
  // 1.5 * 2^23 + 128 rounds half-to-even and leaves q + 128 in the low byte
  uint32_t u[kElems];
#pragma unroll
  for (int k = 0; k < kElems; ++k) {
    const float q0 = y[k] * r;
    const float e = __builtin_fmaf(-q0, sf, y[k]);
    const float q1 = __builtin_fmaf(e, r, q0);
    u[k] = __builtin_bit_cast(uint32_t, q1 + 12583040.0f);
  }
  if (__any(need_clamp)) {
#pragma unroll
    for (int k = 0; k < kElems; ++k) u[k] = min(max(u[k], 0x4B400000u), 0x4B4000FFu);
  }
  // bytes q + 128 -> two's complement by xor 0x80; 4 codes per dword
  uint32_t d[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t lo = __builtin_amdgcn_perm(u[4 * w + 1], u[4 * w], 0x0C0C0400u);
    const uint32_t hi = __builtin_amdgcn_perm(u[4 * w + 3], u[4 * w + 2], 0x0C0C0400u);
    d[w] = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x80808080u;
  }

  if (f.in_range && f.slot >= 0 && f.slot < p.n_slots) {
    const int64_t row = f.slot * p.H + f.head;
    uint8_t* dst = A.codes + row * kRow8 + 8 * lam;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint2*>(dst + 32 * i) = make_uint2(d[2 * i], d[2 * i + 1]);
    if (lam == 0) A.scales[row] = s16;
  }
}

template <int HB>
__device__ __forceinline__ void append8_tensor(const AppendTensor& A, const AppendParams& p) {
  const int lane = threadIdx.x & 63;
  const int lam = lane & 3;
  const int vq = lane >> 2;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WavePos w;
  w.v0 = (blockIdx.x * kWaves + wave) * kVecPerWave;
  if (w.v0 >= (uint32_t)p.TH) return;
  w.t0 = w.v0 / (uint32_t)p.H;
  w.h0 = w.v0 - w.t0 * (uint32_t)p.H;
  quantize_store8<HB>(A, p, fetch_batch(A, p, w, lam, vq), lam);
}

template <int HB0, int HB1>
__global__ __launch_bounds__(kThreads) void append8_kernel(AppendParams p) {
  if (blockIdx.y == 0) append8_tensor<HB0>(p.t[0], p);
  else append8_tensor<HB1>(p.t[1], p);
}

// ---- INT8 read-back ----

struct Gather8Tensor {
  const int8_t* codes;     // [n_slots][H][D]
  const __half* scales;    // [n_slots][H]
  __half* out;             // [T][H][D]
};

struct Gather8Params {
  Gather8Tensor t[2];
  const int64_t* slots;
  int64_t n_slots;
  int32_t TH;
  int32_t H;
};

// One quad per (token, head) vector: lane lam holds channels 32i + 8 lam + j.
template <int HB>
__device__ __forceinline__ void gather8_tensor(const Gather8Tensor& G, const Gather8Params& p) {
  const int lane = threadIdx.x & 63;
  const int lam = lane & 3;
  // TH < 2^31: the vector index splits with a 32-bit division
  const uint32_t v = blockIdx.x * (uint32_t)kVecPerBlock + (threadIdx.x >> 2);
  const bool live = v < (uint32_t)p.TH;
  const uint32_t t = live ? v / (uint32_t)p.H : 0u;
  const int head = live ? (int)(v - t * (uint32_t)p.H) : 0;
  const int64_t slot = live ? p.slots[t] : -1;
  const bool valid = slot >= 0 && slot < p.n_slots;

  float x[kElems];
  float sf = 0.0f;
  if (valid) {
    const int64_t row = slot * p.H + head;
    const int8_t* src = G.codes + row * kRow8 + 8 * lam;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint2 c = *reinterpret_cast<const uint2*>(src + 32 * i);
      const uint32_t w[2] = {c.x, c.y};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[8 * i + j] = (float)(int8_t)(w[j >> 2] >> (8 * (j & 3)));
    }
    sf = __half2float(G.scales[row]);
  } else {
#pragma unroll
    for (int k = 0; k < kElems; ++k) x[k] = 0.0f;
  }
  float o[kElems];
  if constexpr (HB > 0) {
    // integer transform, exact; the lane's sign is folded into c_h * sign
    lane_stage<0>(x);
    const float csg = fwht_rest<HB>(x, lam) * c_h<HB>();
#pragma unroll
    for (int k = 0; k < kElems; ++k) {
      const float tv = opaque(x[k] * sf);            // f32(F(q) * s)
      o[k] = __builtin_fmaf(tv, csg, 0.0f);        // f32(t * c_h); -0 becomes +0
    }
  } else {
#pragma unroll
    for (int k = 0; k < kElems; ++k) o[k] = x[k] * sf;   // exact
  }
  // stage the wave's 16 output rows (4 KB, consecutive vectors) through LDS,
  // then store them as four contiguous 1 KB wave stores; rows padded to 272
  // bytes
  __shared__ uint4 stage[kWaves][kVecPerWave][17];
  const int wv = threadIdx.x >> 6, vq = (threadIdx.x & 63) >> 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint16_t lo = __builtin_bit_cast(uint16_t, __float2half_rn(opaque(o[8 * i + 2 * k])));
      const uint16_t hi =
          __builtin_bit_cast(uint16_t, __float2half_rn(opaque(o[8 * i + 2 * k + 1])));
      wd[k] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    stage[wv][vq][4 * i + lam] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  __builtin_amdgcn_wave_barrier();
  const int ln = threadIdx.x & 63;
  const uint32_t v_first = blockIdx.x * (uint32_t)kVecPerBlock + (uint32_t)wv * kVecPerWave;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (ln >> 4), c = ln & 15;
    const uint4 w = stage[wv][r][c];
    if (v_first + (uint32_t)r < (uint32_t)p.TH)
      store_stream(w, G.out + ((int64_t)v_first + r) * kD + 8 * c);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int HB0, int HB1>
__global__ __launch_bounds__(kThreads) void gather8_kernel(Gather8Params p) {
  if (blockIdx.y == 0) gather8_tensor<HB0>(p.t[0], p);
  else gather8_tensor<HB1>(p.t[1], p);
}

// ---- uncompressed paged cache write ----

struct CacheTensor {
  const uint4* src;        // [T][H][D] 16-bit values, token stride `stride16` x 16 B
  int64_t stride16;
  uint4* cache;            // [n_slots][H][D]
};

struct CacheParams {
  CacheTensor t[2];
  const int64_t* slots;
  int64_t n_slots;
  int64_t n_pieces;        // T * H * 16 (16-byte pieces of a 256-byte row)
  int32_t H;
};

__global__ __launch_bounds__(kThreads) void cache_append_kernel(CacheParams p) {
  const CacheTensor& C = p.t[blockIdx.y];
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= p.n_pieces) return;
  const int64_t vec = i >> 4;
  const int piece = (int)(i & 15);
  int64_t t;
  int head;
  if (p.n_pieces <= INT64_C(16) * UINT32_MAX) {
    // 32-bit division whenever the vector index fits (a 64-bit one is a long
    // emulated sequence ahead of the slot load)
    const uint32_t tv = (uint32_t)vec / (uint32_t)p.H;
    t = tv;
    head = (int)((uint32_t)vec - tv * (uint32_t)p.H);
  } else {
    t = vec / p.H;
    head = (int)(vec - t * p.H);
  }
  const int64_t slot = p.slots[t];
  if (slot < 0 || slot >= p.n_slots) return;
  C.cache[(slot * p.H + head) * 16 + piece] = C.src[t * C.stride16 + head * 16 + piece];
}

// ---- access-pattern control of the INT4 append ----
//
// The INT4 append's grid, loads and stores with none of the method's
// arithmetic: each wave fetches its 16 vectors exactly as the append does
// (fetch_batch: the same 16-byte loads of the fp16 rows and the same slot
// load), folds each 16-byte input piece into one 32-bit word by xor, and
// stores the 64-byte row and the 2-byte scale where the append would store
// the codes and the scale. With kTokenOrder the rows go to row t*H + head
// (token order) instead of the mapped slot, which shows what the same loads
// reach when the destination pages are contiguous.
template <bool kTokenOrder>
__device__ __forceinline__ void pattern_tensor(const AppendTensor& A, const AppendParams& p,
                                               uint32_t bx) {
  const int lane = threadIdx.x & 63;
  const int lam = lane & 3;
  const int vq = lane >> 2;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WavePos w;
  w.v0 = (bx * kWaves + wave) * kVecPerWave;
  if (w.v0 >= (uint32_t)p.TH) return;
  w.t0 = w.v0 / (uint32_t)p.H;
  w.h0 = w.v0 - w.t0 * (uint32_t)p.H;
  const Fetched f = fetch_batch(A, p, w, lam, vq);
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = f.raw[i].x ^ f.raw[i].y ^ f.raw[i].z ^ f.raw[i].w;
  const uint16_t sbits = (uint16_t)(d[0] ^ (d[0] >> 16));
  int64_t row;
  if constexpr (kTokenOrder) {
    row = (int64_t)w.v0 + vq;                  // t * H + head
    if (!f.in_range) return;
  } else {
    if (!(f.in_range && f.slot >= 0 && f.slot < p.n_slots)) return;
    row = f.slot * p.H + f.head;
  }
  uint8_t* dst = A.codes + row * (kD / 2) + 4 * lam;
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t*>(dst + 16 * i) = d[i];
  if (lam == 0) A.scales[row] = __builtin_bit_cast(__half, sbits);
}

// The same grid forms as the append (tensors' blocks alternating in
// dispatch order when the append alternates them).
template <bool kTokenOrder>
__global__ __launch_bounds__(kThreads) void pattern_kernel(AppendParams p) {
  if (gridDim.y == 1 && p.t[1].src != nullptr) {
    if ((blockIdx.x & 1u) == 0) pattern_tensor<kTokenOrder>(p.t[0], p, blockIdx.x >> 1);
    else pattern_tensor<kTokenOrder>(p.t[1], p, blockIdx.x >> 1);
  } else if (blockIdx.y == 0) {
    pattern_tensor<kTokenOrder>(p.t[0], p, blockIdx.x);
  } else {
    pattern_tensor<kTokenOrder>(p.t[1], p, blockIdx.x);
  }
}

}  // namespace controls
}  // namespace sawkv

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

using sawkv::host::aligned;
using sawkv::host::check_geometry;
using sawkv::host::check_output;
using sawkv::host::check_tensor;
using sawkv::host::fail;
using sawkv::host::hb_index;
using sawkv::host::ok;
using sawkv::controls::append8_kernel;
using sawkv::controls::gather8_kernel;

#define SAWKV_TABLE8(K)                                                             \
  {{(void*)&K<0, 0>, nullptr, nullptr, nullptr, nullptr},                           \
   {(void*)&K<16, 0>, (void*)&K<16, 16>, nullptr, nullptr, nullptr},                \
   {(void*)&K<32, 0>, nullptr, (void*)&K<32, 32>, nullptr, nullptr},                \
   {(void*)&K<64, 0>, nullptr, nullptr, (void*)&K<64, 64>, nullptr},                \
   {(void*)&K<128, 0>, nullptr, nullptr, nullptr, (void*)&K<128, 128>}}

const void* const kAppend8[5][5] = SAWKV_TABLE8(append8_kernel);
const void* const kGather8[5][5] = SAWKV_TABLE8(gather8_kernel);

#undef SAWKV_TABLE8

int launch(const void* fn, int grid_y, int64_t blocks, void* params, void* stream) {
  if (fn == nullptr) return fail(SAWKV_EINVAL, "no kernel for this tensor/rotation combination");
  void* args[] = {params};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks, (unsigned)grid_y),
                                       dim3(sawkv::kThreads), args, 0,
                                       reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SAWKV_EHIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int int8_append_impl(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                     const int64_t* slots, int64_t T, int32_t H, int32_t D, void* k_codes,
                     void* v_codes, void* k_scales, void* v_scales, int64_t N_pg, int32_t P,
                     int32_t h, int32_t rot_mode, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, h, rot_mode, slots);
  if (st) return st;
  if (T == 0) return ok();
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
  return launch(kAppend8[hb[0]][hb[1]], n, (p.TH + sawkv::kVecPerBlock - 1) / sawkv::kVecPerBlock,
                &p, stream);
}

int int8_gather_impl(const void* k_codes, const void* v_codes, const void* k_scales,
                     const void* v_scales, int64_t N_pg, int32_t P, const int64_t* slots,
                     int64_t T, int32_t H, int32_t D, void* k_out, void* v_out, int32_t h,
                     int32_t rot_mode, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, h, rot_mode, slots);
  if (st) return st;
  if (T == 0) return ok();
  if (k_out == nullptr && v_out == nullptr) return fail(SAWKV_EINVAL, "both outputs are NULL");
  if (k_out && (st = check_output("k", k_out, k_codes, k_scales))) return st;
  if (v_out && (st = check_output("v", v_out, v_codes, v_scales))) return st;
  sawkv::controls::Gather8Params p{};
  int n = 0, hb[2] = {0, 0};
  if (k_out) {
    p.t[n] = {static_cast<const int8_t*>(k_codes), static_cast<const __half*>(k_scales),
              static_cast<__half*>(k_out)};
    hb[n++] = hb_index(h, rot_mode != SAWKV_ROT_NONE);
  }
  if (v_out) {
    p.t[n] = {static_cast<const int8_t*>(v_codes), static_cast<const __half*>(v_scales),
              static_cast<__half*>(v_out)};
    hb[n++] = hb_index(h, rot_mode == SAWKV_ROT_KV);
  }
  p.slots = slots;
  p.n_slots = N_pg * P;
  p.TH = (int32_t)(T * H);
  p.H = H;
  return launch(kGather8[hb[0]][hb[1]], n, (p.TH + sawkv::kVecPerBlock - 1) / sawkv::kVecPerBlock,
                &p, stream);
}

int cache_append_impl(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                      const int64_t* slots, int64_t T, int32_t H, int32_t D, void* k_cache,
                      void* v_cache, int64_t N_pg, int32_t P, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, 128, SAWKV_ROT_NONE, slots);
  if (st) return st;
  if (T == 0) return ok();
  if (k == nullptr && v == nullptr) return fail(SAWKV_EINVAL, "both k and v are NULL");
  // the cache doubles as "codes" and "scales" for the shared pointer checks
  if (k && (st = check_tensor("k", k, k_stride, k_cache, k_cache, H, D))) return st;
  if (v && (st = check_tensor("v", v, v_stride, v_cache, v_cache, H, D))) return st;
  sawkv::controls::CacheParams p{};
  int n = 0;
  if (k) p.t[n++] = {static_cast<const uint4*>(k), k_stride / 8, static_cast<uint4*>(k_cache)};
  if (v) p.t[n++] = {static_cast<const uint4*>(v), v_stride / 8, static_cast<uint4*>(v_cache)};
  p.slots = slots;
  p.n_slots = N_pg * P;
  p.n_pieces = T * H * 16;
  p.H = H;
  return launch((const void*)&sawkv::controls::cache_append_kernel, n,
                (p.n_pieces + sawkv::kThreads - 1) / sawkv::kThreads, &p, stream);
}

int pattern_impl(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                 const int64_t* slots, int64_t T, int32_t H, int32_t D, void* k_codes,
                 void* v_codes, void* k_scales, void* v_scales, int64_t N_pg, int32_t P,
                 int32_t placement, void* stream) {
  int st = check_geometry(T, H, D, N_pg, P, 128, SAWKV_ROT_NONE, slots);
  if (st) return st;
  if (placement != SAWKV_PLACE_SLOTS && placement != SAWKV_PLACE_TOKEN_ORDER)
    return fail(SAWKV_EINVAL, "placement = %d invalid", placement);
  if (placement == SAWKV_PLACE_TOKEN_ORDER && T > N_pg * P)
    return fail(SAWKV_EINVAL, "token order needs T = %lld <= N_pg*P = %lld slots", (long long)T,
                (long long)(N_pg * P));
  if (T == 0) return ok();
  if (k == nullptr && v == nullptr) return fail(SAWKV_EINVAL, "both k and v are NULL");
  if (k && (st = check_tensor("k", k, k_stride, k_codes, k_scales, H, D))) return st;
  if (v && (st = check_tensor("v", v, v_stride, v_codes, v_scales, H, D))) return st;
  sawkv::AppendParams p{};
  int n = 0;
  if (k)
    p.t[n++] = {static_cast<const __half*>(k), k_stride, static_cast<uint8_t*>(k_codes),
                static_cast<__half*>(k_scales)};
  if (v)
    p.t[n++] = {static_cast<const __half*>(v), v_stride, static_cast<uint8_t*>(v_codes),
                static_cast<__half*>(v_scales)};
  p.slots = slots;
  p.n_slots = N_pg * P;
  p.T = (int32_t)T;
  p.TH = (int32_t)(T * H);
  p.H = H;
  p.h_magic = (uint32_t)(((1u << 20) + (uint32_t)H - 1u) / (uint32_t)H);
  const void* fn = placement == SAWKV_PLACE_SLOTS
                       ? (const void*)&sawkv::controls::pattern_kernel<false>
                       : (const void*)&sawkv::controls::pattern_kernel<true>;
  const int64_t blocks = (p.TH + sawkv::kVecPerBlock - 1) / sawkv::kVecPerBlock;
  if (n == 2 && sawkv::host::alternate_tensors(T, H, D)) return launch(fn, 1, 2 * blocks, &p, stream);
  return launch(fn, n, blocks, &p, stream);
}

}  // namespace

extern "C" {

int sawkv_append_pattern_control(const void* k, const void* v, int64_t k_stride,
                                 int64_t v_stride, const int64_t* slot_mapping, int64_t T,
                                 int32_t H, int32_t D, void* k_codes, void* v_codes,
                                 void* k_scales, void* v_scales, int64_t N_pg, int32_t P,
                                 int32_t placement, void* stream) {
  return pattern_impl(k, v, k_stride, v_stride, slot_mapping, T, H, D, k_codes, v_codes,
                      k_scales, v_scales, N_pg, P, placement, stream);
}

int sawkv_cache_append(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                       const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                       void* k_cache, void* v_cache, int64_t N_pg, int32_t P, void* stream) {
  return cache_append_impl(k, v, k_stride, v_stride, slot_mapping, T, H, D, k_cache, v_cache,
                           N_pg, P, stream);
}

int sawkv_int8_append(const void* k, const void* v, int64_t k_stride, int64_t v_stride,
                      const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                      void* k_codes, void* v_codes, void* k_scales, void* v_scales,
                      int64_t N_pg, int32_t P, int32_t h, int32_t rot_mode, void* stream) {
  return int8_append_impl(k, v, k_stride, v_stride, slot_mapping, T, H, D, k_codes, v_codes,
                          k_scales, v_scales, N_pg, P, h, rot_mode, stream);
}

int sawkv_int8_gather(const void* k_codes, const void* v_codes, const void* k_scales,
                      const void* v_scales, int64_t N_pg, int32_t P,
                      const int64_t* slot_mapping, int64_t T, int32_t H, int32_t D,
                      void* k_out, void* v_out, int32_t h, int32_t rot_mode, void* stream) {
  return int8_gather_impl(k_codes, v_codes, k_scales, v_scales, N_pg, P, slot_mapping, T, H, D,
                          k_out, v_out, h, rot_mode, stream);
}

}  // extern "C"
