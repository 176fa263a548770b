// sawkv decode attention over the paged INT4 pools (gfx950, wave64).
//
// One decode step: every sequence b has one query token with Hq heads; query
// head j reads KV head j / G (G = Hq / H). Keys and values are the INT4 rows
// written by sawkv_quantize_append. The pages place dequantisation inside the
// attention kernel (ainews.cool, "技术深度解析" item 3) and ask that the paged
// layout and fused attention execution be kept (youngju.dev English page, "Why
// the KV Cache Is the Real Bottleneck"); the rotation is orthogonal
// (youngju.dev, "The Rotation Trick - Block-Diagonal Hadamard"), so for a
// rotated key R^T y:  q . (R^T y) = (R q) . y.  The query is rotated once, and
// no key is ever un-rotated; the value side is un-rotated once per output.
//
// Two launches on the caller's stream, sharing a caller-provided workspace:
//
//  chunk    one wave per (sequence, chunk of C tokens, pair of KV heads) when
//           H is even (a wave then reads whole 128-byte lines: both heads'
//           64-byte rows of a token), else per (sequence, chunk, KV head). The wave first
//           prepares its queries: q' = R q (if keys are rotated), scaled by
//           sm_scale * log2(e) and by a power of two 2^sigma that puts
//           max |q'| in [2^13, 2^14), each value split into fp16 hi + lo and
//           laid out as the B operand of the score MFMAs. Then scores on the
//           matrix cores straight from the packed nibbles, an online softmax,
//           and P.V on the matrix cores; it writes the chunk's partial
//           (reference exponent, denominator, unnormalised output).
//  combine  16 lanes per (sequence, query head): merge the chunks (four
//           quads, each over every fourth chunk), divide, un-rotate V (if
//           rotated), round to fp16.
//
// Nibbles on the matrix cores. A code byte holds two two's-complement
// nibbles; xor 0x88 turns them into u = code + 8 in [0, 15]. Masking one
// nibble into the low 10 bits of an fp16 lane gives the subnormal u * 2^-24
// (bits 0-3) or 16u * 2^-24 (bits 4-7): exact values, no conversion
// instruction. The MFMA multiplies subnormal fp16 inputs exactly. The factor
// 16 on odd channels is folded into the other operand (1/16 on the query side,
// a final 1/16 on the value side), and the +8 bias is removed by a per-query
// constant: sum q' (u - 8) = sum q' u - 8 sum q'.
//
// Scores (16x16x32 f16 MFMA, 16 tokens x 16 columns x 32 channels): A =
// codes (row m = token, one code dword per lane per MFMA), B = query
// (column n < G: hi part of query n; G <= n < 2G: lo part; rest 0), so one
// MFMA yields hi and lo dot products in two columns, added with one DPP
// row shift. Lane (g = lane/16, n = lane%16) of the result holds tokens
// 4g + j, j = 0..3, of column n.
//
// Values (16x16x32 MFMA, 16 rows x 16 columns x 32 tokens): A = weights
// p * s_v (row n < G: hi part for query n; G <= n < 2G: lo part), taken
// lane-locally from the score layout (k slot (g, i) is token 16(i/4) + 4g +
// i%4 of the 32-token step); B = value nibbles: lane n loads code dword n
// (channels 8n..8n+7) of its 8 tokens, and MFMA j uses nibble j, so column n
// of MFMA j is channel 8n + j. Hi and lo rows are added once at the end.
//
// Softmax. Scores are kept in log2 units. The reference m tracks the largest
// 4 * score + (bits of s_v >> 8), a cheap upper bound of 4 * log2(p * s_v)
// + 60, so that every weight p * s_v stays below 2^14 in fp16; the reference
// moves only when a new maximum exceeds it by 8 (in log2 units), so the
// rescale of the accumulators is rare.

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <stdio.h>

#include "sawkv.h"
#include "sawkv_device.hpp"
#include "sawkv_host.hpp"

namespace sawkv {
namespace attn {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kStep = 32;              // tokens per loop step (two 16-token tiles)
constexpr int kQWords = 16;            // B-operand dwords per lane (4 MFMAs x 4)

__device__ __forceinline__ f4_t mfma(u4_t a, u4_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}

// Value of lane + S within the lane's row of 16 (0 past the row's end).
template <int S>
__device__ __forceinline__ float row_shl(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                       0, __builtin_bit_cast(int, v), 0x100 + S, 0xF, 0xF, true));
}

// Lanes G..2G-1 of every row take `src` from lane - G; the others keep `old`.
template <int G>
__device__ __forceinline__ uint32_t lo_rows(uint32_t old, uint32_t src) {
  constexpr int bank = G == 8 ? 0xC : G == 4 ? 0x2 : 0x1;
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x110 + G, 0xF, bank, false);
}

// Row exchange on two copies of a value (rows = groups of 16 lanes):
//   v_permlane16_swap a, b: a = [a0, b0, a2, b2], b = [a1, b1, a3, b3]
//   v_permlane32_swap a, b: a = [a0, a1, b0, b1], b = [a2, a3, b2, b3]
// With a = b = v, a op b combines rows (0,1)/(2,3) resp. (0,2)/(1,3). Written
// as inline asm: the compiler folds the builtins' two results into one when
// both inputs are the same value. The s_nop covers the VALU-write ->
// permlane-read hazard (2 wait states), as for DPP.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// max(a, b) as one v_max_f32, without the quieting of signalling NaNs that
// fmaxf adds for operands the compiler cannot prove canonical (select and
// lane-exchange results). Operands here are finite or -inf.
__device__ __forceinline__ float max_raw(float a, float b) {
  float d;
  asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Sum (or max) over the four rows of 16 lanes; every row gets the result.
__device__ __forceinline__ float rows_sum(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = a + b, d = a + b;
  swap32(c, d);
  return c + d;
}

__device__ __forceinline__ float rows_max(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = max_raw(a, b), d = c;
  swap32(c, d);
  return max_raw(c, d);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------------------
// prep: q -> B operand of the score MFMAs
// ---------------------------------------------------------------------------

struct QueryParams {
  const __half* q;
  int64_t q_stride;        // elements between the rows of two sequences
  int32_t h;
  int32_t rot_k;
  float c_h;               // f32(1/sqrt(h))
  float c_sm;              // sm_scale * log2(e)
};

// Column n of the score MFMAs' B operand holds (query of the block, part):
//   single head (PAIR false): n < G hi of query n, G <= n < 2G lo of query n - G
//   head pair (PAIR true, G = 4): query 4 (n / 8) + n % 4, lo when n & 4
//   head pair (PAIR true, G = 8): query n; the hi parts form one operand and
//                                 the lo parts a second one (split_operand)
// where the block's queries are those of its heads in order.
template <int G, bool PAIR>
constexpr bool split_operand() { return PAIR && G == 8; }
template <int G, bool PAIR>
__device__ __forceinline__ int column_query(int n) {
  if constexpr (split_operand<G, PAIR>()) return n;
  else if constexpr (PAIR) return 4 * (n >> 3) + (n & 3);
  else return n < G ? n : (n < 2 * G ? n - G : -1);
}
template <int G, bool PAIR>
__device__ __forceinline__ bool column_hi(int n) {
  if constexpr (split_operand<G, PAIR>()) return true;
  else if constexpr (PAIR) return (n & 4) == 0;
  else return n < G;
}

// Value of lane (lane ^ m), for m a compile-time constant once unrolled:
// DPP moves within a row of 16 lanes for m <= 8 (m = 4 as a half-row mirror,
// lane ^ 7, followed by the quad reversal, lane ^ 3), an LDS permute beyond.
__device__ __forceinline__ float lane_xor(float v, int m) {
  const int b = __builtin_bit_cast(int, v);
  int r;
  if (m == 1) r = __builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true);        // quad_perm 1,0,3,2
  else if (m == 2) r = __builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true);   // quad_perm 2,3,0,1
  else if (m == 4) r = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(b, 0x141, 0xF, 0xF, true),
                                                0x1B, 0xF, 0xF, true);      // half mirror, 3,2,1,0
  else if (m == 8) r = __builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true);  // row_ror 8
  else return __shfl_xor(v, m);
  return __builtin_bit_cast(float, r);
}

// a[k] = a[k] + sg * (a[k] of lane ^ 4) for k < 8, within rows of 16 lanes:
// the half-row mirror (lane ^ 7) into copies, then the quad reversal
// (lane ^ 3) inside the multiply-add. One asm block: its first s_nop covers
// the VALU-write -> DPP-read hazard on a (written before the block), the
// second on the copies, the last on a for whatever DPP-reads it next (the
// compiler does not see the block's writes as vector ALU writes).
__device__ __forceinline__ void xbfly8_lane4(float& a0, float& a1, float& a2, float& a3,
                                             float& a4, float& a5, float& a6, float& a7,
                                             float sg) {
  float t0, t1, t2, t3, t4, t5, t6, t7;
  asm volatile(
      "s_nop 1\n\t"
      "v_mov_b32_dpp %8, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %9, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %10, %2 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %11, %3 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %12, %4 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %13, %5 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %14, %6 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "v_mov_b32_dpp %15, %7 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %8, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %9, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %10, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %11, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %12, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %13, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %14, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %15, %16 quad_perm:[3,2,1,0] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1"
      : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4), "+v"(a5), "+v"(a6), "+v"(a7),
        "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(t5), "=&v"(t6), "=&v"(t7)
      : "v"(sg));
}

// The fp16 query channels of the calling lane, as loaded (CPL / 2 words).
template <int G, bool PAIR>
struct QueryRaw {
  static constexpr int NQ = PAIR ? 2 * G : G;
  static constexpr int CPL = kD / (64 / NQ);
  uint32_t w[CPL / 2];
};

// Issues the load of the calling lane's query channels (see prepare_query for
// the lane layout); rows are 16-byte aligned (q and q_stride).
template <int G, bool PAIR>
__device__ __forceinline__ QueryRaw<G, PAIR> load_query(const QueryParams& p, int64_t b, int hg,
                                                        int lane) {
  using R = QueryRaw<G, PAIR>;
  constexpr int LQ = 64 / R::NQ;
  const int g = lane / LQ, j = lane % LQ;
  const __half* row = p.q + b * p.q_stride + (int64_t)(hg * R::NQ + g) * kD + j * R::CPL;
  R raw;
  if constexpr (R::CPL >= 8) {
#pragma unroll
    for (int c = 0; c < R::CPL / 8; ++c) {
      const uint4 w = reinterpret_cast<const uint4*>(row)[c];
      raw.w[4 * c] = w.x;
      raw.w[4 * c + 1] = w.y;
      raw.w[4 * c + 2] = w.z;
      raw.w[4 * c + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < R::CPL / 2; ++m) raw.w[m] = reinterpret_cast<const uint32_t*>(row)[m];
  }
  return raw;
}

// Query slots per head of the head-pair kernel: 8 for GR = 8, else 4.
template <int GR>
constexpr int pair_slots() { return GR == 8 ? 8 : 4; }

// Head pairs with GR query heads per KV head: the wave holds QS =
// pair_slots<GR>() query slots per head (2 QS in all, the layout
// prepare_query expects). Slot i of head hh (hh = 0, 1) is query
// (2 hp + hh) GR + min(i, GR - 1): with GR < QS the spare slots repeat the
// head's last query, and their results are never written.
template <int GR>
__device__ __forceinline__ QueryRaw<pair_slots<GR>(), true> load_query_pair(
    const QueryParams& p, int64_t b, int hp, int lane) {
  constexpr int QS = pair_slots<GR>();
  using R = QueryRaw<QS, true>;
  constexpr int LQ = 64 / R::NQ;
  const int g = lane / LQ, j = lane % LQ;
  const int qi = (2 * hp + g / QS) * GR + min(g % QS, GR - 1);
  const __half* row = p.q + b * p.q_stride + (int64_t)qi * kD + j * R::CPL;
  R raw;
#pragma unroll
  for (int c = 0; c < R::CPL / 8; ++c) {
    const uint4 w = reinterpret_cast<const uint4*>(row)[c];
    raw.w[4 * c] = w.x;
    raw.w[4 * c + 1] = w.y;
    raw.w[4 * c + 2] = w.z;
    raw.w[4 * c + 3] = w.w;
  }
  return raw;
}

// The B operand of the score MFMAs for the calling lane (bq), and for the
// lane's column n = lane % 16 the accumulator start value (minus 8 times the
// sum of the query's effective multipliers, cinit) and the log2-unit scale F.
// The wave's queries are those of head group `hg` of sequence b: one KV head,
// or a pair of KV heads (PAIR); `raw` is what load_query returned for them.
// xs: NQ x 128 floats of LDS. One wave.
//
// Query g of the wave is held by LQ = 64 / NQ consecutive lanes, CPL = 2 NQ
// contiguous channels per lane, so the Walsh-Hadamard stages of stride < CPL
// are in-lane and the others pair lane j of the query with lane j ^ (s / CPL):
// the lower lane takes fma(a, 1, b) = f32(a + b), the upper fma(b, -1, a) =
// f32(a - b), the same butterflies in the same order as the definition. The
// query's reductions run over its own LQ lanes.
template <int G, bool PAIR>
__device__ __forceinline__ void prepare_query(const QueryParams& p, const QueryRaw<G, PAIR>& raw,
                                              int lane, float (*xs)[kD], u4_t (&bq)[4],
                                              float& cinit_n, float& F_n, u4_t* bq_lo = nullptr) {
  constexpr int NQ = PAIR ? 2 * G : G;          // queries of the wave
  static_assert(!PAIR || G == 4 || G == 8, "head pairs are laid out for 4 or 8 queries per head");
  // split_operand: bq gets the hi parts, bq_lo the lo parts of every column
  constexpr bool kSplit = split_operand<G, PAIR>();
  constexpr int LQ = 64 / NQ;                   // lanes per query
  constexpr int CPL = kD / LQ;                  // channels per lane
  const int g = lane / LQ, j = lane % LQ;

  float x[CPL];
#pragma unroll
  for (int m = 0; m < CPL / 2; ++m) {
    const __half2 hv = __builtin_bit_cast(__half2, raw.w[m]);
    x[2 * m] = __low2float(hv);
    x[2 * m + 1] = __high2float(hv);
  }
  float sgn = 1.0f;              // the lane's sign after the fused stages
  if (p.rot_k) {
#pragma unroll
    for (int s = 1; s < CPL; s <<= 1) {
      if (s < p.h) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          if ((e & s) == 0) {
            const float a = x[e], c = x[e + s];
            x[e] = a + c;
            x[e + s] = a - c;
          }
        }
      }
    }
#pragma unroll
    for (int s = CPL; s < kD; s <<= 1) {
      if (s < p.h) {
        const int m = s / CPL;
        const float sg = (j & m) ? -1.0f : 1.0f;
        if (CPL % 8 == 0 && (m == 1 || m == 2 || m == 4)) {
          // x + sg * partner, one v_fmac_f32_dpp per value: that is sg times
          // f32(sg * x + partner) (rounding is symmetric), so the lane keeps
          // the sign sg and the next stages (whose partners share it) and
          // the scaling below absorb it exactly
#pragma unroll
          for (int e = 0; e < CPL; e += 8) {
            if (m == 1) {
              xbfly8_lane1(x[e], x[e + 1], x[e + 2], x[e + 3], x[e + 4], x[e + 5], x[e + 6],
                           x[e + 7], sg);
            } else if (m == 2) {
              xbfly8_lane2(x[e], x[e + 1], x[e + 2], x[e + 3], x[e + 4], x[e + 5], x[e + 6],
                           x[e + 7], sg);
            } else {
              xbfly8_lane4(x[e], x[e + 1], x[e + 2], x[e + 3], x[e + 4], x[e + 5], x[e + 6],
                           x[e + 7], sg);
            }
          }
          sgn *= sg;
        } else {
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            const float xp = lane_xor(x[e], m);
            x[e] = __builtin_fmaf(x[e], sg, xp);
          }
        }
      }
    }
  }
  const float mul = p.rot_k ? p.c_h * sgn : 1.0f;

  float v[CPL];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    v[e] = x[e] * mul * p.c_sm;
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int o = LQ / 2; o >= 1; o >>= 1) amax = fmaxf(amax, lane_xor(amax, o));
  int ex = 0;
  if (amax > 0.0f) frexpf(amax, &ex);               // amax in [2^(ex-1), 2^ex)
  const int sigma = amax > 0.0f ? 14 - ex : 0;      // max |Q| in [2^13, 2^14)
  float msum = 0.0f;
#pragma unroll
  for (int e = 0; e < CPL; e += 2) {
    const float Q0 = ldexpf(v[e], sigma), Q1 = ldexpf(v[e + 1], sigma);
    // effective multiplier of u: (hi + lo) of Q (even channel) and of Q / 16
    // times 16 (odd channel)
    const _Float16 h0 = (_Float16)Q0;
    const _Float16 l0 = (_Float16)(Q0 - (float)h0);
    const float q16 = Q1 * 0.0625f;
    const _Float16 h1 = (_Float16)q16;
    const _Float16 l1 = (_Float16)(q16 - (float)h1);
    msum += ((float)h0 + (float)l0) + 16.0f * ((float)h1 + (float)l1);
    xs[g][j * CPL + e] = Q0;
    xs[g][j * CPL + e + 1] = q16;
  }
#pragma unroll
  for (int o = LQ / 2; o >= 1; o >>= 1) msum += lane_xor(msum, o);
  const float cinit_g = -8.0f * ldexpf(msum, -24);
  const float sig_g = ldexpf(1.0f, 24 - sigma);
  __syncthreads();

  const int gl = lane >> 4, n = lane & 15;
  uint32_t words[kQWords], words_lo[kQWords];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch0 = 8 * (4 * gl + c) + e, ch1 = ch0 + 4;
      uint32_t w = 0, wl = 0;
      const int qi = column_query<G, PAIR>(n);
      if (qi >= 0) {
        float v[2] = {xs[qi][ch0], xs[qi][ch1]};
        uint16_t bits[2], bits_lo[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const _Float16 hi = (_Float16)v[k];
          const _Float16 lo = (_Float16)(v[k] - (float)hi);
          bits[k] = __builtin_bit_cast(uint16_t, column_hi<G, PAIR>(n) ? hi : lo);
          bits_lo[k] = __builtin_bit_cast(uint16_t, lo);
        }
        w = (uint32_t)bits[0] | ((uint32_t)bits[1] << 16);
        wl = (uint32_t)bits_lo[0] | ((uint32_t)bits_lo[1] << 16);
      }
      words[4 * c + e] = w;
      words_lo[4 * c + e] = wl;
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bq[k] = u4_t{words[4 * k], words[4 * k + 1], words[4 * k + 2], words[4 * k + 3]};
    if constexpr (kSplit)
      bq_lo[k] = u4_t{words_lo[4 * k], words_lo[4 * k + 1], words_lo[4 * k + 2], words_lo[4 * k + 3]};
  }
  {
    const int qi = column_query<G, PAIR>(n);
    const int src = (qi >= 0 ? qi : 0) * LQ;
    const float ci = __shfl(cinit_g, src), f = __shfl(sig_g, src);
    const bool take = qi >= 0 && column_hi<G, PAIR>(n);
    cinit_n = take ? ci : 0.0f;
    F_n = take ? f : 0.0f;
  }
  __syncthreads();                 // xs is reused by the caller's next query group
}

// ---------------------------------------------------------------------------
// chunk: scores, online softmax, P.V over one chunk of one (sequence, head)
// ---------------------------------------------------------------------------

struct ChunkParams {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint16_t* k_scales;
  const uint16_t* v_scales;
  const int32_t* block_tables;
  int64_t bt_stride;
  const int32_t* context_lens;
  QueryParams qp;
  float* part_o;           // [B][NC][Hq][128]
  float* part_ml;          // [B][NC][Hq][2]: reference exponent, denominator
  int64_t N_pg;
  int32_t P, H, Hq, NC, C, max_context;
  uint32_t n_groups;       // B * NC
  // lean form: waves per head pair, sequences, and the merge's view of
  // each sequence (first wave holding its steps, number of such waves)
  int32_t lean_waves, lean_seqs;
  int2* lean_seq;
};

// Registers of one 32-token step as loaded from memory (tiles T = 0, 1 of 16
// tokens; lane (g, n) = (lane / 16, lane % 16)).
struct StepRegs {
  u4_t kq[2];          // K codes of token n of tile T, bytes 16g..16g+15
  uint32_t vd[2][4];   // V code dword n of token 4g + j of tile T
  uint32_t sc;         // one scale: K (lanes 0-31) or V (lanes 32-63) of token
                       // lane % 16 of tile (lane / 16) % 2
  bool ok[2];          // tile starts before the end and has a valid page
};

// Per-lane constants of the chunk loop.
struct Lanes {
  uint32_t k_off;      // byte offset of the lane's K code bytes in a tile
  uint32_t v_off[4];   // byte offsets of the lane's V code dwords
  const uint16_t* s_ptr;  // the lane's scale pool (K for lanes 0-31, else V),
                          // advanced to token lane % 16 of a tile
  bool s_tile1;        // the lane stages a scale of tile 1 (else tile 0)
};

// Buffer resource over [base, base + bytes): raw (untyped) loads with the
// hardware range check, which returns 0 past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Issues the loads of the step at t0 into r. `pages` holds the page id of
// block (blk0 + lane) of the sequence in lane `lane`.
// WIN: the page ids of the range are held 64 at a time, those of pages
// blk0 .. blk0 + 63 in `pages`, the next 64 in `pages_next`; a step's two
// tiles may fall on either side of that boundary.
template <bool BRANCHLESS, bool WIN = false>
__device__ __forceinline__ void load_step(const ChunkParams& p, StepRegs& r, int t0, int t_end,
                                          int blk0, int pages, int h, const Lanes& ln,
                                          int pages_next = -1) {
  const uint32_t row_bytes = (uint32_t)p.H * (kD / 2);
  const uint32_t tile_bytes = 15u * row_bytes + kD / 2;      // reach of a lane's offsets
  int64_t row[2];                                 // first row of each tile (0 if invalid)
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int st = t0 + 16 * T;
    int page = -1;
    if (st < t_end) {
      const int idx = st / p.P - blk0;
      if constexpr (WIN)
        page = idx < 64 ? __builtin_amdgcn_readlane(pages, idx & 63)
                        : __builtin_amdgcn_readlane(pages_next, (idx - 64) & 63);
      else
        page = __builtin_amdgcn_readlane(pages, idx);
    }
    r.ok[T] = page >= 0 && page < p.N_pg;
    const int64_t row0 = r.ok[T] ? ((int64_t)page * p.P + st % p.P) * p.H + h : 0;
    row[T] = row0;
    if (BRANCHLESS || r.ok[T]) {
      // (branchless: an invalid tile gets an empty buffer range, whose loads
      // touch no memory and return zeros)
      const uint32_t reach = r.ok[T] ? tile_bytes : 0u;
      const __amdgpu_buffer_rsrc_t rk = rsrc(p.k_codes + row0 * (kD / 2), reach);
      const __amdgpu_buffer_rsrc_t rv = rsrc(p.v_codes + row0 * (kD / 2), reach);
      r.kq[T] = __builtin_amdgcn_raw_buffer_load_b128(rk, ln.k_off, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r.vd[T][j] = __builtin_amdgcn_raw_buffer_load_b32(rv, ln.v_off[j], 0, 0);
    } else {
      r.kq[T] = u4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j) r.vd[T][j] = 0u;
    }
  }
  // one scale per lane; an invalid tile reads its lane's slot of row 0
  // (in bounds, ignored)
  r.sc = ln.s_ptr[ln.s_tile1 ? row[1] : row[0]];
}

template <int G>
struct Acc {
  float m, mref, l, W;
  f4_t o[8];
};

__device__ __forceinline__ _Float16 half_lo(uint32_t x) {
  return __builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
}
__device__ __forceinline__ _Float16 half_hi(uint32_t x) {
  return __builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// One 32-token step. ks[T] / vs[T]: the K / V scales of tokens 4g..4g+3 of
// tile T as two dwords of fp16 pairs. mask: some tokens may be invalid.
template <int G>
__device__ __forceinline__ void compute_step(const StepRegs& r, const uint32_t (&ks)[2][2],
                                             const uint32_t (&vs)[2][2], const u4_t (&bq)[4],
                                             float cinit, float F, float F4, Acc<G>& a, int g,
                                             int n, int t0, int t_end, bool mask) {
  float lam[2][4], mu[2][4];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    f4_t acc = f4_t{cinit, cinit, cinit, cinit};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      // u = code + 8 = nibble ^ 8, masked into the fp16 lanes (the shift
      // is taken before the xor so each masked word is one 3-input logic op)
      const uint32_t raw = r.kq[T][cc], raw8 = raw >> 8;
      const u4_t av = u4_t{(raw ^ 0x88888888u) & 0x000F000Fu, (raw ^ 0x88888888u) & 0x00F000F0u,
                           (raw8 ^ 0x00888888u) & 0x000F000Fu, (raw8 ^ 0x00888888u) & 0x00F000F0u};
      acc = mfma(av, bq[cc], acc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float s = acc[j] + row_shl<G>(acc[j]);
      const uint32_t kw = ks[T][j >> 1], vw = vs[T][j >> 1];
      lam[T][j] = fmaf((float)((j & 1) ? half_hi(kw) : half_lo(kw)), s, 0.0f);
      const float ub = (float)((j & 1) ? (vw >> 24) : ((vw >> 8) & 0xFFu));
      mu[T][j] = fmaf(F4, lam[T][j], ub);
    }
  }
  if (mask) {
    // token 16 T + 4 g + j of the step is valid iff 4 g < t_end - t0 - 16 T - j
    // (a per-lane value against a wave-uniform one)
    const int rem = __builtin_amdgcn_readfirstlane(t_end - t0);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(r.ok[T] && 4 * g < rem - 16 * T - j)) mu[T][j] = -INFINITY;
  }

  float mx = max3_raw(max3_raw(mu[0][0], mu[0][1], mu[0][2]),
                      max3_raw(mu[0][3], mu[1][0], mu[1][1]),
                      max3_raw(mu[1][2], mu[1][3], -INFINITY));
  mx = rows_max(mx);
  const bool need = n < G && mx > a.m + 32.0f;
  if (__any(need)) {
    const float mn = need ? mx : a.m;
    const float alpha = need ? __builtin_amdgcn_exp2f((a.m - mn) * 0.25f) : 1.0f;
    a.l *= alpha;
    a.W *= alpha;
    // factor of query j (G < 8) or of query j / 4 + j (G = 8, by lane group);
    // both candidates are read as uniform values and selected per lane, so no
    // array is indexed with a lane-dependent value (that would go to scratch)
    const int ab = __builtin_bit_cast(int, alpha);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float f;
      if constexpr (G == 8) {
        const float f0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, j));
        const float f1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, 4 + j));
        f = (g & 1) ? f1 : f0;
      } else {
        f = __builtin_bit_cast(float, __builtin_amdgcn_readlane(ab, j % G));
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) a.o[k][j] *= f;
    }
    a.m = mn;
    a.mref = mn * 0.25f - 20.0f;
  }

  // weights p * s_v, split into fp16 hi + lo for the A operand
  float pr[2][4], w[2][4];
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[T][j] = __builtin_amdgcn_exp2f(fmaf(F, lam[T][j], -a.mref));
      const uint32_t vw = vs[T][j >> 1];
      w[T][j] = fmaf((float)((j & 1) ? half_hi(vw) : half_lo(vw)), pr[T][j], 0.0f);
    }
  if (mask) {
    const int rem = __builtin_amdgcn_readfirstlane(t_end - t0);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(r.ok[T] && 4 * g < rem - 16 * T - j)) pr[T][j] = w[T][j] = 0.0f;
  }
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a.l += pr[T][j];
      a.W += w[T][j];
    }
  // w - hi (exact): one mixed-precision fma each, reading hi as fp16 (the -1
  // is kept opaque so the fma is not folded into a convert and a subtract)
  const float mone = opaque(-1.0f);
  u4_t A;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int T = e >> 1, j0 = 2 * (e & 1);
    const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(w[T][j0], w[T][j0 + 1]));
    const float r0 = fmaf((float)hi[0], mone, w[T][j0]);
    const float r1 = fmaf((float)hi[1], mone, w[T][j0 + 1]);
    const h2_t lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    A[e] = lo_rows<G>(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo));
  }

  // values: lane n holds code dword n of tokens (T, j); MFMA 2*beta (+1) uses
  // the low (high) nibble of byte beta
#pragma unroll
  for (int beta = 0; beta < 4; ++beta) {
    const uint32_t sel = (uint32_t)beta | (0x0Cu << 8) | ((4u + beta) << 16) | (0x0Cu << 24);
    u4_t blo, bhi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int T = e >> 1, j0 = 2 * (e & 1);
      const uint32_t x = __builtin_amdgcn_perm(r.vd[T][j0 + 1], r.vd[T][j0], sel) ^ 0x00880088u;
      blo[e] = x & 0x000F000Fu;
      bhi[e] = x & 0x00F000F0u;
    }
    a.o[2 * beta] = mfma(A, blo, a.o[2 * beta]);
    a.o[2 * beta + 1] = mfma(A, bhi, a.o[2 * beta + 1]);
  }
}

// The step loop of a piece, double-buffered: step t0's registers are in one
// set while the loads of step t0 + step go to the other. The body holds two
// steps, so the two sets alternate without a copy (copying registers whose
// loads are in flight waits for those loads), its loads go out without a
// condition (past the end of the range they get an empty buffer range and
// touch no memory), and the loop has one exit. So every path into a step's
// arithmetic has the same loads issued after that step's own, and the
// compiler's wait before the arithmetic leaves the next step's loads in
// flight; a conditional issue, or a break after each step, made it wait for
// those too, which left no load of the wave in flight while it computed.
// An odd last step is computed after the loop from the set the loop filled.
template <typename Issue, typename Step>
__device__ __forceinline__ void pipelined_steps(const int t_begin, const int t_end, const int step,
                                                StepRegs& ra, StepRegs& rb, Issue&& issue,
                                                Step&& compute) {
  const int nsteps = t_end > t_begin ? (t_end - t_begin + step - 1) / step : 0;
  int t0 = t_begin;
  for (int i = 0; i < nsteps / 2; ++i) {
    issue(rb, t0 + step);
    compute(ra, t0);
    issue(ra, t0 + 2 * step);
    compute(rb, t0 + step);
    t0 += 2 * step;
  }
  if (nsteps & 1) compute(ra, t0);
  // the loads issued past the end are drained here (vmcnt 0, the other
  // counters left alone): a later piece of the same wave then reuses their
  // registers without the compiler holding its loop back for them
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// The plain form: one step of look-ahead issued only while steps remain, the
// loaded set copied forward after each step. The compiler's wait before a
// step's arithmetic also covers the next step's loads (the last step's path,
// which issues none, merges into it), so the wave keeps no load in flight
// while it computes, and the other waves of the SIMD (three for these
// kernels, whose registers the pipelined form would push past 168) cover the
// latency instead. That measured faster than the pipelined form for every
// grouping but eight queries per KV head, and faster than this loop with its
// loads issued on every step (which leaves them in flight at three waves).
template <typename Issue, typename Step>
__device__ __forceinline__ void lookahead_steps(const int t_begin, const int t_end, const int step,
                                                StepRegs& cur, StepRegs& nxt, Issue&& issue,
                                                Step&& compute) {
  for (int t0 = t_begin; t0 < t_end; t0 += step) {
    if (t0 + step < t_end) issue(nxt, t0 + step);
    compute(cur, t0);
    cur = nxt;
  }
}

// Tokens [t_begin, t_end) of sequence b for KV head h, one wave: the
// partial (reference exponent, denominator, weighted values) of the head's G
// queries goes to partial row `part`. t_begin is a multiple of 16. WINDOWS:
// the range may span more than 64 pages (page ids held 64 at a time).
template <int G, bool EARLY, bool WINDOWS>
__device__ __forceinline__ void head_piece(const ChunkParams& p, const int b, const int h,
                                           const int t_begin, const int t_end,
                                           const int64_t part, uint16_t* sstage,
                                           float (*xs)[kD]) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  int lane = threadIdx.x;
  // in the lean kernel's loop over ranges, the lane's offsets are derived
  // anew for every piece rather than held across the loop
  if constexpr (WINDOWS) asm volatile("" : "+v"(lane));
  const int g = lane >> 4, n = lane & 15;

  // page ids of the range's blocks, one per lane, 64 at a time (a chunk
  // spans at most 64, see make_layout)
  int blk0 = t_begin / p.P;
  const int blk_last = (t_end - 1) / p.P;
  const int32_t* bt_row = p.block_tables + (int64_t)b * p.bt_stride;
  int pages = lane <= blk_last - blk0 ? bt_row[blk0 + lane] : -1;
  int pages_next = -1;
  if constexpr (WINDOWS) {
    if (blk_last - blk0 >= 64) pages_next = lane <= blk_last - blk0 - 64 ? bt_row[blk0 + 64 + lane] : -1;
  }
  // the query's load goes out between the page ids and the first step, so
  // each wait takes only what it needs (loads complete in issue order)
  const QueryRaw<G, false> qraw = load_query<G, false>(p.qp, b, h, lane);

  Lanes ln;
  const uint32_t row_bytes = (uint32_t)p.H * (kD / 2);
  ln.k_off = (uint32_t)n * row_bytes + 16u * (uint32_t)g;
#pragma unroll
  for (int j = 0; j < 4; ++j) ln.v_off[j] = (uint32_t)(4 * g + j) * row_bytes + 4u * (uint32_t)n;
  ln.s_ptr = (lane < 32 ? p.k_scales : p.v_scales) + (int64_t)n * p.H;
  ln.s_tile1 = (lane >> 4) & 1;

  Acc<G> a;
  a.m = -INFINITY;
  a.mref = 0.0f;
  a.l = 0.0f;
  a.W = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a.o[k] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // one step of look-ahead: the loads of step t0 + 32 are in flight while
  // step t0 is computed. EARLY: the first step's loads are issued before the
  // query is prepared, which then overlaps their latency.
  StepRegs ra, rb;
  u4_t bq[4];
  float cinit, F;
  if constexpr (EARLY) {
    load_step<true, WINDOWS>(p, ra, t_begin, t_end, blk0, pages, h, ln, pages_next);
    prepare_query<G, false>(p.qp, qraw, lane, xs, bq, cinit, F);
  } else {
    prepare_query<G, false>(p.qp, qraw, lane, xs, bq, cinit, F);
    load_step<false, WINDOWS>(p, ra, t_begin, t_end, blk0, pages, h, ln, pages_next);
  }
  const float F4 = 4.0f * F;
  auto issue = [&](StepRegs& r, const int t1) {
    if constexpr (WINDOWS) {
      // the step's first tile opens the next 64 pages (wave-uniform)
      if (t1 < t_end && t1 / p.P - blk0 >= 64) {
        // (their ids were loaded with the previous window's; the following
        // ones go out now, lanes past the range's last page reading that
        // page's id again: in bounds, and no tile reads those lanes)
        blk0 += 64;
        pages = pages_next;
        pages_next = bt_row[min(blk0 + 64 + lane, blk_last)];
      }
    }
    load_step<false, WINDOWS>(p, r, t1, t_end, blk0, pages, h, ln, pages_next);
  };
  auto step = [&](const StepRegs& r, const int t0) {
    sstage[lane] = (uint16_t)r.sc;
    __builtin_amdgcn_wave_barrier();
    uint32_t ks[2][2], vs[2][2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const uint2 kk = *reinterpret_cast<const uint2*>(&sstage[16 * T + 4 * g]);
      const uint2 vv = *reinterpret_cast<const uint2*>(&sstage[32 + 16 * T + 4 * g]);
      ks[T][0] = kk.x;
      ks[T][1] = kk.y;
      vs[T][0] = vv.x;
      vs[T][1] = vv.y;
    }
    __builtin_amdgcn_wave_barrier();
    const bool mask = !(r.ok[0] && r.ok[1] && t0 + kStep <= t_end);
    compute_step<G>(r, ks, vs, bq, cinit, F, F4, a, g, n, t0, t_end, mask);
  };
  lookahead_steps(t_begin, t_end, kStep, ra, rb, issue, step);

  // ---- chunk partial ----
  float l = rows_sum(a.l);
  float W = rows_sum(a.W);
  f4_t os[8];
  if constexpr (G == 4 || G == 8) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = a.o[k][j], y = a.o[k][j];
        if constexpr (G == 4) swap16(x, y);
        else swap32(x, y);
        os[k][j] = x + y;
      }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) os[k][j] = j < G ? a.o[k][j] + a.o[k][j + G] : 0.0f;
  }
  const int Wb = __builtin_bit_cast(int, W);

  const int64_t head0 = part * p.Hq + (int64_t)h * G;
  const bool writer = G == 8 ? g < 2 : g == 0;
  if (writer) {
#pragma unroll
    for (int j = 0; j < (G < 4 ? G : 4); ++j) {
      const int qi = G == 8 ? 4 * g + j : j;
      float Wv;
      if constexpr (G == 8) {
        const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(Wb, j & 3));
        const float w1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(Wb, 4 + (j & 3)));
        Wv = g ? w1 : w0;
      } else {
        Wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(Wb, j % G));
      }
      float vals[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        vals[k] = os[k][j] * ((k & 1) ? 1048576.0f : 16777216.0f) - 8.0f * Wv;
      f4_t* dst = reinterpret_cast<f4_t*>(p.part_o + (head0 + qi) * kD + 8 * n);
      dst[0] = f4_t{vals[0], vals[1], vals[2], vals[3]};
      dst[1] = f4_t{vals[4], vals[5], vals[6], vals[7]};
    }
  }
  if (g == 0 && n < G) {
    p.part_ml[(head0 + n) * 2] = a.m == -INFINITY ? -INFINITY : a.mref;
    p.part_ml[(head0 + n) * 2 + 1] = l;
  }
}

// One (chunk, sequence, KV head) per block: chunk c covers tokens
// [c C, (c + 1) C) of the sequence.
template <int G, bool EARLY>
__global__ __launch_bounds__(64) void attn_chunk_kernel(ChunkParams p) {
  __shared__ uint16_t sstage[64];
  __shared__ float xs[G][kD];

  // Block -> (chunk, sequence, head). Blocks are dealt to the 8 XCDs in turn
  // (block i to XCD i % 8); the H heads of one (sequence, chunk) get
  // consecutive blocks of one XCD, so the 64-byte rows of neighbouring heads,
  // which share cache lines, meet in one L2.
  const uint32_t bx = blockIdx.x;
  const uint32_t r8 = bx >> 3;
  const int h = (int)(r8 % (uint32_t)p.H);
  const uint32_t grp = (r8 / (uint32_t)p.H) * 8u + (bx & 7u);
  if (grp >= p.n_groups) return;
  // Groups of chunks in dispatch order, counted from the end of each context:
  // group r holds chunk nck - NC + r of every sequence (nck = its chunk
  // count), so whole chunks go first and the partial last chunks (r = NC - 1)
  // last, which keeps the final round of waves short (longest work first).
  const uint32_t nb = p.n_groups / (uint32_t)p.NC;
  // the groups of XCD x are those with grp % 8 == x; offsetting the sequence
  // by r spreads the chunks of one sequence over the XCDs (when nb % 8 == 0
  // group r of sequence b goes to XCD (b + r) % 8), so every XCD gets a share
  // of every context, not whole ones
  const int r = (int)(grp / nb);
  const int b = (int)((grp % nb + nb - (uint32_t)r % nb) % nb);
  int L = p.context_lens[b];
  L = L < 0 ? 0 : (L > p.max_context ? p.max_context : L);
  const int c = (L + p.C - 1) / p.C - p.NC + r;     // chunk index; < 0: none
  if (c < 0) return;
  const int64_t part = (int64_t)b * p.NC + c;      // partial slot (b, c)
  const int t_begin = c * p.C;
  if (t_begin >= L) return;
  const int t_end = min(t_begin + p.C, L);

  head_piece<G, EARLY, false>(p, b, h, t_begin, t_end, part, sstage, xs);
}

// ---------------------------------------------------------------------------
// chunk, head pairs (even H): one wave per (sequence, chunk, pair of KV heads)
// ---------------------------------------------------------------------------
//
// The two heads of a pair hold the two halves of one 128-byte cache line of
// every token, so a wave that owns the pair reads whole lines. A step is 16
// tokens (one page-aligned block) of both heads, as two tiles of 8 tokens.
//
// Scores: MFMA row m of tile tau is token 8 tau + 2 (m % 4) + m / 8 of head
// (m / 4) % 2. With four query slots per head, columns 0-3 / 4-7 hold the
// hi / lo parts of head 0's four queries, 8-11 / 12-15 those of head 1; with
// eight, column n holds query n % 8 of head n / 8, hi parts in one operand
// and lo parts in a second. Result lane (g, n) holds rows 4g + j: tokens
// 8 tau + 2j + g / 2 of head g % 2, so its values are useful when its column
// belongs to that head (n / 8 == g % 2; with four slots also n % 8 < 4).
// Values: k slot (g, i = 4 tau + j) is token 8 tau + 2j + g / 2 of head g % 2,
// so the weights sit in the same lanes as their scores. With four slots rows
// 0-3 / 4-7 of the A operand are head 0's hi / lo weights, rows 8-11 / 12-15
// head 1's; with eight, row n is query n % 8 of head n / 8 and the hi and lo
// weights are two A operands. A row is zero where the slot's head is not the
// row's head.

struct PairLanes {
  uint32_t k_off[2];   // byte offsets of the lane's K code bytes, tiles 0 and 1
  uint32_t v_off[8];   // byte offsets of the lane's V code dwords, slots i
  const uint16_t* s_ptr;  // the lane's scale (loader role), relative to the block
};

// AUX: cache policy of the code loads (0 default, 2 nontemporal).
template <bool BRANCHLESS, int AUX>
__device__ __forceinline__ void load_pair_step(const ChunkParams& p, StepRegs& r, int t0,
                                               int t_end, int blk0, int pages, int h0,
                                               const PairLanes& ln) {
  const uint32_t row_bytes = (uint32_t)p.H * (kD / 2);
  int page = -1;
  if (t0 < t_end) page = __builtin_amdgcn_readlane(pages, t0 / p.P - blk0);
  const bool ok = page >= 0 && page < p.N_pg;
  r.ok[0] = r.ok[1] = ok;
  const int64_t row0 = ok ? ((int64_t)page * p.P + t0 % p.P) * p.H + h0 : 0;
  if (BRANCHLESS || ok) {
    // (branchless: an invalid block gets an empty buffer range, whose loads
    // touch no memory and return zeros)
    const uint32_t reach = ok ? 15u * row_bytes + 2u * (kD / 2) : 0u;   // 16 tokens, two heads
    const __amdgpu_buffer_rsrc_t rk = rsrc(p.k_codes + row0 * (kD / 2), reach);
    const __amdgpu_buffer_rsrc_t rv = rsrc(p.v_codes + row0 * (kD / 2), reach);
#pragma unroll
    for (int T = 0; T < 2; ++T) r.kq[T] = __builtin_amdgcn_raw_buffer_load_b128(rk, ln.k_off[T], 0, AUX);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r.vd[i >> 2][i & 3] = __builtin_amdgcn_raw_buffer_load_b32(rv, ln.v_off[i], 0, AUX);
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T) r.kq[T] = u4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) r.vd[i >> 2][i & 3] = 0u;
  }
  r.sc = ln.s_ptr[row0];       // an invalid block reads row 0 of the pool (ignored)
}

// One 16-token step of a head pair. ks[tau] / vs[tau]: the K / V scales of the
// lane's rows (tokens 8 tau + 2j + g / 2, head g % 2, j = 0..3) as two dwords
// of fp16 pairs. head_ok: the lane's column belongs to its rows' head.
//
// QS = 8 query slots per head: the score columns are the 16 queries (bq their
// hi parts, bq_lo their lo parts, one MFMA chain each, added per element as
// the hi and lo columns are with QS = 4), and the value rows are the 16
// queries too, the hi and the lo weights entering as two MFMAs into the same
// accumulator.
template <int QS>
__device__ __forceinline__ void compute_pair_step(const StepRegs& r, const uint32_t (&ks)[2][2],
                                                  const uint32_t (&vs)[2][2], const u4_t (&bq)[4],
                                                  const u4_t (&bq_lo)[4], float cinit, float F,
                                                  float F4, Acc<QS>& a, int g, int n, bool head_ok,
                                                  int t0, int t_end, bool mask) {
  static_assert(QS == 4 || QS == 8, "query slots per head");
  float lam[2][4], mu[2][4];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    f4_t acc = f4_t{cinit, cinit, cinit, cinit};
    f4_t acl = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      // u = code + 8 = nibble ^ 8, masked into the fp16 lanes (the shift
      // is taken before the xor so each masked word is one 3-input logic op)
      const uint32_t raw = r.kq[T][cc], raw8 = raw >> 8;
      const u4_t av = u4_t{(raw ^ 0x88888888u) & 0x000F000Fu, (raw ^ 0x88888888u) & 0x00F000F0u,
                           (raw8 ^ 0x00888888u) & 0x000F000Fu, (raw8 ^ 0x00888888u) & 0x00F000F0u};
      acc = mfma(av, bq[cc], acc);
      if constexpr (QS == 8) acl = mfma(av, bq_lo[cc], acl);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = QS == 8 ? acc[j] + acl[j] : acc[j] + row_shl<4>(acc[j]);
      const uint32_t kw = ks[T][j >> 1], vw = vs[T][j >> 1];
      lam[T][j] = fmaf((float)((j & 1) ? half_hi(kw) : half_lo(kw)), sc, 0.0f);
      const float ub = (float)((j & 1) ? (vw >> 24) : ((vw >> 8) & 0xFFu));
      mu[T][j] = fmaf(F4, lam[T][j], ub);
    }
  }
  if (mask) {
    // token 8 T + 2 j + g / 2 of the step is valid iff g / 2 < t_end - t0 - 8 T - 2 j
    // (a per-lane value against a wave-uniform one)
    const int rem = __builtin_amdgcn_readfirstlane(t_end - t0);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(r.ok[T] && (g >> 1) < rem - 8 * T - 2 * j)) mu[T][j] = -INFINITY;
  }

  float mx = max3_raw(max3_raw(mu[0][0], mu[0][1], mu[0][2]),
                      max3_raw(mu[0][3], mu[1][0], mu[1][1]),
                      max3_raw(mu[1][2], mu[1][3], -INFINITY));
  mx = rows_max(head_ok ? mx : -INFINITY);
  const bool need = (QS == 8 || (n & 4) == 0) && mx > a.m + 32.0f;
  if (__any(need)) {
    const float mn = need ? mx : a.m;
    const float alpha = need ? __builtin_amdgcn_exp2f((a.m - mn) * 0.25f) : 1.0f;
    a.l *= alpha;
    a.W *= alpha;
    constexpr int NA = 2 * QS;
    float al[NA];
#pragma unroll
    for (int qc = 0; qc < NA; ++qc)
      al[qc] = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha),
                                           QS == 8 ? qc : 8 * (qc >> 2) + (qc & 3)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // QS = 4: rows 4g + j are head g / 2, query j; QS = 8: query 4g + j
      float f;
      if constexpr (QS == 8)
        f = g == 0 ? al[j] : g == 1 ? al[4 + j] : g == 2 ? al[8 + j] : al[12 + j];
      else
        f = (g >> 1) ? al[4 + j] : al[j];
#pragma unroll
      for (int k = 0; k < 8; ++k) a.o[k][j] *= f;
    }
    a.m = mn;
    a.mref = mn * 0.25f - 20.0f;
  }

  float pr[2][4], w[2][4];
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[T][j] = __builtin_amdgcn_exp2f(fmaf(F, lam[T][j], -a.mref));
      const uint32_t vw = vs[T][j >> 1];
      w[T][j] = fmaf((float)((j & 1) ? half_hi(vw) : half_lo(vw)), pr[T][j], 0.0f);
    }
  if (mask) {
    const int rem = __builtin_amdgcn_readfirstlane(t_end - t0);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (!(r.ok[T] && (g >> 1) < rem - 8 * T - 2 * j)) pr[T][j] = w[T][j] = 0.0f;
  }
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a.l += pr[T][j];
      a.W += w[T][j];
    }
  // w - hi (exact): one mixed-precision fma each, reading hi as fp16 (the -1
  // is kept opaque so the fma is not folded into a convert and a subtract)
  const float mone = opaque(-1.0f);
  u4_t A, Alo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int T = e >> 1, j0 = 2 * (e & 1);
    const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(w[T][j0], w[T][j0 + 1]));
    const float r0 = fmaf((float)hi[0], mone, w[T][j0]);
    const float r1 = fmaf((float)hi[1], mone, w[T][j0 + 1]);
    const h2_t lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
    if constexpr (QS == 8) {
      A[e] = head_ok ? __builtin_bit_cast(uint32_t, hi) : 0u;
      Alo[e] = head_ok ? __builtin_bit_cast(uint32_t, lo) : 0u;
    } else {
      // lanes 4-7 and 12-15 of each row take the lo part from lane - 4
      const uint32_t v = (uint32_t)__builtin_amdgcn_update_dpp(
          (int)__builtin_bit_cast(uint32_t, hi), (int)__builtin_bit_cast(uint32_t, lo), 0x114,
          0xF, 0xA, false);
      A[e] = head_ok ? v : 0u;
    }
  }

#pragma unroll
  for (int beta = 0; beta < 4; ++beta) {
    const uint32_t sel = (uint32_t)beta | (0x0Cu << 8) | ((4u + beta) << 16) | (0x0Cu << 24);
    u4_t blo, bhi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int T = e >> 1, j0 = 2 * (e & 1);
      const uint32_t x = __builtin_amdgcn_perm(r.vd[T][j0 + 1], r.vd[T][j0], sel) ^ 0x00880088u;
      blo[e] = x & 0x000F000Fu;
      bhi[e] = x & 0x00F000F0u;
    }
    a.o[2 * beta] = mfma(A, blo, a.o[2 * beta]);
    a.o[2 * beta + 1] = mfma(A, bhi, a.o[2 * beta + 1]);
    if constexpr (QS == 8) {
      a.o[2 * beta] = mfma(Alo, blo, a.o[2 * beta]);
      a.o[2 * beta + 1] = mfma(Alo, bhi, a.o[2 * beta + 1]);
    }
  }
}

// Tokens [t_begin, t_end) of sequence b for head pair hp, one wave: the
// partial (reference exponent, denominator, weighted values) of every query
// of the pair goes to partial row `part`. t_begin is a multiple of 16.
// WINDOWS: the range may span more than 64 pages; the page ids are then held
// 64 at a time (one per lane), the next 64 loaded while the current ones are
// used. Without it the range spans at most 64 pages.
//
// GR: query heads per KV head (1, 2, 4 or 8). The wave computes QS = 4 query
// slots per head for GR <= 4 (see load_query_pair), 8 for GR = 8; with GR = 1
// or 2 the spare slots repeat a query: the extra arithmetic is hidden behind
// the loads, and the wave still reads whole lines.
template <int GR, bool EARLY, bool WINDOWS, bool PIPE>
__device__ __forceinline__ void pair_piece(const ChunkParams& p, const int b, const int hp,
                                           const int t_begin, const int t_end,
                                           const int64_t part, uint16_t* sstage,
                                           float (*xs)[kD]) {
  constexpr int G = pair_slots<GR>();
  static_assert(GR == 1 || GR == 2 || GR == 4 || GR == 8, "queries per KV head");
  // The code loads are nontemporal: in a decode step every layer's pool is
  // read once, so its lines have no later use in the last-level cache and
  // would only displace lines that do (the partials, queries, block tables).
  // Each wave reads whole 128-byte lines (two heads' rows), so no line is
  // shared with another wave. A whole 36-layer decode step (one pool per
  // layer) measured 1.8-2.0 % faster at 1-4 sequences and 7.1 % at 64 than
  // with ordinary loads below three times the cache size, the same at 16 and
  // 256 (where the pool already streamed); one pool read back to back is
  // faster with ordinary loads up to 64 sequences, because it then stays
  // cached between calls.
  constexpr int kAux = 2;
  // PIPE: the pipelined step loop (see pipelined_steps)
  constexpr bool kPipe = PIPE;
  int lane = threadIdx.x;
  // in the lean kernel's loop over ranges, the lane's load offsets are
  // derived anew for every piece instead of being held across the loop (the
  // opaque copy keeps the compiler from hoisting them): eight queries per KV
  // head then fit 167 registers, three waves per SIMD, instead of 187
  if constexpr (WINDOWS) asm volatile("" : "+v"(lane));
  const int g = lane >> 4, n = lane & 15;
  const int h0 = 2 * hp;

  int blk0 = t_begin / p.P;
  const int blk_last = (t_end - 1) / p.P;
  const int32_t* bt_row = p.block_tables + (int64_t)b * p.bt_stride;
  int pages = lane <= blk_last - blk0 ? bt_row[blk0 + lane] : -1;
  int pages_next = -1;
  if constexpr (WINDOWS) {
    if (blk_last - blk0 >= 64) pages_next = lane <= blk_last - blk0 - 64 ? bt_row[blk0 + 64 + lane] : -1;
  }
  // the query's load goes out between the page ids and the first step, so
  // each wait takes only what it needs (loads complete in issue order)
  const QueryRaw<G, true> qraw = load_query_pair<GR>(p.qp, b, hp, lane);
  const bool head_ok = (n >> 3) == (g & 1);

  PairLanes ln;
  const uint32_t row_bytes = (uint32_t)p.H * (kD / 2);
#pragma unroll
  for (int T = 0; T < 2; ++T)
    ln.k_off[T] = (uint32_t)(8 * T + 2 * (n & 3) + (n >> 3)) * row_bytes +
                  (uint32_t)((n >> 2) & 1) * (kD / 2) + 16u * (uint32_t)g;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    ln.v_off[i] = (uint32_t)(8 * (i >> 2) + 2 * (i & 3) + (g >> 1)) * row_bytes +
                  (uint32_t)(g & 1) * (kD / 2) + 4u * (uint32_t)n;
  {
    // loader role: lane l stages tensor l / 32 (K, V), tile (l / 16) % 2, and
    // the reader slot (g' = (l / 4) % 4, j = l % 4): token 8 tau + 2j + g' / 2
    // of head g' % 2
    const int tau = (lane >> 4) & 1, gs = (lane >> 2) & 3, js = lane & 3;
    ln.s_ptr = (lane < 32 ? p.k_scales : p.v_scales) +
               (int64_t)(8 * tau + 2 * js + (gs >> 1)) * p.H + (gs & 1);
  }

  Acc<G> a;
  a.m = -INFINITY;
  a.mref = 0.0f;
  a.l = 0.0f;
  a.W = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a.o[k] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // EARLY: the first step's loads are issued before the query is prepared,
  // which then overlaps their latency
  StepRegs ra, rb;
  u4_t bq[4], bq_lo[4];
  float cinit, F;
  if constexpr (EARLY) {
    load_pair_step<true, kAux>(p, ra, t_begin, t_end, blk0, pages, h0, ln);
    prepare_query<G, true>(p.qp, qraw, lane, xs, bq, cinit, F, bq_lo);
  } else {
    prepare_query<G, true>(p.qp, qraw, lane, xs, bq, cinit, F, bq_lo);
    load_pair_step<false, kAux>(p, ra, t_begin, t_end, blk0, pages, h0, ln);
  }
  const float F4 = 4.0f * F;
  auto issue = [&](StepRegs& r, const int t1) {
    if constexpr (WINDOWS) {
      // the step opens the next 64 pages (wave-uniform)
      if (t1 < t_end && t1 / p.P - blk0 >= 64) {
        // (their ids were loaded with the previous window's; the following
        // ones go out now, lanes past the range's last page reading that
        // page's id again: in bounds, and no tile reads those lanes)
        blk0 += 64;
        pages = pages_next;
        pages_next = bt_row[min(blk0 + 64 + lane, blk_last)];
      }
    }
    load_pair_step<kPipe, kAux>(p, r, t1, t_end, blk0, pages, h0, ln);
  };
  auto step = [&](const StepRegs& r, const int t0) {
    sstage[lane] = (uint16_t)r.sc;
    __builtin_amdgcn_wave_barrier();
    uint32_t ks[2][2], vs[2][2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const uint2 kk = *reinterpret_cast<const uint2*>(&sstage[16 * T + 4 * g]);
      const uint2 vv = *reinterpret_cast<const uint2*>(&sstage[32 + 16 * T + 4 * g]);
      ks[T][0] = kk.x;
      ks[T][1] = kk.y;
      vs[T][0] = vv.x;
      vs[T][1] = vv.y;
    }
    __builtin_amdgcn_wave_barrier();
    const bool mask = !(r.ok[0] && t0 + 16 <= t_end);
    compute_pair_step<G>(r, ks, vs, bq, bq_lo, cinit, F, F4, a, g, n, head_ok, t0, t_end, mask);
  };
  if constexpr (kPipe)
    pipelined_steps(t_begin, t_end, 16, ra, rb, issue, step);
  else
    lookahead_steps(t_begin, t_end, 16, ra, rb, issue, step);

  // ---- partial ----
  const float l = rows_sum(head_ok && (G == 8 || (n & 4) == 0) ? a.l : 0.0f);
  const float W = rows_sum(head_ok && (G == 8 || (n & 4) == 0) ? a.W : 0.0f);
  if constexpr (G == 8) {
    // rows 4g + j of the accumulators and column n of l, W: query 4g + j
    // resp. n of the pair, query head 8 h0 + that index
    float Wq[16];
#pragma unroll
    for (int qc = 0; qc < 16; ++qc)
      Wq[qc] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, W), qc));
    const int64_t head0 = part * p.Hq + (int64_t)h0 * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float Wv = g == 0 ? Wq[j] : g == 1 ? Wq[4 + j] : g == 2 ? Wq[8 + j] : Wq[12 + j];
      float vals[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        vals[k] = a.o[k][j] * ((k & 1) ? 1048576.0f : 16777216.0f) - 8.0f * Wv;
      f4_t* dst = reinterpret_cast<f4_t*>(p.part_o + (head0 + 4 * g + j) * kD + 8 * n);
      dst[0] = f4_t{vals[0], vals[1], vals[2], vals[3]};
      dst[1] = f4_t{vals[4], vals[5], vals[6], vals[7]};
    }
    if (g == 0) {
      p.part_ml[(head0 + n) * 2] = a.m == -INFINITY ? -INFINITY : a.mref;
      p.part_ml[(head0 + n) * 2 + 1] = l;
    }
    return;
  }
  f4_t os[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = a.o[k][j], y = a.o[k][j];
      swap16(x, y);                       // rows 4g + j: hi (g even) + lo (g odd)
      os[k][j] = x + y;
    }
  float Wq[8];
#pragma unroll
  for (int qc = 0; qc < 8; ++qc)
    Wq[qc] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, W),
                                                                 8 * (qc >> 2) + (qc & 3)));
  // query slot j of head hh is query head (h0 + hh) GR + j; spare slots
  // (j >= GR) are not written
  const int64_t head0 = part * p.Hq + (int64_t)h0 * GR;
  if ((g & 1) == 0) {                       // g = 0: head 0, g = 2: head 1
    const int hh = g >> 1;
#pragma unroll
    for (int j = 0; j < (GR < 4 ? GR : 4); ++j) {
      const float Wv = hh ? Wq[4 + j] : Wq[j];
      float vals[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        vals[k] = os[k][j] * ((k & 1) ? 1048576.0f : 16777216.0f) - 8.0f * Wv;
      f4_t* dst = reinterpret_cast<f4_t*>(p.part_o + (head0 + GR * hh + j) * kD + 8 * n);
      dst[0] = f4_t{vals[0], vals[1], vals[2], vals[3]};
      dst[1] = f4_t{vals[4], vals[5], vals[6], vals[7]};
    }
  }
  if (g == 0 && (n & 4) == 0 && (n & 3) < GR) {
    const int64_t qrow = head0 + GR * (n >> 3) + (n & 3);
    p.part_ml[qrow * 2] = a.m == -INFINITY ? -INFINITY : a.mref;
    p.part_ml[qrow * 2 + 1] = l;
  }
}

// One (chunk, sequence, head pair) per block: chunk c covers tokens
// [c C, (c + 1) C) of the sequence.
template <int GR, bool EARLY, bool PIPE>
__global__ __launch_bounds__(64) void attn_chunk_pair_kernel(ChunkParams p) {
  __shared__ uint16_t sstage[64];
  __shared__ float xs[2 * pair_slots<GR>()][kD];
  const int HP = p.H / 2;

  // Block -> (chunk, sequence, head pair), the pairs of one (sequence, chunk)
  // on consecutive blocks of one XCD.
  const uint32_t bx = blockIdx.x;
  const uint32_t r8 = bx >> 3;
  const int hp = (int)(r8 % (uint32_t)HP);
  const uint32_t grp = (r8 / (uint32_t)HP) * 8u + (bx & 7u);
  if (grp >= p.n_groups) return;
  // Groups of chunks in dispatch order, counted from the end of each context:
  // group r holds chunk nck - NC + r of every sequence (nck = its chunk
  // count), so whole chunks go first and the partial last chunks (r = NC - 1)
  // last, which keeps the final round of waves short (longest work first).
  const uint32_t nb = p.n_groups / (uint32_t)p.NC;
  // the groups of XCD x are those with grp % 8 == x; offsetting the sequence
  // by r spreads the chunks of one sequence over the XCDs (when nb % 8 == 0
  // group r of sequence b goes to XCD (b + r) % 8), so every XCD gets a share
  // of every context, not whole ones
  const int r = (int)(grp / nb);
  const int b = (int)((grp % nb + nb - (uint32_t)r % nb) % nb);
  int L = p.context_lens[b];
  L = L < 0 ? 0 : (L > p.max_context ? p.max_context : L);
  const int c = (L + p.C - 1) / p.C - p.NC + r;     // chunk index; < 0: none
  if (c < 0) return;
  const uint32_t part = (uint32_t)b * p.NC + c;    // partial slot (b, c)
  const int t_begin = c * p.C;
  if (t_begin >= L) return;
  const int t_end = min(t_begin + p.C, L);
  pair_piece<GR, EARLY, false, PIPE>(p, b, hp, t_begin, t_end, part, sstage, xs);
}

// Equal work per wave: the 16-token steps of all sequences, in sequence
// order, are split into n ranges of equal length per head pair (wave k takes
// steps [k S / n, (k + 1) S / n) of the S steps); a range covers the end of
// one sequence, whole sequences and the start of another, one partial each,
// in partial row b + k (distinct for every (sequence, wave) that meet, since
// both only grow along the steps). Every wave streams from the first step to
// about the same end, so no round of waves starts or drains while others
// stream. A wave whose range is empty (fewer steps than waves) writes an
// empty partial where the merge may look for one.
//
// Every wave derives the split itself from the context lengths (at most
// kLeanMaxB sequences, 16 per lane): S_b = ceil(L_b / 16) steps per sequence
// (L_b clipped to [0, max_context]), their prefix sums P_b, the sequence and
// local step where its range starts; and for the merge, for each sequence
// whose first step P_b lies in its range, the first wave holding its steps
// (this one) and their number: the wave holding step s is
// floor(((s + 1) n - 1) / S). Wave 0 marks the empty sequences.
constexpr int kLeanMaxB = 1024;

// The split for wave k of n (n = p.lean_waves): returns false if the step has
// no token; else b, s0 = the sequence and local step where the range starts
// and rem = its length in steps (0: an empty range). `writer`: this wave
// records the merge's view of the sequences whose first step lies in its
// range (one head group's waves do).
__device__ __forceinline__ bool lean_range(const ChunkParams& p, const int k, const bool writer,
                                           int& b, int& s0, int64_t& rem) {
  const int lane = threadIdx.x;
  const int N = p.lean_waves;
  // steps of the lane's sequences 16 lane + j, and their sum
  int st[16];
  int lsum = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bb = 16 * lane + j;
    int L = bb < p.lean_seqs ? p.context_lens[bb] : 0;
    L = L < 0 ? 0 : (L > p.max_context ? p.max_context : L);
    st[j] = (L + 15) >> 4;
    lsum += st[j];
  }
  int incl = lsum;                          // inclusive prefix over the lanes
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int excl = incl - lsum;
  const int64_t S = __builtin_amdgcn_readlane(incl, 63);
  const int64_t lo = S > 0 ? (int64_t)k * S / N : 0;
  const int64_t hi = S > 0 ? (int64_t)(k + 1) * S / N : 0;
  if (writer) {
    int pre = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int bb = 16 * lane + j;
      const int64_t Pb = (int64_t)excl + pre;
      if (bb < p.lean_seqs) {
        if (st[j] == 0) {
          if (k == 0) p.lean_seq[bb] = make_int2(0, 0);
        } else if (lo <= Pb && Pb < hi) {
          const int64_t kl = ((Pb + st[j]) * N - 1) / S;
          p.lean_seq[bb] = make_int2(k, (int)(kl - k + 1));
        }
      }
      pre += st[j];
    }
  }
  if (S == 0) return false;
  // the sequence holding step lo: its lane, then its place in the lane
  const uint64_t ball = __ballot(excl <= lo && lo < (int64_t)excl + lsum);
  const int lam = __ffsll((unsigned long long)ball) - 1;
  const int off = (int)(lo - __builtin_amdgcn_readlane(excl, lam));
  b = -1;
  s0 = 0;
  int pre = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int sj = __builtin_amdgcn_readlane(st[j], lam);
    if (b < 0 && off < pre + sj) {
      b = 16 * lam + j;
      s0 = off - pre;
    }
    pre += sj;
  }
  rem = hi - lo;
  return true;
}

// Walks wave k's range from (b, s0) for rem steps, one piece per sequence:
// piece(b, t_begin, t_end) for each.
template <typename Piece>
__device__ __forceinline__ void lean_walk(const ChunkParams& p, int b, int s0, int64_t rem,
                                          Piece&& piece) {
  for (;;) {
    int L = p.context_lens[b];
    L = L < 0 ? 0 : (L > p.max_context ? p.max_context : L);
    const int steps = (L + 15) >> 4;
    const int nstep = (int)min((int64_t)(steps - s0), rem);
    piece(b, 16 * s0, min(16 * (s0 + nstep), L));
    rem -= nstep;
    if (rem <= 0) break;
    // the next sequence with a token (the range ends inside one)
    for (;;) {
      ++b;
      const int Ln = p.context_lens[b];
      if ((Ln < 0 ? 0 : (Ln > p.max_context ? p.max_context : Ln)) > 0) break;
    }
    s0 = 0;
  }
}

// An empty partial (no token) for `nq` queries from query head q0 in row `row`.
__device__ __forceinline__ void lean_empty(const ChunkParams& p, int64_t row, int q0, int nq) {
  if ((int)threadIdx.x < nq) {
    const int64_t r = row * p.Hq + q0 + threadIdx.x;
    p.part_ml[r * 2] = -INFINITY;
    p.part_ml[r * 2 + 1] = 0.0f;
  }
}

template <int GR, bool PIPE>
__global__ __launch_bounds__(64) void attn_lean_pair_kernel(ChunkParams p) {
  __shared__ uint16_t sstage[64];
  __shared__ float xs[2 * pair_slots<GR>()][kD];
  const int HP = p.H / 2;
  // block -> (wave k, head pair): the pairs of one range on one XCD
  const uint32_t bx = blockIdx.x;
  const uint32_t r8 = bx >> 3;
  const int hp = (int)(r8 % (uint32_t)HP);
  const int k = (int)((r8 / (uint32_t)HP) * 8u + (bx & 7u));
  if (k >= p.lean_waves) return;
  int b, s0;
  int64_t rem;
  if (!lean_range(p, k, hp == 0, b, s0, rem)) return;
  if (rem == 0) {
    lean_empty(p, (int64_t)b + k, 2 * hp * GR, 2 * GR);
    return;
  }
  lean_walk(p, b, s0, rem, [&](int bb, int t_begin, int t_end) {
    pair_piece<GR, true, true, PIPE>(p, bb, hp, t_begin, t_end, (int64_t)bb + k, sstage, xs);
  });
}

// The same split for an odd number of KV heads: one wave per (range, head).
template <int G>
__global__ __launch_bounds__(64) void attn_lean_kernel(ChunkParams p) {
  __shared__ uint16_t sstage[64];
  __shared__ float xs[G][kD];
  // block -> (wave k, head): the heads of one range on one XCD
  const uint32_t bx = blockIdx.x;
  const uint32_t r8 = bx >> 3;
  const int h = (int)(r8 % (uint32_t)p.H);
  const int k = (int)((r8 / (uint32_t)p.H) * 8u + (bx & 7u));
  if (k >= p.lean_waves) return;
  int b, s0;
  int64_t rem;
  if (!lean_range(p, k, h == 0, b, s0, rem)) return;
  if (rem == 0) {
    lean_empty(p, (int64_t)b + k, h * G, G);
    return;
  }
  lean_walk(p, b, s0, rem, [&](int bb, int t_begin, int t_end) {
    head_piece<G, true, true>(p, bb, h, t_begin, t_end, (int64_t)bb + k, sstage, xs);
  });
}

// ---------------------------------------------------------------------------
// combine: merge chunks, normalise, un-rotate V, fp16
// ---------------------------------------------------------------------------

struct CombineParams {
  const float* part_o;
  const float* part_ml;
  const int32_t* context_lens;
  __half* out;             // [B][Hq][128]
  int64_t n_vec;           // B * Hq
  int32_t Hq, NC, C, max_context;
  // lean form: per sequence, the first wave holding its steps and the
  // number of such waves (its partials are rows b + first ...); else null
  const int2* lean_seq;
};

// Sum of v over the four quads of a row of 16 lanes (DPP row rotations by 4,
// 8 and 12); every lane of the row gets the total.
__device__ __forceinline__ float quads_sum(float v) {
  const int b = __builtin_bit_cast(int, v);
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x124, 0xF, 0xF, false)) +
         __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false)) +
         __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x12C, 0xF, 0xF, false));
}
__device__ __forceinline__ float quads_max(float v) {
  const int b = __builtin_bit_cast(int, v);
  return fmaxf(fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x124, 0xF, 0xF, false))),
               fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, false)),
                     __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0x12C, 0xF, 0xF, false))));
}

// QPV quads of 4 lanes per output vector: QPV = 4, one row of 16 lanes per
// vector (4 vectors per wave), or QPV = 16, the whole wave on one vector (for
// few vectors with many chunks). Quad qd merges chunks qd, qd + QPV, ...;
// the quads are then merged.
template <int HB, int QPV>
__global__ __launch_bounds__(64) void attn_combine_kernel(CombineParams p) {
  static_assert(QPV == 4 || QPV == 16, "quads per vector");
  const int lane = threadIdx.x, lam = lane & 3;
  const int qd = QPV == 4 ? (lane >> 2) & 3 : lane >> 2;
  const int64_t v = QPV == 4 ? (int64_t)blockIdx.x * 4 + (lane >> 4) : (int64_t)blockIdx.x;
  const bool live = v < p.n_vec;
  int64_t b;
  int qh;
  if (p.n_vec <= (int64_t)UINT32_MAX) {
    // 32-bit division (a 64-bit one is a long emulated sequence that would
    // delay every load of the wave)
    const uint32_t vv = live ? (uint32_t)v : 0u;
    const uint32_t bb = vv / (uint32_t)p.Hq;
    b = bb;
    qh = (int)(vv - bb * (uint32_t)p.Hq);
  } else {
    b = live ? v / p.Hq : 0;
    qh = live ? (int)(v % p.Hq) : 0;
  }
  const int L_raw = live ? p.context_lens[b] : 0;
  // chunk form: chunk c of sequence b in row (b NC + c) Hq + qh; lean form:
  // the j-th wave holding sequence b in row (b + first + j) Hq + qh
  const bool lean = p.lean_seq != nullptr;
  const int2 sk = lean && live ? p.lean_seq[b] : make_int2(0, 0);
  const int64_t base = (lean ? b + sk.x : b * p.NC) * p.Hq + qh;   // piece c adds c * Hq

  // running reference M: a chunk with a larger one rescales what is summed
  float M = -INFINITY;
  float x[kElems];
#pragma unroll
  for (int k = 0; k < kElems; ++k) x[k] = 0.0f;
  float lsum = 0.0f;
  constexpr int kDepth = 4;
  f4_t buf[kDepth][8];
  float2 mlb[kDepth];
  auto fetch = [&](int k, int slot) {
    const int64_t row = base + (int64_t)(qd + QPV * k) * p.Hq;
    mlb[slot] = *reinterpret_cast<const float2*>(p.part_ml + row * 2);
    const f4_t* src = reinterpret_cast<const f4_t*>(p.part_o + row * kD + 8 * lam);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      buf[slot][2 * i] = src[8 * i];
      buf[slot][2 * i + 1] = src[8 * i + 1];
    }
  };
  auto accumulate = [&](int slot) {
    const float ref = mlb[slot].x;
    if (ref == -INFINITY) return;                 // no valid token in the chunk
    if (ref > M) {
      const float r = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - ref);
      lsum *= r;
#pragma unroll
      for (int k = 0; k < kElems; ++k) x[k] *= r;
      M = ref;
    }
    const float sc = __builtin_amdgcn_exp2f(ref - M);
    lsum += sc * mlb[slot].y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * i + j] += sc * buf[slot][2 * i][j];
        x[8 * i + 4 + j] += sc * buf[slot][2 * i + 1][j];
      }
  };

  // Quad qd merges chunks qd + QPV k, k < mine. The whole-wave form (few
  // vectors, many chunks) loads the partials of every chunk slot of the
  // layout without waiting for the context length, so that wait overlaps
  // theirs; slots past the context's last chunk (not written by this call)
  // are loaded but never merged. The 4-lane form waits for the length and
  // loads only the chunks it merges.
  int nfetch = 0;
  if (QPV == 16 && !lean) {
    nfetch = p.NC > qd ? (p.NC - qd + QPV - 1) / QPV : 0;
#pragma unroll
    for (int k = 0; k < kDepth - 1; ++k)
      if (k < nfetch) fetch(k, k);
    __builtin_amdgcn_sched_barrier(0);           // keep the length's wait below these loads
  }
  const int L = L_raw < 0 ? 0 : (L_raw > p.max_context ? p.max_context : L_raw);
  const int nck = lean ? sk.y : (L + p.C - 1) / p.C;
  const int mine = nck > qd ? (nck - qd + QPV - 1) / QPV : 0;
  if (QPV == 4 || lean) {
    nfetch = mine;
#pragma unroll
    for (int k = 0; k < kDepth - 1; ++k)
      if (k < nfetch) fetch(k, k);
  }
  for (int k0 = 0; k0 < nfetch; k0 += kDepth) {
#pragma unroll
    for (int k = 0; k < kDepth; ++k) {
      const int kk = k0 + k;
      if (kk >= nfetch) break;
      if (kk + kDepth - 1 < nfetch) fetch(kk + kDepth - 1, (k + kDepth - 1) % kDepth);
      if (kk < mine) accumulate(k);
    }
  }
  // merge the quads of the vector
  float Mv = quads_max(M);
  if constexpr (QPV == 16) Mv = rows_max(Mv);
  const float rq = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mv);
  lsum = quads_sum(lsum * rq);
#pragma unroll
  for (int k = 0; k < kElems; ++k) x[k] = quads_sum(x[k] * rq);
  if constexpr (QPV == 16) {
    lsum = rows_sum(lsum);
#pragma unroll
    for (int k = 0; k < kElems; ++k) x[k] = rows_sum(x[k]);
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
#pragma unroll
  for (int k = 0; k < kElems; ++k) x[k] *= inv;
  if constexpr (HB > 0) {
    lane_stage<0>(x);
    const float cs = fwht_rest<HB>(x, lam) * c_h<HB>();
#pragma unroll
    for (int k = 0; k < kElems; ++k) x[k] *= cs;
  }
  if (live && qd == 0) {
    u4_t* dst = reinterpret_cast<u4_t*>(p.out + v * kD + 8 * lam);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t wd[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint16_t lo = __builtin_bit_cast(uint16_t, __float2half_rn(x[8 * i + 2 * k]));
        const uint16_t hi = __builtin_bit_cast(uint16_t, __float2half_rn(x[8 * i + 2 * k + 1]));
        wd[k] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      dst[4 * i] = u4_t{wd[0], wd[1], wd[2], wd[3]};
    }
  }
}

}  // namespace attn
}  // namespace sawkv

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

namespace {

using sawkv::host::aligned;
using sawkv::host::fail;
using sawkv::host::ok;

constexpr int64_t kMaxContext = INT64_C(1) << 30;

struct Layout {
  int C;                   // tokens per chunk
  int64_t NC;              // chunks per sequence
  size_t ml, o;            // chunk form: byte offsets of the partials
  // lean form (when the sizes allow it): split plan and partials for at most
  // lean_waves waves per head pair
  bool lean;
  int32_t lean_waves;
  size_t l_seq, l_ml, l_o;
  size_t total;            // bytes for either form
};

// The lean form (equal steps per wave, see attn_lean_pair_kernel) serves
// steps with many tokens per head pair: at least kLeanMinSteps 16-token steps
// if every sequence had max_context tokens (fewer than 2^31, counted in 32
// bits), at most kLeanMaxB sequences (16 per lane of a wave); one wave per
// (range, head pair) for an even number of KV heads, per (range, head) for an
// odd one. Its grid is the resident waves of the device, at most
// kLeanMaxWaves.
// Measured on the decode batch (contexts uniform in [1, 8000], page 16), us
// per call chunk form / lean form for 32 / 64 / 8 query heads: 256 sequences
// 232.1 / 214.0, 251.5 / 237.5, 223.1 / 202.6; 96 sequences (48 000 steps)
// 101.8 / 91.9, 109.0 / 105.6, 94.9 / 85.8; 80 (40 000) 81.2 / 80.9, 94.4 /
// 94.2, 75.4 / 75.5; 64 70.2 / 69.7, 77.0 / 82.0, 66.0 / 65.1; 32 43.9 / 46.9,
// 44.8 / 56.3, 38.6 / 42.8; 64 contexts of 32 768 tokens 409.0 / 382.8.
constexpr int64_t kLeanMinSteps = 40960;
// One wave per (range, head) for odd head counts takes the lean split only
// with at least kLeanMinHeadSteps steps per wave if every sequence had
// max_context tokens (its loop steps are 32 tokens; fewer per wave lose to
// the chunk form). Measured, contexts uniform in [1, 8000], us per call cold,
// chunk form / lean split: 1 KV head (3072 waves) 256 sequences (42 steps per
// wave) 47.8 / 51.9, 1024 sequences (167) 141.1 / 129.1; 3 KV heads (1024
// waves per head) 256 sequences (125) 113.1 / 114.6, 1024 (500) 395.2 / 377.4.
constexpr int64_t kLeanMinHeadSteps = 128;
constexpr int kLeanMaxWaves = 4096;

bool lean_sizes(int64_t B, int64_t max_context) {
  const int64_t steps = B * ((max_context + 15) / 16);
  return B > 0 && B <= sawkv::attn::kLeanMaxB && steps >= kLeanMinSteps &&
         steps < (INT64_C(1) << 31);
}

// head groups of one wave: pairs of KV heads when H is even, else single heads
int32_t head_groups(int32_t H) { return H % 2 == 0 ? H / 2 : H; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Chunk length: 1024 tokens when the step has at least 16384 (sequence,
// chunk, head) items at that length (half the partials to merge, half the
// per-chunk preparations; measured 7 % faster on 64 contexts of 32768 tokens
// and 1.6 % at 256 sequences of up to 8000, but 6 % slower at 192), else
// 512, halved (down to 128) while the step would have fewer than 8192 items,
// so that small batches still spread over every compute unit; 64 only for
// grids too small to fill the chip even at 128 (each wave then pays the
// query preparation for fewer tokens, which costs more than it gains once the
// grid is large enough). A chunk starts at a multiple of C, so it spans at
// most 64 pages (P = 16 divides C) or C / P + 1 <= 33 (P >= 32): one page id
// per lane.
Layout make_layout(int64_t B, int32_t Hq, int32_t H, int64_t max_context) {
  Layout L{};
  int C = B * H * ((max_context + 1023) / 1024) >= 16384 ? 1024 : 512;
  // halve while the step would have fewer than `enough` items; eight queries
  // per KV head run the single-head kernel on such grids, whose waves carry
  // twice the arithmetic of a head pair's per token and prefer longer chunks
  // (64 query heads, µs at 16 / 24 / 48 sequences: 29.8 / 40.2 / 64.2 with
  // 4096 against 33.9 / 46.2 / 69.3 with 8192; 32 query heads lose with 4096).
  // An odd H runs the single-head kernel at every group size and prefers the
  // longer chunks too (cold caches, contexts of up to 8000: 1 KV head x 128 /
  // 256 / 448 sequences 30.5 / 44.0 / 70.6 µs against 33.6 / 48.1 / 79.0;
  // 3 x 80: 47.8 against 57.4; 5 x 48: 44.0 against 54.3; one loss, 3 x 128:
  // 63.3 against 60.6)
  const int64_t enough = (Hq / H == 8 || H % 2 == 1) ? 4096 : 8192;
  while (C > 128 && B * H * ((max_context + C - 1) / C) < enough) C >>= 1;
  // a grid that cannot fill the chip even at 128 tokens (one or two long
  // sequences): halve once more, fewer serial steps per wave
  if (C == 128 && B * H * ((max_context + 127) / 128) < 1024) C = 64;
  L.C = C;
  L.NC = max_context > 0 ? (max_context + C - 1) / C : 1;
  size_t off = 0;
  L.ml = off;
  off = align256(off + (size_t)B * L.NC * Hq * 2 * 4);
  L.o = off;
  off = align256(off + (size_t)B * L.NC * Hq * sawkv::kD * 4);
  L.total = off;
  L.lean = lean_sizes(B, max_context);
  if (L.lean) {
    L.lean_waves = std::max(8, kLeanMaxWaves / head_groups(H));
    const size_t rows = (size_t)(B + L.lean_waves) * Hq;   // partial rows b + k
    size_t lo = 0;
    L.l_seq = lo;
    lo = align256(lo + (size_t)B * 8);
    L.l_ml = lo;
    lo = align256(lo + rows * 2 * 4);
    L.l_o = lo;
    lo = align256(lo + rows * sawkv::kD * 4);
    if (lo > L.total) L.total = lo;
  }
  return L;
}

int check_attn_sizes(int64_t B, int32_t Hq, int32_t H, int32_t D, int64_t max_context) {
  if (B < 0) return fail(SAWKV_EINVAL, "B = %lld is negative", (long long)B);
  if (H <= 0 || Hq <= 0) return fail(SAWKV_EINVAL, "H = %d and Hq = %d must be positive", H, Hq);
  if (Hq % H != 0) return fail(SAWKV_EINVAL, "Hq = %d is not a multiple of H = %d", Hq, H);
  const int32_t G = Hq / H;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SAWKV_EUNSUPPORTED, "Hq / H = %d unsupported (1, 2, 4 or 8)", G);
  if (D != sawkv::kD) return fail(SAWKV_EUNSUPPORTED, "D = %d unsupported (only 128)", D);
  if (H > 256) return fail(SAWKV_EUNSUPPORTED, "H = %d unsupported (at most 256)", H);
  if (max_context < 0) return fail(SAWKV_EINVAL, "max_context = %lld is negative",
                                   (long long)max_context);
  if (max_context > kMaxContext)
    return fail(SAWKV_EUNSUPPORTED, "max_context = %lld too large (at most 2^30)",
                (long long)max_context);
  if (B > (INT64_C(1) << 24))
    return fail(SAWKV_EUNSUPPORTED, "B = %lld too large (at most 2^24)", (long long)B);
  if (B * Hq >= (INT64_C(1) << 33))
    return fail(SAWKV_EUNSUPPORTED, "B * Hq too large for one launch");
  const Layout lay = make_layout(B, Hq, H, max_context);
  // grid of the chunk kernel: ceil(B * NC / 8) * 8 * H blocks
  if (((B * lay.NC + 7) / 8) * 8 * H >= (INT64_C(1) << 31))
    return fail(SAWKV_EUNSUPPORTED, "B * chunks * H too large for one launch");
  return SAWKV_OK;
}

using sawkv::attn::attn_chunk_kernel;
using sawkv::attn::attn_chunk_pair_kernel;
using sawkv::attn::attn_combine_kernel;

int g_index(int32_t G) { return G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3; }

// [first-step order][G]: EARLY instantiations issue the first step's loads
// before preparing the query
const void* const kChunk[2][4] = {
    {(void*)&attn_chunk_kernel<1, false>, (void*)&attn_chunk_kernel<2, false>,
     (void*)&attn_chunk_kernel<4, false>, (void*)&attn_chunk_kernel<8, false>},
    {(void*)&attn_chunk_kernel<1, true>, (void*)&attn_chunk_kernel<2, true>,
     (void*)&attn_chunk_kernel<4, true>, (void*)&attn_chunk_kernel<8, true>}};
// [G index][first-step order]
// The head-pair kernels come with the plain step loop and the pipelined one
// (pipelined_steps), [G index][early][pipelined]. The pipelined loop keeps
// the next step's loads in flight during a step's arithmetic at two waves per
// SIMD instead of three. It pays where a step carries the most arithmetic
// (eight queries per KV head: 64 query heads over 256 contexts of up to 8000
// tokens 247 -> 236 us, over 32 of 32768 cold 229 -> 208 us) and where a
// wave's loads cover much of each token row. With two KV heads a row is the
// pair's 128-byte line, so a 16-token page reads as one 2 KB block (one pair
// over 256 contexts of up to 8000 tokens, 1, 2 or 4 queries per head: 68-74
// -> 64-70 us back to back, 72-78 -> 69-72 us cold; over 64 contexts of
// 32768 113 -> 107 us); with four the pair's line is half of each row (lean
// split, 256 contexts 116-121 -> 109-116 us, 128 contexts 69-72 -> 65 us; the
// chunk form's grids 3 % slower, so they keep the plain loop); with eight a
// wave reads a quarter of every row, and the third wave per SIMD measured
// faster (32 query heads 1-3 % slower pipelined). Eight queries per KV head
// have only the pipelined form.
#define SAWKV_PAIR(GR, PLAIN)                                              \
  {{(void*)&attn_chunk_pair_kernel<GR, false, PLAIN>,                     \
    (void*)&attn_chunk_pair_kernel<GR, false, true>},                     \
   {(void*)&attn_chunk_pair_kernel<GR, true, PLAIN>,                      \
    (void*)&attn_chunk_pair_kernel<GR, true, true>}}
const void* const kChunkPair[4][2][2] = {SAWKV_PAIR(1, false), SAWKV_PAIR(2, false),
                                         SAWKV_PAIR(4, false), SAWKV_PAIR(8, true)};
#undef SAWKV_PAIR

// A grid of at most four rounds of resident chunk waves (3 per SIMD on 256
// compute units) issues each wave's first loads before its query
// preparation: few rounds leave that latency on the critical path. Deeper
// grids hide it behind other waves, and there the early loads measured
// slightly slower.
constexpr int64_t kEarlyIssueBlocks = 4 * 3 * 4 * 256;

// Eight queries per KV head run the head-pair kernel from two rounds of
// resident waves (3 per SIMD on 256 compute units) up; smaller grids finish
// sooner with the single-head kernel's twice as many, shorter waves (which
// read only half of each line). Measured on the 256-sequence decode batch
// (64 query heads, contexts uniform in [1, 8000]), us per call single-head /
// head-pair: 256 sequences (8192 pair blocks) 283 / 252, 128 (8192) 152 /
// 137, 96 (6144) 114 / 110, 64 (4096) 76 / 78, 16 34 / 37, 1 12.5 / 15.4.
constexpr int64_t kPairEightBlocks = 2 * 3 * 4 * 256;

using sawkv::attn::attn_lean_kernel;
using sawkv::attn::attn_lean_pair_kernel;

// [form: single head, head pairs, head pairs pipelined][G index]
const void* const kLean[3][4] = {
    {(void*)&attn_lean_kernel<1>, (void*)&attn_lean_kernel<2>, (void*)&attn_lean_kernel<4>,
     (void*)&attn_lean_kernel<8>},
    {(void*)&attn_lean_pair_kernel<1, false>, (void*)&attn_lean_pair_kernel<2, false>,
     (void*)&attn_lean_pair_kernel<4, false>, (void*)&attn_lean_pair_kernel<8, true>},
    {(void*)&attn_lean_pair_kernel<1, true>, (void*)&attn_lean_pair_kernel<2, true>,
     (void*)&attn_lean_pair_kernel<4, true>, (void*)&attn_lean_pair_kernel<8, true>}};

// Lean waves per head group on the device of `stream`: the waves the device
// keeps resident at once (occupancy of the lean kernel times compute units,
// asked once per device and kernel), at most kLeanMaxWaves over all groups
// and max_per_group per group, a multiple of 8; 0 if the device cannot say.
constexpr int kLeanDevices = 64;
std::mutex g_lean_mu;
int g_lean_resident[kLeanDevices][3][4] = {};

int lean_waves_per_group(hipStream_t stream, int form, int gi, int groups, int max_per_group) {
  int dev = -1;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
      dev >= kLeanDevices)
    return 0;
  int resident;
  {
    std::lock_guard<std::mutex> lock(g_lean_mu);
    resident = g_lean_resident[dev][form][gi];
    if (resident == 0) {
      int per_cu = 0, cus = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kLean[form][gi], 64, 0) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        per_cu = cus = 0;
      resident = per_cu > 0 && cus > 0 ? per_cu * cus : -1;
      g_lean_resident[dev][form][gi] = resident;
    }
  }
  if (resident <= 0) return 0;
  const int per_group = std::min(std::min(resident, kLeanMaxWaves) / groups, max_per_group);
  return per_group / 8 * 8;
}

const void* const kCombine[2][5] = {
    {(void*)&attn_combine_kernel<0, 4>, (void*)&attn_combine_kernel<16, 4>,
     (void*)&attn_combine_kernel<32, 4>, (void*)&attn_combine_kernel<64, 4>,
     (void*)&attn_combine_kernel<128, 4>},
    {(void*)&attn_combine_kernel<0, 16>, (void*)&attn_combine_kernel<16, 16>,
     (void*)&attn_combine_kernel<32, 16>, (void*)&attn_combine_kernel<64, 16>,
     (void*)&attn_combine_kernel<128, 16>}};

int launch64(const void* fn, int64_t blocks, void* params, hipStream_t stream) {
  void* args[] = {params};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(64), args, 0, stream);
  if (e != hipSuccess) return fail(SAWKV_EHIP, "kernel launch: %s", hipGetErrorString(e));
  return SAWKV_OK;
}

int attention_impl(const void* q, int64_t q_stride, const void* k_codes, const void* v_codes,
                   const void* k_scales, const void* v_scales, int64_t N_pg, int32_t P,
                   const int32_t* block_tables, int64_t bt_stride, const int32_t* context_lens,
                   int64_t B, int32_t Hq, int32_t H, int32_t D, int64_t max_context,
                   float sm_scale, int32_t h, int32_t rot_mode, void* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_attn_sizes(B, Hq, H, D, max_context);
  if (st) return st;
  if (P <= 0) return fail(SAWKV_EINVAL, "P = %d must be positive", P);
  if (P % 16 != 0) return fail(SAWKV_EUNSUPPORTED, "P = %d unsupported (a multiple of 16)", P);
  if (N_pg <= 0) return fail(SAWKV_EINVAL, "N_pg = %lld must be positive", (long long)N_pg);
  if (N_pg > INT32_MAX)
    return fail(SAWKV_EUNSUPPORTED, "N_pg = %lld too large (page ids are int32)", (long long)N_pg);
  if (N_pg * P > (INT64_C(1) << 56) / ((int64_t)H * D))
    return fail(SAWKV_EINVAL, "pool of %lld pages x %d slots is too large", (long long)N_pg, P);
  if (h != 16 && h != 32 && h != 64 && h != 128)
    return fail(SAWKV_EUNSUPPORTED, "h = %d unsupported (16, 32, 64 or 128)", h);
  if (rot_mode != SAWKV_ROT_NONE && rot_mode != SAWKV_ROT_K && rot_mode != SAWKV_ROT_KV)
    return fail(SAWKV_EINVAL, "rot_mode = %d invalid", rot_mode);
  if (!(fabsf(sm_scale) <= 3.0e38f)) return fail(SAWKV_EINVAL, "sm_scale is not finite");
  if (bt_stride < (max_context + P - 1) / P)
    return fail(SAWKV_EINVAL, "bt_stride %lld < ceil(max_context / P) = %lld",
                (long long)bt_stride, (long long)((max_context + P - 1) / P));
  if (q_stride < (int64_t)Hq * D)
    return fail(SAWKV_EINVAL, "q_stride %lld < Hq*D = %d", (long long)q_stride, Hq * D);
  if (q_stride % 8 != 0)
    return fail(SAWKV_EALIGN, "q_stride %lld not a multiple of 8", (long long)q_stride);
  if (B == 0) return ok();
  if (!q || !k_codes || !v_codes || !k_scales || !v_scales || !block_tables || !context_lens ||
      !out || !workspace)
    return fail(SAWKV_EINVAL, "a tensor or workspace pointer is NULL");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(k_scales, 16) || !aligned(v_scales, 16) || !aligned(workspace, 256))
    return fail(SAWKV_EALIGN, "q, out and pools must be 16-byte aligned, workspace 256-byte");
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(SAWKV_EALIGN, "block_tables / context_lens not 4-byte aligned");
  const Layout lay = make_layout(B, Hq, H, max_context);
  if (workspace_bytes < lay.total)
    return fail(SAWKV_EINVAL, "workspace of %zu bytes < %zu needed", workspace_bytes, lay.total);

  const int32_t G = Hq / H;
  char* ws = static_cast<char*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  // an even head count: heads are processed in pairs, so that every wave
  // reads whole 128-byte lines (the two heads' 64-byte rows of a token).
  // Measured at 256 sequences against the single-head kernel: 8 query heads
  // 257 -> 228 us, 16 query heads 263 -> 232 us. With eight queries per KV
  // head a head-pair wave holds 16 queries and twice the matrix-core work
  // per step; it pays once the grid has kPairEightBlocks blocks.
  const int64_t pair_blocks = ((B * lay.NC + 7) / 8) * 8 * (H / 2);
  const bool pair = H % 2 == 0 && (G <= 4 || pair_blocks >= kPairEightBlocks);
  const int32_t groups = pair ? H / 2 : H;

  sawkv::attn::ChunkParams cp{};
  cp.k_codes = static_cast<const uint8_t*>(k_codes);
  cp.v_codes = static_cast<const uint8_t*>(v_codes);
  cp.k_scales = static_cast<const uint16_t*>(k_scales);
  cp.v_scales = static_cast<const uint16_t*>(v_scales);
  cp.block_tables = block_tables;
  cp.bt_stride = bt_stride;
  cp.context_lens = context_lens;
  cp.qp.q = static_cast<const __half*>(q);
  cp.qp.q_stride = q_stride;
  cp.qp.h = h;
  cp.qp.rot_k = rot_mode != SAWKV_ROT_NONE;
  cp.qp.c_h = (float)(1.0 / sqrt((double)h));
  cp.qp.c_sm = (float)((double)sm_scale * 1.4426950408889634);
  cp.part_o = reinterpret_cast<float*>(ws + lay.o);
  cp.part_ml = reinterpret_cast<float*>(ws + lay.ml);
  cp.N_pg = N_pg;
  cp.P = P;
  cp.H = H;
  cp.Hq = Hq;
  cp.NC = (int32_t)lay.NC;
  cp.C = lay.C;
  cp.max_context = (int32_t)max_context;
  cp.n_groups = (uint32_t)(B * lay.NC);
  const int hv = rot_mode == SAWKV_ROT_KV ? (h == 16 ? 1 : h == 32 ? 2 : h == 64 ? 3 : 4) : 0;
  sawkv::attn::CombineParams mp{};
  mp.context_lens = context_lens;
  mp.out = static_cast<__half*>(out);
  mp.n_vec = B * Hq;
  mp.Hq = Hq;
  mp.C = lay.C;
  mp.max_context = (int32_t)max_context;

  // the pipelined step loop for every grouping (kChunkPair): two KV heads in
  // either form, four in the lean split (the chunk form's grids there measured
  // 3 % slower pipelined)
  const int pipe = H == 2 ? 1 : 0;
  const int lean_pipe = H == 2 || H == 4 ? 1 : 0;

  // the lean form: split plan, equal-steps waves, merge
  const int lean_pair = H % 2 == 0 ? 1 : 0;
  const int lean_form = lean_pair + lean_pipe;
  const int nwp = lay.lean ? lean_waves_per_group(s, lean_form, g_index(G), head_groups(H),
                                                   lay.lean_waves)
                           : 0;
  if (nwp >= 8 && (lean_pair || B * ((max_context + 15) / 16) >= kLeanMinHeadSteps * nwp)) {
    cp.part_o = reinterpret_cast<float*>(ws + lay.l_o);
    cp.part_ml = reinterpret_cast<float*>(ws + lay.l_ml);
    cp.lean_waves = nwp;
    cp.lean_seqs = (int32_t)B;
    cp.lean_seq = reinterpret_cast<int2*>(ws + lay.l_seq);
    if ((st = launch64(kLean[lean_form][g_index(G)], (int64_t)nwp * head_groups(H), &cp, s)))
      return st;
    mp.part_o = cp.part_o;
    mp.part_ml = cp.part_ml;
    mp.lean_seq = cp.lean_seq;
    mp.NC = 0;
    // a whole wave per vector when a sequence meets many waves (few
    // sequences): nwp / B of them on average
    const bool wide = (int64_t)nwp > 16 * B && B * Hq < 4096;
    if ((st = launch64(kCombine[wide ? 1 : 0][hv], wide ? B * Hq : (B * Hq + 3) / 4, &mp, s)))
      return st;
    return ok();
  }

  const int64_t chunk_blocks = ((B * lay.NC + 7) / 8) * 8 * groups;
  const int early = chunk_blocks <= kEarlyIssueBlocks ? 1 : 0;
  if (max_context > 0 &&
      (st = launch64(pair ? kChunkPair[g_index(G)][early][pipe]
                          : kChunk[early][g_index(G)],
                     chunk_blocks, &cp, s)))
    return st;

  mp.part_o = cp.part_o;
  mp.part_ml = cp.part_ml;
  mp.NC = cp.NC;
  // more chunks than one round of 4-deep loads per quad, over few vectors: a
  // whole wave per vector (16 quads), so each quad merges a quarter as many
  // chunks; otherwise 4 vectors per wave
  const bool wide = lay.NC > 16 && B * Hq < 4096;
  if ((st = launch64(kCombine[wide ? 1 : 0][hv], wide ? B * Hq : (B * Hq + 3) / 4, &mp, s)))
    return st;
  return ok();
}

// ---- the entry point that allocates nothing ----
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the partials live in a file-scope device array of
// kScratchBytes, one copy per GPU, held until the process ends. Host code
// never uses the array's name as an address: its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and
// kept in g_scratch[device].
constexpr size_t kScratchBytes = SAWKV_NOALLOC_MAX_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream`.
int scratch_for(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SAWKV_EHIP, "device of the stream: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SAWKV_EUNSUPPORTED, "device %d outside the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess)
      return fail(SAWKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(SAWKV_EHIP, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess)
        return fail(SAWKV_EHIP, "hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
    }
    if (e != hipSuccess || p == nullptr)
      return fail(SAWKV_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return SAWKV_OK;
}

}  // namespace

extern "C" {

int sawkv_decode_attention_noalloc(const void* q, int64_t q_stride, const void* k_codes,
                                   const void* v_codes, const void* k_scales,
                                   const void* v_scales, int64_t N_pg, int32_t P,
                                   const int32_t* block_tables, int64_t bt_stride,
                                   const int32_t* context_lens, int64_t B, int32_t Hq,
                                   int32_t H, int32_t D, int64_t max_context, float sm_scale,
                                   int32_t h, int32_t rot_mode, void* out, void* stream) {
  int st = check_attn_sizes(B, Hq, H, D, max_context);
  if (st) return st;
  const size_t need = make_layout(B, Hq, H, max_context).total;
  if (need > kScratchBytes)
    return fail(SAWKV_EUNSUPPORTED,
                "these sizes need %zu bytes of partials, more than the %zu-byte static scratch "
                "(use sawkv_decode_attention with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (B > 0 && (st = scratch_for(reinterpret_cast<hipStream_t>(stream), &ws))) return st;
  return attention_impl(q, q_stride, k_codes, v_codes, k_scales, v_scales, N_pg, P,
                        block_tables, bt_stride, context_lens, B, Hq, H, D, max_context,
                        sm_scale, h, rot_mode, out, ws, kScratchBytes, stream);
}

int sawkv_decode_attention_workspace_size(int64_t B, int32_t Hq, int32_t H, int32_t D,
                                          int64_t max_context, size_t* bytes) {
  if (bytes == nullptr) return fail(SAWKV_EINVAL, "bytes is NULL");
  const int st = check_attn_sizes(B, Hq, H, D, max_context);
  if (st) return st;
  *bytes = make_layout(B, Hq, H, max_context).total;
  return ok();
}

int sawkv_decode_attention(const void* q, int64_t q_stride, const void* k_codes,
                           const void* v_codes, const void* k_scales, const void* v_scales,
                           int64_t N_pg, int32_t P, const int32_t* block_tables,
                           int64_t bt_stride, const int32_t* context_lens, int64_t B,
                           int32_t Hq, int32_t H, int32_t D, int64_t max_context,
                           float sm_scale, int32_t h, int32_t rot_mode, void* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(q, q_stride, k_codes, v_codes, k_scales, v_scales, N_pg, P,
                        block_tables, bt_stride, context_lens, B, Hq, H, D, max_context,
                        sm_scale, h, rot_mode, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
