/*
 * sawkv — fused block-diagonal Hadamard rotation + token-wise INT4 append into
 * a paged KV cache, and the matching dequantise / inverse-rotate read-back,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: youngju.dev reading of the SAW-INT4 preprint,
 * sections "Why Naive INT4 Breaks", "The Rotation Trick - Block-Diagonal
 * Hadamard" and the fused-kernel diagram in "The System Is the Design - A
 * Fused Kernel"; gist.science summary "SAW-INT4: System-Aware 4-Bit KV-Cache
 * Quantization for Real-World LLM Serving", §2 Metodologia, BDR items 1-3,
 * and §4 Risultati Sperimentali for h = 128 and keys-only rotation):
 *
 *   for every new token t and head j, for K and (unless skipped) V:
 *     x  = the fp16 head vector, widened to float32 (exact)
 *     y  = f32(c_h * F_h(x))   when the tensor is rotated, else y = x
 *          F_h: Sylvester Walsh-Hadamard butterflies inside each block of h
 *          contiguous channels, strides 1, 2, ..., h/2 in that order, each
 *          (a, b) -> (a + b, a - b) rounded to float32; c_h = f32(1/sqrt(h))
 *     s  = f16(f32(max_i |y_i| / 7)), saturated to 65504
 *     q_i = clamp(rint_half_even(f32(y_i / s)), -8, 7); s == 0 -> q = 0
 *     codes[slot][j][k] = (q_{2k} & 15) | (q_{2k+1} & 15) << 4
 *     scales[slot][j]   = s
 *   where slot = slot_mapping[t] = page * P + offset. Bit-exact against the
 *   float32 IEEE definition above (no FMA contraction, no denormal flush).
 *
 * Pool layout (vLLM-style pages; K and V have separate pools):
 *   codes  uint8   [N_pg][P][H][D/2]   (a token's H rows are contiguous)
 *   scales float16 [N_pg][P][H]
 * Slot s addresses row s of the flat [N_pg*P][H][...] view.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or synchronises, keeps no state between calls
 *     and is safe to call from several host threads. (The one exception,
 *     sawkv_decode_attention_noalloc at the end of this header, keeps its
 *     partial results in a static device array of the library.)
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return. Faults in device memory surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and a status > 0 is returned, with detail
 *     text from sawkv_last_error().
 *   - A slot < 0 or >= N_pg*P is skipped by append and yields a zero row in
 *     gather (no byte outside the addressed rows is ever touched).
 *   - T == 0 returns SAWKV_OK after the size checks, launches nothing and
 *     reads no pointer (NULL tensors are accepted then).
 *   - Caller preconditions not checked: no two tokens of one call share a
 *     slot (the shared rows then hold the bytes of either token, or a mix of
 *     the two at 4-byte granularity; no other row is touched); inputs,
 *     outputs and pools do not overlap; K/V values are finite.
 *   - Supported sizes: D = 128; h in {16, 32, 64, 128}; 1 <= H <= 256;
 *     T*H < 2^31; token strides < 2^26 elements (SAWKV_EUNSUPPORTED otherwise).
 *   - Alignment: every tensor pointer 16-byte aligned, slot_mapping 8-byte
 *     aligned, token strides multiples of 8 elements.
 */
#ifndef SAWKV_H
#define SAWKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAWKV_VERSION 1

enum {
  SAWKV_OK = 0,
  SAWKV_EINVAL = 1,        /* null pointer, negative or inconsistent size   */
  SAWKV_EUNSUPPORTED = 2,  /* D or h outside the supported set              */
  SAWKV_EALIGN = 3,        /* pointer or stride misaligned                  */
  SAWKV_EHIP = 4           /* the HIP runtime refused the launch            */
};

enum {
  SAWKV_ROT_NONE = 0,      /* naive token-wise INT4 for K and V             */
  SAWKV_ROT_K = 1,         /* rotate K only; V is naive INT4                */
  SAWKV_ROT_KV = 2         /* rotate K and V                                */
};

/*
 * Quantise T new tokens of K and V and append them to the paged INT4 pools.
 * (The fused rotation-quantisation-append kernel of the youngju.dev diagram
 * and of the gist.science summary, §2 BDR item 3 and §3 item 3.)
 *
 *   k, v          fp16 [T][H][D]; row (token) t starts at k + t*k_stride
 *                 elements; k_stride, v_stride >= H*D. Either k or v may be
 *                 NULL to skip that tensor (its pool pointers are then
 *                 ignored); not both.
 *   slot_mapping  int64 [T], device memory.
 *   k_codes, v_codes    uint8 [N_pg][P][H][D/2]   (written at mapped rows only)
 *   k_scales, v_scales  fp16  [N_pg][P][H]
 *   h             Hadamard block size; rot_mode one of SAWKV_ROT_*.
 * Returns SAWKV_OK or an error status (nothing launched on error).
 */
int sawkv_quantize_append(const void* k, const void* v,
                          int64_t k_stride, int64_t v_stride,
                          const int64_t* slot_mapping, int64_t T,
                          int32_t H, int32_t D,
                          void* k_codes, void* v_codes,
                          void* k_scales, void* v_scales,
                          int64_t N_pg, int32_t P,
                          int32_t h, int32_t rot_mode,
                          void* stream);

/*
 * Several layers of one decode step in one launch (up to SAWKV_MAX_LAYERS):
 * the same computation as one sawkv_quantize_append call per layer, for
 * layers that share T, H, D, the token strides, slot_mapping and the pool
 * geometry (N_pg, P), each with its own K/V inputs and pools. Meant for
 * decode, where one call per layer is bound by launch overhead; the
 * decode-time append of every new token is the step the pages' fused kernel
 * performs (youngju.dev fused-kernel diagram).
 *
 *   layers    HOST array of n_layers descriptors (read during the call only);
 *             every layer must have k present, or every layer k absent (same
 *             for v); absent tensors are NULL with NULL pools.
 * Validation, ownership and stream behaviour as for sawkv_quantize_append.
 */
#define SAWKV_MAX_LAYERS 64

typedef struct {
  const void* k;         /* fp16 [T][H][D] of this layer, or NULL        */
  const void* v;
  void* k_codes;         /* uint8 [N_pg][P][H][D/2]                      */
  void* v_codes;
  void* k_scales;        /* fp16 [N_pg][P][H]                            */
  void* v_scales;
} sawkv_layer_t;

int sawkv_quantize_append_layers(const sawkv_layer_t* layers, int32_t n_layers,
                                 int64_t k_stride, int64_t v_stride,
                                 const int64_t* slot_mapping, int64_t T,
                                 int32_t H, int32_t D,
                                 int64_t N_pg, int32_t P,
                                 int32_t h, int32_t rot_mode,
                                 void* stream);

/*
 * Read the tokens at slot_mapping back from the pools: y = q * s, then (for
 * rotated tensors) the same normalised Sylvester transform, which is its own
 * inverse (youngju.dev reading, "The Rotation Trick": the rotation is
 * orthogonal and can be undone), then fp16 round-to-nearest-even.
 *
 *   k_out, v_out  fp16 [T][H][D] contiguous; a NULL pair (pool and output)
 *                 skips that tensor; invalid slots give zero rows.
 * The read-back is exact up to the final f16 rounding: every partial sum of
 * q * s fits float32, so the result does not depend on summation order.
 */
int sawkv_dequant_gather(const void* k_codes, const void* v_codes,
                         const void* k_scales, const void* v_scales,
                         int64_t N_pg, int32_t P,
                         const int64_t* slot_mapping, int64_t T,
                         int32_t H, int32_t D,
                         void* k_out, void* v_out,
                         int32_t h, int32_t rot_mode,
                         void* stream);

/*
 * The no-rotation control ("naive" INT4 of the youngju.dev reading, section
 * "Why Naive INT4 Breaks"; the pure-INT4 throughput baseline of gist.science
 * §4): the same bytes, launch geometry and semantics as the two calls above
 * with rot_mode = SAWKV_ROT_NONE, built as separate kernel instantiations.
 */
int sawkv_naive_int4_append(const void* k, const void* v,
                            int64_t k_stride, int64_t v_stride,
                            const int64_t* slot_mapping, int64_t T,
                            int32_t H, int32_t D,
                            void* k_codes, void* v_codes,
                            void* k_scales, void* v_scales,
                            int64_t N_pg, int32_t P,
                            void* stream);

int sawkv_naive_int4_gather(const void* k_codes, const void* v_codes,
                            const void* k_scales, const void* v_scales,
                            int64_t N_pg, int32_t P,
                            const int64_t* slot_mapping, int64_t T,
                            int32_t H, int32_t D,
                            void* k_out, void* v_out,
                            void* stream);

/*
 * Controls: the caches the INT4 cache is compared against (gist.science
 * summary of SAW-INT4, §4 Risultati Sperimentali: accuracy and throughput
 * against a BF16 cache; ainews.cool, the table under "技术深度解析": a uniform
 * INT8 cache). Same tokens, slots, validation, ownership and stream behaviour
 * as sawkv_quantize_append.
 *
 * sawkv_cache_append: the uncompressed paged write. k_cache, v_cache are
 * 16-bit [N_pg][P][H][D] (fp16 or bf16: the 16-bit values are copied
 * unchanged); cache[slot][j] = the token's row j. k or v (with its cache) may
 * be NULL; invalid slots are skipped.
 */
int sawkv_cache_append(const void* k, const void* v,
                       int64_t k_stride, int64_t v_stride,
                       const int64_t* slot_mapping, int64_t T,
                       int32_t H, int32_t D,
                       void* k_cache, void* v_cache,
                       int64_t N_pg, int32_t P,
                       void* stream);

/*
 * sawkv_int8_append: token-wise INT8 with the INT4 path's optional rotation:
 *   s = f16(f32(amax / 127)), q = clamp(rint_half_even(f32(y / s)), -128, 127),
 *   s == 0 -> 0; codes int8 [N_pg][P][H][D] (one byte per channel), scales
 *   fp16 [N_pg][P][H].
 * sawkv_int8_gather: its read-back, f16(f32(c_h * f32(F_h(q) * s))) for a
 *   rotated tensor (F_h(q) of the integer codes is exact), f16(q * s)
 *   otherwise; invalid slots give zero rows. Bit-exact against that
 *   definition.
 */
int sawkv_int8_append(const void* k, const void* v,
                      int64_t k_stride, int64_t v_stride,
                      const int64_t* slot_mapping, int64_t T,
                      int32_t H, int32_t D,
                      void* k_codes, void* v_codes,
                      void* k_scales, void* v_scales,
                      int64_t N_pg, int32_t P,
                      int32_t h, int32_t rot_mode,
                      void* stream);

int sawkv_int8_gather(const void* k_codes, const void* v_codes,
                      const void* k_scales, const void* v_scales,
                      int64_t N_pg, int32_t P,
                      const int64_t* slot_mapping, int64_t T,
                      int32_t H, int32_t D,
                      void* k_out, void* v_out,
                      int32_t h, int32_t rot_mode,
                      void* stream);

/*
 * Access-pattern control of the INT4 append (a measurement control, not part
 * of the method). The pages place the fused append in a data flow bounded by
 * memory bandwidth, with the rotation's arithmetic hidden inside it
 * (gist.science summary, §2 Metodologia, BDR item 3); this call moves the
 * same bytes along the same paths with none of that arithmetic, so its time
 * is what the append's access pattern can reach at all on the device.
 *
 * It runs the append's grid and issues the append's loads (every fp16 row of
 * K and V, 16 bytes per lane, and the slot of every token) and writes, per
 * (token t, head j) vector, a 64-byte row and a 2-byte value:
 *   row word c (c = 0..15, little-endian uint32) = xor of the four uint32
 *       words of the input row's 16-byte piece c
 *   value bits = (word 0) xor (word 0 >> 16), low 16 bits
 * to the codes and scales pools at
 *   placement SAWKV_PLACE_SLOTS:       the row the append writes (slot*H + j;
 *                                      slots < 0 or >= N_pg*P are skipped)
 *   placement SAWKV_PLACE_TOKEN_ORDER: row t*H + j (needs T <= N_pg*P), i.e.
 *                                      the same writes to contiguous pages
 * Arguments, validation and sizes as sawkv_naive_int4_append; placement
 * outside the two values, or T > N_pg*P in token order, is SAWKV_EINVAL.
 */
enum {
  SAWKV_PLACE_SLOTS = 0,
  SAWKV_PLACE_TOKEN_ORDER = 1
};

int sawkv_append_pattern_control(const void* k, const void* v,
                                 int64_t k_stride, int64_t v_stride,
                                 const int64_t* slot_mapping, int64_t T,
                                 int32_t H, int32_t D,
                                 void* k_codes, void* v_codes,
                                 void* k_scales, void* v_scales,
                                 int64_t N_pg, int32_t P,
                                 int32_t placement,
                                 void* stream);

/*
 * Decode attention over the paged INT4 pools: one new query token per
 * sequence attends to every cached token of its sequence. This is the consumer
 * the pages fuse dequantisation into (ainews.cool, "技术深度解析" item 3:
 * dequantisation normally fused with the attention kernel; youngju.dev
 * English page, "Why the KV Cache Is the Real Bottleneck": paged layouts and
 * fused attention must be kept). Computed, for sequence b and query head j
 * (KV head j / G, G = Hq / H):
 *
 *   K_t, V_t = the dequantised rows of token t in the original basis
 *              (q * s, then the inverse rotation for rotated tensors)
 *   out[b][j] = sum_t softmax_t(sm_scale * q[b][j] . K_t) V_t,  fp16
 *
 * over t < min(context_lens[b], max_context); token t lives in page
 * block_tables[b][t / P] at offset t % P. A page id < 0 or >= N_pg masks the
 * page's tokens (nothing is read there); an empty or fully masked context
 * gives a zero row. Keys are never un-rotated: the query is rotated once,
 * since the rotation is orthogonal (youngju.dev, "The Rotation Trick").
 *
 *   q             fp16 [B][Hq][D]; sequence b's row starts at q + b*q_stride
 *                 elements (q_stride >= Hq*D, a multiple of 8)
 *   pools         as written by sawkv_quantize_append with the same h and
 *                 rot_mode (SAWKV_ROT_K: V naive; SAWKV_ROT_KV: both rotated)
 *   block_tables  int32 [B][bt_stride], bt_stride >= ceil(max_context / P);
 *                 entries past a sequence's last page are never read
 *   context_lens  int32 [B], device memory; values above max_context are
 *                 cut to max_context, negative values count as 0
 *   max_context   also sizes the split of the contexts (chunks of up to
 *                 1024 tokens, or, from B x ceil(max_context / 16) >= 40960
 *                 with B <= 1024, equal ranges of 16-token steps over the
 *                 device's resident waves; for an odd H also at least 128
 *                 such steps per wave): pass the batch's longest context,
 *                 not a loose capacity bound
 *   out           fp16 [B][Hq][D] contiguous
 *   workspace     device memory of at least the size that
 *                 sawkv_decode_attention_workspace_size reports for the same
 *                 B, Hq, H, D, max_context; 256-byte aligned; owned by the
 *                 caller and overwritten by the call (one call at a time per
 *                 workspace)
 * Supported: D = 128; Hq / H in {1, 2, 4, 8}; H <= 256; P a multiple of 16;
 * h in {16, 32, 64, 128}; N_pg < 2^31; max_context <= 2^30; B <= 2^24
 * (SAWKV_EUNSUPPORTED otherwise). B == 0 returns SAWKV_OK without reading
 * any pointer. Numerics: float32 accumulation from exact products of the
 * INT4 codes with fp16 hi + lo splits of the query and of the softmax
 * weights; the result is within a few fp16 ulps of the exact attention.
 */
int sawkv_decode_attention_workspace_size(int64_t B, int32_t Hq, int32_t H, int32_t D,
                                          int64_t max_context, size_t* bytes);

int sawkv_decode_attention(const void* q, int64_t q_stride,
                           const void* k_codes, const void* v_codes,
                           const void* k_scales, const void* v_scales,
                           int64_t N_pg, int32_t P,
                           const int32_t* block_tables, int64_t bt_stride,
                           const int32_t* context_lens,
                           int64_t B, int32_t Hq, int32_t H, int32_t D,
                           int64_t max_context, float sm_scale,
                           int32_t h, int32_t rot_mode,
                           void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * sawkv_decode_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, validation and result as
 * sawkv_decode_attention, without the workspace arguments. The partials live
 * in a static device array of SAWKV_NOALLOC_MAX_BYTES inside the library, one
 * copy per GPU, held until the process ends; its address is looked up on the
 * first call on a device (the device of `stream`). The call allocates and
 * frees nothing.
 *   - Sizes whose workspace (sawkv_decode_attention_workspace_size) exceeds
 *     SAWKV_NOALLOC_MAX_BYTES return SAWKV_EUNSUPPORTED, nothing launched
 *     (128 MiB holds e.g. 256 sequences of up to 8000 tokens with 32 query
 *     heads, or 64 sequences of 32768).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (on different streams, or from different threads
 *     without ordering) race and give undefined results. Calls ordered on one
 *     stream are safe. Nothing in the array needs to start at zero.
 */
#define SAWKV_NOALLOC_MAX_BYTES ((size_t)128 << 20)

int sawkv_decode_attention_noalloc(const void* q, int64_t q_stride,
                                   const void* k_codes, const void* v_codes,
                                   const void* k_scales, const void* v_scales,
                                   int64_t N_pg, int32_t P,
                                   const int32_t* block_tables, int64_t bt_stride,
                                   const int32_t* context_lens,
                                   int64_t B, int32_t Hq, int32_t H, int32_t D,
                                   int64_t max_context, float sm_scale,
                                   int32_t h, int32_t rot_mode,
                                   void* out, void* stream);

/* Static text for a status code (never NULL). */
const char* sawkv_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* sawkv_last_error(void);

/* SAWKV_VERSION of the built library. */
int sawkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAWKV_H */
