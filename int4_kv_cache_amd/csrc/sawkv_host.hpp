// Host-side helpers shared by the translation units of libsawkv: the
// per-thread error text behind sawkv_last_error() and pointer alignment.
#pragma once

#include <stdint.h>

namespace sawkv {
namespace host {

extern thread_local char g_err[512];

// Formats the detail text for sawkv_last_error() and returns `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the detail text and returns SAWKV_OK.
int ok();

bool aligned(const void* p, uintptr_t a);

// Size and pointer checks shared by the append / gather style entry points
// (write path, read-back and the controls): status SAWKV_OK or an error with
// detail text.
int check_geometry(int64_t T, int32_t H, int32_t D, int64_t N_pg, int32_t P, int32_t h,
                   int32_t rot_mode, const int64_t* slots);
// Input tensor: stride (elements between tokens) must be in [H*D, 2^26) and a
// multiple of 8; pointers 16-byte aligned, pool pointers non-null.
int check_tensor(const char* name, const void* x, int64_t stride, const void* codes,
                 const void* scales, int32_t H, int32_t D);
// Contiguous output rows of a read-back: pointers 16-byte aligned, pool
// pointers non-null.
int check_output(const char* name, const void* out, const void* codes, const void* scales);

// Whether an append of both tensors dispatches their blocks alternately
// (large inputs) rather than every first-tensor block first.
bool alternate_tensors(int64_t T, int32_t H, int32_t D);

// Kernel-table index of a tensor: 0 = not rotated, 1..4 = h 16/32/64/128.
int hb_index(int32_t h, bool rot);

}  // namespace host
}  // namespace sawkv
