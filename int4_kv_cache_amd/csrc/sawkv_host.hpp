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

}  // namespace host
}  // namespace sawkv
