// Internal helpers shared by the kernels and the runtime of libtiletask.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "tiletask.h"

namespace tt {

// Thread-local message for tt_last_error(). Returns `code` so call sites can
// write `return fail(TT_ERR_ARG, "...")`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define TT_HIP_TRY(expr)                                                        \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ != hipSuccess)                                                       \
      return ::tt::fail(TT_ERR_HIP, "%s failed: %s (%s:%d)", #expr,             \
                        hipGetErrorString(e_), __FILE__, __LINE__);             \
  } while (0)

// Checks the launch that was just issued.
inline int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TT_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return TT_OK;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace tt
