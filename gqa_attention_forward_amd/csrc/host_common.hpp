// Host-side helpers shared by the C ABI source and the kernel dispatch
// sources (defined once, in gqa_api.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.hpp"
#include "gqa.h"

namespace gqa_host {

// Records the thread-local error message and returns `st`.
gqa_status_t fail(gqa_status_t st, const char* fmt, ...);
// GQA_ERR_HIP with the launch error, if the last launch failed.
gqa_status_t check_launch(const char* what);
// Compute units of the current device (queried once per device).
int device_cus();

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The kernel form for `rows` query rows per (b, kv head) at head dim D
// (instantiated in dispatch_d<D>.hip).
template <int D, bool PAGED, bool PARTIAL>
gqa_status_t dispatch_rows(gqa::AttnArgs args, int64_t rows, hipStream_t stream);

// The same at head dim 512 (dispatch_d512.hip): one form for every row count.
template <bool PAGED, bool PARTIAL>
gqa_status_t dispatch_wide(gqa::AttnArgs args, int64_t rows, hipStream_t stream);

#define GQA_EXTERN_DISPATCH(D)                                                              \
  extern template gqa_status_t dispatch_rows<D, false, false>(gqa::AttnArgs, int64_t,       \
                                                              hipStream_t);                 \
  extern template gqa_status_t dispatch_rows<D, false, true>(gqa::AttnArgs, int64_t,        \
                                                             hipStream_t);                  \
  extern template gqa_status_t dispatch_rows<D, true, false>(gqa::AttnArgs, int64_t,        \
                                                             hipStream_t);                  \
  extern template gqa_status_t dispatch_rows<D, true, true>(gqa::AttnArgs, int64_t, hipStream_t);

}  // namespace gqa_host
