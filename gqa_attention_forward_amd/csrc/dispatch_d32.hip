// The attention kernels at head dim 32: explicit instantiations of the
// per-call form choice (launch.hpp), compiled apart from the other head dims.
#include "launch.hpp"

namespace gqa_host {
template gqa_status_t dispatch_rows<32, false, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_rows<32, false, true>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_rows<32, true, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_rows<32, true, true>(gqa::AttnArgs, int64_t, hipStream_t);
}  // namespace gqa_host
