// The attention kernel at head dim 512 (attn_wide.hpp: the head dim split
// across the four waves of a workgroup), compiled apart from the other head
// dims.  Every form -- dense or paged, one pass or split partials -- takes
// 32 query rows per workgroup.
#include "attn_wide.hpp"
#include "launch.hpp"

namespace gqa_host {

template <bool PAGED, bool PARTIAL>
gqa_status_t dispatch_wide(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  using C = gqa::WideCfg;
  args.spw = 1;
  return launch_grid(&gqa::attn_wide_kernel<PAGED, PARTIAL>, C::LDS_BYTES, C::NW * 64, args, rows,
                     C::ROWS, stream);
}

template gqa_status_t dispatch_wide<false, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<false, true>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<true, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<true, true>(gqa::AttnArgs, int64_t, hipStream_t);

}  // namespace gqa_host
