// The attention kernels at head dim 512 (attn_wide.hpp), compiled apart
// from the other head dims.  Groups of up to 32 query rows per (b, kv head)
// (decode, short query blocks) take the kernel that splits the head dim
// across the four waves of a workgroup, 32 rows per workgroup; larger groups
// (prefill) the one whose eight waves each own 16 rows over the whole head
// dim, 128 rows per workgroup sharing each K/V tile.  Both run dense or
// paged, one pass or split partials.
#include "attn_wide.hpp"
#include "launch.hpp"

namespace gqa_host {

template <bool PAGED, bool PARTIAL>
gqa_status_t dispatch_wide(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  args.spw = 1;
  if (rows > gqa::WideCfg::ROWS) {
    using C = gqa::WideRowsCfg;
    return launch_grid(&gqa::attn_wide_rows_kernel<PAGED, PARTIAL>, 0, C::NW * 64, args, rows,
                       C::ROWS, stream);
  }
  using C = gqa::WideCfg;
  return launch_grid(&gqa::attn_wide_kernel<PAGED, PARTIAL>, C::LDS_BYTES, C::NW * 64, args, rows,
                     C::ROWS, stream);
}

template gqa_status_t dispatch_wide<false, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<false, true>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<true, false>(gqa::AttnArgs, int64_t, hipStream_t);
template gqa_status_t dispatch_wide<true, true>(gqa::AttnArgs, int64_t, hipStream_t);

}  // namespace gqa_host
