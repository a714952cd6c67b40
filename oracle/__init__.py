"""fp64 CPU oracle for the grouped-query attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the GPU path: no kernels, helpers, tables or
pre/post-processing.  Its inputs are plain numpy arrays.

Every function here is the plain (non-online) definition written out in
float64, following the pages cited in each docstring:

* AstrAI commit log (gitea, ViperEkura/AstrAI) -- the commit that packs
  HB = min(G, warps) query heads per block, the paged-attention commits and
  the paged decode fix (new-K / new-V pointers for the newest tokens);
* kernbench2 commit log, src/kernbench/benches (git.ywkang.dev) -- the
  tile-granular ring-KV commit (persistent (m, l, O) state, TILE_S_KV) and
  the 2-D mesh all-reduce-mlo commit (associativity of the merge);
* nvfp4-megamoe-kernel commit log, dsv4/kernels/attention (sweetapi.com) --
  the sink-bias, zero-initialised-P, padded-N/kv_len, multi-tile FA2 and
  normalise-once commits.

Parity status: every function is pinned by `tests/test_oracle_pins.py`
(closed forms, invariants, brute force, torch SDPA cross-check).  Nothing
is pinned to printed attention outputs, because the pages print none.
"""

from .attention import (  # noqa: F401
    attention_fp64,
    attention_rows_fp64,
    softmax_weights_fp64,
    splitkv_partials_fp64,
    merge_partials_fp64,
    merge_pair_fp64,
    gather_paged_fp64,
    paged_attention_fp64,
    paged_attention_rows_fp64,
    paged_append_fp64,
)
