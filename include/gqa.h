/*
 * gqa.h -- C ABI of libgqa.so: grouped-query attention forward on AMD MI355X
 * (CDNA4, gfx950).
 *
 *   O = softmax(scale * Q K^T + mask [+ sink]) V
 *
 * Hq query heads share Hkv = Hq / G key/value heads; query head h reads
 * kv head h / G (consecutive groups).  Inputs and output are bf16,
 * accumulation is fp32.  Sources for the operation's definition:
 *
 *  - AstrAI commit log (gitea, ViperEkura/AstrAI): the commit that packs
 *    HB = min(G, warps) query heads per block so each K/V tile streams once
 *    per block; the AttentionParams commits (per-dimension strides, NULL
 *    meaning an optional path is off, q-head/kv-head divisibility and
 *    head-dim contiguity checks, split-KV scratch validated at the binding);
 *    the paged-KV commits (KVSource contiguous vs paged, int32 page tables).
 *  - nvfp4-megamoe-kernel commit log (dsv4/kernels/attention): the commit
 *    that passes the true kv length apart from the padded one; the sink-bias
 *    commit (sink already in the scaled domain); the zero-initialised-P
 *    commit; the multi-tile FA2 and normalise-once commits; the T-stride
 *    commit (query-row stride distinct from head stride); the pure C API +
 *    ctypes loader commits; the single-launch batched decode commit.
 *  - kernbench2 commit log (src/kernbench/benches): the tile-granular
 *    ring-KV and tile-sweep commits (persistent (m, l, O) merged tile by
 *    tile, TILE_S_KV = 1024) and the 2-D mesh all-reduce-mlo commit (the
 *    merge is associative).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers; bf16 tensors are raw 16-bit
 *    bfloat16 values.  Strides are in ELEMENTS; the head-dim stride is 1.
 *  - Dense layout: Q/O [B, Hq, Sq, d], K/V [B, Hkv, Skv, d] addressed by the
 *    (b, h, s) strides passed in `*_stride[3]` (host arrays).
 *  - kv_len: device int32 [B] giving each sequence's true key count, or NULL
 *    meaning Skv for every sequence.  Keys at or past kv_len[b] are never read
 *    into the max, the sum or P.V (padding may hold anything, NaN included).
 *    Values outside [0, Skv] are clamped on the device.
 *  - sink: device fp32 [Hq] of per-head sink logits already in the scaled
 *    domain (an extra softmax column with no value row: it enters the max
 *    and the denominator, is never multiplied by scale), or NULL for none.
 *  - causal: 0 or 1.  Causal masking is aligned bottom-right: query row i of
 *    a sequence with q_len rows and n keys sees keys j <= n - q_len + i.
 *    With q_len == n this is "row i sees keys 0..i".
 *  - A row that sees no key and has no sink gets O = 0.
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).
 *  - A call with no output rows (B * Sq == 0; for paged B, total_q or
 *    max_q_len == 0) is a no-op that returns GQA_OK after the scalar checks;
 *    its pointers are not examined and may be NULL.
 *  - Base pointers must be 16-byte aligned and the (b, h, s) strides of
 *    bf16 tensors multiples of 8 elements, else GQA_ERR_UNSUPPORTED.  The
 *    stride between consecutive key rows of K and V (dense s stride, paged
 *    kv_stride_row, the append form's new_stride_t) must be below 2^25
 *    elements, else GQA_ERR_UNSUPPORTED: a 64-key tile is addressed with
 *    32-bit byte offsets from its first row.
 *    d must be 32, 64, 128, 256 or 512, else GQA_ERR_UNSUPPORTED (the
 *    AstrAI commit log's kernels cover prefill at head dim 32 and decode at
 *    256 besides 64 and 128; the nvfp4-megamoe-kernel commit log's sweep
 *    reaches 512).  The in-kernel merge and the append form take d up to
 *    256.  A launch whose grid would exceed 2^32 - 1
 *    work-items (one dispatch's limit) also returns GQA_ERR_UNSUPPORTED.
 *
 * Ownership: the caller owns all memory and keeps it alive until the work
 * enqueued on `stream` completes.  The library never allocates, frees,
 * synchronises or reads device memory from the host, keeps no pointer after
 * returning, and is reentrant.  Launches are asynchronous and are the only
 * stream operations (no memset or copy), so every entry point can be
 * captured into a HIP graph; a kernel's first launch in the process sets its
 * LDS limit, so call each form once before capturing it.
 *
 * Errors: every function returns a gqa_status_t.  All validation happens
 * before anything is enqueued: on any status other than GQA_OK or
 * GQA_ERR_HIP, nothing was launched and O/workspace are untouched.
 * GQA_ERR_HIP reports a failed launch; for two-kernel calls the first
 * kernel may already be enqueued.  gqa_last_error() gives a message for
 * the last failing call on the calling thread.  Nothing aborts, prints or
 * throws across this boundary.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 2

typedef int32_t gqa_status_t;

#define GQA_OK 0
#define GQA_ERR_INVALID_ARGUMENT 1 /* NULL required pointer, bad dims, Hq % Hkv != 0, bad flag */
#define GQA_ERR_UNSUPPORTED 2      /* d not 32/64/128/256/512, misaligned pointer or stride,
                                      page_size != 64, a group beyond the append/fused limits,
                                      a grid beyond 2^32 - 1 work-items */
#define GQA_ERR_WORKSPACE 3        /* workspace NULL or too small; ticket array too small */
#define GQA_ERR_HIP 4              /* a HIP launch failed; message from hipGetErrorString */

/* GQA_ABI_VERSION of the built library. */
int32_t gqa_abi_version(void);

/* Thread-local message of the last failing call on this thread ("" if none).
 * Valid until the next gqa_* call on the same thread. */
const char* gqa_last_error(void);

/*
 * Bytes of split-KV workspace for B*Hq*Sq query rows over Skv keys split in
 * tiles of tile_s_kv keys: n_split = ceil(Skv / tile_s_kv) partial states
 * (m, l, O~) per row, each (d + 2) fp32 values, rounded up to 256 bytes.
 * Writes 0 when tile_s_kv == 0 (one pass needs no workspace).
 *
 * Workspace layout (also the input of gqa_attention_splitkv_merge), with
 * rows r = (b * Hq + h) * Sq + i:
 *   ml[r][s]    : float2 {m_s, l_s}         at byte 0
 *   ot[r][s][d] : float  O~_s (un-normalised) at byte 8 * rows * n_split
 * m_s is the split's max of scale*q.k (natural-log domain; -inf when the
 * split holds no visible key), l_s = sum_j exp(s_j - m_s), O~_s =
 * sum_j exp(s_j - m_s) v_j (nvfp4-megamoe-kernel commit log, multi-tile FA2
 * commit: P stays un-normalised; kernbench2 benches commit log, tile-granular
 * ring-KV commit: the persistent (m, l, O) state).
 * gqa_attention_splitkv_partial writes every state (O~ = 0 for an empty one).
 * After gqa_attention_prefill or gqa_attention_paged with tile_s_kv > 0 the
 * workspace is scratch: an empty state's O~ may be left unwritten there, as
 * the library's merge gives it weight 0 without reading it.
 */
gqa_status_t gqa_attention_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv,
                                          int64_t d, int32_t tile_s_kv, size_t* bytes);

/*
 * Dense prefill (any Sq >= 1), one query row per (b, h, i).
 *  tile_s_kv == 0 : one pass, one kernel; workspace may be NULL.
 *  tile_s_kv  > 0 : split-KV -- keys cut into tiles of tile_s_kv (a multiple
 *                   of 64), one partial state per tile and row, then a merge
 *                   kernel; needs the workspace above.  Same result up to
 *                   rounding (the merge is associative; a single tile equals
 *                   one pass -- kernbench2 benches commit log, tile sweep).
 */
gqa_status_t gqa_attention_prefill(const void* q, const int64_t q_stride[3],
                                   const void* k, const int64_t k_stride[3],
                                   const void* v, const int64_t v_stride[3],
                                   void* o, const int64_t o_stride[3],
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv,
                                   int32_t d, const int32_t* kv_len, float scale,
                                   const float* sink, int32_t causal, int32_t tile_s_kv,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Single-token decode with split-KV (Sq = 1 implied; causal is a no-op for
 * one trailing query).  tile_s_kv must be a positive multiple of 64
 * (1024 is the pages' TILE_S_KV).  Launches the partial kernel, then the
 * merge kernel, on `stream`.  Q/O strides as for prefill (the s stride is
 * unused but must still be a multiple of 8).
 */
gqa_status_t gqa_attention_decode_splitkv(const void* q, const int64_t q_stride[3],
                                          const void* k, const int64_t k_stride[3],
                                          const void* v, const int64_t v_stride[3],
                                          void* o, const int64_t o_stride[3],
                                          int32_t B, int32_t Hq, int32_t Hkv, int32_t Skv,
                                          int32_t d, const int32_t* kv_len, float scale,
                                          const float* sink, int32_t tile_s_kv,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * A split size for gqa_attention_decode_splitkv (or the paged form with one
 * query token per sequence) when the caller has no better one: the smallest
 * power of two of at least 128 keys for which B * Hkv * ceil(Skv / tile)
 * work units are at most the current device's compute units (capped at
 * 8192).  Short contexts then spread over the chip instead of leaving most
 * of it idle: measured on MI355X at B = 1 and 4, Hq 32, Hkv 8, d 128 over
 * 1K-32K keys it was within 3% of the best split size at every point (B = 1,
 * 1K keys: 9.0 us against 17.8 us with TILE_S_KV = 1024).  Host only; writes
 * *tile_s_kv.  B, Hkv >= 1 and Skv >= 0, else GQA_ERR_INVALID_ARGUMENT.
 */
gqa_status_t gqa_attention_decode_tile(int32_t B, int32_t Hkv, int32_t Skv, int32_t* tile_s_kv);

/*
 * gqa_attention_decode_splitkv in one launch: the split-KV partial states
 * are merged inside the partial kernel instead of by a second kernel.  The
 * pattern is the AstrAI commit log's scale-ring epilogue (after a fence, a
 * counter elects the last block, which finishes the reduction with no extra
 * launch).  Each workgroup writes its partial states, releases them
 * device-wide and takes a ticket for its (b, kv head, q-tile); the workgroup
 * that draws the last ticket merges every split of those rows exactly as the
 * merge kernel does (sink included, one normalisation) and resets the
 * ticket.  Same arguments as gqa_attention_decode_splitkv, plus:
 *
 *  tickets   : device int32 array of n_tickets >= B * Hq entries, all ZERO
 *              before the first call; every call leaves them zero.  Calls
 *              that overlap in time must not share it (nor the workspace).
 *              Too few entries: GQA_ERR_WORKSPACE.
 *
 * Group sizes G = Hq / Hkv up to 32, else GQA_ERR_UNSUPPORTED.
 */
gqa_status_t gqa_attention_decode_splitkv_fused(
    const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
    const void* v, const int64_t v_stride[3], void* o, const int64_t o_stride[3], int32_t B,
    int32_t Hq, int32_t Hkv, int32_t Skv, int32_t d, const int32_t* kv_len, float scale,
    const float* sink, int32_t tile_s_kv, void* workspace, size_t workspace_bytes,
    int32_t* tickets, int64_t n_tickets, void* stream);

/*
 * gqa_attention_decode_splitkv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, and the same
 * kernels and result.  The split-KV partial states go into a scratch buffer
 * of GQA_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU it runs on, kept until the process ends; the call itself
 * allocates nothing.  A call whose partial states,
 * gqa_attention_workspace_size(B, Hq, 1, Skv, d, tile_s_kv) bytes, exceed
 * that size returns GQA_ERR_WORKSPACE before anything is enqueued (the
 * decode of 16 sequences x 32 heads x 8192 keys in splits of 1024 needs
 * 2,129,920 bytes).  Every call on one GPU shares its buffer, which keeps
 * the last call's contents (nothing in it needs to start at zero): calls
 * ordered on one stream are safe, calls that overlap in time on one GPU
 * (other streams, other threads) race and give wrong results.  The first
 * call on each device looks the buffer's address up (hipGetSymbolAddress)
 * with that device current; make it once outside graph capture.
 */
#define GQA_NOALLOC_SCRATCH_BYTES (8u << 20)
gqa_status_t gqa_attention_decode_splitkv_noalloc(
    const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
    const void* v, const int64_t v_stride[3], void* o, const int64_t o_stride[3], int32_t B,
    int32_t Hq, int32_t Hkv, int32_t Skv, int32_t d, const int32_t* kv_len, float scale,
    const float* sink, int32_t tile_s_kv, void* stream);

/*
 * The two phases of split-KV on their own, for callers that place the
 * partial states themselves (for instance KV sharded across devices, with
 * the partials gathered before one merge; the merge is associative -- see
 * the kernbench2 2-D mesh all-reduce-mlo commit).
 *
 * _partial: writes n_split = ceil(Skv / tile_s_kv) partial states per query
 *   row into `workspace` (layout above).  The sink is NOT applied here.
 * _merge:   reads n_split partial states per row from `workspace` and
 *   writes O = sum_s O~_s e^(m_s - M) / (e^(sink - M) + sum_s l_s e^(m_s - M)),
 *   M = max(sink, max_s m_s), normalised exactly once, as bf16.  Splits
 *   with m_s = -inf weigh 0; a row with M = -inf gets 0.
 */
gqa_status_t gqa_attention_splitkv_partial(const void* q, const int64_t q_stride[3],
                                           const void* k, const int64_t k_stride[3],
                                           const void* v, const int64_t v_stride[3],
                                           int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq,
                                           int32_t Skv, int32_t d, const int32_t* kv_len,
                                           float scale, int32_t causal, int32_t tile_s_kv,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

gqa_status_t gqa_attention_splitkv_merge(const void* workspace, size_t workspace_bytes,
                                         void* o, const int64_t o_stride[3], int32_t B,
                                         int32_t Hq, int32_t Sq, int32_t d, int32_t n_split,
                                         const float* sink, void* stream);

/*
 * Ragged-Q, paged-KV attention (AstrAI commit log: packed 3-D inference
 * tensors with a KV cache, int32 page tables, KVSource contiguous vs paged).
 *
 *  q / o        : packed bf16 [total_q, Hq, d]; token t of sequence b is row
 *                 cu_seqlens_q[b] + i, i < q_len_b = cu[b+1] - cu[b].
 *                 Strides (t, h) in elements.
 *  cu_seqlens_q : device int32 [B + 1], cu[0] = 0, non-decreasing,
 *                 every q_len_b <= max_q_len.
 *  k_cache/v_cache : bf16 page pools; key row j of sequence b lives in page
 *                 page_table[b * max_pages_per_seq + j / page_size] at in-page
 *                 row j % page_size, kv head g, addressed as
 *                 page * kv_stride_page + row * kv_stride_row + g * kv_stride_h.
 *                 Default layout [n_pages][page_size][Hkv][d].
 *  page_table   : device int32 [B, max_pages_per_seq]; entries past a
 *                 sequence's last page are never read.
 *  kv_len       : device int32 [B], required.
 *  page_size    : must be 64.
 *  max_q_len    : host bound on q_len_b that sizes the grid (no device read).
 *  tile_s_kv    : 0 = one pass per (sequence, kv head, q-tile); > 0 (a
 *                 multiple of 64) = split-KV over key tiles of that size with
 *                 partial states in `workspace`, merged by a second kernel.
 *                 The workspace is gqa_attention_workspace_size(1, Hq,
 *                 total_q, max_pages_per_seq * page_size, d, tile_s_kv)
 *                 bytes; partial-state rows are r = h * total_q + t.
 * Page ids are trusted: an id outside the pool is undefined behaviour.
 */
gqa_status_t gqa_attention_paged(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                                 const int32_t* cu_seqlens_q, const void* k_cache,
                                 const void* v_cache, int64_t kv_stride_page,
                                 int64_t kv_stride_row, int64_t kv_stride_h,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 const int32_t* kv_len, void* o, int64_t o_stride_t,
                                 int64_t o_stride_h, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t d, int32_t page_size, int32_t total_q,
                                 int32_t max_q_len, float scale, const float* sink,
                                 int32_t causal, int32_t tile_s_kv, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * gqa_attention_paged with the query tokens' own K/V appended in the same
 * launch (AstrAI commit log, the paged decode fix: the decode kernel takes
 * the newest tokens' K/V from separate new-K/new-V pointers instead of the
 * cache).  Besides the gqa_attention_paged arguments:
 *
 *  k_new / v_new : bf16 [total_q, Hkv, d] packed like q, strides (t, h) in
 *                 elements (new_stride_t, new_stride_h; d contiguous; the
 *                 same strides for both; new_stride_t below 2^25).  Token i of sequence b (row
 *                 cu_seqlens_q[b] + i) holds key row j = kv_len[b] - q_len_b
 *                 + i of that sequence: kv_len counts the new tokens, and
 *                 kv_len[b] >= q_len_b (tokens that would land before key
 *                 row 0 are dropped).
 *  k_cache / v_cache : written as well as read: each row j above is stored
 *                 into page page_table[b, j / 64], in-page row j % 64, kv head
 *                 g, so the page must be allocated in page_table.  No other
 *                 cache row is written.  The cache must not overlap k_new,
 *                 v_new, q or o.
 *
 * The output equals writing those rows into the cache first and then calling
 * gqa_attention_paged; the attention reads them from k_new / v_new, so no
 * cache row is read and written in the same launch.  Supported for up to 32
 * query rows per kv head: max_q_len * (Hq / Hkv) <= 32 (decode and short
 * query blocks; the stream kernel), else GQA_ERR_UNSUPPORTED.
 */
gqa_status_t gqa_attention_paged_append(
    const void* q, int64_t q_stride_t, int64_t q_stride_h, const int32_t* cu_seqlens_q,
    void* k_cache, void* v_cache, int64_t kv_stride_page, int64_t kv_stride_row,
    int64_t kv_stride_h, const int32_t* page_table, int32_t max_pages_per_seq,
    const int32_t* kv_len, const void* k_new, const void* v_new, int64_t new_stride_t,
    int64_t new_stride_h, void* o, int64_t o_stride_t, int64_t o_stride_h, int32_t B, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t page_size, int32_t total_q, int32_t max_q_len, float scale,
    const float* sink, int32_t causal, int32_t tile_s_kv, void* workspace,
    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
