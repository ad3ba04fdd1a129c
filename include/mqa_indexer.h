/*
 * mqa_indexer.h -- C ABI of the MI355X (gfx950) lightning-indexer logits library
 * (libmqa_indexer.so).
 *
 * The op (aiter PR 5047 page and aiter PR 5046 page, section "Motivation"):
 *
 *   logits[m, n] = sum_h relu(<Q[m,h,:], K[n,:]>) * kv_scale[n] * weights[m,h]
 *
 * for n inside row m's window and -inf elsewhere, with Q and K in fp8 e4m3fn
 * (OCP E4M3, finite-only), a per-token fp32 K dequant scale, 32 heads and head
 * dim 128.
 *
 * Conventions shared by every call:
 *   - All array arguments are DEVICE pointers owned by the caller, contiguous,
 *     row-major, on the current HIP device.  fp8 arrays are passed as raw
 *     bytes (uint8_t).  Data pointers must be 16-byte aligned, int32 arrays
 *     4-byte aligned.
 *   - The library allocates no device memory.  Between calls it keeps only the
 *     per-thread last-error string, a per-device cache of the gfx950 check
 *     and, for paged_mqa_topk_decode_noalloc, its static scratch array (part
 *     of the loaded code object, not an allocation) and that array's
 *     per-device address.
 *   - Work is enqueued asynchronously on `stream` (NULL = the null stream).  A
 *     call returns before the kernel finishes; outputs are valid once the
 *     stream has been synchronised.
 *   - Return value: MQA_OK (0) or a negative MQA_ERR_* code; on error nothing is
 *     enqueued and mqa_last_error() describes why.  No call aborts the process
 *     and no call falls back to another implementation.
 *   - Integer arrays that live on the device (context_lens, block_tables,
 *     cu_seqlen_ks/ke) cannot be inspected without a synchronisation, so their
 *     documented ranges are preconditions, not checked.  Windows are clamped
 *     into the output row, so no window value can make the kernel write
 *     outside `logits`.
 */
#ifndef MQA_INDEXER_H
#define MQA_INDEXER_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQA_OK 0
#define MQA_ERR_INVALID_ARG (-1) /* NULL/misaligned pointer, bad size, bad tunable */
#define MQA_ERR_UNSUPPORTED (-2) /* shape or device outside mqa_is_supported()    */
#define MQA_ERR_LAUNCH (-3)      /* the HIP runtime rejected the kernel launch     */
#define MQA_ERR_DEVICE (-4)      /* no usable HIP device / device query failed     */

/*
 * Launch tunables.  0 in any field means "use the host heuristic"; every
 * override changes only how the work is split, never a result bit (outputs are
 * bitwise identical across all valid overrides).  Pass NULL for all-heuristic.
 * (Both pages, "Technical Details": the row block, the column / KV split and
 * the wave count are host-chosen and overridable.)
 *
 *   prefill:
 *     ring_depth   1 = every wave streams its own K into registers; 2..7 =
 *                  a workgroup of 4 waves shares each K step through an LDS
 *                  ring of that many steps (head_dim 128 only: 32 heads with
 *                  4 rows per wave, 64 heads with 2 rows and 128 heads with
 *                  1 row at depth 3 or 4; the default at head_dim 128, at
 *                  depth 4, for all but small problems); 0 = the heuristic
 *     block_m      query rows per wave: 1, 2, 4 or 8 (with the ring 4, 2 or
 *                  1 at 32, 64 or 128 heads)
 *     split_n      workgroups per row block along the columns, >= 1
 *     num_warps    waves per workgroup, 1..4: they split the column range
 *                  (4 with the ring, where they split the rows instead)
 *     reverse_rows 1 = dispatch row blocks high-m first, -1 = natural order
 *     (setting block_m or num_warps selects the per-wave kernel unless
 *     ring_depth asks for the ring)
 *   decode:
 *     rows_per_block  next_n rows each wave computes, 1..4 (clamped to
 *                     next_n); a workgroup has ceil(next_n / rows_per_block)
 *                     such waves, all fed from one K stream
 *     split_kv        workgroups per sequence along KV, >= 1
 *     ring_depth      cache blocks each workgroup keeps in its LDS ring
 *                     (requests run ring_depth - 1 blocks ahead), 2..7
 *     (num_warps must be 0 for decode)
 */
typedef struct mqa_tunables {
    int block_m;
    int split_n;
    int num_warps;
    int reverse_rows;
    int rows_per_block;
    int split_kv;
    int ring_depth;
} mqa_tunables;

/*
 * Support gate (both pages, "Technical Details": callers ask before routing a
 * shape to these kernels and go elsewhere instead of failing).  Supported:
 * num_heads 32, 64 or 128 (the head counts the issue page about next_n tiling
 * sweeps) with head_dim 128 or 64 (the head dims of the aiter PR 5046 page's
 * test sweep, "Test Plan").  kv_block_size: 0 asks about prefill; 1, 16, 64 or
 * 128 about paged decode with blocks of that many tokens (at every head count
 * and head dim).  Returns 1 if the current HIP device is gfx950 and the shape
 * is supported, else 0.  Never fails.
 */
int mqa_is_supported(int num_heads, int head_dim, int kv_block_size);

/*
 * Prefill logits over a contiguous, already-gathered K (aiter PR 5046 page,
 * "Motivation" and "Technical Details").
 *
 *   q_fp8        [M, num_heads, head_dim]  fp8 e4m3fn (head_dim 64 or 128)
 *   k_fp8        [N, head_dim]             fp8 e4m3fn
 *   kv_scale     [N]                       fp32, >= 0
 *   weights      [M, num_heads]            fp32
 *   cu_seqlen_ks [M]                       int32
 *   cu_seqlen_ke [M]                       int32
 *   logits       [M, N]                    fp32, written
 *
 * Row m's window is  max(ks[m], 0) <= n < min(ke[m], N)  (empty when ke <= ks,
 * when ke <= 0 or when ks >= N).  clean_logits != 0: every other column of the
 * row is written -inf (the fused fill); clean_logits == 0: only the window is
 * written and all other elements keep their previous contents.
 * kv_scale must be >= 0 (the kernel applies it after the ReLU, once per column).
 * M == 0 or N == 0 is a successful no-op.  M, N < 0, M*N beyond int64 range,
 * NULL or misaligned pointers, or bad tunables -> MQA_ERR_INVALID_ARG; a shape
 * outside the gate -> MQA_ERR_UNSUPPORTED.
 */
int mqa_logits_prefill(const uint8_t *q_fp8, const uint8_t *k_fp8, const float *kv_scale,
                       const float *weights, const int32_t *cu_seqlen_ks,
                       const int32_t *cu_seqlen_ke, float *logits, int M, int N, int num_heads,
                       int head_dim, int clean_logits, const mqa_tunables *tun,
                       hipStream_t stream);

/*
 * Order of the K rows inside a cache block (kv_layout argument):
 *   MQA_KV_SLOT_MAJOR   slot s's head_dim bytes at byte s * head_dim of the
 *                       block
 *   MQA_KV_PRESHUFFLED  the preshuffled (16,16) cache that the aiter PR 5047
 *                       page ("Technical Details") pairs with 64-token blocks:
 *                       the block's slots in groups of 16; a group stores
 *                       16-byte column granule u (bytes 16u..16u+15 of each
 *                       row) of its 16 slots, slot by slot, before granule
 *                       u + 1.  Byte d of slot s is at
 *                       (s/16)*16*head_dim + (d/16)*256 + (s%16)*16 + d%16.
 *                       Needs kv_block_size 16, 64 or 128.
 * The scales follow the K rows in slot order in both layouts.
 */
#define MQA_KV_SLOT_MAJOR 0
#define MQA_KV_PRESHUFFLED 1

/*
 * Paged decode logits (aiter PR 5047 page, "Motivation" and "Technical
 * Details"; the next_n row bound is also spelled out on the issue page about
 * next_n tiling, "The ask").
 *
 *   q_fp8        [batch, next_n, num_heads, head_dim]  fp8 e4m3fn
 *   kv_cache     [num_blocks] blocks of kv_block_size * (head_dim + 4) bytes.
 *                Block i starts at byte i * kv_block_size * (head_dim + 4); its
 *                first kv_block_size * head_dim bytes are the fp8 K rows of
 *                its slots in the order kv_layout names (slot-major: slot s at
 *                byte s * head_dim), the remaining kv_block_size * 4 bytes the
 *                slots' fp32 dequant scales (slot s at byte
 *                kv_block_size * head_dim + 4 s).  For 64-token blocks a block
 *                is 8448 bytes, so every K row stays 16-byte aligned.
 *   weights      [batch * next_n, num_heads]  fp32
 *   context_lens [batch]                      int32
 *   block_tables [batch, max_blocks_per_seq]  int32; entry (b, i) is the
 *                physical block holding positions [i*bs, (i+1)*bs) of
 *                sequence b
 *   logits       [batch * next_n, max_model_len]  fp32, written
 *
 * Row r = b * next_n + j covers positions 0 <= p <= context_lens[b] - next_n + j
 * (none if that bound is negative).  clean_logits != 0 writes -inf at every
 * other position p < max_model_len of the row; clean_logits == 0 writes only
 * the window.
 * Preconditions (not checked, see above): 0 <= context_lens[b] <=
 * min(max_model_len, max_blocks_per_seq * kv_block_size); every table entry
 * with index < ceil(context_lens[b] / kv_block_size) lies in [0, num_blocks).
 * Entries past that are never read.  Scales must be >= 0.  Cache slots past a
 * sequence's context may hold any bytes (NaN included): they never reach an
 * output.
 * kv_block_size 1, 16, 64 or 128 at 32, 64 or 128 heads and head_dim 128 or
 * 64 (at head_dim 64 a block of bs tokens is bs * 68 bytes).  The ring_depth
 * tunable takes 2..7 with kv_block_size 64, 32 heads and head_dim 128, and
 * otherwise 0 or the layout's one depth (4 for kv_block_size 1, else 3).
 * kv_layout MQA_KV_SLOT_MAJOR or MQA_KV_PRESHUFFLED (the latter not with
 * kv_block_size 1).
 * batch == 0 or max_model_len == 0 is a successful no-op.  next_n outside 1..8,
 * a bad kv_layout, negative sizes, NULL or misaligned pointers ->
 * MQA_ERR_INVALID_ARG; a shape, block size or layout outside the gate ->
 * MQA_ERR_UNSUPPORTED.
 */
int paged_mqa_logits_decode(const uint8_t *q_fp8, const uint8_t *kv_cache, const float *weights,
                            const int32_t *context_lens, const int32_t *block_tables,
                            float *logits, int batch, int next_n, int num_heads, int head_dim,
                            int kv_block_size, int kv_layout, int num_blocks,
                            int max_blocks_per_seq, int max_model_len, int clean_logits,
                            const mqa_tunables *tun, hipStream_t stream);

/*
 * Row-wise top-k of a logits matrix: the selection that consumes the indexer
 * (index_topk 2048 or 512 on the aiter PR 5047 page, "Integration" and the
 * serving notes; the issue page about next_n tiling, "Setup").  The pages do
 * not define the selection order; this call uses one total order:
 *
 *   logits   [rows, cols]  fp32, 4-byte aligned
 *   indices  [rows, k]     int32, written
 *
 * Row r's output lists column indices by decreasing value, equal values by
 * increasing column; -inf and NaN entries are never listed (so the -inf
 * written outside each window by clean_logits = 1 excludes those positions);
 * -0.0 counts as equal to +0.0.  When a row has fewer than k listable entries
 * the rest of its output is -1.  1 <= k <= 2048.
 * rows == 0 is a successful no-op; cols == 0 writes all -1.  Negative sizes, k
 * out of range, NULL or misaligned pointers -> MQA_ERR_INVALID_ARG.
 */
int mqa_topk_indices(const float *logits, int rows, int cols, int k, int32_t *indices,
                     hipStream_t stream);

/*
 * mqa_topk_indices with a caller workspace: the same output for every input.
 * mqa_topk_indices gives each row to one workgroup, and one CU streams a row
 * at the rate its outstanding misses allow, so a few long rows leave most of
 * the GPU idle.  With the workspace, long rows (more than 8192 columns, 16-byte
 * aligned: cols a multiple of 4 and logits 16-byte aligned) are split over
 * several workgroups each when there are too few rows to fill the GPU: each
 * keeps the entries of its slice at or above the row's sampled threshold in
 * the row's workspace region, then one workgroup per row gathers and sorts
 * them; a row the sample misjudges is selected from its logits in full.  Other
 * shapes run the one-workgroup-per-row path.
 *
 *   workspace  DEVICE memory of at least mqa_topk_workspace_size(rows, cols)
 *              bytes (8 bytes per row and column plus 256 bytes per row),
 *              256-byte aligned, owned by the caller; contents on entry do not
 *              matter and are clobbered.  Calls that overlap on one workspace
 *              race.  NULL (any workspace_bytes) runs the one-workgroup-per-row
 *              path.
 *
 * Errors as for mqa_topk_indices, plus: a non-NULL workspace that is not
 * 256-byte aligned or is smaller than asked for -> MQA_ERR_INVALID_ARG.
 */
int mqa_topk_indices_ws(const float *logits, int rows, int cols, int k, int32_t *indices,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes mqa_topk_indices_ws needs for rows x cols (0 when rows or
 * cols is not positive, or the size would exceed 2^60).  Host-only, never
 * fails. */
size_t mqa_topk_workspace_size(int rows, int cols);

/*
 * Fused paged decode + row-wise top-k: the indices mqa_topk_indices would
 * return for the logits paged_mqa_logits_decode (clean_logits = 1) would
 * write, without writing those logits (the top-k is the indexer's consumer:
 * aiter PR 5047 page, "Integration"; writing the logits only to read them back
 * is the traffic this avoids).  Same arguments and preconditions as
 * paged_mqa_logits_decode, with
 *
 *   indices    [batch * next_n, k]  int32, written (same order, ties and -1
 *              padding as mqa_topk_indices); 1 <= k <= 2048
 *   workspace  DEVICE memory of at least
 *              paged_mqa_topk_workspace_size(batch, next_n, max_model_len)
 *              bytes (about 8 bytes per row and position: 101 MB for 96 rows
 *              of 131072), 256-byte aligned, owned by the caller; contents on
 *              entry do not matter and are clobbered.  Calls that overlap on one
 *              workspace race.
 *
 * Four kernels on `stream`: a decode of 16 evenly spaced runs of 256
 * positions per sequence (the sample), per-row thresholds from it, the decode
 * of every position keeping only the entries at or above the row's threshold,
 * and a per-row select and sort.  A row whose kept entries cannot hold its top
 * k (the sample misjudged it) is recomputed in full by its select workgroup
 * (its logits into its workspace segment, then an exact radix select), so the
 * output is exact for every input; such rows only take longer.
 * Supported: every head count, head dim, block size and kv_layout that
 * paged_mqa_logits_decode takes; the ring_depth tunable 0 or the logits
 * call's default (4 for kv_block_size 1, else 3); a KV split of
 * at most 1024.  Errors as for paged_mqa_logits_decode (a shape outside its
 * gate -> MQA_ERR_UNSUPPORTED, checked first), plus: k out of range, another
 * ring_depth, NULL or misaligned indices or workspace, a workspace smaller
 * than asked for -> MQA_ERR_INVALID_ARG.
 */
int paged_mqa_topk_decode(const uint8_t *q_fp8, const uint8_t *kv_cache, const float *weights,
                          const int32_t *context_lens, const int32_t *block_tables,
                          int32_t *indices, int batch, int next_n, int num_heads, int head_dim,
                          int kv_block_size, int kv_layout, int num_blocks,
                          int max_blocks_per_seq, int max_model_len, int k, void *workspace,
                          size_t workspace_bytes, const mqa_tunables *tun, hipStream_t stream);

/*
 * paged_mqa_topk_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without the workspace arguments.  The workspace
 * lives in a static device array of MQA_NOALLOC_SCRATCH_BYTES held by the
 * library (one copy per device it runs on, kept until the process ends), so
 * the call makes no allocation of its own; the caller still owns the inputs
 * and `indices`.  Every call on one device shares that array: calls that
 * overlap on a device (several streams or threads) race.  Nothing in it has to
 * start cleared, so a call depends on no earlier call's contents.
 *
 * Errors as for paged_mqa_topk_decode, plus: a problem whose
 * paged_mqa_topk_workspace_size exceeds MQA_NOALLOC_SCRATCH_BYTES (checked
 * first; 128 MiB holds 96 rows of 131072 positions) -> MQA_ERR_INVALID_ARG;
 * the array's device address not available -> MQA_ERR_DEVICE.
 */
#define MQA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int paged_mqa_topk_decode_noalloc(const uint8_t *q_fp8, const uint8_t *kv_cache,
                                  const float *weights, const int32_t *context_lens,
                                  const int32_t *block_tables, int32_t *indices, int batch,
                                  int next_n, int num_heads, int head_dim, int kv_block_size,
                                  int kv_layout, int num_blocks, int max_blocks_per_seq,
                                  int max_model_len, int k, const mqa_tunables *tun,
                                  hipStream_t stream);

/* Workspace bytes paged_mqa_topk_decode needs (0 for sizes it rejects or
 * treats as a no-op).  Host-only, never fails. */
size_t paged_mqa_topk_workspace_size(int batch, int next_n, int max_model_len);

#define MQA_DTYPE_FP32 0
#define MQA_DTYPE_BF16 1

/*
 * K-cache quantise-and-insert: the step that fills the paged cache read by
 * paged_mqa_logits_decode (aiter PR 5047 page, "Motivation": K stored as fp8
 * e4m3fn beside a per-token fp32 dequant scale; the scale is the token's
 * absolute maximum over 448, the largest e4m3fn value).
 *
 *   k             [num_tokens, head_dim]  fp32 (k_dtype MQA_DTYPE_FP32) or
 *                                         bf16 (MQA_DTYPE_BF16); finite values
 *   slot_mapping  [num_tokens]            int64: the cache slot of each token,
 *                                         block * kv_block_size + slot;
 *                                         negative = padding, nothing written
 *   kv_cache      [num_blocks] blocks in the decode layout (K rows in the
 *                 order kv_layout names), updated in place
 *
 * Per token: scale = fp32(max(amax, 1e-12) / 448) (one correctly rounded
 * division), codes = e4m3fn(clamp(k / scale, -448, 448)) rounded to nearest,
 * ties to even, sign kept.  The token's head_dim code bytes and its scale are
 * written to its slot; nothing else in the cache changes.  Slots at or past
 * num_blocks * kv_block_size are skipped as well.  Two tokens mapped to the
 * same slot race (either may win).
 * num_tokens == 0 is a successful no-op.  Negative sizes, a bad k_dtype or
 * kv_layout, NULL or misaligned pointers (k and kv_cache 16-byte,
 * slot_mapping 8-byte) -> MQA_ERR_INVALID_ARG; head_dim other than 128 or 64,
 * kv_block_size not 1, 16, 64 or 128, or the preshuffled layout with
 * kv_block_size 1 -> MQA_ERR_UNSUPPORTED.
 */
int mqa_kcache_quantize_insert(const void *k, int k_dtype, const int64_t *slot_mapping,
                               uint8_t *kv_cache, int num_tokens, int head_dim,
                               int kv_block_size, int kv_layout, int num_blocks,
                               hipStream_t stream);

/* Human-readable reason for this thread's last non-zero return ("" if none). */
const char *mqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MQA_INDEXER_H */
