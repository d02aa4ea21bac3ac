/*
 * qsa.h -- C ABI of libqsa, QSA sparse main-attention prefill on MI355X (gfx950).
 *
 * The operation (page "Qwen4-Exp QSA comes to Huawei's Ascend: inside
 * SGLang's opt-in CANN prefill PR", section "What the pull request actually
 * adds"): every query token t attends only to the physical KV-cache slots its
 * indexer selected,
 *
 *     out[t, h, :] = sum_j softmax_j(scale * q[t,h,:] . k[s_j, g, :]) * v[s_j, g, :]
 *
 * over the entries s_j of slot_idx[t, :] that are not -1, with query head h
 * reading KV head g = h / (Hq / Hkv) (grouped query heads, contiguous groups).
 * BF16 inputs and output, head dim 256 ("Hardware and dtype" bullet), any
 * Hq % Hkv == 0 with no padding of the head ratio ("Head shapes" bullet).  A
 * row with no selected slot -- all -1, or W == 0 -- outputs exactly +0.0
 * ("Sizing bounds" bullet).  Slots may come in any order and -1 may sit
 * anywhere in a row (section "Nine tests that passed, ...").
 *
 * Conventions for every entry point:
 *  - Pointers in the views and the workspace are DEVICE pointers on the
 *    current HIP device; the caller owns all memory.  The library allocates
 *    nothing and keeps no pointer after the call returns.
 *  - Strides are in elements.  The innermost stride must be 1; the other
 *    strides of BF16 views must be multiples of 8 elements (16 bytes) and
 *    their base pointers 16-byte aligned.  Strides may be larger than the
 *    packed size (views of bigger buffers are fine).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work: they return before the kernels run and never synchronize,
 *    except qsa_check_status, which synchronizes `stream`.
 *  - Argument errors are detected on the host before anything is enqueued; the
 *    call then returns a non-zero qsa_status, writes nothing and
 *    qsa_last_error() describes the problem.  There is no fallback path.
 *  - Entries of slot_idx that are neither -1 nor in [0, S) are dropped (never
 *    dereferenced) and counted; qsa_check_status reports them.
 *  - Calls on different streams with different workspaces may run
 *    concurrently; calls sharing a workspace must be stream-ordered.
 *  - A problem whose kernel launches would exceed the 2^32 - 1 work-items
 *    one grid dimension counts (for instance more than 16,777,215 tokens for
 *    the compaction pass, or more than 67,108,863 attention work items of
 *    (token, KV head, block of 16 query heads), times the splits of split
 *    attention) is refused with QSA_ERR_UNSUPPORTED before anything is
 *    enqueued; split such a call.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_NULL = 1,        /* a required pointer is NULL */
    QSA_ERR_SHAPE = 2,       /* sizes disagree or are negative */
    QSA_ERR_STRIDE = 3,      /* innermost stride != 1, misaligned base or stride */
    QSA_ERR_SCALE = 4,       /* scale is NaN or infinite */
    QSA_ERR_WORKSPACE = 5,   /* workspace NULL, misaligned or too small */
    QSA_ERR_SLOT_RANGE = 6,  /* (qsa_check_status) some entry was neither -1 nor in [0, S) */
    QSA_ERR_UNSUPPORTED = 7, /* head dim other than 256, sizes beyond 32-bit limits */
    QSA_ERR_HIP = 8,         /* a HIP runtime call failed */
    QSA_ERR_ALIAS = 9        /* out overlaps an input */
} qsa_status;

/* A strided 3-D BF16 tensor: q and out are [T, Hq, D]; k_cache and v_cache
 * are [S, Hkv, D].  `data` points at element [0][0][0].  The slot stride of
 * k_cache and v_cache (stride[0], in bytes) must be under 4 GiB; larger ones
 * are refused with QSA_ERR_UNSUPPORTED. */
typedef struct qsa_bf16_view {
    void *data;
    int64_t size[3];
    int64_t stride[3];
} qsa_bf16_view;

/* A strided 3-D tensor of FP8 E4M3 codes (one byte per element; OCP "fn"
 * encoding: bias 7, no infinities) for an FP8 KV cache [S, Hkv, D]; strides
 * in elements (= bytes), multiples of 16 apart from the unit innermost one. */
typedef struct qsa_fp8_view {
    void *data;
    int64_t size[3];
    int64_t stride[3];
} qsa_fp8_view;

/* A strided 2-D int32 tensor: slot_idx is [T, W]; -1 means "no slot". */
typedef struct qsa_i32_view {
    const int32_t *data;
    int64_t size[2];
    int64_t stride[2];
} qsa_i32_view;

/* Where the compaction pass leaves its results inside a workspace (byte
 * offsets from the workspace base):
 *   list:  int32 [T][row_stride]; row t holds its count[t] valid slots,
 *          then -1 up to the next multiple of 32.  Order: the row is cut into
 *          runs of 2304 consecutive input entries, kept in input order; inside
 *          a run the valid entries are stably sorted by slot >> r, where
 *          b = max(1, ceil(log2 S)) and r = max(0, b - 7) (at most 128 slot
 *          ranges, ascending; input order within a range);
 *   count: int32 [T], number of valid entries of row t;
 *   n_bad: int32 [T], entries of row t that were neither -1 nor in [0, S);
 *   share: 512 bytes: words the attention writes to pick its layout (see
 *          qsa_sparse_attend), and at byte 384 two int32 words the
 *          compaction writes: the number of cache slots its lists index (S,
 *          or hi - lo for a shard) and a flag it clears, which an attention
 *          over K/V views of fewer slots sets (see qsa_check_status). */
typedef struct qsa_workspace_map {
    int64_t list_offset;
    int64_t row_stride;
    int64_t count_offset;
    int64_t bad_offset;
    int64_t share_offset;
    int64_t total_bytes;
} qsa_workspace_map;

/* Library version string, e.g. "libqsa 0.1.0 gfx950". */
const char *qsa_version(void);

/* Short text for a status code. */
const char *qsa_status_string(qsa_status status);

/* Message for the last non-OK status returned on the calling thread. */
const char *qsa_last_error(void);

/* Workspace bytes needed for T tokens of W selection entries (0 <= T, W <
 * 2^31).  Returns 0 for sizes outside that range. */
size_t qsa_workspace_bytes(int64_t T, int64_t W);

/* The same size under the name of the prefill it serves (qsa_sparse_prefill,
 * qsa_compact_slots, qsa_sparse_attend). */
size_t qsa_sparse_prefill_workspace_bytes(int64_t T, int64_t W);

/* Fill *map with the workspace layout for T, W (see qsa_workspace_map). */
qsa_status qsa_workspace_layout(int64_t T, int64_t W, qsa_workspace_map *map);

/*
 * Index validation and compaction (the -1 rules of the "Sizing bounds"
 * bullet; unordered slots of section "Nine tests that passed, ...").  For
 * every row t of slot_idx [T, W], writes into the workspace the entries in
 * [0, S) grouped into ascending slot ranges (see qsa_workspace_map for the
 * exact order), their count, and the number of invalid entries.  S is the
 * number of cache slots.  Duplicates are kept.  The attention result does
 * not depend on the order of a row; the grouping makes the gathers of one
 * tile fall close together in memory and lets the tokens processed at one
 * time read the same cache rows at about the same time.
 */
qsa_status qsa_compact_slots(const qsa_i32_view *slot_idx, int64_t S,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * qsa_compact_slots for one shard of a cache split by slot ranges: entries in
 * [lo, hi) are kept and stored as slot - lo (the shard's own numbering, so
 * the shard's K/V views start at slot lo).  Entries that are neither -1 nor
 * in [0, S) are counted as invalid exactly as in qsa_compact_slots; valid
 * entries outside [lo, hi) belong to other shards and are skipped silently.
 * Requires 0 <= lo <= hi <= S.  qsa_compact_slots(s, S, ...) is
 * qsa_compact_slot_range(s, S, 0, S, ...).
 */
qsa_status qsa_compact_slot_range(const qsa_i32_view *slot_idx, int64_t S,
                                  int64_t lo, int64_t hi, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Micro-block selections.  QSA selects micro-blocks of consecutive tokens
 * rather than single tokens (page, section "Why QSA is the awkward part, in
 * numbers"; a block size of 4 is the later "block4" work of section "Nine
 * tests that passed, ...").  Reading: block b of the physical cache is slots
 * b * block_size .. b * block_size + block_size - 1, and S must be a multiple
 * of block_size (1..64).  block_idx is [T, W] with -1 for "no block"; an
 * entry that is neither -1 nor in [0, S / block_size) is invalid (dropped,
 * counted).  qsa_compact_blocks fills a workspace for T rows of width
 * W * block_size (size it with qsa_workspace_bytes(T, W * block_size)): the
 * valid blocks, grouped as in qsa_compact_slots by block id, each expanded
 * into its block_size slots in ascending order; count[t] counts slots.
 * qsa_sparse_attend with that width then runs the attention unchanged.
 */
qsa_status qsa_compact_blocks(const qsa_i32_view *block_idx, int64_t S,
                              int32_t block_size, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * The whole prefill for micro-block selections: qsa_compact_blocks followed
 * by qsa_sparse_attend, the same operation and the same conventions
 * (qsa_check_status(workspace, ..., T, W * block_size, ...) reports invalid
 * entries).  With a workspace of qsa_prefill_blocks_workspace_bytes(T, W,
 * block_size) bytes, power-of-two blocks of 4 to 64 slots, W <= 2304 blocks
 * and the sharing of a long prefill (the layout choice of qsa_sparse_attend
 * takes 8 items per CU without an estimate), the compaction writes aligned
 * lists instead, after the standard layout: block ids, not slots, where each
 * token's part of every span of about 2,048 cache slots starts near a fixed
 * place of its row (the gaps masked), so the tokens running at one time reach
 * each part of the cache together; the attention expands every block into
 * its slots.  The result then differs from the plain path's only in the
 * summation order.  A workspace of qsa_workspace_bytes(T, W * block_size)
 * runs the plain path.
 */
size_t qsa_prefill_blocks_workspace_bytes(int64_t T, int64_t W, int32_t block_size);

qsa_status qsa_sparse_prefill_blocks(const qsa_bf16_view *q,
                                     const qsa_bf16_view *k_cache,
                                     const qsa_bf16_view *v_cache,
                                     const qsa_i32_view *block_idx,
                                     int32_t block_size, float scale,
                                     qsa_bf16_view *out, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Gather attention over a workspace already filled by qsa_compact_slots for
 * the same T and W (the softmax(scale * Q K^T) V of the layout-embedding
 * paragraph, restricted to each token's listed slots).  Rows with count 0
 * receive +0.0.  q/out [T, Hq, 256], k_cache/v_cache [S, Hkv, 256]; W is the
 * selection width the workspace was compacted with; scale must be finite.
 * The workspace must have been compacted for at most S cache slots (the S
 * of the compaction, or hi - lo of a shard): every listed slot then lies in
 * the views.  Lists compacted for more slots are not read: the call writes
 * +0.0 rows instead and qsa_check_status reports QSA_ERR_WORKSPACE.
 *
 * Layout choice: the kernel runs 8 items (token, KV head) per CU, which lets
 * the tokens running together share cache rows in L2.  Where the sizes allow
 * little sharing (a cache large against W), a small estimate first samples
 * pairs of neighbouring tokens' lists and counts their common slots; if the
 * tokens share few rows, 4 items per CU are run instead, and if they share
 * many (BF16 caches), the 8 items take their keys through LDS as whole rows
 * (fewer cache rows per load instruction).  Sizes that alone bound the
 * sharing high enough take that form without an estimate.  All layouts give
 * the same bits.  The estimate writes the workspace's share words (the rest
 * of the workspace is only read), so calls on one workspace must not
 * overlap.
 */
qsa_status qsa_sparse_attend(const qsa_bf16_view *q,
                             const qsa_bf16_view *k_cache,
                             const qsa_bf16_view *v_cache, int64_t W,
                             float scale, void *workspace,
                             size_t workspace_bytes, qsa_bf16_view *out,
                             void *stream);

/*
 * The whole sparse prefill: qsa_compact_slots followed by qsa_sparse_attend,
 * enqueued on `stream`.  slot_idx is [T, W] with T = q->size[0].  Pass
 * scale = 1/sqrt(256) for the default scale of the page.  The workspace must
 * hold qsa_workspace_bytes(T, W) bytes, 256-byte aligned.
 */
qsa_status qsa_sparse_prefill(const qsa_bf16_view *q,
                              const qsa_bf16_view *k_cache,
                              const qsa_bf16_view *v_cache,
                              const qsa_i32_view *slot_idx, float scale,
                              qsa_bf16_view *out, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * Split attention and its merge.  The softmax over a token's selected slots
 * can be evaluated over disjoint shares of the slots and combined exactly
 * with a log-sum-exp rescale; this serves decode and other small-T batches
 * (too few (token, KV head) items to fill the GPU, so each item's slots are
 * dealt to several workgroups) and a cache sharded by slot ranges (each
 * shard produces its share, as in the decode context parallelism the page
 * names in section "Where this sits in the Qwen4Exp serving build-out").
 *
 * A partials buffer holds n_parts shares for [T, Hq] rows: FP32 O [n_parts]
 * [T][Hq][256] (not divided by the sum), then FP32 (m, l) [n_parts][T][Hq][2]
 * at the next 256-byte boundary, where m is the running maximum of
 * scale * q.k * log2(e) and l the sum of 2^(score - m).  An empty share has
 * m = -inf, l = 0, O = 0.  qsa_partials_bytes gives the size (256-byte
 * aligned buffer required).
 */
size_t qsa_partials_bytes(int64_t n_parts, int64_t T, int64_t Hq);

/* Deal each item's tiles of a compacted workspace (from qsa_compact_slots or
 * qsa_compact_slot_range, for the same T, W) to `splits` workgroups and write
 * their shares into parts [part_base, part_base + splits) of a partials
 * buffer holding n_parts parts. */
qsa_status qsa_sparse_attend_partial(const qsa_bf16_view *q,
                                     const qsa_bf16_view *k_cache,
                                     const qsa_bf16_view *v_cache, int64_t W,
                                     float scale, const void *workspace,
                                     size_t workspace_bytes, int32_t splits,
                                     int64_t part_base, int64_t n_parts,
                                     void *partials, size_t partials_bytes,
                                     void *stream);

/* out[t,h] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the n_parts
 * shares (M = max_s m_s), rounded to BF16; exactly +0.0 when every share is
 * empty.  out is [T, Hq, 256] and must not overlap the partials. */
qsa_status qsa_merge_partials(const void *partials, size_t partials_bytes,
                              int64_t n_parts, int64_t T, int64_t Hq,
                              qsa_bf16_view *out, void *stream);

/* Splits per item that qsa_sparse_decode uses for these sizes (a pure
 * function of the sizes: about 1,024 workgroups; at least eight 16-slot tiles
 * per split unless that leaves fewer than 512 workgroups; at least four; at
 * most 64 splits). */
int32_t qsa_decode_splits(int64_t T, int64_t W, int32_t Hq, int32_t Hkv);

/* Workspace bytes for qsa_sparse_decode: the area of qsa_workspace_bytes(T, W)
 * (qsa_check_status reads the invalid-entry counts there) followed by the
 * partials of qsa_decode_splits(T, W, Hq, Hkv) shares. */
size_t qsa_decode_workspace_bytes(int64_t T, int64_t W, int32_t Hq, int32_t Hkv);

/*
 * The same operation as qsa_sparse_prefill, organised for few tokens
 * (decode steps, short batches): split attention over qsa_decode_splits
 * shares per item, then the merge.  There is no compaction pass: each share
 * reads its part of the selection row itself, skips -1 and drops (and
 * counts) entries outside [0, S).  Same arguments and conventions as
 * qsa_sparse_prefill; the workspace must hold qsa_decode_workspace_bytes, and
 * qsa_check_status(workspace, ..., T, W, ...) reports the invalid entries.
 * Entries are summed in row order rather than grouped by slot range, so the
 * result can differ from qsa_sparse_prefill's in the last bits.  (An empty
 * cache, S = 0, where no entry is valid, runs the compaction pass instead.)
 */
qsa_status qsa_sparse_decode(const qsa_bf16_view *q,
                             const qsa_bf16_view *k_cache,
                             const qsa_bf16_view *v_cache,
                             const qsa_i32_view *slot_idx, float scale,
                             qsa_bf16_view *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/*
 * qsa_sparse_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and results without the
 * workspace arguments.  Its workspace is a fixed scratch array of
 * qsa_noalloc_scratch_bytes() bytes (64 MiB: enough for 7,810 tokens of 2,051
 * entries) that the library holds in the memory of every GPU it runs on until
 * the process ends; the call allocates nothing.  A selection whose workspace
 * (qsa_workspace_bytes(T, W)) exceeds it is refused with QSA_ERR_UNSUPPORTED.
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (on different streams, or from different threads) race and must not be
 * made.  The array keeps the last call's contents.
 */
size_t qsa_noalloc_scratch_bytes(void);

qsa_status qsa_sparse_prefill_noalloc(const qsa_bf16_view *q,
                                      const qsa_bf16_view *k_cache,
                                      const qsa_bf16_view *v_cache,
                                      const qsa_i32_view *slot_idx, float scale,
                                      qsa_bf16_view *out, void *stream);

/*
 * Synchronizes `stream`, then reads the invalid-entry counts that the last
 * compaction into `workspace` (for T, W), or the last qsa_sparse_decode with
 * it, left.  Writes their total to
 * *n_bad (if not NULL) and returns QSA_ERR_SLOT_RANGE if it is non-zero.
 * Returns QSA_ERR_WORKSPACE instead if an attention since that compaction
 * found the workspace's lists compacted for more cache slots than its K/V
 * views held (and wrote zero rows).
 * This is the only entry point that waits for the device.
 */
qsa_status qsa_check_status(const void *workspace, size_t workspace_bytes,
                            int64_t T, int64_t W, void *stream,
                            int64_t *n_bad);

/*
 * Measurement aid: reads exactly the K and V rows that qsa_sparse_attend
 * would read for this workspace (same slots, same KV heads, same load
 * pattern, one wave per (token, KV head), same residency per CU) and folds
 * them into one checksum word per (token, KV head) in sink[T * Hkv] (device
 * memory, caller-owned): the XOR of the 32-bit words of every read row.  It
 * issues the loads back to back with no attention arithmetic between them;
 * its duration is the cost of the gathers alone issued that way, which the
 * attention itself, pacing its requests, can beat.
 */
qsa_status qsa_gather_only(const qsa_bf16_view *k_cache,
                           const qsa_bf16_view *v_cache, int64_t T,
                           int64_t W, const void *workspace,
                           size_t workspace_bytes, uint32_t *sink,
                           void *stream);

/*
 * Measurement aid: a plain streaming read.  `workgroups` workgroups of 256
 * threads each read bytes_per_workgroup consecutive bytes of the first
 * footprint_bytes of buf with 16-byte loads (workgroup w starting at byte
 * w * bytes_per_workgroup modulo footprint_bytes and wrapping at the end of
 * the footprint), and write the XOR of the 32-bit words they read to
 * sink[w] (device memory, caller-owned, `workgroups` words).  buf must be
 * 16-byte aligned; footprint_bytes and bytes_per_workgroup positive multiples
 * of 16, bytes_per_workgroup <= footprint_bytes.  With a footprint that stays
 * in the L2s, one that fits only the Infinity Cache, and one larger than that,
 * the duration gives the read bandwidth of each level for the attention's
 * 16-byte loads.
 */
qsa_status qsa_stream_read(const void *buf, size_t footprint_bytes,
                           size_t bytes_per_workgroup, int64_t workgroups,
                           uint32_t *sink, void *stream);

/*
 * FP8 KV-cache variant.  The page's section "Where this sits in the Qwen4Exp
 * serving build-out" reports decode measured with an fp8_e4m3 KV cache; the
 * page defines no scaling, so the reading here is one scale per tensor: each
 * K element is decode(code) * k_scale and each V element decode(code) *
 * v_scale.  The computation is otherwise the one of qsa_sparse_attend /
 * qsa_sparse_prefill (q and out stay BF16), with half the gathered bytes.
 * k_scale and v_scale must be finite.
 */
qsa_status qsa_sparse_attend_fp8kv(const qsa_bf16_view *q,
                                   const qsa_fp8_view *k_cache,
                                   const qsa_fp8_view *v_cache, float k_scale,
                                   float v_scale, int64_t W, float scale,
                                   void *workspace, size_t workspace_bytes,
                                   qsa_bf16_view *out, void *stream);

qsa_status qsa_sparse_prefill_fp8kv(const qsa_bf16_view *q,
                                    const qsa_fp8_view *k_cache,
                                    const qsa_fp8_view *v_cache, float k_scale,
                                    float v_scale, const qsa_i32_view *slot_idx,
                                    float scale, qsa_bf16_view *out,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

/*
 * qsa_sparse_decode over an FP8 E4M3 KV cache: the split attention over the
 * raw selection rows and the merge of qsa_sparse_decode, with the cache
 * reading of qsa_sparse_attend_fp8kv (one scale per tensor, element =
 * decode(code) * scale; the page's section "Where this sits in the Qwen4Exp
 * serving build-out" reports decode measured with an fp8_e4m3 KV cache).
 * Arguments as qsa_sparse_prefill_fp8kv; the workspace must hold
 * qsa_decode_workspace_bytes(T, W, Hq, Hkv) bytes, 256-byte aligned, and
 * qsa_check_status(workspace, ..., T, W, ...) reports the invalid entries.
 * k_scale and v_scale must be finite (QSA_ERR_SCALE otherwise).
 */
qsa_status qsa_sparse_decode_fp8kv(const qsa_bf16_view *q,
                                   const qsa_fp8_view *k_cache,
                                   const qsa_fp8_view *v_cache, float k_scale,
                                   float v_scale, const qsa_i32_view *slot_idx,
                                   float scale, qsa_bf16_view *out,
                                   void *workspace, size_t workspace_bytes,
                                   void *stream);

/* qsa_gather_only for an FP8 KV cache (same tiles, waves and loads as
 * qsa_sparse_attend_fp8kv; XOR of the 32-bit words of every read row). */
qsa_status qsa_gather_only_fp8kv(const qsa_fp8_view *k_cache,
                                 const qsa_fp8_view *v_cache, int64_t T,
                                 int64_t W, const void *workspace,
                                 size_t workspace_bytes, uint32_t *sink,
                                 void *stream);

/*
 * QSA indexer and Top-K selection: the step that produces slot_idx (page,
 * section "Why QSA is the awkward part, in numbers": a multi-query indexer,
 * 4 query heads sharing 1 key head, head dim 128, compression ratio 4, a fixed
 * budget; section "Nine tests that passed, ...": causal tails of 0-3
 * positions).  The page gives the structure, not the formulas; readings:
 *  - ik holds one key per block of 4 consecutive positions of the request,
 *    block c = positions 4c .. 4c+3, so C = L / 4 (rounded either way);
 *  - score(t, c) = sum over the 4 heads of max(0, iq[t,h] . ik[c]) (FP32
 *    accumulation of BF16 products);
 *  - a query at position p = positions[t] ranks the complete blocks before it
 *    (4c + 3 <= p) and keeps the `budget` best, ties to the lower c;
 *  - its row of slot_idx [T, 4*budget + 3] lists the positions of the kept
 *    blocks (ascending c, 4 each), then its r = (p+1) % 4 tail positions
 *    p-r+1 .. p, each mapped through slot_of_pos [L] (the request's
 *    position -> physical slot table), then -1.  budget = 512 gives the
 *    2,051-wide rows of the long prefill.
 * Positions outside [0, L) give an all -1 row.  iq is [T, 4, 128], ik
 * [C, 1, 128] (BF16, rows 16-byte aligned); positions, slot_of_pos, scores
 * and slot_idx are device memory.  qsa_indexer_scores writes FP32 [T, C]
 * scores (entries past a query's causal limit are left unspecified) and
 * needs qsa_indexer_scores_bytes(T, C) = T * C * 4 bytes;
 * qsa_indexer_select reads them.  qsa_indexer_topk is the two in one call,
 * with `scores` as caller-owned scratch of that size.
 *
 * qsa_indexer_topk_fused computes the same selection without writing the
 * full score matrix, in caller-owned scratch of
 * qsa_indexer_topk_fused_bytes(T, C) bytes (8-byte aligned): a threshold
 * sampled per token (256 scores of blocks spread over the causal range, the
 * key about sqrt(budget * 4096) * 256 / n from the top, its top 16 bits),
 * the scores recomputed and only those at or above it kept as (score,
 * block) candidates per 1,024-block range, and the exact selection on at
 * most 4,096 candidates.  Rows where the threshold keeps fewer than
 * `budget` or more than 4,096 candidates (or more than 512 in one range)
 * get their full scores and the exact selection, so the result is the same
 * either way.  It takes budgets up to 512 and C up to 262,144 (else
 * QSA_ERR_UNSUPPORTED).  On MI355X it is the slower of the two (the
 * candidate pass is issue-bound, not memory-bound), so qsa_indexer_topk
 * does not use it.
 */
size_t qsa_indexer_scores_bytes(int64_t T, int64_t C);
size_t qsa_indexer_topk_fused_bytes(int64_t T, int64_t C);

qsa_status qsa_indexer_scores(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                              const int32_t *positions, float *scores,
                              size_t scores_bytes, void *stream);

qsa_status qsa_indexer_select(const float *scores, size_t scores_bytes,
                              int64_t T, int64_t C, const int32_t *positions,
                              const int32_t *slot_of_pos, int64_t L,
                              int32_t budget, qsa_i32_view *slot_idx,
                              void *stream);

/* qsa_indexer_scores followed by qsa_indexer_select. */
qsa_status qsa_indexer_topk(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                            const int32_t *positions,
                            const int32_t *slot_of_pos, int64_t L,
                            int32_t budget, float *scores, size_t scores_bytes,
                            qsa_i32_view *slot_idx, void *stream);

/* The same selection by the fused path (scratch: `scratch_bytes` >=
 * qsa_indexer_topk_fused_bytes(T, C)). */
qsa_status qsa_indexer_topk_fused(const qsa_bf16_view *iq, const qsa_bf16_view *ik,
                                  const int32_t *positions,
                                  const int32_t *slot_of_pos, int64_t L,
                                  int32_t budget, void *scratch, size_t scratch_bytes,
                                  qsa_i32_view *slot_idx, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
