/*
 * hwkv.h -- C ABI of the per-head windowed KV cache runtime for MI355X (gfx950).
 *
 * What it implements.  The HeadWiseKV write-up (KnoAI) gives every physical KV
 * head of a global-attention layer a static history window w_h and
 * materialises that policy as real per-head cache residency instead of
 * masking a full cache (sections 摘要 and 核心技术 2 "Grouped-Cache Runtime").
 * Each head owns a block table of ceil(w_h / block_size) blocks, so the memory
 * demand is exact before serving.  This library provides:
 *   - the layout built from per-layer, per-head window vectors and the exact
 *     memory estimate (host only);
 *   - the append of new K/V rows into each head's ring of blocks (device);
 *   - decode attention over exactly the last w_h tokens of each head, GQA,
 *     split over the window and merged (device);
 *   - a chunked-prefill variant: windowed causal attention of a chunk of new
 *     queries over the cache history plus the chunk itself (device).
 *
 * Conventions.
 *   - Every function returns hwkv_status; hwkv_last_error() gives a message
 *     for the last failing call on the calling thread.  No exception crosses
 *     the ABI.
 *   - Every argument is validated on the host before anything is enqueued:
 *     a failing call enqueues nothing.
 *   - Device calls only enqueue kernels on the given HIP stream: no
 *     allocation, no copy, no synchronisation.  They can be captured in a HIP
 *     graph.  Stream order is the only ordering between calls.
 *   - All device memory is owned by the caller.  The library owns only the
 *     host-side hwkv_layout.
 *   - A layout is immutable: changing any window means a new layout (and a
 *     new pool); the write-up's operations table notes that a policy change
 *     requires a restart.
 *   - Alignment (write-up "KV Cache Management in Hybrid Attention LLMs",
 *     section 4.4, which asks for 128- or 256-byte aligned cache pointers):
 *     pool, block table, meta and workspace pointers must be 256-byte aligned;
 *     q, k, v and out 16-byte aligned (128-bit accesses); ctx_len/pos0 8-byte
 *     and seq_slots 4-byte aligned.  Violations return HWKV_ERR_MISALIGNED.
 *   - Kernel-ABI check (same page, section 4.2: a kernel must only read a
 *     cache whose layout it was built for): the meta blob carries the ABI
 *     version and the layout fingerprint, and the cache view states which
 *     fingerprint its blob holds (hwkv_cache.meta_fingerprint).  Every device
 *     call returns HWKV_ERR_ABI_MISMATCH, before enqueueing anything, when
 *     that differs from the fingerprint of the layout it is called with.
 *     The kernels compare the blob itself as well (a view that misstates its
 *     blob): see "Bad device values" below.
 *   - The softmax scale of the attention calls must be finite and > 0
 *     (HWKV_ERR_INVALID_ARG otherwise).
 *
 * Bad device values.  Device arrays (seq_slots, positions, block ids, the
 * meta blob) are the caller's contract; the kernels never trust them for
 * addressing (nothing is read or written outside the pool, the table or the
 * caller's tensors) and turn each violation into a visible result, the same
 * in every kernel:
 *   - a slot outside [0, table_rows): append writes nothing for that
 *     sequence; attention gives NaN rows for it;
 *   - a negative position: append writes nothing for that sequence; decode
 *     (context <= 0) gives zero rows; prefill (pos0 < 0) gives NaN rows;
 *   - a block id outside the pool: append skips the rows that map to it;
 *     an attention query row whose window holds a key stored in that block
 *     comes out NaN (in decode one query row reads the whole window, so all
 *     G query heads of that (sequence, kv head) are NaN; in prefill exactly
 *     the chunk rows whose window reaches that block's keys);
 *   - a meta blob of another layout: append writes nothing; attention writes
 *     NaN over its whole output.
 * The write-up's troubleshooting row locates failures by (layer, head): a
 * NaN output row names them through its position in out.
 *
 * Memory layout of the pool.  Physical block i occupies bytes
 * [i*block_bytes, (i+1)*block_bytes): first block_size K rows of head_dim
 * elements, then block_size V rows.  block_bytes = 2*block_size*head_dim*
 * sizeof(element).  Token t of a head with nb blocks lives in the head's ring
 * block (t / block_size) % nb, row t % block_size.
 *
 * Block tables.  One int32 row of blocks_per_seq entries per cache slot
 * ("sequence row"); head (l, h) owns entries [head_off(l,h),
 * head_off(l,h) + nblocks(l,h)) of the row, heads in layer-major order.  The
 * ids are physical block indices into the pool; any permutation is allowed.
 */
#ifndef HWKV_H
#define HWKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HWKV_ABI_VERSION 3u

typedef enum hwkv_status {
    HWKV_OK = 0,
    HWKV_ERR_INVALID_ARG = 1,  /* bad size, range, null pointer, window < 1 */
    HWKV_ERR_UNSUPPORTED = 2,  /* a valid configuration this build has no kernel for */
    HWKV_ERR_MISALIGNED = 3,   /* a pointer breaks the alignment rules above */
    HWKV_ERR_CAPACITY = 4,     /* pool or workspace smaller than required */
    HWKV_ERR_ABI_MISMATCH = 5, /* meta blob from another layout or ABI version */
    HWKV_ERR_HIP = 6,          /* a HIP launch failed */
    HWKV_ERR_OVERFLOW = 7      /* a size does not fit 64-bit (or int32 ids) */
} hwkv_status;

typedef enum hwkv_dtype {
    HWKV_F32 = 0,
    HWKV_BF16 = 1,
    HWKV_F16 = 2
} hwkv_dtype;

typedef struct hwkv_layout hwkv_layout; /* opaque, host-side, immutable */

typedef struct hwkv_layout_desc {
    uint32_t abi_version;
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t block_size;
    int32_t head_dim;
    int32_t dtype;          /* hwkv_dtype of K, V and q */
    int32_t split_tokens;   /* decode split length S in tokens */
    int32_t max_window;
    int64_t blocks_per_seq; /* entries per block-table row */
    int64_t n_work;         /* decode work items (head, split) over all layers */
    uint64_t block_bytes;
    uint64_t meta_bytes;    /* size of the blob hwkv_meta_fill writes */
    uint64_t fingerprint;   /* hash of every layout parameter and window */
} hwkv_layout_desc;

/* Device-side view of one cache.  A host struct of device pointers, passed by
 * pointer to the device calls. */
typedef struct hwkv_cache {
    void *pool;               /* device, pool_bytes bytes, 256-B aligned */
    uint64_t pool_bytes;      /* must be >= hwkv_mem_estimate(table_rows) */
    const int32_t *block_ids; /* device [table_rows][blocks_per_seq], 256-B aligned */
    int64_t table_rows;       /* number of sequence rows (cache slots) */
    const void *meta;         /* device copy of hwkv_meta_fill, 256-B aligned */
    uint64_t meta_fingerprint; /* fingerprint the blob at meta carries: the
                                  hwkv_layout_desc.fingerprint of the layout
                                  that wrote it (hwkv_meta_fingerprint reads it
                                  from a host copy) */
} hwkv_cache;

/* ABI version compiled into the library (== HWKV_ABI_VERSION of its header).
 * "KV Cache Management in Hybrid Attention LLMs", section 4.2, asks that a
 * kernel reading a cache match the layout of the kernel that wrote it;
 * callers compare this, and the device calls compare the layout
 * fingerprint. */
uint32_t hwkv_abi_version(void);

/* Message of the last failing call on this thread ("" if none).  Capacity
 * errors name the first head that does not fit, in the form of the write-up's
 * operations table: "KV cache block allocation failed at layer X, head Y". */
const char *hwkv_last_error(void);

/* Build a layout from windows[n_layers*n_kv_heads] (layer-major, tokens per
 * head, each >= 1) -- the per-layer kv_head_windows vectors of the write-up's
 * policy YAML (核心技术 2).  Each head gets nblocks = ceil(w / block_size)
 * blocks.  A layout is a host description: any block_size in [1, 1024],
 * head_dim in [1, 1024] and dtype F32, BF16 or F16 can be described and
 * estimated; the device calls report HWKV_ERR_UNSUPPORTED for combinations
 * that have no kernel (append: any block size, rows of whole 16-byte chunks;
 * decode: block sizes 16, 32, 64, 128, 256, GQA groups 1, 2, 3, 4, 6, 8,
 * head_dim 64 or 128 with F32, BF16 or F16 and head_dim 256 with BF16 or
 * F16; prefill: the same block sizes and groups, BF16 or F16, head_dim 64,
 * 128 or 256).  split_tokens is the decode split length S (a multiple of
 * block_size, at most max(block_size, 2048); 0 picks the largest multiple of
 * block_size not above 1024).  The best S depends on the decode launch's
 * workgroup count against the 768 an MI355X holds at once (head_dim 128);
 * measured best: 1024 for 48 layers of one sequence at 112K and for one
 * layer of 4 sequences at 167K, 2048 for one layer of 8 sequences at 32K,
 * 384 for per-layer launches of one sequence.  On success *out owns the
 * layout; free it with hwkv_layout_destroy.  Errors: INVALID_ARG (null,
 * n < 1, window < 1, a size out of range), OVERFLOW. */
hwkv_status hwkv_layout_create(int32_t n_layers, int32_t n_kv_heads,
                               const int32_t *windows, int32_t block_size,
                               int32_t head_dim, hwkv_dtype dtype,
                               int32_t split_tokens, hwkv_layout **out);

void hwkv_layout_destroy(hwkv_layout *layout);

/* Describe a layout.  Optional outputs (may be null): windows_out and
 * nblocks_out [n_layers*n_kv_heads], head_offsets_out [n_layers*n_kv_heads+1]
 * (offset of each head's entries inside a block-table row). */
hwkv_status hwkv_layout_query(const hwkv_layout *layout, hwkv_layout_desc *desc,
                              int32_t *windows_out, int32_t *nblocks_out,
                              int64_t *head_offsets_out);

/* Exact pool bytes for n_seqs sequence rows (write-up 摘要 and 核心技术 2:
 * static per-head windows make the footprint computable before serving):
 *   n_seqs * sum_{l,h} ceil(w/bs) * bs * head_dim * 2 * sizeof(element).
 * Covers K and V blocks only (not tables, meta or workspace). */
hwkv_status hwkv_mem_estimate(const hwkv_layout *layout, int64_t n_seqs,
                              uint64_t *bytes);

/* Whether a pool of pool_bytes holds n_seqs sequence rows of this layout.
 * HWKV_OK if pool_bytes >= hwkv_mem_estimate(n_seqs).  Otherwise
 * HWKV_ERR_CAPACITY: blocks are laid out row by row, heads layer-major inside
 * a row, and *seq_row, *layer, *head (each may be null) receive the first
 * head whose blocks do not fit; the message has the form of the write-up's
 * operations table ("KV cache block allocation failed at layer X, head Y").
 * Every device call runs this check on its cache view. */
hwkv_status hwkv_capacity_check(const hwkv_layout *layout, int64_t n_seqs,
                                uint64_t pool_bytes, int64_t *seq_row,
                                int32_t *layer, int32_t *head);

/* Default block tables into host memory block_ids[n_seqs*blocks_per_seq]:
 * row s gets the consecutive ids [s*blocks_per_seq, (s+1)*blocks_per_seq).
 * This is the per-head BlockTable of the write-up's 核心技术 2 ("Grouped-Cache
 * Runtime": each head's table holds ceil(window / block_size) blocks), with
 * the heads of a sequence laid end to end in layer-major order; any other
 * assignment of distinct ids inside the pool is equally valid.  OVERFLOW if
 * an id would not fit int32. */
hwkv_status hwkv_table_fill(const hwkv_layout *layout, int64_t n_seqs,
                            int32_t *block_ids);

/* Write the layout's device descriptor blob (per-head windows, block counts,
 * table offsets and the decode work list) into host memory meta_host of
 * meta_bytes >= desc.meta_bytes.  The caller copies it to device memory once
 * and passes that copy as hwkv_cache.meta, with hwkv_cache.meta_fingerprint
 * set to the layout's fingerprint.  The blob carries the ABI version and the
 * fingerprint ("KV Cache Management in Hybrid Attention LLMs", section 4.2:
 * kernel-ABI check); kernels given a blob of another layout write nothing
 * (append) or NaN (attention). */
hwkv_status hwkv_meta_fill(const hwkv_layout *layout, void *meta_host,
                           uint64_t meta_bytes);

/* The fingerprint a meta blob carries, read from a host copy of it (e.g. a
 * blob kept with a cache that is restored later): *fingerprint receives the
 * hwkv_layout_desc.fingerprint of the layout that wrote it.  INVALID_ARG for
 * a null pointer or a buffer shorter than the blob header; ABI_MISMATCH when
 * the buffer is not a meta blob or was written under another ABI version. */
hwkv_status hwkv_meta_fingerprint(const void *meta_host, uint64_t meta_bytes,
                                  uint64_t *fingerprint);

/* Device workspace needed by hwkv_decode_split/_merge/_attn for layers
 * [layer_begin, layer_begin+n_layers), n_seqs sequences and n_q_heads query
 * heads: one fp32 record (acc[G][d], m[G], l[G]) per (sequence, work item).
 * The pages fix what decode computes (softmax over each head's window,
 * 摘要 and 核心技术 2) but not how; the workspace belongs to this library's
 * split-K form of it: the window of a head is cut into splits whose partial
 * softmax states are merged exactly, in a fixed order. */
hwkv_status hwkv_workspace_bytes(const hwkv_layout *layout, int32_t layer_begin,
                                 int32_t n_layers, int32_t n_seqs,
                                 int32_t n_q_heads, uint64_t *bytes);

/* Append n_new tokens per sequence: positions [pos0[b], pos0[b]+n_new) of
 * layers [layer_begin, layer_begin+n_layers).  k, v: device
 * [n_layers][n_seqs][n_new][n_kv_heads][head_dim] in the layout's dtype.
 * seq_slots: device int32[n_seqs], the table row of each batch entry, or null
 * for row b.  pos0: device int64[n_seqs].  Each head keeps only its most
 * recent tokens (page 2, "SWA Window": the window shifts as the sequence
 * advances): a head with ring capacity C stores token t in ring block
 * (t/bs)%nblocks, row t%bs, and of this call's tokens only those with
 * t >= pos0+n_new-C are written (older ones would be overwritten in the same
 * call).  Bit copies, no arithmetic.  Device values out of range (slot
 * outside the table, negative position, block id outside the pool) make the
 * affected rows be skipped, never an out-of-bounds access. */
hwkv_status hwkv_append(const hwkv_layout *layout, const hwkv_cache *cache,
                        int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                        const int32_t *seq_slots, const int64_t *pos0,
                        int32_t n_new, const void *k, const void *v,
                        hipStream_t stream);

/* Decode attention, first stage: for each (layer, sequence b, kv head h) the
 * window [max(0, L-w), L) with L = ctx_len[b] (the newest token already
 * appended) is cut into splits of split_tokens tokens; each split writes
 * running max m, sum l and acc = sum_t 2^(s_t-m) v_t for the G = n_q_heads /
 * n_kv_heads query heads of the group (query head i reads kv head i / G),
 * s_t = log2(e) * scale * q_i . k_t.  q: device [n_layers][n_seqs][n_q_heads]
 * [head_dim] in the layout's dtype.  workspace: hwkv_workspace_bytes.
 * scale: finite and > 0.  Arithmetic: q . k sums exact products in fp32;
 * for 16-bit caches the weights 2^(s_t - m) enter acc as 16-bit parts that
 * sum to them within ~2^-22 relative (matrix-core products, fp32
 * accumulation), for fp32 caches as fp32. */
hwkv_status hwkv_decode_split(const hwkv_layout *layout, const hwkv_cache *cache,
                              int32_t layer_begin, int32_t n_layers,
                              int32_t n_seqs, const int32_t *seq_slots,
                              const int64_t *ctx_len, int32_t n_q_heads,
                              const void *q, float scale, void *workspace,
                              uint64_t workspace_bytes, hipStream_t stream);

/* Decode attention, second stage: per (layer, sequence, query head) combine
 * the splits: M = max m_s, o = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s.
 * out: device [n_layers][n_seqs][n_q_heads][head_dim] as out_dtype (F32, or
 * BF16 / F16 rounded to nearest even from fp32).  A sequence with
 * ctx_len <= 0 gets zeros.  Same layer range, n_seqs, ctx_len
 * and workspace as the split stage (the merge reads only the workspace and
 * ctx_len, so n_seqs may exceed the table's rows, as a split stage given
 * seq_slots allows). */
hwkv_status hwkv_decode_merge(const hwkv_layout *layout, const hwkv_cache *cache,
                              int32_t layer_begin, int32_t n_layers,
                              int32_t n_seqs, const int64_t *ctx_len,
                              int32_t n_q_heads, const void *workspace,
                              uint64_t workspace_bytes, void *out,
                              hwkv_dtype out_dtype, hipStream_t stream);

/* Decode attention over exactly the last w_h tokens of every head (write-up
 * 摘要: per-head residency, not a mask): hwkv_decode_split followed by
 * hwkv_decode_merge on the same stream.  Call hwkv_append for the new token
 * first. */
hwkv_status hwkv_decode_attn(const hwkv_layout *layout, const hwkv_cache *cache,
                             int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                             const int32_t *seq_slots, const int64_t *ctx_len,
                             int32_t n_q_heads, const void *q, float scale,
                             void *workspace, uint64_t workspace_bytes, void *out,
                             hwkv_dtype out_dtype, hipStream_t stream);

/* First stage of hwkv_decode_append_attn: hwkv_decode_split at context
 * pos + 1 whose split covering the new token also writes that token's K/V
 * rows (k_new, v_new: device [n_layers][n_seqs][n_kv_heads][head_dim]) into
 * its ring slot and folds them from the arguments.  Follow it with
 * hwkv_decode_merge given ctx_len = pos + 1. */
hwkv_status hwkv_decode_split_append(const hwkv_layout *layout, const hwkv_cache *cache,
                                     int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                     const int32_t *seq_slots, const int64_t *pos,
                                     const void *k_new, const void *v_new,
                                     int32_t n_q_heads, const void *q, float scale,
                                     void *workspace, uint64_t workspace_bytes,
                                     hipStream_t stream);

/* The effect of hwkv_append of one token at position pos[b] (k_new, v_new:
 * device [n_layers][n_seqs][n_kv_heads][head_dim]) followed by
 * hwkv_decode_attn with ctx_len = pos + 1, with the same results bit for bit,
 * in two launches instead of three: the split that covers the new token
 * writes its rows into the ring slot (the slot's previous token lies outside
 * every window that reads the block, page 2 "SWA Window") and folds them from
 * the arguments; the merge stage follows.  workspace: hwkv_workspace_bytes.
 * A sequence with pos < 0 gets zeros and no append; an invalid slot gets NaN
 * and no append. */
hwkv_status hwkv_decode_append_attn(const hwkv_layout *layout, const hwkv_cache *cache,
                                    int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                    const int32_t *seq_slots, const int64_t *pos,
                                    const void *k_new, const void *v_new,
                                    int32_t n_q_heads, const void *q, float scale,
                                    void *workspace, uint64_t workspace_bytes, void *out,
                                    hwkv_dtype out_dtype, hipStream_t stream);

/* hwkv_decode_append_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches and the same results bit for bit, with the
 * split records in a scratch array of HWKV_STATIC_SCRATCH_BYTES that the
 * library keeps on every device it runs on until the process ends, instead
 * of a caller workspace.  The call allocates nothing; the first call on a
 * device looks the array's address up (make it outside graph capture).
 * HWKV_ERR_CAPACITY when hwkv_workspace_bytes of the call exceeds the array
 * (e.g. the 48-layer 112K stack fits up to 5 sequences per call at the
 * default split).  All calls on one device share its array: two such calls
 * that overlap in time on one device (different streams) race; calls on one
 * stream are ordered and safe. */
#define HWKV_STATIC_SCRATCH_BYTES (64ull << 20)
hwkv_status hwkv_decode_append_attn_static(const hwkv_layout *layout,
                                           const hwkv_cache *cache, int32_t layer_begin,
                                           int32_t n_layers, int32_t n_seqs,
                                           const int32_t *seq_slots, const int64_t *pos,
                                           const void *k_new, const void *v_new,
                                           int32_t n_q_heads, const void *q, float scale,
                                           void *out, hwkv_dtype out_dtype,
                                           hipStream_t stream);

/* Device workspace of hwkv_decode_step: the hwkv_workspace_bytes records,
 * padded to 256 bytes, then one uint32 arrival counter per (layer, kv head,
 * sequence).  The counters must be zero before the first hwkv_decode_step on
 * a workspace (zero-fill it once); every call leaves them zero again. */
hwkv_status hwkv_step_workspace_bytes(const hwkv_layout *layout, int32_t layer_begin,
                                      int32_t n_layers, int32_t n_seqs,
                                      int32_t n_q_heads, uint64_t *bytes);

/* One decode step in a single launch: the effect of hwkv_append of one token
 * at position pos[b] (k_new, v_new: device [n_layers][n_seqs][n_kv_heads]
 * [head_dim]) followed by hwkv_decode_attn with ctx_len = pos + 1, with the
 * same results bit for bit.  The split that covers the new token also writes
 * it into its ring slot (that slot's previous token is outside every window
 * that reads the block, page 2 "SWA Window") and takes its K/V rows from the
 * arguments; each split counts its arrival in the workspace and the last one
 * of a head merges, so no separate merge launch is needed.  Two calls that
 * overlap on one workspace race (they share the counters).  A sequence with
 * pos < 0 gets zeros and no append; an invalid slot gets NaN and no append. */
hwkv_status hwkv_decode_step(const hwkv_layout *layout, const hwkv_cache *cache,
                             int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                             const int32_t *seq_slots, const int64_t *pos,
                             const void *k_new, const void *v_new, int32_t n_q_heads,
                             const void *q, float scale, void *workspace,
                             uint64_t workspace_bytes, void *out, hwkv_dtype out_dtype,
                             hipStream_t stream);

/* Device workspace of hwkv_prefill_attn for layer `layer`, n_seqs sequences
 * and chunks of n_chunk rows.  BF16 caches: the fp16 copy of the V rows the
 * call reads, w - 1 + n_chunk rows of head_dim fp16 values per (sequence, kv
 * head), heads in order, sequences in order.  F16 and F32 caches need none
 * (0 bytes).  The pages give no prefill kernel; this buffer belongs to this
 * library's form of it (see hwkv_prefill_attn).  HWKV_ERR_UNSUPPORTED when one
 * head's rows would take 2^31 bytes or more (hwkv_prefill_attn_exact needs no
 * workspace); HWKV_ERR_INVALID_ARG for a layer out of range, n_seqs < 1 or
 * n_chunk < 1. */
hwkv_status hwkv_prefill_workspace_bytes(const hwkv_layout *layout, int32_t layer,
                                         int32_t n_seqs, int32_t n_chunk,
                                         uint64_t *bytes);

/* Chunked prefill of one layer.  The pages define the per-head window (摘要,
 * 核心技术 2; "KV Cache Consistency Practices ...", "SWA Window") but no
 * prefill kernel: this is the same windowed attention for a chunk of new
 * query rows, causal inside the chunk.  Sequence b has history [0, P) in the cache,
 * P = pos0[b], and n_chunk new tokens at [P, P+n_chunk).  Query row r
 * (position p = P + r) of query head i attends to kv head i / G over
 * [max(0, p-w+1), p]: keys before P are read from the cache (only the last
 * w-1 of them can be needed, and the ring holds at least w), keys from P on
 * from k, v.  q: device [n_seqs][n_chunk][n_q_heads][head_dim]; k, v: device
 * [n_seqs][n_chunk][n_kv_heads][head_dim]; out: [n_seqs][n_chunk][n_q_heads]
 * [head_dim] as out_dtype (F32, BF16 or F16).  workspace: device memory of
 * hwkv_prefill_workspace_bytes (256-byte aligned; null allowed when that is
 * 0), scratch of this call only: its contents on return mean nothing, and
 * two calls in flight on one workspace race.  The cache is read, not written: call hwkv_append
 * with the same k, v (n_layers = 1) afterwards, since appending first could
 * overwrite history that earlier rows of the chunk still need.  Runs on
 * MFMA tiles (bf16 or fp16 operands, fp32 accumulation).  scale: finite
 * and > 0.  Bad slots, positions and block ids give NaN rows as stated at
 * the top of this header.
 *
 * Precision of the softmax weights P in the P.V product: they are rounded
 * once to fp16 (11 significant bits; row error a few 1e-4 of the row's
 * largest output on N(0,1) data).  For BF16 caches this needs V in fp16: a
 * first kernel writes the fp16 copy of the V rows the call reads into the
 * workspace (rounded to nearest even, exact for |v| in [2^-14, 65504]).  A
 * query row whose result comes out non-finite (a V element beyond fp16's
 * range) or whose largest magnitude is below 2^-12 of its softmax sum (where
 * the conversion's absolute error, at most 2^-25 per element, could matter)
 * is recomputed as hwkv_prefill_attn_exact does, from the cache's bf16 V, so
 * such inputs cost time, not accuracy.  For BF16 caches the call enqueues
 * three kernels: the fp16 copy, the fp16 pass, which writes such rows as NaN,
 * and a second pass that exits at once unless a row of its workgroup is NaN,
 * in which case it recomputes the workgroup exactly and rewrites those rows
 * (rows that are NaN by the rules above come out NaN again). */
hwkv_status hwkv_prefill_attn(const hwkv_layout *layout, const hwkv_cache *cache,
                              int32_t layer, int32_t n_seqs,
                              const int32_t *seq_slots, const int64_t *pos0,
                              int32_t n_chunk, int32_t n_q_heads, const void *q,
                              const void *k, const void *v, void *workspace,
                              uint64_t workspace_bytes, void *out,
                              hwkv_dtype out_dtype, float scale,
                              hipStream_t stream);

/* hwkv_prefill_attn with the P.V product at ~16-bit precision for BF16
 * caches: P is split into its truncation to bf16 and the remainder rounded
 * to bf16, two bf16 products (row error ~1e-5 of the row's largest output),
 * at about 25-30% more time; one kernel, no workspace.  For F16 caches it is
 * hwkv_prefill_attn.  Same arguments (without the workspace), layouts and
 * errors. */
hwkv_status hwkv_prefill_attn_exact(const hwkv_layout *layout,
                                    const hwkv_cache *cache, int32_t layer,
                                    int32_t n_seqs, const int32_t *seq_slots,
                                    const int64_t *pos0, int32_t n_chunk,
                                    int32_t n_q_heads, const void *q,
                                    const void *k, const void *v, void *out,
                                    hwkv_dtype out_dtype, float scale,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HWKV_H */
