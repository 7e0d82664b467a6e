// Internal declarations shared by the host runtime and the HIP kernels of
// libhwkv.  Nothing here is part of the C ABI (include/hwkv.h is).
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "hwkv.h"

namespace hwkv {

constexpr uint32_t kMetaMagic = 0x564B5748u;  // "HWKV"
constexpr int kDefaultSplitTokens = 1024;
constexpr int kMaxSplitTokens = 2048;
// Split launches of at least this many workgroups write their records with
// non-temporal stores (see rec_put in decode.hip).
constexpr int64_t kStreamedRecordsMinWorkgroups = 2048;
constexpr int kMaxBlockSize = 1024;
constexpr int kMaxHeadDim = 1024;

// Default decode split length: the largest multiple of the block size not
// above 1024 tokens (at least one block).
inline int32_t default_split_tokens(int32_t block_size) {
    const int32_t n = kDefaultSplitTokens / block_size;
    return (n < 1 ? 1 : n) * block_size;
}
constexpr int kMetaAlign = 256;

// Per-head descriptor in the device meta blob (32 bytes, one scalar load).
struct HeadDesc {
    int64_t table_off;   // first entry of this head inside a block-table row
    int32_t window;      // w_h in tokens
    int32_t nblocks;     // ceil(w_h / block_size): ring of nblocks blocks
    int32_t work_off;    // index of this head's first decode work item
    int32_t max_splits;  // ceil(w_h / split_tokens)
    int32_t layer;
    int32_t head;
};
static_assert(sizeof(HeadDesc) == 32, "HeadDesc must stay 32 bytes");

// One decode work item: split `split` of head `head_index` (layer-major).
struct WorkItem {
    int32_t head_index;
    int32_t split;
};

// Header at offset 0 of the meta blob.
struct MetaHeader {
    uint32_t magic;
    uint32_t abi;
    uint64_t fingerprint;
    int32_t n_layers, n_kv_heads, block_size, head_dim;
    int32_t dtype, split_tokens;
    int64_t blocks_per_seq;
    int64_t n_work;
    uint64_t heads_off;       // byte offset of HeadDesc[n_layers*n_kv_heads]
    uint64_t layer_work_off;  // byte offset of int32[n_layers+1]
    uint64_t work_off;        // byte offset of WorkItem[n_work]
    uint64_t order_off;       // byte offset of int32[n_layers][n_kv_heads]
};

}  // namespace hwkv

// The opaque host layout.
struct hwkv_layout {
    int32_t n_layers = 0, n_kv_heads = 0, block_size = 0, head_dim = 0;
    hwkv_dtype dtype = HWKV_BF16;
    int32_t split_tokens = 0;
    int32_t max_window = 0;
    int64_t blocks_per_seq = 0;
    int64_t n_work = 0;
    uint64_t block_bytes = 0;
    uint64_t meta_bytes = 0;
    uint64_t fingerprint = 0;
    std::vector<int32_t> windows, nblocks;
    std::vector<int64_t> head_off;        // n_heads + 1
    std::vector<int32_t> layer_work_off;  // n_layers + 1
    std::vector<hwkv::HeadDesc> heads;
    std::vector<hwkv::WorkItem> work;
    std::vector<int32_t> order;  // per layer: kv heads by window, longest first
    uint64_t heads_off = 0, layer_work_off_bytes = 0, work_off = 0, order_off = 0;
};

namespace hwkv {

// Thread-local error message plumbing (defined in layout.cpp).
hwkv_status fail(hwkv_status st, const std::string& msg);
void clear_error();

inline int elem_bytes(hwkv_dtype dt) { return dt == HWKV_F32 ? 4 : 2; }

// Floats in one decode partial record: acc[G][d], m[G], l[G], padded to 4.
inline int64_t record_floats(int group, int head_dim) {
    int64_t n = (int64_t)group * head_dim + 2 * (int64_t)group;
    return (n + 3) / 4 * 4;
}

// ---------------------------------------------------------------------------
// Kernel argument blocks (passed by value) and launchers (decode.hip,
// append.hip, prefill.hip).
// ---------------------------------------------------------------------------

struct AppendArgs {
    uint8_t* pool;
    uint64_t n_pool_blocks;
    uint64_t block_bytes;
    const int32_t* block_ids;
    int64_t table_rows;
    int64_t blocks_per_seq;
    const uint8_t* meta;
    const HeadDesc* heads;
    uint64_t fingerprint;
    const int32_t* seq_slots;
    const int64_t* pos0;
    const uint8_t* k;
    const uint8_t* v;
    int32_t layer_begin, n_layers, n_seqs, n_new, n_kv_heads;
    int32_t block_size;
    int32_t row_chunks;  // 16-byte chunks per K (or V) row
    int64_t n_chunks;    // total 16-byte chunks of K (same for V)
};

struct DecodeSplitArgs {
    const uint8_t* pool;
    uint64_t n_pool_blocks;
    uint64_t block_bytes;
    const int32_t* block_ids;
    int64_t table_rows;
    int64_t blocks_per_seq;
    const uint8_t* meta;
    const HeadDesc* heads;
    const WorkItem* work;
    uint64_t fingerprint;
    const int32_t* seq_slots;
    const int64_t* ctx_len;
    const uint8_t* q;
    float* ws;
    int32_t work_begin, n_work_range;
    int32_t layer_begin, n_seqs, n_q_heads;
    int32_t split_tokens;
    int32_t rec_floats;
    int32_t tpb_log2;     // log2(block_size / 16): 16-token tiles per block
    float qk_scale_log2;  // scale * log2(e)
    // 1: records are written with non-temporal stores (launches long enough
    // that their write-back would compete with the K/V read stream); 0:
    // ordinary stores, which the merge stage reads back sooner
    int32_t rec_streamed;
    // Appending modes (hwkv_decode_append_attn, hwkv_decode_step): ctx_len
    // then holds the new token's position (context = position + 1) and the
    // token's K/V rows are appended by the split that covers it; in the
    // single-launch step the last split of a head to finish (per-(layer, kv
    // head, sequence) arrival counter) also merges.
    const uint8_t* k_new;
    const uint8_t* v_new;
    uint8_t* pool_w;
    uint32_t* counters;
    void* out;
    int32_t out_kind;  // element type of out (hwkv_dtype): F32, BF16 or F16
    int32_t n_kv_heads;
    int32_t n_layers;
};

struct DecodeMergeArgs {
    const uint8_t* meta;
    const HeadDesc* heads;
    uint64_t fingerprint;
    const int64_t* ctx_len;
    const float* ws;
    void* out;
    int32_t work_begin, n_work_range;
    int32_t layer_begin, n_layers, n_seqs, n_q_heads, n_kv_heads;
    int32_t split_tokens;
    int32_t rec_floats;
    int32_t out_kind;  // element type of out (hwkv_dtype): F32, BF16 or F16
    int32_t ctx_add;  // context = ctx_len[b] + ctx_add (1 when given positions)
    int32_t merge_chunks;  // column chunks per workgroup (set by the launcher)
};

struct PrefillArgs {
    const uint8_t* pool;
    uint64_t n_pool_blocks;
    uint64_t block_bytes;
    const int32_t* block_ids;
    int64_t table_rows;
    int64_t blocks_per_seq;
    const uint8_t* meta;
    const HeadDesc* heads;
    const int32_t* order;  // kv heads of each layer, longest window first
    uint64_t fingerprint;
    const int32_t* seq_slots;
    const int64_t* pos0;
    const uint8_t* q;
    const uint8_t* k;
    const uint8_t* v;
    void* out;
    int32_t layer, n_seqs, n_chunk, n_q_heads, n_kv_heads;
    int32_t out_kind;  // element type of out (hwkv_dtype): F32, BF16 or F16
    int32_t tpb_log2;  // log2(block_size / 16)
    int32_t exact_p;   // bf16 caches: P split into two bf16 products, no fp16 pass
    float qk_scale_log2;
    // bf16 caches, fp16 pass: the workspace holding, per (sequence, kv head),
    // fp16 copies of the V rows of keys [P - w + 1, P + n_chunk) (w - 1 + n_chunk
    // rows, heads in order); v16_seq_rows = rows per sequence
    uint8_t* v16;
    int64_t v16_seq_rows;
};

// Rows of the fp16 V copy one sequence of a prefill call needs:
// sum over the layer's kv heads of (w_h - 1 + n_chunk).
inline int64_t prefill_v16_rows(const hwkv_layout& lay, int32_t layer, int32_t n_chunk) {
    int64_t rows = 0;
    for (int32_t h = 0; h < lay.n_kv_heads; h++)
        rows += (int64_t)lay.windows[(size_t)layer * lay.n_kv_heads + h] - 1 + n_chunk;
    return rows;
}

// Device address of the library's static decode scratch (the records of
// hwkv_decode_append_attn_static) on the device that `stream` runs on: a
// file-scope array of HWKV_STATIC_SCRATCH_BYTES in decode.hip, looked up once
// per device with hipGetSymbolAddress and kept.
hwkv_status static_scratch(hipStream_t stream, void** ptr);

hwkv_status launch_append(const hwkv_layout& lay, const AppendArgs& a, hipStream_t s);
hwkv_status launch_decode_split(const hwkv_layout& lay, int group, const DecodeSplitArgs& a,
                                hipStream_t s);
hwkv_status launch_decode_merge(const hwkv_layout& lay, int group, const DecodeMergeArgs& a,
                                hipStream_t s);
hwkv_status launch_prefill(const hwkv_layout& lay, int group, const PrefillArgs& a,
                           hipStream_t s);
hwkv_status launch_decode_step(const hwkv_layout& lay, int group, const DecodeSplitArgs& a,
                               hipStream_t s);
hwkv_status launch_decode_split_append(const hwkv_layout& lay, int group,
                                       const DecodeSplitArgs& a, hipStream_t s);

// Whether a kernel instance exists for a layout (block size, head_dim, dtype)
// and GQA group size.
bool append_supported(const hwkv_layout& lay);
bool decode_supported(const hwkv_layout& lay, int group);
bool prefill_supported(const hwkv_layout& lay, int group);

}  // namespace hwkv
