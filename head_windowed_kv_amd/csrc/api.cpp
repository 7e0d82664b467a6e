// Device entry points of libhwkv: every argument is validated on the host,
// then the kernels are enqueued on the caller's stream.  Nothing is
// allocated, copied or synchronised here, so each call can be captured in a
// HIP graph (page 1, section 5, and page 2, "Static Topology Constraint":
// the recovery/read path must be fixed at capture time).
#include <math.h>
#include <stdint.h>

#include <string>

#include "hwkv_internal.h"

using namespace hwkv;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

std::string hex64(uint64_t x) {
    static const char* digits = "0123456789abcdef";
    std::string s = "0x";
    for (int i = 60; i >= 0; i -= 4) s += digits[(x >> i) & 15];
    return s;
}

// the softmax scale: finite and positive (a non-positive scale would turn
// the masked scores' -inf into +inf or NaN in the kernels' log2 domain)
hwkv_status check_scale(float scale) {
    if (!(isfinite(scale) && scale > 0.f))
        return fail(HWKV_ERR_INVALID_ARG, "scale must be finite and > 0");
    return HWKV_OK;
}

// Checks shared by every device call: the cache view, its alignment and the
// pool capacity.  A pool smaller than the exact estimate for table_rows rows
// is reported in the form of the write-up's operations table, naming the first
// (layer, head) whose blocks do not fit.
hwkv_status check_cache(const hwkv_layout* L, const hwkv_cache* c) {
    if (!L) return fail(HWKV_ERR_INVALID_ARG, "null layout");
    if (!c) return fail(HWKV_ERR_INVALID_ARG, "null cache view");
    if (!c->pool || !c->block_ids || !c->meta)
        return fail(HWKV_ERR_INVALID_ARG, "cache view has a null pool, block_ids or meta");
    if (!aligned(c->pool, 256) || !aligned(c->block_ids, 256) || !aligned(c->meta, 256))
        return fail(HWKV_ERR_MISALIGNED, "pool, block_ids and meta must be 256-byte aligned");
    if (c->table_rows < 1) return fail(HWKV_ERR_INVALID_ARG, "table_rows must be >= 1");
    // kernel-ABI check ("KV Cache Management in Hybrid Attention LLMs", 4.2):
    // the cache's blob must have been written for this very layout
    if (c->meta_fingerprint != L->fingerprint)
        return fail(HWKV_ERR_ABI_MISMATCH,
                    "the cache's meta blob has fingerprint " + hex64(c->meta_fingerprint) +
                        ", the layout of this call " + hex64(L->fingerprint) +
                        " (another layout, or another ABI version)");
    return hwkv_capacity_check(L, c->table_rows, c->pool_bytes, nullptr, nullptr, nullptr);
}

// reads_table: the call looks rows up in the block table (every stage except
// the merge, which reads only the workspace and the contexts)
hwkv_status check_batch(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                        int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                        bool reads_table = true) {
    if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > L->n_layers)
        return fail(HWKV_ERR_INVALID_ARG, "layer range [" + std::to_string(layer_begin) + ", " +
                                              std::to_string(layer_begin + n_layers) +
                                              ") outside the layout's " +
                                              std::to_string(L->n_layers) + " layers");
    if (n_seqs < 1 || n_seqs > 65535)
        return fail(HWKV_ERR_INVALID_ARG, "n_seqs must be in [1, 65535]");
    if (reads_table && !seq_slots && n_seqs > c->table_rows)
        return fail(HWKV_ERR_INVALID_ARG, "no seq_slots and n_seqs > table_rows");
    if (seq_slots && !aligned(seq_slots, 4))
        return fail(HWKV_ERR_MISALIGNED, "seq_slots must be 4-byte aligned");
    return HWKV_OK;
}

hwkv_status check_group(const hwkv_layout* L, int32_t n_q_heads, int* group) {
    if (n_q_heads < 1 || n_q_heads % L->n_kv_heads != 0)
        return fail(HWKV_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
    *group = n_q_heads / L->n_kv_heads;
    return HWKV_OK;
}

hwkv_status check_workspace(const hwkv_layout* L, int32_t layer_begin, int32_t n_layers,
                            int32_t n_seqs, int32_t n_q_heads, const void* ws,
                            uint64_t ws_bytes) {
    uint64_t need = 0;
    hwkv_status st = hwkv_workspace_bytes(L, layer_begin, n_layers, n_seqs, n_q_heads, &need);
    if (st != HWKV_OK) return st;
    if (!ws) return fail(HWKV_ERR_INVALID_ARG, "null workspace");
    if (!aligned(ws, 256)) return fail(HWKV_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(HWKV_ERR_CAPACITY, "workspace of " + std::to_string(ws_bytes) +
                                           " bytes, need " + std::to_string(need));
    return HWKV_OK;
}

uint64_t pool_blocks(const hwkv_layout* L, const hwkv_cache* c) {
    return c->pool_bytes / L->block_bytes;
}

#define HWKV_TRY(expr)                      \
    do {                                    \
        hwkv_status st_ = (expr);           \
        if (st_ != HWKV_OK) return st_;     \
    } while (0)

}  // namespace

extern "C" {

hwkv_status hwkv_append(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                        int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                        const int64_t* pos0, int32_t n_new, const void* k, const void* v,
                        hipStream_t stream) {
    clear_error();
    HWKV_TRY(check_cache(L, c));
    HWKV_TRY(check_batch(L, c, layer_begin, n_layers, n_seqs, seq_slots));
    if (!append_supported(*L))
        return fail(HWKV_ERR_UNSUPPORTED, "no append kernel for rows of " +
                                              std::to_string(L->head_dim * elem_bytes(L->dtype)) +
                                              " bytes (rows must be a multiple of 16 bytes)");
    if (n_new < 1) return fail(HWKV_ERR_INVALID_ARG, "n_new must be >= 1");
    if (!pos0 || !k || !v) return fail(HWKV_ERR_INVALID_ARG, "null pos0, k or v");
    if (!aligned(pos0, 8)) return fail(HWKV_ERR_MISALIGNED, "pos0 must be 8-byte aligned");
    if (!aligned(k, 16) || !aligned(v, 16))
        return fail(HWKV_ERR_MISALIGNED, "k and v must be 16-byte aligned");
    const uint64_t row_bytes = (uint64_t)L->head_dim * elem_bytes(L->dtype);
    const uint64_t rows = (uint64_t)n_layers * n_seqs * (uint64_t)n_new * L->n_kv_heads;
    if (rows > (uint64_t)1 << 40) return fail(HWKV_ERR_OVERFLOW, "append too large");
    AppendArgs a{};
    a.pool = static_cast<uint8_t*>(c->pool);
    a.n_pool_blocks = pool_blocks(L, c);
    a.block_bytes = L->block_bytes;
    a.block_ids = c->block_ids;
    a.table_rows = c->table_rows;
    a.blocks_per_seq = L->blocks_per_seq;
    a.meta = static_cast<const uint8_t*>(c->meta);
    a.heads = reinterpret_cast<const HeadDesc*>(a.meta + L->heads_off);
    a.fingerprint = L->fingerprint;
    a.seq_slots = seq_slots;
    a.pos0 = pos0;
    a.k = static_cast<const uint8_t*>(k);
    a.v = static_cast<const uint8_t*>(v);
    a.layer_begin = layer_begin;
    a.n_layers = n_layers;
    a.n_seqs = n_seqs;
    a.n_new = n_new;
    a.n_kv_heads = L->n_kv_heads;
    a.block_size = L->block_size;
    a.row_chunks = (int32_t)(row_bytes / 16);
    a.n_chunks = (int64_t)(rows * row_bytes / 16);
    return launch_append(*L, a, stream);
}

static hwkv_status split_args(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                              int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                              const int64_t* ctx_len, int32_t n_q_heads, const void* q,
                              float scale, void* ws, uint64_t ws_bytes, int* group,
                              DecodeSplitArgs* a) {
    HWKV_TRY(check_cache(L, c));
    HWKV_TRY(check_batch(L, c, layer_begin, n_layers, n_seqs, seq_slots));
    HWKV_TRY(check_group(L, n_q_heads, group));
    if (!decode_supported(*L, *group))
        return fail(HWKV_ERR_UNSUPPORTED, "no decode kernel for this block size, dtype, head_dim "
                                          "and GQA group size " + std::to_string(*group));
    HWKV_TRY(check_workspace(L, layer_begin, n_layers, n_seqs, n_q_heads, ws, ws_bytes));
    if (!ctx_len || !q) return fail(HWKV_ERR_INVALID_ARG, "null ctx_len or q");
    if (!aligned(ctx_len, 8)) return fail(HWKV_ERR_MISALIGNED, "ctx_len must be 8-byte aligned");
    if (!aligned(q, 16)) return fail(HWKV_ERR_MISALIGNED, "q must be 16-byte aligned");
    HWKV_TRY(check_scale(scale));
    *a = DecodeSplitArgs{};
    a->pool = static_cast<const uint8_t*>(c->pool);
    a->n_pool_blocks = pool_blocks(L, c);
    a->block_bytes = L->block_bytes;
    a->block_ids = c->block_ids;
    a->table_rows = c->table_rows;
    a->blocks_per_seq = L->blocks_per_seq;
    a->meta = static_cast<const uint8_t*>(c->meta);
    a->heads = reinterpret_cast<const HeadDesc*>(a->meta + L->heads_off);
    a->work = reinterpret_cast<const WorkItem*>(a->meta + L->work_off);
    a->fingerprint = L->fingerprint;
    a->seq_slots = seq_slots;
    a->ctx_len = ctx_len;
    a->q = static_cast<const uint8_t*>(q);
    a->ws = static_cast<float*>(ws);
    a->work_begin = L->layer_work_off[layer_begin];
    a->n_work_range = L->layer_work_off[layer_begin + n_layers] - a->work_begin;
    a->layer_begin = layer_begin;
    a->n_seqs = n_seqs;
    a->n_q_heads = n_q_heads;
    a->split_tokens = L->split_tokens;
    a->rec_floats = (int32_t)record_floats(*group, L->head_dim);
    a->tpb_log2 = 0;
    while ((16 << a->tpb_log2) < L->block_size) a->tpb_log2++;
    a->qk_scale_log2 = scale * 1.4426950408889634f;
    a->rec_streamed = (int64_t)a->n_work_range * n_seqs >= kStreamedRecordsMinWorkgroups;
    return HWKV_OK;
}

static hwkv_status merge_args(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                              int32_t n_layers, int32_t n_seqs, const int64_t* ctx_len,
                              int32_t n_q_heads, const void* ws, uint64_t ws_bytes, void* out,
                              hwkv_dtype out_dtype, int* group, DecodeMergeArgs* a) {
    HWKV_TRY(check_cache(L, c));
    HWKV_TRY(check_batch(L, c, layer_begin, n_layers, n_seqs, nullptr, false));
    HWKV_TRY(check_group(L, n_q_heads, group));
    if (!decode_supported(*L, *group))
        return fail(HWKV_ERR_UNSUPPORTED, "no decode kernel for this block size, dtype, head_dim "
                                          "and GQA group size " + std::to_string(*group));
    HWKV_TRY(check_workspace(L, layer_begin, n_layers, n_seqs, n_q_heads, ws, ws_bytes));
    if (!ctx_len || !out) return fail(HWKV_ERR_INVALID_ARG, "null ctx_len or out");
    if (!aligned(ctx_len, 8)) return fail(HWKV_ERR_MISALIGNED, "ctx_len must be 8-byte aligned");
    if (!aligned(out, 16)) return fail(HWKV_ERR_MISALIGNED, "out must be 16-byte aligned");
    if (out_dtype != HWKV_F32 && out_dtype != HWKV_BF16 && out_dtype != HWKV_F16)
        return fail(HWKV_ERR_INVALID_ARG, "out_dtype must be HWKV_F32, HWKV_BF16 or HWKV_F16");
    *a = DecodeMergeArgs{};
    a->meta = static_cast<const uint8_t*>(c->meta);
    a->heads = reinterpret_cast<const HeadDesc*>(a->meta + L->heads_off);
    a->fingerprint = L->fingerprint;
    a->ctx_len = ctx_len;
    a->ws = static_cast<const float*>(ws);
    a->out = out;
    a->work_begin = L->layer_work_off[layer_begin];
    a->n_work_range = L->layer_work_off[layer_begin + n_layers] - a->work_begin;
    a->layer_begin = layer_begin;
    a->n_layers = n_layers;
    a->n_seqs = n_seqs;
    a->n_q_heads = n_q_heads;
    a->n_kv_heads = L->n_kv_heads;
    a->split_tokens = L->split_tokens;
    a->rec_floats = (int32_t)record_floats(*group, L->head_dim);
    a->out_kind = out_dtype;
    a->ctx_add = 0;
    return HWKV_OK;
}

hwkv_status hwkv_decode_split(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                              int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                              const int64_t* ctx_len, int32_t n_q_heads, const void* q,
                              float scale, void* ws, uint64_t ws_bytes, hipStream_t stream) {
    clear_error();
    int group = 0;
    DecodeSplitArgs a;
    HWKV_TRY(split_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, ctx_len, n_q_heads, q,
                        scale, ws, ws_bytes, &group, &a));
    return launch_decode_split(*L, group, a, stream);
}

hwkv_status hwkv_decode_merge(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                              int32_t n_layers, int32_t n_seqs, const int64_t* ctx_len,
                              int32_t n_q_heads, const void* ws, uint64_t ws_bytes, void* out,
                              hwkv_dtype out_dtype, hipStream_t stream) {
    clear_error();
    int group = 0;
    DecodeMergeArgs a;
    HWKV_TRY(merge_args(L, c, layer_begin, n_layers, n_seqs, ctx_len, n_q_heads, ws, ws_bytes,
                        out, out_dtype, &group, &a));
    return launch_decode_merge(*L, group, a, stream);
}

hwkv_status hwkv_decode_attn(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                             int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                             const int64_t* ctx_len, int32_t n_q_heads, const void* q,
                             float scale, void* ws, uint64_t ws_bytes, void* out,
                             hwkv_dtype out_dtype, hipStream_t stream) {
    clear_error();
    int group = 0;
    DecodeSplitArgs sa;
    DecodeMergeArgs ma;
    // validate both stages before enqueueing either
    HWKV_TRY(split_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, ctx_len, n_q_heads, q,
                        scale, ws, ws_bytes, &group, &sa));
    HWKV_TRY(merge_args(L, c, layer_begin, n_layers, n_seqs, ctx_len, n_q_heads, ws, ws_bytes,
                        out, out_dtype, &group, &ma));
    HWKV_TRY(launch_decode_split(*L, group, sa, stream));
    return launch_decode_merge(*L, group, ma, stream);
}

static hwkv_status split_append_args(const hwkv_layout* L, const hwkv_cache* c,
                                     int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                     const int32_t* seq_slots, const int64_t* pos,
                                     const void* k_new, const void* v_new, int32_t n_q_heads,
                                     const void* q, float scale, void* ws, uint64_t ws_bytes,
                                     int* group, DecodeSplitArgs* a) {
    // pos plays the part of ctx_len (context = pos + 1) in the shared checks
    HWKV_TRY(split_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, n_q_heads, q, scale,
                        ws, ws_bytes, group, a));
    if (!k_new || !v_new) return fail(HWKV_ERR_INVALID_ARG, "null k_new or v_new");
    if (!aligned(k_new, 16) || !aligned(v_new, 16))
        return fail(HWKV_ERR_MISALIGNED, "k_new and v_new must be 16-byte aligned");
    a->k_new = static_cast<const uint8_t*>(k_new);
    a->v_new = static_cast<const uint8_t*>(v_new);
    a->pool_w = static_cast<uint8_t*>(c->pool);
    a->n_kv_heads = L->n_kv_heads;
    a->n_layers = n_layers;
    return HWKV_OK;
}

hwkv_status hwkv_decode_split_append(const hwkv_layout* L, const hwkv_cache* c,
                                     int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                     const int32_t* seq_slots, const int64_t* pos,
                                     const void* k_new, const void* v_new, int32_t n_q_heads,
                                     const void* q, float scale, void* ws, uint64_t ws_bytes,
                                     hipStream_t stream) {
    clear_error();
    int group = 0;
    DecodeSplitArgs sa;
    HWKV_TRY(split_append_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, k_new, v_new,
                               n_q_heads, q, scale, ws, ws_bytes, &group, &sa));
    return launch_decode_split_append(*L, group, sa, stream);
}

static hwkv_status decode_append_attn(const hwkv_layout* L, const hwkv_cache* c,
                                      int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                      const int32_t* seq_slots, const int64_t* pos,
                                      const void* k_new, const void* v_new, int32_t n_q_heads,
                                      const void* q, float scale, void* ws, uint64_t ws_bytes,
                                      void* out, hwkv_dtype out_dtype, hipStream_t stream) {
    int group = 0;
    DecodeSplitArgs sa;
    DecodeMergeArgs ma;
    // validate both stages before enqueueing either
    HWKV_TRY(split_append_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, k_new, v_new,
                               n_q_heads, q, scale, ws, ws_bytes, &group, &sa));
    HWKV_TRY(merge_args(L, c, layer_begin, n_layers, n_seqs, pos, n_q_heads, ws, ws_bytes, out,
                        out_dtype, &group, &ma));
    ma.ctx_add = 1;
    HWKV_TRY(launch_decode_split_append(*L, group, sa, stream));
    return launch_decode_merge(*L, group, ma, stream);
}

hwkv_status hwkv_decode_append_attn(const hwkv_layout* L, const hwkv_cache* c,
                                    int32_t layer_begin, int32_t n_layers, int32_t n_seqs,
                                    const int32_t* seq_slots, const int64_t* pos,
                                    const void* k_new, const void* v_new, int32_t n_q_heads,
                                    const void* q, float scale, void* ws, uint64_t ws_bytes,
                                    void* out, hwkv_dtype out_dtype, hipStream_t stream) {
    clear_error();
    return decode_append_attn(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, k_new, v_new,
                              n_q_heads, q, scale, ws, ws_bytes, out, out_dtype, stream);
}

hwkv_status hwkv_decode_append_attn_static(const hwkv_layout* L, const hwkv_cache* c,
                                           int32_t layer_begin, int32_t n_layers,
                                           int32_t n_seqs, const int32_t* seq_slots,
                                           const int64_t* pos, const void* k_new,
                                           const void* v_new, int32_t n_q_heads, const void* q,
                                           float scale, void* out, hwkv_dtype out_dtype,
                                           hipStream_t stream) {
    clear_error();
    uint64_t need = 0;
    HWKV_TRY(hwkv_workspace_bytes(L, layer_begin, n_layers, n_seqs, n_q_heads, &need));
    if (need > HWKV_STATIC_SCRATCH_BYTES)
        return fail(HWKV_ERR_CAPACITY,
                    "this call needs " + std::to_string(need) + " bytes of split records; the "
                    "static scratch holds " + std::to_string(HWKV_STATIC_SCRATCH_BYTES) +
                    " (fewer layers or sequences per call, or hwkv_decode_append_attn with a "
                    "caller workspace)");
    void* ws = nullptr;
    HWKV_TRY(static_scratch(stream, &ws));
    return decode_append_attn(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, k_new, v_new,
                              n_q_heads, q, scale, ws, HWKV_STATIC_SCRATCH_BYTES, out, out_dtype,
                              stream);
}

hwkv_status hwkv_decode_step(const hwkv_layout* L, const hwkv_cache* c, int32_t layer_begin,
                             int32_t n_layers, int32_t n_seqs, const int32_t* seq_slots,
                             const int64_t* pos, const void* k_new, const void* v_new,
                             int32_t n_q_heads, const void* q, float scale, void* ws,
                             uint64_t ws_bytes, void* out, hwkv_dtype out_dtype,
                             hipStream_t stream) {
    clear_error();
    int group = 0;
    DecodeSplitArgs a;
    uint64_t rec_bytes = 0, need = 0;
    // pos plays the part of ctx_len (context = pos + 1) in the shared checks
    HWKV_TRY(split_args(L, c, layer_begin, n_layers, n_seqs, seq_slots, pos, n_q_heads, q, scale,
                        ws, ws_bytes, &group, &a));
    HWKV_TRY(hwkv_workspace_bytes(L, layer_begin, n_layers, n_seqs, n_q_heads, &rec_bytes));
    HWKV_TRY(hwkv_step_workspace_bytes(L, layer_begin, n_layers, n_seqs, n_q_heads, &need));
    if (ws_bytes < need)
        return fail(HWKV_ERR_CAPACITY, "step workspace of " + std::to_string(ws_bytes) +
                                           " bytes, need " + std::to_string(need));
    if (!k_new || !v_new || !out) return fail(HWKV_ERR_INVALID_ARG, "null k_new, v_new or out");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(out, 16))
        return fail(HWKV_ERR_MISALIGNED, "k_new, v_new and out must be 16-byte aligned");
    if (out_dtype != HWKV_F32 && out_dtype != HWKV_BF16 && out_dtype != HWKV_F16)
        return fail(HWKV_ERR_INVALID_ARG, "out_dtype must be HWKV_F32, HWKV_BF16 or HWKV_F16");
    a.k_new = static_cast<const uint8_t*>(k_new);
    a.v_new = static_cast<const uint8_t*>(v_new);
    a.pool_w = static_cast<uint8_t*>(c->pool);
    a.counters = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + (rec_bytes + 255) / 256 * 256);
    a.out = out;
    a.out_kind = out_dtype;
    a.n_kv_heads = L->n_kv_heads;
    a.n_layers = n_layers;
    return launch_decode_step(*L, group, a, stream);
}

hwkv_status hwkv_prefill_workspace_bytes(const hwkv_layout* L, int32_t layer, int32_t n_seqs,
                                         int32_t n_chunk, uint64_t* bytes) {
    clear_error();
    if (!L || !bytes) return fail(HWKV_ERR_INVALID_ARG, "null layout or bytes");
    if (layer < 0 || layer >= L->n_layers)
        return fail(HWKV_ERR_INVALID_ARG, "layer " + std::to_string(layer) + " outside the layout's " +
                                              std::to_string(L->n_layers) + " layers");
    if (n_seqs < 1 || n_chunk < 1) return fail(HWKV_ERR_INVALID_ARG, "n_seqs and n_chunk must be >= 1");
    *bytes = 0;
    if (L->dtype != HWKV_BF16) return HWKV_OK;  // only bf16 caches take the fp16 copy
    const uint64_t row = (uint64_t)L->head_dim * 2;
    for (int32_t h = 0; h < L->n_kv_heads; h++) {
        const uint64_t rows = (uint64_t)L->windows[(size_t)layer * L->n_kv_heads + h] - 1 + n_chunk;
        if (rows * row >= (1ull << 31))
            return fail(HWKV_ERR_UNSUPPORTED,
                        "kv head " + std::to_string(h) + ": window - 1 + n_chunk = " +
                            std::to_string(rows) + " fp16 V rows take 2^31 bytes or more "
                            "(hwkv_prefill_attn_exact needs no workspace)");
    }
    const uint64_t per_seq = (uint64_t)prefill_v16_rows(*L, layer, n_chunk) * row;
    if (per_seq > UINT64_MAX / (uint64_t)n_seqs)
        return fail(HWKV_ERR_OVERFLOW, "prefill workspace size overflows 64 bits");
    *bytes = per_seq * (uint64_t)n_seqs;
    return HWKV_OK;
}

static hwkv_status prefill_entry(const hwkv_layout* L, const hwkv_cache* c, int32_t layer,
                                 int32_t n_seqs, const int32_t* seq_slots, const int64_t* pos0,
                                 int32_t n_chunk, int32_t n_q_heads, const void* q,
                                 const void* k, const void* v, void* ws, uint64_t ws_bytes,
                                 void* out, hwkv_dtype out_dtype, float scale, bool exact_p,
                                 hipStream_t stream) {
    clear_error();
    HWKV_TRY(check_cache(L, c));
    HWKV_TRY(check_batch(L, c, layer, 1, n_seqs, seq_slots));
    int group = 0;
    HWKV_TRY(check_group(L, n_q_heads, &group));
    if (!prefill_supported(*L, group))
        return fail(HWKV_ERR_UNSUPPORTED, "no prefill kernel for this block size, dtype, "
                                          "head_dim and GQA group size " + std::to_string(group));
    if (n_chunk < 1) return fail(HWKV_ERR_INVALID_ARG, "n_chunk must be >= 1");
    if (!pos0 || !q || !k || !v || !out)
        return fail(HWKV_ERR_INVALID_ARG, "null pos0, q, k, v or out");
    if (!aligned(pos0, 8)) return fail(HWKV_ERR_MISALIGNED, "pos0 must be 8-byte aligned");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(HWKV_ERR_MISALIGNED, "q, k, v and out must be 16-byte aligned");
    if (out_dtype != HWKV_F32 && out_dtype != HWKV_BF16 && out_dtype != HWKV_F16)
        return fail(HWKV_ERR_INVALID_ARG, "out_dtype must be HWKV_F32, HWKV_BF16 or HWKV_F16");
    HWKV_TRY(check_scale(scale));
    uint64_t need = 0;
    if (!exact_p) {
        HWKV_TRY(hwkv_prefill_workspace_bytes(L, layer, n_seqs, n_chunk, &need));
        if (need > 0 && !ws) return fail(HWKV_ERR_INVALID_ARG, "null workspace");
        if (ws && !aligned(ws, 256))
            return fail(HWKV_ERR_MISALIGNED, "workspace must be 256-byte aligned");
        if (ws_bytes < need)
            return fail(HWKV_ERR_CAPACITY, "prefill workspace of " + std::to_string(ws_bytes) +
                                               " bytes, need " + std::to_string(need));
    }
    PrefillArgs a{};
    a.pool = static_cast<const uint8_t*>(c->pool);
    a.n_pool_blocks = pool_blocks(L, c);
    a.block_bytes = L->block_bytes;
    a.block_ids = c->block_ids;
    a.table_rows = c->table_rows;
    a.blocks_per_seq = L->blocks_per_seq;
    a.meta = static_cast<const uint8_t*>(c->meta);
    a.heads = reinterpret_cast<const HeadDesc*>(a.meta + L->heads_off);
    a.order = reinterpret_cast<const int32_t*>(a.meta + L->order_off);
    a.fingerprint = L->fingerprint;
    a.seq_slots = seq_slots;
    a.pos0 = pos0;
    a.q = static_cast<const uint8_t*>(q);
    a.k = static_cast<const uint8_t*>(k);
    a.v = static_cast<const uint8_t*>(v);
    a.out = out;
    a.layer = layer;
    a.n_seqs = n_seqs;
    a.n_chunk = n_chunk;
    a.n_q_heads = n_q_heads;
    a.n_kv_heads = L->n_kv_heads;
    a.out_kind = out_dtype;
    a.tpb_log2 = 0;
    while ((16 << a.tpb_log2) < L->block_size) a.tpb_log2++;
    a.exact_p = exact_p ? 1 : 0;
    a.qk_scale_log2 = scale * 1.4426950408889634f;
    if (need > 0) {
        a.v16 = static_cast<uint8_t*>(ws);
        a.v16_seq_rows = prefill_v16_rows(*L, layer, n_chunk);
    }
    return launch_prefill(*L, group, a, stream);
}

hwkv_status hwkv_prefill_attn(const hwkv_layout* L, const hwkv_cache* c, int32_t layer,
                              int32_t n_seqs, const int32_t* seq_slots, const int64_t* pos0,
                              int32_t n_chunk, int32_t n_q_heads, const void* q, const void* k,
                              const void* v, void* ws, uint64_t ws_bytes, void* out,
                              hwkv_dtype out_dtype, float scale, hipStream_t stream) {
    return prefill_entry(L, c, layer, n_seqs, seq_slots, pos0, n_chunk, n_q_heads, q, k, v, ws,
                         ws_bytes, out, out_dtype, scale, false, stream);
}

hwkv_status hwkv_prefill_attn_exact(const hwkv_layout* L, const hwkv_cache* c, int32_t layer,
                                    int32_t n_seqs, const int32_t* seq_slots,
                                    const int64_t* pos0, int32_t n_chunk, int32_t n_q_heads,
                                    const void* q, const void* k, const void* v, void* out,
                                    hwkv_dtype out_dtype, float scale, hipStream_t stream) {
    return prefill_entry(L, c, layer, n_seqs, seq_slots, pos0, n_chunk, n_q_heads, q, k, v,
                         nullptr, 0, out, out_dtype, scale, true, stream);
}

}  // extern "C"
