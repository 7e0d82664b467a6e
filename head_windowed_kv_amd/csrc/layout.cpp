// Host half of libhwkv: layout construction, the exact memory estimate, the
// default block tables and the device meta blob.  Pure integer arithmetic on
// the host; no HIP runtime call is made here.
//
// Follows the HeadWiseKV write-up (KnoAI), sections 摘要 (static per-head
// windows make the cache demand exact before serving) and 核心技术 2
// "Grouped-Cache Runtime" (each head's block table holds
// ceil(window_size / block_size) blocks; the footprint is computed before
// the server starts).
#include <string.h>

#include <algorithm>
#include <limits>
#include <memory>
#include <new>
#include <string>

#include "hwkv_internal.h"

namespace hwkv {

namespace {
thread_local std::string g_last_error;

uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
    const uint8_t* p = static_cast<const uint8_t*>(data);
    for (size_t i = 0; i < n; i++) {
        h ^= p[i];
        h *= 1099511628211ull;
    }
    return h;
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

bool mul_overflows(uint64_t a, uint64_t b) {
    return a != 0 && b > std::numeric_limits<uint64_t>::max() / a;
}
}  // namespace

hwkv_status fail(hwkv_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

void clear_error() { g_last_error.clear(); }

}  // namespace hwkv

using namespace hwkv;

extern "C" {

uint32_t hwkv_abi_version(void) { return HWKV_ABI_VERSION; }

const char* hwkv_last_error(void) { return g_last_error.c_str(); }

static hwkv_status layout_create(int32_t n_layers, int32_t n_kv_heads, const int32_t* windows,
                                 int32_t block_size, int32_t head_dim, hwkv_dtype dtype,
                                 int32_t split_tokens, hwkv_layout** out);

hwkv_status hwkv_layout_create(int32_t n_layers, int32_t n_kv_heads, const int32_t* windows,
                               int32_t block_size, int32_t head_dim, hwkv_dtype dtype,
                               int32_t split_tokens, hwkv_layout** out) {
    clear_error();
    // the host tables can be large (a work list of up to 2^31 items): an
    // allocation failure is reported, never thrown across the C ABI
    try {
        return layout_create(n_layers, n_kv_heads, windows, block_size, head_dim, dtype,
                             split_tokens, out);
    } catch (const std::bad_alloc&) {
        if (out) *out = nullptr;
        return fail(HWKV_ERR_INVALID_ARG, "out of host memory for the layout tables");
    }
}

static hwkv_status layout_create(int32_t n_layers, int32_t n_kv_heads, const int32_t* windows,
                                 int32_t block_size, int32_t head_dim, hwkv_dtype dtype,
                                 int32_t split_tokens, hwkv_layout** out) {
    if (!out || !windows) return fail(HWKV_ERR_INVALID_ARG, "null windows or out pointer");
    *out = nullptr;
    if (n_layers < 1 || n_kv_heads < 1)
        return fail(HWKV_ERR_INVALID_ARG, "n_layers and n_kv_heads must be >= 1");
    if ((int64_t)n_layers * n_kv_heads > (1 << 24))
        return fail(HWKV_ERR_INVALID_ARG, "more than 2^24 heads");
    if (block_size < 1 || block_size > kMaxBlockSize || head_dim < 1 || head_dim > kMaxHeadDim)
        return fail(HWKV_ERR_INVALID_ARG, "block_size must be in [1, " +
                                              std::to_string(kMaxBlockSize) +
                                              "] and head_dim in [1, " +
                                              std::to_string(kMaxHeadDim) + "]");
    if (dtype != HWKV_F32 && dtype != HWKV_BF16 && dtype != HWKV_F16)
        return fail(HWKV_ERR_INVALID_ARG, "dtype must be HWKV_F32, HWKV_BF16 or HWKV_F16");
    // A layout is a host description (block tables, the exact estimate); any
    // block size and head_dim can be described.  Whether a kernel exists for
    // it is checked by the device calls (HWKV_ERR_UNSUPPORTED there).
    if (split_tokens == 0) split_tokens = default_split_tokens(block_size);
    const int32_t max_split = block_size > kMaxSplitTokens ? block_size : kMaxSplitTokens;
    if (split_tokens < block_size || split_tokens % block_size != 0 || split_tokens > max_split)
        return fail(HWKV_ERR_INVALID_ARG, "split_tokens must be a multiple of block_size in "
                                          "[block_size, max(block_size, " +
                                              std::to_string(kMaxSplitTokens) + ")]");

    const int64_t n_heads = (int64_t)n_layers * n_kv_heads;
    for (int64_t i = 0; i < n_heads; i++) {
        if (windows[i] < 1)
            return fail(HWKV_ERR_INVALID_ARG,
                        "window < 1 at layer " + std::to_string(i / n_kv_heads) + ", head " +
                            std::to_string(i % n_kv_heads));
    }

    std::unique_ptr<hwkv_layout> L(new (std::nothrow) hwkv_layout());
    if (!L) return fail(HWKV_ERR_INVALID_ARG, "out of host memory");
    L->n_layers = n_layers;
    L->n_kv_heads = n_kv_heads;
    L->block_size = block_size;
    L->head_dim = head_dim;
    L->dtype = dtype;
    L->split_tokens = split_tokens;
    L->windows.assign(windows, windows + n_heads);
    L->nblocks.resize(n_heads);
    L->head_off.resize(n_heads + 1);
    L->layer_work_off.resize(n_layers + 1);
    L->heads.resize(n_heads);
    L->block_bytes = 2ull * block_size * head_dim * elem_bytes(dtype);

    int64_t acc = 0, work = 0;
    int32_t maxw = 0;
    for (int64_t i = 0; i < n_heads; i++) {
        const int64_t w = windows[i];
        const int64_t nb = (w + block_size - 1) / block_size;  // ceil(w / bs)
        const int64_t ns = (w + split_tokens - 1) / split_tokens;
        if (i % n_kv_heads == 0) L->layer_work_off[i / n_kv_heads] = (int32_t)work;
        L->nblocks[i] = (int32_t)nb;
        L->head_off[i] = acc;
        HeadDesc& hd = L->heads[i];
        hd.table_off = acc;
        hd.window = (int32_t)w;
        hd.nblocks = (int32_t)nb;
        hd.work_off = (int32_t)work;
        hd.max_splits = (int32_t)ns;
        hd.layer = (int32_t)(i / n_kv_heads);
        hd.head = (int32_t)(i % n_kv_heads);
        acc += nb;
        work += ns;
        if (w > maxw) maxw = (int32_t)w;
        if (work > std::numeric_limits<int32_t>::max() || acc > std::numeric_limits<int32_t>::max())
            return fail(HWKV_ERR_OVERFLOW, "decode work list or blocks per sequence exceed int32");
    }
    L->head_off[n_heads] = acc;
    L->layer_work_off[n_layers] = (int32_t)work;
    L->blocks_per_seq = acc;
    L->n_work = work;
    L->max_window = maxw;
    L->work.resize(work);
    for (int64_t i = 0; i < n_heads; i++)
        for (int32_t j = 0; j < L->heads[i].max_splits; j++)
            L->work[L->heads[i].work_off + j] = WorkItem{(int32_t)i, j};
    // prefill schedules the kv heads of a layer longest window first
    L->order.resize(n_heads);
    for (int32_t l = 0; l < n_layers; l++) {
        int32_t* o = L->order.data() + (int64_t)l * n_kv_heads;
        for (int32_t h = 0; h < n_kv_heads; h++) o[h] = h;
        const int32_t* wl = windows + (int64_t)l * n_kv_heads;
        std::stable_sort(o, o + n_kv_heads, [wl](int32_t x, int32_t y) { return wl[x] > wl[y]; });
    }

    uint64_t h = 1469598103934665603ull;
    const uint32_t abi = HWKV_ABI_VERSION;
    const int32_t params[6] = {n_layers, n_kv_heads, block_size, head_dim, (int32_t)dtype,
                               split_tokens};
    h = fnv1a(h, &abi, sizeof abi);
    h = fnv1a(h, params, sizeof params);
    h = fnv1a(h, windows, (size_t)n_heads * sizeof(int32_t));
    L->fingerprint = h;

    uint64_t off = align_up(sizeof(MetaHeader), kMetaAlign);
    L->heads_off = off;
    off = align_up(off + (uint64_t)n_heads * sizeof(HeadDesc), kMetaAlign);
    L->layer_work_off_bytes = off;
    off = align_up(off + (uint64_t)(n_layers + 1) * sizeof(int32_t), kMetaAlign);
    L->work_off = off;
    off = align_up(off + (uint64_t)work * sizeof(WorkItem), kMetaAlign);
    L->order_off = off;
    off = align_up(off + (uint64_t)n_heads * sizeof(int32_t), kMetaAlign);
    L->meta_bytes = off;

    *out = L.release();
    return HWKV_OK;
}

void hwkv_layout_destroy(hwkv_layout* layout) { delete layout; }

hwkv_status hwkv_layout_query(const hwkv_layout* L, hwkv_layout_desc* desc, int32_t* windows_out,
                              int32_t* nblocks_out, int64_t* head_offsets_out) {
    clear_error();
    if (!L) return fail(HWKV_ERR_INVALID_ARG, "null layout");
    const size_t n_heads = L->windows.size();
    if (desc) {
        memset(desc, 0, sizeof *desc);
        desc->abi_version = HWKV_ABI_VERSION;
        desc->n_layers = L->n_layers;
        desc->n_kv_heads = L->n_kv_heads;
        desc->block_size = L->block_size;
        desc->head_dim = L->head_dim;
        desc->dtype = (int32_t)L->dtype;
        desc->split_tokens = L->split_tokens;
        desc->max_window = L->max_window;
        desc->blocks_per_seq = L->blocks_per_seq;
        desc->n_work = L->n_work;
        desc->block_bytes = L->block_bytes;
        desc->meta_bytes = L->meta_bytes;
        desc->fingerprint = L->fingerprint;
    }
    if (windows_out) memcpy(windows_out, L->windows.data(), n_heads * sizeof(int32_t));
    if (nblocks_out) memcpy(nblocks_out, L->nblocks.data(), n_heads * sizeof(int32_t));
    if (head_offsets_out)
        memcpy(head_offsets_out, L->head_off.data(), (n_heads + 1) * sizeof(int64_t));
    return HWKV_OK;
}

hwkv_status hwkv_mem_estimate(const hwkv_layout* L, int64_t n_seqs, uint64_t* bytes) {
    clear_error();
    if (!L || !bytes) return fail(HWKV_ERR_INVALID_ARG, "null layout or bytes pointer");
    if (n_seqs < 0) return fail(HWKV_ERR_INVALID_ARG, "n_seqs must be >= 0");
    // sum over heads of ceil(w/bs) blocks, each block_bytes = 2*bs*d*sizeof
    const uint64_t per_seq_blocks = (uint64_t)L->blocks_per_seq;
    if (mul_overflows(per_seq_blocks, L->block_bytes))
        return fail(HWKV_ERR_OVERFLOW, "per-sequence bytes overflow 64 bits");
    const uint64_t per_seq = per_seq_blocks * L->block_bytes;
    if (mul_overflows(per_seq, (uint64_t)n_seqs))
        return fail(HWKV_ERR_OVERFLOW, "pool bytes overflow 64 bits");
    *bytes = per_seq * (uint64_t)n_seqs;
    return HWKV_OK;
}

hwkv_status hwkv_capacity_check(const hwkv_layout* L, int64_t n_seqs, uint64_t pool_bytes,
                                int64_t* seq_row, int32_t* layer, int32_t* head) {
    clear_error();
    if (!L) return fail(HWKV_ERR_INVALID_ARG, "null layout");
    if (n_seqs < 0) return fail(HWKV_ERR_INVALID_ARG, "n_seqs must be >= 0");
    uint64_t need = 0;
    hwkv_status st = hwkv_mem_estimate(L, n_seqs, &need);
    if (st != HWKV_OK) return st;
    if (pool_bytes >= need) return HWKV_OK;
    // Blocks are laid out sequence row by row, heads layer-major inside a
    // row: find the first head whose blocks end beyond the pool.
    const uint64_t avail = pool_bytes / L->block_bytes;
    const uint64_t bps = (uint64_t)L->blocks_per_seq;
    const uint64_t row = avail / bps;
    const uint64_t left = avail - row * bps;
    size_t i = 0;
    while (i + 1 < L->nblocks.size() && (uint64_t)(L->head_off[i] + L->nblocks[i]) <= left) i++;
    const int32_t ly = (int32_t)(i / L->n_kv_heads), hh = (int32_t)(i % L->n_kv_heads);
    if (seq_row) *seq_row = (int64_t)row;
    if (layer) *layer = ly;
    if (head) *head = hh;
    return fail(HWKV_ERR_CAPACITY,
                "KV cache block allocation failed at layer " + std::to_string(ly) + ", head " +
                    std::to_string(hh) + ": sequence row " + std::to_string(row) + " needs " +
                    std::to_string(need) + " pool bytes in total, the pool has " +
                    std::to_string(pool_bytes));
}

hwkv_status hwkv_table_fill(const hwkv_layout* L, int64_t n_seqs, int32_t* block_ids) {
    clear_error();
    if (!L || (!block_ids && n_seqs > 0)) return fail(HWKV_ERR_INVALID_ARG, "null argument");
    if (n_seqs < 0) return fail(HWKV_ERR_INVALID_ARG, "n_seqs must be >= 0");
    const int64_t bps = L->blocks_per_seq;
    if (n_seqs > 0 && bps > std::numeric_limits<int32_t>::max() / n_seqs)
        return fail(HWKV_ERR_OVERFLOW, "block ids exceed int32 for " + std::to_string(n_seqs) +
                                           " sequences");
    for (int64_t s = 0; s < n_seqs; s++)
        for (int64_t j = 0; j < bps; j++) block_ids[s * bps + j] = (int32_t)(s * bps + j);
    return HWKV_OK;
}

hwkv_status hwkv_meta_fill(const hwkv_layout* L, void* meta_host, uint64_t meta_bytes) {
    clear_error();
    if (!L || !meta_host) return fail(HWKV_ERR_INVALID_ARG, "null argument");
    if (meta_bytes < L->meta_bytes)
        return fail(HWKV_ERR_CAPACITY, "meta buffer of " + std::to_string(meta_bytes) +
                                           " bytes is smaller than " +
                                           std::to_string(L->meta_bytes));
    uint8_t* base = static_cast<uint8_t*>(meta_host);
    memset(base, 0, L->meta_bytes);
    MetaHeader hdr;
    memset(&hdr, 0, sizeof hdr);
    hdr.magic = kMetaMagic;
    hdr.abi = HWKV_ABI_VERSION;
    hdr.fingerprint = L->fingerprint;
    hdr.n_layers = L->n_layers;
    hdr.n_kv_heads = L->n_kv_heads;
    hdr.block_size = L->block_size;
    hdr.head_dim = L->head_dim;
    hdr.dtype = (int32_t)L->dtype;
    hdr.split_tokens = L->split_tokens;
    hdr.blocks_per_seq = L->blocks_per_seq;
    hdr.n_work = L->n_work;
    hdr.heads_off = L->heads_off;
    hdr.layer_work_off = L->layer_work_off_bytes;
    hdr.work_off = L->work_off;
    hdr.order_off = L->order_off;
    memcpy(base, &hdr, sizeof hdr);
    memcpy(base + L->heads_off, L->heads.data(), L->heads.size() * sizeof(HeadDesc));
    memcpy(base + L->layer_work_off_bytes, L->layer_work_off.data(),
           L->layer_work_off.size() * sizeof(int32_t));
    memcpy(base + L->work_off, L->work.data(), L->work.size() * sizeof(WorkItem));
    memcpy(base + L->order_off, L->order.data(), L->order.size() * sizeof(int32_t));
    return HWKV_OK;
}

hwkv_status hwkv_meta_fingerprint(const void* meta_host, uint64_t meta_bytes,
                                  uint64_t* fingerprint) {
    clear_error();
    if (!meta_host || !fingerprint) return fail(HWKV_ERR_INVALID_ARG, "null argument");
    if (meta_bytes < sizeof(MetaHeader))
        return fail(HWKV_ERR_INVALID_ARG, "a meta blob is at least " +
                                              std::to_string(sizeof(MetaHeader)) + " bytes");
    MetaHeader hdr;
    memcpy(&hdr, meta_host, sizeof hdr);
    if (hdr.magic != kMetaMagic) return fail(HWKV_ERR_ABI_MISMATCH, "not a meta blob");
    if (hdr.abi != HWKV_ABI_VERSION)
        return fail(HWKV_ERR_ABI_MISMATCH, "meta blob written under ABI version " +
                                               std::to_string(hdr.abi) + ", this library is " +
                                               std::to_string(HWKV_ABI_VERSION));
    *fingerprint = hdr.fingerprint;
    return HWKV_OK;
}

hwkv_status hwkv_workspace_bytes(const hwkv_layout* L, int32_t layer_begin, int32_t n_layers,
                                 int32_t n_seqs, int32_t n_q_heads, uint64_t* bytes) {
    clear_error();
    if (!L || !bytes) return fail(HWKV_ERR_INVALID_ARG, "null argument");
    if (layer_begin < 0 || n_layers < 0 || layer_begin + n_layers > L->n_layers)
        return fail(HWKV_ERR_INVALID_ARG, "layer range outside the layout");
    if (n_seqs < 0 || n_q_heads < 1 || n_q_heads % L->n_kv_heads != 0)
        return fail(HWKV_ERR_INVALID_ARG, "n_q_heads must be a positive multiple of n_kv_heads");
    const int group = n_q_heads / L->n_kv_heads;
    const uint64_t items =
        (uint64_t)(L->layer_work_off[layer_begin + n_layers] - L->layer_work_off[layer_begin]);
    const uint64_t rec = (uint64_t)record_floats(group, L->head_dim) * sizeof(float);
    if (mul_overflows(items, rec) || mul_overflows(items * rec, (uint64_t)n_seqs))
        return fail(HWKV_ERR_OVERFLOW, "workspace bytes overflow 64 bits");
    *bytes = items * rec * (uint64_t)n_seqs;
    return HWKV_OK;
}

hwkv_status hwkv_step_workspace_bytes(const hwkv_layout* L, int32_t layer_begin, int32_t n_layers,
                                      int32_t n_seqs, int32_t n_q_heads, uint64_t* bytes) {
    uint64_t rec = 0;
    hwkv_status st = hwkv_workspace_bytes(L, layer_begin, n_layers, n_seqs, n_q_heads, &rec);
    if (st != HWKV_OK) return st;
    // records, then one uint32 arrival counter per (layer, kv head, sequence)
    const uint64_t counters = (uint64_t)n_layers * (uint64_t)L->n_kv_heads * (uint64_t)n_seqs * 4u;
    *bytes = (rec + 255) / 256 * 256 + counters;
    return HWKV_OK;
}

}  // extern "C"
