// Per-head append of new K/V rows into each head's ring of blocks.
//
// HeadWiseKV write-up, 核心技术 2: every head owns ceil(w_h / block_size)
// blocks.  Page 2 ("KV Cache Consistency Practices ..."), "SWA Window": only
// the most recent tokens are kept and the window moves with the sequence.
// Token t of a head with nb blocks of bs tokens is stored in ring block
// (t / bs) % nb, row t % bs, so the ring always holds the newest
// C = bs * nb >= w_h tokens.
//
// Work: a workgroup takes items of consecutive new tokens of one (layer,
// sequence) (grid y = sequence; grid x strides over (layer, token block)
// items).  A token's K row over all KV heads is
// n_kv_heads * row_chunks 16-byte chunks; each thread owns the same
// (head, chunk) in the rows it copies, computed once, so the loop body is a
// table lookup and two 16-byte copies (the same chunk of the K row and of
// the V row) with no division: the ring slot of successive tokens advances
// incrementally.  A thread first loads all of its tokens' chunks, then stores
// them, so each item's reads are in flight together; rows that are not kept
// are neither read nor written.  Reads are coalesced
// (threads in the input's memory order); each head's row lands as one
// contiguous run of 16-byte stores.  Of one call's tokens only those with
// t >= pos0 + n_new - C are written: an older token with the same ring slot
// would be overwritten by a newer one in the same call, and skipping it
// removes the write-write race.
#include <hip/hip_runtime.h>

#include "hwkv_internal.h"

namespace hwkv {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerThread = 4;  // tokens whose chunks a thread moves per item

// Tokens side by side in one pass of the workgroup: whole token rows when a
// row (all KV heads) has at most kThreads chunks, else one.  An item is
// kTokensPerThread passes.
__host__ __device__ inline int tokens_per_pass(int64_t row_chunks_all_heads) {
    return row_chunks_all_heads <= kThreads ? (int)(kThreads / row_chunks_all_heads) : 1;
}

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) return;
    const int b = blockIdx.y;
    const int64_t P = a.pos0[b];
    if (P < 0) return;
    const int64_t slot = a.seq_slots ? (int64_t)a.seq_slots[b] : (int64_t)b;
    if (slot < 0 || slot >= a.table_rows) return;

    const int CPR = a.row_chunks;                         // 16-byte chunks per row
    const int64_t RC = (int64_t)a.n_kv_heads * CPR;       // chunks per token (all heads)
    const int64_t bs = a.block_size;
    const uint64_t ROW = (uint64_t)CPR * 16;
    const int tpp = tokens_per_pass(RC);
    const int item_tok = kTokensPerThread * tpp;
    const int64_t ntb = (a.n_new + item_tok - 1) / item_tok;
    const int64_t n_items = (int64_t)a.n_layers * ntb;
    const int32_t* tbl = a.block_ids + slot * a.blocks_per_seq;

    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int li = (int)(item / ntb);
        const int tok0 = (int)((item - (int64_t)li * ntb) * item_tok);
        const int tok1 = (int)min((int64_t)tok0 + item_tok, (int64_t)a.n_new);
        // first input chunk of token tok0 of (layer li, sequence b)
        const int64_t src0 = ((int64_t)li * a.n_seqs + b) * a.n_new + tok0;
        // this thread's (token offset, chunk of the row) slots in the item
        for (int64_t j0 = RC <= kThreads ? (int64_t)(threadIdx.x % RC) : (int64_t)threadIdx.x;
             j0 < RC; j0 += kThreads) {
            const int ts = RC <= kThreads ? (int)(threadIdx.x / RC) : 0;
            if (ts >= tpp) break;
            const int h = (int)(j0 / CPR), c = (int)(j0 - (int64_t)h * CPR);
            const HeadDesc hd = a.heads[(int64_t)(a.layer_begin + li) * a.n_kv_heads + h];
            // tokens before n_new - C are overwritten later in this call: not
            // read, not written
            const int64_t first_kept = (int64_t)a.n_new - (int64_t)hd.nblocks * bs;
            auto kept = [&](int u) {
                const int64_t tk = (int64_t)tok0 + ts + u * tpp;
                return tk < tok1 && tk >= first_kept;
            };
            auto load = [&](int u, uint4& kc, uint4& vc) {
                if (kept(u)) {
                    const int64_t at = ((src0 + ts + u * tpp) * RC + j0) * 16;
                    kc = *reinterpret_cast<const uint4*>(a.k + at);
                    vc = *reinterpret_cast<const uint4*>(a.v + at);
                }
            };
            static_assert(kTokensPerThread == 4, "four register pairs below");
            uint4 k0{}, v0{}, k1{}, v1{}, k2{}, v2{}, k3{}, v3{};
            load(0, k0, v0);
            load(1, k1, v1);
            load(2, k2, v2);
            load(3, k3, v3);
            // then store them: ring slot of token t = P + tok, advanced by tpp
            const int64_t t = P + tok0 + ts;
            const int64_t blk = t / bs;
            int row = (int)(t - blk * bs);        // < block_size
            int ring = (int)(blk % hd.nblocks);  // < nblocks
            const int ibs = (int)bs;
            auto store = [&](int u, const uint4& kc, const uint4& vc) {
                if (kept(u)) {
                    const int32_t id = tbl[hd.table_off + ring];
                    if (id >= 0 && (uint64_t)id < a.n_pool_blocks) {
                        uint8_t* dst = a.pool + (uint64_t)id * a.block_bytes + (uint64_t)row * ROW +
                                       (uint64_t)c * 16;
                        *reinterpret_cast<uint4*>(dst) = kc;
                        *reinterpret_cast<uint4*>(dst + bs * ROW) = vc;
                    }
                }
                row += tpp;
                if (row >= ibs) {  // crossed into a later block
                    const int q = row / ibs;
                    row -= q * ibs;
                    ring += q;
                    while (ring >= hd.nblocks) ring -= hd.nblocks;
                }
            };
            store(0, k0, v0);
            store(1, k1, v1);
            store(2, k2, v2);
            store(3, k3, v3);
        }
    }
}

}  // namespace

bool append_supported(const hwkv_layout& lay) {
    // a bit copy in 16-byte chunks: any block size, rows of whole chunks
    return ((int64_t)lay.head_dim * elem_bytes(lay.dtype)) % 16 == 0;
}

hwkv_status launch_append(const hwkv_layout& /*lay*/, const AppendArgs& a, hipStream_t s) {
    if (a.n_chunks < 1 || a.n_layers < 1 || a.n_seqs < 1 || a.n_new < 1) return HWKV_OK;
    // items of (layer, block of tokens); the sequences on grid y
    const int64_t item_tok =
        (int64_t)kTokensPerThread * tokens_per_pass((int64_t)a.n_kv_heads * a.row_chunks);
    int64_t items = (int64_t)a.n_layers * ((a.n_new + item_tok - 1) / item_tok);
    if (items > (1 << 20)) items = 1 << 20;  // the kernel strides over the rest
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)items, (unsigned)a.n_seqs), dim3(kThreads), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("append launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

}  // namespace hwkv
