// Per-head append of new K/V rows into each head's ring of blocks.
//
// HeadWiseKV write-up, 核心技术 2: every head owns ceil(w_h / block_size)
// blocks.  Page 2 ("KV Cache Consistency Practices ..."), "SWA Window": only
// the most recent tokens are kept and the window moves with the sequence.
// Token t of a head with nb blocks of bs tokens is stored in ring block
// (t / bs) % nb, row t % bs, so the ring always holds the newest
// C = bs * nb >= w_h tokens.
//
// One thread moves one 16-byte chunk of a K row and the same chunk of the V
// row.  Threads are numbered in the input's memory order
// [layer][seq][token][kv head][chunk], so reads are fully coalesced; each
// head's row lands as one contiguous run of 16-byte stores.  Of one call's
// tokens only those with t >= pos0 + n_new - C are written: an older token
// with the same ring slot would be overwritten by a newer one in the same
// call, and skipping it removes the write-write race.
#include <hip/hip_runtime.h>

#include "hwkv_internal.h"

namespace hwkv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    const int CPR = a.row_chunks;  // 16-byte chunks per row
    const int64_t ROW = (int64_t)CPR * 16;
    const int64_t bs = a.block_size;
    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) return;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < a.n_chunks;
         idx += stride) {
        int64_t rest = idx / CPR;
        const int c = (int)(idx - rest * CPR);
        const int h = (int)(rest % a.n_kv_heads);
        rest /= a.n_kv_heads;
        const int tok = (int)(rest % a.n_new);
        rest /= a.n_new;
        const int b = (int)(rest % a.n_seqs);
        const int li = (int)(rest / a.n_seqs);
        const int64_t P = a.pos0[b];
        if (P < 0) continue;
        const HeadDesc hd = a.heads[(int64_t)(a.layer_begin + li) * a.n_kv_heads + h];
        const int64_t t = P + tok;
        const int64_t cap = (int64_t)hd.nblocks * bs;
        if (t < P + a.n_new - cap) continue;  // overwritten later in this call
        const int64_t slot = a.seq_slots ? (int64_t)a.seq_slots[b] : (int64_t)b;
        if (slot < 0 || slot >= a.table_rows) continue;
        const int32_t id =
            a.block_ids[slot * a.blocks_per_seq + hd.table_off + (t / bs) % hd.nblocks];
        if (id < 0 || (uint64_t)id >= a.n_pool_blocks) continue;
        uint8_t* dst = a.pool + (uint64_t)id * a.block_bytes + (uint64_t)(t % bs) * ROW + c * 16;
        const uint4 kc = *reinterpret_cast<const uint4*>(a.k + idx * 16);
        const uint4 vc = *reinterpret_cast<const uint4*>(a.v + idx * 16);
        *reinterpret_cast<uint4*>(dst) = kc;
        *reinterpret_cast<uint4*>(dst + bs * ROW) = vc;
    }
}

}  // namespace

bool append_supported(const hwkv_layout& lay) {
    // a bit copy in 16-byte chunks: any block size, rows of whole chunks
    return ((int64_t)lay.head_dim * elem_bytes(lay.dtype)) % 16 == 0;
}

hwkv_status launch_append(const hwkv_layout& /*lay*/, const AppendArgs& a, hipStream_t s) {
    int64_t blocks = (a.n_chunks + kThreads - 1) / kThreads;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) return HWKV_OK;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("append launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

}  // namespace hwkv
