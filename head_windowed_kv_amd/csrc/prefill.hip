// Chunked-prefill windowed causal attention on MFMA tiles (gfx950).
//
// HeadWiseKV write-up, 摘要 and 核心技术 2: every KV head h keeps only its
// last w_h tokens, materialised in its own ring of blocks.  For a chunk of n
// new tokens at positions [P, P+n) of one layer, query row p of query head i
// (kv head i / G) attends to the keys [max(0, p-w+1), p]: keys before P come
// from the cache history (the ring), keys from P on from the chunk's own k, v
// arguments (the chunk is appended only afterwards, so no key a query needs
// has been overwritten yet).
//
// Scores and the weighted sum are dense contractions, so they run on MFMA:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = a 32-key slice of the K tile
//                 (row-major in LDS), B = Q^T held in registers; lane l then
//                 owns query column l%32 and 16 of the 32 keys, so the
//                 softmax over keys is in-lane plus one exchange with l^32.
//   O^T = V^T P^T v_mfma_f32_32x32x16_bf16, A = V^T read from the key-major V
//                 tile with ds_read_b64_tr_b16 (the transpose happens in the
//                 LDS read), B = P^T taken straight from the S^T registers; the
//                 key order of the two operands is matched through the
//                 transpose-read addresses.
// P is split into a bf16 high part and a bf16 remainder (two MFMAs): P rounded
// to bf16 alone costs ~2e-3 relative error on near-uniform softmax rows.
//
// Work: a workgroup of 4 waves takes 4 consecutive "units" of one (sequence,
// kv head); unit u is 32 consecutive query positions (u / G) of query head
// (u % G), so the G heads of a GQA group share every K/V tile.  Key tiles of
// 64 positions are staged through LDS (double buffered, rows padded against
// bank conflicts); a wave skips the MFMAs of tiles outside its own band and
// masks only tiles that cross its window start or its causal diagonal.
#include <hip/hip_runtime.h>

#include "hwkv_internal.h"

namespace hwkv {
namespace {

constexpr int kBS = 16;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBK = 64;  // keys per tile
constexpr int kQW = 32;  // query rows per wave
constexpr float kEmptyMax = -1e30f;
constexpr float kLazy = 8.0f;  // raise the running max only when it grows by > 2^8
constexpr int kXcds = 8;       // MI355X dispatches workgroups round robin to 8 XCDs

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct PfCfg {
    static constexpr int ROW = D * 2;         // bytes per K or V row (bf16)
    static constexpr int KS = ROW + 16;       // LDS row stride of the K tile
    static constexpr int VS = ROW + 64;       // LDS row stride of the V tile
    static constexpr int KT = kBK * KS;       // bytes of one K tile
    static constexpr int VT = kBK * VS;       // bytes of one V tile
    static constexpr int BUF = KT + VT;       // one stage
    static constexpr int CPR = ROW / 16;      // 16-byte chunks per row
    static constexpr int CHUNKS = kBK * CPR;  // chunks per K (or V) tile
    static constexpr int PER_T = CHUNKS / kThreads;
    static constexpr int KSTEP = D / 16;      // MFMA k-steps of S^T = K Q^T
    static constexpr int DBLK = D / 32;       // 32-row blocks of O^T
    static_assert(CHUNKS % kThreads == 0, "tile chunks must divide evenly");
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32f(float x) { return __shfl_xor(x, 32, 64); }

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four consecutive bf16 of row (k0 + j/4), columns n0 + 4(j%4) .. +3, read by
// lane j of a 16-lane group; the transpose read hands lane i of the group the
// four rows' elements of column n0 + i.
__device__ __forceinline__ u32x2 tr_read(const uint8_t* lds_v, int row, int col, int vs) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(lds_v + row * vs + col * 2));
    return __builtin_bit_cast(u32x2, r);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
    typedef PfCfg<D> C;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h2 = lane >> 5;   // half of the wave
    const int col = lane & 31;  // query column owned by this lane
    const int n = a.n_chunk;

    // Physical workgroup -> (sequence, kv head, unit group).  Workgroups are
    // handed to the 8 XCDs round robin, so group g of XCD x is physical block
    // 8 g + x.  All unit groups of one (sequence, kv head) go to one XCD (they
    // stream the same K/V tiles through its L2), and (sequence, kv head) pairs
    // are dealt to the XCDs in order of decreasing window, longest first.
    const int n_pb = (n + kQW - 1) / kQW;
    const int n_units = G * n_pb;
    const int n_groups = (n_units + kWaves - 1) / kWaves;
    const int xcd = blockIdx.x % kXcds;
    const int in_xcd = blockIdx.x / kXcds;
    const int pair = (in_xcd / n_groups) * kXcds + xcd;
    const int ug = in_xcd % n_groups;
    if (pair >= a.n_kv_heads * a.n_seqs) return;

    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) return;
    const int rank = pair / a.n_seqs;
    const int b = pair % a.n_seqs;
    const int kvh = a.order[(int64_t)a.layer * a.n_kv_heads + rank];
    const HeadDesc hd = a.heads[(int64_t)a.layer * a.n_kv_heads + kvh];
    const int64_t P = a.pos0[b];
    const int64_t w = hd.window;
    const int64_t slot = a.seq_slots ? (int64_t)a.seq_slots[b] : (int64_t)b;
    const bool seq_ok = P >= 0 && slot >= 0 && slot < a.table_rows;

    // units of this workgroup and of this wave
    const int u0 = ug * kWaves;
    const int u = u0 + wave;
    const bool wave_on = u < n_units;
    const int pb = u / G, qg = u % G;
    const int64_t p0 = P + (int64_t)pb * kQW;  // first query position of the wave
    // key range of the workgroup: union of its units' windows
    const int pb_min = u0 / G;
    const int pb_max = (u0 + kWaves - 1 < n_units ? u0 + kWaves - 1 : n_units - 1) / G;
    const int64_t pmin = P + (int64_t)pb_min * kQW;
    const int64_t pmax_q = P + (int64_t)pb_max * kQW + kQW - 1;
    const int64_t pmax = pmax_q < P + n - 1 ? pmax_q : P + n - 1;
    const int64_t kmin = pmin - w + 1 > 0 ? pmin - w + 1 : 0;
    const int64_t kmax = pmax;
    const int64_t T0 = kmin / kBK;
    const int n_tiles = (int)(kmax / kBK - T0 + 1);
    // key range of this wave
    const int64_t wq_last = p0 + kQW - 1 < P + n - 1 ? p0 + kQW - 1 : P + n - 1;
    const int64_t wk_lo = p0 - w + 1 > 0 ? p0 - w + 1 : 0;
    const int64_t wk_hi = wq_last;

    const int32_t* tbl = a.block_ids + (seq_ok ? slot : 0) * a.blocks_per_seq + hd.table_off;
    const uint32_t nb = (uint32_t)hd.nblocks;
    const int64_t kv_row_stride = (int64_t)a.n_kv_heads * D * 2;  // bytes between chunk rows
    const uint8_t* kc_base = a.k + ((int64_t)b * n * a.n_kv_heads + kvh) * D * 2;
    const uint8_t* vc_base = a.v + ((int64_t)b * n * a.n_kv_heads + kvh) * D * 2;

    // ---- tile staging: 4 threads per key row, each a quarter of the row ----
    constexpr int QB = C::ROW / 4;  // bytes per quarter row
    constexpr int NQ = QB / 16;     // 16-byte chunks per quarter row
    const int lkey = threadIdx.x >> 2;
    const int lq = threadIdx.x & 3;
    u32x4 stK[NQ], stV[NQ];
    // ring block of the first block of the current tile, advanced by 4 per tile
    uint32_t jt = (uint32_t)((T0 * (kBK / kBS)) % nb);
    // Every thread loads unconditionally: a key outside [kmin, kmax] (needed by
    // no query of the workgroup, its score is masked) is read from the
    // clamped position instead, and an id outside the pool from block 0, so
    // all addresses are valid and all data finite for valid caches.  The
    // block id of a tile is fetched one tile ahead of its K/V rows.
    auto key_of = [&](int64_t T) {
        const int64_t t = T * kBK + lkey;
        return t < kmin ? kmin : (t > kmax ? kmax : t);
    };
    auto fetch_id = [&](int64_t T, uint32_t j_first) -> int32_t {
        const int64_t t = key_of(T);
        uint32_t j = j_first + (uint32_t)((t - T * kBK) / kBS);
        while (j >= nb) j -= nb;
        return tbl[t < P ? j : 0];
    };
    auto load_tile = [&](int64_t T, int32_t id) {
        const int64_t t = key_of(T);
        const bool hist = t < P;
        const uint64_t idc = (id >= 0 && (uint64_t)id < a.n_pool_blocks) ? (uint64_t)id : 0;
        const uint8_t* kp = hist ? a.pool + idc * a.block_bytes + (t % kBS) * C::ROW
                                 : kc_base + (t - P) * kv_row_stride;
        const uint8_t* vp = hist ? kp + kBS * C::ROW : vc_base + (t - P) * kv_row_stride;
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            stK[i] = *reinterpret_cast<const u32x4*>(kp + lq * QB + i * 16);
            stV[i] = *reinterpret_cast<const u32x4*>(vp + lq * QB + i * 16);
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t* kb = smem + buf * C::BUF;
        uint8_t* vb = kb + C::KT;
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            *reinterpret_cast<u32x4*>(kb + lkey * C::KS + lq * QB + i * 16) = stK[i];
            *reinterpret_cast<u32x4*>(vb + lkey * C::VS + lq * QB + i * 16) = stV[i];
        }
    };

    // ---- Q^T operands of this wave (query col, head qg): 16 dims per k-step ----
    u32x4 qop[C::KSTEP];
    {
        const int64_t r = p0 - P + col;  // chunk row of this lane's query
        const bool qok = wave_on && r < n;
        const uint8_t* qrow =
            a.q + (((int64_t)b * n + (qok ? r : 0)) * a.n_q_heads + (int64_t)kvh * G + qg) * D * 2;
#pragma unroll
        for (int s = 0; s < C::KSTEP; s++)
            qop[s] = qok ? *reinterpret_cast<const u32x4*>(qrow + (s * 16 + h2 * 8) * 2)
                         : u32x4{0, 0, 0, 0};
    }

    f32x16 oacc[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; db++) oacc[db] = f32x16{};
    // running max in the log2 domain; it is only raised when some lane's tile
    // maximum exceeds it by more than kLazy, so P stays below 2^kLazy
    float m_run = kEmptyMax, l_run = 0.f;
    const float c2 = a.qk_scale_log2;

    // jt: ring block of the first block of tile T0 + it + 1 (advanced by 4 per tile)
    int32_t id_next = 0;
    if (n_tiles > 0) {
        load_tile(T0, fetch_id(T0, jt));
        store_tile(0);
        jt += kBK / kBS;
        while (jt >= nb) jt -= nb;
        if (n_tiles > 1) id_next = fetch_id(T0 + 1, jt);
    }
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(0);  // nothing loaded before the loop is pending in it
    for (int it = 0; it < n_tiles; it++) {
        const int64_t T = T0 + it;
        const int cur = it & 1;
        const bool more = it + 1 < n_tiles;
        if (more) {
            load_tile(T + 1, id_next);
            if (it + 2 < n_tiles) {
                jt += kBK / kBS;
                while (jt >= nb) jt -= nb;
                id_next = fetch_id(T + 2, jt);
            }
        }
        const int64_t kt0 = T * kBK;
        const bool touch = wave_on && kt0 + kBK - 1 >= wk_lo && kt0 <= wk_hi;
        if (touch) {
            const uint8_t* kb = smem + cur * C::BUF;
            const uint8_t* vb = kb + C::KT;
            // S^T for the two 32-key halves of the tile
            // The two 32-key halves are independent accumulation chains; their
            // MFMAs alternate and each K operand is read two steps ahead.
            f32x16 sacc[2] = {f32x16{}, f32x16{}};
            {
                const uint8_t* krow0 = kb + col * C::KS + h2 * 16;
                const uint8_t* krow1 = krow0 + 32 * C::KS;
                u32x4 ka0[C::KSTEP], ka1[C::KSTEP];
#pragma unroll
                for (int s = 0; s < C::KSTEP; s++) {
                    ka0[s] = *reinterpret_cast<const u32x4*>(krow0 + s * 32);
                    ka1[s] = *reinterpret_cast<const u32x4*>(krow1 + s * 32);
                }
#pragma unroll
                for (int s = 0; s < C::KSTEP; s++) {
                    sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(ka0[s]), as_bf16x8(qop[s]), sacc[0], 0, 0, 0);
                    sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        as_bf16x8(ka1[s]), as_bf16x8(qop[s]), sacc[1], 0, 0, 0);
                }
                // order: 4 reads, then (2 reads, 2 MFMAs) per step
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int s = 0; s < C::KSTEP - 2; s++) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            // mask keys outside [pq-w+1, pq]: with u = pq - t, keep 0 <= u < w
            const bool full = kt0 >= wq_last - w + 1 && kt0 + kBK - 1 <= p0;
            if (!full) {
                const int32_t ubase = col - (int32_t)(kt0 - p0) - h2 * 4;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; kb2++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int32_t uu = ubase - (kb2 * 32 + (r >> 2) * 8 + (r & 3));
                        if (!((uint32_t)uu < (uint32_t)w)) sacc[kb2][r] = -INFINITY;
                    }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) mt = fmaxf(mt, sacc[kb2][r]);
            mt = fmaxf(mt, xor32f(mt)) * c2;
            if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy)) {
                const float m_new = fmaxf(m_run, mt);
                const float alpha = fast_exp2(m_run - m_new);
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < C::DBLK; db++)
#pragma unroll
                    for (int r = 0; r < 16; r++) oacc[db][r] *= alpha;
            }
            // P = 2^(s c2 - m) as B operands: high part = P truncated to bf16,
            // low part = the exact remainder rounded to bf16
            u32x4 phi[4], plo[4];
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int kb2 = ks >> 1, half = ks & 1;
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int r0 = (e < 2 ? 2 * half : 2 * half + 1) * 4 + (e & 1) * 2;
                    const float pa = fast_exp2(fmaf(sacc[kb2][r0], c2, -m_run));
                    const float pb2 = fast_exp2(fmaf(sacc[kb2][r0 + 1], c2, -m_run));
                    const uint32_t ua = __float_as_uint(pa), ub = __float_as_uint(pb2);
                    hw[e] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
                    lw[e] = pack_bf16(pa - __uint_as_float(ua & 0xffff0000u),
                                      pb2 - __uint_as_float(ub & 0xffff0000u));
                    l_run += pa + pb2;
                }
                phi[ks] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                plo[ks] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
            // O^T += V^T P^T; V^T operands by transpose reads.  Lane group
            // g16 = lane/16 covers d columns 16*(g16&1) (+32 db) and key
            // offsets 4*(g16>>1) and 8 + 4*(g16>>1) inside each 16-key step.
            const int g16 = lane >> 4, j16 = lane & 15;
            const int rrow = j16 >> 2, rcol = (j16 & 3) * 4;
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const int kbase = (ks >> 1) * 32 + (ks & 1) * 16 + (g16 >> 1) * 4;
                bf16x8 va[C::DBLK];  // this k-step's V^T operands, read before the MFMAs
#pragma unroll
                for (int db = 0; db < C::DBLK; db++) {
                    const int dcol = db * 32 + (g16 & 1) * 16 + rcol;
                    const u32x2 r0 = tr_read(vb, kbase + rrow, dcol, C::VS);
                    const u32x2 r1 = tr_read(vb, kbase + 8 + rrow, dcol, C::VS);
                    va[db] = as_bf16x8(u32x4{r0.x, r0.y, r1.x, r1.y});
                }
#pragma unroll
                for (int db = 0; db < C::DBLK; db++) {
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], as_bf16x8(phi[ks]),
                                                                       oacc[db], 0, 0, 0);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], as_bf16x8(plo[ks]),
                                                                       oacc[db], 0, 0, 0);
                }
            }
        }
        if (more) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- normalise and write this lane's query row ----
    const float l_tot = l_run + xor32f(l_run);
    const int64_t r = p0 - P + col;
    if (!wave_on || r >= n) return;
    const float inv = seq_ok ? 1.0f / l_tot : __builtin_nanf("");
    const int64_t obase = (((int64_t)b * n + r) * a.n_q_heads + (int64_t)kvh * G + qg) * D;
#pragma unroll
    for (int db = 0; db < C::DBLK; db++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int d0 = db * 32 + i * 8 + h2 * 4;
            const f32x4 o = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv,
                             oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv};
            if (a.out_bf16) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) =
                    u32x2{pack_bf16(o.x, o.y), pack_bf16(o.z, o.w)};
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + obase + d0) = o;
            }
        }
}

template <int D, int G>
hwkv_status launch_t(const PrefillArgs& a, hipStream_t s) {
    typedef PfCfg<D> C;
    const int n_pb = (a.n_chunk + kQW - 1) / kQW;
    const int n_units = G * n_pb;
    const int64_t n_groups = (n_units + kWaves - 1) / kWaves;
    const int64_t n_pairs = (int64_t)a.n_kv_heads * a.n_seqs;
    const int64_t blocks = (n_pairs + kXcds - 1) / kXcds * kXcds * n_groups;
    if (blocks > 0x7fffffff) return fail(HWKV_ERR_OVERFLOW, "prefill grid too large");
    dim3 grid((unsigned)blocks);
    const size_t lds = 2 * (size_t)C::BUF;  // two K/V stages, above the 64 KiB default
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<D, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("prefill LDS attribute: ") + hipGetErrorString(e));
    hipLaunchKernelGGL((prefill_kernel<D, G>), grid, dim3(kThreads), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

#define HWKV_FOR_GROUPS(X) X(1) X(2) X(3) X(4) X(6) X(8)

}  // namespace

bool prefill_supported(hwkv_dtype dt, int head_dim, int group) {
    if (dt != HWKV_BF16 || (head_dim != 64 && head_dim != 128)) return false;
    switch (group) {
        case 1: case 2: case 3: case 4: case 6: case 8: return true;
        default: return false;
    }
}

hwkv_status launch_prefill(const hwkv_layout& lay, int group, const PrefillArgs& a,
                           hipStream_t s) {
#define HWKV_CASE(GG) \
    case GG: return lay.head_dim == 128 ? launch_t<128, GG>(a, s) : launch_t<64, GG>(a, s);
    switch (group) {
        HWKV_FOR_GROUPS(HWKV_CASE)
        default: break;
    }
#undef HWKV_CASE
    return fail(HWKV_ERR_UNSUPPORTED, "no prefill kernel for GQA group " + std::to_string(group));
}

}  // namespace hwkv
