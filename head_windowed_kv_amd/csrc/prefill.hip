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
//   O^T = V^T P^T v_mfma_f32_32x32x16_f16 (bf16 in the exact form, below),
//                 A = V^T read from the key-major V
//                 tile with ds_read_b64_tr_b16 (the transpose happens in the
//                 LDS read), B = P^T taken straight from the S^T registers; the
//                 key order of the two operands is matched through the
//                 transpose-read addresses.
// P rounded to bf16 alone costs ~3e-3 relative error on near-uniform softmax
// rows, so the PV product takes P in fp16 (11 significant bits, 8x more
// accurate) on v_mfma_f32_32x32x16_f16.  fp16 caches hold V in fp16 already;
// for bf16 caches a pre-pass converts, once per call, the V rows each
// (sequence, kv head) needs (keys [P - w + 1, P + n)) into an fp16 copy in the
// caller's workspace (exact for |v| in fp16's normal range), and the fast pass
// stages its V tiles from that copy; a row whose result shows a value outside
// that range (non-finite, or very small) is marked and recomputed on the
// stored bf16 tiles with P split into a bf16 high part and a bf16 remainder
// (two MFMAs).  That exact form is also what hwkv_prefill_attn_exact runs
// directly.
//
// head_dim 256: the accumulators and query operands take twice the registers
// (484 VGPRs), so that instance runs one wave per SIMD, with 32 KiB tiles.
//
// Cache blocks of 16 << k tokens: every wave still stages one 16-key slice of
// each 64-key tile; slice u of a head lives in ring block (u >> k) % nblocks,
// at row (u mod 2^k) * 16 of that block.
//
// Work: a workgroup of 4 waves takes 4 consecutive "units" of one (sequence,
// kv head); unit u is 32 consecutive query positions (u / G) of query head
// (u % G), so the G heads of a GQA group share every K/V tile.  Key tiles of
// 64 positions are staged through LDS (double buffered, 16-byte chunks
// swizzled against bank conflicts); every wave runs the workgroup's key range
// (the union of its units' windows, at most a tile or two wider than its
// own) and masks only the tiles that cross its window start or its causal
// diagonal.  Inside a tile the K operands of S^T are read from LDS three
// k-steps ahead of their MFMAs and the V^T operands one k-step ahead, so the
// LDS latency overlaps the matrix work of the same wave.
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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
constexpr int kBF16 = 1, kF16 = 2;  // element kinds (hwkv_dtype values)
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
    static constexpr int TILE = kBK * ROW;    // bytes of one K or V tile in LDS
    static constexpr int CPR = ROW / 16;      // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROW;    // rows per LDS-DMA instruction (64 lanes x 16 B)
    static constexpr int NI = kBS / RPI;      // DMA instructions per 16-key block
    static constexpr int KSTEP = D / 16;      // MFMA k-steps of S^T = K Q^T
    static constexpr int DBLK = D / 32;       // 32-row blocks of O^T
    static_assert(kWaves * kBS == kBK, "each wave stages one 16-key block of a tile");
};

// LDS tiles are unpadded; the 16-byte chunks of a row are permuted by an XOR
// with a function of the row so that the MFMA operand reads hit distinct
// banks: the K reads take one chunk of 16 consecutive rows, the transposed V
// reads 32 bytes of 4 consecutive rows.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return D >= 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    return D >= 128 ? 2 * ((2 * (r & 3)) ^ ((r >> 1) & 1)) : 2 * (r & 3);
}

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations and leaves the other counters alone
template <int n>
constexpr int vmcnt_imm() {
    return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// this lane's value and that of lane l ^ 32, in the two halves of one
// v_permlane32_swap (each lane gets the pair in the same order as its partner)
__device__ __forceinline__ f32x2 with_partner(float x) {
    const u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                     false, false);
    return f32x2{__uint_as_float(r.x), __uint_as_float(r.y)};
}

// NaN-propagating maximum: maps to v_maximum3_f32 chains with no operand
// canonicalisation (fmaxf would first quiet every operand)
__device__ __forceinline__ float fmaximum(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// two fp32 -> packed fp16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// 32x32x16 MFMA on 16-bit operands of element kind T, fp32 accumulation
template <int T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (T == kF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(4))) const int32_t const_i32;

// Four consecutive bf16 at byte address `addr` of the V tile, read by lane j
// of a 16-lane group; the transpose read hands lane i of the group the four
// rows' elements of one column.
__device__ __forceinline__ u32x2 tr_read(const uint8_t* addr) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
    return __builtin_bit_cast(u32x2, r);
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes lds + 16 i
// (the LDS address is the same for the whole wave).  A dword at or beyond the
// resource's byte count reads as zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// Kernel passes.  kFast: P (and, for bf16 caches, V) in fp16, one P.V
// product.  kExact (bf16 caches): P split into a truncated bf16 part and a
// bf16 remainder, two products.  kRedo (bf16 caches): the second launch of
// hwkv_prefill_attn.  kFast writes a row whose result is non-finite or whose
// largest magnitude is below 2^-12 of its softmax sum (where the V
// conversion's absolute error could matter) as NaN; kRedo reads the first
// element of each row of its workgroup, exits at once if none is NaN, and
// otherwise runs the kExact pass and rewrites exactly those rows (a row that
// is NaN by rule, e.g. a bad slot, comes out NaN again).  Keeping the exact
// pass out of the fast kernel leaves it fewer registers to hold.
constexpr int kFast = 0, kExact = 1, kRedo = 2;

// BIG: cache blocks of more than 16 tokens (the 16-token case keeps every
// slice address a compile-time constant).
template <int KT, int D, int G, bool BIG, int PASS>
__global__ __launch_bounds__(kThreads, D > 128 ? 1 : 2) void prefill_kernel(PrefillArgs a) {
    static_assert(KT == kBF16 || PASS == kFast, "fp16 caches have a single pass");
    // the fp16 pass on a bf16 cache reads its V tiles, already in fp16, from
    // the copy the pre-pass wrote; every other pass reads the cache's own V
    constexpr bool V16 = PASS == kFast && KT == kBF16;
    typedef PfCfg<D> C;
    // two stages of K and V tiles; separate objects so that the compiler sees
    // that a DMA into one stage never aliases the reads of the other
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[C::TILE];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[C::TILE];
    __shared__ int s_redo;  // kRedo: some row of the workgroup needs the exact pass
    // per wave: the last history key position it staged from a block whose
    // id lies outside the pool; the rows whose window reaches it are NaN
    __shared__ int64_t s_bad_hi[kWaves];

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

    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) {
        // a meta blob of another layout: its head table cannot be trusted,
        // so the whole grid writes NaN over the whole output
        const int64_t n4 = (int64_t)a.n_seqs * n * a.n_q_heads * (D / 4);
        const float x = __builtin_nanf("");
        for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n4;
             e += (int64_t)gridDim.x * kThreads) {
            if (a.out_kind == kBF16 || a.out_kind == kF16)
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + e * 4) =
                    a.out_kind == kBF16 ? u32x2{pack_bf16(x, x), pack_bf16(x, x)}
                                        : u32x2{pack_f16(x, x), pack_f16(x, x)};
            else
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + e * 4) =
                    f32x4{x, x, x, x};
        }
        return;
    }
    if (pair >= a.n_kv_heads * a.n_seqs) return;
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
    const int64_t T0 = kmin / kBK;
    const int n_tiles = (int)(pmax / kBK - T0 + 1);
    const int64_t wq_last = p0 + kQW - 1 < P + n - 1 ? p0 + kQW - 1 : P + n - 1;

    // kRedo: the rows kFast marked (NaN in their first element)
    bool redo_row = false;
    if constexpr (PASS == kRedo) {
        if (threadIdx.x == 0) s_redo = 0;
        __syncthreads();
        const int64_t r = p0 - P + col;
        if (wave_on && r < n) {
            const int64_t at = (((int64_t)b * n + r) * a.n_q_heads + (int64_t)kvh * G + qg) * D;
            float o0;
            if (a.out_kind == kBF16)
                o0 = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a.out)[at] << 16);
            else if (a.out_kind == kF16)
                o0 = (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(a.out)[at]);
            else
                o0 = reinterpret_cast<const float*>(a.out)[at];
            redo_row = __builtin_isnan(o0);
        }
        if (__builtin_amdgcn_ballot_w64(redo_row) != 0 && lane == 0) s_redo = 1;
        __syncthreads();
        if (!s_redo) return;  // uniform over the workgroup
    }

    const int32_t* tbl = a.block_ids + (seq_ok ? slot : 0) * a.blocks_per_seq + hd.table_off;
    const const_i32* tblc = (const const_i32*)tbl;
    const int32_t nb = hd.nblocks;
    const int64_t stride = (int64_t)a.n_kv_heads * C::ROW;  // bytes between chunk rows
    const uint8_t* kc_base = a.k + ((int64_t)b * n * a.n_kv_heads + kvh) * C::ROW;
    const uint8_t* vc_base = a.v + ((int64_t)b * n * a.n_kv_heads + kvh) * C::ROW;

    // ---- staging: wave w moves the 16-key block w of every tile ----
    // DMA instruction j of a wave fills LDS rows RPI j .. RPI j + RPI - 1 of
    // the block; lane i writes LDS chunk i % CPR of row RPI j + i / CPR, so it
    // fetches the global chunk that the row's swizzle puts there.
    const int lq = lane / C::CPR, la = lane % C::CPR;
    const uint32_t ck = (uint32_t)((la ^ swz_k<D>(lq)) * 16);
    const uint32_t cv = (uint32_t)((la ^ swz_v<D>(lq)) * 16);
    const uint32_t hK = (uint32_t)(lq * C::ROW) + ck, hV = (uint32_t)(lq * C::ROW) + cv;
    const uint32_t cK = (uint32_t)(lq * stride) + ck, cV = (uint32_t)(lq * stride) + cv;
    // the K (V) swizzle of row RPI j + lq differs from that of row lq by
    // xk(j) (xv(j)); xv is zero unless a DMA instruction covers fewer than 4 rows
    auto xk = [](int j) -> uint32_t { return (uint32_t)((swz_k<D>(C::RPI * j) ) * 16); };
    auto xv = [](int j) -> uint32_t { return (uint32_t)((swz_v<D>(C::RPI * j) ) * 16); };
    const int64_t pool_blocks = (int64_t)a.n_pool_blocks;

    // last key of a lost history slice this wave staged (wave-uniform); the
    // start value lies below every window start, positions included
    constexpr int64_t kNoBadKey = -(int64_t(1) << 62);
    int64_t bad_hi = kNoBadKey;
    const int tpb_log2 = BIG ? a.tpb_log2 : 0;  // 16-key slices per cache block = 1 << tpb_log2
    const uint32_t vhalf = ((uint32_t)kBS << tpb_log2) * C::ROW;  // K half of a cache block
    auto issue = [&](uint8_t* slot_base, int64_t X, int32_t id, bool is_v) {
        uint8_t* dst = slot_base + wave * (kBS * C::ROW);
        const int64_t tb = X * kBK + wave * kBS;  // first key of the slice
        const uint32_t sub = ((uint32_t)X * (kBK / kBS) + wave) & ((1u << tpb_log2) - 1u);
        const bool id_ok = id >= 0 && id < pool_blocks;
        // an id outside the pool reads zeros (an empty buffer range), so the
        // rows that mask its keys out see exact zeros, never stale bytes
        const int64_t idc = id_ok ? id : 0;
        if (!id_ok && tb < P) {
            // history keys [tb, min(tb + 16, P)) of this slice are lost
            const int64_t last = (tb + kBS < P ? tb + kBS : P) - 1;
            bad_hi = last > bad_hi ? last : bad_hi;
        }
        const rsrc_t rh = make_rsrc(a.pool + idc * a.block_bytes +
                                        ((is_v ? vhalf : 0u) + sub * (kBS * C::ROW)),
                                    id_ok ? kBS * C::ROW : 0u);
        const uint8_t* cbase = is_v ? vc_base : kc_base;
        if (tb + kBS <= P) {  // history block: every row from the ring block
#pragma unroll
            for (int j = 0; j < C::NI; j++)
                dma16(rh, is_v ? (hV ^ xv(j)) : (hK ^ xk(j)), j * 1024, dst + j * 1024);
        } else if (tb >= P) {
            // rows of the chunk's own k, v; rows past the chunk end read as
            // zero (no query attends to them)
            // (a block wholly past the end gets an empty range)
            const int64_t r0 = tb - P;
            const int64_t rows = n - r0 < kBS ? (n - r0 > 0 ? n - r0 : 0) : kBS;
            const rsrc_t rc = make_rsrc(cbase + r0 * stride, (uint32_t)(rows * stride));
#pragma unroll
            for (int j = 0; j < C::NI; j++)
                dma16(rc, (uint32_t)(j * C::RPI * stride) + (is_v ? (cV ^ xv(j)) : (cK ^ xk(j))), 0,
                      dst + j * 1024);
        } else {
            // the block that holds the chunk start: rows before it from the
            // ring block, rows from it on from the chunk
            const rsrc_t rc = make_rsrc(cbase, (uint32_t)((n < kBS ? n : kBS) * stride));
#pragma unroll
            for (int j = 0; j < C::NI; j++) {
                const int64_t t = tb + C::RPI * j + lq;
                const uint32_t cpart = is_v ? (cv ^ xv(j)) : (ck ^ xk(j));
                if (t < P)
                    dma16(rh, is_v ? (hV ^ xv(j)) : (hK ^ xk(j)), j * 1024, dst + j * 1024);
                else
                    dma16(rc, (uint32_t)((t - P) * stride) + cpart, 0, dst + j * 1024);
            }
        }
    };
    // V16: key t of this (sequence, kv head) is row t - v16_first of its
    // region of the fp16 copy (rows [0, w - 1 + n), fewer than 2^31 bytes);
    // keys before the region (a tile that starts before the window) and past
    // it get offsets beyond the buffer range and read as zero
    const uint8_t* v16_base = nullptr;
    uint32_t v16_bytes = 0;
    int64_t v16_first = 0;
    if constexpr (V16) {
        int64_t off = 0;
        for (int h = 0; h < kvh; h++)
            off += (int64_t)a.heads[(int64_t)a.layer * a.n_kv_heads + h].window - 1 + n;
        v16_base = a.v16 + ((int64_t)b * a.v16_seq_rows + off) * C::ROW;
        v16_bytes = seq_ok ? (uint32_t)((w - 1 + n) * C::ROW) : 0u;
        v16_first = P - (w - 1);
    }
    auto issue_v16 = [&](uint8_t* slot_base, int64_t X) {
        uint8_t* dst = slot_base + wave * (kBS * C::ROW);
        const int64_t tb = X * kBK + wave * kBS;  // first key of the slice
        const rsrc_t r16 = make_rsrc(v16_base, v16_bytes);
        // the whole offset in the range-checked operand (the scalar offset is
        // not checked against the range)
#pragma unroll
        for (int j = 0; j < C::NI; j++) {
            const int64_t i = tb + C::RPI * j + lq - v16_first;  // row of this lane's chunk
            const uint32_t off = i >= 0 ? (uint32_t)(i * C::ROW) + (cv ^ xv(j)) : 0x80000000u;
            dma16(r16, off, 0, dst + j * 1024);
        }
    };

    // ring block of the next slice's id: slice u_next lives in block
    // (u_next >> tpb_log2) % nb; successive tiles advance u by kBK / kBS
    uint32_t u_next = (uint32_t)(T0 * (kBK / kBS) + wave);  // positions < 2^35
    int32_t jw = (int32_t)((u_next >> tpb_log2) % (uint32_t)nb);
    auto next_id = [&]() -> int32_t {
        const int32_t id = tblc[jw];
        const uint32_t u2 = u_next + kBK / kBS;
        jw += (int32_t)((u2 >> tpb_log2) - (u_next >> tpb_log2));
        while (jw >= nb) jw -= nb;
        u_next = u2;
        return id;
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

    // K operand of k-step s for key row 32 kb2 + col: chunk 2 s + h2 of the row
    const uint32_t kx = (uint32_t)(col * C::ROW) + (uint32_t)((h2 ^ swz_k<D>(col)) * 16);
    // V^T operands: lane group g16 = lane/16 covers d columns 16 (g16 & 1)
    // (+32 db) and key offsets 4 (g16 >> 1) and 8 + 4 (g16 >> 1) inside each
    // 16-key step; lane j16 of the group reads row j16/4, columns 4 (j16 % 4)
    const int g16 = lane >> 4, j16 = lane & 15;
    const int rrow = j16 >> 2, rc = j16 & 3;
    uint32_t vaddr[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; db++) {
        const int c16 = db * 4 + (g16 & 1) * 2 + (rc >> 1);
        vaddr[db] = (uint32_t)(((g16 >> 1) * 4 + rrow) * C::ROW) +
                    (uint32_t)((c16 ^ swz_v<D>(rrow)) * 16) + (uint32_t)((rc & 1) * 8);
    }

    auto qk = [&](const uint8_t* kt, f32x16& s0, f32x16& s1) {
        s0 = f32x16{};
        s1 = f32x16{};
        u32x4 ka[C::KSTEP][2];
#pragma unroll
        for (int s = 0; s < C::KSTEP; s++) {
            const uint32_t off = kx ^ (uint32_t)(32 * s);
            ka[s][0] = *reinterpret_cast<const u32x4*>(kt + off);
            ka[s][1] = *reinterpret_cast<const u32x4*>(kt + 32 * C::ROW + off);
        }
#pragma unroll
        for (int s = 0; s < C::KSTEP; s++) {
            s0 = mfma32<KT>(ka[s][0], qop[s], s0);
            s1 = mfma32<KT>(ka[s][1], qop[s], s1);
        }
        // keep the K operand reads three k-steps ahead of the MFMAs that use
        // them (the compiler alone keeps about one, which leaves LDS latency
        // exposed): 6 LDS reads, then 2 MFMAs and 2 reads per k-step
        static_assert(C::KSTEP >= 3, "three k-steps of look-ahead");
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // LDS reads
#pragma unroll
        for (int s = 0; s < C::KSTEP - 3; s++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
    };

    // mask keys outside [pq-w+1, pq] (with u = pq - t, keep 0 <= u < w) and
    // return the tile maximum in the log2 domain
    const float c2 = a.qk_scale_log2;
    auto mask_max = [&](f32x16* sc, int64_t X) -> float {
        const int64_t kt0 = X * kBK;
        const bool full = kt0 >= wq_last - w + 1 && kt0 + kBK - 1 <= p0;
        if (!full) {
            const int32_t ubase = col - (int32_t)(kt0 - p0) - h2 * 4;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; kb2++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int32_t uu = ubase - (kb2 * 32 + (r >> 2) * 8 + (r & 3));
                    if (!((uint32_t)uu < (uint32_t)w)) sc[kb2][r] = -INFINITY;
                }
        }
        float m0 = sc[0][0], m1 = sc[1][0];
#pragma unroll
        for (int r = 1; r < 16; r++) {
            m0 = fmaximum(m0, sc[0][r]);
            m1 = fmaximum(m1, sc[1][r]);
        }
        const f32x2 pr = with_partner(fmaximum(m0, m1));
        return fmaximum(pr.x, pr.y) * c2;
    };

    f32x16 oacc[C::DBLK];
    // running max in the log2 domain; it is only raised when some lane's tile
    // maximum exceeds it by more than kLazy, so P stays below 2^kLazy
    float m_run = kEmptyMax, l_run = 0.f;

    // P = 2^(s c2 - m) of k-step ks (keys 16 ks .. 16 ks + 15) as B operands.
    // F16P: P rounded to fp16, one operand; psum collects the rounded values,
    // so that numerator and denominator use the same weights.  Otherwise high
    // part = P truncated to bf16, low part = the exact remainder rounded to
    // bf16, and psum collects the fp32 P values.
    auto make_p = [&](auto f16p_tag, const f32x16* sc, int ks, u32x4& hi, u32x4& lo,
                      float& psum) {
        constexpr bool F16P = decltype(f16p_tag)::value;
        const int kb2 = ks >> 1, half = ks & 1;
        uint32_t hw[4], lw[4];
        float ps[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r0 = (e < 2 ? 2 * half : 2 * half + 1) * 4 + (e & 1) * 2;
            const float pa = fast_exp2(fmaf(sc[kb2][r0], c2, -m_run));
            const float pb2 = fast_exp2(fmaf(sc[kb2][r0 + 1], c2, -m_run));
            const uint32_t ua = __float_as_uint(pa), ub = __float_as_uint(pb2);
            if constexpr (F16P) {
                hw[e] = pack_f16(pa, pb2);
                lw[e] = 0;
            } else {
                hw[e] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
                lw[e] = pack_bf16(pa - __uint_as_float(ua & 0xffff0000u),
                                  pb2 - __uint_as_float(ub & 0xffff0000u));
                ps[e] = pa + pb2;
            }
        }
        hi = u32x4{hw[0], hw[1], hw[2], hw[3]};
        lo = u32x4{lw[0], lw[1], lw[2], lw[3]};
        if constexpr (F16P) {
            // the row sum of the fp16 weights the P.V product uses, in fp32
            // (v_dot2_f32_f16 against (1, 1))
            const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int e = 0; e < 4; e++)
                psum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, hw[e]), one2, psum, false);
        } else {
            psum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        }
    };

    // V^T operands of k-step ks from transpose reads (fp16 when F16P: an fp16
    // cache, or the pre-pass's fp16 copy of a bf16 cache)
    auto vread = [&](const uint8_t* vt, int ks, u32x4* va) {
        const int roff = ((ks >> 1) * 32 + (ks & 1) * 16) * C::ROW;
#pragma unroll
        for (int db = 0; db < C::DBLK; db++) {
            const u32x2 r0 = tr_read(vt + roff + vaddr[db]);
            const u32x2 r1 = tr_read(vt + roff + 8 * C::ROW + vaddr[db]);
            va[db] = u32x4{r0.x, r0.y, r1.x, r1.y};
        }
    };
    // O^T += V^T P^T for one k-step
    auto pv = [&](auto f16p_tag, const u32x4* va, const u32x4& hi, const u32x4& lo) {
        constexpr bool F16P = decltype(f16p_tag)::value;
        if constexpr (F16P) {
#pragma unroll
            for (int db = 0; db < C::DBLK; db++) oacc[db] = mfma32<kF16>(va[db], hi, oacc[db]);
        } else {
#pragma unroll
            for (int db = 0; db < C::DBLK; db++) oacc[db] = mfma32<KT>(va[db], hi, oacc[db]);
#pragma unroll
            for (int db = 0; db < C::DBLK; db++) oacc[db] = mfma32<KT>(va[db], lo, oacc[db]);
        }
    };

    // ---- software pipeline over key tiles ----
    // Iteration it (tile T = T0 + it) finds S^T of T in registers and K of
    // T + 1, V of T in LDS; it starts the DMA of K of T + 2 and V of T + 1,
    // computes S^T of T + 1 while it exponentiates T, and multiplies P of T
    // into O while it finishes the exponentials and masks T + 1.
    f32x16 sA[2], sB[2];  // S^T of the current and of the next tile, alternating
    float mt = kEmptyMax;
    int32_t idK = 0, idV = 0;
    auto issue_vt = [&](uint8_t* slot_base, int64_t X, int32_t id) {
        if constexpr (V16)
            issue_v16(slot_base, X);
        else
            issue(slot_base, X, id, true);
    };
    auto run = [&](auto f16p_tag) {
        u_next = (uint32_t)(T0 * (kBK / kBS) + wave);
        jw = (int32_t)((u_next >> tpb_log2) % (uint32_t)nb);
        m_run = kEmptyMax;
        l_run = 0.f;
        mt = kEmptyMax;
#pragma unroll
        for (int db = 0; db < C::DBLK; db++) oacc[db] = f32x16{};
        if (n_tiles > 0) {
            const int32_t id0 = next_id();
            issue(sK0, T0, id0, false);
            issue_vt(sV0, T0, id0);
            const int32_t id1 = next_id();
            if (n_tiles > 1) issue(sK1, T0 + 1, id1, false);
            idV = id1;
            idK = next_id();
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (wave_on && n_tiles > 0) {
            qk(sK0, sA[0], sA[1]);
            mt = mask_max(sA, T0);
        }

        auto step = [&](int it, const uint8_t* k_rd, const uint8_t* v_rd, uint8_t* k_dma,
                        uint8_t* v_dma, f32x16* s_cur, f32x16* s_next) {
            const int64_t T = T0 + it;
            // K of T + 1 and V of T have landed (the wait covers this wave's
            // LDS DMA, which the compiler does not track); K of T, V of T - 1
            // are free
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (it + 2 < n_tiles) issue(k_dma, T + 2, idK, false);
            if (it + 1 < n_tiles) issue_vt(v_dma, T + 1, idV);
            idV = idK;
            idK = next_id();
            if (!wave_on) return;
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
            u32x4 phi[4], plo[4];
            float psum = 0.f;
            qk(k_rd, s_next[0], s_next[1]);
            // the V^T operands of each k-step are read one k-step before
            // its P.V MFMAs (two register sets in turn)
            u32x4 vA[C::DBLK], vB[C::DBLK];
            vread(v_rd, 0, vA);
            make_p(f16p_tag, s_cur, 0, phi[0], plo[0], psum);
            vread(v_rd, 1, vB);
            make_p(f16p_tag, s_cur, 1, phi[1], plo[1], psum);
            pv(f16p_tag, vA, phi[0], plo[0]);
            vread(v_rd, 2, vA);
            pv(f16p_tag, vB, phi[1], plo[1]);
            vread(v_rd, 3, vB);
            make_p(f16p_tag, s_cur, 2, phi[2], plo[2], psum);
            pv(f16p_tag, vA, phi[2], plo[2]);
            make_p(f16p_tag, s_cur, 3, phi[3], plo[3], psum);
            pv(f16p_tag, vB, phi[3], plo[3]);
            l_run += psum;
            if (it + 1 < n_tiles) mt = mask_max(s_next, T + 1);
        };
        for (int it = 0; it < n_tiles; it += 2) {
            step(it, sK1, sV0, sK0, sV1, sA, sB);
            if (it + 1 >= n_tiles) break;
            step(it + 1, sK0, sV1, sK1, sV0, sB, sA);
        }
    };

    if constexpr (PASS == kFast)
        run(BoolC<true>{});  // P in fp16, V in fp16 (bf16 caches: from the pre-pass copy)
    else
        run(BoolC<false>{});  // P as a truncated bf16 part and a bf16 remainder

    // kFast on bf16 caches: does this lane's row need the exact pass?
    bool mark = false;
    if constexpr (PASS == kFast && KT == kBF16) {
        float sa = 0.f, mx = 0.f;
#pragma unroll
        for (int db = 0; db < C::DBLK; db++)
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float x = fabsf(oacc[db][i]);
                sa += x;
                mx = fmaxf(mx, x);
            }
        const f32x2 mp = with_partner(mx), sp = with_partner(sa), lp2 = with_partner(l_run);
        const float l_tot2 = lp2.x + lp2.y;
        mark = !(__builtin_isfinite(sp.x + sp.y) && __builtin_isfinite(l_tot2) &&
                 fmaxf(mp.x, mp.y) >= 0x1p-12f * l_tot2);
    }

    // ---- normalise and write this lane's query row ----
    if (lane == 0) s_bad_hi[wave] = bad_hi;
    __syncthreads();
    int64_t lost = s_bad_hi[0];
#pragma unroll
    for (int i = 1; i < kWaves; i++) lost = s_bad_hi[i] > lost ? s_bad_hi[i] : lost;
    const f32x2 lp = with_partner(l_run);
    const float l_tot = lp.x + lp.y;
    const int64_t r = p0 - P + col;
    if (!wave_on || r >= n) return;
    // NaN for a bad sequence, and for a row whose window [p - w + 1, p]
    // reaches a history key held by a block outside the pool
    const bool row_ok = seq_ok && lost < p0 + col - w + 1 && !mark;
    const float inv = row_ok ? 1.0f / l_tot : __builtin_nanf("");
    if (PASS == kRedo && !redo_row) return;  // kFast's row stands
    const int64_t obase = (((int64_t)b * n + r) * a.n_q_heads + (int64_t)kvh * G + qg) * D;
#pragma unroll
    for (int db = 0; db < C::DBLK; db++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int d0 = db * 32 + i * 8 + h2 * 4;
            const f32x4 o = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv,
                             oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv};
            if (a.out_kind == kBF16) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) =
                    u32x2{pack_bf16(o.x, o.y), pack_bf16(o.z, o.w)};
            } else if (a.out_kind == kF16) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + obase + d0) =
                    u32x2{pack_f16(o.x, o.y), pack_f16(o.z, o.w)};
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + obase + d0) = o;
            }
        }
}

// Pre-pass of the fp16 pass on bf16 caches: the fp16 copy of the V rows of
// keys [P - w + 1, P + n) of every (sequence, kv head), keys before P from the
// cache's ring, keys from P on from the chunk's v, rounded to nearest even
// (exact for |v| in fp16's normal range; a value beyond it becomes inf, which
// the fast pass's row check catches).  A key held by a block outside the pool
// gets zeros (its rows come out NaN by the lost-key rule of the main pass);
// keys below 0 and sequences with a bad slot or position are not written
// (never staged).  Grid: x = (sequence, kv head), y strides over the 16-byte
// chunks of its rows.
template <int D>
__global__ __launch_bounds__(256) void prefill_v16_kernel(PrefillArgs a) {
    typedef PfCfg<D> C;
    const int pair = blockIdx.x;
    const int b = pair / a.n_kv_heads, h = pair % a.n_kv_heads;
    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) return;
    const int64_t P = a.pos0[b];
    const int64_t slot = a.seq_slots ? (int64_t)a.seq_slots[b] : (int64_t)b;
    if (P < 0 || slot < 0 || slot >= a.table_rows) return;
    const HeadDesc* hl = a.heads + (int64_t)a.layer * a.n_kv_heads;
    const HeadDesc hd = hl[h];
    const int n = a.n_chunk;
    int64_t off = 0;
    for (int i = 0; i < h; i++) off += (int64_t)hl[i].window - 1 + n;
    uint8_t* dst0 = a.v16 + ((int64_t)b * a.v16_seq_rows + off) * C::ROW;
    const int64_t rows = (int64_t)hd.window - 1 + n, first = P - (hd.window - 1);
    const int32_t* tbl = a.block_ids + slot * a.blocks_per_seq + hd.table_off;
    const int lbs = 4 + a.tpb_log2;  // log2 of the block size
    const uint32_t nb = (uint32_t)hd.nblocks;
    const uint8_t* vbase = a.v + (int64_t)h * C::ROW + (int64_t)b * n * a.n_kv_heads * C::ROW;
    const int64_t crow = (int64_t)a.n_kv_heads * C::ROW;  // bytes between chunk rows
    // U chunks per thread in flight: loads first, then conversions and stores
    constexpr int U = 4;
    const uint64_t n_el = (uint64_t)rows * C::CPR;
    for (uint64_t e0 = (uint64_t)blockIdx.y * (256 * U) + threadIdx.x; e0 < n_el;
         e0 += (uint64_t)gridDim.y * (256 * U)) {
        u32x4 x[U];
        bool keep[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint64_t e = e0 + (uint64_t)u * 256;
            const int64_t i = (int64_t)(e / C::CPR);
            const int c = (int)(e % C::CPR);
            const int64_t t = first + i;
            keep[u] = e < n_el && t >= 0;
            x[u] = u32x4{0u, 0u, 0u, 0u};
            if (!keep[u]) continue;
            if (t < P) {
                const int32_t id = tbl[(uint32_t)(t >> lbs) % nb];
                if (id >= 0 && (uint64_t)id < a.n_pool_blocks)
                    x[u] = *reinterpret_cast<const u32x4*>(
                        a.pool + (uint64_t)id * a.block_bytes +
                        (((int64_t)1 << lbs) + (t & (((int64_t)1 << lbs) - 1))) * C::ROW + c * 16);
            } else {
                x[u] = *reinterpret_cast<const u32x4*>(vbase + (t - P) * crow + c * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (!keep[u]) continue;
            const uint64_t e = e0 + (uint64_t)u * 256;
            u32x4 y;
#pragma unroll
            for (int k = 0; k < 4; k++)
                y[k] = pack_f16(__uint_as_float(x[u][k] << 16),
                                __uint_as_float(x[u][k] & 0xffff0000u));
            *reinterpret_cast<u32x4*>(dst0 + e * 16) = y;
        }
    }
}

template <int D>
hwkv_status launch_v16(const PrefillArgs& a, hipStream_t s) {
    // about 2048 workgroups over the whole grid, at most 256 per pair
    const int64_t pairs = (int64_t)a.n_seqs * a.n_kv_heads;
    if (pairs > 0x7fffffff) return fail(HWKV_ERR_OVERFLOW, "prefill pre-pass grid too large");
    const int64_t per = (2048 + pairs - 1) / pairs;
    dim3 grid((unsigned)pairs, (unsigned)(per < 256 ? per : 256));
    hipLaunchKernelGGL(prefill_v16_kernel<D>, grid, dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("prefill pre-pass launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

template <int T, int D, int G, bool BIG>
hwkv_status launch_pass(const PrefillArgs& a, int pass, hipStream_t s) {
    auto kernel = prefill_kernel<T, D, G, BIG, kFast>;
    if constexpr (T == kBF16)
        kernel = pass == kExact ? prefill_kernel<T, D, G, BIG, kExact>
                 : pass == kRedo ? prefill_kernel<T, D, G, BIG, kRedo>
                                 : prefill_kernel<T, D, G, BIG, kFast>;
    const int n_pb = (a.n_chunk + kQW - 1) / kQW;
    const int n_units = G * n_pb;
    const int64_t n_groups = (n_units + kWaves - 1) / kWaves;
    const int64_t n_pairs = (int64_t)a.n_kv_heads * a.n_seqs;
    const int64_t blocks = (n_pairs + kXcds - 1) / kXcds * kXcds * n_groups;
    if (blocks > 0x7fffffff) return fail(HWKV_ERR_OVERFLOW, "prefill grid too large");
    dim3 grid((unsigned)blocks);
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("prefill launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

// bf16 caches: the exact entry runs kExact; the default entry runs the V
// pre-pass, kFast, and then kRedo (which exits at once unless a workgroup
// holds a marked row).  fp16 caches: one kFast launch.
template <int T, int D, int G>
hwkv_status launch_t(const PrefillArgs& a, hipStream_t s) {
    auto run = a.tpb_log2 > 0 ? launch_pass<T, D, G, true> : launch_pass<T, D, G, false>;
    if (T == kBF16 && a.exact_p) return run(a, kExact, s);
    if (T == kBF16) {
        const hwkv_status st = launch_v16<D>(a, s);
        if (st != HWKV_OK) return st;
    }
    const hwkv_status st = run(a, kFast, s);
    if (st != HWKV_OK || T != kBF16) return st;
    return run(a, kRedo, s);
}

#define HWKV_FOR_GROUPS(X) X(1) X(2) X(3) X(4) X(6) X(8)

}  // namespace

bool prefill_supported(const hwkv_layout& lay, int group) {
    const int bs = lay.block_size;  // powers of two from 16 to 256
    if (bs < kBS || bs > 256 || (bs & (bs - 1)) != 0) return false;
    if (lay.dtype != HWKV_BF16 && lay.dtype != HWKV_F16) return false;
    if (lay.head_dim != 64 && lay.head_dim != 128 && lay.head_dim != 256) return false;
    switch (group) {
        case 1: case 2: case 3: case 4: case 6: case 8: return true;
        default: return false;
    }
}

hwkv_status launch_prefill(const hwkv_layout& lay, int group, const PrefillArgs& a,
                           hipStream_t s) {
    if (lay.head_dim == 256) {  // one wave per SIMD (see the header)
#define HWKV_CASE256(GG)                                                                     \
    case GG:                                                                                 \
        return lay.dtype == HWKV_F16 ? launch_t<kF16, 256, GG>(a, s)                         \
                                     : launch_t<kBF16, 256, GG>(a, s);
        switch (group) {
            HWKV_FOR_GROUPS(HWKV_CASE256)
            default: break;
        }
#undef HWKV_CASE256
        return fail(HWKV_ERR_UNSUPPORTED,
                    "no head_dim 256 prefill kernel for GQA group " + std::to_string(group));
    }
#define HWKV_CASE(GG) \
    case GG:                                                                        \
        if (lay.dtype == HWKV_F16)                                                  \
            return lay.head_dim == 128 ? launch_t<kF16, 128, GG>(a, s)              \
                                       : launch_t<kF16, 64, GG>(a, s);              \
        return lay.head_dim == 128 ? launch_t<kBF16, 128, GG>(a, s)                 \
                                   : launch_t<kBF16, 64, GG>(a, s);
    switch (group) {
        HWKV_FOR_GROUPS(HWKV_CASE)
        default: break;
    }
#undef HWKV_CASE
    return fail(HWKV_ERR_UNSUPPORTED, "no prefill kernel for GQA group " + std::to_string(group));
}

}  // namespace hwkv
