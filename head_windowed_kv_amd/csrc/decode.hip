// Decode attention over exactly the last w_h resident tokens of every KV head
// (HeadWiseKV write-up, 摘要: the policy is materialised as per-head
// residency, not as a mask over a full cache; 核心技术 2: each head reads its
// own block table of ceil(w_h / block_size) blocks).
//
// Stage 1 (split): one workgroup per (work item = (layer, kv head, split),
// sequence).  A split is a run of split_tokens/16 consecutive logical blocks
// of the window [max(0, L-w), L) (cut on block boundaries, the last split
// taking the remainder); the workgroup streams those K/V blocks through the
// head's ring and keeps, for the G query heads of the GQA group, an
// online-softmax state (running max m, sum l, weighted sum acc).  Decode is
// HBM-bound (G flop per byte of 16-bit K/V read), so the design goal is to
// keep enough 128-bit loads in flight and the per-byte arithmetic off the
// critical path.
//
// Work layout inside a workgroup (256 threads = 4 wave64):
//   - a wave processes one 16-token tile (16 rows of K, same of V) at a
//     time, tiles of the split interleaved over the 4 waves, two tiles in
//     flight per wave;
//   - loads: the 64 lanes form groups of 8 (32 for 512-byte rows); group g
//     owns rows g, g+8 of the tile, lane r of a group 16-byte chunks r,
//     r+8, ... of each row, so every load instruction reads whole 128-byte
//     lines.
// 16-bit caches (MFMA block loop): each wave copies the tiles of a pair into
// its own LDS staging area (one K slot, scored before the next tile's K rows
// replace it, and a V slot per tile), issues each tile's next load into the
// same registers as soon as it is staged, and folds the pair in on the
// matrix cores (three waves per SIMD up to head_dim 128): S^T = K Q^T
// on 16x16x32 MFMAs (the 16 columns are the G query heads of the group,
// padded), the online softmax on the S^T registers, O^T += V^T P^T with V^T
// from transposing LDS reads (ds_read_b64_tr_b16) and P split into 16-bit
// parts that sum to it within ~2^-22 (bf16: three parts; fp16: two parts
// of P 2^15).  The per-byte VALU work then no longer grows with G.
// fp32 caches (per-lane loop): q.k partial dots in fp32 FMAs summed over the
// lanes of a group with DPP; each group keeps its own softmax state.
// Either way the partial states are merged across lanes and waves once, at
// the end, in a fixed order (results do not depend on the batch
// composition or on timing).
//
// Stage 2 (merge): per (layer, sequence, kv head), combine the splits:
//   M = max_s m_s;  o = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s.
// Scores are kept in the log2 domain (s * scale * log2 e) so every
// exponential is one v_exp_f32.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "hwkv_internal.h"

// Split records of hwkv_decode_append_attn_static, for callers that cannot
// allocate device memory.  Every device the library runs on holds one copy
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for that device (the name is a host-side
// stand-in there).
static __device__ __align__(256) uint8_t scratch[HWKV_STATIC_SCRATCH_BYTES];

namespace hwkv {

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];  // per device, looked up once
}  // namespace

hwkv_status static_scratch(hipStream_t stream, void** ptr) {
    int cur = -1, dev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) {
        dev = cur;
        if (stream) e = hipStreamGetDevice(stream, &dev);  // the stream's device
    }
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("static scratch: device query: ") +
                                      hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(HWKV_ERR_UNSUPPORTED, "static scratch: device index " + std::to_string(dev) +
                                              " beyond " + std::to_string(kMaxScratchDevices));
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        // the symbol's address on `dev`, looked up with that device current
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(HWKV_ERR_HIP, std::string("static scratch: ") + hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || !p)
            return fail(HWKV_ERR_HIP, std::string("static scratch: hipGetSymbolAddress: ") +
                                          hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return HWKV_OK;
}

namespace {

// The kernels walk every head's window in tiles of kBS = 16 tokens.  A cache
// block of block_size = 16 << tpb_log2 tokens holds 1 << tpb_log2 tiles.
constexpr int kBS = 16;
// element kinds (the values of hwkv_dtype)
constexpr int kF32 = 0, kBF16 = 1, kF16 = 2;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kEmptyMax = -1e30f;  // running max of a state that has seen no token

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16
typedef float f32x4 __attribute__((ext_vector_type(4)));     // 4 fp32
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the N (8, 16 or 32) lanes of a group; every lane of the group
// gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: pairs
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: quads
    x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
    if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: the other 8 of the 16
    if constexpr (N >= 32)
        x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // ^16
    return x;
}

// Lane i gets lane i^8 (rotate a 16-lane row by 8).
__device__ __forceinline__ float xor8(float x) { return dpp<0x128>(x); }
// Lane i gets lane i^16 (swizzle, bit mode: and 0x1f, xor 0x10).
__device__ __forceinline__ float xor16(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---- helpers of the MFMA block loop ----
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16x16x32 MFMA on 16-bit operands of element kind T, fp32 accumulation.
// Lane l holds A[l % 16][8 (l / 16) .. + 7], B[8 (l / 16) .. + 7][l % 16] and
// D[4 (l / 16) .. + 3][l % 16].
template <int T>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (T == kF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Lane j of a 16-lane group reads four consecutive 16-bit elements at `addr`
// (row j / 4, columns 4 (j % 4) .. + 3 of a 4 x 16 block); the transposing
// read hands lane i the four rows' elements of column i.
__device__ __forceinline__ u32x2 tr_read(const uint8_t* addr) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr));
}

// two fp32 -> packed pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{a, b}, f16x2_t));
}
// two fp32 -> packed bf16 pair, truncated (the high halves of the words)
__device__ __forceinline__ uint32_t pack_bf16_trunc(float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// LDS accesses of one wave to its own staging tiles: the hardware performs a
// wave's LDS instructions in order, so only the compiler must keep them so
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Element type traits: a 16-byte chunk holds EPC elements.
template <int T>
struct Elem {
    static constexpr int kBytes = T == kF32 ? 4 : 2;
    typedef typename std::conditional<T == kF32, f32x4, u32x4>::type Chunk;  // 4 fp32 or 8 x 16 bit
};

template <int T, int D, int G>
struct SplitCfg {
    static constexpr int EB = Elem<T>::kBytes;
    static constexpr int ROW = D * EB;  // bytes per K (or V) row
    // lanes per row group: 8 for rows up to 256 bytes, 32 for 512-byte rows
    // (the accumulator of a lane then holds 8 elements per query head)
    static constexpr int LPG = ROW >= 512 ? 32 : 8;
    static constexpr int NC = ROW / (16 * LPG);  // 16-byte chunks per lane per row
    static constexpr int EPC = 16 / EB;          // elements per chunk
    static constexpr int DPL = NC * EPC;         // dims owned per lane
    static constexpr int NG = 64 / LPG;          // row groups per wave
    static constexpr int ROWS = kBS / NG;        // rows per group per tile
    static_assert(NC >= 1 && ROW % (16 * LPG) == 0, "rows of whole lane chunks");
};

// Which loop a cache takes.  In the per-lane form the VALU work per byte
// grows with the GQA group G (a dot product and a multiply-add per element
// and query head) and bounds the kernel from G = 4 on (2.1 TB/s at G = 8 on
// the 48-layer 112K stack); the matrix cores handle a 16-column S^T tile
// whatever G <= 16 is.  At G = 1-3 the MFMA loop streams as fast (head_dim
// 64 / 128) or faster (head_dim 256, where the per-lane form runs one wave
// per SIMD), and its shorter epilogue helps small launches, so every 16-bit
// cache takes it; fp32 caches (no fp32-exact 16-bit operands) keep the
// per-lane form.
template <int T>
constexpr bool mfma_loop() { return T != kF32; }

// Geometry of the MFMA block loop for head_dim D (16-bit elements).
template <int D>
struct MfmaCfg {
    static constexpr int KSTEP = D / 32;      // 16x16x32 k-steps of S^T = K Q^T
    static constexpr int DT = D / 16;         // 16-row tiles of O^T
    static constexpr int CPR = D / 8;         // 16-byte chunks per K or V row
    static constexpr int TILE = kBS * D * 2;  // bytes of one tile's K (or V) rows
    // chunk c of row t sits at chunk c ^ swz(t) of its LDS row
    static __device__ __forceinline__ int swz(int t) { return t & (CPR < 16 ? CPR - 1 : 15); }
};

// Per-lane loop (fp32 caches): partial dot product of one row chunk with one
// query chunk, and element e of a chunk.
template <int T>
__device__ __forceinline__ float chunk_dot(const typename Elem<T>::Chunk& q,
                                           const typename Elem<T>::Chunk& k, float acc) {
    static_assert(T == kF32, "the per-lane loop serves fp32 caches");
    acc = fmaf(q.x, k.x, acc);
    acc = fmaf(q.y, k.y, acc);
    acc = fmaf(q.z, k.z, acc);
    acc = fmaf(q.w, k.w, acc);
    return acc;
}

template <int T>
__device__ __forceinline__ float chunk_elem(const typename Elem<T>::Chunk& v, int e) {
    static_assert(T == kF32, "the per-lane loop serves fp32 caches");
    switch (e) {
        case 0: return v.x;
        case 1: return v.y;
        case 2: return v.z;
        default: return v.w;
    }
}

template <int T, int D, int G>
struct BlockRegs {
    typedef typename Elem<T>::Chunk Chunk;
    typedef SplitCfg<T, D, G> C;
    Chunk k[C::ROWS][C::NC];
    Chunk v[C::ROWS][C::NC];
};

// Issue the loads of one 16-token tile for this lane (rows g + 8*rho,
// chunks r + 8*c).  `tile` points at the tile's first K row; its V rows are
// `vofs` bytes further (block_size K rows separate a block's K and V halves).
// Loads are unconditional: `tile` always points inside the pool (block 0
// stands in for an invalid id), and rows outside the split are masked when
// the tile is folded in.
template <int T, int D, int G>
__device__ __forceinline__ void load_block(BlockRegs<T, D, G>& br, const uint8_t* tile,
                                           uint32_t vofs, int g, int r) {
    typedef SplitCfg<T, D, G> C;
    typedef typename Elem<T>::Chunk Chunk;
#pragma unroll
    for (int rho = 0; rho < C::ROWS; rho++) {
        const uint8_t* krow = tile + (g + C::NG * rho) * C::ROW;
        const uint8_t* vrow = krow + vofs;
#pragma unroll
        for (int c = 0; c < C::NC; c++) {
            br.k[rho][c] =
                __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(krow + (c * C::LPG + r) * 16));
            br.v[rho][c] =
                __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(vrow + (c * C::LPG + r) * 16));
        }
    }
}

// Fold one loaded block into the group's online-softmax state.  FULL: every
// row of the block lies in the split (the common case, no masking).
// Otherwise row rho is used only if valid[rho]; its V chunk is zeroed so that
// stale or uninitialised pool bytes cannot leak in as NaN * 0.
template <int T, int D, int G, bool FULL>
__device__ __forceinline__ void process_block(BlockRegs<T, D, G>& br, const bool* valid,
                                              const typename Elem<T>::Chunk (&qv)[G][SplitCfg<T, D, G>::NC],
                                              float scale_log2, float (&m)[G], float (&l)[G],
                                              float (&acc)[G][SplitCfg<T, D, G>::DPL]) {
    typedef SplitCfg<T, D, G> C;
    typedef typename Elem<T>::Chunk Chunk;
    float s[C::ROWS][G];
#pragma unroll
    for (int rho = 0; rho < C::ROWS; rho++) {
#pragma unroll
        for (int h = 0; h < G; h++) {
            float x = 0.f;
#pragma unroll
            for (int c = 0; c < C::NC; c++) x = chunk_dot<T>(qv[h][c], br.k[rho][c], x);
            x = group_sum<C::LPG>(x);
            s[rho][h] = (FULL || valid[rho]) ? x * scale_log2 : -INFINITY;
        }
        if (!FULL && !valid[rho]) {
#pragma unroll
            for (int c = 0; c < C::NC; c++) br.v[rho][c] = Chunk{};
        }
    }
    float p[C::ROWS][G];
#pragma unroll
    for (int h = 0; h < G; h++) {
        float mx = s[0][h];
#pragma unroll
        for (int rho = 1; rho < C::ROWS; rho++) mx = fmaxf(mx, s[rho][h]);
        if (mx > m[h]) {  // uniform within a group; rare once the max has settled
            const float alpha = fast_exp2(m[h] - mx);
            l[h] *= alpha;
#pragma unroll
            for (int i = 0; i < C::DPL; i++) acc[h][i] *= alpha;
            m[h] = mx;
        }
#pragma unroll
        for (int rho = 0; rho < C::ROWS; rho++) {
            p[rho][h] = fast_exp2(s[rho][h] - m[h]);
            l[h] += p[rho][h];
        }
    }
#pragma unroll
    for (int rho = 0; rho < C::ROWS; rho++) {
#pragma unroll
        for (int c = 0; c < C::NC; c++) {
#pragma unroll
            for (int e = 0; e < C::EPC; e++) {
                const float ve = chunk_elem<T>(br.v[rho][c], e);
#pragma unroll
                for (int h = 0; h < G; h++)
                    acc[h][c * C::EPC + e] = fmaf(p[rho][h], ve, acc[h][c * C::EPC + e]);
            }
        }
    }
}

// Split records.  A large split stage writes them with non-temporal stores:
// records written back from L2 in the middle of the K/V read stream cost ~5%
// of the stream's bandwidth, streamed stores about a third of that.  A small
// launch (one layer at batch 1) is latency-bound instead, and ordinary
// stores let the merge stage read the records back ~4% sooner per step.
__device__ __forceinline__ void rec_put(float* p, float v, bool streamed) {
    if (streamed)
        __builtin_nontemporal_store(v, p);
    else  // an ordinary store, written as a relaxed atomic so that the
          // compiler cannot fold it into the non-temporal one above
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Output row of (layer, sequence, kv head): G query heads x D, fp32, bf16 or fp16.
__device__ __forceinline__ void store_out4(void* out, int kind, int64_t at, f32x4 o) {
    if (kind == kBF16) {
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(o.x) | ((uint32_t)f32_to_bf16_rne(o.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(o.z) | ((uint32_t)f32_to_bf16_rne(o.w) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + at) = make_uint2(lo, hi);
    } else if (kind == kF16) {  // IEEE binary16, round to nearest even
        const f16x2_t a = __builtin_convertvector(float2_t{o.x, o.y}, f16x2_t);
        const f16x2_t b = __builtin_convertvector(float2_t{o.z, o.w}, f16x2_t);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + at) =
            make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b));
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + at) = o;
    }
}

// Merge geometry.  A record's acc[G][D] is NE4 float4 columns, split into DS
// column chunks.  A column's splits are folded by SG split groups (split s by
// group s % SG), each in one pass with a running maximum; the SG partials are
// then rescaled to the common maximum and added in a fixed order.  Every
// workgroup also forms the G softmax denominators the same way.  The same
// operations in the same order serve any grouping of chunks into workgroups
// and the single-launch step's merge, so all give identical bits.
template <int D, int G>
struct MergeCfg {
    static constexpr int NE4 = G * D / 4;
    static constexpr int DS = NE4 >= 64 ? 4 : (NE4 >= 32 ? 2 : 1);
    static constexpr int CPS = NE4 / DS;
    static constexpr int SG = (2048 / NE4) < 1 ? 1 : ((2048 / NE4) > 64 ? 64 : 2048 / NE4);
    static constexpr int PAIRS = NE4 * SG + G * SG;  // (column, group) and (head, group)
    static constexpr int THREADS = PAIRS < 1024 ? (PAIRS + 63) / 64 * 64 : 1024;
    static_assert(NE4 % DS == 0, "merge geometry");
};

// LDS of one merge: the SG groups' partial numerators, denominators and maxima
template <int D, int G>
struct MergeLds {
    f32x4 num[MergeCfg<D, G>::SG][MergeCfg<D, G>::NE4];
    float den[MergeCfg<D, G>::SG][G];
    float mk[MergeCfg<D, G>::SG][G];
};

// factor that takes a partial kept at running maximum `from` to maximum `to`
__device__ __forceinline__ float rescale(float from, float to) {
    return from == to ? 1.f : fast_exp2(from - to);
}

// One pass over the splits s = k, k + SG, ... of column c (query head h):
// running maximum m and num = sum 2^(m_s - m) acc_s[c].
template <int D, int G>
__device__ __forceinline__ f32x4 merge_num_part(const float* rec0, int rec_floats, int ns, int k,
                                                int c) {
    typedef MergeCfg<D, G> M;
    const int h = (c * 4) / D;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
#pragma unroll 8
    for (int s = k; s < ns; s += M::SG) {
        const float* rs = rec0 + (int64_t)s * rec_floats;
        const float ms = rs[G * D + h];
        const f32x4 v = *reinterpret_cast<const f32x4*>(rs + c * 4);
        const float mn = fmaxf(m, ms);
        const float al = rescale(m, mn), f = fast_exp2(ms - mn);
        num.x = fmaf(f, v.x, num.x * al);
        num.y = fmaf(f, v.y, num.y * al);
        num.z = fmaf(f, v.z, num.z * al);
        num.w = fmaf(f, v.w, num.w * al);
        m = mn;
    }
    return num;
}

// The same pass for the denominator of head h: running maximum (returned in
// m) and sum 2^(m_s - m) l_s.
template <int D, int G>
__device__ __forceinline__ float merge_den_part(const float* rec0, int rec_floats, int ns, int k,
                                                int h, float& m) {
    typedef MergeCfg<D, G> M;
    float den = 0.f;
    m = -INFINITY;
#pragma unroll 8
    for (int s = k; s < ns; s += M::SG) {
        const float* rs = rec0 + (int64_t)s * rec_floats;
        const float ms = rs[G * D + h];
        const float ls = rs[G * D + G + h];
        const float mn = fmaxf(m, ms);
        den = fmaf(fast_exp2(ms - mn), ls, den * rescale(m, mn));
        m = mn;
    }
    return den;
}

// Merge of column chunks [ds0, ds1) of one (layer, sequence, kv head) by the
// NTHREADS threads of a workgroup.  obase: output offset of the head's first
// element.
template <int D, int G, int NTHREADS>
__device__ void merge_chunks(MergeLds<D, G>& sm, const float* rec0, int ns, int rec_floats, int ds0,
                             int ds1, void* out, int out_kind, int64_t obase) {
    typedef MergeCfg<D, G> M;
    auto& s_num = sm.num;
    auto& s_den = sm.den;
    auto& s_mk = sm.mk;
    const int t = threadIdx.x;
    const int c0 = ds0 * M::CPS, ncols = (ds1 - ds0) * M::CPS;
    const int npairs = ncols * M::SG + G * M::SG;
    for (int pr = t; pr < npairs; pr += NTHREADS) {
        if (pr < ncols * M::SG) {
            const int cl = pr % ncols, k = pr / ncols;
            s_num[k][cl] = merge_num_part<D, G>(rec0, rec_floats, ns, k, c0 + cl);
        } else {
            const int q = pr - ncols * M::SG;
            const int h = q / M::SG, k = q % M::SG;
            float m;
            s_den[k][h] = merge_den_part<D, G>(rec0, rec_floats, ns, k, h, m);
            s_mk[k][h] = m;
        }
    }
    __syncthreads();
    for (int cl = t; cl < ncols; cl += NTHREADS) {
        const int c = c0 + cl;
        const int h = (c * 4) / D;
        float Mh = s_mk[0][h];
        for (int k = 1; k < M::SG; k++) Mh = fmaxf(Mh, s_mk[k][h]);
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        float dtot = 0.f;
        for (int k = 0; k < M::SG; k++) {
            const float f = fast_exp2(s_mk[k][h] - Mh);
            const f32x4 x = s_num[k][cl];
            tot.x = fmaf(f, x.x, tot.x);
            tot.y = fmaf(f, x.y, tot.y);
            tot.z = fmaf(f, x.z, tot.z);
            tot.w = fmaf(f, x.w, tot.w);
            dtot = fmaf(f, s_den[k][h], dtot);
        }
        store_out4(out, out_kind, obase + c * 4,
                   f32x4{tot.x / dtot, tot.y / dtot, tot.z / dtot, tot.w / dtot});
    }
}

// The merge of one (layer, sequence, kv head) done by the 256 threads of the
// split workgroup that finished last: the same operations in the same order
// as decode_merge_kernel.
template <int D, int G>
__device__ void merge_in_workgroup(MergeLds<D, G>& sm, const float* rec0, int ns, int rec_floats,
                                   void* out, int out_kind, int64_t obase) {
    merge_chunks<D, G, kThreads>(sm, rec0, ns, rec_floats, 0, MergeCfg<D, G>::DS, out, out_kind,
                                 obase);
}

// Split-kernel modes: plain split stage; split stage that also appends the
// new token (hwkv_decode_append_attn); the single-launch step that appends
// and merges by the last-arriving split (hwkv_decode_step).
constexpr int kModePlain = 0, kModeAppend = 1, kModeFused = 2;

// Waves per SIMD the split kernel is built for (a lower bound on occupancy
// the register allocation must allow): three for the MFMA loop up to
// head_dim 128, whose staging takes 48 KiB of LDS per workgroup, so three
// workgroups fit a CU (768 resident on the chip instead of 512); no bound
// otherwise.
template <int T, int D>
constexpr int split_waves_per_simd() { return (mfma_loop<T>() && D <= 128) ? 3 : 1; }

template <int T, int D, int G, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(split_waves_per_simd<T, D>())))
void decode_split_kernel(DecodeSplitArgs a) {
    typedef SplitCfg<T, D, G> C;
    typedef typename Elem<T>::Chunk Chunk;
    constexpr bool FUSED = MODE == kModeFused;     // merges in the last split
    constexpr bool APPENDS = MODE != kModePlain;  // ctx_len holds positions; appends
    constexpr bool MF = mfma_loop<T>();  // MFMA block loop
    static_assert(!MF || G <= 16, "one 16-column S^T tile per GQA group");
    // Partial states the workgroup merge adds up: one per half wave in the
    // per-lane form, one per wave in the MFMA form.  The MFMA form stages, per
    // wave, the K rows of the tile being scored and the V rows of two tiles in
    // LDS (48 KiB per workgroup at head_dim 128, so three workgroups fit a CU);
    // the workgroup merge, and in the single-launch step the merge of a head's
    // splits, reuse that memory once every wave has left its loop.
    constexpr int SLOTS = MF ? kWaves : 2 * kWaves;
    constexpr int kAccBytes = SLOTS * G * D * 4;
    constexpr int kStageBytes = MF ? kWaves * 3 * kBS * C::ROW : 0;
    constexpr int kMergeBytes = FUSED ? (int)sizeof(MergeLds<D, G>) : 0;
    constexpr int kRawBytes = kAccBytes > kStageBytes ? kAccBytes : kStageBytes;
    __shared__ float s_m[kWaves][G];
    __shared__ float s_l[SLOTS][G];
    // appending modes: the new token's K and V rows, parked by the lanes of
    // the wave whose tile holds it and read back by the same lanes
    __shared__ __align__(16) uint8_t s_new[APPENDS ? 2 * C::ROW : 16];
    __shared__ __align__(16) uint8_t s_raw[kRawBytes > kMergeBytes ? kRawBytes : kMergeBytes];
    float(*s_acc)[G * D] = reinterpret_cast<float(*)[G * D]>(s_raw);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int r = lane % C::LPG;  // chunks r, r + LPG, ... of a row
    const int g = lane / C::LPG;  // rows g, g + NG, ... of every tile
    const int b = blockIdx.y;
    const bool streamed = a.rec_streamed != 0;

    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    if (fp != a.fingerprint) {
        // meta of another layout: the split stage leaves no record (the
        // merge stage reports NaN); the fused step writes NaN everywhere
        if constexpr (FUSED) {
            const int64_t n4 = (int64_t)a.n_layers * a.n_seqs * a.n_q_heads * (D / 4);
            const int64_t stride = (int64_t)gridDim.x * gridDim.y * kThreads;
            const float x = __builtin_nanf("");
            for (int64_t e = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
                 e < n4; e += stride)
                store_out4(a.out, a.out_kind, e * 4, f32x4{x, x, x, x});
        }
        return;
    }
    const WorkItem wk = a.work[a.work_begin + blockIdx.x];
    const HeadDesc hd = a.heads[wk.head_index];
    const int64_t L = APPENDS ? a.ctx_len[b] + 1 : a.ctx_len[b];
    const int rel_layer = hd.layer - a.layer_begin;
    const int64_t obase =
        (((int64_t)rel_layer * a.n_seqs + b) * a.n_q_heads + (int64_t)hd.head * G) * D;
    if (L <= 0) {
        if constexpr (FUSED) {  // no context: zeros, as the merge stage writes
            if (wk.split == 0)
                for (int e = threadIdx.x; e < G * D / 4; e += kThreads)
                    store_out4(a.out, a.out_kind, obase + e * 4, f32x4{0.f, 0.f, 0.f, 0.f});
        }
        return;
    }
    // Window [lo, L).  Splits are cut on block boundaries: split j covers
    // the logical blocks [bA + j*SB, bA + (j+1)*SB) with bA = lo / 16 and
    // SB = split_tokens / 16, except that the last split runs to the
    // window's last block.  So only the window's first and last blocks are
    // partial, and the number of splits is ceil(min(w, L) / split_tokens),
    // fixed by (w, L) alone.
    const int64_t lo = L - hd.window > 0 ? L - hd.window : 0;
    const int64_t n_win = L - lo;
    const int64_t ns = (n_win + a.split_tokens - 1) / a.split_tokens;
    if (wk.split >= ns) return;  // beyond a window shorter than w
    const int64_t SB = a.split_tokens / kBS;
    const int64_t bA = lo / kBS, bZ = (L - 1) / kBS;
    const int64_t lb0 = bA + (int64_t)wk.split * SB;
    const int64_t lb1 = wk.split == ns - 1 ? bZ : lb0 + SB - 1;
    float* rec = a.ws + ((int64_t)b * a.n_work_range + blockIdx.x) * a.rec_floats;

    // Fused step: after this workgroup's record is written, count its arrival;
    // the last of the head's ns splits merges all of them and re-arms the
    // counter (nothing waits, so no workgroup can hang on another).  Memory
    // ordering, agent scope (the workgroups run on different XCDs, each with
    // its own L2): the barrier orders every thread's record stores before
    // thread 0's counter increment, which is a release; the workgroup whose
    // increment returns ns - 1 has read the end of that release sequence, so
    // its acquire fence makes every split's record visible, and the barrier
    // after it hands that on to the other threads before they read.
    auto arrive_and_merge = [&]() {
        if constexpr (FUSED) {
            __shared__ uint32_t s_old;
            uint32_t* cnt = a.counters + ((int64_t)rel_layer * a.n_kv_heads + hd.head) * a.n_seqs + b;
            __syncthreads();
            if (threadIdx.x == 0) {
                const uint32_t old =
                    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                if (old == (uint32_t)(ns - 1)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                s_old = old;
            }
            __syncthreads();
            if (s_old != (uint32_t)(ns - 1)) return;
            const float* rec0 =
                a.ws + ((int64_t)b * a.n_work_range + (hd.work_off - a.work_begin)) * a.rec_floats;
            // the merge's LDS: the staging / partial-state memory, which no
            // thread reads any more
            static_assert(sizeof(MergeLds<D, G>) <= sizeof(s_raw), "merge LDS aliases s_raw");
            merge_in_workgroup<D, G>(*reinterpret_cast<MergeLds<D, G>*>(s_raw), rec0, (int)ns,
                                     a.rec_floats, a.out, a.out_kind, obase);
            if (threadIdx.x == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    const int64_t slot = a.seq_slots ? (int64_t)a.seq_slots[b] : (int64_t)b;
    if (slot < 0 || slot >= a.table_rows) {  // invalid slot: an empty record -> NaN output
        for (int e = threadIdx.x; e < G * D; e += kThreads) rec_put(rec + e, 0.f, streamed);
        if (threadIdx.x < G) {
            rec_put(rec + G * D + threadIdx.x, -INFINITY, streamed);
            rec_put(rec + G * D + G + threadIdx.x, 0.f, streamed);
        }
        arrive_and_merge();
        return;
    }
    const int32_t* tbl = a.block_ids + slot * a.blocks_per_seq + hd.table_off;
    const uint32_t nb = (uint32_t)hd.nblocks;

    // Blocks of the split: logical blocks [lb0, lb1]; wave w takes lb0 + w,
    // lb0 + w + 4, ...  Lane i of the wave preloads the physical id of its
    // i-th block, so the loop reads ids with readlane and never waits on
    // the block table.
    const int nblk = (int)(lb1 - lb0 + 1);
    const int my_n = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
    int32_t my_id = -1;
    const int tpb_log2 = a.tpb_log2;  // tiles per block = 1 << tpb_log2
    if (lane < my_n) {
        const uint32_t j = (uint32_t)(((lb0 + wave + (int64_t)lane * kWaves) >> tpb_log2) % nb);
        my_id = tbl[j];
    }
    const uint32_t vofs = (uint32_t)(kBS << tpb_log2) * C::ROW;  // K half of a block

    // Fused step: the new token (position L - 1, logical block bZ) belongs to
    // the last split.  That workgroup writes its K/V rows into the ring slot
    // (the slot's previous token lies outside every window that reads the
    // block) and folds the rows from the arguments, not from the pool.
    const bool new_here = APPENDS && wk.split == ns - 1;
    const int64_t kv_new_off =
        (((int64_t)rel_layer * a.n_seqs + b) * a.n_kv_heads + hd.head) * (int64_t)C::ROW;
    if constexpr (APPENDS) {
        if (new_here && wave == 0 && lane < 2 * (C::ROW / 16)) {
            const int32_t id = tbl[(uint32_t)((bZ >> tpb_log2) % nb)];
            if (id >= 0 && (uint64_t)id < a.n_pool_blocks) {
                const int half = lane / (C::ROW / 16), ch = lane % (C::ROW / 16);
                const int64_t bs = (int64_t)kBS << tpb_log2;
                const uint8_t* src = (half ? a.v_new : a.k_new) + kv_new_off + ch * 16;
                uint8_t* dst = a.pool_w + (uint64_t)id * a.block_bytes +
                               ((int64_t)half * bs + (L - 1) % bs) * C::ROW + ch * 16;
                *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
            }
        }
    }

    const uint64_t nblk_pool = a.n_pool_blocks;
    // physical block i of this wave.  Block 0 stands in for an id outside
    // the pool, so the loads stay in bounds; every block of a split holds
    // tokens of the window, so such an id makes the head's result NaN (the
    // fold poisons the running sum l).
    auto block_ptr = [&](int i, bool& ok) -> const uint8_t* {
        const int32_t id = __builtin_amdgcn_readlane(my_id, i);
        ok = id >= 0 && (uint64_t)id < nblk_pool;
        const uint32_t tile_in_block =
            (uint32_t)(lb0 + wave + (int64_t)i * kWaves) & ((1u << tpb_log2) - 1u);
        return a.pool + (uint64_t)(ok ? id : 0) * a.block_bytes + tile_in_block * (kBS * C::ROW);
    };
    // Appending modes: the new token's rows, from the arguments, replace the
    // loaded rows of its tile (logical tile lb).  The lanes that hold them
    // read their chunks once, before the block loop, and park them in LDS (a
    // load inside the loop would make its wait, the wait counter being in
    // order, drain the tile loads issued before it; registers would cost the
    // third wave per SIMD).
    const int new_row = (int)((L - 1) % kBS);
    // lane holds that row in the wave whose tiles include logical tile bZ
    const bool new_lane = new_here && (new_row - g) % C::NG == 0 &&
                          (int)((bZ - lb0) % kWaves) == wave;
    if constexpr (APPENDS) {
        if (new_lane) {
#pragma unroll
            for (int c = 0; c < C::NC; c++) {
                const int ch = (c * C::LPG + r) * 16;
                *reinterpret_cast<Chunk*>(s_new + ch) =
                    *reinterpret_cast<const Chunk*>(a.k_new + kv_new_off + ch);
                *reinterpret_cast<Chunk*>(s_new + C::ROW + ch) =
                    *reinterpret_cast<const Chunk*>(a.v_new + kv_new_off + ch);
            }
        }
    }
    auto put_new_row = [&](BlockRegs<T, D, G>& br, int64_t lb) {
        if constexpr (APPENDS) {
            if (new_lane && lb == bZ) {
#pragma unroll
                for (int rho = 0; rho < C::ROWS; rho++) {
                    if (g + C::NG * rho == new_row) {
#pragma unroll
                        for (int c = 0; c < C::NC; c++) {
                            const int ch = (c * C::LPG + r) * 16;
                            br.k[rho][c] = *reinterpret_cast<const Chunk*>(s_new + ch);
                            br.v[rho][c] = *reinterpret_cast<const Chunk*>(s_new + C::ROW + ch);
                        }
                    }
                }
            }
        }
    };

    if constexpr (MF) {
        // ---- MFMA block loop ----
        // A wave takes its tiles in pairs.  Each tile's K and V rows go from
        // registers into the wave's own LDS staging area (one K slot, scored
        // before the next tile's K rows replace it; a V slot per tile), and
        // the load of the tile two ahead is issued into the same registers at
        // once; the pair is then folded in from LDS while those loads are in
        // flight:
        //   S^T = K Q^T     head_dim / 32 16x16x32 MFMAs per tile; column
        //                   j of the 16 is query head j of the group (Q^T
        //                   operand zero beyond G); lane l holds tokens
        //                   4 (l / 16) .. + 3 of column l % 16;
        //   O^T += V^T P^T  one 16x16x32 MFMA per 16 rows of O^T and P part;
        //                   the 32 keys of the pair are ordered so that the
        //                   S^T registers of the two tiles are the B operand
        //                   as they stand, and V^T comes from transposing
        //                   LDS reads.
        // P = 2^(s - m) enters the products in parts that sum to it almost
        // exactly: for bf16 caches a truncated high part, a truncated middle
        // part and the rounded rest (relative error below 2^-22); for fp16
        // caches the fp16 value of P 2^15 and its rounded remainder (P 2^15
        // stays in fp16's normal range down to P = 2^-29; the 2^15 is taken
        // out of the accumulator at the end).  l sums P in fp32.
        typedef MfmaCfg<D> F;
        const int col = lane & 15;  // S^T and O^T column (query head of the group)
        const int g16 = lane >> 4;  // output rows 4 g16 .. + 3 of each 16-row tile
        u32x4 qop[F::KSTEP];        // Q^T: dims 32 s + 8 g16 .. + 7 of head col
        {
            const int64_t qoff =
                (((int64_t)rel_layer * a.n_seqs + b) * a.n_q_heads + (int64_t)hd.head * G) * D;
            const uint8_t* qrow = a.q + (qoff + (int64_t)(col < G ? col : 0) * D) * 2;
#pragma unroll
            for (int s = 0; s < F::KSTEP; s++)
                qop[s] = col < G ? *reinterpret_cast<const u32x4*>(qrow + (32 * s + 8 * g16) * 2)
                                 : u32x4{0, 0, 0, 0};
        }
        f32x4 oacc[F::DT];
#pragma unroll
        for (int t = 0; t < F::DT; t++) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m = kEmptyMax, l = 0.f;  // state of column col (same in the 4 lane groups)

        // staging area of this wave: the K rows of the tile being scored,
        // then the V rows of tile 0 and of tile 1
        uint8_t* const stage = s_raw + wave * (3 * F::TILE);
        uint32_t koff[F::KSTEP];  // K operand of k-step s: row col, chunk 4 s + g16
#pragma unroll
        for (int s = 0; s < F::KSTEP; s++)
            koff[s] = (uint32_t)(col * C::ROW + (((4 * s + g16) ^ F::swz(col)) * 16));
        // V^T operand of rows 16 t .. + 15 of O^T: this lane's transposing
        // read covers row 4 g16 + col / 4, dims 16 t + 4 (col % 4) .. + 3
        const int vrow = 4 * g16 + (col >> 2);
        uint32_t voff[F::DT];
#pragma unroll
        for (int t = 0; t < F::DT; t++)
            voff[t] = (uint32_t)(vrow * C::ROW +
                                 (((2 * t + ((col & 3) >> 1)) ^ F::swz(vrow)) * 16) + (col & 1) * 8);

        // rows of a loaded tile into the staging area; V rows outside the
        // window (all rows when the block id was outside the pool) are
        // written as zeros, so that stale pool bytes cannot enter as NaN * 0
        auto stage_put = [&](const BlockRegs<T, D, G>& br, int tau, int64_t lb, bool ok) {
            uint8_t* kst = stage;
            uint8_t* vst = stage + (1 + tau) * F::TILE;
            const int64_t first = lb * kBS;
            const bool full = ok && first >= lo && first + kBS <= L;
#pragma unroll
            for (int rho = 0; rho < C::ROWS; rho++) {
                const int row = g + C::NG * rho;
                const bool keep = full || (ok && first + row >= lo && first + row < L);
#pragma unroll
                for (int c = 0; c < C::NC; c++) {
                    const uint32_t off =
                        (uint32_t)(row * C::ROW + (((c * C::LPG + r) ^ F::swz(row)) * 16));
                    *reinterpret_cast<Chunk*>(kst + off) = br.k[rho][c];
                    *reinterpret_cast<Chunk*>(vst + off) = keep ? br.v[rho][c] : Chunk{};
                }
            }
        };
        auto stage_zero_v = [&](int tau) {  // V rows of a tile the pair does not have
            uint8_t* vst = stage + (1 + tau) * F::TILE;
#pragma unroll
            for (int c = 0; c < F::TILE / (64 * 16); c++)
                *reinterpret_cast<u32x4*>(vst + (c * 64 + lane) * 16) = u32x4{0, 0, 0, 0};
        };
        auto scores = [&]() -> f32x4 {  // S^T of the tile whose K rows are staged
            const uint8_t* kst = stage;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < F::KSTEP; k++)
                s = mfma16<T>(*reinterpret_cast<const u32x4*>(kst + koff[k]), qop[k], s);
            return s;
        };
        // fold the staged pair (tiles i and i + 1 of this wave) into the state
        auto fold_pair = [&](int i, bool okA, bool okB, bool hasB, const f32x4& sA,
                             const f32x4& sB) {
            const int64_t pA = (lb0 + wave + (int64_t)i * kWaves) * kBS + 4 * g16;
            const int64_t pB = pA + kWaves * kBS;
            float sv[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                sv[e] = (okA && pA + e >= lo && pA + e < L) ? sA[e] * a.qk_scale_log2 : -INFINITY;
                sv[4 + e] = (hasB && okB && pB + e >= lo && pB + e < L)
                                ? sB[e] * a.qk_scale_log2
                                : -INFINITY;
            }
            float mx = sv[0];
#pragma unroll
            for (int e = 1; e < 8; e++) mx = fmaxf(mx, sv[e]);
            mx = fmaxf(mx, xor16(mx));
            mx = fmaxf(mx, xor32(mx));
            if (__builtin_amdgcn_ballot_w64(mx > m)) {  // rare once the maxima have settled
                const float mn = fmaxf(m, mx);
                const float alpha = fast_exp2(m - mn);
                l *= alpha;
#pragma unroll
                for (int t = 0; t < F::DT; t++) oacc[t] *= alpha;
                m = mn;
            }
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                p[e] = fast_exp2(sv[e] - m);
                l += p[e];
            }
            u32x4 part[3];
            constexpr int NP = T == kF16 ? 2 : 3;
            if constexpr (T == kF16) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float x0 = p[2 * q] * 32768.f, x1 = p[2 * q + 1] * 32768.f;
                    hw[q] = pack_f16_rne(x0, x1);
                    const f16x2_t h = __builtin_bit_cast(f16x2_t, hw[q]);
                    lw[q] = pack_f16_rne(x0 - (float)h.x, x1 - (float)h.y);
                }
                part[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                part[1] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            } else {
                uint32_t hw[4], mw[4], lw[4];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float x0 = p[2 * q], x1 = p[2 * q + 1];
                    hw[q] = pack_bf16_trunc(x0, x1);
                    const float r0 = x0 - bf16_lo(hw[q]), r1 = x1 - bf16_hi(hw[q]);
                    mw[q] = pack_bf16_trunc(r0, r1);
                    lw[q] = pack_bf16_rne(r0 - bf16_lo(mw[q]), r1 - bf16_hi(mw[q]));
                }
                part[0] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                part[1] = u32x4{mw[0], mw[1], mw[2], mw[3]};
                part[2] = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
#pragma unroll
            for (int t = 0; t < F::DT; t++) {
                const u32x2 v0 = tr_read(stage + F::TILE + voff[t]);
                const u32x2 v1 = tr_read(stage + 2 * F::TILE + voff[t]);
                const u32x4 va = u32x4{v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                for (int k = 0; k < NP; k++) oacc[t] = mfma16<T>(va, part[k], oacc[t]);
            }
            if (!okA || (hasB && !okB)) l = __builtin_nanf("");  // an id outside the pool
        };

        BlockRegs<T, D, G> bufA, bufB;
        bool okA = false, okB = false;
        if (my_n > 0) load_block<T, D, G>(bufA, block_ptr(0, okA), vofs, g, r);
        if (my_n > 1) load_block<T, D, G>(bufB, block_ptr(1, okB), vofs, g, r);
        for (int i = 0; i < my_n; i += 2) {
            const bool hasB = i + 1 < my_n;
            const int64_t lbA = lb0 + wave + (int64_t)i * kWaves;
            wave_lds_order();  // after the previous pair's LDS reads
            const bool curA = okA, curB = okB;
            put_new_row(bufA, lbA);
            stage_put(bufA, 0, lbA, curA);
            if (i + 2 < my_n) load_block<T, D, G>(bufA, block_ptr(i + 2, okA), vofs, g, r);
            wave_lds_order();
            const f32x4 sA = scores();
            wave_lds_order();  // tile 1's K rows replace tile 0's after its scores
            f32x4 sB = {0.f, 0.f, 0.f, 0.f};
            if (hasB) {
                put_new_row(bufB, lbA + kWaves);
                stage_put(bufB, 1, lbA + kWaves, curB);
            } else {
                stage_zero_v(1);
            }
            if (i + 3 < my_n) load_block<T, D, G>(bufB, block_ptr(i + 3, okB), vofs, g, r);
            wave_lds_order();
            if (hasB) sB = scores();
            fold_pair(i, curA, curB, hasB, sA, sB);
        }

        // ---- merge the 4 wave states of the workgroup, in a fixed order ----
        if (lane < G) s_m[wave][lane] = m;
        __syncthreads();  // every wave has also left its loop: s_acc may reuse the staging
        const int hq = col < G ? col : 0;
        float MW = s_m[0][hq];
#pragma unroll
        for (int w = 1; w < kWaves; w++) MW = fmaxf(MW, s_m[w][hq]);
        const float f = fast_exp2(m - MW);
        const float fo = T == kF16 ? f * (1.f / 32768.f) : f;
        float lh = l * f;
        lh += xor16(lh);
        lh += xor32(lh);
        if (col < G) {
#pragma unroll
            for (int t = 0; t < F::DT; t++)
#pragma unroll
                for (int e = 0; e < 4; e++) s_acc[wave][col * D + 16 * t + 4 * g16 + e] = oacc[t][e] * fo;
        }
        if (lane < G) s_l[wave][lane] = lh;
        __syncthreads();
    } else {
        // ---- per-lane block loop ----
        // query chunks of the G heads of this group
        Chunk qv[G][C::NC];
        {
            const int64_t qoff =
                (((int64_t)rel_layer * a.n_seqs + b) * a.n_q_heads + (int64_t)hd.head * G) * D;
            const uint8_t* qb = a.q + qoff * C::EB;
#pragma unroll
            for (int h = 0; h < G; h++)
#pragma unroll
                for (int c = 0; c < C::NC; c++)
                    qv[h][c] = *reinterpret_cast<const Chunk*>(qb + (h * D) * C::EB + (c * C::LPG + r) * 16);
        }

        float m[G], l[G], acc[G][C::DPL];
#pragma unroll
        for (int h = 0; h < G; h++) {
            m[h] = kEmptyMax;
            l[h] = 0.f;
#pragma unroll
            for (int i = 0; i < C::DPL; i++) acc[h][i] = 0.f;
        }

        auto fold = [&](BlockRegs<T, D, G>& br, int i, bool ok) {
            const int64_t lb = lb0 + wave + (int64_t)i * kWaves;
            const int64_t first = lb * kBS;
            put_new_row(br, lb);
            if (ok && first >= lo && first + kBS <= L) {
                process_block<T, D, G, true>(br, nullptr, qv, a.qk_scale_log2, m, l, acc);
            } else {
                bool valid[C::ROWS];
#pragma unroll
                for (int rho = 0; rho < C::ROWS; rho++) {
                    const int64_t pos = first + g + C::NG * rho;
                    valid[rho] = ok && pos >= lo && pos < L;
                }
                process_block<T, D, G, false>(br, valid, qv, a.qk_scale_log2, m, l, acc);
                if (!ok) {  // an id outside the pool: NaN for every query head of the group
#pragma unroll
                    for (int h = 0; h < G; h++) l[h] = __builtin_nanf("");
                }
            }
        };

        // Two blocks per iteration: both blocks' loads (16 KiB per wave) are
        // issued before either is folded in.
        for (int i = 0; i < my_n; i += 2) {
            BlockRegs<T, D, G> bufA, bufB;
            bool okA, okB = false;
            load_block<T, D, G>(bufA, block_ptr(i, okA), vofs, g, r);
            if (i + 1 < my_n) load_block<T, D, G>(bufB, block_ptr(i + 1, okB), vofs, g, r);
            fold(bufA, i, okA);
            if (i + 1 < my_n) fold(bufB, i + 1, okB);
        }

        // ---- merge the 32 group states of the workgroup, in a fixed order ----
#pragma unroll
        for (int h = 0; h < G; h++) {
            float M = m[h];
            if constexpr (C::LPG <= 8) M = fmaxf(M, xor8(M));
            if constexpr (C::LPG <= 16) M = fmaxf(M, xor16(M));
            M = fmaxf(M, xor32(M));
            if (lane == 0) s_m[wave][h] = M;
        }
        __syncthreads();
#pragma unroll
        for (int h = 0; h < G; h++) {
            float MW = s_m[0][h];
#pragma unroll
            for (int w = 1; w < kWaves; w++) MW = fmaxf(MW, s_m[w][h]);
            const float f = fast_exp2(m[h] - MW);
            float lh = l[h] * f;
            if constexpr (C::LPG <= 8) lh += xor8(lh);
            if constexpr (C::LPG <= 16) lh += xor16(lh);
#pragma unroll
            for (int i = 0; i < C::DPL; i++) {
                float x = acc[h][i] * f;
                if constexpr (C::LPG <= 8) x += xor8(x);
                if constexpr (C::LPG <= 16) x += xor16(x);
                acc[h][i] = x;
            }
            if ((lane & 31) < C::LPG) {  // the first group of each half wave holds its sums
                const int sl = wave * 2 + (lane >> 5);
#pragma unroll
                for (int c = 0; c < C::NC; c++)
#pragma unroll
                    for (int e = 0; e < C::EPC; e++)
                        s_acc[sl][h * D + (c * C::LPG + r) * C::EPC + e] = acc[h][c * C::EPC + e];
                if (r == 0) s_l[sl][h] = lh;
            }
        }
        __syncthreads();
    }
    for (int e = threadIdx.x; e < G * D; e += kThreads) {
        float sum = 0.f;
#pragma unroll
        for (int sl = 0; sl < SLOTS; sl++) sum += s_acc[sl][e];
        rec_put(rec + e, sum, streamed);
    }
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float MW = s_m[0][h];
        float lsum = 0.f;
#pragma unroll
        for (int w = 1; w < kWaves; w++) MW = fmaxf(MW, s_m[w][h]);
#pragma unroll
        for (int sl = 0; sl < SLOTS; sl++) lsum += s_l[sl][h];
        rec_put(rec + G * D + h, MW, streamed);
        rec_put(rec + G * D + G + h, lsum, streamed);
    }
    arrive_and_merge();
}

// One workgroup per (layer, sequence, kv head) and group of a.merge_chunks
// column chunks: all DS chunks in one workgroup when there are many heads to
// merge, one chunk per workgroup when there are few (a single layer).
template <int D, int G>
__global__ __launch_bounds__((MergeCfg<D, G>::THREADS)) void decode_merge_kernel(DecodeMergeArgs a) {
    typedef MergeCfg<D, G> M;
    const int groups = M::DS / a.merge_chunks;
    const int ds0 = (blockIdx.x % groups) * a.merge_chunks;
    const int hrel = blockIdx.x / groups;  // kv head within the layer range
    const int b = blockIdx.y;
    const int rel_layer = hrel / a.n_kv_heads;
    const int head = hrel % a.n_kv_heads;
    const int64_t obase =
        (((int64_t)rel_layer * a.n_seqs + b) * a.n_q_heads + (int64_t)head * G) * D;

    const uint64_t fp = *reinterpret_cast<const uint64_t*>(a.meta + 8);
    const int64_t L = a.ctx_len[b] + a.ctx_add;
    if (fp != a.fingerprint || L <= 0) {
        const float x = fp != a.fingerprint ? __builtin_nanf("") : 0.f;
        for (int c = ds0 * M::CPS + (int)threadIdx.x; c < (ds0 + a.merge_chunks) * M::CPS;
             c += M::THREADS)
            store_out4(a.out, a.out_kind, obase + c * 4, f32x4{x, x, x, x});
        return;
    }
    const HeadDesc hd = a.heads[a.layer_begin * a.n_kv_heads + hrel];
    const int64_t n = L < hd.window ? L : hd.window;
    const int ns = (int)((n + a.split_tokens - 1) / a.split_tokens);
    const float* rec0 =
        a.ws + ((int64_t)b * a.n_work_range + (hd.work_off - a.work_begin)) * a.rec_floats;
    __shared__ MergeLds<D, G> s_merge;
    merge_chunks<D, G, M::THREADS>(s_merge, rec0, ns, a.rec_floats, ds0, ds0 + a.merge_chunks, a.out,
                                   a.out_kind, obase);
}

template <int T, int D, int G, int MODE>
hwkv_status launch_split_t(const DecodeSplitArgs& a, hipStream_t s) {
    dim3 grid((unsigned)a.n_work_range, (unsigned)a.n_seqs);
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, MODE>), grid, dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string(MODE == kModeFused ? "decode step launch: "
                                                                  : "decode split launch: ") +
                                      hipGetErrorString(e));
    return HWKV_OK;
}

template <int D, int G>
hwkv_status launch_merge_t(const DecodeMergeArgs& a, hipStream_t s) {
    // few heads to merge (e.g. one layer): one column chunk per workgroup
    DecodeMergeArgs b = a;
    const int64_t heads = (int64_t)a.n_layers * a.n_kv_heads * a.n_seqs;
    b.merge_chunks = heads >= 256 ? MergeCfg<D, G>::DS : 1;
    const int groups = MergeCfg<D, G>::DS / b.merge_chunks;
    dim3 grid((unsigned)(a.n_layers * a.n_kv_heads * groups), (unsigned)a.n_seqs);
    hipLaunchKernelGGL((decode_merge_kernel<D, G>), grid, dim3(MergeCfg<D, G>::THREADS), 0, s, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(HWKV_ERR_HIP, std::string("decode merge launch: ") + hipGetErrorString(e));
    return HWKV_OK;
}

// Instances: group sizes 1..4 and 6, 8 for every element kind and head dim.
#define HWKV_FOR_GROUPS(X) X(1) X(2) X(3) X(4) X(6) X(8)

}  // namespace

bool decode_supported(const hwkv_layout& lay, int group) {
    // block sizes: powers of two from 16 to 256 (whole 16-token tiles)
    const int bs = lay.block_size;
    if (bs < kBS || bs > 256 || (bs & (bs - 1)) != 0) return false;
    if (lay.dtype != HWKV_F32 && lay.dtype != HWKV_BF16 && lay.dtype != HWKV_F16) return false;
    if (lay.head_dim != 64 && lay.head_dim != 128 && lay.head_dim != 256) return false;
    if (lay.head_dim == 256 && lay.dtype == HWKV_F32) return false;
    switch (group) {
        case 1: case 2: case 3: case 4: case 6: case 8: return true;
        default: return false;
    }
}

template <int MODE>
hwkv_status launch_split_any(const hwkv_layout& lay, int group, const DecodeSplitArgs& a,
                             hipStream_t s) {
    if (a.n_work_range <= 0) return HWKV_OK;
    if (lay.head_dim == 256) {  // 16-bit caches
        const bool f16 = lay.dtype == HWKV_F16;
#define HWKV_CASE256(GG)                                                                     \
    case GG:                                                                                 \
        return f16 ? launch_split_t<kF16, 256, GG, MODE>(a, s)                               \
                   : launch_split_t<kBF16, 256, GG, MODE>(a, s);
        switch (group) {
            HWKV_CASE256(1) HWKV_CASE256(2) HWKV_CASE256(3) HWKV_CASE256(4) HWKV_CASE256(6)
            HWKV_CASE256(8)
            default: break;
        }
#undef HWKV_CASE256
        return fail(HWKV_ERR_UNSUPPORTED, "no head_dim 256 decode kernel for GQA group " +
                                              std::to_string(group));
    }
    const bool d128 = lay.head_dim == 128;
#define HWKV_CASE(GG)                                                                        \
    case GG:                                                                                 \
        if (lay.dtype == HWKV_BF16)                                                          \
            return d128 ? launch_split_t<kBF16, 128, GG, MODE>(a, s)                        \
                        : launch_split_t<kBF16, 64, GG, MODE>(a, s);                        \
        if (lay.dtype == HWKV_F16)                                                           \
            return d128 ? launch_split_t<kF16, 128, GG, MODE>(a, s)                         \
                        : launch_split_t<kF16, 64, GG, MODE>(a, s);                         \
        return d128 ? launch_split_t<kF32, 128, GG, MODE>(a, s)                             \
                    : launch_split_t<kF32, 64, GG, MODE>(a, s);
    switch (group) {
        HWKV_FOR_GROUPS(HWKV_CASE)
        default: break;
    }
#undef HWKV_CASE
    return fail(HWKV_ERR_UNSUPPORTED, "no decode kernel for GQA group " + std::to_string(group));
}

hwkv_status launch_decode_split(const hwkv_layout& lay, int group, const DecodeSplitArgs& a,
                                hipStream_t s) {
    return launch_split_any<kModePlain>(lay, group, a, s);
}

hwkv_status launch_decode_split_append(const hwkv_layout& lay, int group,
                                       const DecodeSplitArgs& a, hipStream_t s) {
    return launch_split_any<kModeAppend>(lay, group, a, s);
}

hwkv_status launch_decode_step(const hwkv_layout& lay, int group, const DecodeSplitArgs& a,
                               hipStream_t s) {
    return launch_split_any<kModeFused>(lay, group, a, s);
}

hwkv_status launch_decode_merge(const hwkv_layout& lay, int group, const DecodeMergeArgs& a,
                                hipStream_t s) {
    if (lay.head_dim == 256) {
        switch (group) {
            case 1: return launch_merge_t<256, 1>(a, s);
            case 2: return launch_merge_t<256, 2>(a, s);
            case 3: return launch_merge_t<256, 3>(a, s);
            case 4: return launch_merge_t<256, 4>(a, s);
            case 6: return launch_merge_t<256, 6>(a, s);
            case 8: return launch_merge_t<256, 8>(a, s);
            default: break;
        }
        return fail(HWKV_ERR_UNSUPPORTED, "no head_dim 256 merge kernel for GQA group " +
                                              std::to_string(group));
    }
#define HWKV_CASE(GG)                                                                        \
    case GG:                                                                                 \
        return lay.head_dim == 128 ? launch_merge_t<128, GG>(a, s) : launch_merge_t<64, GG>(a, s);
    switch (group) {
        HWKV_FOR_GROUPS(HWKV_CASE)
        default: break;
    }
#undef HWKV_CASE
    return fail(HWKV_ERR_UNSUPPORTED, "no decode kernel for GQA group " + std::to_string(group));
}

}  // namespace hwkv
