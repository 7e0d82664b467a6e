// Drives every entry point of the C ABI through its host-side work (layout
// construction, estimates, tables, validation, argument marshalling) under
// the address and undefined-behaviour sanitizers.  Device pointers are fake,
// suitably aligned addresses: the kernel launchers are stand-ins that never
// touch them.  Exit status 0 means every expectation held; the sanitizers
// abort the process on the first report.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "hwkv.h"

namespace hwkv {
extern int g_launches;
}

static int failures = 0;
#define EXPECT(cond)                                                             \
    do {                                                                         \
        if (!(cond)) {                                                           \
            fprintf(stderr, "line %d: expectation failed: %s (%s)\n", __LINE__, #cond, \
                    hwkv_last_error());                                          \
            failures++;                                                          \
        }                                                                        \
    } while (0)

template <class T>
static T* fake(uintptr_t mib) {
    return reinterpret_cast<T*>(mib << 20);
}

// every host call on one layout, and every device entry point both with a
// rejected argument and with arguments that pass validation
static void exercise(int L, int H, const std::vector<int32_t>& w, int bs, int d, hwkv_dtype dt,
                     int split, int G) {
    hwkv_layout* lay = nullptr;
    if (hwkv_layout_create(L, H, w.data(), bs, d, dt, split, &lay) != HWKV_OK) {
        fprintf(stderr, "layout_create failed: %s\n", hwkv_last_error());
        failures++;
        return;
    }
    hwkv_layout_desc desc;
    EXPECT(hwkv_layout_query(lay, &desc, nullptr, nullptr, nullptr) == HWKV_OK);
    std::vector<int32_t> wq(L * H), nb(L * H);
    std::vector<int64_t> off(L * H + 1);
    EXPECT(hwkv_layout_query(lay, &desc, wq.data(), nb.data(), off.data()) == HWKV_OK);
    EXPECT(wq == w);
    int64_t bps = 0;
    for (int i = 0; i < L * H; i++) {
        EXPECT(nb[i] == (w[i] + bs - 1) / bs);
        EXPECT(off[i] == bps);
        bps += nb[i];
    }
    EXPECT(off[L * H] == bps && desc.blocks_per_seq == bps);

    const int64_t n_seqs = 3;
    uint64_t est = 0;
    EXPECT(hwkv_mem_estimate(lay, n_seqs, &est) == HWKV_OK);
    const uint64_t esz = dt == HWKV_F32 ? 4 : 2;
    EXPECT(est == (uint64_t)n_seqs * (uint64_t)bps * (uint64_t)bs * (uint64_t)d * 2 * esz);
    int64_t row = -1;
    int32_t fl = -1, fh = -1;
    EXPECT(hwkv_capacity_check(lay, n_seqs, est, &row, &fl, &fh) == HWKV_OK);
    EXPECT(hwkv_capacity_check(lay, n_seqs, est - 1, &row, &fl, &fh) == HWKV_ERR_CAPACITY);
    EXPECT(strstr(hwkv_last_error(), "layer") != nullptr);
    uint64_t big = 0;
    EXPECT(hwkv_mem_estimate(lay, INT64_MAX / 2, &big) == HWKV_ERR_OVERFLOW);

    std::vector<int32_t> tbl((size_t)(n_seqs * bps));
    EXPECT(hwkv_table_fill(lay, n_seqs, tbl.data()) == HWKV_OK);
    for (int64_t i = 0; i < n_seqs * bps; i++) EXPECT(tbl[i] == (int32_t)i);
    std::vector<uint8_t> meta(desc.meta_bytes);
    EXPECT(hwkv_meta_fill(lay, meta.data(), meta.size()) == HWKV_OK);
    EXPECT(hwkv_meta_fill(lay, meta.data(), meta.size() - 1) != HWKV_OK);

    const int nq = H * G;
    uint64_t ws = 0, sws = 0;
    EXPECT(hwkv_workspace_bytes(lay, 0, L, (int32_t)n_seqs, nq, &ws) == HWKV_OK);
    EXPECT(hwkv_step_workspace_bytes(lay, 0, L, (int32_t)n_seqs, nq, &sws) == HWKV_OK);
    EXPECT(sws >= ws);
    EXPECT(hwkv_workspace_bytes(lay, 0, L + 1, (int32_t)n_seqs, nq, &ws) != HWKV_OK);
    EXPECT(hwkv_workspace_bytes(lay, 0, L, (int32_t)n_seqs, nq + 1, &ws) != HWKV_OK);
    EXPECT(hwkv_step_workspace_bytes(lay, 0, L, (int32_t)n_seqs, nq, &sws) == HWKV_OK);
    // prefill: bf16 caches take an fp16 copy of the V rows, other dtypes none
    uint64_t pws = 1, pws7 = 1;
    EXPECT(hwkv_prefill_workspace_bytes(lay, L - 1, (int32_t)n_seqs, 77, &pws) == HWKV_OK);
    EXPECT(hwkv_prefill_workspace_bytes(lay, 0, (int32_t)n_seqs, 7, &pws7) == HWKV_OK);
    {
        uint64_t rows = 0;
        for (int h = 0; h < H; h++) rows += (uint64_t)w[(size_t)(L - 1) * H + h] - 1 + 77;
        EXPECT(pws == (dt == HWKV_BF16 ? (uint64_t)n_seqs * rows * (uint64_t)d * 2 : 0));
    }
    EXPECT(hwkv_prefill_workspace_bytes(lay, L, (int32_t)n_seqs, 7, &pws7) != HWKV_OK);
    EXPECT(hwkv_prefill_workspace_bytes(lay, 0, (int32_t)n_seqs, 0, &pws7) != HWKV_OK);
    EXPECT(hwkv_prefill_workspace_bytes(lay, 0, (int32_t)n_seqs, 7, nullptr) != HWKV_OK);
    EXPECT(hwkv_prefill_workspace_bytes(lay, 0, (int32_t)n_seqs, 7, &pws7) == HWKV_OK);

    uint64_t mfp = 0;
    EXPECT(hwkv_meta_fingerprint(meta.data(), meta.size(), &mfp) == HWKV_OK);
    EXPECT(mfp == desc.fingerprint);
    EXPECT(hwkv_meta_fingerprint(meta.data(), 16, &mfp) == HWKV_ERR_INVALID_ARG);
    EXPECT(hwkv_meta_fingerprint(nullptr, meta.size(), &mfp) == HWKV_ERR_INVALID_ARG);
    std::vector<uint8_t> junk(meta.size(), 0);
    EXPECT(hwkv_meta_fingerprint(junk.data(), junk.size(), &mfp) == HWKV_ERR_ABI_MISMATCH);

    hwkv_cache c = {fake<void>(1024), est, fake<const int32_t>(2048), n_seqs,
                    fake<const void>(2049), mfp};
    hwkv_cache small = c;
    small.pool_bytes = est - 1;
    void* wsp = fake<void>(4096);
    const int32_t* slots = fake<const int32_t>(5000);
    const int64_t* pos = fake<const int64_t>(5001);
    const void* q = fake<const void>(5002);
    const void* k = fake<const void>(5003);
    const void* v = fake<const void>(5004);
    void* out = fake<void>(5005);
    const int ns = (int)n_seqs;
    const int before = hwkv::g_launches;

    // accepted calls (the stand-in launchers count them)
    EXPECT(hwkv_append(lay, &c, 0, L, ns, slots, pos, 5, k, v, nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_split(lay, &c, 0, L, ns, slots, pos, nq, q, 0.1f, wsp, ws, nullptr) ==
           HWKV_OK);
    EXPECT(hwkv_decode_merge(lay, &c, 0, L, ns, pos, nq, wsp, ws, out, HWKV_BF16, nullptr) ==
           HWKV_OK);
    EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns, slots, pos, nq, q, 0.1f, wsp, ws, out, HWKV_F32,
                            nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_split_append(lay, &c, 0, L, ns, nullptr, pos, k, v, nq, q, 0.1f, wsp, ws,
                                    nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_append_attn(lay, &c, 0, L, ns, slots, pos, k, v, nq, q, 0.1f, wsp, ws, out,
                                   HWKV_F16, nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_step(lay, &c, 0, L, ns, slots, pos, k, v, nq, q, 0.1f, wsp, sws, out,
                            HWKV_F32, nullptr) == HWKV_OK);
    if (ws <= HWKV_STATIC_SCRATCH_BYTES)
        EXPECT(hwkv_decode_append_attn_static(lay, &c, 0, L, ns, slots, pos, k, v, nq, q, 0.1f,
                                              out, HWKV_BF16, nullptr) == HWKV_OK);
    EXPECT(hwkv_prefill_attn(lay, &c, L - 1, ns, slots, pos, 77, nq, q, k, v, wsp, pws, out,
                             HWKV_BF16, 0.1f, nullptr) == HWKV_OK);
    EXPECT(hwkv_prefill_attn_exact(lay, &c, 0, ns, nullptr, pos, 1, nq, q, k, v, out, HWKV_F32,
                                   0.1f, nullptr) == HWKV_OK);
    // the merge reads only the workspace and the contexts: a batch larger
    // than the table (several entries reading one slot) is accepted
    EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns + 2, slots, pos, nq, q, 0.1f, wsp, 2 * ws, out,
                            HWKV_F32, nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_merge(lay, &c, 0, L, ns + 2, pos, nq, wsp, 2 * ws, out, HWKV_F32,
                             nullptr) == HWKV_OK);
    EXPECT(hwkv_decode_append_attn(lay, &c, 0, L, ns + 2, slots, pos, k, v, nq, q, 0.1f, wsp,
                                   2 * ws, out, HWKV_BF16, nullptr) == HWKV_OK);
    EXPECT(hwkv::g_launches > before);

    // rejected calls: nothing launched
    const int mid = hwkv::g_launches;
    EXPECT(hwkv_append(lay, &small, 0, L, ns, slots, pos, 5, k, v, nullptr) == HWKV_ERR_CAPACITY);
    EXPECT(hwkv_append(lay, &c, 0, L, ns, slots, pos, 0, k, v, nullptr) != HWKV_OK);
    EXPECT(hwkv_append(lay, &c, 0, L + 1, ns, slots, pos, 1, k, v, nullptr) != HWKV_OK);
    EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns, slots, pos, nq, q, 0.1f, wsp, ws - 1, out,
                            HWKV_F32, nullptr) != HWKV_OK);
    EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns, slots, pos, nq + 1, q, 0.1f, wsp, ws, out,
                            HWKV_F32, nullptr) != HWKV_OK);
    EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns, slots, pos, nq, (const char*)q + 2, 0.1f, wsp, ws,
                            out, HWKV_F32, nullptr) == HWKV_ERR_MISALIGNED);
    EXPECT(hwkv_decode_step(lay, &c, 0, L, ns, slots, pos, k, v, nq, q, 0.1f, wsp, ws - 1, out,
                            HWKV_F32, nullptr) != HWKV_OK);
    EXPECT(hwkv_prefill_attn(lay, &c, L, ns, slots, pos, 7, nq, q, k, v, wsp, pws7, out,
                             HWKV_F32, 0.1f, nullptr) != HWKV_OK);
    if (pws7 > 0) {  // a short or missing prefill workspace
        EXPECT(hwkv_prefill_attn(lay, &c, 0, ns, slots, pos, 7, nq, q, k, v, wsp, pws7 - 1, out,
                                 HWKV_F32, 0.1f, nullptr) == HWKV_ERR_CAPACITY);
        EXPECT(hwkv_prefill_attn(lay, &c, 0, ns, slots, pos, 7, nq, q, k, v, nullptr, pws7, out,
                                 HWKV_F32, 0.1f, nullptr) == HWKV_ERR_INVALID_ARG);
    }
    EXPECT(hwkv_prefill_attn_exact(lay, &c, 0, ns, slots, pos, 0, nq, q, k, v, out, HWKV_F32,
                                   0.1f, nullptr) != HWKV_OK);
    EXPECT(hwkv_prefill_attn(lay, nullptr, 0, ns, slots, pos, 7, nq, q, k, v, wsp, pws7, out,
                             HWKV_F32, 0.1f, nullptr) != HWKV_OK);
    // the static scratch refuses a call whose records exceed it
    EXPECT(hwkv_decode_append_attn_static(lay, &c, 0, L, 65535, slots, pos, k, v, nq, q, 0.1f,
                                          out, HWKV_F32, nullptr) == HWKV_ERR_CAPACITY);
    EXPECT(strstr(hwkv_last_error(), "static scratch") != nullptr);
    // a view whose blob belongs to another layout (kernel-ABI check)
    hwkv_cache other = c;
    other.meta_fingerprint ^= 1;
    EXPECT(hwkv_append(lay, &other, 0, L, ns, slots, pos, 5, k, v, nullptr) ==
           HWKV_ERR_ABI_MISMATCH);
    EXPECT(hwkv_decode_attn(lay, &other, 0, L, ns, slots, pos, nq, q, 0.1f, wsp, ws, out,
                            HWKV_F32, nullptr) == HWKV_ERR_ABI_MISMATCH);
    EXPECT(hwkv_decode_merge(lay, &other, 0, L, ns, pos, nq, wsp, ws, out, HWKV_F32, nullptr) ==
           HWKV_ERR_ABI_MISMATCH);
    EXPECT(hwkv_decode_step(lay, &other, 0, L, ns, slots, pos, k, v, nq, q, 0.1f, wsp, sws, out,
                            HWKV_F32, nullptr) == HWKV_ERR_ABI_MISMATCH);
    EXPECT(hwkv_prefill_attn(lay, &other, 0, ns, slots, pos, 7, nq, q, k, v, wsp, pws7, out,
                             HWKV_F32, 0.1f, nullptr) == HWKV_ERR_ABI_MISMATCH);
    // the softmax scale must be finite and positive
    const float bad_scales[3] = {0.0f, -0.5f, __builtin_nanf("")};
    for (float sc : bad_scales) {
        EXPECT(hwkv_decode_attn(lay, &c, 0, L, ns, slots, pos, nq, q, sc, wsp, ws, out, HWKV_F32,
                                nullptr) == HWKV_ERR_INVALID_ARG);
        EXPECT(hwkv_decode_step(lay, &c, 0, L, ns, slots, pos, k, v, nq, q, sc, wsp, sws, out,
                                HWKV_F32, nullptr) == HWKV_ERR_INVALID_ARG);
        EXPECT(hwkv_prefill_attn(lay, &c, 0, ns, slots, pos, 7, nq, q, k, v, wsp, pws7, out,
                                 HWKV_F32, sc, nullptr) == HWKV_ERR_INVALID_ARG);
    }
    EXPECT(hwkv::g_launches == mid);
    hwkv_layout_destroy(lay);
}

int main() {
    EXPECT(hwkv_abi_version() == HWKV_ABI_VERSION);
    EXPECT(hwkv_last_error() != nullptr);

    // the printed policy's layer 0, and a seeded 48-layer draw from its levels
    exercise(1, 8, {4096, 4096, 16384, 16384, 65536, 65536, 65536, 65536}, 16, 128, HWKV_BF16, 0,
             3);
    std::mt19937 rng(7);
    const int32_t levels[4] = {1024, 4096, 16384, 65536};
    std::vector<int32_t> w48(48 * 8);
    for (auto& x : w48) x = levels[rng() % 4];
    exercise(48, 8, w48, 16, 128, HWKV_BF16, 1024, 3);
    // ragged windows, other block sizes, head dims and dtypes
    std::vector<int32_t> wr(3 * 5);
    for (auto& x : wr) x = 1 + (int32_t)(rng() % 5000);
    exercise(3, 5, wr, 16, 64, HWKV_F32, 64, 2);
    exercise(3, 5, wr, 32, 256, HWKV_F16, 0, 8);
    exercise(3, 5, wr, 256, 128, HWKV_BF16, 512, 1);
    exercise(2, 2, {1, 1, 3, 2}, 1, 16, HWKV_F32, 0, 4);

    // rejected layouts
    hwkv_layout* lay = nullptr;
    const int32_t ok_w[2] = {64, 16}, bad_w[2] = {64, 0}, huge_w[2] = {INT32_MAX, INT32_MAX};
    EXPECT(hwkv_layout_create(1, 2, nullptr, 16, 128, HWKV_BF16, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(0, 2, ok_w, 16, 128, HWKV_BF16, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, bad_w, 16, 128, HWKV_BF16, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, ok_w, 0, 128, HWKV_BF16, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, ok_w, 16, 0, HWKV_BF16, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, ok_w, 16, 128, (hwkv_dtype)9, 0, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, ok_w, 16, 128, HWKV_BF16, 24, &lay) != HWKV_OK);
    EXPECT(hwkv_layout_create(1, 2, ok_w, 16, 128, HWKV_BF16, 0, nullptr) != HWKV_OK);
    if (hwkv_layout_create(1, 2, huge_w, 1024, 1024, HWKV_F32, 0, &lay) == HWKV_OK) {
        uint64_t b = 0;
        EXPECT(hwkv_mem_estimate(lay, INT64_MAX / 4, &b) == HWKV_ERR_OVERFLOW);
        hwkv_layout_destroy(lay);
    }
    hwkv_layout_destroy(nullptr);

    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("host ABI under sanitizers: ok (%d stand-in launches)\n", hwkv::g_launches);
    return 0;
}
