// Fused block-sparse attention forward for 128-row query tiles over 128-key
// KV tiles, for launches with few work items (dense attention at S = 4k):
// two KV streams of whole tiles, each stream single-buffered.
//
// What is computed: FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// ref_masked_sdpa_fp32 (per-wave arithmetic in wave_engine.h). The two-stream
// split of a query tile's list with an FP32 merge follows that page's fork
// notes; the merge is the split-KV combination of page
// "BlackwellMultiHeadLatentAttentionForwardFP8" (reduction_kernel).
//
// Schedule. Wave w and wave w+4 own the same 32 rows; group 0 (waves 0-3)
// takes the first half of the list, group 1 the second. Both groups
// alternate MFMA phases (M_j: O += V_{j-1} P_{j-1}, S_j = K_j Q^T, 64 MFMAs
// per wave as in the 256-row kernel) and softmax phases, group 1 one phase
// behind, with a workgroup barrier after every phase ("window"):
//
//     window:   0      1      2      3     ...
//     group 0:  M_0    V_0    M_1    V_1   ...
//     group 1:  -      M_0    V_0    M_1   ...
//
// Each group holds one K and one V tile in LDS (4 tiles = 128 KB at D = 128).
// After group g's M_j both of its buffers are free for one window, in which
// its K_{j+1} and V_j are fetched with direct-to-LDS loads and waited for
// before the window's barrier (the K/V of a dense head are L2-resident).
// Which waves issue which loads is set by measurement (see the note at the
// loads below). At the end group 1 hands its partial rows to group 0
// through LDS, which merges and writes O and LSE.
#include "device_common.h"
#include "vsa_internal.h"
#include "wave_engine.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kIdxCap2t = 8192;  // CSR row entries staged in LDS (>= the largest idx_ld)

template <int D, bool PARTIAL>
__global__ __launch_bounds__(512) void vsa_fwd_2t_kernel(FwdParams prm) {
    constexpr int BQ = 128;
    constexpr int BKV = 128;
    using E = WaveEngine<BKV, D>;
    using G = TileGeom<BKV, D>;
    using F = TileFetch<BKV, D, 4>;  // a tile is fetched by the four waves of the other group
    constexpr int GROUP_LDS = 2 * G::TILE;  // K, V of one group
    static_assert(4 * E::STATE_WORDS * 64 * 4 <= 2 * GROUP_LDS, "merge exchange must fit in the tile buffers");
    __shared__ __attribute__((aligned(1024))) char smem[2 * GROUP_LDS + kIdxCap2t * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31;

    const int wi = xcd_contiguous_block();
    if (wi >= prm.n_work) return;
    const int item = prm.work ? prm.work[wi] : wi;
    if (item < 0 || item >= prm.n_items) return;

    const int p = item % prm.nq;
    const int bh = item / prm.nq;
    const int h = bh % prm.H;
    const int b = bh / prm.H;
    const int S = prm.S;
    const int64_t tok_stride = (int64_t)prm.H * D;  // o is contiguous
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld;
    const int ldc = prm.ld < kIdxCap2t ? prm.ld : kIdxCap2t;
    int n = prm.cnt[item];
    n = n < 0 ? 0 : (n > ldc ? ldc : n);
    const int nkv = prm.nkv;
    const int q0 = p * BQ + (wave & 3) * 32;
    // group 0: entries [0, N0), group 1: [N0, n)
    const int N0 = (n + 1) / 2, N1 = n - N0;
    const int ng = grp ? N1 : N0;

    E e;
    e.init(smem, lane, prm.scale_log2);
    e.load_q(prm.q + (int64_t)b * prm.qs[0] + (int64_t)(q0 + l32) * prm.qs[1] + (int64_t)h * prm.qs[2]);

    int* lidx = (int*)(smem + 2 * GROUP_LDS);
    for (int i = tid; i < ldc; i += 512) lidx[i] = stage_entry<PARTIAL>(irow[i], nkv, BKV, prm.kv_valid);
    e.q_ready();

    auto valid = [&](int t) { return t >= 0 && t < nkv; };
    const char* kbase = (const char*)(prm.k + (int64_t)b * prm.ks[0] + (int64_t)h * prm.ks[2]);
    const char* vbase = (const char*)(prm.v + (int64_t)b * prm.vs[0] + (int64_t)h * prm.vs[2]);
    const int kt_bytes = (int)(prm.ks[1] * 2), vt_bytes = (int)(prm.vs[1] * 2);  // K and V row strides
    const F fetch(smem, wave & 3, lane, kt_bytes, vt_bytes);
    auto tile_at = [&](const char* base, int row_bytes, int t) {
        return uniform_ptr(base + (int64_t)(valid(t) ? t : 0) * BKV * row_bytes);
    };
    // buffers of group g
    auto kbuf = [](int g) { return g * GROUP_LDS; };
    auto vbuf = [](int g) { return g * GROUP_LDS + G::TILE; };
    // list entry of tile j of group g, and its valid keys
    auto entry = [&](int g, int j) { return __builtin_amdgcn_readfirstlane(lidx[(g ? N0 : 0) + j]); };
    auto tile_of = [&](int g, int j) { return entry_tile<PARTIAL>(entry(g, j)); };
    auto keys_of = [&](int g, int j) { return entry_keys<PARTIAL>(entry(g, j), BKV); };

    // K_0 of each group, fetched by that group before the first window; its
    // tile index is read from the CSR row in global memory, since the staged
    // copy is not visible to every wave before the barrier
    if (ng > 0)
        fetch.all(kbuf(grp), tile_at(kbase, kt_bytes, __builtin_amdgcn_readfirstlane(irow[grp ? N0 : 0])), kt_bytes, kLayoutK);
    wait_global_loads();
    lds_barrier();

    // Where the tile loads go. Group 0 (waves 0-3, the older wave on each
    // SIMD) fetches its own K_{j+1} and V_j during its softmax V_j, and group
    // 1's V_{j-1} during its M_j, spread over the MFMA steps; group 1 fetches
    // its own K_{j+1} during its softmax V_j. Loads issued by the younger
    // wave of a SIMD while the older one runs its softmax were measured to
    // stretch that MFMA phase by a third, so group 1 issues none in its
    // MFMA phases; each group's softmax runs beside a longer MFMA phase and
    // has the slack for its loads.
    auto k_loads = [&](int g, int kj) {  // BPW hooks: K_kj of group g, if it exists
        const bool dk = kj < (g ? N1 : N0);
        const char* kt = dk ? tile_at(kbase, kt_bytes, tile_of(g, kj)) : nullptr;
        const int kd = kbuf(g);
        return [=, &fetch](int i) { if (dk) fetch.block(kd, kt, kt_bytes, kLayoutK, i); };
    };
    auto v_loads = [&](int g, int vj) {  // BPW hooks: V_vj of group g, if it exists
        const bool dv = vj >= 0 && vj < (g ? N1 : N0);
        const char* vt = dv ? tile_at(vbase, vt_bytes, tile_of(g, vj)) : nullptr;
        const int vd = vbuf(g);
        return [=, &fetch](int i) { if (dv) fetch.block(vd, vt, vt_bytes, kLayoutV, i); };
    };
    auto issue = [](const auto& hooks) {
#pragma unroll
        for (int i = 0; i < F::BPW; ++i) hooks(i);
    };
    auto softmax_ok = [&](int j) __attribute__((always_inline)) {
        const int nv = keys_of(grp, j);
        if (PARTIAL && nv > 0 && nv < BKV) e.mask_keys(nv);
        return nv > 0;
    };

    // Group g runs M_j in window 2j + g and its softmax V_j in window
    // 2j + 1 + g, for j = 0 .. ng (M_ng is the PV of its last tile). Each
    // group's loop body is M_j then V_j, so that S (live from M_j to V_j) and
    // P (from V_j to M_{j+1}) never both cross the back-edge; every wave
    // passes the same number of barriers (the shorter side pads).
    const int b0 = n > 0 ? 2 * N0 + 2 : 0, b1 = n > 0 ? 2 * N1 + 3 : 0;
    const int total = b0 > b1 ? b0 : b1;
    int nbar = 0;
    auto bar = [&]() {
        lds_barrier();
        ++nbar;
    };
    if (n > 0) {
        if (grp == 0) {
            // N0 >= 1 and N0 >= N1
            e.template mfma_phase<false, true>(0, kbuf(0));  // M_0
            bar();
            issue(k_loads(0, 1));
            issue(v_loads(0, 0));
            e.softmax(softmax_ok(0));  // V_0
            wait_global_loads();
            bar();
            int j = 1;
            for (; j < N0; ++j) {
                e.template mfma_phase<true, true, F::BPW>(vbuf(0), kbuf(0), v_loads(1, j - 1));  // M_j
                wait_global_loads();
                bar();
                issue(k_loads(0, j + 1));
                issue(v_loads(0, j));
                e.softmax(softmax_ok(j));  // V_j
                wait_global_loads();
                bar();
            }
            e.template mfma_phase<true, false, F::BPW>(vbuf(0), 0, v_loads(1, j - 1));  // M_N0
            wait_global_loads();
            bar();
            bar();
        } else {
            bar();
            if (N1 > 0) {
                e.template mfma_phase<false, true>(0, kbuf(1));  // M_0
                bar();
                issue(k_loads(1, 1));
                e.softmax(softmax_ok(0));  // V_0
                wait_global_loads();
                bar();
                int j = 1;
                for (; j < N1; ++j) {
                    e.template mfma_phase<true, true>(vbuf(1), kbuf(1));  // M_j
                    bar();
                    issue(k_loads(1, j + 1));
                    e.softmax(softmax_ok(j));  // V_j
                    wait_global_loads();
                    bar();
                }
                e.template mfma_phase<true, false>(vbuf(1), 0);  // M_N1
                bar();
                bar();
            }
        }
    }
    while (nbar < total) bar();

    // merge the two streams' partial rows; the tile buffers are free now
    float* xch = (float*)smem + (wave & 3) * E::STATE_WORDS * 64;
    if (grp == 1) e.export_state(xch);
    lds_barrier();
    if (grp == 0) {
        e.merge_state(xch);
        e.store(prm.o + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D,
                prm.lse + ((int64_t)b * prm.H + h) * S + q0 + l32);
    }
}

template <int D>
hipError_t launch_2t(const FwdParams& p, hipStream_t stream) {
    if (p.kv_valid) hipLaunchKernelGGL((vsa_fwd_2t_kernel<D, true>), dim3(p.n_work), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((vsa_fwd_2t_kernel<D, false>), dim3(p.n_work), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_2t(int head_dim, const FwdParams& p, hipStream_t stream) {
    if (p.n_work <= 0) return hipSuccess;
    if (head_dim == 128) return launch_2t<128>(p, stream);
    if (head_dim == 64) return launch_2t<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace vsa
