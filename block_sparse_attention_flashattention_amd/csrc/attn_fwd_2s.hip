// Fused block-sparse attention forward for 128-row query tiles on gfx950:
// two KV streams per query tile, one per wave group, in alternating phases.
//
// What is computed: FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// ref_masked_sdpa_fp32 (per-wave arithmetic in wave_engine.h). The split of
// one query tile's KV list into two streams whose (max, sum, O) partials are
// merged in fp32 follows that page's fork notes (single-Q-block, two-KV-stream
// schedule with an FP32 online-softmax merge); the merge itself is the
// split-KV combination of page "BlackwellMultiHeadLatentAttentionForwardFP8"
// (reduction_kernel: rescale each partial to the larger max).
//
// Schedule. All eight waves work on the same 128 query rows: wave w and wave
// w+4 own rows [32*(w%4), +32). The tile's KV list, cut into 64-key
// sub-tiles, is split in two halves: group 0 (waves 0-3) takes the first,
// group 1 (waves 4-7) the second. Each group runs MFMA phases (PV of its
// previous sub-tile, QK of its current one) and softmax phases; group 1 is
// one phase behind group 0 and every phase ends in a workgroup barrier, so on
// each SIMD one wave issues MFMAs while the other runs the softmax. Each group
// has its own double-buffered K/V sub-tiles in LDS and fetches them itself
// with direct-to-LDS loads issued at the start of its MFMA phase M_j (K_{j+1},
// V_j) and waited for at the end of its softmax phase V_j. At the end group 1
// hands its partial rows to group 0 through LDS, which merges and writes O and
// LSE.
#include "device_common.h"
#include "vsa_internal.h"
#include "wave_engine.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kIdxCap2s = 8192;  // CSR row entries staged in LDS (>= the largest idx_ld)

template <int D, bool PARTIAL>
__global__ __launch_bounds__(512) void vsa_fwd_2s_kernel(FwdParams prm) {
    constexpr int BQ = 128;
    constexpr int SUB = 64;  // keys per sub-tile
    using E = WaveEngine<SUB, D>;
    using G = TileGeom<SUB, D>;
    constexpr int GROUP_LDS = 4 * G::TILE;  // K[2], V[2] of one group
    static_assert(4 * E::STATE_WORDS * 64 * 4 <= 2 * GROUP_LDS, "merge exchange must fit in the tile buffers");
    __shared__ __attribute__((aligned(1024))) char smem[2 * GROUP_LDS + kIdxCap2s * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
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
    // The count, the CSR row and Q are fetched at once; the row is read up
    // to its allocated length ld, so it does not wait for the count.
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld;
    const int ldc = prm.ld < kIdxCap2s ? prm.ld : kIdxCap2s;
    int n = prm.cnt[item];
    n = n < 0 ? 0 : (n > ldc ? ldc : n);
    const int nkv = prm.nkv;
    const int block_kv = prm.block_kv;
    const int R = block_kv / SUB;  // sub-tiles per CSR tile (1 or 2)
    const int q0 = p * BQ + (wave & 3) * 32;

    // this group's stream: sub-tiles [first, first + ng)
    const int N = n * R;
    const int N0 = (N + 1) / 2, N1 = N - N0;
    const int first = grp ? N0 : 0;
    const int ng = grp ? N1 : N0;

    E e;
    e.init(smem, lane, prm.scale_log2);
    e.load_q(prm.q + (int64_t)b * prm.qs[0] + (int64_t)(q0 + l32) * prm.qs[1] + (int64_t)h * prm.qs[2]);

    int* lidx = (int*)(smem + 2 * GROUP_LDS);
    for (int i = tid; i < ldc; i += 512) lidx[i] = stage_entry<PARTIAL>(irow[i], nkv, block_kv, prm.kv_valid);
    e.q_ready();

    // sub-tile j of this stream -> CSR entry and 64-key offset inside it
    // CSR tile of sub-tile j, and its valid keys within this sub-tile
    auto tile_of = [&](int j) { return entry_tile<PARTIAL>(__builtin_amdgcn_readfirstlane(lidx[(first + j) / R])); };
    auto valid = [&](int t) { return t >= 0 && t < nkv; };
    auto keys_of = [&](int j) {
        if constexpr (!PARTIAL) return valid(tile_of(j)) ? SUB : 0;
        const int nv = entry_keys<PARTIAL>(__builtin_amdgcn_readfirstlane(lidx[(first + j) / R]), block_kv) -
                       ((first + j) % R) * SUB;
        return nv < 0 ? 0 : (nv > SUB ? SUB : nv);
    };
    const char* kbase = (const char*)(prm.k + (int64_t)b * prm.ks[0] + (int64_t)h * prm.ks[2]);
    const char* vbase = (const char*)(prm.v + (int64_t)b * prm.vs[0] + (int64_t)h * prm.vs[2]);
    const int kt_bytes = (int)(prm.ks[1] * 2), vt_bytes = (int)(prm.vs[1] * 2);  // K and V row strides
    using F = TileFetch<SUB, D, 4>;
    const int fw = wave & 3;  // this wave's index among the waves fetching its stream's tiles
    const F fetch(smem, fw, lane, kt_bytes, vt_bytes);
    // sub-tile j of this stream in CSR tile t; out-of-range tiles load tile 0
    // and contribute nothing
    auto sub_ptr = [&](const char* base, int row_bytes, int t, int j) {
        const int64_t row0 = (int64_t)(valid(t) ? t : 0) * block_kv + ((first + j) % R) * SUB;
        return uniform_ptr(base + row0 * row_bytes);
    };
    auto tile_ptr = [&](const char* base, int row_bytes, int j) { return sub_ptr(base, row_bytes, tile_of(j), j); };
    const int gbase = grp * GROUP_LDS;
    auto kbuf = [&](int j) { return gbase + (j & 1) * G::TILE; };
    auto vbuf = [&](int j) { return gbase + (2 + (j & 1)) * G::TILE; };
    // The loads of M_j (K_{j+1} if it exists, then V_j) are spread over the
    // MFMA phase, one 1 KB block per hook.
    auto loads = [&](int j) {
        const char* kt = tile_ptr(kbase, kt_bytes, j + 1);
        const char* vt = tile_ptr(vbase, vt_bytes, j);
        const int kd = kbuf(j + 1), vd = vbuf(j);
        return [=, &fetch](int i) {
            if (i < F::BPW) fetch.block(kd, kt, kt_bytes, false, i);
            else fetch.block(vd, vt, vt_bytes, true, i - F::BPW);
        };
    };
    auto v_loads = [&](int j) {
        const char* vt = tile_ptr(vbase, vt_bytes, j);
        const int vd = vbuf(j);
        return [=, &fetch](int i) { fetch.block(vd, vt, vt_bytes, true, i); };
    };
    auto pv = [&](int j) { e.template mfma_phase<true, false>(vbuf(j), 0); };
    auto softmax = [&](int j) {
        const int nv = keys_of(j);
        if (PARTIAL && nv > 0 && nv < SUB) e.mask_keys(nv);
        e.softmax(nv > 0);
    };

    // Every wave passes the same number of barriers: group 0 uses 2*N0 + 2,
    // group 1 (one phase later) 2*N1 + 3; the shorter one pads at the end.
    const int total = max(2 * N0 + 2, 2 * N1 + 3);
    int nbar = 0;
    auto bar = [&]() {
        lds_barrier();
        ++nbar;
    };

    // K_0 of this stream, addressed straight from the CSR row in memory; the
    // barrier then publishes both it and the staged row.
    if (ng > 0) {
        const int t0 = __builtin_amdgcn_readfirstlane(irow[first / R]);
        fetch.all(kbuf(0), sub_ptr(kbase, kt_bytes, t0, 0), kt_bytes, false);
    }
    wait_global_loads();
    bar();
    if (grp == 1) bar();
    // M_j fetches K_{j+1} and V_j; the last M_j has no K to fetch and is peeled
    // so that the loop body has no branch per load.
    if (ng > 0) {
        if (ng > 1) e.template mfma_phase<false, true, 2 * F::BPW>(0, kbuf(0), loads(0));   // M_0
        else e.template mfma_phase<false, true, F::BPW>(0, kbuf(0), v_loads(0));
        bar();
        softmax(0);                              // V_0
        wait_global_loads();
        bar();
        for (int j = 1; j < ng - 1; ++j) {
            e.template mfma_phase<true, true, 2 * F::BPW>(vbuf(j - 1), kbuf(j), loads(j));  // M_j
            bar();
            softmax(j);                          // V_j
            wait_global_loads();
            bar();
        }
        if (ng > 1) {
            e.template mfma_phase<true, true, F::BPW>(vbuf(ng - 2), kbuf(ng - 1), v_loads(ng - 1));
            bar();
            softmax(ng - 1);
            wait_global_loads();
            bar();
        }
        pv(ng - 1);                              // M_n
        bar();
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
hipError_t launch_2s(const FwdParams& p, hipStream_t stream) {
    if (p.kv_valid) hipLaunchKernelGGL((vsa_fwd_2s_kernel<D, true>), dim3(p.n_work), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((vsa_fwd_2s_kernel<D, false>), dim3(p.n_work), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_2s(int block_kv, int head_dim, const FwdParams& p, hipStream_t stream) {
    if (p.n_work <= 0) return hipSuccess;
    if (block_kv != 64 && block_kv != 128) return hipErrorInvalidValue;
    if (head_dim == 128) return launch_2s<128>(p, stream);
    if (head_dim == 64) return launch_2s<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace vsa
