// Fused block-sparse attention forward for 256-row query tiles on gfx950:
// eight waves in two groups that alternate between matrix-core work and
// softmax work ("ping-pong").
//
// What is computed: FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// ref_masked_sdpa_fp32 (per-wave arithmetic in wave_engine.h).
//
// Schedule. Waves 0-3 (group 0) own query rows [0,128) of the tile, waves
// 4-7 (group 1) rows [128,256); each SIMD runs one wave of each group. Work
// per KV tile j is split into an MFMA phase M_j (O += V_{j-1} P_{j-1}, then
// S_j = K_j Q^T) and a softmax phase V_j (S_j into bf16 P_j, rescale of O).
// Group 1 runs one phase behind group 0, and every phase ends in a workgroup
// barrier, so while one wave of a SIMD issues MFMAs the other issues exp/FMA
// work:
//
//     phase:    0     1     2     3     4   ...  2n    2n+1
//     group 0:  M_0   V_0   M_1   V_1   M_2 ...  M_n
//     group 1:  -     M_0   V_0   M_1   V_1 ...  V_n-1 M_n
//
// Both groups read the same K and V tiles, double-buffered in LDS and fetched
// with direct-to-LDS 16-byte loads: K_{j+1} by group 1 and V_j by group 0,
// both issued at the start of phase 2j and waited for at the end of phase
// 2j+1, two phases before first use.
#include "device_common.h"
#include "vsa_internal.h"
#include "wave_engine.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kIdxCap = 8192;  // CSR row entries staged in LDS (>= the largest idx_ld)

template <int BKV, int D, bool PARTIAL>
__global__ __launch_bounds__(512) void vsa_fwd_pp_kernel(FwdParams prm) {
    using E = WaveEngine<BKV, D>;
    using G = TileGeom<BKV, D>;
    constexpr int BQ = 256;
    constexpr int LDS_TILES = 4 * G::TILE;  // K[2], V[2]
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TILES + kIdxCap * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int grp = wave >> 2;
    const int l32 = lane & 31;

    const int wi = xcd_contiguous_block();
    if (wi >= prm.n_work) return;
    // With split lists, workgroup wi serves part wi % splits of work entry
    // wi / splits and takes the list entries part, part + splits, ...
    const int SP = prm.splits;
    const int slot = SP == 1 ? wi : wi / SP;
    const int part = wi - slot * SP;
    const int item = prm.work ? prm.work[slot] : slot;
    if (item < 0 || item >= prm.n_items) return;

    const int p = item % prm.nq;
    const int bh = item / prm.nq;
    const int h = bh % prm.H;
    const int b = bh / prm.H;
    const int S = prm.S;
    const int64_t tok_stride = (int64_t)prm.H * D;  // o is contiguous
    // The count, the CSR row, Q and the first K tile are all fetched at once
    // (none of these loads waits for another; the row is read up to its
    // allocated length ld, so it does not need the count first).
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld + part;
    const int ldp = prm.ld > part ? (prm.ld - part + SP - 1) / SP : 0;  // this part's slots of the row
    const int ldc = ldp < kIdxCap ? ldp : kIdxCap;
    // (a part with no slot reads a valid address and ignores the value)
    const int first_raw = __builtin_amdgcn_readfirstlane(*(ldp > 0 ? irow : prm.idx));
    const int first_tile = ldp > 0 ? first_raw : -1;
    int n = prm.cnt[item];
    const int nkv = prm.nkv;
    const int q0 = p * BQ + wave * 32;
    auto valid = [&](int t) { return t >= 0 && t < nkv; };
    const char* kbase = (const char*)(prm.k + (int64_t)b * prm.ks[0] + (int64_t)h * prm.ks[2]);
    const char* vbase = (const char*)(prm.v + (int64_t)b * prm.vs[0] + (int64_t)h * prm.vs[2]);
    const int kt_bytes = (int)(prm.ks[1] * 2), vt_bytes = (int)(prm.vs[1] * 2);  // K and V row strides
    using F = TileFetch<BKV, D, 4>;  // a tile is fetched by the four waves of one group
    const F fetch(smem, wave & 3, lane, kt_bytes, vt_bytes);
    // out-of-range entries load tile 0 and contribute nothing
    auto tile_at = [&](const char* base, int row_bytes, int t) {
        return uniform_ptr(base + (int64_t)(valid(t) ? t : 0) * BKV * row_bytes);
    };

    E e;
    e.init(smem, lane, prm.scale_log2);
    e.load_q(prm.q + (int64_t)b * prm.qs[0] + (int64_t)(q0 + l32) * prm.qs[1] + (int64_t)h * prm.qs[2]);

    // Stage this tile's CSR row in LDS: list entries are then read with
    // uniform LDS loads, which do not wait on outstanding global loads.
    int* lidx = (int*)(smem + LDS_TILES);
    for (int i = tid; i < ldc; i += 512) lidx[i] = stage_entry<PARTIAL>(irow[(int64_t)i * SP], nkv, BKV, prm.kv_valid);
    e.q_ready();
    // group 1 fetches K_0 (buffer 0 is free); an empty row fetches it too
    if (grp == 1) fetch.all(0, tile_at(kbase, kt_bytes, first_tile), kt_bytes, false);
    n = n < 0 ? 0 : (n > prm.ld ? prm.ld : n);
    n = n > part ? (n - part + SP - 1) / SP : 0;  // this part's entries
    n = n > ldc ? ldc : n;
    wait_global_loads();
    lds_barrier();

    // Tile index and valid key count of list entry j (uniform; -1 / 0 when
    // the entry is out of range).
    auto tile_of = [&](int j) { return entry_tile<PARTIAL>(__builtin_amdgcn_readfirstlane(lidx[j])); };
    auto keys_of = [&](int j) { return entry_keys<PARTIAL>(__builtin_amdgcn_readfirstlane(lidx[j]), BKV); };
    auto tile_ptr = [&](const char* base, int row_bytes, int j) { return tile_at(base, row_bytes, tile_of(j)); };
    // LDS byte offsets of the K and V buffers used for list entry j
    auto kbuf = [](int j) { return (j & 1) * G::TILE; };
    auto vbuf = [](int j) { return (2 + (j & 1)) * G::TILE; };
    // Tile loads are spread over a phase (one 1 KB block per hook) so that
    // the eight waves' loads do not queue up at the start of the phase.
    auto v_loads = [&](int j) {
        const char* tile = tile_ptr(vbase, vt_bytes, j);
        return [=, &fetch](int i) { fetch.block(vbuf(j), tile, vt_bytes, true, i); };
    };
    auto k_loads = [&](int j) {
        const char* tile = tile_ptr(kbase, kt_bytes, j);
        return [=, &fetch](int i) { fetch.block(kbuf(j), tile, kt_bytes, false, i); };
    };
    auto pv = [&](int j) { e.template mfma_phase<true, false>(vbuf(j), 0); };
    // softmax of list entry j, masking a partial tile's missing keys first
    auto softmax_of = [&](int j) {
        const int nv = keys_of(j);
        if (PARTIAL && nv > 0 && nv < BKV) e.mask_keys(nv);
        return nv > 0;
    };
    auto softmax = [&](int j) { e.softmax(softmax_of(j)); };

    // Both groups pass 2(n+1) barriers after the prologue. Each group has its own loop so that
    // S (live from M_j to V_j) and P (live from V_j to M_{j+1}) never both
    // cross a loop back-edge, and the first and last tiles are peeled so the
    // steady-state MFMA phase (PV_{j-1} then QK_j) is one basic block.
    if (grp == 0) {
        if (n > 0) {
            e.template mfma_phase<false, true, F::BPW>(0, kbuf(0), v_loads(0));                // M_0
            lds_barrier();
            softmax(0);                          // V_0
            wait_global_loads();
            lds_barrier();
            for (int j = 1; j < n; ++j) {
                e.template mfma_phase<true, true, F::BPW>(vbuf(j - 1), kbuf(j), v_loads(j));   // M_j
                lds_barrier();
                softmax(j);                      // V_j
                wait_global_loads();
                lds_barrier();
            }
            pv(n - 1);                           // M_n
        }
        lds_barrier();
        lds_barrier();
    } else {
        if (n > 0) {
            if (n > 1) fetch.all(kbuf(1), tile_ptr(kbase, kt_bytes, 1), kt_bytes, false);
            lds_barrier();
            e.template mfma_phase<false, true>(0, kbuf(0));                                    // M_0
            wait_global_loads();
            lds_barrier();
            // the last tile has no K_{j+1} to fetch: peeled, so the loop body has no branch per load
            for (int j = 1; j < n - 1; ++j) {
                e.template softmax<F::BPW>(softmax_of(j - 1), k_loads(j + 1));  // V_{j-1}
                lds_barrier();
                e.template mfma_phase<true, true>(vbuf(j - 1), kbuf(j));            // M_j
                wait_global_loads();
                lds_barrier();
            }
            if (n > 1) {
                softmax(n - 2);                  // V_{n-2}
                lds_barrier();
                e.template mfma_phase<true, true>(vbuf(n - 2), kbuf(n - 1));        // M_{n-1}
                wait_global_loads();
                lds_barrier();
            }
            softmax(n - 1);                      // V_{n-1}
            lds_barrier();
            pv(n - 1);                           // M_n
            lds_barrier();
        } else {
            lds_barrier();
            lds_barrier();
        }
    }

    if (SP > 1) {
        // Split list: every part publishes its rows (device-scope stores,
        // then a wait for them), and the last part of the item to arrive
        // merges all parts in part order, so the result does not depend on
        // which one that is, and writes O and LSE. Nothing waits on another
        // workgroup, and no fence invalidates the caches that the other
        // workgroups are reading K and V through.
        constexpr int64_t WORDS = (int64_t)E::STATE_WORDS * 64;
        e.template export_state<true>(prm.ws_partial + ((int64_t)wi * 8 + wave) * WORDS);
        wait_global_loads();  // the stores have reached the coherence point
        lds_barrier();
        int* flag = (int*)smem;  // the tile buffers are free now
        if (tid == 0) {
            const int last = __hip_atomic_fetch_add(prm.ws_counter + item, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT) == SP - 1;
            if (last) __hip_atomic_store(prm.ws_counter + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *flag = last;
        }
        lds_barrier();
        if (__builtin_amdgcn_readfirstlane(*flag) == 0) return;
        const float* parts = prm.ws_partial + ((int64_t)slot * SP * 8 + wave) * WORDS;
        e.template import_state<true>(parts);
        for (int q = 1; q < SP; ++q) e.template merge_state<true>(parts + (int64_t)q * 8 * WORDS);
    }
    e.store(prm.o + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D,
            prm.lse + ((int64_t)b * prm.H + h) * S + q0 + l32);
}

template <int BKV, int D>
hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
    if (p.kv_valid) hipLaunchKernelGGL((vsa_fwd_pp_kernel<BKV, D, true>), dim3(p.n_work), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((vsa_fwd_pp_kernel<BKV, D, false>), dim3(p.n_work), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_pp(int block_kv, int head_dim, const FwdParams& p, hipStream_t stream) {
    if (p.n_work <= 0) return hipSuccess;
    if (block_kv == 128 && head_dim == 128) return launch_pp<128, 128>(p, stream);
    if (block_kv == 128 && head_dim == 64) return launch_pp<128, 64>(p, stream);
    if (block_kv == 64 && head_dim == 128) return launch_pp<64, 128>(p, stream);
    if (block_kv == 64 && head_dim == 64) return launch_pp<64, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace vsa
