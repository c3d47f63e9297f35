// Fused block-sparse attention forward for 64- and 128-row query tiles on
// gfx950 with independent waves: every wave owns 32 query rows and runs its
// own MFMA / softmax sequence; the matrix core is kept busy by the second
// wave on each SIMD, which belongs to another workgroup.
//
// What is computed: FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// ref_masked_sdpa_fp32 (per-wave arithmetic in wave_engine.h: online softmax
// in base 2 with the lazily skipped correction of page
// "BlackwellMultiHeadLatentAttentionForwardFP8").
//
// Schedule. The tile's KV list is walked in sub-tiles of SUB keys (64 for
// 128-row tiles, 32 for 64-row tiles). Step j of a wave is the MFMA phase
// O += V_{j-1} P_{j-1}, S_j = K_j Q^T, then the softmax of S_j; the step's
// direct-to-LDS loads (K_{j+1}, V_j, a share of each per wave) are spread
// over the MFMA phase, and the step ends by waiting for them and a workgroup
// barrier. K and V are double-buffered, so a workgroup needs 4*SUB*D*2 bytes
// of LDS plus its staged list (sized at launch): two 128-row or four 64-row
// workgroups fit a compute unit, and every wave stays within 256 registers,
// so each SIMD runs two waves that are not in lock step.
#include "device_common.h"
#include "vsa_internal.h"
#include "wave_engine.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kIdxCapIw = 8192;  // CSR row entries staged in LDS (at most)

template <int BQ>
constexpr int iw_sub() { return BQ == 64 ? 32 : 64; }
template <int BQ, int D>
constexpr int iw_tiles_bytes() { return 4 * iw_sub<BQ>() * D * 2; }

template <int BQ, int D, bool PARTIAL>
__global__ __launch_bounds__(BQ * 2, 2) void vsa_fwd_iw_kernel(FwdParams prm) {
    constexpr int NW = BQ / 32;
    constexpr int SUB = iw_sub<BQ>();
    using E = WaveEngine<SUB, D>;
    using G = TileGeom<SUB, D>;
    using F = TileFetch<SUB, D, NW>;  // every wave fetches a share of each sub-tile
    static_assert(4 * G::TILE == iw_tiles_bytes<BQ, D>(), "launch sizes the LDS from iw_tiles_bytes");
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // K[2], V[2], then the list

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // the count, the CSR row, Q and the first K sub-tile are fetched at once
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld + part;
    const int ldp = prm.ld > part ? (prm.ld - part + SP - 1) / SP : 0;  // this part's slots of the row
    const int ldc = ldp < kIdxCapIw ? ldp : kIdxCapIw;
    // (a part with no slot reads a valid address and ignores the value)
    const int first_raw = __builtin_amdgcn_readfirstlane(*(ldp > 0 ? irow : prm.idx));
    const int first_tile = ldp > 0 ? first_raw : -1;
    int n = prm.cnt[item];
    const int nkv = prm.nkv;
    const int block_kv = prm.block_kv;
    const int R = block_kv / SUB;  // sub-tiles per CSR tile
    const int q0 = p * BQ + wave * 32;
    auto valid = [&](int t) { return t >= 0 && t < nkv; };
    const char* kbase = (const char*)(prm.k + (int64_t)b * prm.ks[0] + (int64_t)h * prm.ks[2]);
    const char* vbase = (const char*)(prm.v + (int64_t)b * prm.vs[0] + (int64_t)h * prm.vs[2]);
    const int kt_bytes = (int)(prm.ks[1] * 2), vt_bytes = (int)(prm.vs[1] * 2);  // K and V row strides
    const F fetch(smem, wave, lane, kt_bytes, vt_bytes);
    // sub-tile r of CSR tile t; out-of-range tiles load tile 0 and contribute nothing
    auto sub_ptr = [&](const char* base, int row_bytes, int t, int r) {
        return uniform_ptr(base + ((int64_t)(valid(t) ? t : 0) * block_kv + r * SUB) * row_bytes);
    };

    E e;
    e.init(smem, lane, prm.scale_log2);
    e.load_q(prm.q + (int64_t)b * prm.qs[0] + (int64_t)(q0 + l32) * prm.qs[1] + (int64_t)h * prm.qs[2]);

    int* lidx = (int*)(smem + 4 * G::TILE);
    for (int i = tid; i < ldc; i += BQ * 2)
        lidx[i] = stage_entry<PARTIAL>(irow[(int64_t)i * SP], nkv, block_kv, prm.kv_valid);
    e.q_ready();
    fetch.all(0, sub_ptr(kbase, kt_bytes, first_tile, 0), kt_bytes, kLayoutK);
    n = n < 0 ? 0 : (n > prm.ld ? prm.ld : n);
    n = n > part ? (n - part + SP - 1) / SP : 0;  // this part's entries
    n = n > ldc ? ldc : n;
    const int N = n * R;
    wait_global_loads();
    lds_barrier();

    auto entry = [&](int j) { return __builtin_amdgcn_readfirstlane(lidx[j / R]); };
    auto src = [&](const char* base, int row_bytes, int j) {
        return sub_ptr(base, row_bytes, entry_tile<PARTIAL>(entry(j)), j % R);
    };
    auto keys = [&](int j) {
        const int nv = entry_keys<PARTIAL>(entry(j), block_kv) - (j % R) * SUB;
        return nv < 0 ? 0 : (nv > SUB ? SUB : nv);
    };
    auto kbuf = [](int j) { return (j & 1) * G::TILE; };
    auto vbuf = [](int j) { return (2 + (j & 1)) * G::TILE; };
    // loads of step j: K_{j+1} (if dk) in hooks 0..BPW-1, V_j in hooks BPW..2*BPW-1
    auto loads = [&](int j, bool dk) {
        const char* kt = dk ? src(kbase, kt_bytes, j + 1) : nullptr;
        const char* vt = src(vbase, vt_bytes, j);
        const int kd = kbuf(j + 1), vd = vbuf(j);
        return [=, &fetch](int i) {
            if (i < F::BPW) {
                if (dk) fetch.block(kd, kt, kt_bytes, kLayoutK, i);
            } else {
                fetch.block(vd, vt, vt_bytes, kLayoutV, i - F::BPW);
            }
        };
    };
    auto softmax = [&](int j) __attribute__((always_inline)) {
        const int nv = keys(j);
        if (PARTIAL && nv > 0 && nv < SUB) e.mask_keys(nv);
        e.softmax(nv > 0);
    };

    if (N > 0) {
        e.template mfma_phase<false, true, 2 * F::BPW>(0, kbuf(0), loads(0, N > 1));  // S_0
        softmax(0);
        wait_global_loads();
        lds_barrier();
        int j = 1;
        for (; j + 1 < N; ++j) {
            e.template mfma_phase<true, true, 2 * F::BPW>(vbuf(j - 1), kbuf(j), loads(j, true));
            softmax(j);
            wait_global_loads();
            lds_barrier();
        }
        if (j < N) {  // the last sub-tile: no K to fetch
            e.template mfma_phase<true, true, 2 * F::BPW>(vbuf(j - 1), kbuf(j), loads(j, false));
            softmax(j);
            wait_global_loads();
            lds_barrier();
        }
        e.template mfma_phase<true, false>(vbuf(N - 1), 0);  // O += V_{N-1} P_{N-1}
    }
    if (SP > 1) {
        // Split list: every part publishes its rows (device-scope stores,
        // then a wait for them), and the last part of the item to arrive
        // merges all parts in part order, so the result does not depend on
        // which one that is, and writes O and LSE. Nothing waits on another
        // workgroup, and no fence invalidates the caches that the other
        // workgroups are reading K and V through.
        constexpr int64_t WORDS = (int64_t)E::STATE_WORDS * 64;
        e.template export_state<true>(prm.ws_partial + ((int64_t)wi * NW + wave) * WORDS);
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
        const float* parts = prm.ws_partial + ((int64_t)slot * SP * NW + wave) * WORDS;
        e.template import_state<true>(parts);
        for (int q = 1; q < SP; ++q) e.template merge_state<true>(parts + (int64_t)q * NW * WORDS);
    }
    e.store(prm.o + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D,
            prm.lse + ((int64_t)b * prm.H + h) * S + q0 + l32);
}

template <int BQ, int D>
hipError_t launch_iw_d(const FwdParams& p, hipStream_t stream) {
    const int lds = iw_tiles_bytes<BQ, D>() + 4 * (p.ld < kIdxCapIw ? p.ld : kIdxCapIw);
    auto kernel = p.kv_valid ? vsa_fwd_iw_kernel<BQ, D, true> : vsa_fwd_iw_kernel<BQ, D, false>;
    if (lds > 65536) {
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kernel), lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(p.n_work), dim3(BQ * 2), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_iw(int block_q, int head_dim, const FwdParams& p, hipStream_t stream) {
    if (p.n_work <= 0) return hipSuccess;
    if (block_q == 128) return head_dim == 128 ? launch_iw_d<128, 128>(p, stream) : launch_iw_d<128, 64>(p, stream);
    if (block_q == 64) return head_dim == 128 ? launch_iw_d<64, 128>(p, stream) : launch_iw_d<64, 64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace vsa
