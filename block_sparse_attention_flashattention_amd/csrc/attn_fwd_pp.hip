// Fused block-sparse attention forward for 256-row query tiles on gfx950:
// eight waves in two groups that alternate between matrix-core work and
// softmax work ("ping-pong").
//
// What is computed is the same as in attn_fwd.hip (FastVideo page "[perf]
// Add fine-grained FA4 VSA kernels", ref_masked_sdpa_fp32; base-2 online
// softmax with a lazily rescaled accumulator as in the softmax/correction
// split of page "BlackwellMultiHeadLatentAttentionForwardFP8").
//
// Schedule. Waves 0-3 (group 0) own query rows [0,128) of the tile, waves
// 4-7 (group 1) rows [128,256); each SIMD runs one wave of each group. Work
// per KV tile j is split into an MFMA phase M_j (O += V_{j-1} P_{j-1}, then
// S_j = K_j Q^T) and a VALU phase V_j (softmax of S_j into bf16 P_j and the
// accumulator rescale). Group 1 runs one phase behind group 0, and every
// phase ends in a workgroup barrier, so while one wave of a SIMD issues MFMAs
// the other issues exp/FMA work:
//
//     phase:    0     1     2     3     4   ...  2n    2n+1
//     group 0:  M_0   V_0   M_1   V_1   M_2 ...  M_n
//     group 1:  -     M_0   V_0   M_1   V_1 ...  V_n-1 M_n
//
// K and V tiles are double-buffered in LDS and fetched with direct-to-LDS
// 16-byte loads (global_load_lds_dwordx4): K_{j+1} by group 1 and V_j by
// group 0, both issued at the start of phase 2j and waited for at the end of
// phase 2j+1, two phases before first use. Both tiles are stored
// row-major with 16-byte chunks XOR-swizzled on the global side. K rows feed
// the A operand of S^T = K Q^T with ds_read_b128; V feeds the A operand of
// O^T = V^T P^T through the transposing read ds_read_b64_tr_b16: with lane j
// of a 16-lane group addressing row (kv0 + j/4), columns d0 + 4*(j%4) .. +3,
// lane i receives column d0 + i of rows kv0 .. kv0+3. The V swizzle spreads
// the 8 rows x 64 bytes of one such read over all 64 banks.
#include <type_traits>

#include "device_common.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using namespace dev;

template <int BKV, int D>
struct PP {
    static constexpr int BQ = 256;
    static constexpr int NT = 512;
    static constexpr int ROW_BYTES = D * 2;        // bytes per K or V row in LDS
    static constexpr int NC = D / 8;               // 16-byte chunks per row
    static constexpr int TILE = BKV * ROW_BYTES;   // bytes per K (or V) tile
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
    static constexpr int BLOCKS_PER_WAVE = TILE / 1024 / 4;   // 1 KB loads per wave of a group
    static constexpr int DC = D / 16;              // QK^T k-steps
    static constexpr int NB = BKV / 32;            // 32-key blocks of S^T
    static constexpr int DB = D / 32;              // 32-wide d blocks of O^T
    static constexpr int KC = BKV / 16;            // PV k-steps
    static constexpr int LDS_TILES = 4 * TILE;     // K[2], V[2]
    static constexpr int IDX_CAP = 8192;           // CSR row entries staged in LDS
    static constexpr int LDS_BYTES = LDS_TILES + IDX_CAP * 4;
    static_assert(NC == 8 || NC == 16, "head_dim 64 or 128");
    static_assert(BLOCKS_PER_WAVE >= 1 && TILE % 4096 == 0, "tile must split over four waves");
};

// 16-byte-chunk swizzles (XOR, an involution: LDS position <-> global chunk).
template <int NC>
__device__ __forceinline__ int swz_k(int row) {
    // 16 consecutive rows of one chunk column land in 16 distinct bank groups
    if constexpr (NC == 16) return row & 15;
    else return (row >> 1) & 7;
}
template <int NC>
__device__ __forceinline__ int swz_v(int row) {
    // the 8 rows x 4 chunks of one transposing read cover every bank group twice
    if constexpr (NC == 16) return (row & 3) << 2;
    else return ((row >> 1) & 1) << 2;
}

// Scheduling pins for one MFMA phase (see mfma_phase in the kernel): the LDS
// reads of the first RING steps, then per step its MFMA followed by the reads
// of the step RING ahead. Masks: 0x100 LDS read, 0x008 MFMA.
template <bool PV, bool QK>
constexpr int step_reads(int st) {
    return (PV && (!QK || (st & 1) == 0)) ? 2 : 1;  // PV: two 8-byte transposing reads
}
template <bool PV, bool QK, int RING, int NS, int ST = 0>
__device__ __forceinline__ void pin_mfma_schedule() {
    if constexpr (ST == 0) {
        constexpr int pre = step_reads<PV, QK>(0) + step_reads<PV, QK>(1) + step_reads<PV, QK>(2) +
                            step_reads<PV, QK>(3);
        static_assert(RING == 4, "prefetch count assumes a ring of 4");
        __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
    }
    if constexpr (ST < NS) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (ST + RING < NS) {
            constexpr int r = step_reads<PV, QK>(ST + RING);
            __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
        }
        pin_mfma_schedule<PV, QK, RING, NS, ST + 1>();
    }
}

template <int BKV, int D>
__global__ __launch_bounds__(512) void vsa_fwd_pp_kernel(FwdParams prm) {
    using C = PP<BKV, D>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int grp = wave >> 2;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
    // give each XCD a contiguous run of the work list instead, so that the
    // tiles it works on concurrently share K/V tiles in its own L2.
    int wi;
    {
        const int nwg = gridDim.x, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
        const int per = nwg / 8, rem = nwg % 8;
        wi = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    }
    if (wi >= prm.n_work) return;
    const int item = prm.work ? prm.work[wi] : wi;
    if (item < 0 || item >= prm.n_items) return;

    const int p = item % prm.nq;
    const int bh = item / prm.nq;
    const int h = bh % prm.H;
    const int b = bh / prm.H;
    const int S = prm.S;
    const int64_t tok_stride = (int64_t)prm.H * D;
    int n = prm.cnt[item];
    n = n < 0 ? 0 : (n > prm.ld ? prm.ld : n);
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld;
    const int nkv = prm.nkv;

    // Q^T operand: lane holds query row l32 of this wave, d in [c*16 + hi*8, +8)
    const int q0 = p * C::BQ + wave * 32;
    bf16x8 qreg[C::DC];
    {
        const uint16_t* qp = prm.q + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D + hi * 8;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) qreg[c] = *(const bf16x8*)(qp + c * 16);
    }

    const uint16_t* kbase = prm.k + (int64_t)b * S * tok_stride + (int64_t)h * D;
    const uint16_t* vbase = prm.v + (int64_t)b * S * tok_stride + (int64_t)h * D;
    // LDS byte offsets of the K and V buffers used for list entry j
    auto kbuf = [](int j) { return (j & 1) * C::TILE; };
    auto vbuf = [](int j) { return (2 + (j & 1)) * C::TILE; };

    // Stage this tile's CSR row in LDS: list entries are then read with
    // uniform LDS loads, which do not wait on outstanding global loads.
    int* lidx = (int*)(smem + C::LDS_TILES);
    n = n > C::IDX_CAP ? C::IDX_CAP : n;
    for (int e = tid; e < n; e += C::NT) lidx[e] = irow[e];
    lds_barrier();

    // Tile index of list entry j (uniform); out-of-range entries load tile 0
    // and contribute nothing.
    auto tile_of = [&](int j) { return __builtin_amdgcn_readfirstlane(lidx[j]); };
    auto valid = [&](int t) { return t >= 0 && t < nkv; };

    // One wave's share of a tile fetched by its group: BLOCKS_PER_WAVE 1 KB
    // direct-to-LDS loads, each from a uniform row base plus a 32-bit
    // per-lane offset.
    const int tok_bytes = (int)(tok_stride * 2);
    auto issue_tile = [&](const uint16_t* base, int dst, int t, bool v_layout) {
        const char* tile = (const char*)base + (int64_t)(valid(t) ? t : 0) * BKV * tok_bytes;
        const int gw = wave & 3;
        const int rl = lane / C::NC, pos = lane % C::NC;
#pragma unroll
        for (int i = 0; i < C::BLOCKS_PER_WAVE; ++i) {
            const int blk = gw * C::BLOCKS_PER_WAVE + i;
            const int row = blk * C::ROWS_PER_KB + rl;
            const int c = pos ^ (v_layout ? swz_v<C::NC>(row) : swz_k<C::NC>(row));
            const char* src = tile + (int64_t)(blk * C::ROWS_PER_KB) * tok_bytes;
            const uint32_t off = (uint32_t)(rl * tok_bytes + c * 16);
            lds_dma16(src, off, lds_addr(smem + dst + blk * 1024));
        }
    };

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
    f32x16 sacc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) sacc[nb] = f32x16{};
    bf16x8 pk[C::KC];
#pragma unroll
    for (int g = 0; g < C::KC; ++g) pk[g] = bf16x8{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    // Per-lane LDS byte offsets of the MFMA A operands. Within one operand
    // loop the swizzle depends on the lane only (row offsets of a 32-key block
    // or a 16-key chunk are multiples of the swizzle period), so every read is
    // "buffer + per-lane offset + compile-time constant".
    int koff[C::DC];   // K row l32, chunk 2c+hi; + nb*32 rows
#pragma unroll
    for (int c = 0; c < C::DC; ++c) koff[c] = l32 * C::ROW_BYTES + (((2 * c + hi) ^ swz_k<C::NC>(l32)) << 4);
    int voff[C::DB];   // transposing read of d-block db; + (g*16 + r*8) rows
    {
        const int G = lane >> 4, i = lane & 15;
        const int row = (G >> 1) * 4 + (i >> 2);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
            const int d = db * 32 + (G & 1) * 16 + 4 * (i & 3);
            voff[db] = row * C::ROW_BYTES + (((d >> 3) ^ swz_v<C::NC>(row)) << 4) + (d & 7) * 2;
        }
    }

    // MFMA phase. Steps are O^T += V^T P^T products (PV, over the V tile at
    // LDS offset vb) and S^T = K Q^T products (QK, over the K tile at kb);
    // when both run they alternate 1:1 so consecutive MFMAs use independent
    // accumulators. Each step's A operand (two transposing 8-byte reads for
    // PV, one 16-byte read for QK) is fetched RING steps ahead into a
    // register ring, so LDS latency is hidden behind the MFMAs in flight.
    constexpr int RING = 4;
    auto mfma_phase = [&](auto pv_on, auto qk_on, int vb, int kb) {
        constexpr bool PV = decltype(pv_on)::value;
        constexpr bool QK = decltype(qk_on)::value;
        constexpr int NPV = PV ? C::DB * C::KC : 0;
        constexpr int NQK = QK ? C::NB * C::DC : 0;
        constexpr int NS = NPV + NQK;
        // step s -> (is_pv, item); PV item i = (g = i / DB, db = i % DB),
        // QK item i = (c = i / NB, nb = i % NB)
        auto is_pv = [](int st) { return PV && (!QK || (st & 1) == 0); };
        auto item = [](int st) { return (PV && QK) ? (st >> 1) : st; };
        auto load = [&](int st) -> bf16x8 {
            const int i = item(st);
            if (is_pv(st)) {
                const int g = i / C::DB, db = i % C::DB;
                const char* base = smem + vb + voff[db] + (g * 16) * C::ROW_BYTES;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
                const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * C::ROW_BYTES));
                return __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                const int c = i / C::NB, nb = i % C::NB;
                return *(const bf16x8*)(smem + kb + koff[c] + nb * 32 * C::ROW_BYTES);
            }
        };
        if constexpr (QK) {
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) sacc[nb] = f32x16{};
        }
        bf16x8 ring[RING];
#pragma unroll
        for (int st = 0; st < RING && st < NS; ++st) ring[st] = load(st);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const bf16x8 a = ring[st % RING];
            if (st + RING < NS) ring[st % RING] = load(st + RING);
            const int i = item(st);
            if (is_pv(st)) {
                const int g = i / C::DB, db = i % C::DB;
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[g], oacc[db], 0, 0, 0);
            } else {
                const int c = i / C::NB, nb = i % C::NB;
                sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc[nb], 0, 0, 0);
            }
        }
        pin_mfma_schedule<PV, QK, RING, NS>();
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    auto pv = [&](int vb) { mfma_phase(yes{}, no{}, vb, 0); };
    auto qk = [&](int kb) { mfma_phase(no{}, yes{}, 0, kb); };
    auto pv_qk = [&](int vb, int kb) { mfma_phase(yes{}, yes{}, vb, kb); };

    // softmax of S_j into pk (bf16), with the lazy rescale of O and l
    auto softmax = [&](bool ok) {
        if (!ok) {
#pragma unroll
            for (int g = 0; g < C::KC; ++g) pk[g] = bf16x8{};
            return;
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
        mx = halfwave_max(mx);
        const float m_new = fmaxf(m_run, mx * prm.scale_log2);
        if (__any(m_new > m_run + kRescaleThreshold)) {
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
        }
        float lsum = 0.0f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = fast_exp2(fmaf(sacc[nb][half * 8 + 2 * e], prm.scale_log2, -m_run));
                    const float p1 = fast_exp2(fmaf(sacc[nb][half * 8 + 2 * e + 1], prm.scale_log2, -m_run));
                    lsum += p0 + p1;
                    w[e] = pack_bf16x2(p0, p1);
                }
                pk[nb * 2 + half] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l_run += lsum;
    };

    // prologue: group 1 fetches K_0
    if (grp == 1 && n > 0) {
        issue_tile(kbase, kbuf(0), tile_of(0), false);
        wait_global_loads();
    }
    lds_barrier();

    // Both groups pass 2(n+1) barriers. Each group has its own loop so that
    // S (live from M_j to V_j) and P (live from V_j to M_{j+1}) never both
    // cross a loop back-edge, and the first and last tiles are peeled so the
    // steady-state MFMA phase (PV_{j-1} then QK_j) is one basic block whose
    // two independent accumulator sets the scheduler can interleave.
    // Tile fetches: group 1 issues K_{j+1} at the start of phase 2j (its
    // softmax phase), group 0 issues V_j at the start of phase 2j (its MFMA
    // phase); both wait at the end of phase 2j+1, so every load has two
    // phases to land before its first use in phase 2j+2.
    if (grp == 0) {
        if (n > 0) {
            issue_tile(vbase, vbuf(0), tile_of(0), true);
            qk(kbuf(0));                                   // M_0
            lds_barrier();
            softmax(valid(tile_of(0)));                    // V_0
            wait_global_loads();
            lds_barrier();
            for (int j = 1; j < n; ++j) {
                issue_tile(vbase, vbuf(j), tile_of(j), true);
                pv_qk(vbuf(j - 1), kbuf(j));               // M_j
                lds_barrier();
                softmax(valid(tile_of(j)));                // V_j
                wait_global_loads();
                lds_barrier();
            }
            pv(vbuf(n - 1));                               // M_n
        }
        lds_barrier();
        lds_barrier();
    } else {
        if (n > 0) {
            if (n > 1) issue_tile(kbase, kbuf(1), tile_of(1), false);
            lds_barrier();
            qk(kbuf(0));                                   // M_0
            wait_global_loads();
            lds_barrier();
            for (int j = 1; j < n; ++j) {
                if (j + 1 < n) issue_tile(kbase, kbuf(j + 1), tile_of(j + 1), false);
                softmax(valid(tile_of(j - 1)));            // V_{j-1}
                lds_barrier();
                pv_qk(vbuf(j - 1), kbuf(j));               // M_j
                wait_global_loads();
                lds_barrier();
            }
            softmax(valid(tile_of(n - 1)));                // V_{n-1}
            lds_barrier();
            pv(vbuf(n - 1));                               // M_n
            lds_barrier();
        } else {
            lds_barrier();
            lds_barrier();
        }
    }

    // epilogue: O = O^T / l (bf16, RNE), LSE = (m + log2 l) ln 2
    const float l_tot = halfwave_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* orow = prm.o + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
            const int d0 = db * 32 + jg * 8 + hi * 4;
            u32x2 w;
            w[0] = pack_bf16x2(oacc[db][jg * 4 + 0] * inv, oacc[db][jg * 4 + 1] * inv);
            w[1] = pack_bf16x2(oacc[db][jg * 4 + 2] * inv, oacc[db][jg * 4 + 3] * inv);
            *(u32x2*)(orow + d0) = w;
        }
    }
    if (hi == 0) {
        const float lse = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        prm.lse[((int64_t)b * prm.H + h) * S + q0 + l32] = lse;
    }
}

template <int BKV, int D>
hipError_t launch_pp(const FwdParams& p, hipStream_t stream) {
    using C = PP<BKV, D>;
    hipLaunchKernelGGL((vsa_fwd_pp_kernel<BKV, D>), dim3(p.n_work), dim3(C::NT), 0, stream, p);
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
