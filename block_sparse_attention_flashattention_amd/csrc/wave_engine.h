// Per-wave machinery of the phase-alternating ("ping-pong") forward kernels
// on gfx950: one wave owns 32 query rows and accumulates
//     S^T = K Q^T   and   O^T += V^T P^T
// with v_mfma_f32_32x32x16_bf16 over KV tiles staged in LDS.
//
// Layout facts used throughout (32x32x16 MFMA, wave64; l = lane):
//  * A operand: lane l supplies row (l % 32), 8 consecutive k slots of half
//    (l / 32); B operand: lane l supplies column (l % 32), same k slots.
//  * Result: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column
//    (l % 32).
// With S^T (keys x queries) each lane therefore holds 16 scores of query row
// (l % 32) per 32-key block, so the row max/sum is an in-lane reduction plus
// one exchange between the half-waves, and the bf16-packed probabilities are
// directly the B operand of O^T = V^T P^T, whose accumulator is again indexed
// by query column, making the per-row rescale lane-uniform.
//
// Online softmax in base 2 with scale*log2(e) folded into one FMA, a running
// row max and row sum, and a correction of O that is skipped while the max
// grows by at most kRescaleThreshold (page "BlackwellMultiHeadLatentAttention
// ForwardFP8", softmax / correction / skip_correction_threshold; what is
// computed: FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// ref_masked_sdpa_fp32).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.h"

namespace vsa {
namespace dev {

// 16-byte-chunk XOR swizzles (involutions: LDS position <-> global chunk).
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

// Swizzle for tiles read both ways (16-byte row reads of 16 consecutive rows
// and transposing reads of 8 rows x 4 chunks), as the backward pass reads Q,
// dO and K: conflict-free for both, since it is injective on 16 consecutive
// rows (same-parity rows for NC = 8) and sends the rows of a transposing read
// to distinct 4-chunk groups.
template <int NC>
__device__ __forceinline__ int swz_d(int row) {
    if constexpr (NC == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// LDS tile layouts: K (row reads), V (transposing reads), D (both).
enum TileLayout : int { kLayoutK = 0, kLayoutV = 1, kLayoutD = 2 };

// Scheduling pins for MFMA steps [S0, S1) of one MFMA phase of NS steps:
// per step its MFMA followed by the LDS reads of the step RING ahead; with
// PRE, first the reads of the first RING steps (the ring fill). The pins of
// one scheduling region must describe exactly that region's reads and MFMAs.
// Masks: 0x100 LDS read, 0x008 MFMA.
template <bool PV, bool QK>
constexpr int step_reads(int st) {
    return (PV && (!QK || (st & 1) == 0)) ? 2 : 1;  // PV: two 8-byte transposing reads
}
template <bool PV, bool QK, int RING, int NS>
constexpr int ring_fill_reads() {
    int r = 0;
    for (int st = 0; st < RING && st < NS; ++st) r += step_reads<PV, QK>(st);
    return r;
}
template <bool PV, bool QK, int RING, int NS, int S0, int S1, bool PRE>
__device__ __forceinline__ void pin_mfma_steps() {
    if constexpr (PRE) __builtin_amdgcn_sched_group_barrier(0x100, ring_fill_reads<PV, QK, RING, NS>(), 0);
    if constexpr (S0 < S1) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (S0 + RING < NS) {
            constexpr int r = step_reads<PV, QK>(S0 + RING);
            __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
        }
        pin_mfma_steps<PV, QK, RING, NS, S0 + 1, S1, false>();
    }
}

// K/V tile geometry in LDS: BKV rows of D bf16, row-major, 16-byte chunks
// swizzled with swz_k (K) or swz_v (V).
template <int BKV, int D>
struct TileGeom {
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int NC = D / 8;               // 16-byte chunks per row
    static constexpr int TILE = BKV * ROW_BYTES;   // bytes per tile
    static constexpr int ROWS_PER_KB = 1024 / ROW_BYTES;
    static_assert(NC == 8 || NC == 16, "head_dim 64 or 128");
    static_assert(TILE % 1024 == 0, "tiles are fetched in 1 KB blocks");
};

// Tile fetch: the tile is split into 1 KB blocks shared out over the WPF
// waves that fetch it (wave gw takes blocks [gw*BPW, (gw+1)*BPW)); each block
// is one direct-to-LDS 16-byte-per-lane load from a uniform row base plus a
// 32-bit per-lane offset. `tile` points at row 0 of the tile for this head;
// consecutive rows are tok_bytes apart (v_tok_bytes for the V layout).
//
// A lane's offset within its block depends on the block only through the
// swizzle, which repeats every KP blocks for K and is the same for every
// block for V; the KP + 1 offsets are computed once, so issuing a block costs
// no vector ALU work (the row base and the LDS address are scalar).
template <int BKV, int D, int WPF>
struct TileFetch {
    using G = TileGeom<BKV, D>;
    static constexpr int BPW = G::TILE / 1024 / WPF;  // blocks per wave
    static_assert(BPW >= 1 && G::TILE % (1024 * WPF) == 0, "tile must split evenly over the waves");
    // swizzle period in blocks: swz_k depends on row % 16 (NC=16) or row % 16 / 2 (NC=8)
    static constexpr int KP = 16 / G::ROWS_PER_KB;

    int gw;
    uint32_t lds0;  // LDS byte address of the tile buffers' base
    uint32_t koff[KP];
    uint32_t doff[KP];
    uint32_t voff;

    __device__ __forceinline__ TileFetch(const char* smem, int gw_, int lane, int tok_bytes, int v_tok_bytes = -1)
        : gw(gw_), lds0(lds_addr(smem)) {
        if (v_tok_bytes < 0) v_tok_bytes = tok_bytes;
        const int rl = lane / G::NC, pos = lane % G::NC;
#pragma unroll
        for (int k = 0; k < KP; ++k) {
            const int row = ((gw * BPW + k) % KP) * G::ROWS_PER_KB + rl;
            koff[k] = (uint32_t)(rl * tok_bytes + ((pos ^ swz_k<G::NC>(row)) << 4));
            doff[k] = (uint32_t)(rl * tok_bytes + ((pos ^ swz_d<G::NC>(row)) << 4));
        }
        voff = (uint32_t)(rl * v_tok_bytes + ((pos ^ swz_v<G::NC>(rl)) << 4));
    }
    // block i (0 <= i < BPW) of this wave's share; dst is the tile buffer's
    // byte offset from the base; layout is a TileLayout
    __device__ __forceinline__ void block(int dst, const char* tile, int tok_bytes, int layout, int i) const {
        const int blk = gw * BPW + i;
        const char* src = tile + (int64_t)(blk * G::ROWS_PER_KB) * tok_bytes;
        const uint32_t off = layout == kLayoutV ? voff : (layout == kLayoutD ? doff[i % KP] : koff[i % KP]);
        lds_dma16(src, off, lds0 + (uint32_t)(dst + blk * 1024));
    }
    // this wave's whole share
    __device__ __forceinline__ void all(int dst, const char* tile, int tok_bytes, int layout) const {
#pragma unroll
        for (int i = 0; i < BPW; ++i) block(dst, tile, tok_bytes, layout, i);
    }
};

// Hook that issues nothing (phases without interleaved loads).
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

template <int BKV, int D>
struct WaveEngine {
    using G = TileGeom<BKV, D>;
    static constexpr int DC = D / 16;    // QK^T k-steps
    static constexpr int NB = BKV / 32;  // 32-key blocks of S^T
    static constexpr int DB = D / 32;    // 32-wide d blocks of O^T
    static constexpr int KC = BKV / 16;  // PV k-steps
    // operand prefetch distance (MFMA steps): deeper for 32-key sub-tiles,
    // whose MFMA phases are short enough for the fill to show
    static constexpr int RING = BKV <= 32 ? 6 : 4;
    // fp32 words per lane exchanged when two waves merge their partial rows
    static constexpr int STATE_WORDS = DB * 16 + 2;

    char* smem;
    int lane, l32, hi;
    float scale_log2;
    bf16x8 qreg[DC];
    f32x16 oacc[DB];
    f32x16 sacc[NB];
    bf16x8 pk[KC];
    int koff[DC];  // K operand: row l32, chunk 2c+hi (+ nb*32 rows)
    int voff[DB];  // V transposing read of d-block db (+ (g*16 + r*8) rows)
    float m_run, l_run;

    __device__ __forceinline__ void init(char* smem_, int lane_, float scale_log2_) {
        smem = smem_;
        lane = lane_;
        l32 = lane & 31;
        hi = lane >> 5;
        scale_log2 = scale_log2_;
        // Within one operand loop the swizzle depends on the lane only (row
        // offsets of a 32-key block or a 16-key chunk are multiples of the
        // swizzle period), so every read is buffer + per-lane offset + constant.
#pragma unroll
        for (int c = 0; c < DC; ++c) koff[c] = l32 * G::ROW_BYTES + (((2 * c + hi) ^ swz_k<G::NC>(l32)) << 4);
        // Transposing read: lane j of a 16-lane group addresses row
        // (kv0 + j/4), columns d0 + 4*(j%4) .. +3; lane i then receives column
        // d0 + i of rows kv0 .. kv0+3. Rows kv0 = g*16 + r*8 + 4*(l/32) give
        // the k slots the S^T accumulator holds for half-wave l/32.
        {
            const int grp16 = lane >> 4, i = lane & 15;
            const int row = (grp16 >> 1) * 4 + (i >> 2);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = db * 32 + (grp16 & 1) * 16 + 4 * (i & 3);
                voff[db] = row * G::ROW_BYTES + (((d >> 3) ^ swz_v<G::NC>(row)) << 4) + (d & 7) * 2;
            }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[nb] = f32x16{};
#pragma unroll
        for (int g = 0; g < KC; ++g) pk[g] = bf16x8{};
        m_run = -__builtin_inff();
        l_run = 0.0f;
    }

    // Q^T operand: qrow points at d = 0 of this lane's query row (l32 of the
    // wave's 32 rows) for this head.
    __device__ __forceinline__ void load_q(const uint16_t* qrow) {
        const uint16_t* qp = qrow + hi * 8;
#pragma unroll
        for (int c = 0; c < DC; ++c) qreg[c] = *(const bf16x8*)(qp + c * 16);
    }

    // Makes the compiler wait for the Q loads here. Its wait counting does not
    // see the direct-to-LDS loads issued through inline asm, so a Q register
    // first used after some of them would get a wait that also covers those
    // tile loads; consuming Q before the first tile load avoids that.
    __device__ __forceinline__ void q_ready() const {
#pragma unroll
        for (int c = 0; c < DC; ++c) asm volatile("" ::"v"(qreg[c]));
    }

    // MFMA phase: PV steps (O^T += V^T P^T over the V tile at LDS offset vb)
    // and/or QK steps (S^T = K Q^T over the K tile at kb). When both run they
    // alternate 1:1 so consecutive MFMAs use independent accumulators; each
    // step's A operand is fetched RING steps ahead into a register ring.
    // hook(0..NH-1) is called at evenly spaced step boundaries (hook 0 before
    // the first MFMA) to spread other work, such as tile loads, over the phase.
    template <bool PV, bool QK, int NH = 0, typename Hook = NoHook>
    __device__ __forceinline__ void mfma_phase(int vb, int kb, Hook&& hook = Hook{}) {
        constexpr int NPV = PV ? DB * KC : 0;
        constexpr int NQK = QK ? NB * DC : 0;
        constexpr int NS = NPV + NQK;
        static_assert(NH <= NS, "at most one hook per MFMA step");
        // step -> (is_pv, item); PV item i = (g = i / DB, db = i % DB), QK
        // item i = (c = i / NB, nb = i % NB)
        auto is_pv = [](int st) { return PV && (!QK || (st & 1) == 0); };
        auto item = [](int st) { return (PV && QK) ? (st >> 1) : st; };
        auto load = [&](int st) -> bf16x8 {
            const int i = item(st);
            if (is_pv(st)) {
                const int g = i / DB, db = i % DB;
                const char* base = smem + vb + voff[db] + (g * 16) * G::ROW_BYTES;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)base);
                const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + 8 * G::ROW_BYTES));
                return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                const int c = i / NB, nb = i % NB;
                return *(const bf16x8*)(smem + kb + koff[c] + nb * 32 * G::ROW_BYTES);
            }
        };
        // Raised issue priority for the phase: where another wave on the
        // SIMD runs its softmax, this wave's MFMAs and operand reads go first.
        __builtin_amdgcn_s_setprio(1);
        if constexpr (QK) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) sacc[nb] = f32x16{};
        }
        bf16x8 ring[RING];
#pragma unroll
        for (int st = 0; st < RING && st < NS; ++st) ring[st] = load(st);
        // steps [S0, S1)
        auto steps = [&]<int S0, int S1, bool PRE>() {
#pragma unroll
            for (int st = S0; st < S1; ++st) {
                const bf16x8 a = ring[st % RING];
                if (st + RING < NS) ring[st % RING] = load(st + RING);
                const int i = item(st);
                if (is_pv(st)) {
                    const int g = i / DB, db = i % DB;
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[g], oacc[db], 0, 0, 0);
                } else {
                    const int c = i / NB, nb = i % NB;
                    sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc[nb], 0, 0, 0);
                }
            }
            pin_mfma_steps<PV, QK, RING, NS, S0, S1, PRE>();
        };
        if constexpr (NH == 0) {
            steps.template operator()<0, NS, true>();
        } else {
            // the ring fill forms its own scheduling region before hook 0
            pin_mfma_steps<PV, QK, RING, NS, 0, 0, true>();
            [&]<int... H>(std::integer_sequence<int, H...>) {
                ((hook(H), steps.template operator()<H * NS / NH, (H + 1) * NS / NH, false>()), ...);
            }(std::make_integer_sequence<int, NH>{});
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // Partial tile: scores of keys at or past nv (0 < nv < BKV) become -inf,
    // so those keys take no part in the softmax.
    __device__ __forceinline__ void mask_keys(int nv) {
        // key of register r in 32-key block nb: nb*32 + 8*(r/4) + 4*hi + r%4.
        // Compared as (compile-time part) >= nv - 4*hi, so that no per-lane
        // key table is formed (it would be hoisted out of the KV loop).
        const int lim = nv - 4 * hi;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (nb * 32 + 8 * (r >> 2) + (r & 3) >= lim) sacc[nb][r] = -__builtin_inff();
    }

    // Softmax of the scores in sacc into pk (bf16), with the lazy rescale of
    // O and l. A tile with no valid key (ok == false: a list entry out of
    // range, or a partial tile with no valid key) contributes nothing.
    // hook(0..NH-1) is spread over the exponentials (and is called on
    // skipped tiles too).
    template <int NH = 0, typename Hook = NoHook>
    __device__ __forceinline__ void softmax(bool ok, Hook&& hook = Hook{}) {
        constexpr int CHUNKS = NB * 2;  // 8-score blocks per lane
        if (!ok) {
#pragma unroll
            for (int g = 0; g < KC; ++g) pk[g] = bf16x8{};
#pragma unroll
            for (int i = 0; i < NH; ++i) hook(i);
            return;
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
        mx = halfwave_max(mx);
        const float m_new = fmaxf(m_run, mx * scale_log2);
        if (__any(m_new > m_run + kRescaleThreshold)) {
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        float lsum = 0.0f;
#pragma unroll
        for (int ch = 0; ch < CHUNKS; ++ch) {
            // hooks h with floor(h * CHUNKS / NH) == ch run before chunk ch
            if constexpr (NH > 0) {
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    if (h * CHUNKS / NH == ch) hook(h);
            }
            const int nb = ch >> 1, half = ch & 1;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(sacc[nb][half * 8 + 2 * e], scale_log2, -m_run));
                const float p1 = fast_exp2(fmaf(sacc[nb][half * 8 + 2 * e + 1], scale_log2, -m_run));
                lsum += p0 + p1;
                w[e] = pack_bf16x2(p0, p1);
            }
            pk[ch] = __builtin_bit_cast(bf16x8, w);
        }
        l_run += lsum;
    }

    // Partial-row exchange between two waves that own the same rows (same
    // lane -> row/column mapping): words[e * 64 + lane], e < STATE_WORDS.
    // DEV: between workgroups through global memory, with device-scope
    // stores and loads (written through to and read from the device's
    // coherence point), so that no cache-wide fence is needed; the writer
    // waits for its stores before it signals.
    template <bool DEV>
    static __device__ __forceinline__ void put(float* p, float v) {
        if constexpr (DEV) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else *p = v;
    }
    template <bool DEV>
    static __device__ __forceinline__ float get(const float* p) {
        if constexpr (DEV) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else return *p;
    }
    template <bool DEV = false>
    __device__ __forceinline__ void export_state(float* words) const {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) put<DEV>(&words[(db * 16 + r) * 64 + lane], oacc[db][r]);
        put<DEV>(&words[(DB * 16) * 64 + lane], m_run);
        put<DEV>(&words[(DB * 16 + 1) * 64 + lane], l_run);
    }
    // Replace this wave's state by an exported one.
    template <bool DEV = false>
    __device__ __forceinline__ void import_state(const float* words) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = get<DEV>(&words[(db * 16 + r) * 64 + lane]);
        m_run = get<DEV>(&words[(DB * 16) * 64 + lane]);
        l_run = get<DEV>(&words[(DB * 16 + 1) * 64 + lane]);
    }
    // Merge another wave's partial state (exported above) into this one:
    // both sums are rescaled to the larger of the two (stale) maxima.
    template <bool DEV = false>
    __device__ __forceinline__ void merge_state(const float* words) {
        const float m1 = get<DEV>(&words[(DB * 16) * 64 + lane]);
        const float l1 = get<DEV>(&words[(DB * 16 + 1) * 64 + lane]);
        const float m = fmaxf(m_run, m1);
        const float a0 = m == -__builtin_inff() ? 0.0f : fast_exp2(m_run - m);
        const float a1 = m == -__builtin_inff() ? 0.0f : fast_exp2(m1 - m);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + get<DEV>(&words[(db * 16 + r) * 64 + lane]) * a1;
        l_run = l_run * a0 + l1 * a1;
        m_run = m;
    }

    // Epilogue: O = O^T / l (bf16, RNE) into orow (d = 0 of this lane's query
    // row), LSE = (m + log2 l) ln 2 into *lse_row (lanes of half-wave 0).
    // A row with no selected key gives O = 0 and LSE = -inf.
    __device__ __forceinline__ void store(uint16_t* orow, float* lse_row) const {
        const float l_tot = halfwave_sum(l_run);
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int jg = 0; jg < 4; ++jg) {
                const int d0 = db * 32 + jg * 8 + hi * 4;
                u32x2 w;
                w[0] = pack_bf16x2(oacc[db][jg * 4 + 0] * inv, oacc[db][jg * 4 + 1] * inv);
                w[1] = pack_bf16x2(oacc[db][jg * 4 + 2] * inv, oacc[db][jg * 4 + 3] * inv);
                *(u32x2*)(orow + d0) = w;
            }
        }
        if (hi == 0) *lse_row = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
};

}  // namespace dev
}  // namespace vsa
