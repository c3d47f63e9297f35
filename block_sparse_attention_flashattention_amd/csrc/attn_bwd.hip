// Block-sparse attention backward pass on gfx950: dQ, dK and dV.
//
// What is computed: the gradients of FastVideo page "[perf] Add fine-grained
// FA4 VSA kernels", ref_masked_sdpa_fp32 (the masked softmax attention the
// forward computes). With P the masked row softmax of scale * Q K^T
// (recomputed from the forward's LSE), O the forward output and dO given:
//     D_i  = dO_i . O_i
//     dS   = P * (dO V^T - D)          (elementwise, per row i)
//     dV   = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K
//
// Schedule (no atomics, deterministic): dK and dV come from one workgroup per
// KV tile that walks the query tiles selecting it (the Q-direction lists of
// the page's FA4 block_sparsity.py backward) and accumulates in registers;
// dQ comes from one workgroup per query tile that walks the forward list, as
// the split-dQ form of the FlashAttention backward does. Both recompute P.
// The dQ kernel runs first: it also forms D and LSE * log2(e) for its rows
// (it holds dO already), which the dK/dV kernel then reads.
//
// Operand layouts follow the forward (wave_engine.h): 32x32x16 bf16 MFMA,
// lane l / register r of a result holds row 8*(r/4) + 4*(l/32) + r%4 and
// column l%32. A result used as a B operand keeps that row order in its k
// slots, and the A operand that meets it is read with transposing LDS reads
// whose rows follow the same order. Tiles read both by rows and transposed
// (Q and dO for dK/dV, K for dQ) use the swz_d swizzle.
#include "device_common.h"
#include "vsa_internal.h"
#include "wave_engine.h"

namespace vsa {
namespace {

using namespace dev;

constexpr int kIdxCapBwd = 8192;  // list entries staged in LDS (at most)

// Keys per dQ step: 32 for 64-row tiles, so that four of those two-wave
// workgroups fit a compute unit's LDS; 64 otherwise.
template <int BQ>
constexpr int dq_sub() { return BQ == 64 ? 32 : 64; }
// LDS of the two kernels: two stages of streamed tiles, then the staged list
// (its length is known at launch only, so the LDS is sized then).
template <int BQ, int D>
constexpr int dq_stage_bytes() { return 2 * dq_sub<BQ>() * D * 2; }
constexpr int kDkvQs = 32;  // query rows per dK/dV step
template <int D>
constexpr int dkv_stage_bytes() { return 2 * kDkvQs * D * 2 + 2 * kDkvQs * 4; }

// Per-lane LDS offsets for the operand reads of one tile layout.
template <int D>
struct OperandOffsets {
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int NC = D / 8;
    static constexpr int DC = D / 16;
    static constexpr int DB = D / 32;
    int row[DC];   // 16-byte row read of row l%32, chunk 2c + hi (add 32*ROW_BYTES per 32-row block)
    int trl[DB];   // transposing read, rows 4*hi + (0..3) of a 16-row group, d block db
    int trh[DB];   // the same 8 rows further down
    template <int LAYOUT>
    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, hi = lane >> 5;
        auto swz = [](int r) {
            if constexpr (LAYOUT == kLayoutD) return swz_d<NC>(r);
            else if constexpr (LAYOUT == kLayoutV) return swz_v<NC>(r);
            else return swz_k<NC>(r);
        };
#pragma unroll
        for (int c = 0; c < DC; ++c) row[c] = l32 * ROW_BYTES + (((2 * c + hi) ^ swz(l32)) << 4);
        const int grp16 = lane >> 4, i = lane & 15;
        const int r0 = (grp16 >> 1) * 4 + (i >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + (grp16 & 1) * 16 + 4 * (i & 3);
            trl[db] = r0 * ROW_BYTES + (((d >> 3) ^ swz(r0)) << 4) + (d & 7) * 2;
            trh[db] = (r0 + 8) * ROW_BYTES + (((d >> 3) ^ swz(r0 + 8)) << 4) + (d & 7) * 2;
        }
    }
};

// A operand of 16 k slots taken from rows g*16 + {4*hi + 0..3, 8 + 4*hi + 0..3}
// of the tile at byte offset base, d block db (transposing reads).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* smem, int base, const OperandOffsets<D>& off, int db, int g) {
    const char* p = smem + base + g * 16 * OperandOffsets<D>::ROW_BYTES;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + off.trl[db]));
    const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + off.trh[db]));
    return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

// OperandOffsets in one register per kind, for kernels short of registers.
// The row-read offsets of chunk pairs c and the transposing-read offsets of
// d blocks db differ from the first ones only in chunk bits (c << 5 and
// db << 6: the chunk index is 2c ^ hi, and the swizzles and row terms leave
// those bits alone), so each is formed by an XOR onto the tile base, which
// must be a multiple of 256 bytes.
template <int D>
struct CompactOffsets {
    static constexpr int ROW_BYTES = D * 2;
    int row0, trl0, trh0;
    template <int LAYOUT>
    __device__ __forceinline__ void init(int lane) {
        OperandOffsets<D> full;
        full.template init<LAYOUT>(lane);
        row0 = full.row[0];
        trl0 = full.trl[0];
        trh0 = full.trh[0];
    }
    // byte offset of the row read of chunk pair c in the tile at `base`
    __device__ __forceinline__ int row(int base, int c) const { return (base + row0) ^ (c << 5); }
};

template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* smem, int base, const CompactOffsets<D>& off, int db, int g) {
    const char* p = smem + g * 16 * CompactOffsets<D>::ROW_BYTES;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + ((base + off.trl0) ^ (db << 6))));
    const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + ((base + off.trh0) ^ (db << 6))));
    return __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
}

// B operand registers of 32 token rows: lane l holds row l%32, d = 16c + 8*hi + (0..7).
template <int DC>
__device__ __forceinline__ void load_rows(bf16x8 (&reg)[DC], const uint16_t* row_ptr, int hi) {
    const uint16_t* p = row_ptr + hi * 8;
#pragma unroll
    for (int c = 0; c < DC; ++c) reg[c] = *(const bf16x8*)(p + c * 16);
}

// Store a transposed accumulator (rows d, column = this lane's token row) as
// bf16 times mul into the token row at dst (d = 0 of the row).
template <int DB>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16 (&acc)[DB], float mul, int hi) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
            const int d0 = db * 32 + jg * 8 + hi * 4;
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][jg * 4 + 0] * mul, acc[db][jg * 4 + 1] * mul);
            w[1] = pack_bf16x2(acc[db][jg * 4 + 2] * mul, acc[db][jg * 4 + 3] * mul);
            *(u32x2*)(dst + d0) = w;
        }
    }
}

// Split lists: every part of a work item publishes its accumulators (NA
// 16-float blocks per lane) with device-scope stores, waits for them, then
// bumps the item's counter; the last part to arrive returns true with the sum
// of all parts, taken in part order so that the result does not depend on
// which part that is, and resets the counter. The others return false. mine:
// this wave's slot; parts: part 0's slot for this wave, part q at q * stride.
// smem is free LDS (the tile stages, after the last step).
template <int NA>
__device__ __forceinline__ bool merge_parts(f32x16 (&acc)[NA], float* mine, const float* parts, int64_t stride,
                                            int SP, int32_t* counter, char* smem, int tid) {
    const int lane = tid & 63;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            __hip_atomic_store(&mine[(a * 16 + r) * 64 + lane], acc[a][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_global_loads();  // the stores have reached the coherence point
    lds_barrier();
    int* flag = (int*)smem;
    if (tid == 0) {
        const int last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == SP - 1;
        if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    lds_barrier();
    if (__builtin_amdgcn_readfirstlane(*flag) == 0) return false;
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[a][r] = __hip_atomic_load(&parts[(a * 16 + r) * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int q = 1; q < SP; ++q) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[a][r] += __hip_atomic_load(&parts[q * stride + (a * 16 + r) * 64 + lane], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
}

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    // element strides between batches, tokens and heads of q, k, v and dout
    // (row r of head h in batch b starts at b*s[0] + r*s[1] + h*s[2]); o, dq,
    // dk, dv and the per-row terms are contiguous
    int64_t qs[3], ks[3], vs[3], ds[3];
    int32_t strided;  // any of them not the contiguous [B, S, H, D] layout
    const float* lse;         // forward LSE [B,H,S]
    float* aux;               // [2][B*H*S]: D, then LSE*log2(e); written by the dQ kernel
    const int32_t* idx;       // forward CSR [B,H,nq,ld]
    const int32_t* cnt;
    const int32_t* qidx;      // Q-direction CSR [B,H,nkv,q_ld]
    const int32_t* qcnt;
    const int32_t* kv_valid;  // [nkv] or null
    const int32_t* work_q;    // dQ work list (flat (b*H + h)*nq + p)
    const int32_t* work_kv;   // dK/dV work list (flat (b*H + h)*nkv + n)
    uint16_t *dq, *dk, *dv;
    int32_t n_items_q, n_items_kv;
    // split lists (1 = off): workgroup wi serves part wi % splits of work
    // entry wi / splits; per-item counters and partial accumulators
    int32_t splits_q, splits_kv;
    int32_t *ws_counter_q, *ws_counter_kv;
    float *ws_q, *ws_kv;
    int32_t S, H, nq, nkv, ld, q_ld, block_q, block_kv;
    int32_t n_rows;           // B*H*S
    float scale, scale_log2;
};

// ----------------------------------------------------------------------- dQ
// One workgroup per query tile of BQ rows, BQ/32 waves of 32 rows. The KV
// list is walked in 64-key steps (32 for 64-row tiles); per step K (swz_d:
// row reads for S^T = K Q^T, transposing reads for dQ^T += K^T dS^T) and V
// (row reads for dP^T = V dO^T) are fetched for the next step while this one
// is computed. Every variant stays within 256 registers per wave, so each
// SIMD runs two waves (of one workgroup at 256 rows, of two or four smaller
// ones otherwise).
template <int BQ, int D, bool PARTIAL, bool SPLIT>
__global__ __launch_bounds__(BQ * 2, 2) void vsa_bwd_dq_kernel(BwdParams prm) {
    constexpr int NW = BQ / 32;
    constexpr int SUB = dq_sub<BQ>();
    using G = TileGeom<SUB, D>;
    using F = TileFetch<SUB, D, NW>;
    using OO = OperandOffsets<D>;
    constexpr int DC = D / 16, DB = D / 32, NB = SUB / 32, KC = SUB / 16;
    constexpr int STAGE = 2 * G::TILE;  // K, V
    static_assert(STAGE == dq_stage_bytes<BQ, D>(), "launch sizes the LDS from dq_stage_bytes");
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // 2 stages, then the list

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = xcd_contiguous_block();
    const int SP = SPLIT ? prm.splits_q : 1;  // built apart so the unsplit loop keeps its registers
    if (wi >= prm.n_items_q * SP) return;
    const int slot = SP == 1 ? wi : wi / SP;
    const int part = wi - slot * SP;  // takes list entries part, part + SP, ...
    const int item = prm.work_q ? prm.work_q[slot] : slot;
    if (item < 0 || item >= prm.n_items_q) return;
    const int p = item % prm.nq, bh = item / prm.nq, h = bh % prm.H, b = bh / prm.H;
    const int S = prm.S, nkv = prm.nkv, block_kv = prm.block_kv;
    const int64_t tok_stride = (int64_t)prm.H * D;  // o and dq are contiguous
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld + part;
    const int ldp = prm.ld > part ? (prm.ld - part + SP - 1) / SP : 0;  // this part's slots of the row
    const int ldc = ldp < kIdxCapBwd ? ldp : kIdxCapBwd;
    int n = prm.cnt[item];
    n = n < 0 ? 0 : (n > prm.ld ? prm.ld : n);
    n = n > part ? (n - part + SP - 1) / SP : 0;  // this part's entries
    n = n > ldc ? ldc : n;
    const int R = block_kv / SUB;
    const int steps = n * R;
    const int q0 = p * BQ + wave * 32;
    const int64_t qrow = ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D;  // o, dq
    const int64_t qin = (int64_t)b * prm.qs[0] + (int64_t)(q0 + l32) * prm.qs[1] + (int64_t)h * prm.qs[2];
    const int64_t doin = (int64_t)b * prm.ds[0] + (int64_t)(q0 + l32) * prm.ds[1] + (int64_t)h * prm.ds[2];

    bf16x8 qreg[DC], doreg[DC];
    load_rows<DC>(qreg, prm.q + qin, hi);
    load_rows<DC>(doreg, prm.dout + doin, hi);
    const int64_t arow = (int64_t)bh * S + q0 + l32;
    // D_i = dO_i . O_i (this lane's half of the row, then both half-waves) and
    // LSE_i * log2(e) (+inf for a row without keys, so that exp2(s - lse2) = 0);
    // part 0 also writes both to aux for the dK/dV kernel, launched after this one
    float dval, lse2;
    {
        bf16x8 oreg[DC];
        load_rows<DC>(oreg, prm.o + qrow, hi);
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)oreg[c][e], (float)doreg[c][e], acc);
        dval = halfwave_sum(acc);
        const float l = prm.lse[arow];
        lse2 = l == -__builtin_inff() ? __builtin_inff() : l * 1.4426950408889634f;
        if (part == 0 && hi == 0) {
            prm.aux[arow] = dval;
            prm.aux[(int64_t)prm.n_rows + arow] = lse2;
        }
    }

    int* lidx = (int*)(smem + 2 * STAGE);
    for (int i = tid; i < ldc; i += BQ * 2)
        lidx[i] = stage_entry<PARTIAL>(irow[(int64_t)i * SP], nkv, block_kv, prm.kv_valid);
    // consume every loaded register before the first tile load (the compiler's
    // wait counting does not see the inline-asm tile loads)
#pragma unroll
    for (int c = 0; c < DC; ++c) asm volatile("" ::"v"(qreg[c]), "v"(doreg[c]));
    asm volatile("" ::"v"(dval), "v"(lse2));
    wait_global_loads();
    lds_barrier();

    OO ko, vo;
    ko.template init<kLayoutD>(lane);
    vo.template init<kLayoutK>(lane);
    const int kt_bytes = (int)(prm.ks[1] * 2), vt_bytes = (int)(prm.vs[1] * 2);  // K and V row strides
    const F kfetch(smem, wave, lane, kt_bytes), vfetch(smem, wave, lane, vt_bytes);
    const char* kbase = (const char*)(prm.k + (int64_t)b * prm.ks[0] + (int64_t)h * prm.ks[2]);
    const char* vbase = (const char*)(prm.v + (int64_t)b * prm.vs[0] + (int64_t)h * prm.vs[2]);
    auto entry = [&](int j) { return __builtin_amdgcn_readfirstlane(lidx[j / R]); };
    auto step_ptr = [&](const char* base, int row_bytes, int j) {
        const int t = entry_tile<PARTIAL>(entry(j));
        const int64_t row0 = (int64_t)(t >= 0 && t < nkv ? t : 0) * block_kv + (j % R) * SUB;
        return uniform_ptr(base + row0 * row_bytes);
    };
    auto fetch_step = [&](int j) {
        const int st = (j & 1) * STAGE;
        kfetch.all(st, step_ptr(kbase, kt_bytes, j), kt_bytes, kLayoutD);
        vfetch.all(st + G::TILE, step_ptr(vbase, vt_bytes, j), vt_bytes, kLayoutK);
    };

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    if (steps > 0) fetch_step(0);
    for (int j = 0; j < steps; ++j) {
        wait_global_loads();
        lds_barrier();  // step j's tiles are in LDS; step j-1's buffers are free
        if (j + 1 < steps) fetch_step(j + 1);
        const int e = entry(j);
        const int t = entry_tile<PARTIAL>(e);
        int nv = (t >= 0 && t < nkv) ? entry_keys<PARTIAL>(e, block_kv) - (j % R) * SUB : 0;
        nv = nv < 0 ? 0 : (nv > SUB ? SUB : nv);
        if (nv == 0) continue;  // uniform: every wave skips the same step
        const int kb = (j & 1) * STAGE, vb = kb + G::TILE;
        // MFMA blocks at raised issue priority, the exp / dS work at normal
        // priority: the other workgroup's wave on the SIMD fills the gaps
        __builtin_amdgcn_s_setprio(1);
        f32x16 s[NB], dp[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            s[nb] = f32x16{};
            dp[nb] = f32x16{};
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const bf16x8 ka = *(const bf16x8*)(smem + kb + ko.row[c] + nb * 32 * OO::ROW_BYTES);
                s[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], s[nb], 0, 0, 0);
                const bf16x8 va = *(const bf16x8*)(smem + vb + vo.row[c] + nb * 32 * OO::ROW_BYTES);
                dp[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, doreg[c], dp[nb], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // dS^T = P^T (dP^T - D), P^T = exp2(S^T * scale*log2e - LSE*log2e); keys at or past nv do not exist
        bf16x8 pk[KC];
#pragma unroll
        for (int ch = 0; ch < KC; ++ch) {
            const int nb = ch >> 1, half = ch & 1;
            u32x4 w;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float ds[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int r = half * 8 + 2 * e2 + u;
                    const int key = nb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const float pr = fast_exp2(fmaf(s[nb][r], prm.scale_log2, -lse2));
                    ds[u] = (PARTIAL && key >= nv) ? 0.0f : pr * (dp[nb][r] - dval);
                }
                w[e2] = pack_bf16x2(ds[0], ds[1]);
            }
            pk[ch] = __builtin_bit_cast(bf16x8, w);
        }
        // dQ^T += K^T dS^T
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int g = 0; g < KC; ++g)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(smem, kb, ko, db, g), pk[g], dq[db], 0,
                                                                 0, 0);
        __builtin_amdgcn_s_setprio(0);
    }
    if (SPLIT) {
        float* mine = prm.ws_q + ((int64_t)wi * NW + wave) * (DB * 16 * 64);
        const float* parts = prm.ws_q + ((int64_t)slot * SP * NW + wave) * (DB * 16 * 64);
        if (!merge_parts<DB>(dq, mine, parts, (int64_t)NW * DB * 16 * 64, SP, prm.ws_counter_q + item, smem, tid))
            return;
    }
    store_rows<DB>(prm.dq + qrow, dq, prm.scale, hi);
}

// -------------------------------------------------------------------- dK, dV
// One workgroup per KV tile of BKV rows, BKV/32 waves of 32 key rows; K and V
// rows stay in registers. The tile's Q-direction list is walked in 32-row
// query steps: Q and dO (swz_d: row reads for S = Q K^T and dP = dO V^T,
// transposing reads for dK^T += Q^T dS and dV^T += dO^T P) and the rows'
// D and LSE are fetched for the next step while this one is computed.
// 32-row steps keep a 128-key workgroup within 256 registers per wave, so two
// workgroups share a compute unit and each SIMD has a second wave whose MFMAs
// can run while this one computes exponentials.
template <int BKV, int D, bool PARTIAL, bool SPLIT, bool STRIDED>
__global__ __launch_bounds__(BKV * 2, 2) void vsa_bwd_dkv_kernel(BwdParams prm) {
    constexpr int NW = BKV / 32;
    constexpr int QS = kDkvQs;  // query rows per step
    using G = TileGeom<QS, D>;
    using F = TileFetch<QS, D, NW>;
    using OO = OperandOffsets<D>;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int STAGE = 2 * G::TILE + 2 * QS * 4;  // Q, dO, D[QS], lse2[QS]
    static_assert(STAGE == dkv_stage_bytes<D>(), "launch sizes the LDS from dkv_stage_bytes");
    extern __shared__ __attribute__((aligned(1024))) char smem[];  // 2 stages, then the list

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = xcd_contiguous_block();
    const int SP = SPLIT ? prm.splits_kv : 1;  // built apart so the unsplit loop keeps its registers
    if (wi >= prm.n_items_kv * SP) return;
    const int slot = SP == 1 ? wi : wi / SP;
    const int part = wi - slot * SP;  // takes list entries part, part + SP, ...
    const int item = prm.work_kv ? prm.work_kv[slot] : slot;
    if (item < 0 || item >= prm.n_items_kv) return;
    const int nt = item % prm.nkv, bh = item / prm.nkv, h = bh % prm.H, b = bh / prm.H;
    const int S = prm.S, nq = prm.nq, block_q = prm.block_q;
    const int64_t tok_stride = (int64_t)prm.H * D;  // dk and dv are contiguous
    const int32_t* qrow_list = prm.qidx + (int64_t)item * prm.q_ld + part;
    const int ldp = prm.q_ld > part ? (prm.q_ld - part + SP - 1) / SP : 0;  // this part's slots of the row
    const int ldc = ldp < kIdxCapBwd ? ldp : kIdxCapBwd;
    int n = prm.qcnt[item];
    n = n < 0 ? 0 : (n > prm.q_ld ? prm.q_ld : n);
    n = n > part ? (n - part + SP - 1) / SP : 0;  // this part's entries
    n = n > ldc ? ldc : n;
    const int RQ = block_q / QS;
    const int steps = n * RQ;
    const int kv0 = nt * BKV + wave * 32;
    const int64_t krow = ((int64_t)b * S + kv0 + l32) * tok_stride + (int64_t)h * D;  // dk, dv
    // (built apart for contiguous inputs, where Q and dO share one row stride
    // and one set of tile-fetch offsets)
    const int64_t kin =
        STRIDED ? (int64_t)b * prm.ks[0] + (int64_t)(kv0 + l32) * prm.ks[1] + (int64_t)h * prm.ks[2] : krow;
    const int64_t vin =
        STRIDED ? (int64_t)b * prm.vs[0] + (int64_t)(kv0 + l32) * prm.vs[1] + (int64_t)h * prm.vs[2] : krow;
    // valid keys of this wave's column (partial tiles)
    int nv_tile = BKV;
    if constexpr (PARTIAL) {
        const int nvt = prm.kv_valid[nt];
        nv_tile = nvt < 0 ? 0 : (nvt > BKV ? BKV : nvt);
    }
    const bool key_ok = wave * 32 + l32 < nv_tile;

    bf16x8 kreg[DC], vreg[DC];
    load_rows<DC>(kreg, prm.k + kin, hi);
    load_rows<DC>(vreg, prm.v + vin, hi);

    int* lq = (int*)(smem + 2 * STAGE);
    for (int i = tid; i < ldc; i += BKV * 2) {
        const int m = qrow_list[(int64_t)i * SP];
        lq[i] = (m >= 0 && m < nq) ? m : -1;
    }
#pragma unroll
    for (int c = 0; c < DC; ++c) asm volatile("" ::"v"(kreg[c]), "v"(vreg[c]));
    wait_global_loads();
    lds_barrier();

    // compact offsets: the full set left this kernel a few registers short,
    // and the spill reload inside the step waited on the next step's tile loads
    CompactOffsets<D> qo;
    qo.template init<kLayoutD>(lane);
    // Q and dO row strides
    const int qt_bytes = STRIDED ? (int)(prm.qs[1] * 2) : (int)(tok_stride * 2);
    const int dt_bytes = STRIDED ? (int)(prm.ds[1] * 2) : qt_bytes;
    const F qfetch(smem, wave, lane, qt_bytes), dfetch(smem, wave, lane, dt_bytes);
    const int64_t qb0 = STRIDED ? (int64_t)b * prm.qs[0] + (int64_t)h * prm.qs[2] : (int64_t)b * S * tok_stride + h * D;
    const int64_t db0 = STRIDED ? (int64_t)b * prm.ds[0] + (int64_t)h * prm.ds[2] : qb0;
    const char* qbase = (const char*)(prm.q + qb0);
    const char* dbase = (const char*)(prm.dout + db0);
    const float* dvec = prm.aux + (int64_t)bh * S;
    const float* lvec = prm.aux + (int64_t)prm.n_rows + (int64_t)bh * S;
    auto entry = [&](int j) { return __builtin_amdgcn_readfirstlane(lq[j / RQ]); };
    auto fetch_step = [&](int j) {
        const int m = entry(j);
        const int r0 = (m >= 0 ? m : 0) * block_q + (j % RQ) * QS;  // first query row of the step
        const int st = (j & 1) * STAGE;
        qfetch.all(st, uniform_ptr(qbase + (int64_t)r0 * qt_bytes), qt_bytes, kLayoutD);
        dfetch.all(st + G::TILE, uniform_ptr(dbase + (int64_t)r0 * dt_bytes), dt_bytes, kLayoutD);
        if (wave == 0 && lane < QS / 4) {
            // D and lse2 of the step's rows: 256 bytes each, 16 bytes per lane
            const uint32_t dst = qfetch.lds0 + (uint32_t)(st + 2 * G::TILE);
            lds_dma16(dvec + r0, (uint32_t)(lane * 16), dst);
            lds_dma16(lvec + r0, (uint32_t)(lane * 16), dst + QS * 4);
        }
    };

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    if (steps > 0) fetch_step(0);
    for (int j = 0; j < steps; ++j) {
        wait_global_loads();
        lds_barrier();
        if (j + 1 < steps) fetch_step(j + 1);
        if (entry(j) < 0) continue;  // uniform
        const int qb = (j & 1) * STAGE, ob = qb + G::TILE, ab = qb + 2 * G::TILE;
        // S = Q K^T and dP = dO V^T for every 32-row block of the step first,
        // then per block the exp/dS work and the dV, dK products
        f32x16 s[QS / 32], dp[QS / 32];
        __builtin_amdgcn_s_setprio(1);  // MFMA blocks at raised issue priority, as in the dQ kernel
#pragma unroll
        for (int qs = 0; qs < QS / 32; ++qs) {
            s[qs] = f32x16{};
            dp[qs] = f32x16{};
        }
#pragma unroll
        for (int c = 0; c < DC; ++c)
#pragma unroll
            for (int qs = 0; qs < QS / 32; ++qs) {
                const bf16x8 qa = *(const bf16x8*)(smem + qo.row(qb, c) + qs * 32 * OO::ROW_BYTES);
                s[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[c], s[qs], 0, 0, 0);
                const bf16x8 oa = *(const bf16x8*)(smem + qo.row(ob, c) + qs * 32 * OO::ROW_BYTES);
                dp[qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vreg[c], dp[qs], 0, 0, 0);
            }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int qs = 0; qs < QS / 32; ++qs) {
            // rows q = qs*32 + 8*(r/4) + 4*hi + r%4: their D and lse2, four at a time
            bf16x8 pp[2], ps[2];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                u32x4 wp, wsd;
#pragma unroll
                for (int k4 = 0; k4 < 2; ++k4) {
                    const int qr = qs * 32 + 8 * (half * 2 + k4) + 4 * hi;
                    const f32x4 dd = *(const f32x4*)(smem + ab + qr * 4);
                    const f32x4 ll = *(const f32x4*)(smem + ab + QS * 4 + qr * 4);
                    float pv[4], dsv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int r = (half * 2 + k4) * 4 + u;
                        const float pr = fast_exp2(fmaf(s[qs][r], prm.scale_log2, -ll[u]));
                        const bool off = PARTIAL && !key_ok;
                        pv[u] = off ? 0.0f : pr;
                        dsv[u] = off ? 0.0f : pr * (dp[qs][r] - dd[u]);
                    }
                    wp[k4 * 2] = pack_bf16x2(pv[0], pv[1]);
                    wp[k4 * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
                    wsd[k4 * 2] = pack_bf16x2(dsv[0], dsv[1]);
                    wsd[k4 * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
                }
                pp[half] = __builtin_bit_cast(bf16x8, wp);
                ps[half] = __builtin_bit_cast(bf16x8, wsd);
            }
            // dV^T += dO^T P, dK^T += Q^T dS over the 32 rows (two 16-row k chunks)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(smem, ob, qo, db, qs * 2 + g), pp[g],
                                                                     dv[db], 0, 0, 0);
                    dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(smem, qb, qo, db, qs * 2 + g), ps[g],
                                                                     dk[db], 0, 0, 0);
                }
            __builtin_amdgcn_s_setprio(0);
        }
    }
    if (SPLIT) {
        constexpr int64_t W = 2 * DB * 16 * 64;  // dK, then dV
        f32x16 acc[2 * DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            acc[db] = dk[db];
            acc[DB + db] = dv[db];
        }
        float* mine = prm.ws_kv + ((int64_t)wi * NW + wave) * W;
        const float* parts = prm.ws_kv + ((int64_t)slot * SP * NW + wave) * W;
        if (!merge_parts<2 * DB>(acc, mine, parts, (int64_t)NW * W, SP, prm.ws_counter_kv + item, smem, tid)) return;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            dk[db] = acc[db];
            dv[db] = acc[DB + db];
        }
    }
    store_rows<DB>(prm.dk + krow, dk, prm.scale, hi);
    store_rows<DB>(prm.dv + krow, dv, 1.0f, hi);
}

// Launch with `lds` bytes of dynamic LDS (allowing more than the default
// limit once per kernel when needed).
template <typename K>
hipError_t launch_dyn(K kernel, int grid, int threads, int lds, const BwdParams& p, hipStream_t stream) {
    if (lds > 65536) {
        const hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kernel), lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), lds, stream, p);
    return hipGetLastError();
}

template <int D, bool PARTIAL, bool SPLIT>
hipError_t launch_dq_s(const BwdParams& p, hipStream_t stream) {
    const int list = 4 * (p.ld < kIdxCapBwd ? p.ld : kIdxCapBwd);
    const int grid = p.n_items_q * p.splits_q;
    switch (p.block_q) {
        case 64:
            return launch_dyn(vsa_bwd_dq_kernel<64, D, PARTIAL, SPLIT>, grid, 128, 2 * dq_stage_bytes<64, D>() + list, p,
                              stream);
        case 128:
            return launch_dyn(vsa_bwd_dq_kernel<128, D, PARTIAL, SPLIT>, grid, 256,
                              2 * dq_stage_bytes<128, D>() + list, p, stream);
        case 256:
            return launch_dyn(vsa_bwd_dq_kernel<256, D, PARTIAL, SPLIT>, grid, 512,
                              2 * dq_stage_bytes<256, D>() + list, p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool PARTIAL>
hipError_t launch_dq_d(const BwdParams& p, hipStream_t stream) {
    if (p.n_items_q <= 0) return hipSuccess;
    return p.splits_q > 1 ? launch_dq_s<D, PARTIAL, true>(p, stream) : launch_dq_s<D, PARTIAL, false>(p, stream);
}

template <int D, bool PARTIAL, bool SPLIT, bool STRIDED>
hipError_t launch_dkv_s(const BwdParams& p, hipStream_t stream) {
    const int lds = 2 * dkv_stage_bytes<D>() + 4 * (p.q_ld < kIdxCapBwd ? p.q_ld : kIdxCapBwd);
    const int grid = p.n_items_kv * p.splits_kv;
    switch (p.block_kv) {
        case 64: return launch_dyn(vsa_bwd_dkv_kernel<64, D, PARTIAL, SPLIT, STRIDED>, grid, 128, lds, p, stream);
        case 128: return launch_dyn(vsa_bwd_dkv_kernel<128, D, PARTIAL, SPLIT, STRIDED>, grid, 256, lds, p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool PARTIAL>
hipError_t launch_dkv_d(const BwdParams& p, hipStream_t stream) {
    if (p.n_items_kv <= 0) return hipSuccess;
    if (p.strided)
        return p.splits_kv > 1 ? launch_dkv_s<D, PARTIAL, true, true>(p, stream)
                               : launch_dkv_s<D, PARTIAL, false, true>(p, stream);
    return p.splits_kv > 1 ? launch_dkv_s<D, PARTIAL, true, false>(p, stream)
                           : launch_dkv_s<D, PARTIAL, false, false>(p, stream);
}

}  // namespace

bool bwd_supported(int block_q, int block_kv, int head_dim) {
    return (block_q == 64 || block_q == 128 || block_q == 256) && (block_kv == 64 || block_kv == 128) &&
           (head_dim == 64 || head_dim == 128);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.dout = a.dout;
    p.o = a.o;
    p.lse = a.lse;
    for (int i = 0; i < 3; ++i) {
        const int64_t contiguous[3] = {(int64_t)a.S * a.H * a.D, (int64_t)a.H * a.D, (int64_t)a.D};
        p.qs[i] = a.strides ? a.strides[i] : contiguous[i];
        p.ks[i] = a.strides ? a.strides[3 + i] : contiguous[i];
        p.vs[i] = a.strides ? a.strides[6 + i] : contiguous[i];
        p.ds[i] = a.strides ? a.strides[9 + i] : contiguous[i];
    }
    p.strided = 0;
    for (int i = 0; i < 3; ++i) {
        const int64_t contiguous[3] = {(int64_t)a.S * a.H * a.D, (int64_t)a.H * a.D, (int64_t)a.D};
        if (p.qs[i] != contiguous[i] || p.ks[i] != contiguous[i] || p.vs[i] != contiguous[i] || p.ds[i] != contiguous[i])
            p.strided = 1;
    }
    p.aux = a.aux;
    p.idx = a.idx;
    p.cnt = a.cnt;
    p.qidx = a.qidx;
    p.qcnt = a.qcnt;
    p.kv_valid = a.kv_valid;
    p.work_q = a.work_q;
    p.work_kv = a.work_kv;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.S = a.S;
    p.H = a.H;
    p.nq = a.S / a.block_q;
    p.nkv = a.S / a.block_kv;
    p.ld = a.ld;
    p.q_ld = a.q_ld;
    p.block_q = a.block_q;
    p.block_kv = a.block_kv;
    p.n_rows = a.B * a.H * a.S;
    p.n_items_q = a.B * a.H * p.nq;
    p.n_items_kv = a.B * a.H * p.nkv;
    p.scale = a.scale;
    p.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    p.splits_q = a.splits_q > 1 ? a.splits_q : 1;
    p.splits_kv = a.splits_kv > 1 ? a.splits_kv : 1;
    p.ws_counter_q = a.ws_counter_q;
    p.ws_counter_kv = a.ws_counter_kv;
    p.ws_q = a.ws_q;
    p.ws_kv = a.ws_kv;
    // the dQ kernel forms D and LSE*log2(e) for every row, which the dK/dV kernel reads
    const bool partial = a.kv_valid != nullptr;
    hipError_t e;
    if (a.D == 128) {
        e = partial ? launch_dq_d<128, true>(p, stream) : launch_dq_d<128, false>(p, stream);
        if (e != hipSuccess) return e;
        return partial ? launch_dkv_d<128, true>(p, stream) : launch_dkv_d<128, false>(p, stream);
    }
    e = partial ? launch_dq_d<64, true>(p, stream) : launch_dq_d<64, false>(p, stream);
    if (e != hipSuccess) return e;
    return partial ? launch_dkv_d<64, true>(p, stream) : launch_dkv_d<64, false>(p, stream);
}

}  // namespace vsa
