// Fused block-sparse attention forward for gfx950 (CDNA4).
//
// What is computed (FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// benchmarks/bench_vsa_blackwell.py, ref_masked_sdpa_fp32): for each query
// tile p of head h, O = softmax(scale * Q K^T over the selected KV tiles) V and
// the per-row natural-log LSE. The online softmax runs in base 2 with
// scale*log2(e) folded into one multiply, keeps a running row max and row sum,
// and rescales the accumulator only when the max has grown by more than a
// threshold (page "BlackwellMultiHeadLatentAttentionForwardFP8": softmax,
// correction and its skip_correction_threshold).
//
// Design (one workgroup per work-list entry = one query tile):
//  * BQ/32 waves; wave w owns query rows [w*32, w*32+32) of the tile.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    lane l then holds 16 scores of query row (l%32) per 32-key block, so the
//    row max/sum is an in-lane reduction plus one exchange between the two
//    half-waves. Q^T stays in VGPRs for the whole tile (B operand).
//  * O^T = V^T P^T with the same instruction: the score accumulator,
//    exponentiated and packed to bf16, is directly the B operand (no
//    shuffles), and the per-row rescale factor is lane-uniform.
//  * K is staged to LDS row-major, V transposed (V^T, keys of each 16-key
//    group in the order the score accumulator holds them); 16-byte chunks are
//    XOR-swizzled by row so 16 consecutive rows of one chunk column hit
//    distinct bank groups. The next KV tile is fetched into VGPRs while the
//    current one is consumed.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.6931471805599453f;
// A stale row max is kept while the new tile max exceeds it by at most this
// many powers of two, so un-normalised probabilities stay <= 2^8.
constexpr float kRescaleThreshold = 8.0f;

// Chunk-column XOR swizzle for a row of NC 16-byte chunks.
template <int NC>
__device__ __forceinline__ int swz(int row) {
    if constexpr (NC >= 16) {
        return row & 15;
    } else if constexpr (NC == 8) {
        return (row >> 1) & 7;
    } else {
        static_assert(NC == 4, "unsupported row width");
        return (row >> 2) & 3;
    }
}

// Byte offset of 16-byte chunk c of row r in a swizzled LDS matrix.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int r, int c) {
    constexpr int NC = ROW_BYTES / 16;
    return r * ROW_BYTES + ((c ^ swz<NC>(r)) << 4);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int BQ, int BKV, int D>
struct Cfg {
    static constexpr int WAVES = BQ / 32;
    static constexpr int NT = WAVES * 64;  // == BQ * 2 (launch bound)
    static constexpr int DC = D / 16;          // 16-wide d chunks (QK^T k-steps)
    static constexpr int NB = BKV / 32;        // 32-key blocks of S^T
    static constexpr int DB = D / 32;          // 32-wide d blocks of O^T
    static constexpr int KC = BKV / 16;        // 16-key chunks (PV k-steps)
    static constexpr int K_ROW = D * 2;        // bytes per K row in LDS
    static constexpr int V_ROW = BKV * 2;      // bytes per V^T row in LDS
    static constexpr int K_CPR = D / 8;        // 16-byte chunks per K row
    static constexpr int K_LOADS = BKV * K_CPR / NT;
    static constexpr int V_UNITS = (BKV / 4) * (D / 8);   // 4 keys x 8 dims
    static constexpr int V_LOADS = (V_UNITS + NT - 1) / NT;
    static constexpr int LDS_BYTES = BKV * D * 2 * 2;
    static_assert(BKV * K_CPR % NT == 0, "K staging must divide evenly");
};

// Next tile-list position >= j whose tile index is in range (uniform).
__device__ __forceinline__ int next_valid(const int32_t* irow, int j, int n, int nkv) {
    while (j < n) {
        int t = __builtin_amdgcn_readfirstlane(irow[j]);
        if (t >= 0 && t < nkv) break;
        ++j;
    }
    return j;
}

template <int BQ, int BKV, int D>
__global__ __launch_bounds__(BQ * 2) void vsa_fwd_kernel(FwdParams prm) {
    using C = Cfg<BQ, BKV, D>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    char* Ks = smem;
    char* Vs = smem + BKV * D * 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int wi = blockIdx.x;
    if (wi >= prm.n_work) return;
    const int item = prm.work ? prm.work[wi] : wi;
    if (item < 0 || item >= prm.n_items) return;

    const int p = item % prm.nq;
    const int bh = item / prm.nq;
    const int h = bh % prm.H;
    const int b = bh / prm.H;
    const int S = prm.S;
    const int64_t tok_stride = (int64_t)prm.H * D;  // elements between tokens
    int n = prm.cnt[item];
    n = n < 0 ? 0 : (n > prm.ld ? prm.ld : n);
    const int32_t* irow = prm.idx + (int64_t)item * prm.ld;

    // ---- Q^T operand: lane holds query row (l32) d-chunks [c*16 + hi*8, +8) ----
    const int q0 = p * BQ + wave * 32;
    bf16x8 qreg[C::DC];
    {
        const uint16_t* qp = prm.q + ((int64_t)b * S + q0 + l32) * tok_stride + (int64_t)h * D + hi * 8;
#pragma unroll
        for (int c = 0; c < C::DC; ++c) qreg[c] = *(const bf16x8*)(qp + c * 16);
    }

    f32x16 oacc[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    const uint16_t* kbase = prm.k + (int64_t)b * S * tok_stride + (int64_t)h * D;
    const uint16_t* vbase = prm.v + (int64_t)b * S * tok_stride + (int64_t)h * D;

    u32x4 kst[C::K_LOADS];
    u32x4 vst[C::V_LOADS][4];

    auto load_tile = [&](int t) {
        const int64_t row0 = (int64_t)t * BKV;
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) {
            const int e = tid + i * C::NT;
            const int r = e / C::K_CPR, c = e % C::K_CPR;
            kst[i] = *(const u32x4*)(kbase + (row0 + r) * tok_stride + c * 8);
        }
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i) {
            const int u = tid + i * C::NT;
            if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
                const int d8 = u % (D / 8), kv4 = u / (D / 8);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vst[i][r] = *(const u32x4*)(vbase + (row0 + kv4 * 4 + r) * tok_stride + d8 * 8);
            }
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < C::K_LOADS; ++i) {
            const int e = tid + i * C::NT;
            const int r = e / C::K_CPR, c = e % C::K_CPR;
            *(u32x4*)(Ks + lds_off<C::K_ROW>(r, c)) = kst[i];
        }
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i) {
            const int u = tid + i * C::NT;
            if (C::V_UNITS % C::NT == 0 || u < C::V_UNITS) {
                const int d8 = u % (D / 8), kv4 = u / (D / 8);
                // keys kv4*4..+3 sit at positions g*16 + hh*8 + a*4 .. +3 of each V^T row,
                // where key-in-group = a*8 + hh*4 + (0..3): the order of the score
                // accumulator rows seen by one half-wave.
                const int kl = (kv4 * 4) & 15;
                const int g = (kv4 * 4) >> 4;
                const int a = kl >> 3, hh = (kl >> 2) & 1;
                const int chunk = g * 2 + hh;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const int m = c >> 1;
                    uint32_t w0, w1;
                    if (c & 1) {
                        w0 = (vst[i][0][m] >> 16) | (vst[i][1][m] & 0xffff0000u);
                        w1 = (vst[i][2][m] >> 16) | (vst[i][3][m] & 0xffff0000u);
                    } else {
                        w0 = (vst[i][0][m] & 0xffffu) | (vst[i][1][m] << 16);
                        w1 = (vst[i][2][m] & 0xffffu) | (vst[i][3][m] << 16);
                    }
                    *(u32x2*)(Vs + lds_off<C::V_ROW>(d8 * 8 + c, chunk) + a * 8) = u32x2{w0, w1};
                }
            }
        }
    };

    int j = next_valid(irow, 0, n, prm.nkv);
    if (j < n) load_tile(__builtin_amdgcn_readfirstlane(irow[j]));
    while (j < n) {
        const int jn = next_valid(irow, j + 1, n, prm.nkv);
        __syncthreads();  // every wave is done reading the previous tile
        store_tile();
        __syncthreads();
        if (jn < n) load_tile(__builtin_amdgcn_readfirstlane(irow[jn]));

        // ---- S^T = K Q^T : NB blocks of 32 keys x 32 query rows ----
        f32x16 sacc[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            sacc[nb] = f32x16{};
            const int krow = nb * 32 + l32;
#pragma unroll
            for (int c = 0; c < C::DC; ++c) {
                const bf16x8 a = *(const bf16x8*)(Ks + lds_off<C::K_ROW>(krow, 2 * c + hi));
                sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], sacc[nb], 0, 0, 0);
            }
        }

        // ---- online softmax (base 2) for query row l32 ----
        float mx = sacc[0][0];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_tile = mx * prm.scale_log2;
        const float m_new = fmaxf(m_run, m_tile);
        if (__any(m_new > m_run + kRescaleThreshold)) {
            const float alpha = fast_exp2(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
        }
        bf16x8 pk[C::KC];
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

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
#pragma unroll
            for (int g = 0; g < C::KC; ++g) {
                const bf16x8 a = *(const bf16x8*)(Vs + lds_off<C::V_ROW>(db * 32 + l32, 2 * g + hi));
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[g], oacc[db], 0, 0, 0);
            }
        }
        j = jn;
    }

    // ---- epilogue: O = O^T / l (bf16, RNE), LSE = (m + log2 l) ln 2 ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
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

template <int BQ, int BKV, int D>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
    using C = Cfg<BQ, BKV, D>;
    if (p.n_work <= 0) return hipSuccess;
    hipLaunchKernelGGL((vsa_fwd_kernel<BQ, BKV, D>), dim3(p.n_work), dim3(C::NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool fwd_supported(int block_q, int block_kv, int head_dim) {
    const bool bq = block_q == 64 || block_q == 128 || block_q == 256;
    const bool bkv = block_kv == 64 || block_kv == 128;
    const bool d = head_dim == 64 || head_dim == 128;
    return bq && bkv && d;
}

hipError_t launch_fwd(int block_q, int block_kv, int head_dim, const FwdParams& p, hipStream_t stream) {
#define VSA_CASE(BQ, BKV, D) \
    if (block_q == BQ && block_kv == BKV && head_dim == D) return launch<BQ, BKV, D>(p, stream);
    VSA_CASE(64, 64, 64)
    VSA_CASE(64, 64, 128)
    VSA_CASE(64, 128, 64)
    VSA_CASE(64, 128, 128)
#undef VSA_CASE
    if (block_q == 128) return launch_fwd_2s(block_kv, head_dim, p, stream);
    if (block_q == 256) return launch_fwd_pp(block_kv, head_dim, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace vsa
