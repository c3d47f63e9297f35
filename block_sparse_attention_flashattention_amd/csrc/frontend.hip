// Mask front-end for gfx950: logical block mask -> physical block CSR, and
// the count-sorted work list.
//
// Exact expansion (FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
// benchmarks/bench_vsa_blackwell.py, expand_exact256_mask and arm_fa4):
// physical Q tile p reads logical row floor(p / q_ratio); every selected
// logical KV cell t becomes physical tiles t*kv_ratio .. t*kv_ratio +
// kv_ratio-1, listed in ascending order. The selected token pairs are exactly
// those of the logical mask.
#include "vsa_internal.h"

namespace vsa {
namespace {

// One wave per physical CSR row: 64 mask bytes per step, ballot + prefix
// popcount to place each selected cell. With valid key counts per physical
// KV tile (VALID), a tile with no valid key is left out of the list: each
// lane counts the non-empty tiles of its cell and a wave prefix sum places
// them.
template <bool VALID>
__global__ __launch_bounds__(256) void mask_to_csr_kernel(const uint8_t* __restrict__ mask, int n_rows,
                                                          int nq_logical, int nkv_logical, int q_ratio,
                                                          int kv_ratio, int nq_physical,
                                                          const int32_t* __restrict__ kv_valid,
                                                          int32_t* __restrict__ idx, int ld,
                                                          int32_t* __restrict__ cnt,
                                                          int32_t* __restrict__ overflow) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= n_rows) return;
    const int p = row % nq_physical;
    const int bh = row / nq_physical;
    const uint8_t* mrow = mask + ((int64_t)bh * nq_logical + p / q_ratio) * nkv_logical;
    int32_t* orow = idx + (int64_t)row * ld;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int running = 0;  // physical tiles listed so far
    for (int base = 0; base < nkv_logical; base += 64) {
        const int t = base + lane;
        const bool sel = t < nkv_logical && mrow[t] != 0;
        if constexpr (!VALID) {
            const uint64_t bal = __ballot(sel);
            if (sel) {
                const int pos = (running + __popcll(bal & below)) * kv_ratio;
                for (int r = 0; r < kv_ratio; ++r)
                    if (pos + r < ld) orow[pos + r] = t * kv_ratio + r;
            }
            running += __popcll(bal);
        } else {
            unsigned keep = 0;  // bit r: physical tile t*kv_ratio + r has a valid key
            if (sel)
                for (int r = 0; r < kv_ratio; ++r) keep |= (kv_valid[t * kv_ratio + r] > 0 ? 1u : 0u) << r;
            const int m = __popc(keep);
            int x = m;  // inclusive prefix sum of m over the wave
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off);
                if (lane >= off) x += y;
            }
            int pos = running + x - m;
            for (int r = 0; r < kv_ratio; ++r)
                if ((keep >> r) & 1u) {
                    if (pos < ld) orow[pos] = t * kv_ratio + r;
                    ++pos;
                }
            running += __shfl(x, 63);
        }
    }
    if (lane == 0) {
        const int c = VALID ? running : running * kv_ratio;
        cnt[row] = c;
        if (c > ld && overflow) *overflow = 1;
    }
}

// Lanes of the wave whose key equals this lane's key (among active lanes).
template <int KEY_BITS>
__device__ __forceinline__ uint64_t same_key_lanes(int key, bool active) {
    uint64_t m = __ballot(active);
#pragma unroll
    for (int bit = 0; bit < KEY_BITS; ++bit) {
        const bool set = (key >> bit) & 1;
        const uint64_t bb = __ballot(set);
        m &= set ? bb : ~bb;
    }
    return m;
}

// Stable counting sort of item indices by count, largest count first, within
// one segment of `seg` consecutive items per workgroup (segment blockIdx.x
// covers items [blockIdx.x*seg, +seg) and is written to the same positions
// of the work list). Wave w of the WAVES waves owns a contiguous part of the
// segment; per-wave histograms give each wave its own output offsets, and
// within a wave the rank among equal keys comes from ballots, so the result
// is deterministic and equal keys keep ascending item order.
//
// With a gate, the list is built only if (*gate == 0) == run_if_zero;
// otherwise every entry is -1, which the attention kernels skip. This lets
// the device choose between two schedules without a host round trip.
template <int WAVES, int BINS, int KEY_BITS>
__global__ __launch_bounds__(WAVES * 64) void worklist_kernel(const int32_t* __restrict__ cnt_all, int seg,
                                                             int max_cnt, int32_t* __restrict__ work_all,
                                                             const int32_t* __restrict__ gate, int run_if_zero) {
    const int32_t* cnt = cnt_all + (int64_t)blockIdx.x * seg;
    int32_t* work = work_all + (int64_t)blockIdx.x * seg;
    const int first_item = blockIdx.x * seg;
    const int n = seg;
    __shared__ int hist[WAVES][BINS];
    __shared__ int wave_total[WAVES];
    constexpr int NT = WAVES * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (gate != nullptr && ((*gate == 0) != (run_if_zero != 0))) {
        for (int i = tid; i < n; i += NT) work[i] = -1;
        return;
    }
    const int nbins = max_cnt + 1;
    for (int i = tid; i < WAVES * BINS; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();

    const int part = (n + WAVES - 1) / WAVES;
    const int beg = min(n, wave * part);
    const int end = min(n, beg + part);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // Phase 1: per-wave histogram of clamped counts.
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const bool act = i < end;
        int key = act ? cnt[i] : 0;
        key = key < 0 ? 0 : (key > max_cnt ? max_cnt : key);
        const uint64_t same = same_key_lanes<KEY_BITS>(key, act);
        if (act && (same & below) == 0) hist[wave][key] += __popcll(same);
    }
    __syncthreads();

    // Phase 2: exclusive scan over keys in descending order; each thread owns
    // PER consecutive positions (position o <-> key max_cnt - o).
    constexpr int PER = (BINS + NT - 1) / NT;
    int local_sum = 0;
    for (int k = 0; k < PER; ++k) {
        const int o = tid * PER + k;
        if (o < nbins) {
            const int key = max_cnt - o;
            for (int w = 0; w < WAVES; ++w) local_sum += hist[w][key];
        }
    }
    int incl = local_sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int run = incl - local_sum;
    for (int w = 0; w < wave; ++w) run += wave_total[w];
    for (int k = 0; k < PER; ++k) {
        const int o = tid * PER + k;
        if (o < nbins) {
            const int key = max_cnt - o;
            for (int w = 0; w < WAVES; ++w) {
                const int c = hist[w][key];
                hist[w][key] = run;
                run += c;
            }
        }
    }
    __syncthreads();

    // Phase 3: scatter in item order.
    for (int base = beg; base < end; base += 64) {
        const int i = base + lane;
        const bool act = i < end;
        int key = act ? cnt[i] : 0;
        key = key < 0 ? 0 : (key > max_cnt ? max_cnt : key);
        const uint64_t same = same_key_lanes<KEY_BITS>(key, act);
        const int pos = act ? hist[wave][key] + __popcll(same & below) : 0;
        if (act) work[pos] = first_item + i;
        if (act && (same & below) == 0) hist[wave][key] += __popcll(same);
    }
}

// Q-direction lists for the backward pass (the per-KV-tile lists of the query
// tiles that select the tile, "transposed from forward" in the FastVideo
// page's FA4 block_sparsity.py). One workgroup per (batch, head): the
// selection is marked in an LDS bitmap [KV tile][Q tile], a chunk of KV tiles
// at a time, then one wave per KV tile lists the set bits in ascending order
// with ballot + prefix popcount.
constexpr int kTransposeLdsWords = 16384;  // 64 KB bitmap per chunk

__global__ __launch_bounds__(1024) void csr_transpose_kernel(const int32_t* __restrict__ idx,
                                                             const int32_t* __restrict__ cnt, int nq, int nkv, int ld,
                                                             int32_t* __restrict__ q_idx, int q_ld,
                                                             int32_t* __restrict__ q_cnt,
                                                             int32_t* __restrict__ overflow) {
    __shared__ uint32_t bits[kTransposeLdsWords];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wpr = (nq + 31) / 32;                 // bitmap words per KV tile
    const int chunk = kTransposeLdsWords / wpr;     // KV tiles per pass (>= 1: host checks wpr)
    const int32_t* crow = idx + (int64_t)bh * nq * ld;
    const int32_t* ccnt = cnt + (int64_t)bh * nq;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int n0 = 0; n0 < nkv; n0 += chunk) {
        const int n1 = min(nkv, n0 + chunk);
        for (int w = tid; w < (n1 - n0) * wpr; w += 1024) bits[w] = 0u;
        __syncthreads();
        for (int e = tid; e < nq * ld; e += 1024) {
            const int m = e / ld, slot = e % ld;
            int c = ccnt[m];
            c = c < 0 ? 0 : (c > ld ? ld : c);
            if (slot >= c) continue;
            const int t = crow[e];
            if (t >= n0 && t < n1) atomicOr(&bits[(t - n0) * wpr + (m >> 5)], 1u << (m & 31));
        }
        __syncthreads();
        for (int n = n0 + wave; n < n1; n += 16) {
            const uint32_t* row = bits + (n - n0) * wpr;
            int32_t* orow = q_idx + ((int64_t)bh * nkv + n) * q_ld;
            int running = 0;
            for (int base = 0; base < nq; base += 64) {
                const int m = base + lane;
                const bool sel = m < nq && ((row[m >> 5] >> (m & 31)) & 1u);
                const uint64_t bal = __ballot(sel);
                const int pos = running + __popcll(bal & below);
                if (sel && pos < q_ld) orow[pos] = m;
                running += __popcll(bal);
            }
            if (lane == 0) {
                q_cnt[(int64_t)bh * nkv + n] = running;
                if (running > q_ld && overflow) *overflow = 1;
            }
        }
        __syncthreads();
    }
}

// Pairing of query tiles (2p, 2p+1) onto tiles twice as tall (FastVideo page:
// the Q64 children of one Q256 row share their KV list and run on the
// Q128/KV64 schedule). One wave per pair: row p of the output takes row 2p's
// count and stored entries; a pair whose counts or stored entries differ adds
// one to *unpaired (zeroed by zero_kernel before this launch).
__global__ __launch_bounds__(256) void pair_q_tiles_kernel(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ cnt, int n_pairs, int ld,
                                                           int32_t* __restrict__ out_idx,
                                                           int32_t* __restrict__ out_cnt,
                                                           int32_t* __restrict__ unpaired) {
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (pair >= n_pairs) return;
    const int c0 = cnt[2 * (int64_t)pair], c1 = cnt[2 * (int64_t)pair + 1];
    const int n = c0 < 0 ? 0 : (c0 > ld ? ld : c0);
    const int32_t* r0 = idx + 2 * (int64_t)pair * ld;
    const int32_t* r1 = r0 + ld;
    int32_t* o = out_idx + (int64_t)pair * ld;
    bool differ = false;
    for (int base = 0; base < n; base += 64) {
        const int j = base + lane;
        if (j < n) {
            const int32_t t = r0[j];
            o[j] = t;
            differ |= t != r1[j];
        }
    }
    differ = __ballot(differ) != 0ull || c0 != c1;
    if (lane == 0) {
        out_cnt[pair] = c0;
        if (differ) atomicAdd(unpaired, 1);
    }
}

__global__ void zero_kernel(int32_t* p) { *p = 0; }

// p[0, n) = 0, grid-stride (clears split counters without a memset node, so
// that a captured graph replays it like any other kernel).
__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// Gates of a two-level pairing from the mismatch counts of level 1 (a) and
// level 2 (b): the 256-row list runs iff a + b == 0, the 128-row list iff
// a == 0 and b != 0 (both as "run if the gate is zero").
__global__ void pair_gates_kernel(const int32_t* a, const int32_t* b, int32_t* gate256, int32_t* gate128) {
    const int32_t x = *a, y = *b;
    *gate256 = (x == 0 && y == 0) ? 0 : 1;
    *gate128 = (x == 0 && y != 0) ? 0 : 1;
}

// Valid keys per physical KV tile from valid tokens per logical KV block:
// tile r of block T keeps clamp(vbs[T] - r*block_kv, 0, block_kv).
__global__ void expand_valid_kernel(const int32_t* vbs, int n_out, int kv_ratio, int block_kv, int32_t* out) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_out) return;
    const int r = i % kv_ratio;
    const int v = vbs[i / kv_ratio] - r * block_kv;
    out[i] = v < 0 ? 0 : (v > block_kv ? block_kv : v);
}

}  // namespace

hipError_t launch_mask_to_csr(const uint8_t* mask, int batch, int heads, int nq_logical, int nkv_logical,
                              int q_ratio, int kv_ratio, int nq_physical, const int32_t* kv_valid, int32_t* idx,
                              int ld, int32_t* cnt, int32_t* overflow, hipStream_t stream) {
    const int n_rows = batch * heads * nq_physical;
    if (n_rows <= 0) return hipSuccess;
    if (kv_valid)
        hipLaunchKernelGGL(mask_to_csr_kernel<true>, dim3((n_rows + 3) / 4), dim3(256), 0, stream, mask, n_rows,
                           nq_logical, nkv_logical, q_ratio, kv_ratio, nq_physical, kv_valid, idx, ld, cnt, overflow);
    else
        hipLaunchKernelGGL(mask_to_csr_kernel<false>, dim3((n_rows + 3) / 4), dim3(256), 0, stream, mask, n_rows,
                           nq_logical, nkv_logical, q_ratio, kv_ratio, nq_physical, kv_valid, idx, ld, cnt, overflow);
    return hipGetLastError();
}

hipError_t launch_build_worklist(const int32_t* cnt, int n_items, int segment, int max_cnt, int32_t* work,
                                 hipStream_t stream, const int32_t* gate, bool run_if_zero) {
    if (n_items <= 0) return hipSuccess;
    const int n_seg = n_items / segment;
    if (max_cnt < 2048) {
        hipLaunchKernelGGL((worklist_kernel<4, 2048, 11>), dim3(n_seg), dim3(256), 0, stream, cnt, segment, max_cnt,
                           work, gate, (int)run_if_zero);
    } else {
        hipLaunchKernelGGL((worklist_kernel<1, 8192, 13>), dim3(n_seg), dim3(64), 0, stream, cnt, segment, max_cnt,
                           work, gate, (int)run_if_zero);
    }
    return hipGetLastError();
}

hipError_t launch_pair_q_tiles(const int32_t* idx, const int32_t* cnt, int n_pairs, int ld, int32_t* out_idx,
                               int32_t* out_cnt, int32_t* unpaired, hipStream_t stream) {
    hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(1), 0, stream, unpaired);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_pairs <= 0) return e;
    hipLaunchKernelGGL(pair_q_tiles_kernel, dim3((n_pairs + 3) / 4), dim3(256), 0, stream, idx, cnt, n_pairs, ld,
                       out_idx, out_cnt, unpaired);
    return hipGetLastError();
}

hipError_t launch_pair_gates(const int32_t* a, const int32_t* b, int32_t* gate256, int32_t* gate128,
                             hipStream_t stream) {
    hipLaunchKernelGGL(pair_gates_kernel, dim3(1), dim3(1), 0, stream, a, b, gate256, gate128);
    return hipGetLastError();
}

hipError_t launch_csr_transpose(const int32_t* idx, const int32_t* cnt, int batch_heads, int nq, int nkv, int ld,
                                int32_t* q_idx, int q_ld, int32_t* q_cnt, int32_t* overflow, hipStream_t stream) {
    if (batch_heads <= 0 || nkv <= 0) return hipSuccess;
    hipLaunchKernelGGL(csr_transpose_kernel, dim3(batch_heads), dim3(1024), 0, stream, idx, cnt, nq, nkv, ld, q_idx,
                       q_ld, q_cnt, overflow);
    return hipGetLastError();
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_expand_valid(const int32_t* vbs, int nkv_logical, int kv_ratio, int block_kv, int32_t* kv_valid,
                               hipStream_t stream) {
    const int n = nkv_logical * kv_ratio;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(expand_valid_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, vbs, n, kv_ratio, block_kv,
                       kv_valid);
    return hipGetLastError();
}

}  // namespace vsa
