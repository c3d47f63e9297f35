// Internal declarations shared by the translation units of libvsa_attn.so.
// Not part of the public ABI (that is include/vsa_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

namespace vsa {

// Arguments of the fused forward kernel. All pointers are device pointers.
struct FwdParams {
    const uint16_t* q;       // [B, S, H, D] bf16 bits
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* idx;      // [B, H, nq, ld]
    const int32_t* cnt;      // [B, H, nq]
    const int32_t* work;     // [n_work] flat (b*H + h)*nq + p; may be null = identity
    const int32_t* kv_valid; // [nkv] valid leading keys per KV tile; null = all tiles full
    uint16_t* o;             // [B, S, H, D] bf16 bits
    float* lse;              // [B, H, S]
    // element strides of q, k and v between batches, tokens and heads (row r
    // of head h in batch b starts at b*s[0] + r*s[1] + h*s[2]; head_dim is
    // contiguous); o and lse are contiguous
    int64_t qs[3], ks[3], vs[3];
    int32_t n_work;
    int32_t n_items;         // B * H * nq
    int32_t S, H, nq, nkv, ld;
    int32_t block_kv;        // tokens per KV tile of the CSR
    float scale_log2;        // softmax scale * log2(e)
    // Split lists (256-row tiles only): work entry w is served by workgroups
    // w*splits .. w*splits + splits-1, part q taking list entries q, q+splits, ...;
    // partial states go to ws_partial, the last part to finish merges them
    // (ws_counter: one int per item, zero between launches).
    int32_t splits;
    int32_t* ws_counter;
    float* ws_partial;
};

// Launch the forward kernel for one (block_q, block_kv, head_dim); returns
// hipSuccess or the launch error. Shapes are validated by the caller.
hipError_t launch_fwd(int block_q, int block_kv, int head_dim, const FwdParams& p, hipStream_t stream);

// 256-row query tiles: the two-group ping-pong kernel (attn_fwd_pp.hip).
hipError_t launch_fwd_pp(int block_kv, int head_dim, const FwdParams& p, hipStream_t stream);
// 128-row query tiles: the two-KV-stream ping-pong kernel (attn_fwd_2s.hip).
hipError_t launch_fwd_2s(int block_kv, int head_dim, const FwdParams& p, hipStream_t stream);
// 64-row query tiles: the four-KV-stream ping-pong kernel (attn_fwd_4s.hip).
hipError_t launch_fwd_4s(int block_kv, int head_dim, const FwdParams& p, hipStream_t stream);

// 128-row query tiles over 128-key tiles, whole-tile streams (attn_fwd_2t.hip).
hipError_t launch_fwd_2t(int head_dim, const FwdParams& p, hipStream_t stream);
// 64- and 128-row query tiles with independent waves (attn_fwd_iw.hip).
hipError_t launch_fwd_iw(int block_q, int head_dim, const FwdParams& p, hipStream_t stream);

// Let `kernel` be launched with `bytes` of dynamic LDS (above the default
// limit); remembered per kernel. Host only.
inline hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
    static std::mutex mutex;
    static std::vector<std::pair<const void*, int>> allowed;
    std::lock_guard<std::mutex> lock(mutex);
    for (auto& a : allowed)
        if (a.first == kernel && a.second >= bytes) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) allowed.emplace_back(kernel, bytes);
    return e;
}

// Compute units of the current device (cached per device; 0 if unknown). Host only.
inline int device_cu_count() {
    static std::mutex mutex;
    static std::vector<int> counts;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mutex);
    if ((int)counts.size() <= dev) counts.resize(dev + 1, 0);
    if (counts[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) counts[dev] = n;
    }
    return counts[dev];
}

// Work items per compute unit from which 64- and 128-row tiles run the
// independent-wave kernel rather than the eight-wave multi-stream ones.
constexpr int kIwItemsPerCu = 8;

// Whether launch_fwd has a kernel for this configuration.
bool fwd_supported(int block_q, int block_kv, int head_dim);

// Arguments of the backward pass (attn_bwd.hip). aux: [2 * B*H*S] fp32
// scratch (D, LSE*log2 e); work lists as for the forward.
struct BwdArgs {
    const uint16_t *q, *k, *v, *o, *dout;
    // element strides of q, k, v and dout as (batch, token, head), 12 values
    // (head_dim contiguous); null: all four contiguous [B, S, H, D]. o, dq, dk
    // and dv are contiguous.
    const int64_t* strides = nullptr;
    const float* lse;
    float* aux;
    const int32_t *idx, *cnt;    // forward CSR
    const int32_t *qidx, *qcnt;  // Q-direction CSR
    const int32_t* kv_valid;
    const int32_t *work_q, *work_kv;
    uint16_t *dq, *dk, *dv;
    int32_t B, S, H, D, ld, q_ld, block_q, block_kv;
    float scale;
    // split lists (1 = off) and their workspaces (counters zero on entry)
    int32_t splits_q = 1, splits_kv = 1;
    int32_t *ws_counter_q = nullptr, *ws_counter_kv = nullptr;
    float *ws_q = nullptr, *ws_kv = nullptr;
};
// Accumulator floats per wave that a split backward part publishes.
inline int bwd_split_words_q(int head_dim) { return head_dim / 32 * 16 * 64; }
inline int bwd_split_words_kv(int head_dim) { return 2 * head_dim / 32 * 16 * 64; }
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
bool bwd_supported(int block_q, int block_kv, int head_dim);

// Front-end launches (frontend.hip).
// kv_valid (may be null): valid keys per physical KV tile; tiles without one
// are left out of the lists.
hipError_t launch_mask_to_csr(const uint8_t* mask, int batch, int heads, int nq_logical, int nkv_logical,
                              int q_ratio, int kv_ratio, int nq_physical, const int32_t* kv_valid, int32_t* idx,
                              int ld, int32_t* cnt, int32_t* overflow, hipStream_t stream);
// With a gate, the list is built only if (*gate == 0) == run_if_zero, and
// is all -1 (skipped by the kernels) otherwise.
hipError_t launch_build_worklist(const int32_t* cnt, int n_items, int segment, int max_cnt, int32_t* work,
                                 hipStream_t stream, const int32_t* gate = nullptr, bool run_if_zero = true);
// Query tiles (2p, 2p+1) -> tile p of twice the height; *unpaired = number of
// pairs whose lists differ (zeroed by the launch itself, in stream order).
hipError_t launch_pair_gates(const int32_t* a, const int32_t* b, int32_t* gate256, int32_t* gate128,
                             hipStream_t stream);
hipError_t launch_pair_q_tiles(const int32_t* idx, const int32_t* cnt, int n_pairs, int ld, int32_t* out_idx,
                               int32_t* out_cnt, int32_t* unpaired, hipStream_t stream);
// Q-direction CSR for the backward pass; nq must be <= 32 * kTransposeMaxWords.
hipError_t launch_csr_transpose(const int32_t* idx, const int32_t* cnt, int batch_heads, int nq, int nkv, int ld,
                                int32_t* q_idx, int q_ld, int32_t* q_cnt, int32_t* overflow, hipStream_t stream);
constexpr int kTransposeMaxWords = 16384;
// p[0, n) = 0 by a kernel (no memset node).
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t stream);
hipError_t launch_expand_valid(const int32_t* vbs, int nkv_logical, int kv_ratio, int block_kv, int32_t* kv_valid,
                               hipStream_t stream);

constexpr int kWorklistMaxCnt = 8191;
// Largest CSR row length the forward kernels accept (rows are staged in LDS).
constexpr int kMaxIdxLd = 8191;
// Staged CSR entries pack the tile index (low kTileBits bits) with the
// number of invalid keys of a partial tile (the bits above), so a sequence
// may hold fewer than 2^kTileBits KV tiles.
constexpr int kTileBits = 22;
constexpr int kMaxTilesPartial = 1 << kTileBits;

}  // namespace vsa
