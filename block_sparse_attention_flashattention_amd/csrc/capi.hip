// C ABI of libvsa_attn.so: argument validation, dispatch and the per-device
// work-list buffer. The operations are specified in include/vsa_attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "vsa_attn.h"
#include "vsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
    return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

#define VSA_REQUIRE(cond, code, ...)          \
    do {                                      \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

// Validation shared by both forward entry points.
int32_t check_fwd(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* cnt,
                  const int32_t* kv_valid, int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim,
                  int32_t idx_ld, int32_t block_q, int32_t block_kv, float scale, const void* o, const float* lse) {
    VSA_REQUIRE(q && k && v && idx && cnt && o && lse, VSA_ERR_INVALID_ARG, "null tensor pointer");
    VSA_REQUIRE(batch >= 1 && seqlen >= 1 && heads >= 1 && head_dim >= 1, VSA_ERR_INVALID_ARG,
                "batch, seqlen, heads and head_dim must be >= 1");
    VSA_REQUIRE(block_q >= 1 && block_kv >= 1, VSA_ERR_INVALID_ARG, "block sizes must be >= 1");
    VSA_REQUIRE(seqlen % block_q == 0 && seqlen % block_kv == 0, VSA_ERR_INVALID_ARG,
                "seqlen %d must be divisible by block_q %d and block_kv %d", seqlen, block_q, block_kv);
    VSA_REQUIRE(idx_ld >= 1, VSA_ERR_INVALID_ARG, "idx_ld must be >= 1");
    VSA_REQUIRE(idx_ld <= vsa::kMaxIdxLd, VSA_ERR_UNSUPPORTED, "idx_ld %d exceeds the supported maximum %d", idx_ld,
                vsa::kMaxIdxLd);
    VSA_REQUIRE(isfinite(scale) && scale > 0.0f, VSA_ERR_INVALID_ARG, "scale must be finite and > 0");
    VSA_REQUIRE(vsa::fwd_supported(block_q, block_kv, head_dim), VSA_ERR_UNSUPPORTED,
                "no kernel for block_q=%d block_kv=%d head_dim=%d (supported: block_q in {64,128,256}, "
                "block_kv in {64,128}, head_dim in {64,128})",
                block_q, block_kv, head_dim);
    VSA_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(o, 16), VSA_ERR_INVALID_ARG,
                "q, k, v, o must be 16-byte aligned");
    VSA_REQUIRE(aligned(lse, 4) && aligned(idx, 4) && aligned(cnt, 4), VSA_ERR_INVALID_ARG,
                "lse, kv_block_idx, kv_block_cnt must be 4-byte aligned");
    const int64_t n_items = (int64_t)batch * heads * (seqlen / block_q);
    VSA_REQUIRE(n_items <= INT32_MAX, VSA_ERR_INVALID_ARG, "batch*heads*seqlen/block_q exceeds int32");
    VSA_REQUIRE((int64_t)batch * seqlen <= INT32_MAX, VSA_ERR_INVALID_ARG, "batch*seqlen exceeds int32");
    VSA_REQUIRE(seqlen / block_kv < vsa::kMaxTilesPartial, VSA_ERR_UNSUPPORTED,
                "seqlen/block_kv must be below %d KV tiles", vsa::kMaxTilesPartial);
    VSA_REQUIRE(aligned(kv_valid, 4), VSA_ERR_INVALID_ARG, "kv_valid must be 4-byte aligned");
    return VSA_OK;
}

vsa::FwdParams make_params(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* cnt,
                           const int32_t* kv_valid, int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim,
                           int32_t idx_ld, int32_t block_q, int32_t block_kv, float scale, const int32_t* work,
                           int32_t n_work, void* o, float* lse) {
    vsa::FwdParams p;
    p.q = (const uint16_t*)q;
    p.k = (const uint16_t*)k;
    p.v = (const uint16_t*)v;
    p.idx = idx;
    p.cnt = cnt;
    p.work = work;
    p.kv_valid = kv_valid;
    p.o = (uint16_t*)o;
    p.lse = lse;
    p.n_work = n_work;
    p.S = seqlen;
    p.H = heads;
    p.nq = seqlen / block_q;
    p.nkv = seqlen / block_kv;
    p.ld = idx_ld;
    p.block_kv = block_kv;
    p.n_items = batch * heads * p.nq;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    p.splits = 1;
    p.ws_counter = nullptr;
    p.ws_partial = nullptr;
    // contiguous [B, S, H, D]
    const int64_t hs = head_dim, ts = (int64_t)heads * head_dim, bs = (int64_t)seqlen * ts;
    for (int64_t* x : {p.qs, p.ks, p.vs}) {
        x[0] = bs;
        x[1] = ts;
        x[2] = hs;
    }
    return p;
}

// Strides of vsa_attn_fwd_strided (q, k, v: batch, token, head, in elements):
// every row must start on a 16-byte boundary, a row stride must fit the
// kernels' 32-bit row offsets, and rows of one tensor must not overlap.
int32_t check_strides(const int64_t* s, int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim,
                      int n_tensors = 3) {
    VSA_REQUIRE(s, VSA_ERR_INVALID_ARG, "null stride array");
    const char* name[4] = {"q", "k", "v", "dout"};
    for (int t = 0; t < n_tensors; ++t) {
        const int64_t bs = s[3 * t], ts = s[3 * t + 1], hs = s[3 * t + 2];
        VSA_REQUIRE(bs >= 0 && ts >= 0 && hs >= 0, VSA_ERR_INVALID_ARG, "%s strides must be >= 0", name[t]);
        VSA_REQUIRE(bs % 8 == 0 && ts % 8 == 0 && hs % 8 == 0, VSA_ERR_INVALID_ARG,
                    "%s strides (%lld, %lld, %lld) must be multiples of 8 elements (16 bytes)", name[t],
                    (long long)bs, (long long)ts, (long long)hs);
        VSA_REQUIRE(ts <= ((int64_t)1 << 24), VSA_ERR_UNSUPPORTED, "%s token stride %lld exceeds 2^24", name[t],
                    (long long)ts);
        // No order or overlap is required of the three strides: the tensors
        // are only read, so a [batch, heads, seqlen, head_dim] buffer seen as
        // [B, S, H, D] (token stride head_dim) and K, V broadcast over the
        // heads (head stride 0) are fine.
    }
    (void)batch;
    (void)seqlen;
    (void)heads;
    (void)head_dim;
    return VSA_OK;
}

// Library-owned device buffers, one per (device, stream, purpose), grown on
// demand. Keying by stream lets calls on different streams run at the same
// time; calls on one stream are ordered by it. A buffer that is too small is
// replaced by a larger one, and the old one is kept until vsa_release
// (freeing it here would wait for the device).
enum BufKind : int { kBufWork = 0, kBufBwd, kBufPair, kBufCoal, kBufSplit, kBufBwdSplit };
struct DeviceBuffer {
    void* ptr = nullptr;
    size_t bytes = 0;
    size_t zeroed = 0;  // split workspaces: leading bytes known to hold zero counters
};
std::mutex g_buf_mutex;
std::map<std::tuple<int, uintptr_t, int>, DeviceBuffer> g_bufs;
std::vector<void*> g_retired;  // superseded buffers, freed by vsa_release

int32_t stream_buffer_locked(int kind, hipStream_t stream, size_t bytes, DeviceBuffer** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    DeviceBuffer& b = g_bufs[std::make_tuple(dev, (uintptr_t)stream, kind)];
    if (b.bytes < bytes) {
        // grow by at least a quarter, in 64 KiB steps, so that slowly growing
        // calls do not replace the buffer every time
        size_t want = bytes > b.bytes + b.bytes / 4 ? bytes : b.bytes + b.bytes / 4;
        want = (want + 65535) / 65536 * 65536;
        void* p = nullptr;
        e = hipMalloc(&p, want);
        if (e != hipSuccess) return hip_fail(e, "hipMalloc(library buffer)");
        if (b.ptr) g_retired.push_back(b.ptr);
        b.ptr = p;
        b.bytes = want;
        b.zeroed = 0;
    }
    *out = &b;
    return VSA_OK;
}

int32_t stream_buffer(int kind, hipStream_t stream, size_t bytes, void** out) {
    std::lock_guard<std::mutex> lock(g_buf_mutex);
    DeviceBuffer* b = nullptr;
    const int32_t rc = stream_buffer_locked(kind, stream, bytes, &b);
    if (rc == VSA_OK) *out = b->ptr;
    return rc;
}

// Workspace of a split-list launch: counter_bytes of per-item counters
// followed by the partial states. The kernels return every counter they use
// to 0, but the bytes past the previous call's counters held partial states,
// so the counters are cleared (by a kernel, on the stream) whenever they
// reach beyond the bytes known to be zero (a new buffer holds none).
std::atomic<int32_t> g_max_splits{4};  // vsa_set_max_splits
int32_t split_buffer(int kind, size_t counter_bytes, size_t bytes, hipStream_t stream, void** out) {
    std::lock_guard<std::mutex> lock(g_buf_mutex);
    DeviceBuffer* b = nullptr;
    int32_t rc = stream_buffer_locked(kind, stream, bytes, &b);
    if (rc != VSA_OK) return rc;
    if (b->zeroed < counter_bytes) {
        const hipError_t e = vsa::launch_fill_zero((int32_t*)b->ptr, (int64_t)(counter_bytes / 4), stream);
        if (e != hipSuccess) return hip_fail(e, "split counter clear launch");
    }
    b->zeroed = counter_bytes;  // past them the partial states are written
    *out = b->ptr;
    return VSA_OK;
}

// Split choice and workspace layout of one vsa_attn_fwd call: with too few
// work items to occupy every compute unit, each list is split over 2 or 4
// workgroups (partial states merged by the last one). 256-row tiles run one
// workgroup per compute unit; 64-row tiles go to the independent-wave
// kernel, four per compute unit. (128-row tiles with few items measured
// faster on the two-stream kernel unsplit.)
struct FwdSplit {
    int splits = 1;
    size_t counter_bytes = 0;  // one int32 per item, padded to 256 bytes
    size_t partial_bytes = 0;  // partial (O, max, sum) states of every part
};
FwdSplit plan_split(int64_t n_items, int block_q, int head_dim, int max_splits) {
    FwdSplit f;
    const int cus = vsa::device_cu_count();
    if (block_q == 256) {
        while (f.splits < max_splits && n_items * f.splits * 2 <= cus) f.splits *= 2;
    } else if (block_q == 64 && n_items < (int64_t)vsa::kIwItemsPerCu * cus) {
        while (f.splits < max_splits && n_items * f.splits < 4LL * cus) f.splits *= 2;
    }
    if (f.splits > 1) {
        f.counter_bytes = ((size_t)n_items * sizeof(int32_t) + 255) / 256 * 256;
        const size_t state_words = (size_t)(head_dim / 32 * 16 + 2) * 64;  // per wave
        f.partial_bytes = (size_t)n_items * f.splits * (block_q / 32) * state_words * sizeof(float);
    }
    return f;
}

// Scratch of vsa_attn_fwd_noalloc: one copy per device, held until the
// process ends. Layout: [counters | work list | partial states]; the counter
// region is only ever written by split launches, which leave every counter
// they use at zero, so it is cleared once per device.
constexpr size_t kScratchBytes = 16u << 20;
constexpr size_t kScratchCounterBytes = 256u << 10;
static __device__ __align__(256) char scratch[kScratchBytes];
struct ScratchState {
    char* ptr = nullptr;        // device address of this device's copy of `scratch`
    bool counters_zero = false; // a clearing launch has been enqueued outside graph capture
};
std::vector<ScratchState> g_scratch;  // per device, under g_buf_mutex

int32_t scratch_for_device(hipStream_t stream, char** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_buf_mutex);
    if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1);
    ScratchState& s = g_scratch[dev];
    if (s.ptr == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        s.ptr = (char*)p;
    }
    if (!s.counters_zero) {
        // Under graph capture the clearing kernel becomes part of the graph
        // (and runs at every replay), so it is enqueued again next time.
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
        e = vsa::launch_fill_zero((int32_t*)s.ptr, (int64_t)(kScratchCounterBytes / 4), stream);
        if (e != hipSuccess) return hip_fail(e, "scratch counter clear launch");
        if (cap == hipStreamCaptureStatusNone) s.counters_zero = true;
    }
    *out = s.ptr;
    return VSA_OK;
}

// The body shared by vsa_attn_fwd and vsa_attn_fwd_noalloc: the work list
// (count-sorted within each batch and head) into `work`, then the kernel,
// with split lists over `counters` / `partial` when splits > 1.
int32_t run_fwd(const void* q, const void* k, const void* v, const int32_t* idx, const int32_t* cnt,
                const int32_t* kv_valid, int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim,
                int32_t idx_ld, int32_t block_q, int32_t block_kv, float scale, void* o, float* lse, hipStream_t st,
                int32_t* work, int splits, int32_t* counters, float* partial, const int64_t* strides = nullptr) {
    const int32_t n_items = batch * heads * (seqlen / block_q);
    // one segment per (batch, head): heads stay contiguous in the list
    hipError_t e = vsa::launch_build_worklist(cnt, n_items, seqlen / block_q, idx_ld, work, st);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    vsa::FwdParams p = make_params(q, k, v, idx, cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, block_q,
                                   block_kv, scale, work, n_items, o, lse);
    if (strides) {
        for (int i = 0; i < 3; ++i) {
            p.qs[i] = strides[i];
            p.ks[i] = strides[3 + i];
            p.vs[i] = strides[6 + i];
        }
    }
    if (splits > 1) {
        p.splits = splits;
        p.ws_counter = counters;
        p.ws_partial = partial;
        p.n_work = n_items * splits;
    }
    e = vsa::launch_fwd(block_q, block_kv, head_dim, p, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return VSA_OK;
}

}  // namespace

namespace vsa {
// Sustained MFMA rate and shader clock on random / zero operands, or beside
// softmax-shaped vector work (mode 0 / 1 / 2; measure.hip). Synchronises.
hipError_t measure_mfma(int mode, int iters, hipStream_t stream, float* tflops, float* clock_mhz);
}  // namespace vsa

extern "C" {

int32_t vsa_abi_version(void) { return 12; }

int32_t vsa_set_max_splits(int32_t max_splits) {
    const int32_t m = max_splits >= 4 ? 4 : (max_splits >= 2 ? 2 : 1);
    return g_max_splits.exchange(m);
}

int32_t vsa_measure_mfma(int32_t mode, int32_t iters, float* tflops, float* clock_mhz, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(tflops && clock_mhz, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(mode >= 0 && mode <= 2, VSA_ERR_INVALID_ARG, "mode must be 0, 1 or 2");
    VSA_REQUIRE(iters >= 1 && iters <= 2000000, VSA_ERR_INVALID_ARG, "iters must be in [1, 2000000]");
    const hipError_t e = vsa::measure_mfma(mode, iters, (hipStream_t)stream, tflops, clock_mhz);
    if (e != hipSuccess) return hip_fail(e, "MFMA rate measurement");
    return VSA_OK;
}

const char* vsa_status_string(int32_t status) {
    switch (status) {
        case VSA_OK: return "VSA_OK";
        case VSA_ERR_INVALID_ARG: return "VSA_ERR_INVALID_ARG";
        case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
        case VSA_ERR_HIP: return "VSA_ERR_HIP";
        default: return "VSA_ERR_UNKNOWN";
    }
}

const char* vsa_last_error(void) { return g_last_error; }

int32_t vsa_mask_to_csr(const uint8_t* mask, int32_t batch, int32_t heads, int32_t nq_logical, int32_t nkv_logical,
                        int32_t logical_block_q, int32_t logical_block_kv, int32_t block_q, int32_t block_kv,
                        const int32_t* kv_valid, int32_t* kv_block_idx, int32_t idx_ld, int32_t* kv_block_cnt,
                        int32_t* overflow, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(mask && kv_block_idx && kv_block_cnt, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(batch >= 1 && heads >= 1 && nq_logical >= 1 && nkv_logical >= 1, VSA_ERR_INVALID_ARG,
                "batch, heads, nq_logical, nkv_logical must be >= 1");
    VSA_REQUIRE(logical_block_q >= 1 && logical_block_kv >= 1 && block_q >= 1 && block_kv >= 1,
                VSA_ERR_INVALID_ARG, "block sizes must be >= 1");
    VSA_REQUIRE(logical_block_q % block_q == 0 && logical_block_kv % block_kv == 0, VSA_ERR_INVALID_ARG,
                "physical tile %dx%d must divide the logical block %dx%d", block_q, block_kv, logical_block_q,
                logical_block_kv);
    VSA_REQUIRE((int64_t)nq_logical * logical_block_q == (int64_t)nkv_logical * logical_block_kv,
                VSA_ERR_INVALID_ARG, "query and key sequence lengths differ");
    VSA_REQUIRE(idx_ld >= 1, VSA_ERR_INVALID_ARG, "idx_ld must be >= 1");
    VSA_REQUIRE(aligned(kv_block_idx, 4) && aligned(kv_block_cnt, 4) && aligned(overflow, 4) && aligned(kv_valid, 4),
                VSA_ERR_INVALID_ARG, "index buffers and kv_valid must be 4-byte aligned");
    const int64_t q_ratio = logical_block_q / block_q, kv_ratio = logical_block_kv / block_kv;
    const int64_t nq_phys = (int64_t)nq_logical * q_ratio;
    const int64_t rows = (int64_t)batch * heads * nq_phys;
    VSA_REQUIRE(rows <= INT32_MAX / 4 && (int64_t)nkv_logical * kv_ratio <= INT32_MAX, VSA_ERR_INVALID_ARG,
                "problem too large");
    hipError_t e = vsa::launch_mask_to_csr(mask, batch, heads, nq_logical, nkv_logical, (int)q_ratio, (int)kv_ratio,
                                           (int)nq_phys, kv_valid, kv_block_idx, idx_ld, kv_block_cnt, overflow,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mask_to_csr launch");
    return VSA_OK;
}

int32_t vsa_build_worklist(const int32_t* kv_block_cnt, int32_t n_items, int32_t segment, int32_t max_cnt,
                           int32_t* work_list, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(n_items >= 0, VSA_ERR_INVALID_ARG, "n_items must be >= 0");
    VSA_REQUIRE(segment >= 1 && (n_items == 0 || n_items % segment == 0), VSA_ERR_INVALID_ARG,
                "segment must be >= 1 and divide n_items");
    VSA_REQUIRE(max_cnt >= 0 && max_cnt <= vsa::kWorklistMaxCnt, VSA_ERR_INVALID_ARG, "max_cnt must be in [0, %d]",
                vsa::kWorklistMaxCnt);
    if (n_items == 0) return VSA_OK;
    VSA_REQUIRE(kv_block_cnt && work_list, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(aligned(kv_block_cnt, 4) && aligned(work_list, 4), VSA_ERR_INVALID_ARG, "buffers must be 4-byte aligned");
    hipError_t e = vsa::launch_build_worklist(kv_block_cnt, n_items, segment, max_cnt, work_list, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    return VSA_OK;
}

int32_t vsa_attn_fwd_worklist(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                              const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                              int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                              float scale, const int32_t* work_list, int32_t n_work, void* o, float* lse,
                              void* stream) {
    g_last_error[0] = 0;
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                           block_q, block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    VSA_REQUIRE(n_work >= 0, VSA_ERR_INVALID_ARG, "n_work must be >= 0");
    if (n_work == 0) return VSA_OK;
    VSA_REQUIRE(work_list && aligned(work_list, 4), VSA_ERR_INVALID_ARG, "work_list must be a 4-byte aligned pointer");
    vsa::FwdParams p = make_params(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim,
                                   idx_ld, block_q, block_kv, scale, work_list, n_work, o, lse);
    hipError_t e = vsa::launch_fwd(block_q, block_kv, head_dim, p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
    return VSA_OK;
}

int32_t vsa_attn_fwd(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                     const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                     int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv, float scale,
                     void* o, float* lse, void* stream) {
    return vsa_attn_fwd_strided(q, k, v, nullptr, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads,
                                head_dim, idx_ld, block_q, block_kv, scale, o, lse, stream);
}

int32_t vsa_attn_fwd_strided(const void* q, const void* k, const void* v, const int64_t* qkv_strides,
                             const int32_t* kv_block_idx, const int32_t* kv_block_cnt, const int32_t* kv_valid,
                             int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim, int32_t idx_ld,
                             int32_t block_q, int32_t block_kv, float scale, void* o, float* lse, void* stream) {
    g_last_error[0] = 0;
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                           block_q, block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    if (qkv_strides) {
        rc = check_strides(qkv_strides, batch, seqlen, heads, head_dim);
        if (rc != VSA_OK) return rc;
    }
    VSA_REQUIRE(idx_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED,
                "idx_ld %d exceeds the work-list sort limit %d; use vsa_attn_fwd_worklist", idx_ld,
                vsa::kWorklistMaxCnt);
    hipStream_t st = (hipStream_t)stream;
    const int32_t n_items = batch * heads * (seqlen / block_q);
    int32_t* work = nullptr;
    rc = stream_buffer(kBufWork, st, (size_t)n_items * sizeof(int32_t), (void**)&work);
    if (rc != VSA_OK) return rc;
    const FwdSplit f = plan_split(n_items, block_q, head_dim, g_max_splits.load());
    void* ws = nullptr;
    if (f.splits > 1) {
        rc = split_buffer(kBufSplit, f.counter_bytes, f.counter_bytes + f.partial_bytes, st, &ws);
        if (rc != VSA_OK) return rc;
    }
    return run_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, block_q,
                   block_kv, scale, o, lse, st, work, f.splits, (int32_t*)ws,
                   ws ? (float*)((char*)ws + f.counter_bytes) : nullptr, qkv_strides);
}

int32_t vsa_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                             const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                             int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                             float scale, void* o, float* lse, void* stream) {
    g_last_error[0] = 0;
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                           block_q, block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    VSA_REQUIRE(idx_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED,
                "idx_ld %d exceeds the work-list sort limit %d", idx_ld, vsa::kWorklistMaxCnt);
    const int64_t n_items = (int64_t)batch * heads * (seqlen / block_q);
    const size_t work_bytes = ((size_t)n_items * sizeof(int32_t) + 255) / 256 * 256;
    const size_t room = kScratchBytes - kScratchCounterBytes;
    VSA_REQUIRE(work_bytes <= room, VSA_ERR_UNSUPPORTED,
                "%lld work items need %zu bytes of scratch; vsa_attn_fwd_noalloc holds %zu (at most %zu items)",
                (long long)n_items, work_bytes, room, room / sizeof(int32_t));
    hipStream_t st = (hipStream_t)stream;
    char* base = nullptr;
    rc = scratch_for_device(st, &base);
    if (rc != VSA_OK) return rc;
    // Split as vsa_attn_fwd would, with fewer parts (or none) where the
    // partial states would not fit beside the work list.
    FwdSplit f = plan_split(n_items, block_q, head_dim, g_max_splits.load());
    while (f.splits > 1 && (f.counter_bytes > kScratchCounterBytes || f.partial_bytes > room - work_bytes)) {
        const int parts = f.splits / 2;
        f = plan_split(n_items, block_q, head_dim, parts);
    }
    int32_t* work = (int32_t*)(base + kScratchCounterBytes);
    float* partial = (float*)(base + kScratchCounterBytes + work_bytes);
    return run_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, block_q,
                   block_kv, scale, o, lse, st, work, f.splits, f.splits > 1 ? (int32_t*)base : nullptr,
                   f.splits > 1 ? partial : nullptr);
}

int32_t vsa_pair_q_tiles(const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t batch, int32_t heads,
                         int32_t nq, int32_t idx_ld, int32_t* paired_idx, int32_t* paired_cnt, int32_t* unpaired,
                         void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(kv_block_idx && kv_block_cnt && paired_idx && paired_cnt && unpaired, VSA_ERR_INVALID_ARG,
                "null pointer");
    VSA_REQUIRE(batch >= 1 && heads >= 1 && nq >= 2 && nq % 2 == 0, VSA_ERR_INVALID_ARG,
                "batch and heads must be >= 1 and nq a positive even number (got nq=%d)", nq);
    VSA_REQUIRE(idx_ld >= 1, VSA_ERR_INVALID_ARG, "idx_ld must be >= 1");
    VSA_REQUIRE((int64_t)batch * heads * nq * idx_ld <= INT32_MAX, VSA_ERR_INVALID_ARG, "problem too large");
    VSA_REQUIRE(aligned(kv_block_idx, 4) && aligned(kv_block_cnt, 4) && aligned(paired_idx, 4) &&
                    aligned(paired_cnt, 4) && aligned(unpaired, 4),
                VSA_ERR_INVALID_ARG, "index buffers must be 4-byte aligned");
    hipError_t e = vsa::launch_pair_q_tiles(kv_block_idx, kv_block_cnt, batch * heads * (nq / 2), idx_ld, paired_idx,
                                            paired_cnt, unpaired, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pair_q_tiles launch");
    return VSA_OK;
}

int32_t vsa_attn_fwd_paired(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                            const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                            int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_kv, float scale, void* o,
                            float* lse, void* stream) {
    g_last_error[0] = 0;
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, 64,
                           block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    VSA_REQUIRE(idx_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED, "idx_ld %d exceeds the work-list sort limit %d",
                idx_ld, vsa::kWorklistMaxCnt);
    if (seqlen % 128 != 0 || !vsa::fwd_supported(128, block_kv, head_dim))  // nothing to pair
        return vsa_attn_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, 64,
                            block_kv, scale, o, lse, stream);
    const int nq = seqlen / 64;
    const int64_t n_items = (int64_t)batch * heads * nq, n_pairs = n_items / 2;
    // [unpaired, pad to 256 B][paired cnt][work 128][work 64][paired idx]
    const size_t words = 64 + (size_t)n_pairs * 2 + (size_t)n_items + (size_t)n_pairs * idx_ld;
    void* buf = nullptr;
    rc = stream_buffer(kBufPair, (hipStream_t)stream, words * sizeof(int32_t), &buf);
    if (rc != VSA_OK) return rc;
    int32_t* unpaired = (int32_t*)buf;
    int32_t* pcnt = unpaired + 64;
    int32_t* work128 = pcnt + n_pairs;
    int32_t* work64 = work128 + n_pairs;
    int32_t* pidx = work64 + n_items;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = vsa::launch_pair_q_tiles(kv_block_idx, kv_block_cnt, (int)n_pairs, idx_ld, pidx, pcnt, unpaired, st);
    if (e != hipSuccess) return hip_fail(e, "pair_q_tiles launch");
    // Exactly one of the two schedules gets a non-empty work list: the
    // 128-row one if every pair agrees, else the native 64-row one.
    e = vsa::launch_build_worklist(pcnt, (int)n_pairs, nq / 2, idx_ld, work128, st, unpaired, true);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    e = vsa::launch_build_worklist(kv_block_cnt, (int)n_items, nq, idx_ld, work64, st, unpaired, false);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    vsa::FwdParams p128 = make_params(q, k, v, pidx, pcnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld, 128,
                                      block_kv, scale, work128, (int32_t)n_pairs, o, lse);
    e = vsa::launch_fwd(128, block_kv, head_dim, p128, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch (128-row tiles)");
    vsa::FwdParams p64 = make_params(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim,
                                     idx_ld, 64, block_kv, scale, work64, (int32_t)n_items, o, lse);
    e = vsa::launch_fwd(64, block_kv, head_dim, p64, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch (64-row tiles)");
    return VSA_OK;
}

int32_t vsa_attn_fwd_coalesced(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                               const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                               int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                               float scale, void* o, float* lse, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(block_q == 64 || block_q == 128, VSA_ERR_UNSUPPORTED,
                "vsa_attn_fwd_coalesced takes block_q 64 or 128 (got %d)", block_q);
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                           block_q, block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    VSA_REQUIRE(idx_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED, "idx_ld %d exceeds the work-list sort limit %d",
                idx_ld, vsa::kWorklistMaxCnt);
    if (seqlen % 256 != 0) {  // no 256-row tiles
        if (block_q == 64)
            return vsa_attn_fwd_paired(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim,
                                       idx_ld, block_kv, scale, o, lse, stream);
        return vsa_attn_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                            block_q, block_kv, scale, o, lse, stream);
    }
    const int nq = seqlen / block_q;
    const int64_t n_items = (int64_t)batch * heads * nq;
    const int64_t n128 = block_q == 64 ? n_items / 2 : n_items;  // 128-row tiles
    const int64_t n256 = n128 / 2;                                // 256-row tiles
    // [a, b, gate256, gate128, pad to 256 B][cnt128][idx128][cnt256][idx256][work256][work128][work64]
    // (cnt128 / idx128 only when pairing from 64 rows)
    const size_t words = 64 + (block_q == 64 ? (size_t)n128 * (1 + idx_ld) : 0) + (size_t)n256 * (1 + idx_ld) +
                         (size_t)n256 + (size_t)n128 + (block_q == 64 ? (size_t)n_items : 0);
    void* buf = nullptr;
    rc = stream_buffer(kBufCoal, (hipStream_t)stream, words * sizeof(int32_t), &buf);
    if (rc != VSA_OK) return rc;
    int32_t* ctr_a = (int32_t*)buf;
    int32_t* ctr_b = ctr_a + 1;
    int32_t* gate256 = ctr_a + 2;
    int32_t* gate128 = ctr_a + 3;
    int32_t* w = ctr_a + 64;
    const int32_t *idx128 = kv_block_idx, *cnt128 = kv_block_cnt;  // the 128-row CSR
    if (block_q == 64) {
        cnt128 = w;
        idx128 = w + n128;
        w += (size_t)n128 * (1 + idx_ld);
    }
    int32_t* cnt256 = w;
    int32_t* idx256 = w + n256;
    w += (size_t)n256 * (1 + idx_ld);
    int32_t* work256 = w;
    int32_t* work128 = work256 + n256;
    int32_t* work64 = work128 + n128;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (block_q == 64) {
        // level 1 (64 -> 128 rows) counts into a, level 2 (128 -> 256) into b
        e = vsa::launch_pair_q_tiles(kv_block_idx, kv_block_cnt, (int)n128, idx_ld, (int32_t*)idx128,
                                     (int32_t*)cnt128, ctr_a, st);
        if (e != hipSuccess) return hip_fail(e, "pair_q_tiles launch");
        e = vsa::launch_pair_q_tiles(idx128, cnt128, (int)n256, idx_ld, idx256, cnt256, ctr_b, st);
        if (e != hipSuccess) return hip_fail(e, "pair_q_tiles launch");
        e = vsa::launch_pair_gates(ctr_a, ctr_b, gate256, gate128, st);
        if (e != hipSuccess) return hip_fail(e, "pair gates launch");
    } else {
        e = vsa::launch_pair_q_tiles(kv_block_idx, kv_block_cnt, (int)n256, idx_ld, idx256, cnt256, ctr_a, st);
        if (e != hipSuccess) return hip_fail(e, "pair_q_tiles launch");
    }
    // exactly one schedule gets a non-empty work list
    e = vsa::launch_build_worklist(cnt256, (int)n256, seqlen / 256, idx_ld, work256, st,
                                   block_q == 64 ? gate256 : ctr_a, true);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    e = vsa::launch_build_worklist(cnt128, (int)n128, seqlen / 128, idx_ld, work128, st,
                                   block_q == 64 ? gate128 : ctr_a, block_q == 64);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    if (block_q == 64) {
        e = vsa::launch_build_worklist(kv_block_cnt, (int)n_items, nq, idx_ld, work64, st, ctr_a, false);
        if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    }
    vsa::FwdParams p256 = make_params(q, k, v, idx256, cnt256, kv_valid, batch, seqlen, heads, head_dim, idx_ld, 256,
                                      block_kv, scale, work256, (int32_t)n256, o, lse);
    e = vsa::launch_fwd(256, block_kv, head_dim, p256, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch (256-row tiles)");
    vsa::FwdParams p128 = make_params(q, k, v, idx128, cnt128, kv_valid, batch, seqlen, heads, head_dim, idx_ld, 128,
                                      block_kv, scale, work128, (int32_t)n128, o, lse);
    e = vsa::launch_fwd(128, block_kv, head_dim, p128, st);
    if (e != hipSuccess) return hip_fail(e, "attention kernel launch (128-row tiles)");
    if (block_q == 64) {
        vsa::FwdParams p64 = make_params(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads,
                                         head_dim, idx_ld, 64, block_kv, scale, work64, (int32_t)n_items, o, lse);
        e = vsa::launch_fwd(64, block_kv, head_dim, p64, st);
        if (e != hipSuccess) return hip_fail(e, "attention kernel launch (64-row tiles)");
    }
    return VSA_OK;
}

int32_t vsa_csr_transpose(const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t batch, int32_t heads,
                          int32_t nq, int32_t nkv, int32_t idx_ld, int32_t* q_block_idx, int32_t q_ld,
                          int32_t* q_block_cnt, int32_t* overflow, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(kv_block_idx && kv_block_cnt && q_block_idx && q_block_cnt, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(batch >= 1 && heads >= 1 && nq >= 1 && nkv >= 1, VSA_ERR_INVALID_ARG,
                "batch, heads, nq and nkv must be >= 1");
    VSA_REQUIRE(idx_ld >= 1 && q_ld >= 1, VSA_ERR_INVALID_ARG, "idx_ld and q_ld must be >= 1");
    VSA_REQUIRE(nq <= 32 * vsa::kTransposeMaxWords, VSA_ERR_UNSUPPORTED, "nq %d exceeds %d", nq,
                32 * vsa::kTransposeMaxWords);
    VSA_REQUIRE((int64_t)batch * heads * nq * idx_ld <= INT32_MAX &&
                    (int64_t)batch * heads * nkv * q_ld <= INT32_MAX && (int64_t)nq * idx_ld <= INT32_MAX,
                VSA_ERR_INVALID_ARG, "problem too large");
    VSA_REQUIRE(aligned(kv_block_idx, 4) && aligned(kv_block_cnt, 4) && aligned(q_block_idx, 4) &&
                    aligned(q_block_cnt, 4) && aligned(overflow, 4),
                VSA_ERR_INVALID_ARG, "index buffers must be 4-byte aligned");
    hipError_t e = vsa::launch_csr_transpose(kv_block_idx, kv_block_cnt, batch * heads, nq, nkv, idx_ld, q_block_idx,
                                             q_ld, q_block_cnt, overflow, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "csr_transpose launch");
    return VSA_OK;
}

int32_t vsa_expand_valid(const int32_t* vbs, int32_t nkv_logical, int32_t logical_block_kv, int32_t block_kv,
                         int32_t* kv_valid, void* stream) {
    g_last_error[0] = 0;
    VSA_REQUIRE(nkv_logical >= 0, VSA_ERR_INVALID_ARG, "nkv_logical must be >= 0");
    VSA_REQUIRE(logical_block_kv >= 1 && block_kv >= 1 && logical_block_kv % block_kv == 0, VSA_ERR_INVALID_ARG,
                "block_kv %d must divide logical_block_kv %d", block_kv, logical_block_kv);
    const int64_t n = (int64_t)nkv_logical * (logical_block_kv / block_kv);
    VSA_REQUIRE(n <= INT32_MAX, VSA_ERR_INVALID_ARG, "too many tiles");
    if (n == 0) return VSA_OK;
    VSA_REQUIRE(vbs && kv_valid, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(aligned(vbs, 4) && aligned(kv_valid, 4), VSA_ERR_INVALID_ARG, "buffers must be 4-byte aligned");
    hipError_t e = vsa::launch_expand_valid(vbs, nkv_logical, logical_block_kv / block_kv, block_kv, kv_valid,
                                            (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "expand_valid launch");
    return VSA_OK;
}

int32_t vsa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t idx_ld,
                     const int32_t* q_block_idx, const int32_t* q_block_cnt, int32_t q_ld, const int32_t* kv_valid,
                     int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim, int32_t block_q,
                     int32_t block_kv, float scale, void* dq, void* dk, void* dv, void* stream) {
    return vsa_attn_bwd_strided(q, k, v, o, lse, dout, nullptr, kv_block_idx, kv_block_cnt, idx_ld, q_block_idx,
                                q_block_cnt, q_ld, kv_valid, batch, seqlen, heads, head_dim, block_q, block_kv, scale,
                                dq, dk, dv, stream);
}

int32_t vsa_attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, const int64_t* strides, const int32_t* kv_block_idx,
                             const int32_t* kv_block_cnt, int32_t idx_ld, const int32_t* q_block_idx,
                             const int32_t* q_block_cnt, int32_t q_ld, const int32_t* kv_valid, int32_t batch,
                             int32_t seqlen, int32_t heads, int32_t head_dim, int32_t block_q, int32_t block_kv,
                             float scale, void* dq, void* dk, void* dv, void* stream) {
    g_last_error[0] = 0;
    int32_t rc = check_fwd(q, k, v, kv_block_idx, kv_block_cnt, kv_valid, batch, seqlen, heads, head_dim, idx_ld,
                           block_q, block_kv, scale, o, lse);
    if (rc != VSA_OK) return rc;
    if (strides) {
        rc = check_strides(strides, batch, seqlen, heads, head_dim, 4);
        if (rc != VSA_OK) return rc;
    }
    VSA_REQUIRE(dout && dq && dk && dv && q_block_idx && q_block_cnt, VSA_ERR_INVALID_ARG, "null pointer");
    VSA_REQUIRE(aligned(dout, 16) && aligned(dq, 16) && aligned(dk, 16) && aligned(dv, 16), VSA_ERR_INVALID_ARG,
                "dout, dq, dk, dv must be 16-byte aligned");
    VSA_REQUIRE(aligned(q_block_idx, 4) && aligned(q_block_cnt, 4), VSA_ERR_INVALID_ARG,
                "q_block_idx, q_block_cnt must be 4-byte aligned");
    VSA_REQUIRE(q_ld >= 1 && q_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED, "q_ld must be in [1, %d]",
                vsa::kWorklistMaxCnt);
    VSA_REQUIRE(idx_ld <= vsa::kWorklistMaxCnt, VSA_ERR_UNSUPPORTED, "idx_ld %d exceeds %d", idx_ld,
                vsa::kWorklistMaxCnt);
    VSA_REQUIRE(vsa::bwd_supported(block_q, block_kv, head_dim), VSA_ERR_UNSUPPORTED,
                "no backward kernel for block_q=%d block_kv=%d head_dim=%d", block_q, block_kv, head_dim);
    const int64_t rows = (int64_t)batch * heads * seqlen;
    const int32_t nq = seqlen / block_q, nkv = seqlen / block_kv;
    const int32_t items_q = batch * heads * nq, items_kv = batch * heads * nkv;
    void* buf = nullptr;
    rc = stream_buffer(kBufBwd, (hipStream_t)stream, (size_t)rows * 2 * sizeof(float) + ((size_t)items_q + items_kv) * sizeof(int32_t),
                       &buf);
    if (rc != VSA_OK) return rc;
    float* aux = (float*)buf;
    int32_t* work_q = (int32_t*)(aux + rows * 2);
    int32_t* work_kv = work_q + items_q;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = vsa::launch_build_worklist(kv_block_cnt, items_q, nq, idx_ld, work_q, st);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    e = vsa::launch_build_worklist(q_block_cnt, items_kv, nkv, q_ld, work_kv, st);
    if (e != hipSuccess) return hip_fail(e, "build_worklist launch");
    vsa::BwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (const uint16_t*)o;
    a.dout = (const uint16_t*)dout;
    a.strides = strides;
    a.lse = lse;
    a.aux = aux;
    a.idx = kv_block_idx;
    a.cnt = kv_block_cnt;
    a.qidx = q_block_idx;
    a.qcnt = q_block_cnt;
    a.kv_valid = kv_valid;
    a.work_q = work_q;
    a.work_kv = work_kv;
    a.dq = (uint16_t*)dq;
    a.dk = (uint16_t*)dk;
    a.dv = (uint16_t*)dv;
    a.B = batch;
    a.S = seqlen;
    a.H = heads;
    a.D = head_dim;
    a.ld = idx_ld;
    a.q_ld = q_ld;
    a.block_q = block_q;
    a.block_kv = block_kv;
    a.scale = scale;
    // Fewer work items than two waves per SIMD: split each list over 2 or 4
    // workgroups whose fp32 accumulators the last one sums (deterministic).
    const int64_t waves = 8LL * vsa::device_cu_count();
    const int max_splits = g_max_splits.load();
    while (a.splits_q < max_splits && (int64_t)items_q * a.splits_q * (block_q / 32) < waves) a.splits_q *= 2;
    while (a.splits_kv < max_splits && (int64_t)items_kv * a.splits_kv * (block_kv / 32) < waves) a.splits_kv *= 2;
    if (a.splits_q > 1 || a.splits_kv > 1) {
        const size_t cq = ((size_t)items_q * sizeof(int32_t) + 255) / 256 * 256;
        const size_t ckv = ((size_t)items_kv * sizeof(int32_t) + 255) / 256 * 256;
        const size_t wq = a.splits_q > 1 ? (size_t)items_q * a.splits_q * (block_q / 32) *
                                               vsa::bwd_split_words_q(head_dim) * sizeof(float)
                                         : 0;
        const size_t wkv = a.splits_kv > 1 ? (size_t)items_kv * a.splits_kv * (block_kv / 32) *
                                                 vsa::bwd_split_words_kv(head_dim) * sizeof(float)
                                           : 0;
        void* ws = nullptr;
        rc = split_buffer(kBufBwdSplit, cq + ckv, cq + ckv + wq + wkv, st, &ws);
        if (rc != VSA_OK) return rc;
        a.ws_counter_q = (int32_t*)ws;
        a.ws_counter_kv = (int32_t*)((char*)ws + cq);
        a.ws_q = (float*)((char*)ws + cq + ckv);
        a.ws_kv = (float*)((char*)ws + cq + ckv + wq);
    }
    e = vsa::launch_bwd(a, st);
    if (e != hipSuccess) return hip_fail(e, "backward kernel launch");
    return VSA_OK;
}

void vsa_release(void) {
    std::lock_guard<std::mutex> lock(g_buf_mutex);
    for (auto& kv : g_bufs)
        if (kv.second.ptr) (void)hipFree(kv.second.ptr);
    g_bufs.clear();
    for (void* p : g_retired) (void)hipFree(p);
    g_retired.clear();
}

}  // extern "C"
