/*
 * vsa_attn.h -- block-sparse attention (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libvsa_attn.so. Every entry point takes plain pointers and sizes;
 * no framework types cross this boundary.
 *
 * The operation (FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
 * benchmarks/bench_vsa_blackwell.py, functions ref_masked_sdpa_fp32 and
 * arm_fa4): for every batch b, head h and query token i,
 *
 *     A(i)  = union over selected KV tiles t of query tile floor(i/block_q)
 *             of the key tokens [t*block_kv, (t+1)*block_kv)
 *     O_i   = softmax_j in A(i) (scale * q_i . k_j) applied to v_j
 *     LSE_i = ln sum_{j in A(i)} exp(scale * q_i . k_j)
 *
 * Dense attention is the case where every query tile selects every KV tile.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 *  - Tensors are dense, row-major and contiguous (vsa_attn_fwd_strided and
 *    vsa_attn_bwd_strided also take q, k, v and dout as strided views):
 *      q, k, v, o      [batch, seqlen, heads, head_dim]  bf16 (raw 16-bit)
 *      lse             [batch, heads, seqlen]            fp32
 *      kv_block_idx    [batch, heads, seqlen/block_q, idx_ld]  int32
 *      kv_block_cnt    [batch, heads, seqlen/block_q]          int32
 *    This is the per-query-tile list form of FA4's block-sparse tensors
 *    (FastVideo page, fa4 block_sparsity.py, BlockSparseTensorsTorch full_block_cnt /
 *    full_block_idx, including the "compact" last dimension idx_ld that
 *    only needs to hold the largest count).
 *  - Pointers named in a signature are DEVICE pointers unless stated. The
 *    caller owns every buffer; the library never frees or retains them.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream). All
 *    GPU work is enqueued asynchronously on it; no call synchronises the
 *    host with the device.
 *  - Every call works on the calling thread's current HIP device
 *    (hipSetDevice); the stream and every device pointer must belong to it.
 *  - Library-owned scratch (work lists, split workspaces, the backward's
 *    per-row terms) is kept per device AND per stream: calls on different
 *    streams never share it and may run at the same time; calls on one
 *    stream are ordered by it. A buffer that must grow is replaced with
 *    hipMalloc; the old one is not freed (hipFree would wait for the device)
 *    but kept until vsa_release. Buffers are keyed by the stream handle, so
 *    a stream destroyed while its work still runs must not be followed by a
 *    new stream that reuses its handle before that work ends.
 *  - Arguments are validated on the host before anything is launched. A
 *    call returns VSA_OK, or a negative vsa_status_t and enqueues nothing.
 *    vsa_last_error() then returns a message naming the failed check.
 *  - Device-data contract: row (b,h,p) uses kv_block_idx entries
 *    [0, min(cnt, idx_ld)); entries must be distinct tile indices in
 *    [0, seqlen/block_kv), in any order. Kernels never read outside
 *    [0, idx_ld) and skip tile indices outside [0, seqlen/block_kv) rather
 *    than read out of bounds; a row with count 0 yields O = 0 and
 *    LSE = -inf (as the split-KV epilogue on page
 *    "BlackwellMultiHeadLatentAttentionForwardFP8", write_empty_output).
 *    Duplicate entries are counted twice.
 *  - Partial tiles (optional): kv_valid [seqlen/block_kv] int32, shared by
 *    every batch and head, gives the number of valid leading key tokens of
 *    each KV tile; the rest of the tile is padding that no query attends to.
 *    This is the per-block valid size `vbs` of the FastVideo page's VSA
 *    wrapper (block_sparse_attn_256_bshd(q, k, v, mask, vbs)), per physical
 *    tile (see vsa_expand_valid). NULL means every tile is full. Values are
 *    clamped to [0, block_kv]; a query row left with no valid key gets O = 0
 *    and LSE = -inf.
 */
#ifndef VSA_ATTN_H
#define VSA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VSA_OK = 0,
    VSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, non-divisible shape */
    VSA_ERR_UNSUPPORTED = -2, /* valid but not implemented (tile shape, head_dim) */
    VSA_ERR_HIP = -3          /* a HIP runtime call or kernel launch failed */
} vsa_status_t;

/* Version of this ABI; bumped on any signature change. */
int32_t vsa_abi_version(void);

/* Static string for a status code. */
const char* vsa_status_string(int32_t status);

/* Message of the last failed call on the calling host thread ("" if none). */
const char* vsa_last_error(void);

/*
 * vsa_mask_to_csr -- mask front-end, step 1: exact expansion + block CSR.
 *
 * Source: FastVideo page, bench_vsa_blackwell.py, expand_exact256_mask (repeat every
 * logical row block_q-fold and column block_kv-fold, which keeps the
 * selected token pairs) and arm_fa4 (per physical Q tile, the ascending
 * indices of its selected physical KV tiles, and their count).
 *
 *   mask           [batch, heads, nq_logical, nkv_logical] uint8, nonzero =
 *                  selected; logical cells are logical_block_q x
 *                  logical_block_kv tokens.
 *   block_q/kv     physical tile shape; must divide the logical block sizes.
 *                  seqlen = nq_logical*logical_block_q must equal
 *                  nkv_logical*logical_block_kv.
 *   kv_valid       optional [seqlen/block_kv] int32 (may be NULL): valid
 *                  key tokens per physical KV tile, as passed to the forward
 *                  (see vsa_expand_valid). A selected tile with no valid key
 *                  (kv_valid <= 0) is left out of the list, so no kernel
 *                  fetches or multiplies it; the selected token pairs are
 *                  unchanged (such a tile has none).
 *   kv_block_idx   out [batch, heads, seqlen/block_q, idx_ld]: ascending
 *                  physical KV tile indices; slots past the count are not
 *                  written.
 *   kv_block_cnt   out [batch, heads, seqlen/block_q]: number of listed
 *                  physical KV tiles (the true count, even if > idx_ld).
 *   overflow       optional out (device int32, may be NULL): set to 1 if
 *                  any row's count exceeds idx_ld (that row then keeps only
 *                  its first idx_ld tiles); never cleared by this call.
 */
int32_t vsa_mask_to_csr(const uint8_t* mask, int32_t batch, int32_t heads, int32_t nq_logical,
                        int32_t nkv_logical, int32_t logical_block_q, int32_t logical_block_kv,
                        int32_t block_q, int32_t block_kv, const int32_t* kv_valid, int32_t* kv_block_idx,
                        int32_t idx_ld, int32_t* kv_block_cnt, int32_t* overflow, void* stream);

/*
 * vsa_build_worklist -- mask front-end, step 2: count-sorted work list.
 *
 * Source: page "BlackwellMultiHeadLatentAttentionForwardFP8" (persistent
 * tile scheduling over a device work list instead of a plain grid). The
 * order is longest-first for load balance, within segments: with
 * segment = nq (one segment per batch and head) each head's query tiles stay
 * together, so the K/V tiles they share stay cached; segment = n_items sorts
 * the whole list.
 *
 *   kv_block_cnt  [n_items] int32 (the flattened [batch, heads, nq] counts)
 *   segment       items per segment; must divide n_items
 *   max_cnt       counts are clamped to [0, max_cnt] for ordering (pass the
 *                 idx_ld the counts belong to); 0 <= max_cnt <= 8191.
 *   work_list     out [n_items] int32: entry i of segment s is the flat index
 *                 (b*heads + h)*nq + p of the segment's item with the i-th
 *                 largest clamped count; equal counts keep ascending index
 *                 order. Segments stay in ascending order. Deterministic.
 */
int32_t vsa_build_worklist(const int32_t* kv_block_cnt, int32_t n_items, int32_t segment, int32_t max_cnt,
                           int32_t* work_list, void* stream);

/*
 * vsa_csr_transpose -- Q-direction lists for the backward pass: for every KV
 * tile, the query tiles that select it (FastVideo page, FA4 block_sparsity.py,
 * normalize_block_sparse_config_bwd: the backward walks per-KV-tile lists of
 * query tiles, "transposed from forward").
 *
 *   kv_block_idx / kv_block_cnt  forward CSR [batch, heads, nq, idx_ld] /
 *                  [batch, heads, nq] (row m uses entries [0, min(cnt, idx_ld))).
 *   q_block_idx    out [batch, heads, nkv, q_ld]: ascending query tile indices;
 *                  slots past the count are not written.
 *   q_block_cnt    out [batch, heads, nkv]: the true count (even if > q_ld).
 *   overflow       optional out (device int32, may be NULL): set to 1 if a
 *                  count exceeds q_ld; never cleared by this call.
 *   Forward entries outside [0, nkv) are ignored. nq <= 524288.
 */
int32_t vsa_csr_transpose(const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t batch, int32_t heads,
                          int32_t nq, int32_t nkv, int32_t idx_ld, int32_t* q_block_idx, int32_t q_ld,
                          int32_t* q_block_cnt, int32_t* overflow, void* stream);

/*
 * vsa_expand_valid -- valid key tokens per physical KV tile from valid tokens
 * per logical KV block (the variable block sizes `vbs` of the FastVideo
 * page's VSA wrapper): a logical block of logical_block_kv positions holding
 * vbs[T] valid tokens first, then padding, splits into
 * logical_block_kv/block_kv physical tiles, tile r keeping
 * clamp(vbs[T] - r*block_kv, 0, block_kv) valid tokens.
 *
 *   vbs        [nkv_logical] int32, each in [0, logical_block_kv]
 *   kv_valid   out [nkv_logical * logical_block_kv / block_kv] int32
 *   block_kv must divide logical_block_kv.
 */
int32_t vsa_expand_valid(const int32_t* vbs, int32_t nkv_logical, int32_t logical_block_kv, int32_t block_kv,
                         int32_t* kv_valid, void* stream);

/*
 * vsa_attn_fwd -- fused block-sparse attention forward (O and LSE).
 *
 * Source: FastVideo page, bench_vsa_blackwell.py, ref_masked_sdpa_fp32 (what is
 * computed) and arm_fa4 / the _flash_attn_fwd call (the tile-list input and
 * outputs). Online softmax in base 2 with scale*log2(e) folded into one
 * multiply (page "BlackwellMultiHeadLatentAttentionForwardFP8", softmax
 * and correction warps). bf16 inputs, fp32 accumulation, bf16 O rounded to
 * nearest even, fp32 LSE in natural log.
 *
 *   block_q x block_kv in {64,128,256} x {64,128}; head_dim in {64, 128};
 *   seqlen divisible by both; seqlen/block_kv < 2^22; 0 < scale < inf;
 *   1 <= idx_ld <= 8191;
 *   kv_valid: NULL or per-tile valid key counts (see the conventions above).
 *   Kernels read the whole CSR row [0, idx_ld) of every listed query tile.
 *   Builds the work list (count-sorted within each batch and head, segment
 *   = seqlen/block_q) in a library-owned device buffer (one per device and
 *   stream, grown on demand, released by vsa_release) and then runs the
 *   kernel in that order; see vsa_attn_fwd_worklist for the kernel alone.
 *   With block_q = 256 and fewer than half as many query tiles as the GPU
 *   has compute units, or block_q = 64 and fewer than 8 query tiles per
 *   compute unit, each tile's list is split over 2 or 4 workgroups
 *   whose partial rows are merged with the log-sum-exp rule (page
 *   "BlackwellMultiHeadLatentAttentionForwardFP8", split-KV reduction):
 *   the last workgroup of a tile to finish merges all parts in part order,
 *   so results stay deterministic. This uses another library-owned buffer
 *   (per device and stream) of about 17 KB per 32 rows and part.
 */
int32_t vsa_attn_fwd(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                     const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                     int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                     float scale, void* o, float* lse, void* stream);

/*
 * vsa_attn_fwd_strided -- vsa_attn_fwd with q, k and v given as strided views
 * (for example the three slices of a packed QKV projection), read in place.
 *
 * Source: FastVideo page, arm_fa4 / the _flash_attn_fwd call, whose q, k, v
 * are tensors with their own strides.
 *
 *   qkv_strides: host array of 9 int64, the strides in elements of q, k and
 *   v in that order, each as (batch, token, head): row r of head h in batch
 *   b of q starts at element b*s[0] + r*s[1] + h*s[2], and its head_dim
 *   elements are contiguous. NULL = contiguous [B, S, H, D] (vsa_attn_fwd).
 *   Every stride is >= 0 and a multiple of 8 elements (rows start on 16-byte
 *   boundaries, as q, k, v must) and the token stride is at most 2^24
 *   elements; VSA_ERR_INVALID_ARG / VSA_ERR_UNSUPPORTED otherwise. The
 *   strides need no particular order and rows may coincide, since q, k and
 *   v are only read: a [batch, heads, seqlen, head_dim] buffer viewed as
 *   [B, S, H, D] (token stride head_dim, head stride seqlen*head_dim), and
 *   k, v broadcast over the heads (head stride 0: every query head attends
 *   to the same keys and values, as in multi-query attention) are both
 *   valid. Every row addressed must lie inside the caller's allocation. q, k
 *   and v may overlap one another; o and lse stay contiguous and must not
 *   overlap the inputs. Otherwise as vsa_attn_fwd: same kernels,
 *   work list, splits and buffers, and results bitwise equal to vsa_attn_fwd
 *   on contiguous copies of the same values.
 */
int32_t vsa_attn_fwd_strided(const void* q, const void* k, const void* v, const int64_t* qkv_strides,
                             const int32_t* kv_block_idx, const int32_t* kv_block_cnt, const int32_t* kv_valid,
                             int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim, int32_t idx_ld,
                             int32_t block_q, int32_t block_kv, float scale, void* o, float* lse, void* stream);

/*
 * vsa_attn_fwd_noalloc -- vsa_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc during a step.
 *
 * Same arguments, result and kernels as vsa_attn_fwd, but it never calls
 * hipMalloc or hipFree: the work list and split-list workspace live in a
 * fixed 16 MiB device array of the library (one copy per GPU, held until
 * the process ends). Limits: at most 4,128,768 work items
 * (batch*heads*seqlen/block_q), else VSA_ERR_UNSUPPORTED; a launch that
 * vsa_attn_fwd would split over more parts than the array's room for
 * partial states allows is split over fewer parts, or not at all (results
 * then differ from vsa_attn_fwd's by rounding only). Every call on one GPU
 * shares that GPU's array, whatever the stream: calls that overlap in time
 * on one GPU race and must be ordered by the caller (one stream, or events).
 * The first call on a GPU (outside graph capture) also enqueues a small
 * kernel that clears the array's counters; under capture that kernel is
 * part of the captured work.
 */
int32_t vsa_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                             const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                             int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                             float scale, void* o, float* lse, void* stream);

/*
 * vsa_attn_fwd_worklist -- the attention kernel alone, over a caller-built
 * work list (for example from vsa_build_worklist). Each entry is a flat
 * index (b*heads + h)*(seqlen/block_q) + p in [0, batch*heads*seqlen/block_q);
 * entries outside that range are skipped. Only the Q tiles listed are
 * written, once per listing. n_work >= 0.
 */
int32_t vsa_attn_fwd_worklist(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                              const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch,
                              int32_t seqlen, int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q,
                              int32_t block_kv, float scale, const int32_t* work_list, int32_t n_work, void* o,
                              float* lse, void* stream);

/*
 * vsa_pair_q_tiles -- pair query tiles (2p, 2p+1) onto tiles twice as tall.
 *
 * Source: FastVideo page, README of the fine-grained VSA kernels and the
 * notes of bench_vsa_blackwell.py: at the Q256 API boundary the Q64 children
 * of one logical row have identical KV lists and are paired onto the
 * physical Q128/KV64 schedule; distinct Q64 lists keep the native kernel.
 *
 *   kv_block_idx / kv_block_cnt   CSR of nq query tiles (nq even, >= 2)
 *   paired_idx     out [batch, heads, nq/2, idx_ld]: row p holds the first
 *                  min(count, idx_ld) entries of row 2p (slots past them
 *                  are not written)
 *   paired_cnt     out [batch, heads, nq/2]: the count of row 2p
 *   unpaired       out, one device int32: the number of pairs whose counts
 *                  or stored entries (compared in order) differ; written in
 *                  stream order, no host synchronisation.
 * The paired CSR selects the same token pairs as the input iff *unpaired
 * is 0.
 */
int32_t vsa_pair_q_tiles(const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t batch, int32_t heads,
                         int32_t nq, int32_t idx_ld, int32_t* paired_idx, int32_t* paired_cnt, int32_t* unpaired,
                         void* stream);

/*
 * vsa_attn_fwd_paired -- vsa_attn_fwd for a 64-row query tile CSR that runs
 * adjacent tiles as 128-row tiles when every pair has identical lists.
 *
 * Same arguments as vsa_attn_fwd with block_q = 64. The pairing
 * (vsa_pair_q_tiles) and the choice are made on the device: the 128-row
 * kernel runs over the paired CSR if every pair agrees, otherwise the
 * native 64-row kernel runs over the input; the other launch finds an empty
 * work list. Either way O and LSE are those of the input CSR (the 128-row
 * kernel splits each list over two streams instead of four, so the
 * rounding order differs). If seqlen is not a multiple of 128 this is
 * vsa_attn_fwd. Uses a library-owned device buffer (per device and stream)
 * of about 4*(batch*heads*seqlen/64)*(idx_ld/2 + 2) bytes.
 */
int32_t vsa_attn_fwd_paired(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                            const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                            int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_kv, float scale, void* o,
                            float* lse, void* stream);

/*
 * vsa_attn_fwd_coalesced -- vsa_attn_fwd for a 64- or 128-row query tile CSR
 * that runs adjacent tiles with identical lists as one tile up to 256 rows
 * tall.
 *
 * Source: as vsa_pair_q_tiles (FastVideo page, fine-grained VSA kernels:
 * the query-tile children of one Q256 logical row share their KV list and
 * are paired onto taller physical tiles), applied level by level up to the
 * Q256 row itself.
 *
 * Same arguments as vsa_attn_fwd, with block_q 64 or 128 (else
 * VSA_ERR_UNSUPPORTED). Pairing levels: 64 -> 128 -> 256 rows for
 * block_q = 64, 128 -> 256 for block_q = 128; a level applies only if every
 * pair of that level has equal counts and equal stored entries in order
 * (vsa_pair_q_tiles), so the selected token pairs never change. The levels
 * and the choice of schedule are made on the device: exactly one of the
 * 256-row, 128-row and (for block_q = 64) 64-row kernels gets a non-empty
 * work list. O and LSE are those of the input CSR; the per-row arithmetic
 * follows the kernel that runs (the 256-row and the many-entry 128-row
 * kernels run the same steps per row). If seqlen is not a multiple of 256
 * this is vsa_attn_fwd_paired (block_q 64) or vsa_attn_fwd (block_q 128).
 * Partial tiles (kv_valid) are supported as in vsa_attn_fwd. Uses a
 * library-owned device buffer (per device and stream) of about
 * 4*(batch*heads*seqlen/block_q)*(idx_ld + 3) bytes. idx_ld must not
 * exceed the work-list sort limit (8191).
 */
int32_t vsa_attn_fwd_coalesced(const void* q, const void* k, const void* v, const int32_t* kv_block_idx,
                               const int32_t* kv_block_cnt, const int32_t* kv_valid, int32_t batch, int32_t seqlen,
                               int32_t heads, int32_t head_dim, int32_t idx_ld, int32_t block_q, int32_t block_kv,
                               float scale, void* o, float* lse, void* stream);

/*
 * vsa_attn_bwd -- backward pass: dQ, dK and dV of vsa_attn_fwd.
 *
 * Source: the gradient of the FastVideo page's ref_masked_sdpa_fp32 (the function the
 * forward computes); the backward walks, per KV tile, the query tiles that
 * select it (FA4 block_sparsity.py, normalize_block_sparse_config_bwd). With
 * P recomputed from the forward's LSE, D_i = dO_i . O_i, dS = P (dO V^T - D):
 * dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K. Deterministic: dK and dV
 * of a KV tile accumulate in one workgroup over its query tiles in list
 * order, dQ of a query tile in one workgroup over its KV tiles in list order;
 * no floating-point atomics. bf16 in and out, fp32 accumulation. When the
 * query tiles (or KV tiles) number fewer than two waves per SIMD of the GPU,
 * each list is split over 2 or 4 workgroups (at most vsa_set_max_splits):
 * each publishes its fp32 partial sums, and the last to finish adds all
 * parts in part order, so results stay deterministic on a given GPU.
 *
 *   q, k, v, o, dout, dq, dk, dv   [batch, seqlen, heads, head_dim] bf16
 *                  (o: the forward output; dq, dk, dv written, every row)
 *   lse            [batch, heads, seqlen] fp32 from the forward
 *   kv_block_idx / kv_block_cnt / idx_ld   the forward CSR
 *   q_block_idx / q_block_cnt / q_ld       its transpose (vsa_csr_transpose)
 *   kv_valid       as for the forward (NULL: full tiles); padding keys get
 *                  dK = dV = 0
 *   Same shape limits as vsa_attn_fwd; q_ld, idx_ld <= 8191. Uses a
 *   library-owned device buffer of 8*batch*heads*seqlen bytes plus the work
 *   lists, and with split lists another of 4*head_dim bytes per token row and
 *   part for dQ and twice that for dK and dV (both per device and stream).
 *   Padding tokens of partial tiles must hold finite values.
 */
int32_t vsa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     const int32_t* kv_block_idx, const int32_t* kv_block_cnt, int32_t idx_ld,
                     const int32_t* q_block_idx, const int32_t* q_block_cnt, int32_t q_ld, const int32_t* kv_valid,
                     int32_t batch, int32_t seqlen, int32_t heads, int32_t head_dim, int32_t block_q,
                     int32_t block_kv, float scale, void* dq, void* dk, void* dv, void* stream);

/*
 * vsa_attn_bwd_strided -- vsa_attn_bwd with q, k, v and dout given as
 * strided views (for example the slices of a packed QKV projection, or
 * [batch, heads, seqlen, head_dim] tensors), read in place.
 *
 * Source: as vsa_attn_bwd; the pages' interface takes tensors with their own
 * strides (FastVideo page, arm_fa4 / _flash_attn_fwd).
 *
 *   strides: host array of 12 int64, the element strides of q, k, v and dout
 *   in that order, each as (batch, token, head), with the same meaning and
 *   limits as in vsa_attn_fwd_strided (>= 0, multiples of 8, token stride at
 *   most 2^24, any order, rows may coincide); NULL = all four contiguous
 *   (vsa_attn_bwd). o, lse, dq, dk and dv stay contiguous. Otherwise as
 *   vsa_attn_bwd: same kernels, buffers and split lists, and results bitwise
 *   equal to vsa_attn_bwd on contiguous copies of the same values. With k, v
 *   broadcast over the heads (head stride 0), dk and dv hold each head's
 *   gradient; their sum over the heads is the gradient of the shared tensor.
 */
int32_t vsa_attn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, const int64_t* strides, const int32_t* kv_block_idx,
                             const int32_t* kv_block_cnt, int32_t idx_ld, const int32_t* q_block_idx,
                             const int32_t* q_block_cnt, int32_t q_ld, const int32_t* kv_valid, int32_t batch,
                             int32_t seqlen, int32_t heads, int32_t head_dim, int32_t block_q, int32_t block_kv,
                             float scale, void* dq, void* dk, void* dv, void* stream);

/* Free the library-owned buffers (every device and stream, including the
 * ones superseded by growth). Must not run while library work is in flight
 * or another thread is inside a library call. The no-alloc array of
 * vsa_attn_fwd_noalloc is not affected. */
void vsa_release(void);

/*
 * vsa_set_max_splits -- the most parts (1, 2 or 4; other values are rounded
 * down to one of those, values below 2 give 1) into which vsa_attn_fwd and
 * vsa_attn_bwd may split a work item's list when a launch has too few work
 * items to fill the GPU. The default is 4. Whether a launch splits depends
 * on the GPU's compute unit count, and a split changes the fp32 summation
 * order, so 1 gives results that are bit-identical across GPU models (at
 * some speed when items are few). Process-wide; takes effect for calls that
 * start after it returns. Returns the previous value.
 */
int32_t vsa_set_max_splits(int32_t max_splits);

/*
 * vsa_measure_mfma -- a measurement aid for the roofline the forward is
 * reported against, not part of the attention operation: what this device's
 * matrix cores sustain on v_mfma_f32_32x32x16_bf16 when every compute unit
 * runs it back to back. Under such a load the shader clock is set by the
 * power the chip draws, which depends on the operand bits, so the published
 * dense peak (top clock) is not what bf16 data drawn like Q, K and V gets.
 *   mode 0: operands drawn from N(0,1) in bf16, two MFMA waves per SIMD;
 *   mode 1: all-zero operands, otherwise as mode 0;
 *   mode 2: per SIMD one wave issues the MFMAs of mode 0 while the other
 *           issues softmax-shaped vector work (fma, exp2, add, max, bf16
 *           pack; about 4.5 instructions per MFMA of its partner), the phase
 *           split of the forward kernels.
 * iters (1 .. 2,000,000) is the number of 8-MFMA iterations per MFMA wave
 * (200,000 take about 60 ms). Host outputs: *tflops = MFMA flops / elapsed
 * time between HIP events around the launch; *clock_mhz = the mean over
 * waves of shader cycles (s_memtime) per real time (s_memrealtime, 100 MHz).
 * Unlike every other entry point this call synchronises: it allocates and
 * frees two small device buffers and waits for the kernel on `stream`.
 * Returns VSA_OK, VSA_ERR_INVALID_ARG (null output, mode or iters out of
 * range) or VSA_ERR_HIP.
 */
int32_t vsa_measure_mfma(int32_t mode, int32_t iters, float* tflops, float* clock_mhz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_ATTN_H */
