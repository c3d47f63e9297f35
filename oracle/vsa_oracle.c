/*
 * Block-sparse masked SDPA oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct CPU implementation of the forward pass that
 * the GPU library computes. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library; the product
 * path never does. It shares no code with the GPU library.
 *
 * Definition followed (FastVideo page "[perf] Add fine-grained FA4 VSA
 * kernels", benchmarks/bench_vsa_blackwell.py, function ref_masked_sdpa_fp32):
 * per head, fp32 scores (Q K^T) * scale; every query token i may attend to the
 * key tokens of the KV tiles its Q tile selects (a boolean token mask made by
 * repeating the block mask over the tile sizes); unselected scores become
 * -inf; a row softmax; then the product with V. True fp32 arithmetic is used
 * (the page disables TF32 for this reference). Row log-sum-exp is the natural
 * log of the sum of exp over the same masked fp32 scores (cf. page
 * "BlackwellMultiHeadLatentAttentionForwardFP8", write_empty_output: a row
 * with no selected key gives O = 0 and LSE = -inf).
 *
 * Block mask input is the per-Q-tile list form used by FA4's block-sparse
 * interface (FastVideo page, fa4 block_sparsity.py, BlockSparseTensorsTorch full_block_*):
 * kv_block_idx [B,H,NQ,ld] int32 (row p uses entries [0, cnt)), kv_block_cnt
 * [B,H,NQ] int32. Entries may be in any order; they must be distinct and in
 * [0, S/block_kv).
 *
 * Partial tiles (optional kv_valid [S/block_kv] int32, shared by all batches
 * and heads): only the first kv_valid[t] key tokens of KV tile t exist, the
 * rest of the tile is padding that no query attends to. This is the variable
 * block size input `vbs` of the FastVideo page's VSA wrapper
 * (block_sparse_attn_256_bshd(q, k, v, mask, vbs)), stated per physical tile;
 * kv_valid = NULL means every tile is full. A query row whose selected tiles
 * hold no valid key is an empty row (O = 0, LSE = -inf).
 *
 * Evaluation order is fixed and independent of the tile shape: the selected
 * key tokens of a row are visited in ascending token order and every sum over
 * the head dimension runs d = 0..D-1. Hence two masks that select the same
 * token pairs (for example a 256x256 mask and its exact expansion to 128x64 or
 * 64x64 tiles) give bit-identical results.
 *
 * Built with plain gcc -O2 (no -ffast-math); OpenMP parallelises over rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_IDX_RANGE (-2)
#define ORACLE_ERR_IDX_DUP (-3)
#define ORACLE_ERR_CNT (-4)
#define ORACLE_ERR_NOMEM (-5)

static float bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * For one CSR row, allow[t] = number of leading key tokens of KV tile t the
 * row may attend to: 0 for tiles the row does not select, kv_valid[t] (or
 * the whole tile) for selected ones. Returns an error code.
 */
static int mark_tiles(const int32_t* idx_row, int32_t n, int32_t ld, int32_t nkv, const int32_t* kv_valid,
                      int32_t block_kv, int32_t* allow) {
    if (n < 0 || n > ld) return ORACLE_ERR_CNT;
    for (int32_t t = 0; t < nkv; ++t) allow[t] = -1;
    for (int32_t e = 0; e < n; ++e) {
        int32_t t = idx_row[e];
        if (t < 0 || t >= nkv) return ORACLE_ERR_IDX_RANGE;
        if (allow[t] >= 0) return ORACLE_ERR_IDX_DUP;
        allow[t] = kv_valid ? kv_valid[t] : block_kv;
    }
    for (int32_t t = 0; t < nkv; ++t)
        if (allow[t] < 0) allow[t] = 0;
    return ORACLE_OK;
}

/* May a query of this row attend to key token j? */
static int allowed(const int32_t* allow, int block_kv, int j) { return (j % block_kv) < allow[j / block_kv]; }

/* kv_valid entries must lie in [0, block_kv]. */
static int check_valid(const int32_t* kv_valid, int nkv, int block_kv) {
    if (!kv_valid) return ORACLE_OK;
    for (int t = 0; t < nkv; ++t)
        if (kv_valid[t] < 0 || kv_valid[t] > block_kv) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/*
 * Softmax weights of one query row over the key tokens (ascending order).
 * On return: s[j] holds the weight of key token j for every selected j, keys
 * that are not selected hold 0, *m the row max of the scores, *l the sum of
 * exp(score - max). Returns the number of selected keys.
 */
static int64_t row_weights(const uint16_t* q, const uint16_t* k, int S, int H, int D, int b, int h, int i,
                           const int32_t* allow, int nkv, int block_kv, float scale, float* qf, float* s,
                           float* m_out, float* l_out) {
    const int64_t tok = (int64_t)H * D;
    const uint16_t* qrow = q + ((int64_t)b * S + i) * tok + (int64_t)h * D;
    for (int d = 0; d < D; ++d) qf[d] = bf16_to_f32(qrow[d]);

    /* scores = (q . k) * scale over selected keys; masked keys -> -inf */
    float m = -INFINITY;
    int64_t nsel = 0;
    for (int t = 0; t < nkv; ++t) {
        for (int jj = 0; jj < block_kv; ++jj) {
            int j = t * block_kv + jj;
            if (!allowed(allow, block_kv, j)) {
                s[j] = -INFINITY;
                continue;
            }
            const uint16_t* krow = k + ((int64_t)b * S + j) * tok + (int64_t)h * D;
            float acc = 0.0f;
            for (int d = 0; d < D; ++d) acc += qf[d] * bf16_to_f32(krow[d]);
            s[j] = acc * scale;
            if (s[j] > m) m = s[j];
            ++nsel;
        }
    }
    /* softmax along the row: exp(s - max) / sum */
    float l = 0.0f;
    if (nsel > 0) {
        for (int j = 0; j < S; ++j) {
            if (!allowed(allow, block_kv, j)) {
                s[j] = 0.0f;
                continue;
            }
            s[j] = expf(s[j] - m);
            l += s[j];
        }
        for (int j = 0; j < S; ++j)
            if (allowed(allow, block_kv, j)) s[j] = s[j] / l;
    } else {
        for (int j = 0; j < S; ++j) s[j] = 0.0f;
    }
    *m_out = m;
    *l_out = l;
    return nsel;
}

/*
 * Forward pass for a list of query rows.
 *   q, k, v : bf16 bit patterns, [B, S, H, D] contiguous
 *   kv_block_idx / kv_block_cnt : block CSR at tile shape block_q x block_kv
 *   kv_valid : valid key tokens per KV tile [S/block_kv], or NULL (all full)
 *   rows    : flat row ids (b*H + h)*S + i, or NULL for all B*H*S rows in
 *             that order
 *   o       : [n_rows, D] fp32 output; lse : [n_rows] fp32 output
 *   n_threads <= 0 uses the OpenMP default
 * Returns 0, or a negative error code if any row's CSR entry is invalid.
 */
int vsa_oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* kv_block_idx,
                         const int32_t* kv_block_cnt, const int32_t* kv_valid, int B, int S, int H, int D, int ld,
                         int block_q, int block_kv, float scale, const int64_t* rows, int64_t n_rows, float* o,
                         float* lse, int n_threads) {
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || block_q <= 0 || block_kv <= 0 || ld < 0) return ORACLE_ERR_ARG;
    if (S % block_q || S % block_kv) return ORACLE_ERR_ARG;
    const int nq = S / block_q, nkv = S / block_kv;
    if (check_valid(kv_valid, nkv, block_kv) != ORACLE_OK) return ORACLE_ERR_ARG;
    const int64_t total = (int64_t)B * H * S;
    if (rows == NULL) n_rows = total;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
    (void)n_threads;
#endif

#pragma omp parallel num_threads(n_threads)
    {
        float* s = (float*)malloc(sizeof(float) * (size_t)S);
        float* qf = (float*)malloc(sizeof(float) * (size_t)D);
        int32_t* allow = (int32_t*)malloc(sizeof(int32_t) * (size_t)nkv);
        if (!s || !qf || !allow) {
#pragma omp critical
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t flat = rows ? rows[r] : r;
                float* orow = o + r * D;
                if (flat < 0 || flat >= total) {
#pragma omp critical
                    status = ORACLE_ERR_ARG;
                    continue;
                }
                int i = (int)(flat % S);
                int h = (int)((flat / S) % H);
                int b = (int)(flat / ((int64_t)S * H));
                int p = i / block_q;
                int64_t crow = ((int64_t)b * H + h) * nq + p;
                int rc = mark_tiles(kv_block_idx + crow * ld, kv_block_cnt[crow], ld, nkv, kv_valid, block_kv, allow);
                if (rc != ORACLE_OK) {
#pragma omp critical
                    status = rc;
                    continue;
                }
                float m, l;
                int64_t nsel = row_weights(q, k, S, H, D, b, h, i, allow, nkv, block_kv, scale, qf, s, &m, &l);
                /* out = softmax(scores) @ v, keys in ascending order */
                for (int d = 0; d < D; ++d) orow[d] = 0.0f;
                if (nsel > 0) {
                    const int64_t tok = (int64_t)H * D;
                    for (int j = 0; j < S; ++j) {
                        if (!allowed(allow, block_kv, j)) continue;
                        const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                        float w = s[j];
                        for (int d = 0; d < D; ++d) orow[d] += w * bf16_to_f32(vrow[d]);
                    }
                    lse[r] = m + logf(l);
                } else {
                    lse[r] = -INFINITY;
                }
            }
        }
        free(s);
        free(qf);
        free(allow);
    }
    return status;
}

/*
 * Softmax weights of one query row (flat id (b*H + h)*S + i) over all S key
 * tokens: probs[j] = 0 for unselected keys. Used to check the oracle's own
 * invariants (rows sum to one, zero outside the mask).
 */
int vsa_oracle_probs_row(const uint16_t* q, const uint16_t* k, const int32_t* kv_block_idx,
                         const int32_t* kv_block_cnt, const int32_t* kv_valid, int B, int S, int H, int D, int ld,
                         int block_q, int block_kv, float scale, int64_t flat_row, float* probs) {
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || block_q <= 0 || block_kv <= 0 || ld < 0) return ORACLE_ERR_ARG;
    if (S % block_q || S % block_kv) return ORACLE_ERR_ARG;
    if (flat_row < 0 || flat_row >= (int64_t)B * H * S) return ORACLE_ERR_ARG;
    const int nq = S / block_q, nkv = S / block_kv;
    if (check_valid(kv_valid, nkv, block_kv) != ORACLE_OK) return ORACLE_ERR_ARG;
    int i = (int)(flat_row % S);
    int h = (int)((flat_row / S) % H);
    int b = (int)(flat_row / ((int64_t)S * H));
    int64_t crow = ((int64_t)b * H + h) * nq + i / block_q;
    int32_t* allow = (int32_t*)malloc(sizeof(int32_t) * (size_t)nkv);
    float* qf = (float*)malloc(sizeof(float) * (size_t)D);
    if (!allow || !qf) {
        free(allow);
        free(qf);
        return ORACLE_ERR_NOMEM;
    }
    int rc = mark_tiles(kv_block_idx + crow * ld, kv_block_cnt[crow], ld, nkv, kv_valid, block_kv, allow);
    if (rc == ORACLE_OK) {
        float m, l;
        row_weights(q, k, S, H, D, b, h, i, allow, nkv, block_kv, scale, qf, probs, &m, &l);
    }
    free(allow);
    free(qf);
    return rc;
}


/* ------------------------------------------------------------------------
 * Backward pass (gradients of O with respect to Q, K and V), the standard
 * softmax-attention derivative applied to the same masked fp32 scores as the
 * forward (FastVideo page "[perf] Add fine-grained FA4 VSA kernels",
 * benchmarks/bench_vsa_blackwell.py, ref_masked_sdpa_fp32: the gradient of
 * that function; the page's block_sparsity.py, normalize_block_sparse_config_
 * bwd, sets up the same computation over the transposed, Q-direction lists).
 * With P the masked row softmax of scale * Q K^T, O = P V and dO given:
 *     dV_j  = sum_i P_ij dO_i
 *     dP_ij = dO_i . v_j,   D_i = dO_i . O_i = sum_j P_ij dP_ij
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
 * Everything is computed here from q, k, v, dO and the mask (O, P and D are
 * recomputed in fp32, not taken from a forward run). Sums over keys run in
 * ascending key order, sums over queries in ascending query order, and the
 * head dimension d = 0..D-1, independent of the tile shape.
 * ------------------------------------------------------------------------ */

/* Query tile p's row may attend to key tile t?  Scans the CSR row. */
static int row_selects(const int32_t* idx_row, int32_t n, int32_t t) {
    for (int32_t e = 0; e < n; ++e)
        if (idx_row[e] == t) return 1;
    return 0;
}

/* P_i (in s, zero outside the mask), O_i (fp32) and D_i for one query row. */
static int64_t row_prob_out(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout, int S,
                            int H, int D, int b, int h, int i, const int32_t* allow, int nkv, int block_kv,
                            float scale, float* qf, float* s, float* o, float* d_out) {
    float m, l;
    int64_t nsel = row_weights(q, k, S, H, D, b, h, i, allow, nkv, block_kv, scale, qf, s, &m, &l);
    const int64_t tok = (int64_t)H * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0f;
    if (nsel > 0) {
        for (int j = 0; j < S; ++j) {
            if (!allowed(allow, block_kv, j)) continue;
            const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;
            for (int d = 0; d < D; ++d) o[d] += s[j] * bf16_to_f32(vrow[d]);
        }
    }
    const uint16_t* drow = dout + ((int64_t)b * S + i) * tok + (int64_t)h * D;
    float dd = 0.0f;
    for (int d = 0; d < D; ++d) dd += bf16_to_f32(drow[d]) * o[d];
    *d_out = dd;
    return nsel;
}

/*
 * dQ for a list of query rows (flat (b*H + h)*S + i, or NULL for all rows):
 * dq [n_rows, D] fp32.
 */
int vsa_oracle_bwd_dq_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                           const int32_t* kv_block_idx, const int32_t* kv_block_cnt, const int32_t* kv_valid, int B,
                           int S, int H, int D, int ld, int block_q, int block_kv, float scale, const int64_t* rows,
                           int64_t n_rows, float* dq, int n_threads) {
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || block_q <= 0 || block_kv <= 0 || ld < 0) return ORACLE_ERR_ARG;
    if (S % block_q || S % block_kv) return ORACLE_ERR_ARG;
    const int nq = S / block_q, nkv = S / block_kv;
    if (check_valid(kv_valid, nkv, block_kv) != ORACLE_OK) return ORACLE_ERR_ARG;
    const int64_t total = (int64_t)B * H * S;
    if (rows == NULL) n_rows = total;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
    (void)n_threads;
#endif
#pragma omp parallel num_threads(n_threads)
    {
        float* s = (float*)malloc(sizeof(float) * (size_t)S);
        float* qf = (float*)malloc(sizeof(float) * (size_t)D);
        float* o = (float*)malloc(sizeof(float) * (size_t)D);
        float* dof = (float*)malloc(sizeof(float) * (size_t)D);
        int32_t* allow = (int32_t*)malloc(sizeof(int32_t) * (size_t)nkv);
        if (!s || !qf || !o || !dof || !allow) {
#pragma omp critical
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t flat = rows ? rows[r] : r;
                float* dqrow = dq + r * D;
                if (flat < 0 || flat >= total) {
#pragma omp critical
                    status = ORACLE_ERR_ARG;
                    continue;
                }
                int i = (int)(flat % S);
                int h = (int)((flat / S) % H);
                int b = (int)(flat / ((int64_t)S * H));
                int64_t crow = ((int64_t)b * H + h) * nq + i / block_q;
                int rc = mark_tiles(kv_block_idx + crow * ld, kv_block_cnt[crow], ld, nkv, kv_valid, block_kv, allow);
                if (rc != ORACLE_OK) {
#pragma omp critical
                    status = rc;
                    continue;
                }
                float di;
                row_prob_out(q, k, v, dout, S, H, D, b, h, i, allow, nkv, block_kv, scale, qf, s, o, &di);
                const int64_t tok = (int64_t)H * D;
                const uint16_t* drow = dout + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                for (int d = 0; d < D; ++d) dof[d] = bf16_to_f32(drow[d]);
                for (int d = 0; d < D; ++d) dqrow[d] = 0.0f;
                for (int j = 0; j < S; ++j) {
                    if (!allowed(allow, block_kv, j)) continue;
                    const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                    const uint16_t* krow = k + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                    float dp = 0.0f;
                    for (int d = 0; d < D; ++d) dp += dof[d] * bf16_to_f32(vrow[d]);
                    const float ds = s[j] * (dp - di);
                    for (int d = 0; d < D; ++d) dqrow[d] += ds * bf16_to_f32(krow[d]);
                }
                for (int d = 0; d < D; ++d) dqrow[d] *= scale;
            }
        }
        free(s);
        free(qf);
        free(o);
        free(dof);
        free(allow);
    }
    return status;
}

/*
 * dK and dV for a list of key rows (flat (b*H + h)*S + j, or NULL for all):
 * dk, dv [n_rows, D] fp32. For key j the sums run over the query rows i that
 * may attend to it, in ascending order; each such row's softmax and D_i are
 * recomputed.
 */
int vsa_oracle_bwd_dkv_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                            const int32_t* kv_block_idx, const int32_t* kv_block_cnt, const int32_t* kv_valid, int B,
                            int S, int H, int D, int ld, int block_q, int block_kv, float scale, const int64_t* rows,
                            int64_t n_rows, float* dk, float* dv, int n_threads) {
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || block_q <= 0 || block_kv <= 0 || ld < 0) return ORACLE_ERR_ARG;
    if (S % block_q || S % block_kv) return ORACLE_ERR_ARG;
    const int nq = S / block_q, nkv = S / block_kv;
    if (check_valid(kv_valid, nkv, block_kv) != ORACLE_OK) return ORACLE_ERR_ARG;
    const int64_t total = (int64_t)B * H * S;
    if (rows == NULL) n_rows = total;
    int status = ORACLE_OK;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
    (void)n_threads;
#endif
#pragma omp parallel num_threads(n_threads)
    {
        float* s = (float*)malloc(sizeof(float) * (size_t)S);
        float* qf = (float*)malloc(sizeof(float) * (size_t)D);
        float* o = (float*)malloc(sizeof(float) * (size_t)D);
        int32_t* allow = (int32_t*)malloc(sizeof(int32_t) * (size_t)nkv);
        if (!s || !qf || !o || !allow) {
#pragma omp critical
            status = ORACLE_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t flat = rows ? rows[r] : r;
                float* dkrow = dk + r * D;
                float* dvrow = dv + r * D;
                if (flat < 0 || flat >= total) {
#pragma omp critical
                    status = ORACLE_ERR_ARG;
                    continue;
                }
                int j = (int)(flat % S);
                int h = (int)((flat / S) % H);
                int b = (int)(flat / ((int64_t)S * H));
                const int64_t tok = (int64_t)H * D;
                const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                for (int d = 0; d < D; ++d) dkrow[d] = 0.0f;
                for (int d = 0; d < D; ++d) dvrow[d] = 0.0f;
                for (int p = 0; p < nq; ++p) {
                    int64_t crow = ((int64_t)b * H + h) * nq + p;
                    int32_t n = kv_block_cnt[crow];
                    if (n < 0 || n > ld) {
#pragma omp critical
                        status = ORACLE_ERR_CNT;
                        break;
                    }
                    if (!row_selects(kv_block_idx + crow * ld, n, j / block_kv)) continue;
                    int rc = mark_tiles(kv_block_idx + crow * ld, n, ld, nkv, kv_valid, block_kv, allow);
                    if (rc != ORACLE_OK) {
#pragma omp critical
                        status = rc;
                        break;
                    }
                    if (!allowed(allow, block_kv, j)) continue; /* padding key of a partial tile */
                    for (int i = p * block_q; i < (p + 1) * block_q; ++i) {
                        float di;
                        row_prob_out(q, k, v, dout, S, H, D, b, h, i, allow, nkv, block_kv, scale, qf, s, o, &di);
                        const uint16_t* drow = dout + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                        float dp = 0.0f;
                        for (int d = 0; d < D; ++d) dp += bf16_to_f32(drow[d]) * bf16_to_f32(vrow[d]);
                        const float pij = s[j];
                        const float ds = pij * (dp - di);
                        /* qf holds row i of Q (filled by row_weights) */
                        for (int d = 0; d < D; ++d) dkrow[d] += ds * qf[d];
                        for (int d = 0; d < D; ++d) dvrow[d] += pij * bf16_to_f32(drow[d]);
                    }
                }
                for (int d = 0; d < D; ++d) dkrow[d] *= scale;
            }
        }
        free(s);
        free(qf);
        free(o);
        free(allow);
    }
    return status;
}


/*
 * All three gradients for every row, one head at a time, in two passes that
 * are each parallel over rows:
 *   1. every query row i (ascending keys j): P_ij, D_i, dS_ij and dQ_i;
 *      P_ij and dS_ij are kept for the keys the row sees;
 *   2. every key row j: dK_j = scale * sum_i dS_ij q_i and dV_j =
 *      sum_i P_ij dO_i over the query rows i that see j, in ascending i.
 * These are the same sums, in the same order and with the same fp32
 * operations, as vsa_oracle_bwd_dq_rows and vsa_oracle_bwd_dkv_rows (whose
 * results this reproduces bit for bit, only faster). dq, dk, dv:
 * [B, S, H, D] fp32.
 */
int vsa_oracle_bwd_full(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                        const int32_t* kv_block_idx, const int32_t* kv_block_cnt, const int32_t* kv_valid, int B, int S,
                        int H, int D, int ld, int block_q, int block_kv, float scale, float* dq, float* dk, float* dv,
                        int n_threads) {
    if (B <= 0 || S <= 0 || H <= 0 || D <= 0 || block_q <= 0 || block_kv <= 0 || ld < 0) return ORACLE_ERR_ARG;
    if (S % block_q || S % block_kv) return ORACLE_ERR_ARG;
    const int nq = S / block_q, nkv = S / block_kv;
    if (check_valid(kv_valid, nkv, block_kv) != ORACLE_OK) return ORACLE_ERR_ARG;
#ifdef _OPENMP
    if (n_threads <= 0) n_threads = omp_get_max_threads();
#else
    (void)n_threads;
#endif
    const int64_t tok = (int64_t)H * D;
    /* per query tile p: allow[p*nkv + t] keys of tile t it sees, first[p*nkv + t]
     * the position of tile t's first key among the keys the row sees (ascending) */
    int32_t* allow = (int32_t*)malloc(sizeof(int32_t) * (size_t)nq * nkv);
    int64_t* first = (int64_t*)malloc(sizeof(int64_t) * (size_t)nq * nkv);
    int64_t* row_off = (int64_t*)malloc(sizeof(int64_t) * ((size_t)S + 1));
    if (!allow || !first || !row_off) {
        free(allow);
        free(first);
        free(row_off);
        return ORACLE_ERR_NOMEM;
    }
    float* pst = NULL; /* P_ij of every (row, seen key), rows back to back */
    float* dst = NULL; /* dS_ij, same layout */
    size_t cap = 0;
    int status = ORACLE_OK;
    for (int bh = 0; bh < B * H && status == ORACLE_OK; ++bh) {
        const int b = bh / H, h = bh % H;
        for (int p = 0; p < nq && status == ORACLE_OK; ++p) {
            const int64_t crow = ((int64_t)b * H + h) * nq + p;
            status = mark_tiles(kv_block_idx + crow * ld, kv_block_cnt[crow], ld, nkv, kv_valid, block_kv,
                                allow + (size_t)p * nkv);
            int64_t acc = 0;
            for (int t = 0; t < nkv; ++t) {
                first[(size_t)p * nkv + t] = acc;
                acc += allow[(size_t)p * nkv + t];
            }
        }
        if (status != ORACLE_OK) break;
        row_off[0] = 0;
        for (int i = 0; i < S; ++i) {
            const int p = i / block_q;
            row_off[i + 1] = row_off[i] + first[(size_t)p * nkv + nkv - 1] + allow[(size_t)p * nkv + nkv - 1];
        }
        const size_t need = (size_t)row_off[S];
        if (need > cap) {
            free(pst);
            free(dst);
            cap = need;
            pst = (float*)malloc(sizeof(float) * (cap ? cap : 1));
            dst = (float*)malloc(sizeof(float) * (cap ? cap : 1));
            if (!pst || !dst) {
                status = ORACLE_ERR_NOMEM;
                break;
            }
        }
        /* pass 1: query rows */
#pragma omp parallel num_threads(n_threads)
        {
            float* s = (float*)malloc(sizeof(float) * (size_t)S);
            float* qf = (float*)malloc(sizeof(float) * (size_t)D);
            float* o = (float*)malloc(sizeof(float) * (size_t)D);
            float* dof = (float*)malloc(sizeof(float) * (size_t)D);
            if (!s || !qf || !o || !dof) {
#pragma omp critical
                status = ORACLE_ERR_NOMEM;
            } else {
#pragma omp for schedule(dynamic, 16)
                for (int i = 0; i < S; ++i) {
                    const int32_t* al = allow + (size_t)(i / block_q) * nkv;
                    float* dqrow = dq + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                    float di;
                    row_prob_out(q, k, v, dout, S, H, D, b, h, i, al, nkv, block_kv, scale, qf, s, o, &di);
                    const uint16_t* drow = dout + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                    for (int d = 0; d < D; ++d) dof[d] = bf16_to_f32(drow[d]);
                    for (int d = 0; d < D; ++d) dqrow[d] = 0.0f;
                    int64_t pos = row_off[i];
                    for (int j = 0; j < S; ++j) {
                        if (!allowed(al, block_kv, j)) continue;
                        const uint16_t* vrow = v + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                        const uint16_t* krow = k + ((int64_t)b * S + j) * tok + (int64_t)h * D;
                        float dp = 0.0f;
                        for (int d = 0; d < D; ++d) dp += dof[d] * bf16_to_f32(vrow[d]);
                        const float pij = s[j];
                        const float ds = pij * (dp - di);
                        for (int d = 0; d < D; ++d) dqrow[d] += ds * bf16_to_f32(krow[d]);
                        pst[pos] = pij;
                        dst[pos] = ds;
                        ++pos;
                    }
                    for (int d = 0; d < D; ++d) dqrow[d] *= scale;
                }
            }
            free(s);
            free(qf);
            free(o);
            free(dof);
        }
        if (status != ORACLE_OK) break;
        /* pass 2: key rows, summing over the query rows that see them in
         * ascending order (query tiles ascending, rows within a tile ascending) */
#pragma omp parallel for schedule(dynamic, 16) num_threads(n_threads)
        for (int j = 0; j < S; ++j) {
            const int t = j / block_kv, r = j % block_kv;
            float* dkrow = dk + ((int64_t)b * S + j) * tok + (int64_t)h * D;
            float* dvrow = dv + ((int64_t)b * S + j) * tok + (int64_t)h * D;
            for (int d = 0; d < D; ++d) dkrow[d] = 0.0f;
            for (int d = 0; d < D; ++d) dvrow[d] = 0.0f;
            for (int p = 0; p < nq; ++p) {
                if (r >= allow[(size_t)p * nkv + t]) continue;
                const int64_t at = first[(size_t)p * nkv + t] + r;
                for (int i = p * block_q; i < (p + 1) * block_q; ++i) {
                    const uint16_t* qrow = q + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                    const uint16_t* drow = dout + ((int64_t)b * S + i) * tok + (int64_t)h * D;
                    const float pij = pst[row_off[i] + at];
                    const float ds = dst[row_off[i] + at];
                    for (int d = 0; d < D; ++d) dkrow[d] += ds * bf16_to_f32(qrow[d]);
                    for (int d = 0; d < D; ++d) dvrow[d] += pij * bf16_to_f32(drow[d]);
                }
            }
            for (int d = 0; d < D; ++d) dkrow[d] *= scale;
        }
    }
    free(pst);
    free(dst);
    free(allow);
    free(first);
    free(row_off);
    return status;
}
