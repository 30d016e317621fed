/*
 * CPU oracle for dynamic block-sparse self-attention.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, fp64 definition that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it. The GPU library does not include, link or
 * call anything here, and nothing here comes from the GPU library.
 *
 * What the method computes, per the pages:
 *   [KC] "知识卡片：600倍加速，720p视频实时生成！单卡也能带的动14B模型"
 *        (ai.cheesepanini.fun knowledge card), section 方法/产品要点, item
 *        动态稀疏量化注意力: Query/Key block means give a quick estimate of which
 *        attention blocks matter; at run time only the activated key blocks are
 *        computed; typical sparsity 80-90 % (about 10-20 % of blocks kept); the
 *        sparse path is combined with SageAttention2 into an FP8 path.
 *   [AO] "单卡 RTX 5090 跑 Wan2.2-A14B：720p 视频生成只要 3.8 秒" (aoyii.com),
 *        section 四步拆解, step 3 动态稀疏注意力: the same, and inside the selected
 *        blocks the computation stays dense.
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *   - block score = dot product of the two block means scaled by 1/sqrt(D);
 *   - a fixed count k = min(n, max(1, ceil(r*n - 1e-6))) of key blocks per query
 *     block, per (batch, head); ties go to the lower block index;
 *   - the last block may be partial: its mean divides by its valid token count, and
 *     its missing keys do not exist (they are never zero-padded);
 *   - dropped blocks contribute nothing; the softmax renormalises over kept keys;
 *     softmax scale 1/sqrt(D), no causal mask;
 *   - a query block with an empty kept list produces a zero output row;
 *   - FP8 is OCP E4M3FN with round-to-nearest-even, one fp32 scale = absmax/448 per
 *     (batch, head, token block) for Q and for K separately (scale 1 when absmax=0).
 *   - Full FP8 path (P and V in E4M3 as well; the pages name SageAttention2 but give
 *     none of its steps): V has one fp32 scale per (batch, head, channel) over the whole
 *     sequence; the softmax runs online over the kept keys in list order, 64 keys at a
 *     time, and each 64-key sub-tile's weights 2^(x - m) <= 1 (x the logit in log2 units,
 *     m the running maximum after that sub-tile) are stored as E4M3FN codes of 448 times
 *     the weight; the normaliser is the sum of the stored weights. That sub-tile schedule
 *     is one kernel's order of work, so it serves as a diagnostic; the full FP8 path is
 *     graded against oracle_attention_fp8_qkv (exact softmax over the dequantised Q, K and
 *     V) with a bound on what rounding the weights to E4M3 can change, which holds for any
 *     order and reference point.
 *
 * Layouts: tensors are [B, H, S, D] row-major; bf16 values are passed as their raw
 * 16-bit patterns. Block i of a sequence is tokens [i*block, min(S,(i+1)*block)).
 * All arithmetic is fp64 (bf16 and E4M3 values widen exactly).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- element access --------------------------------------------------------------- */

/* bf16 is the top half of an IEEE binary32 pattern; widening is exact. */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit floating point, E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits; exponent field 0 is subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN;
 * the largest finite magnitude is S.1111.110 = 448. */
double oracle_e4m3_value(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Nearest E4M3FN code to x, ties to the even code (even mantissa), magnitudes above 448
 * go to 448. The 127 non-negative finite codes increase with their value, so a binary
 * search over the code values finds the two neighbours of |x|. */
uint8_t oracle_e4m3_encode(double x) {
    uint8_t sign = (x < 0.0 || (x == 0.0 && signbit(x))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (isnan(x)) return 0x7F;
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 0x7E;               /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_value((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - oracle_e4m3_value((uint8_t)lo), dhi = oracle_e4m3_value((uint8_t)hi) - a;
    int pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = (lo % 2 == 0) ? lo : hi;  /* tie: even mantissa */
    return (uint8_t)(sign | pick);
}

/* A tensor as the attention definition reads it: either bf16 bits, or E4M3 codes with
 * one scale per (batch*head, block), or (chan_scale) one scale per (batch*head, channel). */
typedef struct {
    const uint16_t* bf16;
    const uint8_t* e4m3;
    const float* scale;
    const float* chan_scale;
    int64_t S, D, block, nblk;
} tensor_t;

/* Every code's value, taken from oracle_e4m3_value once per attention call (a lookup, so
 * that decoding does not dominate the oracle's run time; the values are the same). */
static double e4m3_table[256];

static void fill_e4m3_table(void) {
    for (int c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_value((uint8_t)c);
}

static double load(const tensor_t* T, int64_t bh, int64_t t, int64_t d) {
    int64_t off = (bh * T->S + t) * T->D + d;
    if (T->bf16) return bf16_value(T->bf16[off]);
    double sc = T->chan_scale ? (double)T->chan_scale[bh * T->D + d]
                              : (double)T->scale[bh * T->nblk + t / T->block];
    return e4m3_table[T->e4m3[off]] * sc;
}

/* ---- block partition and the k rule ----------------------------------------------- */

int32_t oracle_num_blocks(int32_t S, int32_t block) {
    if (S < 1 || block < 1) return 0;
    return (int32_t)(((int64_t)S + block - 1) / block);
}

/* Kept key blocks per query block: the pages keep about 10-20 % of blocks; the count is
 * the ratio times the block count, rounded up (with a 1e-6 guard against binary
 * representation error), clamped to [1, n]. Returns 0 for invalid input. */
int32_t oracle_num_kept(int32_t n, double keep_ratio) {
    if (n < 1 || !(keep_ratio > 0.0) || keep_ratio > 1.0) return 0;
    double k = ceil(keep_ratio * (double)n - 1e-6);
    if (k < 1.0) k = 1.0;
    if (k > (double)n) k = (double)n;
    return (int32_t)k;
}

/* ---- step 1: block means of Q or K ([KC] 动态稀疏量化注意力: importance from block-level means) */

void oracle_pool(const uint16_t* x, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                 double* xbar /* [B*H, n, D] */) {
    int64_t n = oracle_num_blocks(S, block), rows = (int64_t)B * H * n;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t bh = r / n, i = r % n;
        int64_t t0 = i * block, t1 = t0 + block < S ? t0 + block : S;
        for (int64_t d = 0; d < D; ++d) {
            double sum = 0.0;
            for (int64_t t = t0; t < t1; ++t) sum += bf16_value(x[(bh * S + t) * D + d]);
            xbar[r * D + d] = sum / (double)(t1 - t0);
        }
    }
}

/* ---- step 2: block-pair importance from the means ---------------------------------- */

void oracle_scores(const double* qbar, const double* kbar, int32_t BH, int32_t n, int32_t D,
                   double* s /* [BH, n, n] */) {
    double inv = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < (int64_t)BH * n; ++r) {
        int64_t bh = r / n;
        for (int64_t j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qbar[r * D + d] * kbar[(bh * n + j) * D + d];
            s[r * n + j] = dot * inv;
        }
    }
}

/* ---- step 3: keep the k most important key blocks of every query block ------------ */

typedef struct { double s; int32_t j; } cand_t;

/* Order: higher score first; equal scores, lower block index first. */
static int by_score_then_index(const void* a, const void* b) {
    const cand_t* x = (const cand_t*)a;
    const cand_t* y = (const cand_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_int(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x > y) - (x < y);
}

/* col_idx[row*k .. row*k+k) = the kept blocks of row, ascending. gap[row] = k-th largest
 * score minus (k+1)-th largest (+inf when k = n). */
void oracle_select(const double* s, int32_t rows, int32_t n, int32_t k, int32_t* col_idx,
                   double* gap) {
#pragma omp parallel
    {
        cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)n);
#pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            for (int32_t j = 0; j < n; ++j) { c[j].s = s[r * n + j]; c[j].j = j; }
            qsort(c, (size_t)n, sizeof(cand_t), by_score_then_index);
            for (int32_t m = 0; m < k; ++m) col_idx[r * k + m] = c[m].j;
            qsort(col_idx + r * k, (size_t)k, sizeof(int32_t), by_int);
            if (gap) gap[r] = (k < n) ? c[k - 1].s - c[k].s : INFINITY;
        }
        free(c);
    }
}

/* ---- step 4: attention over the kept blocks only ----------------------------------- */

/* For every requested query token, softmax(Q_t K_u^T / sqrt(D)) V_u over the keys u of
 * the kept blocks of t's block ([AO] 动态稀疏注意力: dense inside the selected blocks).
 * tokens[m] = bh*S + t; NULL means all B*H*S tokens in order. out is [ntok, D].
 * dev (optional, [ntok, 3, D]) receives, per output element, the spread of the values
 * around it: sum_u p_u |v_ud - o_d|, sum_u |v_ud - o_d| and sqrt(sum_u p_u^2 (v_ud - o_d)^2)
 * (p the softmax weights); the full FP8 path's error bound is built from them. */
static void attention_core(const tensor_t* Q, const tensor_t* K, const tensor_t* V, int64_t BH,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const int64_t* tokens, int64_t ntok, double* out, double* dev) {
    int64_t S = Q->S, D = Q->D, block = Q->block, n = Q->nblk;
    double inv = 1.0 / sqrt((double)D);
    (void)BH;
    fill_e4m3_table();
#pragma omp parallel
    {
        double* logit = (double*)malloc(sizeof(double) * (size_t)S);
        int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)S);
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 16)
        for (int64_t m = 0; m < ntok; ++m) {
            int64_t flat = tokens ? tokens[m] : m;
            int64_t bh = flat / S, t = flat % S, row = bh * n + t / block;
            double* o = out + m * D;
            int64_t nk = 0;
            for (int32_t p = row_ptr[row]; p < row_ptr[row + 1]; ++p) {
                int64_t j = col_idx[p], u0 = j * block, u1 = u0 + block < S ? u0 + block : S;
                for (int64_t u = u0; u < u1; ++u) key[nk++] = u;
            }
            for (int64_t d = 0; d < D; ++d) { qrow[d] = load(Q, bh, t, d); o[d] = 0.0; }
            if (dev)  /* an empty row has no spread */
                for (int64_t d = 0; d < 3 * D; ++d) dev[m * 3 * D + d] = 0.0;
            if (nk == 0) continue;
            double mx = -INFINITY;
            for (int64_t a = 0; a < nk; ++a) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qrow[d] * load(K, bh, key[a], d);
                logit[a] = dot * inv;
                if (logit[a] > mx) mx = logit[a];
            }
            double denom = 0.0;
            for (int64_t a = 0; a < nk; ++a) { logit[a] = exp(logit[a] - mx); denom += logit[a]; }
            for (int64_t a = 0; a < nk; ++a) {
                double p = logit[a] / denom;
                for (int64_t d = 0; d < D; ++d) o[d] += p * load(V, bh, key[a], d);
            }
            if (dev) {
                double* dv = dev + m * 3 * D;
                for (int64_t a = 0; a < nk; ++a) {
                    double p = logit[a] / denom;
                    for (int64_t d = 0; d < D; ++d) {
                        double e = fabs(load(V, bh, key[a], d) - o[d]);
                        dv[d] += p * e;
                        dv[D + d] += e;
                        dv[2 * D + d] += p * p * e * e;
                    }
                }
                for (int64_t d = 0; d < D; ++d) dv[2 * D + d] = sqrt(dv[2 * D + d]);
            }
        }
        free(logit); free(key); free(qrow);
    }
}

void oracle_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int32_t B,
                      int32_t H, int32_t S, int32_t D, int32_t block, const int32_t* row_ptr,
                      const int32_t* col_idx, const int64_t* tokens, int64_t ntok, double* out) {
    int64_t n = oracle_num_blocks(S, block);
    tensor_t Q = {q, NULL, NULL, NULL, S, D, block, n}, K = {k, NULL, NULL, NULL, S, D, block, n},
             V = {v, NULL, NULL, NULL, S, D, block, n};
    if (!tokens) ntok = (int64_t)B * H * S;
    attention_core(&Q, &K, &V, (int64_t)B * H, row_ptr, col_idx, tokens, ntok, out, NULL);
}

/* ---- FP8 path ([KC] 动态稀疏量化注意力: SageAttention2 FP8 sparse path) ------------ */

/* Per (batch*head, block): scale = absmax/448 in fp32 (1 when the block is all zero);
 * code = nearest E4M3FN to x/scale, the division done in IEEE fp32. */
void oracle_quantize_fp8(const uint16_t* x, int32_t B, int32_t H, int32_t S, int32_t D,
                         int32_t block, uint8_t* codes, float* scale /* [B*H, n] */) {
    int64_t n = oracle_num_blocks(S, block), rows = (int64_t)B * H * n;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t bh = r / n, i = r % n;
        int64_t t0 = i * block, t1 = t0 + block < S ? t0 + block : S;
        float amax = 0.0f;
        for (int64_t off = (bh * S + t0) * D; off < (bh * S + t1) * D; ++off) {
            float a = fabsf((float)bf16_value(x[off]));
            if (a > amax) amax = a;
        }
        float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        scale[r] = sc;
        for (int64_t off = (bh * S + t0) * D; off < (bh * S + t1) * D; ++off) {
            float y = (float)bf16_value(x[off]) / sc;
            codes[off] = oracle_e4m3_encode((double)y);
        }
    }
}

/* Attention with Q and K given as E4M3 codes and per-block scales, V as bf16 (the
 * quantised path; a diagnostic that separates quantisation error from kernel error). */
void oracle_attention_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                          const float* k_scale, const uint16_t* v, int32_t B, int32_t H,
                          int32_t S, int32_t D, int32_t block, const int32_t* row_ptr,
                          const int32_t* col_idx, const int64_t* tokens, int64_t ntok,
                          double* out) {
    int64_t n = oracle_num_blocks(S, block);
    tensor_t Q = {NULL, q8, q_scale, NULL, S, D, block, n}, K = {NULL, k8, k_scale, NULL, S, D, block, n},
             V = {v, NULL, NULL, NULL, S, D, block, n};
    if (!tokens) ntok = (int64_t)B * H * S;
    attention_core(&Q, &K, &V, (int64_t)B * H, row_ptr, col_idx, tokens, ntok, out, NULL);
}

/* ---- Full FP8 path: P and V in E4M3 as well -------------------------------------------
 * [KC] 动态稀疏量化注意力 and [AO] step 3: the sparse path is combined with SageAttention2
 * into an FP8 attention path. The quantisation steps below are this implementation's
 * reading (see the header): they are not on the pages. */

/* Per (batch*head, channel d): scale = absmax over all S tokens / 448 in fp32 (1 when the
 * channel is all zero); code = nearest E4M3FN to v/scale, the division in IEEE fp32.
 * codes keep the [B, H, S, D] layout of v. */
void oracle_quantize_v_fp8(const uint16_t* v, int32_t B, int32_t H, int32_t S, int32_t D,
                           uint8_t* codes, float* scale /* [B*H, D] */) {
    int64_t BH = (int64_t)B * H;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < BH * D; ++r) {
        int64_t bh = r / D, d = r % D;
        float amax = 0.0f;
        for (int64_t t = 0; t < S; ++t) {
            float a = fabsf((float)bf16_value(v[(bh * S + t) * D + d]));
            if (a > amax) amax = a;
        }
        float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        scale[r] = sc;
        for (int64_t t = 0; t < S; ++t) {
            int64_t off = (bh * S + t) * D + d;
            float y = (float)bf16_value(v[off]) / sc;
            codes[off] = oracle_e4m3_encode((double)y);
        }
    }
}

/* The full FP8 path's operands without its weight rounding: exact softmax attention (fp64)
 * over Q and K dequantised from E4M3 codes with their per-(batch*head, block) scales and V
 * dequantised with its per-(batch*head, channel) scales. Rounding the softmax weights to
 * E4M3 moves each weight by at most 2^-4 of itself (or by an absolute amount below the
 * smallest subnormal step, for weights in the subnormal range), whatever the order in which a
 * kernel visits the keys and wherever it takes its reference point, so this result together
 * with the spread terms in dev bounds every such kernel. dev as in attention_core. */
void oracle_attention_fp8_qkv(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                              const float* k_scale, const uint8_t* v8, const float* v_scale,
                              int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              const int64_t* tokens, int64_t ntok, double* out, double* dev) {
    int64_t n = oracle_num_blocks(S, block);
    tensor_t Q = {NULL, q8, q_scale, NULL, S, D, block, n}, K = {NULL, k8, k_scale, NULL, S, D, block, n},
             V = {NULL, v8, NULL, v_scale, S, D, block, n};
    if (!tokens) ntok = (int64_t)B * H * S;
    attention_core(&Q, &K, &V, (int64_t)B * H, row_ptr, col_idx, tokens, ntok, out, dev);
}

/* Attention with Q, K (per-block scales) and V (per-channel scales) as E4M3 codes and the
 * softmax weights stored as E4M3 as well. For every requested query token t of query
 * block i: walk the kept blocks of row i in list order; split each block's keys into
 * sub-tiles of 64 (the last may be shorter); for each sub-tile
 *   x_u   = (q_t . k_u) log2(e) / sqrt(D)              (dequantised codes, fp64)
 *   m'    = max(m, max_u x_u);  O *= 2^(m - m'),  l *= 2^(m - m')   (0 while m = -inf)
 *   w_u   = value(E4M3(448 * 2^(x_u - m'))) / 448
 *   l    += sum_u w_u;  O += sum_u w_u v_u             (v_u dequantised)
 *   m     = m'
 * and return O / l (zeros for an empty list). Entries outside [0, n) are skipped. */
void oracle_attention_fp8_full(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                               const float* k_scale, const uint8_t* v8, const float* v_scale,
                               int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                               const int32_t* row_ptr, const int32_t* col_idx,
                               const int64_t* tokens, int64_t ntok, double* out) {
    const int64_t n = oracle_num_blocks(S, block), KT = 64;
    const double log2e = 1.4426950408889634073599, inv = 1.0 / sqrt((double)D);
    if (!tokens) ntok = (int64_t)B * H * S;
#pragma omp parallel
    {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        double* x = (double*)malloc(sizeof(double) * (size_t)KT);
#pragma omp for schedule(dynamic, 16)
        for (int64_t mi = 0; mi < ntok; ++mi) {
            int64_t flat = tokens ? tokens[mi] : mi;
            int64_t bh = flat / S, t = flat % S, row = bh * n + t / block;
            double* o = out + mi * D;
            double qs = (double)q_scale[bh * n + t / block];
            for (int64_t d = 0; d < D; ++d) {
                qrow[d] = oracle_e4m3_value(q8[(bh * S + t) * D + d]) * qs;
                o[d] = 0.0;
            }
            double m = -INFINITY, l = 0.0;
            for (int32_t p = row_ptr[row]; p < row_ptr[row + 1]; ++p) {
                int64_t j = col_idx[p];
                if (j < 0 || j >= n) continue;
                double ks = (double)k_scale[bh * n + j];
                int64_t u_end = (j + 1) * block < S ? (j + 1) * block : S;
                for (int64_t u0 = j * block; u0 < u_end; u0 += KT) {
                    int64_t u1 = u0 + KT < u_end ? u0 + KT : u_end;
                    double mt = -INFINITY;
                    for (int64_t u = u0; u < u1; ++u) {
                        double dot = 0.0;
                        for (int64_t d = 0; d < D; ++d)
                            dot += qrow[d] * oracle_e4m3_value(k8[(bh * S + u) * D + d]) * ks;
                        x[u - u0] = dot * inv * log2e;
                        if (x[u - u0] > mt) mt = x[u - u0];
                    }
                    double m_new = mt > m ? mt : m;
                    double alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new);
                    l *= alpha;
                    for (int64_t d = 0; d < D; ++d) o[d] *= alpha;
                    for (int64_t u = u0; u < u1; ++u) {
                        double w = oracle_e4m3_value(oracle_e4m3_encode(448.0 * exp2(x[u - u0] - m_new))) / 448.0;
                        l += w;
                        for (int64_t d = 0; d < D; ++d)
                            o[d] += w * oracle_e4m3_value(v8[(bh * S + u) * D + d]) * (double)v_scale[bh * D + d];
                    }
                    m = m_new;
                }
            }
            if (l > 0.0)
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
            else
                for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        }
        free(qrow); free(x);
    }
}

/* ---- RMSNorm and 3D RoPE of a Q or K projection ---------------------------------------
 * [KC] 方法/产品要点, item 高效推理算子, and [AO] 四步拆解, step 4 (融合内核): 3D RoPE and
 * RMSNorm run as fused kernels, to save temporaries and memory round trips. Neither page
 * gives a formula, so the following readings define the operation:
 *   - x is a projection's output, bf16 [B, S, H*D] (token-major); w is bf16 [H*D];
 *   - RMSNorm over the H*D channels of a token: x_c / sqrt(mean over c of x_c^2 + eps) * w_c;
 *   - 3D RoPE inside each head: its D channels split into three contiguous segments for the
 *     frame, height and width axes, of sizes D - 4*floor(D/6), 2*floor(D/6), 2*floor(D/6);
 *     in a segment of size Da, channels 2i and 2i+1 are turned by the angle
 *     p * theta^(-2i/Da) (p = the token's coordinate on that axis):
 *     (u, v) -> (u cos a - v sin a, u sin a + v cos a);
 *   - token s of the latent grid (Gt, Gh, Gw), row-major, is at (s / (Gh*Gw), (s / Gw) % Gh,
 *     s % Gw);
 *   - the result, [B, H, S, D], is rounded once to bf16 (nearest, ties to even).
 * The block means of the rounded result are oracle_pool of it. */

/* Nearest bf16 to a finite x (ties to even), as its 16-bit pattern. bf16 keeps 8
 * significant bits down to 2^-126 and a fixed spacing of 2^-133 below. */
uint16_t oracle_round_bf16(double x) {
    if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
    int e;
    (void)frexp(x, &e);               /* 2^(e-1) <= |x| < 2^e */
    int lsb = e - 8;
    if (lsb < -133) lsb = -133;
    double r = ldexp(nearbyint(ldexp(x, -lsb)), lsb);  /* default mode: ties to even */
    float f = (float)r;                /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_norm_rope(const uint16_t* x /* [B, S, H*D] */, const uint16_t* w /* [H*D] */, int32_t B,
                      int32_t S, int32_t H, int32_t D, int32_t gt, int32_t gh, int32_t gw, double eps,
                      double theta, double* y /* [B, H, S, D] or NULL */,
                      uint16_t* y16 /* [B, H, S, D] or NULL */) {
    const int64_t C = (int64_t)H * D;
    const int64_t seg[3] = {D - 4 * (D / 6), 2 * (D / 6), 2 * (D / 6)};
    (void)gt;
#pragma omp parallel for schedule(static)
    for (int64_t bs = 0; bs < (int64_t)B * S; ++bs) {
        const int64_t b = bs / S, s = bs % S;
        const uint16_t* xr = x + bs * C;
        double ms = 0.0;
        for (int64_t c = 0; c < C; ++c) ms += bf16_value(xr[c]) * bf16_value(xr[c]);
        ms /= (double)C;
        const double inv = 1.0 / sqrt(ms + eps);
        const int64_t pos[3] = {s / ((int64_t)gh * gw), (s / gw) % gh, s % gw};
        for (int64_t h = 0; h < H; ++h) {
            int64_t off = 0;
            for (int a = 0; a < 3; ++a) {
                for (int64_t i = 0; i < seg[a] / 2; ++i) {
                    const int64_t c0 = h * D + off + 2 * i;
                    const double u = bf16_value(xr[c0]) * inv * bf16_value(w[c0]);
                    const double v = bf16_value(xr[c0 + 1]) * inv * bf16_value(w[c0 + 1]);
                    const double ang = (double)pos[a] * pow(theta, -2.0 * (double)i / (double)seg[a]);
                    const double r0 = u * cos(ang) - v * sin(ang), r1 = u * sin(ang) + v * cos(ang);
                    const int64_t o = ((b * H + h) * S + s) * D + off + 2 * i;
                    if (y) { y[o] = r0; y[o + 1] = r1; }
                    if (y16) { y16[o] = oracle_round_bf16(r0); y16[o + 1] = oracle_round_bf16(r1); }
                }
                off += seg[a];
            }
        }
    }
}
