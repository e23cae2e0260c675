/*
 * fsa_oracle.c -- plain fp64 CPU definition of top-k selected block-sparse
 * attention (prefill) and top-k gathered paged-KV decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, link or
 * call this file: only the test suite, the package smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code with the HIP library.
 *
 * What is computed (the plain definition; every step is written out, there is
 * no blocking, fusion or reordering beyond it):
 *
 *  - Head mapping: query head h reads kv head h / (Hq / Hkv).  (Stated with
 *    the 6-q-head / 2-kv-head example in the MQA/GQA paragraph of the
 *    flash_attn_func docstring, flash-attention-npu page.)
 *  - Causal mask aligned to the bottom-right corner: row i of a sequence with
 *    S_q queries and S_k keys sees key j iff j <= i + S_k - S_q.  A row with
 *    no visible key outputs zeros.  (Same docstring, causal paragraph and its
 *    2x5 / 5x2 examples; FlashAttention basic-usage page section 4.2.)
 *  - Selection: per (query token, kv head) a list of key-block ids of
 *    block_size keys each; the row attends to the keys of the listed blocks
 *    only.  The list is read as a SET: ids outside [0, ceil(S_k/bs)) are
 *    skipped (-1 is the invalid-index value of the Ascend SFA tiling struct)
 *    and a repeated id counts once.  (FSA page: selected attention with
 *    block_size / topk; Ascend SFA blog: gather the top-k K/V rows, then run
 *    ordinary attention on them.)
 *  - Scores s_j = scale * <q, k_j>; LSE = ln sum_j exp(s_j), the natural log
 *    of the softmax normaliser (flash_attn_func docstring, softmax_lse);
 *    O = sum_j exp(s_j - LSE) v_j.  Empty row: O = 0, LSE = -inf.
 *  - Decode: one query per sequence; the list holds cache positions t, read
 *    as a set; t is skipped unless 0 <= t < cache_seqlens[b].  Position t
 *    lives in page block_table[b, t / page_size] at row t % page_size of the
 *    cache [num_pages, page_size, Hkv, d] (flash_attn_with_kvcache
 *    docstring: k_cache / block_table / cache_seqlens).  A position whose
 *    page slot lies beyond max_pages_per_seq or whose page id is outside
 *    [0, num_pages) is skipped as well.
 *  - Merge of partial results over a partition of the key set:
 *    LSE = ln sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i (the split-KV
 *    reduction of the flash-sparse-attn feature list and of the Ascend SFA
 *    decode-reduction core).
 *
 * Inputs q/k/v are bfloat16 bit patterns; they are widened exactly to fp64.
 * All arithmetic is fp64.  Rows are independent and run in parallel (OpenMP).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* Sort and drop repeats in place; returns the new length. */
static int64_t sort_unique(int64_t* v, int64_t n) {
    if (n <= 1) return n;
    qsort(v, (size_t)n, sizeof(int64_t), cmp_i64);
    int64_t w = 1;
    for (int64_t r = 1; r < n; ++r)
        if (v[r] != v[w - 1]) v[w++] = v[r];
    return w;
}

/*
 * Attention of one query row over the key rows found at element offsets
 * key_off[0..nkeys) of k and v (each row d contiguous values).
 * s is scratch of nkeys doubles.
 */
static void attend(const uint16_t* qrow, const uint16_t* k, const uint16_t* v,
                   const int64_t* key_off, int64_t nkeys, int d, double scale,
                   double* s, double* out, double* lse) {
    if (nkeys == 0) {
        for (int c = 0; c < d; ++c) out[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        const uint16_t* kr = k + key_off[j];
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += widen_bf16(qrow[c]) * widen_bf16(kr[c]);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) sum += exp(s[j] - m);
    double L = m + log(sum);
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        double p = exp(s[j] - L);
        const uint16_t* vr = v + key_off[j];
        for (int c = 0; c < d; ++c) out[c] += p * widen_bf16(vr[c]);
    }
    *lse = L;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads later oracle calls use (n <= 0: every core OpenMP sees). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
#else
    (void)n;
#endif
}

/*
 * Prefill.  q [total_q, Hq, d], k/v [total_k, Hkv, d] (bf16 bits),
 * blk_idx [total_q, Hkv, topk], cu_q/cu_k [batch + 1].
 * tokens: global query-token ids to evaluate (NULL: all total_q tokens, then
 * ntok must equal total_q).  out [ntok, Hq, d], lse [ntok, Hq] (fp64).
 * Returns 0, or -1 on bad arguments.
 */
int oracle_selected_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const int32_t* blk_idx, const int32_t* cu_q, const int32_t* cu_k,
                             int32_t batch, int32_t Hq, int32_t Hkv, int32_t d,
                             int32_t block_size, int32_t topk, double scale, int32_t causal,
                             const int64_t* tokens, int64_t ntok, double* out, double* lse) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || block_size <= 0 ||
        topk < 0)
        return -1;
    const int G = Hq / Hkv;
    const int64_t total_q = cu_q[batch];
    if (tokens == NULL && ntok != total_q) return -1;
    int bad = 0;
#pragma omp parallel
    {
        int64_t* blocks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1) *
                                         (size_t)block_size);
        double* s = (double*)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1) *
                                    (size_t)block_size);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < ntok; ++r) {
            int64_t t = tokens ? tokens[r] : r;
            if (t < 0 || t >= total_q) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            /* sequence containing token t */
            int sq_id = 0;
            while (sq_id + 1 < batch && cu_q[sq_id + 1] <= t) ++sq_id;
            const int64_t i = t - cu_q[sq_id];
            const int64_t Sq = cu_q[sq_id + 1] - cu_q[sq_id];
            const int64_t Sk = cu_k[sq_id + 1] - cu_k[sq_id];
            const int64_t nblk = (Sk + block_size - 1) / block_size;
            for (int g = 0; g < Hkv; ++g) {
                /* the selected block set */
                int64_t nb = 0;
                const int32_t* lst = blk_idx + (t * Hkv + g) * (int64_t)topk;
                for (int e = 0; e < topk; ++e)
                    if (lst[e] >= 0 && lst[e] < nblk) blocks[nb++] = lst[e];
                nb = sort_unique(blocks, nb);
                /* the visible keys of those blocks */
                int64_t nk = 0;
                for (int64_t bi = 0; bi < nb; ++bi) {
                    for (int64_t j = blocks[bi] * block_size;
                         j < (blocks[bi] + 1) * block_size && j < Sk; ++j) {
                        if (causal && j > i + Sk - Sq) continue;
                        keys[nk++] = ((cu_k[sq_id] + j) * Hkv + g) * (int64_t)d;
                    }
                }
                for (int hh = 0; hh < G; ++hh) {
                    int h = g * G + hh;
                    attend(q + (t * Hq + h) * (int64_t)d, k, v, keys, nk, d, scale, s,
                           out + (r * Hq + h) * (int64_t)d, lse + r * Hq + h);
                }
            }
        }
        free(blocks);
        free(keys);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Backward of selected attention: the gradients of sum(dO * O) with respect to
 * q, k and v, O being the forward above (the training use of selected
 * attention on the FSA page).  For each row (token i, q head h) with visible
 * key set J (exactly the forward's), P_j = exp(s_j - LSE), O = sum_j P_j v_j
 * and, by the chain rule through the softmax,
 *   D = sum_c dO_c O_c,  dP_j = <dO, v_j>,  dS_j = P_j (dP_j - D),
 *   dq = scale * sum_j dS_j k_j,  dk_j += scale * dS_j q,  dv_j += P_j dO.
 * Inputs as in oracle_selected_attn_fwd plus dout [total_q, Hq, d] (bf16
 * bits); outputs dq [total_q, Hq, d], dk and dv [total_k, Hkv, d] (fp64),
 * every element written (keys no row sees get 0).  Work is split over
 * (sequence, kv head) pairs, whose dk / dv rows are disjoint.
 */
int oracle_selected_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const uint16_t* dout, const int32_t* blk_idx, const int32_t* cu_q,
                             const int32_t* cu_k, int32_t batch, int32_t Hq, int32_t Hkv,
                             int32_t d, int32_t block_size, int32_t topk, double scale,
                             int32_t causal, double* dq, double* dk, double* dv) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || block_size <= 0 ||
        topk < 0)
        return -1;
    const int G = Hq / Hkv;
    const int64_t total_q = cu_q[batch], total_k = cu_k[batch];
    memset(dq, 0, sizeof(double) * (size_t)total_q * Hq * d);
    memset(dk, 0, sizeof(double) * (size_t)total_k * Hkv * d);
    memset(dv, 0, sizeof(double) * (size_t)total_k * Hkv * d);
    const int64_t cap = (int64_t)(topk > 0 ? topk : 1) * block_size;
#pragma omp parallel
    {
        int64_t* blocks = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)cap);
        double* p = (double*)malloc(sizeof(double) * (size_t)cap);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int sq_id = 0; sq_id < batch; ++sq_id) {
            for (int g = 0; g < Hkv; ++g) {
                const int64_t Sq = cu_q[sq_id + 1] - cu_q[sq_id];
                const int64_t Sk = cu_k[sq_id + 1] - cu_k[sq_id];
                const int64_t nblk = (Sk + block_size - 1) / block_size;
                for (int64_t i = 0; i < Sq; ++i) {
                    const int64_t t = cu_q[sq_id] + i;
                    int64_t nb = 0;
                    const int32_t* lst = blk_idx + (t * Hkv + g) * (int64_t)topk;
                    for (int e = 0; e < topk; ++e)
                        if (lst[e] >= 0 && lst[e] < nblk) blocks[nb++] = lst[e];
                    nb = sort_unique(blocks, nb);
                    int64_t nk = 0;
                    for (int64_t bi = 0; bi < nb; ++bi)
                        for (int64_t j = blocks[bi] * block_size;
                             j < (blocks[bi] + 1) * block_size && j < Sk; ++j) {
                            if (causal && j > i + Sk - Sq) continue;
                            keys[nk++] = (cu_k[sq_id] + j) * Hkv + g;     /* key row */
                        }
                    if (nk == 0) continue;
                    for (int hh = 0; hh < G; ++hh) {
                        const int h = g * G + hh;
                        const uint16_t* qr = q + (t * Hq + h) * (int64_t)d;
                        const uint16_t* dor = dout + (t * Hq + h) * (int64_t)d;
                        double m = -INFINITY;
                        for (int64_t j = 0; j < nk; ++j) {
                            const uint16_t* kr = k + keys[j] * d;
                            double dot = 0.0;
                            for (int c = 0; c < d; ++c) dot += widen_bf16(qr[c]) * widen_bf16(kr[c]);
                            p[j] = scale * dot;
                            if (p[j] > m) m = p[j];
                        }
                        double sum = 0.0;
                        for (int64_t j = 0; j < nk; ++j) sum += exp(p[j] - m);
                        const double lse = m + log(sum);
                        for (int c = 0; c < d; ++c) o[c] = 0.0;
                        for (int64_t j = 0; j < nk; ++j) {
                            p[j] = exp(p[j] - lse);
                            const uint16_t* vr = v + keys[j] * d;
                            for (int c = 0; c < d; ++c) o[c] += p[j] * widen_bf16(vr[c]);
                        }
                        double D = 0.0;
                        for (int c = 0; c < d; ++c) D += widen_bf16(dor[c]) * o[c];
                        double* dqr = dq + (t * Hq + h) * (int64_t)d;
                        for (int64_t j = 0; j < nk; ++j) {
                            const uint16_t* kr = k + keys[j] * d;
                            const uint16_t* vr = v + keys[j] * d;
                            double dp = 0.0;
                            for (int c = 0; c < d; ++c) dp += widen_bf16(dor[c]) * widen_bf16(vr[c]);
                            const double ds = p[j] * (dp - D);
                            double* dkr = dk + keys[j] * d;
                            double* dvr = dv + keys[j] * d;
                            for (int c = 0; c < d; ++c) {
                                dqr[c] += scale * ds * widen_bf16(kr[c]);
                                dkr[c] += scale * ds * widen_bf16(qr[c]);
                                dvr[c] += p[j] * widen_bf16(dor[c]);
                            }
                        }
                    }
                }
            }
        }
        free(blocks);
        free(keys);
        free(p);
        free(o);
    }
    return 0;
}

/*
 * Local (sliding-window) attention, dense within the window.  Row i of a
 * sequence with S_q queries and S_k keys attends to every key j with
 *   i + S_k - S_q - left <= j <= i + S_k - S_q + right,   0 <= j < S_k,
 * where a negative left or right leaves that side unlimited (window_size =
 * (left, right) of the flash_attn_func docstring, flash-attention-npu page;
 * (-1, 0) is causal attention, FlashAttention tutorial page section 4.3; the
 * FSA page's sliding-window branch is the causal window (window - 1, 0)).
 * Same layouts and conventions as oracle_selected_attn_fwd.
 */
int oracle_window_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* cu_q, const int32_t* cu_k, int32_t batch, int32_t Hq,
                           int32_t Hkv, int32_t d, int64_t left, int64_t right, double scale,
                           const int64_t* tokens, int64_t ntok, double* out, double* lse) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0) return -1;
    const int G = Hq / Hkv;
    const int64_t total_q = cu_q[batch];
    if (tokens == NULL && ntok != total_q) return -1;
    int64_t max_sk = 1;
    for (int b = 0; b < batch; ++b)
        if (cu_k[b + 1] - cu_k[b] > max_sk) max_sk = cu_k[b + 1] - cu_k[b];
    int bad = 0;
#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)max_sk);
        double* s = (double*)malloc(sizeof(double) * (size_t)max_sk);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < ntok; ++r) {
            int64_t t = tokens ? tokens[r] : r;
            if (t < 0 || t >= total_q) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int sq_id = 0;
            while (sq_id + 1 < batch && cu_q[sq_id + 1] <= t) ++sq_id;
            const int64_t i = t - cu_q[sq_id];
            const int64_t Sq = cu_q[sq_id + 1] - cu_q[sq_id];
            const int64_t Sk = cu_k[sq_id + 1] - cu_k[sq_id];
            const int64_t c = i + Sk - Sq;               /* the row's aligned key position */
            for (int g = 0; g < Hkv; ++g) {
                int64_t nk = 0;
                for (int64_t j = 0; j < Sk; ++j) {
                    if (left >= 0 && j < c - left) continue;
                    if (right >= 0 && j > c + right) continue;
                    keys[nk++] = ((cu_k[sq_id] + j) * Hkv + g) * (int64_t)d;
                }
                for (int hh = 0; hh < G; ++hh) {
                    int h = g * G + hh;
                    attend(q + (t * Hq + h) * (int64_t)d, k, v, keys, nk, d, scale, s,
                           out + (r * Hq + h) * (int64_t)d, lse + r * Hq + h);
                }
            }
        }
        free(keys);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Top-k decode.  q [batch, Hq, d]; k_cache/v_cache [num_pages, page_size, Hkv, d];
 * tok_idx [batch, Hkv, topk]; block_table [batch, max_pages]; cache_seqlens [batch].
 * seqs: batch entries to evaluate (NULL: all, nseq == batch).
 * out [nseq, Hq, d], lse [nseq, Hq].
 */
int oracle_topk_decode(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                       const int32_t* tok_idx, const int32_t* block_table,
                       const int32_t* cache_seqlens, int32_t batch, int32_t Hq, int32_t Hkv,
                       int32_t d, int32_t page_size, int32_t max_pages, int32_t num_pages,
                       int32_t topk, double scale, const int64_t* seqs, int64_t nseq,
                       double* out, double* lse) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || page_size <= 0 ||
        max_pages < 0 || topk < 0)
        return -1;
    if (seqs == NULL && nseq != batch) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < nseq; ++r) {
            for (int g = 0; g < Hkv; ++g) {
                int64_t b = seqs ? seqs[r] : r;
                if (b < 0 || b >= batch) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                const int64_t L = cache_seqlens[b];
                const int32_t* lst = tok_idx + (b * Hkv + g) * (int64_t)topk;
                int64_t n = 0;
                for (int e = 0; e < topk; ++e) {
                    int64_t t = lst[e];
                    if (t < 0 || t >= L) continue;
                    if (t / page_size >= max_pages) continue;
                    int64_t page = block_table[b * max_pages + t / page_size];
                    if (page < 0 || page >= num_pages) continue;
                    pos[n++] = t;
                }
                n = sort_unique(pos, n);
                for (int64_t e = 0; e < n; ++e) {
                    int64_t t = pos[e];
                    int64_t page = block_table[b * max_pages + t / page_size];
                    keys[e] = ((page * page_size + t % page_size) * Hkv + g) * (int64_t)d;
                }
                for (int hh = 0; hh < G; ++hh) {
                    int h = g * G + hh;
                    attend(q + (b * Hq + h) * (int64_t)d, k_cache, v_cache, keys, n, d, scale,
                           s, out + (r * Hq + h) * (int64_t)d, lse + r * Hq + h);
                }
            }
        }
        free(pos);
        free(keys);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * FP8 E4M3 byte -> value, exactly (the torch.float8_e4m3fn format the
 * FlashAttention tutorial page lists among its dtypes: 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
 * subnormals m * 2^-9; no infinities; S.1111.111 is NaN).
 */
static double widen_e4m3(uint8_t bits) {
    const int sgn = bits >> 7, e = (bits >> 3) & 15, m = bits & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -v : v;
}

double oracle_e4m3_value(uint8_t bits) { return widen_e4m3(bits); }

/*
 * Top-k decode over an FP8 (E4M3) paged cache with dequantisation factors
 * (the q_descale / k_descale / v_descale arguments of the FP8 path in the
 * flash-attention-npu page's v3 docstrings; the flash-sparse-attn page's
 * fused-quant decode).  The stored byte x of K (or V) of sequence b, kv head
 * g stands for e4m3(x) * k_descale[b * Hkv + g] (NULL: factor 1); q stays
 * bf16.  Everything else is the bf16 decode above: the list is a set of
 * valid positions, scores s_j = scale * <q, k_j>, LSE = ln sum exp s_j,
 * O = sum exp(s_j - LSE) v_j.
 */
int oracle_topk_decode_fp8(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache,
                           const float* k_descale, const float* v_descale,
                           const int32_t* tok_idx, const int32_t* block_table,
                           const int32_t* cache_seqlens, int32_t batch, int32_t Hq, int32_t Hkv,
                           int32_t d, int32_t page_size, int32_t max_pages, int32_t num_pages,
                           int32_t topk, double scale, const int64_t* seqs, int64_t nseq,
                           double* out, double* lse) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || page_size <= 0 ||
        max_pages < 0 || topk < 0)
        return -1;
    if (seqs == NULL && nseq != batch) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < nseq; ++r) {
            for (int g = 0; g < Hkv; ++g) {
                int64_t b = seqs ? seqs[r] : r;
                if (b < 0 || b >= batch) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                const double kd = k_descale ? (double)k_descale[b * Hkv + g] : 1.0;
                const double vd = v_descale ? (double)v_descale[b * Hkv + g] : 1.0;
                const int64_t L = cache_seqlens[b];
                const int32_t* lst = tok_idx + (b * Hkv + g) * (int64_t)topk;
                int64_t n = 0;
                for (int e = 0; e < topk; ++e) {
                    int64_t t = lst[e];
                    if (t < 0 || t >= L) continue;
                    if (t / page_size >= max_pages) continue;
                    int64_t page = block_table[b * max_pages + t / page_size];
                    if (page < 0 || page >= num_pages) continue;
                    pos[n++] = t;
                }
                n = sort_unique(pos, n);
                for (int hh = 0; hh < G; ++hh) {
                    const int h = g * G + hh;
                    const uint16_t* qrow = q + (b * Hq + h) * (int64_t)d;
                    double* o = out + (r * Hq + h) * (int64_t)d;
                    double* l = lse + r * Hq + h;
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    if (n == 0) {
                        *l = -INFINITY;
                        continue;
                    }
                    double m = -INFINITY;
                    for (int64_t j = 0; j < n; ++j) {
                        const int64_t t = pos[j];
                        const int64_t page = block_table[b * max_pages + t / page_size];
                        const uint8_t* kr =
                            k_cache + ((page * page_size + t % page_size) * Hkv + g) * (int64_t)d;
                        double dot = 0.0;
                        for (int c = 0; c < d; ++c) dot += widen_bf16(qrow[c]) * (widen_e4m3(kr[c]) * kd);
                        s[j] = scale * dot;
                        if (s[j] > m) m = s[j];
                    }
                    double sum = 0.0;
                    for (int64_t j = 0; j < n; ++j) sum += exp(s[j] - m);
                    const double L2 = m + log(sum);
                    for (int64_t j = 0; j < n; ++j) {
                        const int64_t t = pos[j];
                        const int64_t page = block_table[b * max_pages + t / page_size];
                        const uint8_t* vr =
                            v_cache + ((page * page_size + t % page_size) * Hkv + g) * (int64_t)d;
                        const double p = exp(s[j] - L2);
                        for (int c = 0; c < d; ++c) o[c] += p * (widen_e4m3(vr[c]) * vd);
                    }
                    *l = L2;
                }
            }
        }
        free(pos);
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Block-index producer: NSA-style selection of the blocks a query token
 * attends to, from a compressed view of the keys (FSA page, quick start:
 * kernel_size 32 / kernel_stride 16 summaries of the keys, block_size 64,
 * topk, init_blocks, local_blocks).  The pages name these parameters only;
 * each step below is the plain reading stated beside it.
 *
 *  1. Compressed keys.  Window j of a sequence covers keys
 *     [j*stride, j*stride + ksize); windows exist while they fit inside the
 *     sequence.  Its summary is the mean of its ksize keys (per kv head) --
 *     the weight-free form of a learned summary -- stored as bf16 with
 *     round-to-nearest-even: the quick start runs the whole module, and so
 *     every tensor it forms, compressed keys included, in torch.bfloat16
 *     (module .to(torch.bfloat16), bf16 input x), and torch's cast to bf16
 *     rounds to nearest even.
 *  2. Compressed attention.  Row (token i, q head h) sees window j when the
 *     whole window lies in its causal past: j*stride + ksize - 1 <= i + S_k -
 *     S_q.  p_j = softmax over the visible windows of scale * <q, c_j>; a row
 *     with no visible window has p = 0.
 *  3. Block importance.  Each window's probability is spread evenly over its
 *     keys; block b (keys [b*bs, b*bs + bs)) collects the mass of its keys,
 *     summed over the q heads of the kv head's group (the list is shared by
 *     the group):  I[b] = sum_h sum_j p_hj * |window j n block b| / ksize.
 *  4. Selection (the init / local vocabulary of the quick start).  With
 *     qb = floor((i + S_k - S_q) / bs) (no list when negative): blocks
 *     0 .. init-1 (those <= qb), then the local blocks qb, qb-1, ... (local
 *     of them, >= 0, not yet listed), truncated to topk; the remaining slots
 *     take the candidates b in [init, qb - local + 1) of largest I[b], ties
 *     to the smaller b, listed by decreasing importance; -1 pads the rest.
 *
 * q [total_q, Hq, d], k [total_k, Hkv, d] bf16; tokens / ntok as above.
 * blk_idx [ntok, Hkv, topk] int32.  scores: NULL, or [ntok, Hkv, nb_max]
 * fp64 receiving I (0 beyond the sequence's blocks), nb_max =
 * ceil(max S_k / bs).
 */
static uint16_t round_bf16(double x) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int oracle_block_select(const uint16_t* q, const uint16_t* k, const int32_t* cu_q,
                        const int32_t* cu_k, int32_t batch, int32_t Hq, int32_t Hkv, int32_t d,
                        int32_t ksize, int32_t stride, int32_t bs, int32_t topk, int32_t init,
                        int32_t local, double scale, const int64_t* tokens, int64_t ntok,
                        int32_t* blk_idx, double* scores) {
    if (batch < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0 || ksize <= 0 ||
        stride <= 0 || bs <= 0 || topk <= 0 || init < 0 || local < 0)
        return -1;
    const int G = Hq / Hkv;
    const int64_t total_q = cu_q[batch];
    if (tokens == NULL && ntok != total_q) return -1;
    int64_t max_sk = 0;
    for (int b = 0; b < batch; ++b)
        if (cu_k[b + 1] - cu_k[b] > max_sk) max_sk = cu_k[b + 1] - cu_k[b];
    const int64_t nb_max = (max_sk + bs - 1) / bs;
    const int64_t ncmp_max = max_sk >= ksize ? (max_sk - ksize) / stride + 1 : 0;

    /* step 1: compressed keys of every sequence, [batch][ncmp_max][Hkv][d] */
    uint16_t* cmp = (uint16_t*)calloc((size_t)(batch * ncmp_max * Hkv * d) + 1, sizeof(uint16_t));
    if (cmp == NULL) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < batch; ++b)
        for (int64_t j = 0; j < ncmp_max; ++j) {
            const int64_t Sk = cu_k[b + 1] - cu_k[b];
            const int64_t ncmp = Sk >= ksize ? (Sk - ksize) / stride + 1 : 0;
            if (j >= ncmp) continue;
            for (int g = 0; g < Hkv; ++g)
                for (int c = 0; c < d; ++c) {
                    double sum = 0.0;
                    for (int r = 0; r < ksize; ++r)
                        sum += widen_bf16(k[((cu_k[b] + j * stride + r) * Hkv + g) * (int64_t)d + c]);
                    cmp[(((int64_t)b * ncmp_max + j) * Hkv + g) * d + c] = round_bf16(sum / ksize);
                }
        }

    int bad = 0;
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)(ncmp_max + 1));
        double* imp = (double*)malloc(sizeof(double) * (size_t)(nb_max + 1));
        char* used = (char*)malloc((size_t)(nb_max + 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < ntok; ++r) {
            const int64_t t = tokens ? tokens[r] : r;
            if (t < 0 || t >= total_q) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int b = 0;
            while (b + 1 < batch && cu_q[b + 1] <= t) ++b;
            const int64_t i = t - cu_q[b];
            const int64_t Sq = cu_q[b + 1] - cu_q[b];
            const int64_t Sk = cu_k[b + 1] - cu_k[b];
            const int64_t c = i + Sk - Sq;                    /* aligned key position */
            const int64_t nblk = (Sk + bs - 1) / bs;
            const int64_t ncmp = Sk >= ksize ? (Sk - ksize) / stride + 1 : 0;
            int64_t nvis = 0;                                 /* visible windows: 0 .. nvis-1 */
            if (c - ksize + 1 >= 0) nvis = (c - ksize + 1) / stride + 1;
            if (nvis > ncmp) nvis = ncmp;
            for (int g = 0; g < Hkv; ++g) {
                for (int64_t x = 0; x < nblk; ++x) imp[x] = 0.0;
                for (int hh = 0; hh < G && nvis > 0; ++hh) {
                    const int h = g * G + hh;
                    const uint16_t* qr = q + (t * Hq + h) * (int64_t)d;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < nvis; ++j) {              /* step 2 */
                        const uint16_t* cj = cmp + (((int64_t)b * ncmp_max + j) * Hkv + g) * d;
                        double dot = 0.0;
                        for (int e = 0; e < d; ++e) dot += widen_bf16(qr[e]) * widen_bf16(cj[e]);
                        p[j] = scale * dot;
                        if (p[j] > m) m = p[j];
                    }
                    double l = 0.0;
                    for (int64_t j = 0; j < nvis; ++j) {
                        p[j] = exp(p[j] - m);
                        l += p[j];
                    }
                    for (int64_t j = 0; j < nvis; ++j) {              /* step 3 */
                        const int64_t k0 = j * stride, k1 = j * stride + ksize;
                        for (int64_t x = k0 / bs; x * bs < k1 && x < nblk; ++x) {
                            const int64_t lo = k0 > x * bs ? k0 : x * bs;
                            const int64_t hi = k1 < x * bs + bs ? k1 : x * bs + bs;
                            imp[x] += (p[j] / l) * (double)(hi - lo) / ksize;
                        }
                    }
                }
                if (scores != NULL)
                    for (int64_t x = 0; x < nb_max; ++x)
                        scores[(r * Hkv + g) * nb_max + x] = x < nblk ? imp[x] : 0.0;
                /* step 4 */
                int32_t* out = blk_idx + (r * Hkv + g) * (int64_t)topk;
                for (int e = 0; e < topk; ++e) out[e] = -1;
                if (c < 0) continue;
                const int64_t qb = c / bs < nblk - 1 ? c / bs : nblk - 1;
                for (int64_t x = 0; x < nblk; ++x) used[x] = 0;
                int n = 0;
                for (int64_t x = 0; x < init && x <= qb && n < topk; ++x) {
                    out[n++] = (int32_t)x;
                    used[x] = 1;
                }
                for (int64_t y = 0; y < local && n < topk; ++y) {
                    const int64_t x = qb - y;
                    if (x < 0) break;
                    if (used[x]) continue;
                    out[n++] = (int32_t)x;
                    used[x] = 1;
                }
                const int64_t lo = init, hi = qb - local + 1;
                while (n < topk) {
                    int64_t best = -1;
                    for (int64_t x = lo; x < hi; ++x) {
                        if (used[x]) continue;
                        if (best < 0 || imp[x] > imp[best]) best = x;   /* ties: smaller x */
                    }
                    if (best < 0) break;
                    out[n++] = (int32_t)best;
                    used[best] = 1;
                }
            }
        }
        free(p);
        free(imp);
        free(used);
    }
    free(cmp);
    return bad ? -1 : 0;
}

/*
 * Merge n partial results (lse_parts[n], o_parts[n, d]) of one row computed on
 * disjoint key subsets.  An empty part carries LSE = -inf and adds nothing.
 */
void oracle_lse_merge(int64_t n, int32_t d, const double* lse_parts, const double* o_parts,
                      double* lse, double* o) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (lse_parts[i] > m) m = lse_parts[i];
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (m == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double sum = 0.0;
    for (int64_t i = 0; i < n; ++i) sum += exp(lse_parts[i] - m);
    double L = m + log(sum);
    for (int64_t i = 0; i < n; ++i) {
        double w = exp(lse_parts[i] - L);
        for (int c = 0; c < d; ++c) o[c] += w * o_parts[i * d + c];
    }
    *lse = L;
}
