/*
 * CPU oracle for the CSA2 hierarchical sparse attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * HIP path is checked against.  It shares no code, header, table or constant
 * with the HIP library; only the tests, the smoke check and the benchmark's CPU
 * baseline may load it.
 *
 * Sources (DeepSeek-V4.1-Flash write-ups):
 *   [P2] fupanwang.com article, section "三个方向一起压小缓存" (the three layer
 *        modes, the hierarchical sparse indexer and its figure caption, the FP4
 *        indexer, OCP MXFP4 main KV, FP8 sliding-window KV); section
 *        "后 20 层干脆共用一份 KV" (128-token sliding window).
 *   [P3] dreamax.pages.dev notes, CSA2 paragraph (Full / Reindex / Reuse).
 * Numeric rules the pages leave open are fixed as follows (each is one of the
 * readings listed in the design notes):
 *   - indexer score = one 128-d dot product of the FP4 query and key, with each
 *     32-element block summed exactly (integers in half-units) and the four
 *     scaled block sums added in fp32 in block order ((v0+v1)+v2)+v3;
 *   - blocks are 8 aligned positions; a block's score is the maximum over its
 *     visible positions; blocks and positions rank by (score desc, id asc);
 *   - the pool keeps min(n_pool, #blocks) blocks; top-k keeps min(k, #pool);
 *     outputs are ascending and padded with -1;
 *   - attention: one softmax over the selected latent rows and the window rows,
 *     value = key, scale sm_scale, computed in double, stored as float.
 *   - scores compare by their IEEE-754 total order (-0 below +0).
 *   - cache write: an entry at ratio m is the weighted sum of its m token rows
 *     with the caller's per-token weights, in fp32, tokens in order, each
 *     product rounded before its addition; the sum is then stored with the
 *     MXFP4 encoder below (NaN elements do not count towards amax, an infinite
 *     amax takes E = 127).
 *
 * Pins: every function here is checked in tests/ against brute force, closed
 * forms, library routines or published format tables (see the test docstrings).
 */
#include "csa2_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* O1-O2: E2M1 and E8M0 (OCP Microscaling Formats v1.0)               */
/* ------------------------------------------------------------------ */

/* E2M1 code -> value.  bit3 sign, bits 2..1 exponent (bias 1), bit0 mantissa. */
static const double kE2M1[16] = {
    0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0};

double orc_e2m1_value(unsigned code) { return kE2M1[code & 15u]; }

/* E2M1 code -> value in half-units (value * 2), an integer in [-12, 12]. */
static int e2m1_half_units(unsigned code) { return (int)(kE2M1[code & 15u] * 2.0); }

/* E8M0 byte -> 2^(byte-127); 0xFF is NaN. */
double orc_e8m0_scale(unsigned byte) {
    if ((byte & 255u) == 255u) return NAN;
    return ldexp(1.0, (int)(byte & 255u) - 127);
}

/* FP8 E4M3 (OCP E4M3FN): bias 7, 3 mantissa bits, S.1111.111 is NaN, no inf. */
double orc_e4m3_value(unsigned code) {
    code &= 255u;
    double sign = (code & 0x80u) ? -1.0 : 1.0;
    unsigned e = (code >> 3) & 15u, m = code & 7u;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) return sign * ldexp((double)m, -9);          /* subnormal: m/8 * 2^-6 */
    return sign * ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

/* O3: MXFP4 encode of one 32-element block (rule E = floor(log2 amax) - 2). */
void orc_mxfp4_encode_block(const double* x, uint8_t* codes16, uint8_t* scale) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
    if (amax == 0.0) {
        for (int i = 0; i < 16; ++i) codes16[i] = 0;
        *scale = 0;
        return;
    }
    int E = ilogb(amax) - 2;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
    *scale = (uint8_t)(E + 127);
    for (int i = 0; i < 32; ++i) {
        double y = x[i] / ldexp(1.0, E);
        /* nearest of the 8 non-negative E2M1 values; on a tie take the even
           mantissa (code bit 0 clear); beyond 6 saturate */
        int best = 0;
        for (int c = 1; c < 8; ++c) {
            double dc = fabs(fabs(y) - kE2M1[c]), db = fabs(fabs(y) - kE2M1[best]);
            if (dc < db || (dc == db && (c % 2) == 0)) best = c;
        }
        if (fabs(y) >= 6.0) best = 7;
        unsigned code = (unsigned)best;
        if (y < 0.0 && best != 0) code |= 8u;
        if (i % 2 == 0) codes16[i / 2] = (uint8_t)code;
        else codes16[i / 2] = (uint8_t)(codes16[i / 2] | (code << 4));
    }
}

/* O4: E4M3 encode, round to nearest even over the table of finite values. */
uint8_t orc_e4m3_encode(double x) {
    if (isnan(x)) return 0x7F;
    if (x >= 448.0) return 0x7E;
    if (x <= -448.0) return 0xFE;
    int best = -1;
    double bestd = 0.0;
    for (int c = 0; c < 256; ++c) {
        double v = orc_e4m3_value((unsigned)c);
        if (isnan(v)) continue;
        if ((signbit(v) != 0) != (signbit(x) != 0)) continue;   /* same sign only */
        double d = fabs(x - v);
        if (best < 0 || d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------ */
/* O5: indexer score                                                  */
/* ------------------------------------------------------------------ */
float orc_score(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc, const uint8_t* ks) {
    float v[4];
    for (int b = 0; b < 4; ++b) {
        int isum = 0;                                 /* exact, |isum| <= 32*144 */
        for (int i = 32 * b; i < 32 * b + 32; ++i) {
            unsigned cq = (i % 2 == 0) ? (qc[i / 2] & 15u) : (qc[i / 2] >> 4);
            unsigned ck = (i % 2 == 0) ? (kc[i / 2] & 15u) : (kc[i / 2] >> 4);
            isum += e2m1_half_units(cq) * e2m1_half_units(ck);
        }
        /* (hq/2 * 2^(eq-127)) * (hk/2 * 2^(ek-127)) summed = isum * 2^(eq+ek-256) */
        int e = (int)qs[b] + (int)ks[b] - 256;
        v[b] = ldexpf((float)isum, e);
    }
    volatile float s = v[0] + v[1];
    s = s + v[2];
    s = s + v[3];
    float out = s;
    /* A score that is not a number (two block values overflowing to opposite
       infinities) is the positive quiet NaN 0x7FC00000, whatever NaN the host's
       adder produced, so that its place in the total order is fixed. */
    if (isnan(out)) {
        uint32_t u = 0x7FC00000u;
        memcpy(&out, &u, 4);
    }
    return out;
}

/* ------------------------------------------------------------------ */
/* ordering helpers                                                   */
/* ------------------------------------------------------------------ */
/* IEEE-754 total order of a float as an unsigned key (larger key = larger). */
uint32_t orc_order_key(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef struct { uint32_t key; int64_t id; } ranked_t;

/* (key desc, id asc) */
static int cmp_rank(const void* a, const void* b) {
    const ranked_t* x = (const ranked_t*)a;
    const ranked_t* y = (const ranked_t*)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    if (x->id != y->id) return x->id < y->id ? -1 : 1;
    return 0;
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

/* Keep the first k of the ranked list, emit their ids ascending, pad with -1. */
static void emit_first_k_ascending(ranked_t* r, int64_t n, int64_t k, int32_t* out, int64_t out_len) {
    qsort(r, (size_t)n, sizeof(ranked_t), cmp_rank);
    int64_t keep = k < n ? k : n;
    int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (size_t)(keep > 0 ? keep : 1));
    for (int64_t i = 0; i < keep; ++i) ids[i] = r[i].id;
    qsort(ids, (size_t)keep, sizeof(int64_t), cmp_i64);
    for (int64_t i = 0; i < out_len; ++i) out[i] = i < keep ? (int32_t)ids[i] : -1;
    free(ids);
}

/* ------------------------------------------------------------------ */
/* simple thread pool over rows                                       */
/* ------------------------------------------------------------------ */
typedef void (*row_fn)(void* ctx, int64_t row);
typedef struct { row_fn fn; void* ctx; int64_t n; int64_t next; pthread_mutex_t mu; } pool_t;

static void* pool_worker(void* arg) {
    pool_t* p = (pool_t*)arg;
    for (;;) {
        pthread_mutex_lock(&p->mu);
        int64_t r = p->next++;
        pthread_mutex_unlock(&p->mu);
        if (r >= p->n) break;
        p->fn(p->ctx, r);
    }
    return NULL;
}

static void parallel_rows(row_fn fn, void* ctx, int64_t n, int threads) {
    pool_t p;
    p.fn = fn; p.ctx = ctx; p.n = n; p.next = 0;
    pthread_mutex_init(&p.mu, NULL);
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > n) threads = (int)(n > 0 ? n : 1);
    pthread_t tid[256];
    int started = 0;
    for (int t = 1; t < threads; ++t)
        if (pthread_create(&tid[started], NULL, pool_worker, &p) == 0) ++started;
    pool_worker(&p);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------ */
/* O5-O8: Full layer                                                   */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint8_t *qc, *qs, *kc, *ks;
    const int32_t* n_visible;
    int M; int64_t N_max; int n_pool; int k;
    float* scores; float* block_max; int32_t* pool_blocks; int32_t* idx;
    int64_t nblk_max;
    int global_topk;
    float** pre;              /* when set: each row's scores, computed beforehand */
    int64_t parts;            /* position ranges per row when scoring beforehand */
} full_ctx;

/* O5 for row r over positions [j0, j1): s[j] for each of them. */
static void score_range(const full_ctx* c, int64_t r, int64_t j0, int64_t j1, float* s) {
    int64_t seq = r / c->M;
    const uint8_t* qc = c->qc + r * 64;
    const uint8_t* qs = c->qs + r * 4;
    const uint8_t* kc = c->kc + seq * c->N_max * 64;
    const uint8_t* ks = c->ks + seq * c->N_max * 4;
    for (int64_t j = j0; j < j1; ++j) s[j] = orc_score(qc, qs, kc + j * 64, ks + j * 4);
}

/* Task t of the scoring beforehand: part t % parts of row t / parts. */
static void score_part(void* vctx, int64_t t) {
    full_ctx* c = (full_ctx*)vctx;
    int64_t r = t / c->parts, part = t % c->parts;
    int64_t nv = c->n_visible[r];
    score_range(c, r, nv * part / c->parts, nv * (part + 1) / c->parts, c->pre[r]);
}

static void full_row(void* vctx, int64_t r) {
    full_ctx* c = (full_ctx*)vctx;
    int64_t nv = c->n_visible[r];
    /* O5: every visible position */
    float* s = c->pre ? c->pre[r] : (float*)malloc(sizeof(float) * (size_t)(nv > 0 ? nv : 1));
    if (!c->pre) score_range(c, r, 0, nv, s);
    if (c->scores)
        for (int64_t j = 0; j < nv; ++j) c->scores[r * c->N_max + j] = s[j];
    /* O6: block b = positions [8b, 8b+8) that are visible; max by total order */
    int64_t nblk = (nv + 7) / 8;
    ranked_t* blocks = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(nblk > 0 ? nblk : 1));
    for (int64_t b = 0; b < nblk; ++b) {
        uint32_t best = 0;
        float bestf = 0.f;
        for (int64_t j = 8 * b; j < 8 * b + 8 && j < nv; ++j) {
            if (j == 8 * b || orc_order_key(s[j]) > best) { best = orc_order_key(s[j]); bestf = s[j]; }
        }
        blocks[b].key = best;
        blocks[b].id = b;
        if (c->block_max) c->block_max[r * c->nblk_max + b] = bestf;
    }
    /* O7: pool = first min(n_pool, nblk) blocks by (max desc, id asc) */
    int32_t* pool = c->pool_blocks + r * c->n_pool;
    emit_first_k_ascending(blocks, nblk, c->n_pool, pool, c->n_pool);
    if (c->idx && c->k > 0) {
        /* O8: top-k over the pool's visible positions by (score desc, pos asc).
           With global_topk set, rank every visible position instead (the two are
           equal for a Full layer when the pool keeps >= k blocks). */
        ranked_t* cand = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(nv > 0 ? nv : 1));
        int64_t nc = 0;
        if (c->global_topk) {
            for (int64_t j = 0; j < nv; ++j) { cand[nc].key = orc_order_key(s[j]); cand[nc].id = j; ++nc; }
        } else {
            for (int i = 0; i < c->n_pool; ++i) {
                if (pool[i] < 0) continue;
                for (int64_t j = 8 * (int64_t)pool[i]; j < 8 * (int64_t)pool[i] + 8 && j < nv; ++j) {
                    cand[nc].key = orc_order_key(s[j]);
                    cand[nc].id = j;
                    ++nc;
                }
            }
        }
        emit_first_k_ascending(cand, nc, c->k, c->idx + r * c->k, c->k);
        free(cand);
    }
    free(blocks);
    if (!c->pre) free(s);
}

int orc_index_full(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const int32_t* n_visible, int B, int M, int64_t N_max,
                   int n_pool, int k, float* scores, float* block_max, int32_t* pool_blocks,
                   int32_t* idx, int global_topk, int threads) {
    if (B < 0 || M < 0 || N_max < 0 || n_pool < 0 || k < 0 || !pool_blocks) return -1;
    for (int64_t r = 0; r < (int64_t)B * M; ++r)
        if (n_visible[r] < 0 || n_visible[r] > N_max) return -1;
    full_ctx c = {q_codes, q_scales, k_codes, k_scales, n_visible, M, N_max, n_pool, k,
                  scores, block_max, pool_blocks, idx, (N_max + 7) / 8, global_topk, NULL, 1};
    int64_t R = (int64_t)B * M;
    if (threads > R && R > 0) {
        /* fewer rows than threads: score each row's position ranges on all of
           them first, then run the rest of each row (O6-O8) as usual */
        c.parts = (4 * (int64_t)threads + R - 1) / R;
        c.pre = (float**)malloc(sizeof(float*) * (size_t)R);
        for (int64_t r = 0; r < R; ++r)
            c.pre[r] = (float*)malloc(sizeof(float) * (size_t)(n_visible[r] > 0 ? n_visible[r] : 1));
        parallel_rows(score_part, &c, R * c.parts, threads);
        parallel_rows(full_row, &c, R, threads);
        for (int64_t r = 0; r < R; ++r) free(c.pre[r]);
        free(c.pre);
        return 0;
    }
    parallel_rows(full_row, &c, R, threads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O9: Reindex - score only the pool's positions                      */
/* ------------------------------------------------------------------ */
typedef struct {
    const uint8_t *qc, *qs, *kc, *ks;
    const int32_t *pool_blocks, *n_visible;
    int n_pool, M; int64_t N_max;
    float* pool_scores;
} pool_ctx;

static void pool_row(void* vctx, int64_t r) {
    pool_ctx* c = (pool_ctx*)vctx;
    int64_t seq = r / c->M;
    int64_t nv = c->n_visible[r];
    for (int i = 0; i < c->n_pool; ++i) {
        int64_t b = c->pool_blocks[r * c->n_pool + i];
        for (int t = 0; t < 8; ++t) {
            int64_t j = 8 * b + t;
            float v = -INFINITY;
            if (b >= 0 && j < nv)
                v = orc_score(c->qc + r * 64, c->qs + r * 4, c->kc + (seq * c->N_max + j) * 64,
                              c->ks + (seq * c->N_max + j) * 4);
            c->pool_scores[(r * c->n_pool + i) * 8 + t] = v;
        }
    }
}

int orc_index_pool(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                   const uint8_t* k_scales, const int32_t* pool_blocks, int n_pool,
                   const int32_t* n_visible, int B, int M, int64_t N_max, float* pool_scores, int threads) {
    if (B < 0 || M < 0 || n_pool < 0) return -1;
    pool_ctx c = {q_codes, q_scales, k_codes, k_scales, pool_blocks, n_visible, n_pool, M, N_max, pool_scores};
    parallel_rows(pool_row, &c, (int64_t)B * M, threads);
    return 0;
}

/* O8 over a pool-score array: slot 8i+t is position 8*pool[i]+t when pool[i]
   >= 0 and the position is visible. */
typedef struct {
    const float* pool_scores; const int32_t* pool_blocks; const int32_t* n_visible;
    int n_pool, k; int32_t* idx;
} topk_ctx;

static void topk_row(void* vctx, int64_t r) {
    topk_ctx* c = (topk_ctx*)vctx;
    ranked_t* cand = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(8 * c->n_pool + 1));
    int64_t nc = 0, nv = c->n_visible[r];
    for (int i = 0; i < c->n_pool; ++i) {
        int64_t b = c->pool_blocks[r * c->n_pool + i];
        if (b < 0) continue;
        for (int t = 0; t < 8; ++t) {
            int64_t j = 8 * b + t;
            if (j >= nv) continue;
            cand[nc].key = orc_order_key(c->pool_scores[(r * c->n_pool + i) * 8 + t]);
            cand[nc].id = j;
            ++nc;
        }
    }
    emit_first_k_ascending(cand, nc, c->k, c->idx + r * c->k, c->k);
    free(cand);
}

int orc_topk_pool(const float* pool_scores, const int32_t* pool_blocks, int n_pool,
                  const int32_t* n_visible, int64_t R, int k, int32_t* idx, int threads) {
    if (R < 0 || n_pool < 0 || k < 0) return -1;
    topk_ctx c = {pool_scores, pool_blocks, n_visible, n_pool, k, idx};
    parallel_rows(topk_row, &c, R, threads);
    return 0;
}

/* O8 over a full score array [R][N_max], positions < n_visible. */
typedef struct { const float* scores; const int32_t* n_visible; int64_t N_max; int k; int32_t* idx; } topkf_ctx;

static void topkf_row(void* vctx, int64_t r) {
    topkf_ctx* c = (topkf_ctx*)vctx;
    int64_t nv = c->n_visible[r];
    ranked_t* cand = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(nv > 0 ? nv : 1));
    for (int64_t j = 0; j < nv; ++j) { cand[j].key = orc_order_key(c->scores[r * c->N_max + j]); cand[j].id = j; }
    emit_first_k_ascending(cand, nv, c->k, c->idx + r * c->k, c->k);
    free(cand);
}

int orc_topk_full(const float* scores, const int32_t* n_visible, int64_t R, int64_t N_max, int k,
                  int32_t* idx, int threads) {
    if (R < 0 || k < 0) return -1;
    topkf_ctx c = {scores, n_visible, N_max, k, idx};
    parallel_rows(topkf_row, &c, R, threads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O11: sparse + window attention in double                           */
/* ------------------------------------------------------------------ */
typedef struct {
    const float* q; const uint8_t *cc, *cs; const int32_t* idx; int k;
    const uint8_t* win; const int32_t *win_start, *win_len; int win_max;
    int M, H, Tw; int64_t N_max; float sm_scale; float* out;
} attn_ctx;

static void decode_latent_row(const uint8_t* codes, const uint8_t* scales, double* v) {
    for (int i = 0; i < 512; ++i) {
        unsigned code = (i % 2 == 0) ? (codes[i / 2] & 15u) : (codes[i / 2] >> 4);
        v[i] = orc_e2m1_value(code) * orc_e8m0_scale(scales[i / 32]);
    }
}

/* The row's attention set: the decoded values of its entries in order, the
   selected latent rows then the window rows; returns how many (vals holds room
   for k + win_max rows). */
static int row_values(const attn_ctx* c, int64_t r, double* vals) {
    int64_t seq = r / c->M;
    /* the row's window: rows win_start .. win_start + n - 1 of its sequence's
       window store, n = min(win_len, win_max) (a negative length is empty) */
    int nw = c->win_max > 0 ? c->win_len[r] : 0;
    if (nw < 0) nw = 0;
    if (nw > c->win_max) nw = c->win_max;
    int ne = 0;
    /* the selected latent rows (value = key); an index outside the cache
       [0, N_max) names no entry and is left out */
    for (int j = 0; j < c->k; ++j) {
        int64_t p = c->idx[r * c->k + j];
        if (p < 0 || p >= c->N_max) continue;
        const uint8_t* codes = c->cc + (seq * c->N_max + p) * 256;
        const uint8_t* scales = c->cs + (seq * c->N_max + p) * 16;
        decode_latent_row(codes, scales, vals + 512 * (size_t)ne);
        ++ne;
    }
    /* the sliding-window rows (FP8, value = key); a row outside the window
       store [0, Tw) names no entry and is left out */
    for (int t = 0; t < nw; ++t) {
        int64_t wr = (int64_t)c->win_start[r] + t;
        if (wr < 0 || wr >= c->Tw) continue;
        const uint8_t* row = c->win + (seq * (int64_t)c->Tw + wr) * 512;
        for (int i = 0; i < 512; ++i) vals[512 * (size_t)ne + i] = orc_e4m3_value(row[i]);
        ++ne;
    }
    return ne;
}

/* O11 for head h of row r over the row's ne values; z: room for ne doubles. */
static void attn_head(const attn_ctx* c, int64_t r, int h, const double* vals, int ne, double* z) {
    const float* qh = c->q + (r * c->H + h) * 512;
    float* oh = c->out + (r * c->H + h) * 512;
    if (ne == 0) {
        for (int d = 0; d < 512; ++d) oh[d] = 0.f;
        return;
    }
    double m = -INFINITY;
    for (int i = 0; i < ne; ++i) {
        double dot = 0.0;
        for (int d = 0; d < 512; ++d) dot += (double)qh[d] * vals[512 * (size_t)i + d];
        z[i] = dot * (double)c->sm_scale;
        if (z[i] > m) m = z[i];
    }
    double l = 0.0;
    for (int i = 0; i < ne; ++i) { z[i] = exp(z[i] - m); l += z[i]; }
    for (int d = 0; d < 512; ++d) {
        double o = 0.0;
        for (int i = 0; i < ne; ++i) o += z[i] * vals[512 * (size_t)i + d];
        oh[d] = (float)(o / l);
    }
}

static size_t row_capacity(const attn_ctx* c) {
    int cap = c->k + (c->win_max > 0 ? c->win_max : 0);
    return (size_t)(cap > 0 ? cap : 1);
}

static void attn_row(void* vctx, int64_t r) {
    attn_ctx* c = (attn_ctx*)vctx;
    double* vals = (double*)malloc(sizeof(double) * 512 * row_capacity(c));
    double* z = (double*)malloc(sizeof(double) * row_capacity(c));
    int ne = row_values(c, r, vals);
    for (int h = 0; h < c->H; ++h) attn_head(c, r, h, vals, ne, z);
    free(z);
    free(vals);
}

/* Fewer rows than threads: each row's values decoded first (task = row), then
   one task per (row, head). */
typedef struct { attn_ctx* c; double** vals; int* ne; } attn_split_ctx;

static void attn_decode_task(void* vctx, int64_t r) {
    attn_split_ctx* a = (attn_split_ctx*)vctx;
    a->ne[r] = row_values(a->c, r, a->vals[r]);
}

static void attn_head_task(void* vctx, int64_t t) {
    attn_split_ctx* a = (attn_split_ctx*)vctx;
    int64_t r = t / a->c->H;
    int h = (int)(t % a->c->H);
    double* z = (double*)malloc(sizeof(double) * row_capacity(a->c));
    attn_head(a->c, r, h, a->vals[r], a->ne[r], z);
    free(z);
}

int orc_sparse_attn(const float* q, const uint8_t* c_codes, const uint8_t* c_scales, const int32_t* idx,
                    int k, const uint8_t* win, const int32_t* win_start, const int32_t* win_len, int win_max,
                    int B, int M, int64_t N_max, int H, int Tw, float sm_scale, float* out, int threads) {
    if (B < 0 || M < 0 || H <= 0 || k < 0 || Tw < 0 || win_max < 0) return -1;
    attn_ctx c = {q, c_codes, c_scales, idx, k, win, win_start, win_len, win_max, M, H, Tw, N_max, sm_scale, out};
    int64_t R = (int64_t)B * M;
    if (threads > R && R > 0) {
        attn_split_ctx a = {&c, (double**)malloc(sizeof(double*) * (size_t)R), (int*)malloc(sizeof(int) * (size_t)R)};
        for (int64_t r = 0; r < R; ++r) a.vals[r] = (double*)malloc(sizeof(double) * 512 * row_capacity(&c));
        parallel_rows(attn_decode_task, &a, R, threads);
        parallel_rows(attn_head_task, &a, R * H, threads);
        for (int64_t r = 0; r < R; ++r) free(a.vals[r]);
        free(a.vals);
        free(a.ne);
        return 0;
    }
    parallel_rows(attn_row, &c, R, threads);
    return 0;
}

/* ------------------------------------------------------------------ */
/* O13: cache write (CSA2 ratio-m compression, quantize-on-write)      */
/* ------------------------------------------------------------------ */
/* [P2] every m consecutive tokens are stored as one entry, a merge weighted by
   the layer's compression weights, entries do not overlap; entry e of row
   length D is sum_j w[m e + j] x[m e + j], j = 0..m-1, in fp32 in that order
   (this file is compiled without contraction, so the product and the sum are
   two roundings).  w == NULL means every weight is 1. */
int orc_merge_f32(const float* x, const float* w, int64_t n_entries, int ratio, int D, float* out) {
    if (n_entries < 0 || ratio < 1 || D < 1) return -1;
    for (int64_t e = 0; e < n_entries; ++e) {
        for (int d = 0; d < D; ++d) {
            float s = 0.0f;
            for (int j = 0; j < ratio; ++j) {
                int64_t tok = e * ratio + j;
                float wj = w ? w[tok] : 1.0f;
                float p = x[tok * (int64_t)D + d] * wj;
                s = (j == 0) ? p : s + p;
            }
            out[e * (int64_t)D + d] = s;
        }
    }
    return 0;
}

/* [P2] the main KV and indexer keys are stored in MXFP4: the merged entries
   through O3, 32 elements at a time (a float is exact as a double). */
int orc_cache_write_mxfp4(const float* x, const float* w, int64_t n_entries, int ratio, int D, uint8_t* codes,
                          uint8_t* scales) {
    if (D < 32 || D % 32 != 0) return -1;
    float* m = (float*)malloc(sizeof(float) * (size_t)D);
    if (!m) return -2;
    double blk[32];
    for (int64_t e = 0; e < n_entries; ++e) {
        if (orc_merge_f32(x + e * (int64_t)ratio * D, w ? w + e * ratio : NULL, 1, ratio, D, m) != 0) {
            free(m);
            return -1;
        }
        for (int b = 0; b < D / 32; ++b) {
            for (int i = 0; i < 32; ++i) blk[i] = (double)m[32 * b + i];
            orc_mxfp4_encode_block(blk, codes + e * (int64_t)(D / 2) + 16 * b, scales + e * (int64_t)(D / 32) + b);
        }
    }
    free(m);
    return 0;
}

/* [P2] the sliding-window KV is stored in FP8: every value through O4. */
void orc_cache_write_e4m3(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode((double)x[i]);
}
