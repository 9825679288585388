/*
 * Seeded synthetic inputs for the CSA2 hierarchical sparse attention step.
 *
 * This module only prepares data: it draws iid N(0,1) values and stores them in
 * the storage formats the cached state uses on the pages (DeepSeek-V4.1-Flash
 * write-up on fupanwang.com, section "三个方向一起压小缓存": indexer query/key in
 * FP4, main KV in OCP MXFP4, sliding-window KV in FP8).  It performs none of the
 * attention step's arithmetic (no scoring, selection or softmax).
 *
 * Random numbers: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11) with the published round constants,
 * followed by the Box-Muller transform in double precision.  Every normal is a
 * pure function of (seed, tensor id, row, column), so any slice of any tensor can
 * be regenerated independently and the output does not depend on the thread
 * count.
 *
 * Storage encodings used here (input preparation only):
 *   MXFP4 (OCP Microscaling Formats spec v1.0): blocks of 32 elements share an
 *     E8M0 scale byte 127+E with E = floor(log2(amax)) - 2 (E2M1's largest
 *     exponent is 2); each element is x/2^E rounded to the nearest E2M1 value,
 *     ties to the even mantissa, saturating at +-6.  Element 2i is the low
 *     nibble of byte i.  An all-zero block stores scale byte 0.
 *   FP8 E4M3 (OCP "E4M3FN"): bias 7, no infinities, max 448; round to nearest
 *     even, saturate to +-448.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox-4x32-10 ---------------- */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += PHILOX_W0;
        k1 += PHILOX_W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void synth_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
    philox4x32_10(ctr, key, out);
}

/* Four normals for counter (col/4, row_lo, row_hi, tensor). */
static void normals4(uint64_t seed, uint32_t tensor, uint64_t row, uint64_t col4, double z[4]) {
    uint32_t ctr[4] = {(uint32_t)col4, (uint32_t)row, (uint32_t)(row >> 32), tensor};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t x[4];
    philox4x32_10(ctr, key, x);
    const double two32 = 4294967296.0;
    const double twopi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)x[2 * p] + 1.0) / two32;   /* (0, 1] */
        double u2 = (double)x[2 * p + 1] / two32;       /* [0, 1) */
        double r = sqrt(-2.0 * log(u1));
        z[2 * p] = r * cos(twopi * u2);
        z[2 * p + 1] = r * sin(twopi * u2);
    }
}

/* One row of `cols` normals (cols a multiple of 4). */
static void normal_row(uint64_t seed, uint32_t tensor, uint64_t row, int cols, double* out) {
    double z[4];
    for (int c = 0; c < cols; c += 4) {
        normals4(seed, tensor, row, (uint64_t)(c / 4), z);
        out[c] = z[0]; out[c + 1] = z[1]; out[c + 2] = z[2]; out[c + 3] = z[3];
    }
}

/* ---------------- storage encoders (input preparation) ---------------- */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* nearest E2M1 magnitude index for |y|, ties to even mantissa, saturating */
static unsigned e2m1_mag_index(double a) {
    if (!(a < 6.0)) return 7;
    unsigned best = 0;
    double bestd = a;
    for (unsigned i = 1; i < 8; ++i) {
        double d = fabs(a - kE2M1Mag[i]);
        if (d < bestd || (d == bestd && (i & 1u) == 0u)) { best = i; bestd = d; }
    }
    return best;
}

void synth_mxfp4_encode_block(const double* x, uint8_t* codes16, uint8_t* scale) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) { double a = fabs(x[i]); if (a > amax) amax = a; }
    if (amax == 0.0) {
        memset(codes16, 0, 16);
        *scale = 0;
        return;
    }
    int e = ilogb(amax) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (uint8_t)(e + 127);
    for (int i = 0; i < 32; i += 2) {
        unsigned c[2];
        for (int j = 0; j < 2; ++j) {
            double y = ldexp(x[i + j], -e);
            unsigned m = e2m1_mag_index(fabs(y));
            c[j] = m | ((y < 0.0 && m != 0) ? 8u : 0u);
        }
        codes16[i / 2] = (uint8_t)(c[0] | (c[1] << 4));
    }
}

uint8_t synth_e4m3_encode(double x) {
    if (x != x) return 0x7F;
    unsigned sign = signbit(x) ? 0x80u : 0u;
    double a = fabs(x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    /* candidate grid: exponent field 0 (subnormal, step 2^-9) or 1..15 */
    int e = (a < 0.015625) ? -6 : ilogb(a);       /* 2^-6 is the smallest normal */
    if (e < -6) e = -6;
    double step = ldexp(1.0, e - 3);
    double q = a / step;                             /* exact: power-of-two division */
    double fl = floor(q);
    double fr = q - fl;
    double m = fl;
    if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) m = fl + 1.0;
    double v = m * step;
    if (v >= 448.0) return (uint8_t)(sign | 0x7E);
    if (v == 0.0) return (uint8_t)sign;
    /* re-derive fields from the exact value v */
    int ev = ilogb(v);
    unsigned code;
    if (ev < -6) {
        code = (unsigned)(v / ldexp(1.0, -9));         /* subnormal mantissa 1..7 */
    } else {
        unsigned mant = (unsigned)((v / ldexp(1.0, ev) - 1.0) * 8.0);
        code = ((unsigned)(ev + 7) << 3) | mant;
    }
    return (uint8_t)(sign | code);
}

/* ---------------- tensor generators ---------------- */
typedef struct {
    uint64_t seed;
    uint32_t tensor;
    uint64_t row0, nrows;     /* rows [row0, row0+nrows) of the logical tensor */
    int cols;
    int kind;                 /* 0 mxfp4, 1 e4m3, 2 f32, 3 mxfp4 ratio-2 merged */
    uint32_t logit_tensor;    /* kind 3: tensor id of the per-token merge logits */
    uint8_t* codes; uint8_t* scales; uint8_t* bytes; float* f32;
    uint64_t t0, t1;          /* thread's row range (relative) */
} job_t;

void synth_merge_weights(uint64_t seed, uint32_t logit_tensor, uint64_t row, double* w);

static void merged_row(const job_t* j, uint64_t row, double* out, double* tmp) {
    /* entry row = w0 * token(2row) + w1 * token(2row+1); w = softmax(l0, l1) */
    double w[2];
    synth_merge_weights(j->seed, j->logit_tensor, row, w);
    normal_row(j->seed, j->tensor, 2 * row, j->cols, out);
    normal_row(j->seed, j->tensor, 2 * row + 1, j->cols, tmp);
    for (int c = 0; c < j->cols; ++c) out[c] = w[0] * out[c] + w[1] * tmp[c];
}

static void* run_job(void* arg) {
    job_t* j = (job_t*)arg;
    double* row = (double*)malloc(sizeof(double) * (size_t)j->cols * 2);
    double* tmp = row + j->cols;
    for (uint64_t r = j->t0; r < j->t1; ++r) {
        uint64_t g = j->row0 + r;
        if (j->kind == 3) merged_row(j, g, row, tmp);
        else normal_row(j->seed, j->tensor, g, j->cols, row);
        if (j->kind == 0 || j->kind == 3) {
            int nb = j->cols / 32;
            for (int b = 0; b < nb; ++b)
                synth_mxfp4_encode_block(row + 32 * b, j->codes + r * (uint64_t)(j->cols / 2) + 16 * b,
                                         j->scales + r * (uint64_t)nb + b);
        } else if (j->kind == 1) {
            for (int c = 0; c < j->cols; ++c) j->bytes[r * (uint64_t)j->cols + c] = synth_e4m3_encode(row[c]);
        } else {
            for (int c = 0; c < j->cols; ++c) j->f32[r * (uint64_t)j->cols + c] = (float)row[c];
        }
    }
    free(row);
    return NULL;
}

static int run_threads(job_t proto, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if ((uint64_t)threads > proto.nrows) threads = proto.nrows ? (int)proto.nrows : 1;
    pthread_t tid[64];
    job_t jobs[64];
    uint64_t per = (proto.nrows + threads - 1) / threads;
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        jobs[t] = proto;
        jobs[t].t0 = per * t;
        jobs[t].t1 = per * (t + 1) < proto.nrows ? per * (t + 1) : proto.nrows;
        if (jobs[t].t0 >= jobs[t].t1) break;
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) != 0) { run_job(&jobs[t]); continue; }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    return 0;
}

/* rows x cols (cols % 32 == 0) MXFP4: codes [rows][cols/2], scales [rows][cols/32] */
int synth_mxfp4(uint64_t seed, uint32_t tensor, uint64_t row0, uint64_t nrows, int cols,
                uint8_t* codes, uint8_t* scales, int threads) {
    if (cols <= 0 || cols % 32) return -1;
    job_t j; memset(&j, 0, sizeof j);
    j.seed = seed; j.tensor = tensor; j.row0 = row0; j.nrows = nrows; j.cols = cols; j.kind = 0;
    j.codes = codes; j.scales = scales;
    return run_threads(j, threads);
}

/* ratio-2 merged entries: entry r = softmax-weighted mean of tokens 2r, 2r+1 */
int synth_mxfp4_merged2(uint64_t seed, uint32_t tensor, uint32_t logit_tensor, uint64_t row0, uint64_t nrows,
                        int cols, uint8_t* codes, uint8_t* scales, int threads) {
    if (cols <= 0 || cols % 32) return -1;
    job_t j; memset(&j, 0, sizeof j);
    j.seed = seed; j.tensor = tensor; j.logit_tensor = logit_tensor; j.row0 = row0; j.nrows = nrows;
    j.cols = cols; j.kind = 3; j.codes = codes; j.scales = scales;
    return run_threads(j, threads);
}

int synth_e4m3(uint64_t seed, uint32_t tensor, uint64_t row0, uint64_t nrows, int cols, uint8_t* out, int threads) {
    if (cols <= 0 || cols % 4) return -1;
    job_t j; memset(&j, 0, sizeof j);
    j.seed = seed; j.tensor = tensor; j.row0 = row0; j.nrows = nrows; j.cols = cols; j.kind = 1; j.bytes = out;
    return run_threads(j, threads);
}

int synth_f32(uint64_t seed, uint32_t tensor, uint64_t row0, uint64_t nrows, int cols, float* out, int threads) {
    if (cols <= 0 || cols % 4) return -1;
    job_t j; memset(&j, 0, sizeof j);
    j.seed = seed; j.tensor = tensor; j.row0 = row0; j.nrows = nrows; j.cols = cols; j.kind = 2; j.f32 = out;
    return run_threads(j, threads);
}

/* raw normals in double (for tests of the distribution and of the merge) */
int synth_normals(uint64_t seed, uint32_t tensor, uint64_t row0, uint64_t nrows, int cols, double* out) {
    if (cols <= 0 || cols % 4) return -1;
    for (uint64_t r = 0; r < nrows; ++r) normal_row(seed, tensor, row0 + r, cols, out + r * (uint64_t)cols);
    return 0;
}

/* the merge weights (w0, w1) for entry row r: one scalar N(0,1) logit per token,
   token t uses lane t%4 of the Philox draw at (row t/4, column 0) */
void synth_merge_weights(uint64_t seed, uint32_t logit_tensor, uint64_t row, double* w) {
    uint64_t t0 = 2 * row, t1 = 2 * row + 1;
    double la[4], lb[4];
    normals4(seed, logit_tensor, t0 >> 2, 0, la);
    normals4(seed, logit_tensor, t1 >> 2, 0, lb);
    double l0 = la[t0 & 3], l1 = lb[t1 & 3];
    double mx = l0 > l1 ? l0 : l1;
    double e0 = exp(l0 - mx), e1 = exp(l1 - mx);
    w[0] = e0 / (e0 + e1);
    w[1] = e1 / (e0 + e1);
}

/* merge weights of entries [row0, row0 + nrows) as float32 pairs:
   out[2r], out[2r+1] = (float)w0, (float)w1 of entry row0 + r */
void synth_merge_weights_f32(uint64_t seed, uint32_t logit_tensor, uint64_t row0, uint64_t nrows, float* out) {
    double w[2];
    for (uint64_t r = 0; r < nrows; ++r) {
        synth_merge_weights(seed, logit_tensor, row0 + r, w);
        out[2 * r] = (float)w[0];
        out[2 * r + 1] = (float)w[1];
    }
}
