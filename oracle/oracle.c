/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the LoRA-bypass linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code with the GPU library: its dtype
 * policy, its rounding and its contractions are written here from the
 * definitions, independently of the HIP kernels.
 *
 * What it computes (all arithmetic in IEEE binary64, rounding only at the
 * declared boundaries):
 *
 *   policy   -- LyCORIS "Precision" page, section "Dtype policy": compute
 *               dtype is the 16-bit type when any operand is 16-bit, else
 *               fp32; output dtype is the promotion of every operand's dtype;
 *               fp16 together with bf16 is rejected as a caller bug.
 *   cast     -- matmul operands (x, W, down, up) are rounded from their
 *               stored value to the compute dtype (exact when equal).  The
 *               bias is not a matmul operand and keeps its stored value.
 *   h        -- h = x_c . down_c^T summed in fp64, then rounded to the
 *               compute (storage) dtype before the second dot, as the eager
 *               two-Linear chain does (same page, "Measured accuracy").
 *   lora     -- y = round_out( x_c.W_c^T + scale * h_r.up_c^T + b ), one
 *               final rounding.
 *   linear   -- Luminal FP16 page, "What Was Fixed": the projection
 *               p = x.W^T (fp32 compute) is rounded to the output dtype,
 *               then the bias is added and the sum rounded again; the bias is
 *               never fused across the projection's rounding boundary.
 *   merge    -- the LoRA merge W' = round_out( W + scale * up_c . down_c ):
 *               the original weight is the "input" of the same dtype policy
 *               and, like the bias, not a matmul operand (it keeps its stored
 *               value); up and down are cast to the compute dtype; one
 *               rounding (LyCORIS "Precision" page, "Dtype policy" and the
 *               merge figure of "Measured accuracy").
 *   backward -- the gradients of x, down and up for a given dy (LyCORIS
 *               "Precision" page, "Dtype policy": each gradient in its own
 *               leaf's dtype; "VRAM": h recomputed, up.down and its gradient
 *               never formed).  W and the bias are the frozen base layer.
 *               h and the gradient at h, gh = scale * dy_c . up_c, are each
 *               rounded once to the storage dtype before their second dots,
 *               as the forward rounds h; dx, dDown and dUp round once.
 *   dora     -- the row norms of the merged weight, RN_fp32(||W + scale up_c.down_c||_2)
 *               per row (the cached DoRA state of the "VRAM" section), and
 *               the DoRA forward y = round_out((m/norm) (x_c.W_c^T +
 *               scale h_r.up_c^T) + b): the magnitude vector m scales the
 *               LoRA product of each output feature, the bias is added after.
 *   rounding -- IEEE round-to-nearest, ties-to-even, directly from fp64 (never
 *               via fp32), gradual underflow, overflow to +-inf at or beyond
 *               max + half an ulp, NaN propagated.
 *
 * Sums run over k in increasing order.  Products of two fp16/bf16 values,
 * and of two fp32 values, are exact in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3 };
enum { OR_OK = 0, OR_MIXED_HALF = 1, OR_INVALID = 2 };

/* ---- formats ------------------------------------------------------------ */

/* p = significand bits (incl. the implicit one), emin = exponent of the
 * smallest normal, emax = exponent of the largest finite value. */
static int fmt(int dt, int* p, int* emin, int* emax) {
    switch (dt) {
    case OR_F16:  *p = 11; *emin = -14;  *emax = 15;  return 0;
    case OR_BF16: *p = 8;  *emin = -126; *emax = 127; return 0;
    case OR_F32:  *p = 24; *emin = -126; *emax = 127; return 0;
    default: return -1;
    }
}

/* Round v (binary64) to the nearest value of format dt, ties to even.
 * Returned as the binary64 value of the result. */
double oracle_round(double v, int dt) {
    int p, emin, emax;
    if (fmt(dt, &p, &emin, &emax)) return NAN;
    if (isnan(v)) return v;
    if (v == 0.0 || isinf(v)) return v;
    double a = fabs(v);
    /* largest finite value and the overflow threshold max + ulp(max)/2 */
    double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (a >= maxv + ldexp(1.0, emax - p)) return copysign(INFINITY, v);
    int ex;
    frexp(a, &ex);                  /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                 /* floor(log2(a)) */
    if (e < emin) e = emin;         /* subnormal range: fixed quantum */
    double q = ldexp(1.0, e - p + 1);   /* spacing of the format around a */
    double n = a / q;               /* exact: division by a power of two */
    double fl = floor(n);
    double d = n - fl;              /* exact fractional part */
    if (d > 0.5 || (d == 0.5 && fmod(fl, 2.0) == 1.0)) fl += 1.0;
    return copysign(fl * q, v);
}

/* Stored element -> exact binary64 value. */
static double widen(const void* base, int dt, int64_t i) {
    if (dt == OR_F32) return (double)((const float*)base)[i];
    uint16_t b = ((const uint16_t*)base)[i];
    if (dt == OR_BF16) {
        uint32_t u = (uint32_t)b << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    /* fp16: 1 sign, 5 exponent, 10 fraction bits */
    int s = b >> 15, e = (b >> 10) & 0x1f, m = b & 0x3ff;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

double oracle_widen(const void* base, int dt, int64_t i) { return widen(base, dt, i); }

/* Store a value that is already representable in dt. */
static void store(void* base, int dt, int64_t i, double v) {
    if (dt == OR_F32) { ((float*)base)[i] = (float)v; return; }
    uint16_t bits;
    if (dt == OR_BF16) {
        float f = (float)v;            /* exact: v is a bf16 value */
        uint32_t u;
        memcpy(&u, &f, 4);
        bits = isnan(v) ? (uint16_t)0x7fc0 : (uint16_t)(u >> 16);
    } else {
        uint16_t s = signbit(v) ? 0x8000 : 0;
        double a = fabs(v);
        if (isnan(v)) bits = 0x7e00;
        else if (isinf(v)) bits = s | 0x7c00;
        else if (a == 0.0) bits = s;
        else {
            int ex;
            frexp(a, &ex);
            int e = ex - 1;
            if (e < -14) bits = s | (uint16_t)ldexp(a, 24);           /* subnormal: a / 2^-24 */
            else bits = s | (uint16_t)((e + 15) << 10) | (uint16_t)(ldexp(a, 10 - e) - 1024.0);
        }
    }
    ((uint16_t*)base)[i] = bits;
}

void oracle_store(void* base, int dt, int64_t i, double v) { store(base, dt, i, v); }

/* Array forms of the three element helpers above. */
void oracle_round_n(const double* in, double* out, int64_t n, int dt) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_round(in[i], dt);
}
void oracle_widen_n(const void* base, int dt, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = widen(base, dt, i);
}
void oracle_store_n(void* base, int dt, const double* in, int64_t n) {
    for (int64_t i = 0; i < n; ++i) store(base, dt, i, in[i]);
}

/* ---- dtype policy ------------------------------------------------------- */

int oracle_resolve(const int* dts, int n, int* compute, int* output) {
    if (!dts || n <= 0) return OR_INVALID;
    int h16 = 0, hbf = 0, h32 = 0;
    for (int i = 0; i < n; ++i) {
        if (dts[i] == OR_F16) h16 = 1;
        else if (dts[i] == OR_BF16) hbf = 1;
        else if (dts[i] == OR_F32) h32 = 1;
        else return OR_INVALID;
    }
    if (h16 && hbf) return OR_MIXED_HALF;
    int c = h16 ? OR_F16 : (hbf ? OR_BF16 : OR_F32);
    if (compute) *compute = c;
    if (output) *output = h32 ? OR_F32 : c;
    return OR_OK;
}

/* ---- the forward ---------------------------------------------------------- */

typedef struct {
    /* problem */
    const void *x, *w, *b, *down, *up;
    int x_dt, w_dt, b_dt, down_dt, up_dt;
    int64_t M, N, K, r;
    double scale;
    int lora;                    /* 1: LoRA bypass, 0: plain affine (two roundings) */
    int c_dt, o_dt;
    /* cast operands, binary64 */
    const double *wc, *dc, *uc;  /* [N,K], [r,K], [N,r] */
    /* rows to evaluate */
    const int64_t* rows;
    int64_t nrows;
    /* outputs, [nrows][N] / [nrows][r]; any may be NULL */
    void* y;
    double* ref;
    double* hr;
    /* work split */
    int64_t lo, hi;
} job_t;

static void* run_rows(void* arg) {
    job_t* J = (job_t*)arg;
    const int64_t N = J->N, K = J->K, r = J->r;
    double* xc = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double* h = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    for (int64_t i = J->lo; i < J->hi; ++i) {
        int64_t m = J->rows ? J->rows[i] : i;
        for (int64_t k = 0; k < K; ++k) xc[k] = oracle_round(widen(J->x, J->x_dt, m * K + k), J->c_dt);
        if (J->lora) {
            for (int64_t j = 0; j < r; ++j) {
                double s = 0.0;
                for (int64_t k = 0; k < K; ++k) s += xc[k] * J->dc[j * K + k];
                h[j] = oracle_round(s, J->c_dt);               /* h rounded before the second dot */
                if (J->hr) J->hr[i * r + j] = h[j];
            }
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            const double* wr = J->wc + n * K;
            for (int64_t k = 0; k < K; ++k) acc += xc[k] * wr[k];
            double bias = J->b ? widen(J->b, J->b_dt, n) : 0.0;
            double v;
            if (J->lora) {
                double f = 0.0;
                for (int64_t j = 0; j < r; ++j) f += h[j] * J->uc[n * r + j];
                v = acc + J->scale * f + bias;
            } else {
                v = oracle_round(acc, J->o_dt) + bias;         /* projection rounded, then bias */
            }
            if (J->ref) J->ref[i * N + n] = v;
            if (J->y) store(J->y, J->o_dt, i * N + n, oracle_round(v, J->o_dt));
        }
    }
    free(xc);
    free(h);
    return NULL;
}

static double* cast_all(const void* src, int dt, int c_dt, int64_t n) {
    double* d = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) d[i] = oracle_round(widen(src, dt, i), c_dt);
    return d;
}

/*
 * Evaluate the forward for the given rows.
 *   lora = 0: plain affine (down/up/r/scale ignored).
 *   rows = NULL evaluates rows 0..nrows-1.
 *   y (o_dt storage), ref (value before the final rounding), hr (h rounded,
 *   LoRA only) are written as [nrows][N] / [nrows][r]; each may be NULL.
 *   b may be NULL (no bias).  Returns OR_OK, OR_MIXED_HALF or OR_INVALID and
 *   the resolved dtypes in *c_out / *o_out.
 */
int oracle_forward(int lora,
                   const void* x, int x_dt, const void* w, int w_dt, const void* b, int b_dt,
                   const void* down, int down_dt, const void* up, int up_dt, int64_t r, double scale,
                   int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                   void* y, double* ref, double* hr, int nthreads, int* c_out, int* o_out) {
    int dts[5], n = 0;
    dts[n++] = x_dt;
    dts[n++] = w_dt;
    if (b) dts[n++] = b_dt;
    if (lora) { dts[n++] = down_dt; dts[n++] = up_dt; }
    int c_dt, o_dt;
    int st = oracle_resolve(dts, n, &c_dt, &o_dt);
    if (st != OR_OK) return st;
    if (c_out) *c_out = c_dt;
    if (o_out) *o_out = o_dt;
    if (M < 0 || N < 0 || K < 0 || r < 0 || nrows < 0) return OR_INVALID;
    if (!lora) r = 0;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return OR_INVALID;
    if (!rows && nrows > M) return OR_INVALID;

    double* wc = cast_all(w, w_dt, c_dt, N * K);
    double* dc = lora ? cast_all(down, down_dt, c_dt, r * K) : NULL;
    double* uc = lora ? cast_all(up, up_dt, c_dt, N * r) : NULL;

    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        job_t* J = &jobs[t];
        J->x = x; J->w = w; J->b = b; J->down = down; J->up = up;
        J->x_dt = x_dt; J->w_dt = w_dt; J->b_dt = b_dt; J->down_dt = down_dt; J->up_dt = up_dt;
        J->M = M; J->N = N; J->K = K; J->r = r; J->scale = scale; J->lora = lora;
        J->c_dt = c_dt; J->o_dt = o_dt;
        J->wc = wc; J->dc = dc; J->uc = uc;
        J->rows = rows; J->nrows = nrows;
        J->y = y; J->ref = ref; J->hr = hr;
        J->lo = nrows * t / nthreads;
        J->hi = nrows * (t + 1) / nthreads;
    }
    int* started = (int*)calloc((size_t)nthreads, sizeof(int));
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&th[t], NULL, run_rows, &jobs[t]) == 0;
    run_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        else run_rows(&jobs[t]);      /* no thread: run the share here */
    }
    free(started);
    free(jobs);
    free(th);
    free(wc);
    free(dc);
    free(uc);
    return OR_OK;
}

/* ---- the merge ------------------------------------------------------------ */

typedef struct {
    const void* w;
    int w_dt, o_dt;
    int64_t N, K, r;
    double scale;
    const double *dc, *uc;       /* [r,K], [N,r] cast to compute, binary64 */
    const int64_t* rows;
    void* out;                   /* [nrows][K], o_dt storage */
    double* ref;                 /* [nrows][K] before the rounding */
    int64_t lo, hi;
} merge_job_t;

static void* merge_rows(void* arg) {
    merge_job_t* J = (merge_job_t*)arg;
    const int64_t K = J->K, r = J->r;
    for (int64_t i = J->lo; i < J->hi; ++i) {
        const int64_t n = J->rows ? J->rows[i] : i;
        for (int64_t k = 0; k < K; ++k) {
            double d = 0.0;
            for (int64_t j = 0; j < r; ++j) d += J->uc[n * r + j] * J->dc[j * K + k];
            const double v = widen(J->w, J->w_dt, n * K + k) + J->scale * d;
            if (J->ref) J->ref[i * K + k] = v;
            if (J->out) store(J->out, J->o_dt, i * K + k, oracle_round(v, J->o_dt));
        }
    }
    return NULL;
}

/*
 * The LoRA merge for the given rows n of W [N,K]: down [r,K], up [N,r].
 *   rows = NULL evaluates rows 0..nrows-1; out / ref are [nrows][K], either
 *   may be NULL.  Returns OR_OK, OR_MIXED_HALF or OR_INVALID and the
 *   resolved dtypes (over W, down, up) in *c_out / *o_out.
 */
int oracle_merge(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt, int64_t r,
                 double scale, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, void* out, double* ref,
                 int nthreads, int* c_out, int* o_out) {
    int dts[3] = {w_dt, down_dt, up_dt};
    int c_dt, o_dt;
    int st = oracle_resolve(dts, 3, &c_dt, &o_dt);
    if (st != OR_OK) return st;
    if (c_out) *c_out = c_dt;
    if (o_out) *o_out = o_dt;
    if (N < 0 || K < 0 || r < 0 || nrows < 0) return OR_INVALID;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= N) return OR_INVALID;
    if (!rows && nrows > N) return OR_INVALID;
    double* dc = cast_all(down, down_dt, c_dt, r * K);
    double* uc = cast_all(up, up_dt, c_dt, N * r);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    merge_job_t* jobs = (merge_job_t*)calloc((size_t)nthreads, sizeof(merge_job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int* started = (int*)calloc((size_t)nthreads, sizeof(int));
    for (int t = 0; t < nthreads; ++t) {
        merge_job_t* J = &jobs[t];
        J->w = w; J->w_dt = w_dt; J->o_dt = o_dt;
        J->N = N; J->K = K; J->r = r; J->scale = scale;
        J->dc = dc; J->uc = uc; J->rows = rows; J->out = out; J->ref = ref;
        J->lo = nrows * t / nthreads;
        J->hi = nrows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        started[t] = pthread_create(&th[t], NULL, merge_rows, &jobs[t]) == 0;
    merge_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        else merge_rows(&jobs[t]);
    }
    free(started);
    free(jobs);
    free(th);
    free(dc);
    free(uc);
    return OR_OK;
}

/* ---- the backward ---------------------------------------------------------- */

/* Run fn(ctx, lo, hi) over [0, n) split into nthreads contiguous shares. */
typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
    range_fn fn;
    void* ctx;
    int64_t lo, hi;
} range_job_t;

static void* run_range(void* arg) {
    range_job_t* J = (range_job_t*)arg;
    J->fn(J->ctx, J->lo, J->hi);
    return NULL;
}

static void par_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
    if (n <= 0) return;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = (int)n;
    range_job_t* jobs = (range_job_t*)calloc((size_t)nthreads, sizeof(range_job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    int* started = (int*)calloc((size_t)nthreads, sizeof(int));
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = n * t / nthreads;
        jobs[t].hi = n * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t) started[t] = pthread_create(&th[t], NULL, run_range, &jobs[t]) == 0;
    run_range(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        else run_range(&jobs[t]);
    }
    free(started);
    free(jobs);
    free(th);
}

typedef struct {
    int64_t M, N, K, r;
    double scale;
    int c_dt, x_dt, down_dt, up_dt;
    /* operands rounded to the compute dtype, binary64 */
    const double *xc, *wc, *dc, *uc, *gc;   /* [M,K], [N,K], [r,K], [N,r], [M,N] */
    /* rank columns evaluated for d_down and d_up */
    const int64_t* js;
    int64_t nj;
    /* h_r and gh_r for every token, columns js: [M][nj] */
    double *hj, *ghj;
    /* dx rows */
    const int64_t* dx_rows;
    double* ghrow;                           /* [n_dx][r] gh_r of the dx rows */
    void* dx;
    double *dx_ref, *dx_rss;
    /* d_down[js][dd_cols], d_up[du_rows][js] */
    const int64_t *dd_cols, *du_rows;
    int64_t n_dd, n_du;
    void *d_down, *d_up;
    double *dd_ref, *du_ref, *dd_rss, *du_rss;
} bwd_t;

/* h_r[m][j] = round_c(sum_k x_c[m,k] down_c[j,k]) -- the forward's h, recomputed */
static double bwd_h(const bwd_t* B, int64_t m, int64_t j) {
    double s = 0.0;
    for (int64_t k = 0; k < B->K; ++k) s += B->xc[m * B->K + k] * B->dc[j * B->K + k];
    return oracle_round(s, B->c_dt);
}

/* gh_r[m][j] = round_c(scale * sum_n dy_c[m,n] up_c[n,j]): the gradient at h,
 * rounded to the storage dtype before its own second dots */
static double bwd_gh(const bwd_t* B, int64_t m, int64_t j) {
    double s = 0.0;
    for (int64_t n = 0; n < B->N; ++n) s += B->gc[m * B->N + n] * B->uc[n * B->r + j];
    return oracle_round(B->scale * s, B->c_dt);
}

static void bwd_tokens(void* ctx, int64_t lo, int64_t hi) {
    bwd_t* B = (bwd_t*)ctx;
    for (int64_t m = lo; m < hi; ++m)
        for (int64_t t = 0; t < B->nj; ++t) {
            if (B->hj) B->hj[m * B->nj + t] = bwd_h(B, m, B->js[t]);
            if (B->ghj) B->ghj[m * B->nj + t] = bwd_gh(B, m, B->js[t]);
        }
}

/* dx[m,k] = round_x( sum_n dy_c[m,n] W_c[n,k] + sum_j gh_r[m,j] down_c[j,k] ) */
static void bwd_dx(void* ctx, int64_t lo, int64_t hi) {
    bwd_t* B = (bwd_t*)ctx;
    const int64_t N = B->N, K = B->K, r = B->r;
    for (int64_t i = lo; i < hi; ++i) {
        const int64_t m = B->dx_rows[i];
        double* gh = B->ghrow + i * r;
        for (int64_t j = 0; j < r; ++j) gh[j] = bwd_gh(B, m, j);
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0, q = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double t = B->gc[m * N + n] * B->wc[n * K + k];
                s += t;
                q += t * t;
            }
            double f = 0.0;
            for (int64_t j = 0; j < r; ++j) {
                const double t = gh[j] * B->dc[j * K + k];
                f += t;
                q += t * t;
            }
            const double v = s + f;
            if (B->dx_ref) B->dx_ref[i * K + k] = v;
            if (B->dx_rss) B->dx_rss[i * K + k] = sqrt(q);
            if (B->dx) store(B->dx, B->x_dt, i * K + k, oracle_round(v, B->x_dt));
        }
    }
}

/* d_down[j,k] = round_down( sum_m gh_r[m,j] x_c[m,k] ), over the columns k listed */
static void bwd_ddown(void* ctx, int64_t lo, int64_t hi) {
    bwd_t* B = (bwd_t*)ctx;
    for (int64_t c = lo; c < hi; ++c) {
        const int64_t k = B->dd_cols[c];
        for (int64_t t = 0; t < B->nj; ++t) {
            double s = 0.0, q = 0.0;
            for (int64_t m = 0; m < B->M; ++m) {
                const double u = B->ghj[m * B->nj + t] * B->xc[m * B->K + k];
                s += u;
                q += u * u;
            }
            if (B->dd_ref) B->dd_ref[t * B->n_dd + c] = s;
            if (B->dd_rss) B->dd_rss[t * B->n_dd + c] = sqrt(q);
            if (B->d_down) store(B->d_down, B->down_dt, t * B->n_dd + c, oracle_round(s, B->down_dt));
        }
    }
}

/* d_up[n,j] = round_up( scale * sum_m dy_c[m,n] h_r[m,j] ), over the rows n listed */
static void bwd_dup(void* ctx, int64_t lo, int64_t hi) {
    bwd_t* B = (bwd_t*)ctx;
    for (int64_t i = lo; i < hi; ++i) {
        const int64_t n = B->du_rows[i];
        for (int64_t t = 0; t < B->nj; ++t) {
            double s = 0.0, q = 0.0;
            for (int64_t m = 0; m < B->M; ++m) {
                const double u = B->gc[m * B->N + n] * B->hj[m * B->nj + t];
                s += u;
                q += u * u;
            }
            const double v = B->scale * s;
            if (B->du_ref) B->du_ref[i * B->nj + t] = v;
            if (B->du_rss) B->du_rss[i * B->nj + t] = fabs(B->scale) * sqrt(q);
            if (B->d_up) store(B->d_up, B->up_dt, i * B->nj + t, oracle_round(v, B->up_dt));
        }
    }
}

/*
 * The LoRA-bypass backward: the gradients of x, down and up given dy, the
 * gradient of y (LyCORIS "Precision" page: "Dtype policy" -- each gradient
 * comes back in its own leaf's dtype -- and "VRAM" -- h is recomputed, the
 * product up.down and its gradient are never formed).  W and the bias are the
 * frozen base layer: they get no gradient; the bias dtype (0: none) only
 * takes part in the policy, so that the compute dtype is the forward's.
 * The policy runs over (x, W, b, down, up, dy); with c the compute dtype:
 *
 *   h_r   = round_c( x_c . down_c^T )                  as in the forward
 *   gh_r  = round_c( scale * dy_c . up_c )             [M, r], rounded once
 *   dx    = round_x( dy_c . W_c + gh_r . down_c )      [M, K]
 *   dDown = round_down( gh_r^T . x_c )                 [r, K]
 *   dUp   = round_up( scale * dy_c^T . h_r )           [N, r]
 *
 * every sum in binary64, rounding only where written.  Outputs, each
 * optional (NULL):
 *   dx / dx_ref      [n_dx][K]  for the token rows dx_rows
 *   gh_rows          [n_dx][r]  gh_r of those rows
 *   d_down / dd_ref  [nj][n_dd] for the rank rows js and the columns dd_cols
 *   d_up / du_ref    [n_du][nj] for the rows du_rows and the rank columns js
 * With each *_ref goes *_rss, the root-sum-square of the terms of that
 * output's final sum (for error bounds of an fp32 evaluation; NULL: skipped).
 * Returns OR_OK, OR_MIXED_HALF or OR_INVALID, and the compute dtype.
 */
int oracle_backward(const void* x, int x_dt, const void* w, int w_dt, int b_dt, const void* down, int down_dt,
                    const void* up, int up_dt, int64_t r, double scale, const void* dy, int dy_dt, int64_t M,
                    int64_t N, int64_t K, const int64_t* dx_rows, int64_t n_dx, void* dx, double* dx_ref,
                    double* gh_rows, const int64_t* js, int64_t nj, const int64_t* dd_cols, int64_t n_dd,
                    void* d_down, double* dd_ref, const int64_t* du_rows, int64_t n_du, void* d_up,
                    double* du_ref, double* dx_rss, double* dd_rss, double* du_rss, int nthreads, int* c_out) {
    int dts[6], nd = 0;
    dts[nd++] = x_dt;
    dts[nd++] = w_dt;
    if (b_dt) dts[nd++] = b_dt;
    dts[nd++] = down_dt;
    dts[nd++] = up_dt;
    dts[nd++] = dy_dt;
    int c_dt, o_dt;
    int st = oracle_resolve(dts, nd, &c_dt, &o_dt);
    if (st != OR_OK) return st;
    if (c_out) *c_out = c_dt;
    if (M < 0 || N < 0 || K < 0 || r < 0 || n_dx < 0 || nj < 0 || n_dd < 0 || n_du < 0) return OR_INVALID;
    for (int64_t i = 0; i < n_dx; ++i) if (dx_rows[i] < 0 || dx_rows[i] >= M) return OR_INVALID;
    for (int64_t i = 0; i < nj; ++i) if (js[i] < 0 || js[i] >= r) return OR_INVALID;
    for (int64_t i = 0; i < n_dd; ++i) if (dd_cols[i] < 0 || dd_cols[i] >= K) return OR_INVALID;
    for (int64_t i = 0; i < n_du; ++i) if (du_rows[i] < 0 || du_rows[i] >= N) return OR_INVALID;

    bwd_t B;
    memset(&B, 0, sizeof(B));
    B.M = M; B.N = N; B.K = K; B.r = r; B.scale = scale;
    B.c_dt = c_dt; B.x_dt = x_dt; B.down_dt = down_dt; B.up_dt = up_dt;
    double* xc = cast_all(x, x_dt, c_dt, M * K);
    double* wc = cast_all(w, w_dt, c_dt, N * K);
    double* dc = cast_all(down, down_dt, c_dt, r * K);
    double* uc = cast_all(up, up_dt, c_dt, N * r);
    double* gc = cast_all(dy, dy_dt, c_dt, M * N);
    B.xc = xc; B.wc = wc; B.dc = dc; B.uc = uc; B.gc = gc;
    B.js = js; B.nj = nj;
    const int need_tokens = nj > 0 && (n_dd > 0 || n_du > 0);
    double* hj = need_tokens && n_du > 0 ? (double*)malloc(sizeof(double) * (size_t)(M * nj > 0 ? M * nj : 1)) : NULL;
    double* ghj = need_tokens && n_dd > 0 ? (double*)malloc(sizeof(double) * (size_t)(M * nj > 0 ? M * nj : 1)) : NULL;
    B.hj = hj; B.ghj = ghj;
    if (need_tokens) par_for(M, nthreads, bwd_tokens, &B);

    double* ghr = (double*)malloc(sizeof(double) * (size_t)(n_dx * r > 0 ? n_dx * r : 1));
    B.dx_rows = dx_rows; B.ghrow = ghr; B.dx = dx; B.dx_ref = dx_ref; B.dx_rss = dx_rss;
    par_for(n_dx, nthreads, bwd_dx, &B);
    if (gh_rows) memcpy(gh_rows, ghr, sizeof(double) * (size_t)(n_dx * r));

    B.dd_cols = dd_cols; B.n_dd = n_dd; B.d_down = d_down; B.dd_ref = dd_ref; B.dd_rss = dd_rss;
    if (ghj) par_for(n_dd, nthreads, bwd_ddown, &B);
    B.du_rows = du_rows; B.n_du = n_du; B.d_up = d_up; B.du_ref = du_ref; B.du_rss = du_rss;
    if (hj) par_for(n_du, nthreads, bwd_dup, &B);

    free(xc); free(wc); free(dc); free(uc); free(gc);
    free(hj); free(ghj); free(ghr);
    return OR_OK;
}

/* ---- DoRA ------------------------------------------------------------------- */

/* The row norms of the merged weight, before its rounding: for each row n,
 *   norm_n = RN_fp32( || W[n,:] + scale * (up_c . down_c)[n,:] ||_2 )
 * with the merge's policy over (W, down, up): W keeps its stored value, up and
 * down are rounded to the compute dtype (LyCORIS "Precision" page, "VRAM": the
 * DoRA row norms are the small cached state, one fp32 value per row).  The sum
 * of squares is binary64 in k order and its square root the binary64 one. */
typedef struct {
    const void* w;
    int w_dt;
    int64_t N, K, r;
    double scale;
    const double *dc, *uc;
    const int64_t* rows;
    float* norms;
    double* exact;
} dnorm_t;

static void dora_norm_rows(void* ctx, int64_t lo, int64_t hi) {
    dnorm_t* D = (dnorm_t*)ctx;
    const int64_t K = D->K, r = D->r;
    for (int64_t i = lo; i < hi; ++i) {
        const int64_t n = D->rows ? D->rows[i] : i;
        double q = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double d = 0.0;
            for (int64_t j = 0; j < r; ++j) d += D->uc[n * r + j] * D->dc[j * K + k];
            const double v = widen(D->w, D->w_dt, n * K + k) + D->scale * d;
            q += v * v;
        }
        const double s = sqrt(q);
        if (D->exact) D->exact[i] = s;
        if (D->norms) D->norms[i] = (float)oracle_round(s, OR_F32);
    }
}

int oracle_dora_norms(const void* w, int w_dt, const void* down, int down_dt, const void* up, int up_dt, int64_t r,
                      double scale, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, float* norms,
                      double* exact, int nthreads, int* c_out) {
    int dts[3] = {w_dt, down_dt, up_dt};
    int c_dt, o_dt;
    int st = oracle_resolve(dts, 3, &c_dt, &o_dt);
    if (st != OR_OK) return st;
    if (c_out) *c_out = c_dt;
    if (N < 0 || K < 0 || r < 0 || nrows < 0) return OR_INVALID;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= N) return OR_INVALID;
    if (!rows && nrows > N) return OR_INVALID;
    dnorm_t D;
    memset(&D, 0, sizeof D);
    D.w = w; D.w_dt = w_dt; D.N = N; D.K = K; D.r = r; D.scale = scale;
    double* dc = cast_all(down, down_dt, c_dt, r * K);
    double* uc = cast_all(up, up_dt, c_dt, N * r);
    D.dc = dc; D.uc = uc; D.rows = rows; D.norms = norms; D.exact = exact;
    par_for(nrows, nthreads, dora_norm_rows, &D);
    free(dc);
    free(uc);
    return OR_OK;
}

/* The DoRA forward for the given rows of x, with norms = the fp32 row norms
 * above (computed here from W, down and up):
 *   y = round_out( (m_n / norm_n) * (x_c . W_c^T + scale * h_r . up_c^T)_n + b_n )
 * The policy runs over (x, W, b, down, up, m); h_r is the LoRA forward's;
 * m_n / norm_n is one binary64 division, the bias is added after the
 * magnitude scaling, one final rounding. */
typedef struct {
    const void *x, *b, *m;
    int x_dt, b_dt, m_dt, c_dt, o_dt;
    int64_t N, K, r;
    double scale;
    const double *wc, *dc, *uc;
    const float* norms;          /* [N] */
    const int64_t* rows;
    void* y;
    double* ref;
} dfwd_t;

static void dora_fwd_rows(void* ctx, int64_t lo, int64_t hi) {
    dfwd_t* D = (dfwd_t*)ctx;
    const int64_t N = D->N, K = D->K, r = D->r;
    double* xc = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double* h = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    for (int64_t i = lo; i < hi; ++i) {
        const int64_t m = D->rows ? D->rows[i] : i;
        for (int64_t k = 0; k < K; ++k) xc[k] = oracle_round(widen(D->x, D->x_dt, m * K + k), D->c_dt);
        for (int64_t j = 0; j < r; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k) s += xc[k] * D->dc[j * K + k];
            h[j] = oracle_round(s, D->c_dt);
        }
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, f = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += xc[k] * D->wc[n * K + k];
            for (int64_t j = 0; j < r; ++j) f += h[j] * D->uc[n * r + j];
            const double g = widen(D->m, D->m_dt, n) / (double)D->norms[n];
            const double bias = D->b ? widen(D->b, D->b_dt, n) : 0.0;
            const double v = g * (acc + D->scale * f) + bias;
            if (D->ref) D->ref[i * N + n] = v;
            if (D->y) store(D->y, D->o_dt, i * N + n, oracle_round(v, D->o_dt));
        }
    }
    free(xc);
    free(h);
}

int oracle_dora_forward(const void* x, int x_dt, const void* w, int w_dt, const void* b, int b_dt, const void* down,
                        int down_dt, const void* up, int up_dt, const void* mag, int m_dt, int64_t r, double scale,
                        int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, void* y, double* ref,
                        float* norms_out, int nthreads, int* c_out, int* o_out) {
    int dts[6], nd = 0;
    dts[nd++] = x_dt;
    dts[nd++] = w_dt;
    if (b) dts[nd++] = b_dt;
    dts[nd++] = down_dt;
    dts[nd++] = up_dt;
    dts[nd++] = m_dt;
    int c_dt, o_dt;
    int st = oracle_resolve(dts, nd, &c_dt, &o_dt);
    if (st != OR_OK) return st;
    if (c_out) *c_out = c_dt;
    if (o_out) *o_out = o_dt;
    if (M < 0 || N < 0 || K < 0 || r < 0 || nrows < 0) return OR_INVALID;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return OR_INVALID;
    if (!rows && nrows > M) return OR_INVALID;
    float* norms = (float*)malloc(sizeof(float) * (size_t)(N > 0 ? N : 1));
    st = oracle_dora_norms(w, w_dt, down, down_dt, up, up_dt, r, scale, N, K, NULL, N, norms, NULL, nthreads, NULL);
    if (st != OR_OK) { free(norms); return st; }
    if (norms_out) memcpy(norms_out, norms, sizeof(float) * (size_t)N);
    dfwd_t D;
    memset(&D, 0, sizeof D);
    D.x = x; D.b = b; D.m = mag; D.x_dt = x_dt; D.b_dt = b_dt; D.m_dt = m_dt; D.c_dt = c_dt; D.o_dt = o_dt;
    D.N = N; D.K = K; D.r = r; D.scale = scale;
    double* wc = cast_all(w, w_dt, c_dt, N * K);
    double* dc = cast_all(down, down_dt, c_dt, r * K);
    double* uc = cast_all(up, up_dt, c_dt, N * r);
    D.wc = wc; D.dc = dc; D.uc = uc; D.norms = norms; D.rows = rows; D.y = y; D.ref = ref;
    par_for(nrows, nthreads, dora_fwd_rows, &D);
    free(wc); free(dc); free(uc); free(norms);
    return OR_OK;
}
