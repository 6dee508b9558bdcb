/*
 * Float64 reference ("oracle") for the RWKV-7 WKV time-mix recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. This file is compiled and called by the test
 * suite, by the smoke check and by the benchmark's CPU-baseline leg. It shares
 * no code, header or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes (per batch b and head h, state S is N x N, row i = value
 * index, column j = key index):
 *
 *     sa_i      = sum_j S_ij a_j                      (S of the previous token)
 *     S_ij     <- S_ij w_j + sa_i b_j + v_i k_j
 *     y_i       = sum_j S_ij r_j                      (S after the update)
 *
 * i.e. S_t = S_{t-1} (diag(w_t) + a_t b_t^T) + v_t k_t^T and y_t = S_t r_t.
 * Sources:
 *   - RWKV-7 G0 7.2B notes (lshu.cn/news/198401), section 7.1 "x070 architecture,
 *     the two core operators": the state is decayed by w, gets the state*a*b
 *     term and the v k^T outer product, and is then read out with r; the kernel
 *     slots are a = -kk and b = kk*a_lr.
 *   - same page, section 3.3 "vocabulary and loading details": the per-layer
 *     WKV state is an [H, N, N] float32 tensor initialised to zero.
 *   - RWKV-LM README (oa0.com/c/1004164), "RWKV introduction": a state of None
 *     starts fresh and a returned state resumes the sequence.
 *
 * Readings taken where the pages leave a step open:
 *   - decay multiplies key columns j (right-multiplication by diag(w));
 *   - sa uses the state before this token's update;
 *   - y is read after the update;
 *   - inputs are widened exactly (bf16 bits << 16, or float) to double and every
 *     accumulation is double, in index order, with no fused multiply-add
 *     (build with -ffp-contract=off).
 *
 * Layouts: r,w,k,v,a,b,y are [B,T,H,N] row-major; state_in / state_out are
 * [B,H,N,N] row-major with element (i,j) = S_ij.
 *
 * 16-bit stored states (the reduced-precision decode state; the RWKV-8 ROSA
 * note, trdm.cn/news/547794, "why states are worth quantising", gives the state
 * size as a function of the bits per element Q): state_in may be bfloat16 or
 * IEEE binary16 bits, widened exactly, and wkv7_oracle_round16 rounds a float64
 * state to either format, to nearest with ties to even, as the definition of
 * that rounding states it (scale by the quantum of the value's binade, round
 * the quotient to the nearest integer, even on ties, scale back).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_F16 = 3 };

/* IEEE binary16: sign bit, 5 exponent bits with bias 15, 10 fraction bits;
 * exponent field 0 holds zero and the subnormals (fraction * 2^-24). */
static double widen_f16(uint16_t h)
{
    const double sign = (h & 0x8000u) ? -1.0 : 1.0;
    const int e = (h >> 10) & 31;
    const int m = h & 1023;
    if (e == 0)
        return sign * ldexp((double)m, -24);
    if (e == 31)
        return m ? NAN : sign * INFINITY;
    return sign * ldexp((double)(1024 + m), e - 25);
}

static double widen(const void *p, int dtype, size_t idx)
{
    if (dtype == ORC_F32)
        return (double)((const float *)p)[idx];
    if (dtype == ORC_F16)
        return widen_f16(((const uint16_t *)p)[idx]);
    if (dtype == ORC_BF16) {
        /* bfloat16 is the upper half of an IEEE binary32 word. */
        uint32_t u = ((uint32_t)((const uint16_t *)p)[idx]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double *)p)[idx];
}

typedef struct {
    const void *r, *w, *k, *v, *a, *b; /* [B,T,H,N], dtype in_dtype */
    const void *state_in;              /* [B,H,N,N] or NULL, dtype st_dtype */
    double *y;                         /* [B,T,H,N] */
    double *state_out;                 /* [B,H,N,N] or NULL */
    int64_t B, T, H, N;
    int in_dtype, st_dtype;
    int64_t next_unit; /* shared work counter, guarded by lock */
    pthread_mutex_t lock;
} job_t;

static void run_unit(job_t *J, int64_t unit, double *S, double *vec)
{
    const int64_t N = J->N, T = J->T, H = J->H;
    const int64_t bb = unit / H, hh = unit % H;
    double *r = vec, *w = vec + N, *k = vec + 2 * N, *v = vec + 3 * N;
    double *a = vec + 4 * N, *b = vec + 5 * N;

    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < N; ++j)
            S[i * N + j] = J->state_in
                               ? widen(J->state_in, J->st_dtype, (size_t)(unit * N * N + i * N + j))
                               : 0.0;

    for (int64_t t = 0; t < T; ++t) {
        const size_t base = (size_t)(((bb * T + t) * H + hh) * N);
        for (int64_t j = 0; j < N; ++j) {
            r[j] = widen(J->r, J->in_dtype, base + j);
            w[j] = widen(J->w, J->in_dtype, base + j);
            k[j] = widen(J->k, J->in_dtype, base + j);
            v[j] = widen(J->v, J->in_dtype, base + j);
            a[j] = widen(J->a, J->in_dtype, base + j);
            b[j] = widen(J->b, J->in_dtype, base + j);
        }
        for (int64_t i = 0; i < N; ++i) {
            double *Si = S + i * N;
            double sa = 0.0;
            for (int64_t j = 0; j < N; ++j)
                sa += Si[j] * a[j];
            for (int64_t j = 0; j < N; ++j)
                Si[j] = Si[j] * w[j] + sa * b[j] + v[i] * k[j];
            double yi = 0.0;
            for (int64_t j = 0; j < N; ++j)
                yi += Si[j] * r[j];
            J->y[base + i] = yi;
        }
    }
    if (J->state_out)
        memcpy(J->state_out + unit * N * N, S, sizeof(double) * (size_t)(N * N));
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *S = (double *)malloc(sizeof(double) * (size_t)(J->N * J->N));
    double *vec = (double *)malloc(sizeof(double) * (size_t)(6 * J->N));
    if (!S || !vec) {
        free(S);
        free(vec);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= J->B * J->H)
            break;
        run_unit(J, unit, S, vec);
    }
    free(S);
    free(vec);
    return NULL;
}

/*
 * Runs the recurrence over all B*H (batch, head) units with `nthreads` POSIX
 * threads (each unit is independent). Returns 0 on success, -1 on bad
 * arguments, -2 if a thread or its buffers could not be created.
 */
int wkv7_oracle_f64(const void *r, const void *w, const void *k, const void *v,
                    const void *a, const void *b, const void *state_in, double *y,
                    double *state_out, int64_t B, int64_t T, int64_t H, int64_t N,
                    int in_dtype, int st_dtype, int nthreads)
{
    if (!r || !w || !k || !v || !a || !b || !y || B < 0 || T < 0 || H < 0 || N <= 0)
        return -1;
    if (in_dtype < ORC_F32 || in_dtype > ORC_F64 || st_dtype < ORC_F32 || st_dtype > ORC_F16)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    job_t J;
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b;
    J.state_in = state_in; J.y = y; J.state_out = state_out;
    J.B = B; J.T = T; J.H = H; J.N = N;
    J.in_dtype = in_dtype; J.st_dtype = st_dtype;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (B * H < nthreads)
        nthreads = (int)(B * H > 0 ? B * H : 1);

    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int status = 0, started = 0;
    if (!tid) {
        pthread_mutex_destroy(&J.lock);
        return -2;
    }
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &J) != 0) {
            status = -2;
            break;
        }
        ++started;
    }
    if (started == 0 && status == 0)
        status = -2;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret)
            status = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return status;
}

/*
 * Round x to the nearest number with `prec` significant bits whose leading bit
 * weighs at least 2^emin (below that the quantum stays 2^(emin - prec + 1):
 * the subnormal range), ties to even; anything beyond maxv becomes infinite.
 */
static double round_to_format(double x, int prec, int emin, double maxv)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    int e;
    frexp(x, &e); /* |x| = f 2^e with 0.5 <= f < 1: the leading bit weighs 2^(e-1) */
    int lead = e - 1;
    if (lead < emin)
        lead = emin;
    const double quantum = ldexp(1.0, lead - (prec - 1));
    const double r = rint(x / quantum) * quantum; /* rint: nearest, ties to even */
    return fabs(r) > maxv ? copysign(INFINITY, x) : r;
}

static uint16_t encode_bf16(double r)
{
    if (isnan(r))
        return 0x7FC0u;
    const float f = (float)r; /* exact: every bfloat16 value is a binary32 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint16_t encode_f16(double r)
{
    if (isnan(r))
        return 0x7E00u;
    const uint16_t sign = signbit(r) ? 0x8000u : 0u;
    const double m = fabs(r);
    if (isinf(m))
        return sign | 0x7C00u;
    if (m < ldexp(1.0, -14)) /* zero or subnormal: fraction = m / 2^-24 */
        return sign | (uint16_t)(m * ldexp(1.0, 24));
    int e;
    frexp(m, &e);
    const int lead = e - 1; /* -14 .. 15 */
    const uint16_t frac = (uint16_t)((m * ldexp(1.0, -lead) - 1.0) * 1024.0);
    return sign | (uint16_t)((lead + 15) << 10) | frac;
}

/*
 * Round n float64 values to a 16-bit state format and write the encodings.
 * fmt 1: bfloat16 (8 significant bits, binary32 exponent range, largest finite
 * value (2 - 2^-7) 2^127); fmt 3: IEEE binary16 (11 significant bits, normal
 * leading exponents -14..15, largest finite value 65504). Returns 0, or -1 for
 * an unknown format or bad arguments.
 */
int wkv7_oracle_round16(const double *x, uint16_t *out, int64_t n, int fmt)
{
    if ((!x || !out) && n > 0)
        return -1;
    if (fmt != ORC_BF16 && fmt != ORC_F16)
        return -1;
    for (int64_t i = 0; i < n; ++i) {
        if (fmt == ORC_BF16)
            out[i] = encode_bf16(round_to_format(x[i], 8, -126, ldexp(255.0, 120)));
        else
            out[i] = encode_f16(round_to_format(x[i], 11, -14, 65504.0));
    }
    return 0;
}

/* Widen n 16-bit state encodings (fmt 1 bfloat16, fmt 3 binary16) to float64. */
int wkv7_oracle_widen16(const uint16_t *bits, double *out, int64_t n, int fmt)
{
    if ((!bits || !out) && n > 0)
        return -1;
    if (fmt != ORC_BF16 && fmt != ORC_F16)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        out[i] = widen(bits, fmt, (size_t)i);
    return 0;
}

/*
 * Backward of the recurrence (reverse-mode derivatives, float64), for training
 * (RWKV-7 G0 7.2B notes, section 7.2: the training code runs the same WKV-7
 * operator forward and backward). Given dy = dL/dy_t for every token and
 * dS_T = dL/dS_T for the final state (NULL: zero), it returns dL/dr, dL/dw,
 * dL/dk, dL/dv, dL/da, dL/db ([B,T,H,N]) and dL/dS_0 ([B,H,N,N]).
 *
 * It keeps every state S_t of the forward pass and walks the tokens backwards
 * with G = dL/dS_t. With M_t = diag(w_t) + a_t b_t^T:
 *   y_t = S_t r_t                 ->  G += dy_t r_t^T,       dr_t = S_t^T dy_t
 *   S_t = S_{t-1} M_t + v_t k_t^T ->  dv_t = G k_t,          dk_t = G^T v_t,
 *                                     dM_t = S_{t-1}^T G,    dw_t = diag(dM_t),
 *                                     da_t = dM_t b_t = S_{t-1}^T (G b_t),
 *                                     db_t = dM_t^T a_t = G^T (S_{t-1} a_t),
 *                                     G <- G M_t^T = G diag(w_t) + (G b_t) a_t^T
 * and dL/dS_0 is G after the first token.
 */
typedef struct {
    const void *r, *w, *k, *v, *a, *b; /* [B,T,H,N], dtype in_dtype */
    const void *state_in;              /* [B,H,N,N] or NULL, dtype st_dtype */
    const double *dy;                  /* [B,T,H,N] */
    const double *dstate_out;          /* [B,H,N,N] or NULL */
    double *dr, *dw, *dk, *dv, *da, *db; /* [B,T,H,N] */
    double *dstate_in;                 /* [B,H,N,N] or NULL */
    int64_t B, T, H, N;
    int in_dtype, st_dtype;
    int64_t next_unit;
    pthread_mutex_t lock;
} bjob_t;

static int run_bwd_unit(bjob_t *J, int64_t unit)
{
    const int64_t N = J->N, T = J->T, H = J->H;
    const int64_t bb = unit / H, hh = unit % H;
    const size_t NN = (size_t)(N * N);
    double *Sall = (double *)malloc(sizeof(double) * NN * (size_t)(T + 1));
    double *G = (double *)malloc(sizeof(double) * NN);
    double *vec = (double *)malloc(sizeof(double) * (size_t)(9 * N));
    if (!Sall || !G || !vec) {
        free(Sall);
        free(G);
        free(vec);
        return -2;
    }
    double *r = vec, *w = vec + N, *k = vec + 2 * N, *v = vec + 3 * N, *a = vec + 4 * N, *b = vec + 5 * N;
    double *dyv = vec + 6 * N, *gb = vec + 7 * N, *sa = vec + 8 * N;

    for (size_t e = 0; e < NN; ++e)
        Sall[e] = J->state_in ? widen(J->state_in, J->st_dtype, (size_t)unit * NN + e) : 0.0;
    for (int64_t t = 0; t < T; ++t) { /* forward, keeping S_t in Sall[t + 1] */
        const size_t base = (size_t)(((bb * T + t) * H + hh) * N);
        for (int64_t j = 0; j < N; ++j) {
            w[j] = widen(J->w, J->in_dtype, base + j);
            k[j] = widen(J->k, J->in_dtype, base + j);
            v[j] = widen(J->v, J->in_dtype, base + j);
            a[j] = widen(J->a, J->in_dtype, base + j);
            b[j] = widen(J->b, J->in_dtype, base + j);
        }
        const double *Sp = Sall + (size_t)t * NN;
        double *Sc = Sall + (size_t)(t + 1) * NN;
        for (int64_t i = 0; i < N; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < N; ++j)
                s += Sp[i * N + j] * a[j];
            for (int64_t j = 0; j < N; ++j)
                Sc[i * N + j] = Sp[i * N + j] * w[j] + s * b[j] + v[i] * k[j];
        }
    }

    for (size_t e = 0; e < NN; ++e)
        G[e] = J->dstate_out ? J->dstate_out[(size_t)unit * NN + e] : 0.0;
    for (int64_t t = T - 1; t >= 0; --t) {
        const size_t base = (size_t)(((bb * T + t) * H + hh) * N);
        for (int64_t j = 0; j < N; ++j) {
            r[j] = widen(J->r, J->in_dtype, base + j);
            w[j] = widen(J->w, J->in_dtype, base + j);
            k[j] = widen(J->k, J->in_dtype, base + j);
            v[j] = widen(J->v, J->in_dtype, base + j);
            a[j] = widen(J->a, J->in_dtype, base + j);
            b[j] = widen(J->b, J->in_dtype, base + j);
            dyv[j] = J->dy[base + j];
        }
        const double *Sp = Sall + (size_t)t * NN;       /* S_{t-1} */
        const double *Sc = Sall + (size_t)(t + 1) * NN; /* S_t */
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j)
                G[i * N + j] += dyv[i] * r[j];
        for (int64_t j = 0; j < N; ++j) {
            double s_dr = 0.0, s_dk = 0.0, s_dw = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                s_dr += Sc[i * N + j] * dyv[i];
                s_dk += G[i * N + j] * v[i];
                s_dw += Sp[i * N + j] * G[i * N + j];
            }
            J->dr[base + j] = s_dr;
            J->dk[base + j] = s_dk;
            J->dw[base + j] = s_dw;
        }
        for (int64_t i = 0; i < N; ++i) {
            double s_dv = 0.0, s_gb = 0.0, s_sa = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                s_dv += G[i * N + j] * k[j];
                s_gb += G[i * N + j] * b[j];
                s_sa += Sp[i * N + j] * a[j];
            }
            J->dv[base + i] = s_dv;
            gb[i] = s_gb;
            sa[i] = s_sa;
        }
        for (int64_t j = 0; j < N; ++j) {
            double s_da = 0.0, s_db = 0.0;
            for (int64_t i = 0; i < N; ++i) {
                s_da += Sp[i * N + j] * gb[i];
                s_db += G[i * N + j] * sa[i];
            }
            J->da[base + j] = s_da;
            J->db[base + j] = s_db;
        }
        for (int64_t i = 0; i < N; ++i)
            for (int64_t j = 0; j < N; ++j)
                G[i * N + j] = G[i * N + j] * w[j] + gb[i] * a[j];
    }
    if (J->dstate_in)
        memcpy(J->dstate_in + (size_t)unit * NN, G, sizeof(double) * NN);
    free(Sall);
    free(G);
    free(vec);
    return 0;
}

static void *bworker(void *arg)
{
    bjob_t *J = (bjob_t *)arg;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t unit = J->next_unit++;
        pthread_mutex_unlock(&J->lock);
        if (unit >= J->B * J->H)
            break;
        if (run_bwd_unit(J, unit) != 0)
            return (void *)1;
    }
    return NULL;
}

/* Backward over all B*H units with `nthreads` threads. Returns 0, -1 on bad arguments, -2 on allocation failure. */
int wkv7_oracle_bwd_f64(const void *r, const void *w, const void *k, const void *v, const void *a,
                        const void *b, const void *state_in, const double *dy, const double *dstate_out,
                        double *dr, double *dw, double *dk, double *dv, double *da, double *db,
                        double *dstate_in, int64_t B, int64_t T, int64_t H, int64_t N, int in_dtype,
                        int st_dtype, int nthreads)
{
    if (!r || !w || !k || !v || !a || !b || !dy || !dr || !dw || !dk || !dv || !da || !db)
        return -1;
    if (B < 0 || T < 0 || H < 0 || N <= 0 || in_dtype < ORC_F32 || in_dtype > ORC_F64 || st_dtype < ORC_F32 ||
        st_dtype > ORC_F16)
        return -1;
    bjob_t J;
    J.r = r; J.w = w; J.k = k; J.v = v; J.a = a; J.b = b;
    J.state_in = state_in; J.dy = dy; J.dstate_out = dstate_out;
    J.dr = dr; J.dw = dw; J.dk = dk; J.dv = dv; J.da = da; J.db = db; J.dstate_in = dstate_in;
    J.B = B; J.T = T; J.H = H; J.N = N;
    J.in_dtype = in_dtype; J.st_dtype = st_dtype;
    J.next_unit = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1)
        nthreads = 1;
    if (B * H < nthreads)
        nthreads = (int)(B * H > 0 ? B * H : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    int status = 0, started = 0;
    if (!tid) {
        pthread_mutex_destroy(&J.lock);
        return -2;
    }
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, bworker, &J) != 0) {
            status = -2;
            break;
        }
        ++started;
    }
    if (started == 0 && status == 0)
        status = -2;
    for (int i = 0; i < started; ++i) {
        void *ret = NULL;
        pthread_join(tid[i], &ret);
        if (ret)
            status = -2;
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return status;
}
