/*
 * gret_oracle.c -- fp64 CPU oracle for multi-head gated retention (gRet).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library path may include, link or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header or constant with the HIP
 * kernels.
 *
 * What it computes (page "YOCO 完全拆解：Decoder-Decoder 架构如何让 KV Cache 只存一次",
 * section "路线二：Multi-Head Gated Retention", the state/output recurrence, and
 * section "单 token Decode 的实现骨架", where a decode step scales the old state
 * by the exponential of the gate value and adds the key/value outer product):
 *
 *   for every (batch b, head h) independently, with S a dk x dv matrix:
 *     S <- state_in[b,h]  (zero when no initial state is given)
 *     for n = 0 .. N-1:
 *       g       = exp(log_gamma[b,h,n])          (exp(-inf) = 0 exactly)
 *       S[i][j] = g * S[i][j] + k[n][i] * v[n][j]
 *       out[n][j] = sum_i q[n][i] * S[i][j]       (reads the updated state)
 *     state_out[b,h] <- S
 *
 * The section "Prefill 与 Decode 为什么使用两种计算形态" states that the chunkwise
 * form is the same formula associated differently, not an approximation, so
 * this plain recurrence is the reference for both prefill and decode.
 *
 * Everything is carried in double precision. Inputs are read exactly as the
 * GPU reads them (fp32, or bf16 bit patterns widened exactly) and widened to
 * double element by element; no input is ever rounded.
 *
 * Layouts (row-major, contiguous): q,k [B,H,N,dk], v [B,H,N,dv],
 * log_gamma [B,H,N], state [B,H,dk,dv] with S[i][j] pairing key dim i with
 * value dim j.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Exact widening of one stored element to double. */
static inline double widen(const void* base, int64_t idx, int dtype) {
    if (dtype == ORACLE_F32) {
        return (double)((const float*)base)[idx];
    }
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One (b,h) head over N positions.
 *   s      : dk*dv doubles, holds the initial state on entry, the final on exit
 *   krow, vrow, qrow, orow : scratch rows of dk / dv / dk / dv doubles
 *   out    : N*dv doubles or NULL
 *   cmp    : optional N*dv values (dtype cmp_dtype) to compare against; the
 *            max |cmp - ref| and max |ref| over the head go to stats[0], [1]
 */
static void run_head(const void* q, const void* k, const void* v, int dtype,
                     const float* lg, double* s, int64_t N, int64_t dk,
                     int64_t dv, double* out, const void* cmp, int cmp_dtype,
                     double* stats, double* krow, double* vrow, double* qrow,
                     double* orow) {
    double max_diff = 0.0, max_ref = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        const double g = exp((double)lg[n]);
        for (int64_t i = 0; i < dk; ++i) {
            krow[i] = widen(k, n * dk + i, dtype);
            qrow[i] = widen(q, n * dk + i, dtype);
        }
        for (int64_t j = 0; j < dv; ++j) {
            vrow[j] = widen(v, n * dv + j, dtype);
            orow[j] = 0.0;
        }
        for (int64_t i = 0; i < dk; ++i) {
            double* srow = s + i * dv;
            const double ki = krow[i];
            const double qi = qrow[i];
            for (int64_t j = 0; j < dv; ++j) {
                srow[j] = g * srow[j] + ki * vrow[j];
                orow[j] += qi * srow[j];
            }
        }
        if (out) memcpy(out + n * dv, orow, (size_t)dv * sizeof(double));
        if (cmp) {
            for (int64_t j = 0; j < dv; ++j) {
                const double r = orow[j];
                const double d = fabs(widen(cmp, n * dv + j, cmp_dtype) - r);
                if (fabs(r) > max_ref) max_ref = fabs(r);
                if (d > max_diff || d != d) max_diff = (d != d) ? INFINITY : d;
            }
        }
    }
    if (stats) {
        stats[0] = max_diff;
        stats[1] = max_ref;
    }
}

/*
 * Prefill over every (b,h) head (OpenMP across heads).
 *   state_in  : double [B*H, dk, dv] or NULL (zero initial state); fp32
 *               states are widened exactly by the caller
 *   state_out : double [B*H, dk, dv], required
 *   out       : double [B*H, N, dv] or NULL
 *   cmp, cmp_dtype, stats : optional comparison; stats is [B*H, 2]
 *   nthreads  : OpenMP threads (<= 0: runtime default)
 * Returns 0, or -1 on a bad argument / failed allocation.
 */
int gret_oracle_prefill_f64(const void* q, const void* k, const void* v,
                            int in_dtype, const float* log_gamma,
                            const double* state_in, double* state_out,
                            double* out, const void* cmp, int cmp_dtype,
                            double* stats, int64_t BH, int64_t N, int64_t dk,
                            int64_t dv, int nthreads) {
    if (!q || !k || !v || !log_gamma || !state_out) return -1;
    if (BH < 0 || N < 0 || dk <= 0 || dv <= 0) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16) return -1;
    if (cmp && (!stats || (cmp_dtype != ORACLE_F32 && cmp_dtype != ORACLE_BF16))) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t x = 0; x < BH; ++x) {
        double* scratch = (double*)malloc((size_t)(2 * dk + 2 * dv) * sizeof(double));
        if (!scratch) {
            failed |= 1;
            continue;
        }
        double* s = state_out + x * dk * dv;
        for (int64_t e = 0; e < dk * dv; ++e)
            s[e] = state_in ? state_in[x * dk * dv + e] : 0.0;
        const size_t isz = in_dtype == ORACLE_F32 ? 4 : 2;
        const size_t csz = cmp_dtype == ORACLE_F32 ? 4 : 2;
        run_head((const char*)q + (size_t)(x * N * dk) * isz,
                 (const char*)k + (size_t)(x * N * dk) * isz,
                 (const char*)v + (size_t)(x * N * dv) * isz, in_dtype,
                 log_gamma + x * N, s, N, dk, dv, out ? out + x * N * dv : NULL,
                 cmp ? (const char*)cmp + (size_t)(x * N * dv) * csz : NULL,
                 cmp_dtype, stats ? stats + 2 * x : NULL, scratch,
                 scratch + dk, scratch + dk + dv, scratch + 2 * dk + dv);
        free(scratch);
    }
    return failed ? -1 : 0;
}

/*
 * One recurrent decode step for BH independent heads: the same loop body as
 * above for a single position. The state is carried in double and updated in
 * place.
 *   q,k [BH,dk], v [BH,dv] (dtype in_dtype), log_gamma [BH] fp32,
 *   state [BH,dk,dv] double (in/out), out [BH,dv] double.
 */
int gret_oracle_decode_f64(const void* q, const void* k, const void* v,
                           int in_dtype, const float* log_gamma, double* state,
                           double* out, int64_t BH, int64_t dk, int64_t dv,
                           int nthreads) {
    if (!q || !k || !v || !log_gamma || !state || !out) return -1;
    if (BH < 0 || dk <= 0 || dv <= 0) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(| : failed)
#endif
    for (int64_t x = 0; x < BH; ++x) {
        double* scratch = (double*)malloc((size_t)(2 * dk + 2 * dv) * sizeof(double));
        if (!scratch) {
            failed |= 1;
            continue;
        }
        const size_t isz = in_dtype == ORACLE_F32 ? 4 : 2;
        run_head((const char*)q + (size_t)(x * dk) * isz,
                 (const char*)k + (size_t)(x * dk) * isz,
                 (const char*)v + (size_t)(x * dv) * isz, in_dtype,
                 log_gamma + x, state + x * dk * dv, 1, dk, dv, out + x * dv,
                 NULL, 0, NULL, scratch, scratch + dk, scratch + dk + dv,
                 scratch + 2 * dk + dv);
        free(scratch);
    }
    return failed ? -1 : 0;
}

int gret_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
