/*
 * ssd_oracle.c -- plain fp64 CPU reference for the Mamba-2 SSD forward pass.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  It shares nothing
 * with the HIP library: no headers, no helpers, no constants.
 *
 * What it computes, token by token, for every (batch b, head h) with group
 * g = h / (nheads / ngroups) and a P x N state matrix s (s = init_state[b,h]
 * or zero):
 *
 *     alpha_t = exp(dt[b,t,h] * A[h])                          (decay a_t = dt_t A)
 *     s      <- alpha_t * s + dt[b,t,h] * x[b,t,h,:] (outer) B[b,t,g,:]
 *     y[b,t,h,:] = s @ C[b,t,g,:] + D[h] * x[b,t,h,:]
 *     final_state[b,h] = s after the last token
 *
 * The output line is the recurrence printed in devin.kr "NVIDIA CUDA Tile로
 * Mamba-2 순방향 전달 커널 가속화", section "Mamba-2 아키텍처의 핵심 연산"
 * (core operations): y_t = c_t^T h_t + D x_t, where h_t is the fixed-size state
 * carried from token to token.  That section names the per-token decay a_t
 * and its running sum G but does not print the state update; the update used
 * here is the standard discretised Mamba-2 update above (exp(dt A) decay, dt-
 * weighted outer product of x_t and b_t), read so that y_t sees the state
 * AFTER token t has been absorbed (same index t on both sides of the printed
 * output equation).
 *
 * Arithmetic is fp64 with libm exp(); inputs arrive as fp32 arrays holding
 * exactly the values the GPU reads (bf16 values are widened exactly).
 * No chunking, no log space, no exp2: those belong to the fast method, whose
 * results must equal this one up to rounding.
 *
 * Optional debug outputs:
 *   chunk_states [B,H,T,P,N]: the state just before token c*Q of each chunk c
 *                  (state at the start of chunk c), T = ceil(L/Q).
 *   ssd_oracle_chunk_cumsum: G[b,h,t] = (1/ln 2) * sum_{k=cQ}^{t} dt[b,k,h] A[h]
 *                  for t in chunk c -- the within-chunk running sum of a_t in
 *                  base-2 log space (same page, section "세 가지 핵심 커널 구현"
 *                  (three kernels): chunk_cumsum sums a_t inside each chunk and
 *                  scales by log2(e) so later steps can use exp2).
 *
 * Return value: 0 on success, -1 on a bad argument (nothing written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_fwd(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                   int64_t dstate, int64_t ngroups,
                   const float* x, const float* dt, const float* A,
                   const float* Bm, const float* Cm, const float* D,
                   const float* init_state, double* y, double* final_state,
                   int64_t chunk_size, double* chunk_states, int nthreads)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || nheads % ngroups != 0)
        return -1;
    if (!x || !dt || !A || !Bm || !Cm || !y || !final_state)
        return -1;
    if (chunk_states && chunk_size <= 0)
        return -1;
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int64_t heads_per_group = H / G;
    const int64_t T = chunk_states ? (L + chunk_size - 1) / chunk_size : 0;
    if (nthreads <= 0) nthreads = 1;

    int status = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (int64_t bh = 0; bh < batch * H; ++bh) {
        const int64_t b = bh / H, h = bh % H, g = h / heads_per_group;
        double* s = (double*)malloc((size_t)(P * N) * sizeof(double));
        if (!s) {
#pragma omp atomic write
            status = -1;
            continue;
        }
        if (init_state) {
            const float* s0 = init_state + (b * H + h) * P * N;
            for (int64_t i = 0; i < P * N; ++i) s[i] = (double)s0[i];
        } else {
            memset(s, 0, (size_t)(P * N) * sizeof(double));
        }
        const double a_h = (double)A[h];
        const double d_h = D ? (double)D[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            if (chunk_states && t % chunk_size == 0) {
                double* dst = chunk_states + ((b * H + h) * T + t / chunk_size) * P * N;
                memcpy(dst, s, (size_t)(P * N) * sizeof(double));
            }
            const double dtv = (double)dt[(b * L + t) * H + h];
            const double alpha = exp(dtv * a_h);
            const float* xt = x + ((b * L + t) * H + h) * P;
            const float* bt = Bm + ((b * L + t) * G + g) * N;
            const float* ct = Cm + ((b * L + t) * G + g) * N;
            double* yt = y + ((b * L + t) * H + h) * P;
            for (int64_t p = 0; p < P; ++p) {
                const double u = dtv * (double)xt[p];
                double* row = s + p * N;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    row[n] = alpha * row[n] + u * (double)bt[n];
                    acc += row[n] * (double)ct[n];
                }
                yt[p] = acc + d_h * (double)xt[p];
            }
        }
        memcpy(final_state + (b * H + h) * P * N, s, (size_t)(P * N) * sizeof(double));
        free(s);
    }
    return status;
}

int ssd_oracle_chunk_cumsum(int64_t batch, int64_t seqlen, int64_t nheads, int64_t chunk_size,
                            const float* dt, const float* A, double* G_out)
{
    if (batch <= 0 || seqlen <= 0 || nheads <= 0 || chunk_size <= 0 || !dt || !A || !G_out)
        return -1;
    const int64_t L = seqlen, H = nheads;
    const double inv_ln2 = 1.0 / log(2.0);
    for (int64_t b = 0; b < batch; ++b)
        for (int64_t h = 0; h < H; ++h) {
            double run = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                if (t % chunk_size == 0) run = 0.0;
                run += (double)dt[(b * L + t) * H + h] * (double)A[h];
                G_out[(b * H + h) * L + t] = run * inv_ln2;
            }
        }
    return 0;
}
