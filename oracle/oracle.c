/*
 * oracle.c -- float64 CPU oracle for the selective-scan forward and the
 * Mamba-2 scalar-decay (SSD) forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it is the plain definition written out as a
 * sequential loop, one (batch, channel) row (or one (batch, head) pair) at a
 * time, in float64.
 *
 * Sources (web pages on selective state-space models, cited by title and
 * section):
 *   [ybb]  "Mamba状态空间模型的硬件感知推理优化：从选择性扫描到并行前缀和"
 *          (ybb.press/llm/14642): section 1 gives the recurrence h_t = A h_{t-1}
 *          + B x_t with output y_t = C h_t; section 3.1 computes the per-step
 *          decay as exp(A * softplus(dt)) inside one fused kernel and adds the
 *          skip term D*x to the output; section 4 gives the Mamba-2 scalar
 *          per-step decay h_t = a_t h_{t-1} + b_t x_t.
 *   [mhpq] essay at www.mhpq.cn/news/984979: section 2.2 gives the continuous
 *          LTI system x' = Ax + Bu, y = Cx + Du and the zero-order-hold step
 *          A_d = exp(A dt); section 3.1 makes A diagonal so the exponential is
 *          taken per state element.
 *   [csdn] "从硬件感知到算法革命：Mamba如何重塑序列建模的计算效率"
 *          (tencentcloud.csdn.net): section 2 makes the step size
 *          Delta = softplus(linear(x)) input-dependent; section 3 lists the
 *          block steps, with the SSM output merged with a SiLU gate branch.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes):
 *   - B is discretised by the step size alone: deltaB_u = delta * B_t * u_t.
 *   - softplus is applied to (delta_raw + delta_bias); no threshold, the
 *     float64 form max(x,0) + log1p(exp(-|x|)) is exact to rounding.
 *   - gating multiplies the whole output (C.h + D*u) by silu(z) = z*sigmoid(z).
 *   - the state starts at h0 (zero unless given) and h_last is the state after
 *     the final step.
 *   - the sum over the state index n runs in ascending n.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 * Rows are independent, so OpenMP over rows gives results bitwise identical
 * to a single thread.
 */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), written so neither branch overflows. */
static double oracle_softplus(double x)
{
    double ax = x < 0.0 ? -x : x;
    return (x > 0.0 ? x : 0.0) + log1p(exp(-ax));
}

/* silu(z) = z * sigmoid(z) ([csdn] section 3: SiLU activation on the gate). */
static double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

double oracle_softplus_f64(double x) { return oracle_softplus(x); }
double oracle_silu_f64(double z) { return oracle_silu(z); }

/*
 * Selective scan forward ([ybb] sections 1 and 3.1; [mhpq] sections 2.2, 3.1;
 * [csdn] section 2).  For every batch b and channel d independently:
 *
 *   h = h0[b,d,:]  (or 0)
 *   for t in 0..L-1:
 *       dl   = softplus(delta[b,d,t] + delta_bias[d])
 *       h[n] = exp(dl * A[d,n]) * h[n] + dl * B[b,n,t] * u[b,d,t]
 *       yv   = sum_n C[b,n,t] * h[n] + Dskip[d] * u[b,d,t]
 *       y[b,d,t] = z ? yv * silu(z[b,d,t]) : yv
 *   h_last[b,d,:] = h
 *
 * Layouts (row-major, contiguous):
 *   u, delta, z, y : (batch, D, L)
 *   B, C           : (batch, N, L)
 *   A              : (D, N)
 *   delta_bias, Dskip : (D)           (nullable -> 0)
 *   z              : nullable -> no gate
 *   h0, h_last     : (batch, D, N)    (h0 nullable -> 0; h_last nullable)
 */
void oracle_selective_scan_f64(int64_t batch, int64_t L, int64_t D, int64_t N,
                               const double *u, const double *delta,
                               const double *delta_bias, const double *A,
                               const double *B, const double *C,
                               const double *Dskip, const double *z,
                               const double *h0, double *y, double *h_last,
                               int nthreads)
{
    int64_t rows = batch * D;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / D, d = r % D;
        double hbuf[1024];
        double *h = hbuf;              /* N <= 1024 is enforced by the caller */
        const double *ur = u + r * L;
        const double *dr = delta + r * L;
        const double *zr = z ? z + r * L : NULL;
        const double *Bb = B + b * N * L;
        const double *Cb = C + b * N * L;
        const double *Ad = A + d * N;
        double bias = delta_bias ? delta_bias[d] : 0.0;
        double skip = Dskip ? Dskip[d] : 0.0;
        double *yr = y + r * L;
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[r * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dl = oracle_softplus(dr[t] + bias);
            double ut = ur[t];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double dA = exp(dl * Ad[n]);
                double dBu = dl * Bb[n * L + t] * ut;
                h[n] = dA * h[n] + dBu;
                acc += Cb[n * L + t] * h[n];
            }
            double yv = acc + skip * ut;
            if (zr) yv = yv * oracle_silu(zr[t]);
            yr[t] = yv;
        }
        if (h_last)
            for (int64_t n = 0; n < N; ++n) h_last[r * N + n] = h[n];
    }
}

/*
 * Mamba-2 scalar-decay (SSD) forward ([ybb] section 4: the decay a_t is one
 * scalar per step shared by every state element of a head).  For every batch
 * b and head h (group g = h / (H/G)) independently:
 *
 *   S[p][n] = h0[b,h,p,n] (or 0)
 *   for t in 0..L-1:
 *       dl = softplus(dt[b,t,h] + dt_bias[h])
 *       a  = exp(dl * A[h])
 *       S[p][n] = a * S[p][n] + dl * x[b,t,h,p] * B[b,t,g,n]
 *       y[b,t,h,p] = sum_n C[b,t,g,n] * S[p][n] + Dskip[h] * x[b,t,h,p]
 *       if z: y[b,t,h,p] *= silu(z[b,t,h,p])
 *   h_last[b,h,:,:] = S
 *
 * The optional gate multiplies the whole output, skip term included, as in
 * the selective scan (the tencentcloud.csdn.net article on Mamba, section 3:
 * a SiLU branch gates the SSM output).
 *
 * Layouts: x, z, y (batch, L, H, P); dt (batch, L, H); B, C (batch, L, G, N);
 * A, dt_bias, Dskip (H); h0, h_last (batch, H, P, N).
 */
void oracle_ssd_f64(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                    int64_t G, const double *x, const double *dt,
                    const double *dt_bias, const double *A, const double *B,
                    const double *C, const double *Dskip, const double *z,
                    const double *h0, double *y, double *h_last, int nthreads)
{
    int64_t pairs = batch * H;
    int64_t heads_per_group = H / G;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int64_t r = 0; r < pairs; ++r) {
        int64_t b = r / H, hh = r % H;
        int64_t g = hh / heads_per_group;
        double Sbuf[65536];            /* P*N <= 65536 is enforced by the caller */
        double *S = Sbuf;
        double bias = dt_bias ? dt_bias[hh] : 0.0;
        double skip = Dskip ? Dskip[hh] : 0.0;
        for (int64_t i = 0; i < P * N; ++i)
            S[i] = h0 ? h0[r * P * N + i] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dl = oracle_softplus(dt[(b * L + t) * H + hh] + bias);
            double a = exp(dl * A[hh]);
            const double *xt = x + ((b * L + t) * H + hh) * P;
            const double *Bt = B + ((b * L + t) * G + g) * N;
            const double *Ct = C + ((b * L + t) * G + g) * N;
            double *yt = y + ((b * L + t) * H + hh) * P;
            const double *zt = z ? z + ((b * L + t) * H + hh) * P : 0;
            for (int64_t p = 0; p < P; ++p) {
                double acc = 0.0;
                double dx = dl * xt[p];
                for (int64_t n = 0; n < N; ++n) {
                    S[p * N + n] = a * S[p * N + n] + dx * Bt[n];
                    acc += Ct[n] * S[p * N + n];
                }
                yt[p] = acc + skip * xt[p];
                if (zt) yt[p] *= oracle_silu(zt[p]);
            }
        }
        if (h_last)
            for (int64_t i = 0; i < P * N; ++i) h_last[r * P * N + i] = S[i];
    }
}

/*
 * Causal depthwise convolution of width K followed by SiLU, the local
 * convolution the Mamba block applies to its SSM branch before the scan
 * ([csdn] section 3: a local convolution captures short-range patterns,
 * kernel size 4, SiLU activation; [mlqm] section 3.3: d_conv = 4).  For every
 * batch b, channel d and step t:
 *
 *   u[b,d,t] = silu(conv_b[d] + sum_{k=0..K-1} conv_w[d,k] * x[b,d,t-(K-1)+k])
 *
 * with x = 0 before the first step (causal: step t sees steps t-K+1 .. t).
 * Layouts: x, u (batch, D, L); conv_w (D, K); conv_b (D) nullable -> 0.
 */
void oracle_conv1d_silu_f64(int64_t batch, int64_t D, int64_t L, int64_t K,
                            const double *x, const double *conv_w,
                            const double *conv_b, double *u)
{
    for (int64_t r = 0; r < batch * D; ++r) {
        int64_t d = r % D;
        const double *xr = x + r * L;
        const double *w = conv_w + d * K;
        double bias = conv_b ? conv_b[d] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double acc = bias;
            for (int64_t k = 0; k < K; ++k) {
                int64_t s = t - (K - 1) + k;
                if (s >= 0) acc += w[k] * xr[s];
            }
            u[r * L + t] = oracle_silu(acc);
        }
    }
}

/*
 * Backward of the selective scan: the reverse-mode derivative of the loop of
 * oracle_selective_scan_f64 (the recurrence of [ybb] sections 1 and 3.1 and
 * [mhpq] section 2.2; the forward + backward training use of the block in
 * [mlqm] section 3.2).  Given the output gradients dy (batch, D, L) and
 * dh_last (batch, D, N) (nullable -> 0), it forms the gradients of every
 * input.  For each row (b, d), the states h_t of the row are recomputed
 * forward and kept; then, with x_t = delta + bias, dl_t = softplus(x_t),
 * a_t[n] = exp(dl_t A[d,n]), s_t = sum_n C_t[n] h_t[n] + D u_t and
 * y_t = s_t silu(z_t), for t = L-1 down to 0:
 *
 *   ds_t     = dy_t silu(z_t)                    dz_t = dy_t s_t silu'(z_t)
 *   dh_t[n]  = ds_t C_t[n] + a_{t+1}[n] dh_{t+1}[n]   (dh_L := dh_last)
 *   dC_t[n] += ds_t h_t[n]                       dD    += ds_t u_t
 *   dA[n]   += dh_t[n] h_{t-1}[n] a_t[n] dl_t    dB_t[n] += dh_t[n] dl_t u_t
 *   du_t     = ds_t D + sum_n dh_t[n] dl_t B_t[n]
 *   d(dl_t)  = sum_n dh_t[n] (h_{t-1}[n] a_t[n] A[n] + B_t[n] u_t)
 *   ddelta_t = d(dl_t) sigmoid(x_t)              dbias += ddelta_t
 *
 * and dh0 = a_0 dh_0.  silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).
 * dB, dC sum over channels, dA, dD, dbias over batches.  Outputs: du,
 * ddelta, dz like u (dz only when z is given); dB, dC like B; dA like A;
 * dD, ddelta_bias (D); dh0 like h0.  Every output but du and ddelta is
 * nullable.  Single-threaded; rows in order, so sums are deterministic.
 */
void oracle_selective_scan_bwd_f64(int64_t batch, int64_t L, int64_t D, int64_t N,
                                   const double *u, const double *delta,
                                   const double *delta_bias, const double *A,
                                   const double *B, const double *C,
                                   const double *Dskip, const double *z,
                                   const double *h0, const double *dy,
                                   const double *dh_last, double *du, double *ddelta,
                                   double *ddelta_bias, double *dA, double *dB,
                                   double *dC, double *dD, double *dz, double *dh0)
{
    double *hist = (double *)malloc(sizeof(double) * (size_t)((L + 1) * N));
    double *dh = (double *)malloc(sizeof(double) * (size_t)N);
    double *gB = (double *)calloc((size_t)(batch * N * L), sizeof(double));
    double *gC = (double *)calloc((size_t)(batch * N * L), sizeof(double));
    double *gA = (double *)calloc((size_t)(D * N), sizeof(double));
    double *gD = (double *)calloc((size_t)D, sizeof(double));
    double *gbias = (double *)calloc((size_t)D, sizeof(double));
    for (int64_t r = 0; r < batch * D; ++r) {
        int64_t b = r / D, d = r % D;
        const double *ur = u + r * L, *dr = delta + r * L;
        const double *Ad = A + d * N;
        const double *Bb = B + b * N * L, *Cb = C + b * N * L;
        double bias = delta_bias ? delta_bias[d] : 0.0;
        double skip = Dskip ? Dskip[d] : 0.0;
        /* forward: hist[(t + 1) N + n] = h_t[n], hist[n] = the initial state */
        for (int64_t n = 0; n < N; ++n) hist[n] = h0 ? h0[r * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dl = oracle_softplus(dr[t] + bias);
            for (int64_t n = 0; n < N; ++n)
                hist[(t + 1) * N + n] = exp(dl * Ad[n]) * hist[t * N + n] +
                                        dl * Bb[n * L + t] * ur[t];
        }
        /* reverse: dh carries a_{t+1} dh_{t+1} into step t */
        for (int64_t n = 0; n < N; ++n) dh[n] = dh_last ? dh_last[r * N + n] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            double x = dr[t] + bias;
            double dl = oracle_softplus(x);
            double sig = 1.0 / (1.0 + exp(-x));
            double dyt = dy[r * L + t];
            double ds = dyt;
            if (z) {
                double zt = z[r * L + t];
                double sz = 1.0 / (1.0 + exp(-zt));
                double s = skip * ur[t];
                for (int64_t n = 0; n < N; ++n) s += Cb[n * L + t] * hist[(t + 1) * N + n];
                ds = dyt * oracle_silu(zt);
                if (dz) dz[r * L + t] = dyt * s * sz * (1.0 + zt * (1.0 - sz));
            }
            gD[d] += ds * ur[t];
            double dut = ds * skip;
            double ddl = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double Bt = Bb[n * L + t];
                double a = exp(dl * Ad[n]);
                double hprev = hist[t * N + n];
                dh[n] += ds * Cb[n * L + t];
                gC[b * N * L + n * L + t] += ds * hist[(t + 1) * N + n];
                gA[d * N + n] += dh[n] * hprev * a * dl;
                gB[b * N * L + n * L + t] += dh[n] * dl * ur[t];
                dut += dh[n] * dl * Bt;
                ddl += dh[n] * (hprev * a * Ad[n] + Bt * ur[t]);
                dh[n] *= a;
            }
            du[r * L + t] = dut;
            ddelta[r * L + t] = ddl * sig;
            gbias[d] += ddl * sig;
        }
        if (dh0)
            for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = dh[n];
    }
    for (int64_t i = 0; i < batch * N * L; ++i) {
        if (dB) dB[i] = gB[i];
        if (dC) dC[i] = gC[i];
    }
    for (int64_t i = 0; i < D * N; ++i)
        if (dA) dA[i] = gA[i];
    for (int64_t i = 0; i < D; ++i) {
        if (dD) dD[i] = gD[i];
        if (ddelta_bias) ddelta_bias[i] = gbias[i];
    }
    free(hist); free(dh); free(gB); free(gC); free(gA); free(gD); free(gbias);
}
