/*
 * oracle.c -- plain fp64 CPU definition of Mamba's selective SSM scan (S6) and of its
 * one-token recurrent step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes, and where the pages define it:
 *   - Keras/TensorFlow tutorial page ("Mamba SSM concept and implementation in Keras and
 *     TensorFlow"), function `selective_scan`: A_bar = exp(delta * A) per (t, d, n), the
 *     input term delta * u * B (Euler form for B; the zero-order-hold formulas on that page
 *     did not survive extraction), the inclusive recurrence h_t = A_bar_t h_{t-1} + B_bar_t
 *     u_t from h_0 = 0 (the page's unrolled sum assumes h0 = 0), y_t = sum_n C_t h_t, then
 *     the D skip y + u * D.
 *   - Same page, `MambaBlock.ssm`: delta = softplus(delta_projection(...)) where the
 *     projection carries a bias, so delta = softplus(delta_raw + bias).
 *   - Same page, `MambaBlock.call`: the SSM output is multiplied by swish(res) = silu(z)
 *     after the D skip, so out = (C.h + D u) * silu(z).
 *   - mamba-jax README and the upstream README (generation): the recurrent mode carries the
 *     state token by token; one token of it is the loop body below with L = 1.
 * Arithmetic is IEEE fp64 throughout, sequential in t; rows (batch, channel) are
 * independent and are the only thing run in parallel.
 *
 * A scan may also start from a given state h_0 instead of zeros (prefill continued in chunks:
 * the recurrence itself is unchanged, only its first h_{t-1} differs), and a row may be shorter
 * than L (row_len[r], sequences of different lengths in one batch): its steps stop there, its
 * outputs past the end are 0 and last_state is the state after its own last step.
 *
 * Parity pins (all in tests/test_oracle_pins.py, each independent of this loop): the L = 1
 * closed form; the LTI case against a brute-force convolution with kernel
 * K_k = sum_n C_n exp(k delta A_n) delta B_n; the unrolled time-varying sum with exponents
 * summed directly; the tutorial's own suffix-sum / ratio formulation; linearity in u; A = 0
 * against numpy.cumsum; the memoryless limit; causality; gate / skip / bias placement;
 * the decode step chained L times against the scan; softplus and silu against numpy/scipy.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), written as max(x, 0) + log1p(e^-|x|) so it neither
 * overflows nor loses digits for very negative x.  (tutorial page, tf.nn.softplus) */
static double sp(double x) { return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* silu(v) = v * sigmoid(v) = v / (1 + e^-v)  (tutorial page, tf.nn.swish) */
static double silu(double v) { return v / (1.0 + exp(-v)); }

void oracle_softplus(const double* x, double* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = sp(x[i]);
}

void oracle_silu(const double* x, double* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = silu(x[i]);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Forward selective scan over R independent rows.
 *   row_batch[r]      batch index b of row r (selects B[b], C[b])
 *   u, delta, z       R x L (z may be NULL: no gate); delta is the raw value before bias
 *   A                 R x N (A of the row's channel)
 *   Bm, Cm            Bt x N x L
 *   D, bias           R (either may be NULL: treated as 0)
 *   softplus_flag     nonzero: delta = softplus(delta_raw + bias); zero: delta_raw + bias
 *   out               R x L
 *   last_state        R x N, h_L (may be NULL)
 * Returns 0, or -1 for a bad size.
 */
int oracle_selective_scan(int64_t R, int64_t N, int64_t L, int64_t Bt,
                          const int64_t* row_batch,
                          const double* u, const double* delta, const double* z,
                          const double* A, const double* Bm, const double* Cm,
                          const double* D, const double* bias, int softplus_flag,
                          const double* h0, const int64_t* row_len, double* out,
                          double* last_state, int nthreads) {
    if (R < 0 || N <= 0 || L < 0 || Bt <= 0) return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t b = row_batch[r];
        if (b < 0 || b >= Bt) { bad = 1; continue; }
        double* h = (double*)calloc((size_t)N, sizeof(double)); /* h_0 = 0 ... */
        if (!h) { bad = 1; continue; }
        if (h0)                                                  /* ... or the given state */
            for (int64_t n = 0; n < N; ++n) h[n] = h0[r * N + n];
        const double* Ar = A + r * N;
        const double* Bb = Bm + b * N * L;
        const double* Cb = Cm + b * N * L;
        const double Dr = D ? D[r] : 0.0;
        const double br = bias ? bias[r] : 0.0;
        const int64_t Lr = row_len ? (row_len[r] < 0 ? 0 : (row_len[r] > L ? L : row_len[r])) : L;
        for (int64_t t = Lr; t < L; ++t) out[r * L + t] = 0.0;           /* past the row's end */
        for (int64_t t = 0; t < Lr; ++t) {
            const double ut = u[r * L + t];
            const double pre = delta[r * L + t] + br;
            const double dt = softplus_flag ? sp(pre) : pre;
            double y = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double abar = exp(dt * Ar[n]);          /* A_bar = exp(delta A) */
                h[n] = abar * h[n] + dt * Bb[n * L + t] * ut;  /* + delta B u        */
                y += Cb[n * L + t] * h[n];                     /* C . h_t            */
            }
            y += Dr * ut;                                      /* D skip             */
            out[r * L + t] = z ? y * silu(z[r * L + t]) : y;   /* gate after skip    */
        }
        if (last_state)
            for (int64_t n = 0; n < N; ++n) last_state[r * N + n] = h[n];
        free(h);
    }
    return bad ? -1 : 0;
}

/*
 * Gradients of the forward scan (h_0 = 0): given dout = dL/dout for a scalar loss L, the
 * adjoint (reverse-mode) pass of the recurrence above, written out step by step.  The pages
 * define only the forward; this is its derivative, taken by the chain rule through
 *   pre = delta_raw + bias,  dt = softplus(pre) (d dt / d pre = sigmoid(pre)) or dt = pre,
 *   abar_n = exp(dt A_n),  h_t = abar h_{t-1} + dt B_t u_t,  y_t = C_t.h_t + D u_t,
 *   out_t = y_t silu(z_t)   (d silu / dz = s (1 + z (1 - s)), s = sigmoid(z)).
 * With G_t = dL/dh_t (total), G_t = dy_t C_t + abar_{t+1} G_{t+1}; every input's gradient
 * collects its terms from the steps that use it.  h_t is stored for the whole row (the
 * plainest route; no recomputation).
 *
 * Outputs, all overwritten:
 *   du, ddelta         R x L   (ddelta is w.r.t. delta_raw)
 *   dz                 R x L   (only when z is given)
 *   dA                 R x N   row's contribution (the channel's gradient sums its rows)
 *   dD, dbias          R       row's contribution (computed even when D / bias is NULL,
 *                              i.e. the gradient at D = 0 / bias = 0)
 *   dB, dC             Bt x N x L, summed over the R rows
 * magnitude != 0 replaces every term added into an output by its absolute value (G and h
 * themselves stay signed), giving sum |terms| per output element: the scale a rounding-error
 * bound for a re-associated fp32 evaluation of the same sums is proportional to.
 * The forward may start from h0 (R x N) and stop at row_len[r] (as in the forward above); dlast
 * (R x N) is dL/d last_state when the loss also depends on the final state (it seeds the adjoint
 * at the row's last step), and dh0 (R x N, written when not NULL) is dL/dh0.  Steps past a row's
 * end take no part: their du, ddelta, dz are 0.
 * Not pinned by the pages (they print no gradient); pinned in the tests by central finite
 * differences of the forward above, an L = 1 closed form and linearity in dout.
 */
int oracle_selective_scan_bwd(int64_t R, int64_t N, int64_t L, int64_t Bt,
                              const int64_t* row_batch,
                              const double* u, const double* delta, const double* z,
                              const double* A, const double* Bm, const double* Cm,
                              const double* D, const double* bias, int softplus_flag,
                              const double* h0, const int64_t* row_len, const double* dlast,
                              const double* dout, double* du, double* ddelta, double* dz,
                              double* dA, double* dB, double* dC, double* dD, double* dbias,
                              double* dh0, int magnitude, int nthreads) {
    if (R < 0 || N <= 0 || L < 0 || Bt <= 0) return -1;
    set_threads(nthreads);
    const size_t nbc = (size_t)(Bt * N * L);
    const int nt = oracle_max_threads();
    /* each thread's share of dB / dC, added into the outputs in thread order at the end */
    double* shares = (double*)calloc((size_t)nt * 2 * (nbc ? nbc : 1), sizeof(double));
    if (!shares) return -1;
    int bad = 0;
#pragma omp parallel reduction(| : bad)
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        double* accB = shares + (size_t)tid * 2 * (nbc ? nbc : 1);
        double* accC = accB + (nbc ? nbc : 1);
        double* hs = (double*)malloc((size_t)((L + 1) * N) * sizeof(double)); /* h_0 .. h_L */
        double* ys = (double*)malloc((size_t)(L ? L : 1) * sizeof(double));
        double* g = (double*)malloc((size_t)N * sizeof(double));
        if (tid >= nt || !hs || !ys || !g) bad = 1;
#define ACC(dst, term) ((dst) += magnitude ? fabs(term) : (term))
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < R; ++r) {
            if (bad) continue;
            const int64_t b = row_batch[r];
            if (b < 0 || b >= Bt) { bad = 1; continue; }
            const double* Ar = A + r * N;
            const double* Bb = Bm + b * N * L;
            const double* Cb = Cm + b * N * L;
            const double Dr = D ? D[r] : 0.0;
            const double br = bias ? bias[r] : 0.0;
            const int64_t Lr = row_len ? (row_len[r] < 0 ? 0 : (row_len[r] > L ? L : row_len[r])) : L;
            for (int64_t t = Lr; t < L; ++t) {  /* past the row's end */
                du[r * L + t] = 0.0; ddelta[r * L + t] = 0.0;
                if (z) dz[r * L + t] = 0.0;
            }
            /* forward, keeping every h_t and y_t (for magnitude: y's sum of |terms|) */
            for (int64_t n = 0; n < N; ++n) hs[n] = h0 ? h0[r * N + n] : 0.0;
            for (int64_t t = 0; t < Lr; ++t) {
                const double ut = u[r * L + t];
                const double pre = delta[r * L + t] + br;
                const double dt = softplus_flag ? sp(pre) : pre;
                const double* hp = hs + t * N;
                double* hc = hs + (t + 1) * N;
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    hc[n] = exp(dt * Ar[n]) * hp[n] + dt * Bb[n * L + t] * ut;
                    ACC(y, Cb[n * L + t] * hc[n]);
                }
                ACC(y, Dr * ut);
                ys[t] = y;
            }
            /* reverse */
            double dDr = 0.0, dbr = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                g[n] = dlast ? dlast[r * N + n] : 0.0;  /* G and h stay signed in either mode */
                dA[r * N + n] = 0.0;
            }
            for (int64_t t = Lr - 1; t >= 0; --t) {
                const double ut = u[r * L + t];
                const double pre = delta[r * L + t] + br;
                const double dt = softplus_flag ? sp(pre) : pre;
                const double dsp = softplus_flag ? 1.0 / (1.0 + exp(-pre)) : 1.0;
                const double go = dout[r * L + t];
                double dy = go;
                if (z) {
                    const double zt = z[r * L + t];
                    const double s = 1.0 / (1.0 + exp(-zt));
                    dy = go * zt * s;                                   /* dout silu(z) */
                    const double dgate = go * s * (1.0 + zt * (1.0 - s)); /* dout silu'(z) */
                    dz[r * L + t] = magnitude ? fabs(dgate) * ys[t] : dgate * ys[t];
                }
                double dut = 0.0, ddt = 0.0;
                ACC(dut, Dr * dy);
                ACC(dDr, dy * ut);
                const double* hp = hs + t * N;        /* h_{t-1} */
                const double* hc = hs + (t + 1) * N;  /* h_t     */
                for (int64_t n = 0; n < N; ++n) {
                    const double Bn = Bb[n * L + t], Cn = Cb[n * L + t];
                    const double G = dy * Cn + g[n];  /* dL/dh_t */
                    const double abar = exp(dt * Ar[n]);
                    const double ah = abar * hp[n];
                    ACC(ddt, G * Ar[n] * ah);         /* through abar = exp(dt A) */
                    ACC(ddt, G * Bn * ut);            /* through dt B u           */
                    ACC(dA[r * N + n], G * dt * ah);
                    ACC(accB[(b * N + n) * L + t], G * dt * ut);
                    ACC(accC[(b * N + n) * L + t], dy * hc[n]);
                    ACC(dut, G * dt * Bn);
                    g[n] = abar * G;                  /* dL/dh_{t-1} from this step */
                }
                du[r * L + t] = dut;
                const double dpre = ddt * dsp;
                ddelta[r * L + t] = dpre;
                dbr += dpre;
            }
            if (dD) dD[r] = dDr;
            if (dbias) dbias[r] = dbr;
            if (dh0)
                for (int64_t n = 0; n < N; ++n) dh0[r * N + n] = magnitude ? fabs(g[n]) : g[n];
        }
#undef ACC
        free(hs); free(ys); free(g);
    }
    for (size_t i = 0; i < nbc; ++i) { dB[i] = 0.0; dC[i] = 0.0; }
    for (int k = 0; k < nt; ++k) {
        const double* sB = shares + (size_t)k * 2 * (nbc ? nbc : 1);
        const double* sC = sB + (nbc ? nbc : 1);
        for (size_t i = 0; i < nbc; ++i) { dB[i] += sB[i]; dC[i] += sC[i]; }
    }
    free(shares);
    return bad ? -1 : 0;
}

/*
 * Causal depthwise conv1d with optional silu, the step in front of the scan in the tutorial
 * page's `MambaBlock` (a Keras Conv1D with groups = channels, kernel_size 4, bias, channels-first
 * data and padding='causal', then swish; the upstream README's d_conv = 4 "local convolution
 * width").  Keras's Conv1D is a cross-correlation and 'causal' pads K - 1 zeros on the left, so
 *     y[t] = bias + sum_{k=0}^{K-1} w[k] * x[t - (K-1) + k],   x[t < 0] = state (else 0)
 * and w[K-1] multiplies the current input.  Over R rows of length L:
 *   x, out       R x L
 *   w            R x K (the row's channel weights), bias R (may be NULL)
 *   state_in     R x (K-1): the inputs before t = 0, oldest first (NULL: zeros)
 *   state_out    R x (K-1): the last K-1 inputs (from state_in too when L < K-1), or NULL
 *   silu_flag    nonzero: out = silu(y)
 */
int oracle_causal_conv1d(int64_t R, int64_t L, int64_t K, const double* x, const double* w,
                         const double* bias, const double* state_in, int silu_flag, double* out,
                         double* state_out, int nthreads) {
    if (R < 0 || L < 0 || K < 1) return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < R; ++r) {
        /* the row with its K - 1 predecessors in front: ext[j] = x[j - (K-1)] */
        double* ext = (double*)malloc((size_t)(L + K - 1) * sizeof(double));
        if (!ext) { bad = 1; continue; }
        for (int64_t j = 0; j < K - 1; ++j) ext[j] = state_in ? state_in[r * (K - 1) + j] : 0.0;
        for (int64_t t = 0; t < L; ++t) ext[K - 1 + t] = x[r * L + t];
        for (int64_t t = 0; t < L; ++t) {
            double y = bias ? bias[r] : 0.0;
            for (int64_t k = 0; k < K; ++k) y += w[r * K + k] * ext[t + k];
            out[r * L + t] = silu_flag ? silu(y) : y;
        }
        if (state_out)
            for (int64_t j = 0; j < K - 1; ++j) state_out[r * (K - 1) + j] = ext[L + j];
        free(ext);
    }
    return bad ? -1 : 0;
}

/*
 * One recurrent (decode) step over R rows, state updated in place.
 *   state      R x N (in/out)
 *   x, dt, z   R (z may be NULL); dt is raw, softplus(dt + dt_bias) is always applied
 *   A          R x N
 *   Bm, Cm     Bt x N (this token's B and C)
 *   D, dt_bias R (may be NULL: 0)
 *   out        R
 */
int oracle_state_update(int64_t R, int64_t N, int64_t Bt, const int64_t* row_batch,
                        double* state, const double* x, const double* dt, const double* z,
                        const double* A, const double* Bm, const double* Cm,
                        const double* D, const double* dt_bias, double* out, int nthreads) {
    if (R < 0 || N <= 0 || Bt <= 0) return -1;
    set_threads(nthreads);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < R; ++r) {
        const int64_t b = row_batch[r];
        if (b < 0 || b >= Bt) { bad = 1; continue; }
        double* h = state + r * N;
        const double d = sp(dt[r] + (dt_bias ? dt_bias[r] : 0.0));
        double y = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            h[n] = exp(d * A[r * N + n]) * h[n] + d * Bm[b * N + n] * x[r];
            y += Cm[b * N + n] * h[n];
        }
        y += (D ? D[r] : 0.0) * x[r];
        out[r] = z ? y * silu(z[r]) : y;
    }
    return bad ? -1 : 0;
}

/*
 * Mamba-2's SSD layer (the upstream README's Mamba-2 block, whose state size is usually 64 or 128,
 * and its pointer to a minimal SSD module; the pages give no equations for it).  Reading: the same
 * selective recurrence as oracle_selective_scan with Mamba-2's tied parameters --
 *   - heads h of P channels each; the head's A is one scalar A[h], the same for every channel p
 *     and every state n;
 *   - one delta per (batch, time, head), shared by the head's P channels:
 *     delta = softplus(dt + dt_bias[h]) (or dt + dt_bias with the flag off);
 *   - B and C per (batch, time, group), G groups, heads taken in contiguous blocks of H / G
 *     (head h reads group h / (H / G));
 *   - Euler input term delta B x, inclusive h_t, y = C.h_t + D[h] x, out = y silu(z).
 * Layouts: x, z, out (Bt, L, H, P); dt (Bt, L, H); B, C (Bt, L, G, N); A, D, dt_bias (H);
 * h0, last_state (Bt, H, P, N).  Only the (batch, head) pairs listed in `pairs` (flat
 * b * H + h, n_pairs of them) are computed (NULL: all); out and last_state are written in the
 * full layouts at those pairs only.  With magnitude != 0 every term is added in absolute value
 * (|x|, |B|, |C|, |D|, |h0|, |silu(z)|; the decays are positive already): the per-element scale
 * M that bounds the rounding error of any other summation order.
 */
int oracle_ssd_scan(int64_t Bt, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                    const double* x, const double* dt, const double* A, const double* Bm,
                    const double* Cm, const double* D, const double* z, const double* dt_bias,
                    int softplus_flag, const double* h0, const int64_t* pairs, int64_t n_pairs,
                    double* out, double* last_state, int magnitude, int nthreads) {
    if (Bt < 0 || L < 0 || H <= 0 || P <= 0 || G <= 0 || N <= 0 || H % G != 0) return -1;
    set_threads(nthreads);
    const int64_t hpg = H / G;  /* heads per group */
    const int64_t total = pairs ? n_pairs : Bt * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t k = 0; k < total; ++k) {
        const int64_t bh = pairs ? pairs[k] : k;
        if (bh < 0 || bh >= Bt * H) { bad = 1; continue; }
        const int64_t b = bh / H, h = bh % H, g = h / hpg;
        double* st = (double*)malloc((size_t)(P * N) * sizeof(double));
        if (!st) { bad = 1; continue; }
        for (int64_t i = 0; i < P * N; ++i) {
            const double v = h0 ? h0[(b * H + h) * P * N + i] : 0.0;
            st[i] = magnitude ? fabs(v) : v;
        }
        const double a = A[h];
        const double Dh = D ? D[h] : 0.0;
        const double bias = dt_bias ? dt_bias[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double pre = dt[(b * L + t) * H + h] + bias;
            const double delta = softplus_flag ? sp(pre) : pre;
            const double abar = exp(delta * a);                      /* A_bar = exp(delta A[h]) */
            const double* Bt_ = Bm + ((b * L + t) * G + g) * N;
            const double* Ct_ = Cm + ((b * L + t) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const int64_t xi = ((b * L + t) * H + h) * P + p;
                const double xv = magnitude ? fabs(x[xi]) : x[xi];
                double* hp = st + p * N;
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double Bn = magnitude ? fabs(Bt_[n]) : Bt_[n];
                    const double Cn = magnitude ? fabs(Ct_[n]) : Ct_[n];
                    hp[n] = abar * hp[n] + delta * Bn * xv;              /* + delta B x */
                    y += Cn * hp[n];                                    /* C . h_t     */
                }
                y += (magnitude ? fabs(Dh) : Dh) * xv;                 /* D skip      */
                if (z) {
                    const double s = silu(z[xi]);
                    y *= magnitude ? fabs(s) : s;                       /* gate after skip */
                }
                out[xi] = y;
            }
        }
        if (last_state)
            for (int64_t i = 0; i < P * N; ++i) last_state[(b * H + h) * P * N + i] = st[i];
        free(st);
    }
    return bad ? -1 : 0;
}
