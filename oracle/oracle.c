/*
 * CPU oracle for the Mamba selective scan -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, sequential definition of what the HIP path
 * computes, written in fp64.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load it.  It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Inputs are fp32 arrays (bf16 inputs arrive already widened to their exact
 * fp32 values); every operation below is carried out in double precision and
 * results are returned in double.  Build with -ffp-contract=off so that each
 * line is evaluated exactly as written (no fused multiply-add contraction),
 * which makes the step function and the scan bitwise comparable.
 *
 * What is computed, and where the pages state it
 * ----------------------------------------------
 * - The recurrence h_t = dA_t * h_{t-1} + dBx_t with a caller-given initial
 *   state h_0 (zero when absent): "Adding Initial Value Support to Selective
 *   Scan Forward Kernel" (state-spaces/mamba issue 285), the opening question
 *   (h_t = A*h_{t-1} + Bx with h_0 fixed at 0, asking for an initial value).
 * - Discretisation dA_t = exp(delta_t * A[d,n]): same page, the later reply
 *   that gives the scan element as the pair (exp(delta*A), hidden_state) and
 *   the backward note that uses exp(delta_0 * A); dBx_t = delta_t*B_t[n]*x_t
 *   is the additive term of that pair.
 * - The initial state enters as the pair (1, h0), i.e. it is h before step 1,
 *   not a decay factor: same page, the reply that corrects the (h0, 0) seed to
 *   (1, h0).  Here that is simply "h starts at h0".
 * - Output y_t = sum_n C_t[n] h_t[n] + D[d] x_t, gated by silu(z_t) when z is
 *   given: "ggml : add GPU support for Mamba models" (llama.cpp issue 6758):
 *   the ssm_d {d_inner} tensor in compilade's ctx_layer diff, and jploski's
 *   report that ggml_silu(ctx, z) is applied to the z half of xz.  The scan is
 *   inclusive (y_t uses h_t after token t): the mamba page's InclusiveScan.
 * - Inputs are not modified and the final state is a separate output: the
 *   llama.cpp page, compilade's note that ggml_ssm_scan no longer modifies its
 *   inputs and returns the final state with its output.
 * - Optionally the step size is delta + delta_bias[d] (per head for SSD) and
 *   then softplus(v) = log(1 + e^v): the fused dt-bias/softplus input
 *   transform of Mamba's scan (the bias is a model tensor on the llama.cpp
 *   page); off by default.
 * - Backward (gradients of the scan): the mamba page's replies on the
 *   backward kernel -- states recomputed by a forward scan, gradients of the
 *   states carried by a reverse scan over dy * C, the gradient of the initial
 *   state dh * exp(delta_0 * A).  The remaining gradients are the chain rule
 *   through the same recurrence (see oracle_scan_bwd).
 * - Decode (single-token state update, Megatron's selective_state_update in
 *   "Clean up SSM ops directory structure - #6444"): the same step with L = 1,
 *   state updated in place.
 * - Mamba-2 SSD: the same recurrence per (b, head, p) with a scalar A per head,
 *   so dA_t = exp(dt_t * A[h]) for every n, and B/C shared by the heads of a
 *   group (head h uses group h / (H/G)): the SSD kernel family of the Megatron
 *   page, the head-group naming and repeat_interleave of "Tensor-parallel SSM
 *   #333", and the groups-divide-heads rule of "Current Implementation of TP in
 *   MambaMixer2".  The chunked SSD algorithm reaches this recurrence exactly
 *   (up to rounding order); the chunk length does not enter the definition.
 *
 * - Short causal convolution ahead of the scan (ggml's SSM_CONV op of the
 *   llama.cpp page, whose signature ggml_ssm_conv(ctx, s, x, c) and tensor
 *   shapes s {d_conv-1, d_inner, n_seqs}, x {d_inner, n_seq_tokens, n_seqs},
 *   c {d_conv, d_inner} appear in compilade's test patch; the conv bias
 *   tensor ssm_conv1d_b {d_inner} in the ctx_layer diff; the concat of the
 *   carried state with the new tokens in compilade's im2col/concat notes;
 *   Megatron's causal_conv1d_update for the decode step): per channel the
 *   state holds the previous d_conv - 1 inputs, oldest first; the window
 *   xp = [state, x] gives y_t = sum_k c[d][k] xp[t + k] (+ bias, then the
 *   optional SiLU), and the new state is the last d_conv - 1 entries of xp.
 *
 * Layouts: row-major, last index fastest.
 *   scan:   x, delta, z: (B, L, D); Bm, Cm: (B, L, N); A: (D, N); D_skip: (D);
 *           h0: (B, D, N)
 *   step:   state: (S, D, N); x, delta, z: (S, D); Bm, Cm: (S, N)
 *   SSD:    x, z: (B, L, H, P); dt: (B, L, H); A, D_skip: (H); Bm, Cm:
 *           (B, L, G, N); h0: (B, H, P, N)
 *   conv:   x, y: (B, L, D); w: (D, K); bias: (D); state: (B, D, K-1)
 * Outputs are written per requested channel so that a test can evaluate a
 * sample of channels of a full-size problem:
 *   y_out[k*L + t] and h_out[k*N + n] for the k-th requested channel.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

static double silu(double v) { return v / (1.0 + exp(-v)); }

/*
 * The step size as the scan uses it: delta + delta_bias[c] when a bias is
 * given, then softplus(v) = log(1 + e^v) when asked (Mamba's dt projection
 * bias and softplus; the bias tensor exists as a model tensor on the
 * llama.cpp page).  Both off: delta unchanged.
 */
static double step_size(double v, const float *delta_bias, int64_t c, int softplus)
{
    if (delta_bias) v += (double)delta_bias[c];
    if (softplus) v = v > 30.0 ? v : log1p(exp(v));
    return v;
}

/*
 * Mamba-1 selective scan for channels c = b*D + d listed in `channels`.
 * D_skip, z and h0 may be NULL (no skip term, no gate, zero initial state).
 */
void oracle_scan(int64_t B, int64_t L, int64_t D, int64_t N,
                 const float *x, const float *delta, const float *A,
                 const float *Bm, const float *Cm, const float *D_skip,
                 const float *z, const float *h0,
                 const int64_t *channels, int64_t n_channels,
                 double *y_out, double *h_out,
                 const float *delta_bias, int delta_softplus)
{
    (void)B;
    for (int64_t k = 0; k < n_channels; ++k) {
        const int64_t b = channels[k] / D;
        const int64_t d = channels[k] % D;
        double *h = h_out + k * N;  /* running state h[n] of this channel */
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? (double)h0[(b * D + d) * N + n] : 0.0;

        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = b * L + t;           /* token (b, t) */
            const double dl = step_size(delta[row * D + d], delta_bias, d, delta_softplus);
            const double u = x[row * D + d];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double dA = exp(dl * (double)A[d * N + n]);
                const double dBx = dl * (double)Bm[row * N + n] * u;
                h[n] = dA * h[n] + dBx;
                acc += (double)Cm[row * N + n] * h[n];
            }
            double v = acc;
            if (D_skip) v += (double)D_skip[d] * u;
            if (z) v *= silu((double)z[row * D + d]);
            y_out[k * L + t] = v;
        }
    }
}

/*
 * Gradients of oracle_scan (the backward of the mamba page's middle replies:
 * the forward states are recomputed, then a reverse-time pass carries the
 * adjoint of the state -- fed by dy * C at every token and decayed by
 * exp(delta * A) from one token to the one before -- and the gradient of h0
 * is exp(delta_0 * A) times the adjoint at the first token).
 *
 * With u_t = delta_t x_t, a_t = exp(delta_t A), h_t = a_t h_{t-1} + u_t B_t,
 * q_t = sum_n C_t h_t + D x_t and y_t = q_t silu(z_t), and g_t = dy_t
 * silu(z_t) the gradient reaching q_t, the adjoint of the state is
 *   lam_t = g_t C_t + a_{t+1} lam_{t+1},  lam_{L-1} = g C + dh_final,
 * and per token
 *   ddelta_t = sum_n lam_t (A a_t h_{t-1} + B_t x_t)   (times the softplus
 *              slope sigmoid(delta + bias) when softplus is on)
 *   dx_t     = sum_n lam_t delta_t B_t + D g_t
 *   dz_t     = dy_t q_t silu'(z_t)
 *   dB_t    += lam_t delta_t x_t,   dC_t += g_t h_t   (summed over channels)
 *   dA      += lam_t delta_t a_t h_{t-1},  dD += g_t x_t,  dbias += ddelta_t
 *   dh0      = a_0 lam_0.
 * Inputs as oracle_scan, plus dy (B, L, D) and dh_final (B, D, N) (NULL =
 * zero).  Per requested channel k: dx, ddelta, dz rows at [k * L + t] and
 * dh0 at [k * N + n] (overwritten); dA (D, N), dD (D), dbias (D), dB and dC
 * (B, L, N) are ADDED TO (the caller zeroes them), with the contributions of
 * the requested channels only.  z NULL: no gate and dz untouched.
 */
void oracle_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N,
                     const float *x, const float *delta, const float *A,
                     const float *Bm, const float *Cm, const float *D_skip,
                     const float *z, const float *h0,
                     const float *dy, const float *dh_final,
                     const float *delta_bias, int delta_softplus,
                     const int64_t *channels, int64_t n_channels,
                     double *dx, double *ddelta, double *dz, double *dh0,
                     double *dA, double *dD, double *dbias, double *dB, double *dC)
{
    (void)B;
    double *h = (double *)malloc((size_t)((L + 1) * N > 0 ? (L + 1) * N : 1) * sizeof(double));
    double *lam = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t k = 0; k < n_channels; ++k) {
        const int64_t b = channels[k] / D;
        const int64_t d = channels[k] % D;
        /* forward: h[(t + 1) * N + n] is the state after token t */
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? (double)h0[(b * D + d) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t row = b * L + t;
            const double dl = step_size(delta[row * D + d], delta_bias, d, delta_softplus);
            const double xv = x[row * D + d];
            for (int64_t n = 0; n < N; ++n) {
                const double a = exp(dl * (double)A[d * N + n]);
                h[(t + 1) * N + n] = a * h[t * N + n] + dl * (double)Bm[row * N + n] * xv;
            }
        }
        /* reverse */
        for (int64_t n = 0; n < N; ++n)
            lam[n] = dh_final ? (double)dh_final[(b * D + d) * N + n] : 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
            const int64_t row = b * L + t;
            const double raw = delta[row * D + d];
            const double dl = step_size(raw, delta_bias, d, delta_softplus);
            const double xv = x[row * D + d];
            const double dyv = dy[row * D + d];
            double q = 0.0;
            for (int64_t n = 0; n < N; ++n)
                q += (double)Cm[row * N + n] * h[(t + 1) * N + n];
            if (D_skip) q += (double)D_skip[d] * xv;
            double g = dyv;
            if (z) {
                const double zv = z[row * D + d];
                const double sg = 1.0 / (1.0 + exp(-zv));
                g = dyv * zv * sg;
                dz[k * L + t] = dyv * q * sg * (1.0 + zv * (1.0 - sg));
            }
            double ddl = 0.0, dxv = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double An = A[d * N + n];
                const double Bn = Bm[row * N + n];
                const double a = exp(dl * An);
                lam[n] += g * (double)Cm[row * N + n];
                dC[row * N + n] += g * h[(t + 1) * N + n];
                dB[row * N + n] += lam[n] * dl * xv;
                ddl += lam[n] * (An * a * h[t * N + n] + Bn * xv);
                dA[d * N + n] += lam[n] * dl * a * h[t * N + n];
                dxv += lam[n] * dl * Bn;
                lam[n] *= a;
            }
            if (D_skip) {
                dxv += (double)D_skip[d] * g;
                dD[d] += g * xv;
            }
            if (delta_softplus) {
                const double v = raw + (delta_bias ? (double)delta_bias[d] : 0.0);
                ddl *= 1.0 / (1.0 + exp(-v));
            }
            dx[k * L + t] = dxv;
            ddelta[k * L + t] = ddl;
            dbias[d] += ddl;
        }
        for (int64_t n = 0; n < N; ++n)
            dh0[k * N + n] = lam[n];
    }
    free(lam);
    free(h);
}

/*
 * One decode step for S sequences: the scan body with L = 1, state updated in
 * place (fp64 state so a test can chain steps without fp32 rounding).
 */
void oracle_state_update(int64_t S, int64_t D, int64_t N, double *state,
                         const float *x, const float *delta, const float *A,
                         const float *Bm, const float *Cm, const float *D_skip,
                         const float *z, double *y,
                         const float *delta_bias, int delta_softplus)
{
    for (int64_t s = 0; s < S; ++s) {
        for (int64_t d = 0; d < D; ++d) {
            double *h = state + (s * D + d) * N;
            const double dl = step_size(delta[s * D + d], delta_bias, d, delta_softplus);
            const double u = x[s * D + d];
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double dA = exp(dl * (double)A[d * N + n]);
                const double dBx = dl * (double)Bm[s * N + n] * u;
                h[n] = dA * h[n] + dBx;
                acc += (double)Cm[s * N + n] * h[n];
            }
            double v = acc;
            if (D_skip) v += (double)D_skip[d] * u;
            if (z) v *= silu((double)z[s * D + d]);
            y[s * D + d] = v;
        }
    }
}

/*
 * Mamba-2 SSD: the recurrence per channel c = (b*H + h)*P + p with scalar
 * A[h] and B/C of group g = h / (H/G).  D_skip, z, h0 may be NULL.
 */
void oracle_ssd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                const float *x, const float *dt, const float *A,
                const float *Bm, const float *Cm, const float *D_skip,
                const float *z, const float *h0,
                const int64_t *channels, int64_t n_channels,
                double *y_out, double *h_out,
                const float *dt_bias, int dt_softplus)
{
    (void)B;
    const int64_t heads_per_group = H / G;
    for (int64_t k = 0; k < n_channels; ++k) {
        const int64_t c = channels[k];
        const int64_t p = c % P;
        const int64_t hd = (c / P) % H;
        const int64_t b = c / (P * H);
        const int64_t g = hd / heads_per_group;
        double *h = h_out + k * N;
        for (int64_t n = 0; n < N; ++n)
            h[n] = h0 ? (double)h0[((b * H + hd) * P + p) * N + n] : 0.0;

        for (int64_t t = 0; t < L; ++t) {
            const int64_t tok = b * L + t;
            const double dl = step_size(dt[tok * H + hd], dt_bias, hd, dt_softplus);
            const double u = x[(tok * H + hd) * P + p];
            const double dA = exp(dl * (double)A[hd]);
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double dBx = dl * (double)Bm[(tok * G + g) * N + n] * u;
                h[n] = dA * h[n] + dBx;
                acc += (double)Cm[(tok * G + g) * N + n] * h[n];
            }
            double v = acc;
            if (D_skip) v += (double)D_skip[hd] * u;
            if (z) v *= silu((double)z[(tok * H + hd) * P + p]);
            y_out[k * L + t] = v;
        }
    }
}

/*
 * Causal convolution of width K over L tokens for every (b, d).  state0 may
 * be NULL (zeros), bias may be NULL; act = 1 applies SiLU to the output.
 * y: (B, L, D); state_out: (B, D, K-1), the last K-1 entries of [state0, x].
 */
void oracle_conv1d(int64_t B, int64_t L, int64_t D, int64_t K,
                   const float *x, const float *w, const float *bias,
                   const float *state0, int act, double *y, double *state_out)
{
    const int64_t W = K - 1 + L;  /* length of the padded sequence */
    double *xp = (double *)malloc((size_t)(W > 0 ? W : 1) * sizeof(double));
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t d = 0; d < D; ++d) {
            for (int64_t j = 0; j < K - 1; ++j)
                xp[j] = state0 ? (double)state0[(b * D + d) * (K - 1) + j] : 0.0;
            for (int64_t t = 0; t < L; ++t)
                xp[K - 1 + t] = x[(b * L + t) * D + d];
            for (int64_t t = 0; t < L; ++t) {
                double v = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    v += (double)w[d * K + k] * xp[t + k];
                if (bias) v += (double)bias[d];
                if (act) v = silu(v);
                y[(b * L + t) * D + d] = v;
            }
            for (int64_t j = 0; j < K - 1; ++j)
                state_out[(b * D + d) * (K - 1) + j] = xp[L + j];
        }
    }
    free(xp);
}

/*
 * One decode step of the causal convolution for S sequences: window =
 * [state, x_t], y = sum_k w[d][k] window[k] (+ bias, SiLU), and the state
 * drops its oldest entry and appends x_t (fp64 state, updated in place).
 */
void oracle_conv1d_update(int64_t S, int64_t D, int64_t K, double *state,
                          const float *x, const float *w, const float *bias,
                          int act, double *y)
{
    for (int64_t s = 0; s < S; ++s) {
        for (int64_t d = 0; d < D; ++d) {
            double *st = state + (s * D + d) * (K - 1);
            const double xt = x[s * D + d];
            double v = 0.0;
            for (int64_t k = 0; k < K - 1; ++k)
                v += (double)w[d * K + k] * st[k];
            v += (double)w[d * K + K - 1] * xt;
            if (bias) v += (double)bias[d];
            if (act) v = silu(v);
            y[s * D + d] = v;
            for (int64_t k = 0; k + 1 < K - 1; ++k)
                st[k] = st[k + 1];
            if (K > 1) st[K - 2] = xt;
        }
    }
}
