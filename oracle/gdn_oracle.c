/*
 * gdn_oracle.c -- plain CPU oracle for the Gated-Delta-Net (GDN) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (per batch element b and head h, independently):
 *
 *     S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = S_t q_t / sqrt(d_k)
 *
 * with S a d_v x d_k matrix (row i is output channel i, so o = S q).  The
 * method is the GDN linear-attention recurrence that the librediffusion PR #21
 * page ("feat(sana): in-tree SANA-Streaming V2V DiT (GDN linear-attention) +
 * C-API", section "What's added") implements as a CUDA kernel, and whose
 * per-token inputs q, k, v, beta, decay are the arguments of the SANA-WM
 * camera-GDN method in the sglang source record (page "errors.standardbeagle
 * .com ... sana-wm-triton-camera-gdn-backend-unavailable", field sourceCode).
 * Neither page prints the update; the formula above is the gated delta rule
 * written out, taken as the definition.  beta (b) and decay (a) are plain
 * values in [0, 1], not logits.
 *
 * Layouts (row-major, contiguous, the same as the device library's):
 *   q, k  [B, T, H, d_k]     v, out  [B, T, H, d_v]
 *   beta, decay  [B, T, H]   state   [B, H, d_v, d_k]
 *
 * Functions:
 *   oracle_forward_f64   sequential recurrence in float64 (the graded oracle)
 *   oracle_forward_f32   the same loop in float32 (shows the fp32 error floor)
 *   oracle_bidi_f64      causal scan + reversed causal scan, summed in f64
 *   oracle_chunkwise_f64 the chunked (UT-transform) form of the same algebra,
 *                        in float64, for brute-force agreement with the above
 *   oracle_dense_f64     tiny brute force: S_t from explicit products of the
 *                        per-token transition matrices M_t = a_t (I - b_t k k^T)
 *
 * Built with -O2 -ffp-contract=off and no fast-math; OpenMP threads run over
 * the (b, h) pairs, which are independent.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Offset of token (b, t, h) in a [B, T, H, d] tensor. */
static size_t tok(long b, long t, long h, long T, long H, long d)
{
    return (size_t)(((b * T + t) * H + h) * d);
}

/* Offset of gate (b, t, h) in a [B, T, H] tensor. */
static size_t gate(long b, long t, long h, long T, long H)
{
    return (size_t)((b * T + t) * H + h);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One (b, h) pair of the sequential recurrence in float64.  When reverse is
 * non-zero the time index runs T-1 .. 0 instead of 0 .. T-1; this is exactly
 * "run the causal recurrence on the time-reversed sequence, then reverse the
 * outputs back", the second half of the bidirectional form.  When accumulate
 * is non-zero the outputs are added into out instead of stored.
 */
static void seq_head_f64(int b, int h, int H, long T, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *beta, const double *decay,
                         const double *state_in, double *out, double *state_out,
                         int reverse, int accumulate)
{
    double *S = (double *)calloc((size_t)dv * dk, sizeof(double));
    double *u = (double *)malloc((size_t)dv * sizeof(double));
    const double scale = 1.0 / sqrt((double)dk);
    if (state_in) {
        memcpy(S, state_in + ((size_t)b * H + h) * dv * dk,
               (size_t)dv * dk * sizeof(double));
    }
    for (long s = 0; s < T; ++s) {
        const long t = reverse ? T - 1 - s : s;
        const double *kt = k + tok(b, t, h, T, H, dk);
        const double *qt = q + tok(b, t, h, T, H, dk);
        const double *vt = v + tok(b, t, h, T, H, dv);
        const double bt = beta[gate(b, t, h, T, H)];
        const double at = decay[gate(b, t, h, T, H)];
        double *ot = out + tok(b, t, h, T, H, dv);
        /* u = S k */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kt[j];
            u[i] = acc;
        }
        /* S = a (S - b u k^T) + b v k^T,  i.e.  a S (I - b k k^T) + b v k^T */
        for (int i = 0; i < dv; ++i) {
            for (int j = 0; j < dk; ++j) {
                double *sij = &S[(size_t)i * dk + j];
                *sij = at * (*sij - bt * u[i] * kt[j]) + bt * vt[i] * kt[j];
            }
        }
        /* o = S q / sqrt(d_k) */
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qt[j];
            if (accumulate) ot[i] += acc * scale;
            else ot[i] = acc * scale;
        }
    }
    if (state_out) {
        memcpy(state_out + ((size_t)b * H + h) * dv * dk, S,
               (size_t)dv * dk * sizeof(double));
    }
    free(u);
    free(S);
}

/*
 * Causal recurrence over T tokens, float64.  state_in may be NULL (zero
 * initial state); state_out may be NULL (final state discarded).
 */
void oracle_forward_f64(int B, long T, int H, int dk, int dv,
                        const double *q, const double *k, const double *v,
                        const double *beta, const double *decay,
                        const double *state_in, double *out, double *state_out)
{
    int bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        seq_head_f64(bh / H, bh % H, H, T, dk, dv, q, k, v, beta, decay,
                     state_in, out, state_out, 0, 0);
    }
}

/*
 * Bidirectional form: out = fwd(x; S=0) + R(fwd(R(x); S=0)), R reversing the
 * time axis.  Token t is counted by both directions.  The sum is in float64;
 * no state is returned.  (SANA-WM bidirectional variant, FlashDreams
 * "SANA-WM" page, section "Bidirectional variant": a complete clip in one
 * pass; the sglang record names the kernel cam_scan_bidi_chunkwise.)
 */
void oracle_bidi_f64(int B, long T, int H, int dk, int dv,
                     const double *q, const double *k, const double *v,
                     const double *beta, const double *decay, double *out)
{
    int bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        seq_head_f64(bh / H, bh % H, H, T, dk, dv, q, k, v, beta, decay,
                     NULL, out, NULL, 0, 0);
        seq_head_f64(bh / H, bh % H, H, T, dk, dv, q, k, v, beta, decay,
                     NULL, out, NULL, 1, 1);
    }
}

/* The same sequential loop with float32 storage and arithmetic. */
void oracle_forward_f32(int B, long T, int H, int dk, int dv,
                        const float *q, const float *k, const float *v,
                        const float *beta, const float *decay,
                        const float *state_in, float *out, float *state_out)
{
    int bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        float *S = (float *)calloc((size_t)dv * dk, sizeof(float));
        float *u = (float *)malloc((size_t)dv * sizeof(float));
        const float scale = 1.0f / sqrtf((float)dk);
        if (state_in) {
            memcpy(S, state_in + ((size_t)b * H + h) * dv * dk,
                   (size_t)dv * dk * sizeof(float));
        }
        for (long t = 0; t < T; ++t) {
            const float *kt = k + tok(b, t, h, T, H, dk);
            const float *qt = q + tok(b, t, h, T, H, dk);
            const float *vt = v + tok(b, t, h, T, H, dv);
            const float bt = beta[gate(b, t, h, T, H)];
            const float at = decay[gate(b, t, h, T, H)];
            float *ot = out + tok(b, t, h, T, H, dv);
            for (int i = 0; i < dv; ++i) {
                float acc = 0.0f;
                for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * kt[j];
                u[i] = acc;
            }
            for (int i = 0; i < dv; ++i) {
                for (int j = 0; j < dk; ++j) {
                    float *sij = &S[(size_t)i * dk + j];
                    *sij = at * (*sij - bt * u[i] * kt[j]) + bt * vt[i] * kt[j];
                }
            }
            for (int i = 0; i < dv; ++i) {
                float acc = 0.0f;
                for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * qt[j];
                ot[i] = acc * scale;
            }
        }
        if (state_out) {
            memcpy(state_out + ((size_t)b * H + h) * dv * dk, S,
                   (size_t)dv * dk * sizeof(float));
        }
        free(u);
        free(S);
    }
}

/*
 * Chunked form, float64.  Inside a chunk of n <= C tokens starting from state
 * S0, write nu_i = b_i (v_i - a_i S_{i-1} k_i), so that S_i = a_i S_{i-1} +
 * nu_i k_i^T.  Unrolling gives S_i = gam_i S0 + sum_{j<=i} G_ij nu_j k_j^T with
 * gam_i = a_0 ... a_i and G_ij = a_{j+1} ... a_i (G_ii = 1).  Substituting
 * back, the nu's solve the unit lower-triangular system
 *     (I + A) N = diag(b) V - diag(b gam) K S0^T,
 *     A_ij = b_i G_ij (k_i . k_j)   for j < i,
 * i.e. N = U - W S0^T with Tm = (I + A)^-1, W = Tm diag(b gam) K and
 * U = Tm diag(b) V.  Then
 *     O   = (diag(gam) Q S0^T + P N) / sqrt(d_k),  P_ij = G_ij (q_i . k_j), j <= i
 *     S_n = gam_{n-1} S0 + N^T diag(G_{n-1, .}) K.
 * The decay products are formed as plain products (no logarithms), so a
 * token with a = 0 is exact.  A final chunk shorter than C uses n < C rows.
 */
static void chunk_head_f64(int b, int h, int H, long T, int dk, int dv, int C,
                           const double *q, const double *k, const double *v,
                           const double *beta, const double *decay,
                           const double *state_in, double *out, double *state_out)
{
    const double scale = 1.0 / sqrt((double)dk);
    double *S = (double *)calloc((size_t)dv * dk, sizeof(double));
    double *G = (double *)malloc((size_t)C * C * sizeof(double));
    double *gam = (double *)malloc((size_t)C * sizeof(double));
    double *A = (double *)malloc((size_t)C * C * sizeof(double));
    double *Tm = (double *)malloc((size_t)C * C * sizeof(double));
    double *W = (double *)malloc((size_t)C * dk * sizeof(double));
    double *U = (double *)malloc((size_t)C * dv * sizeof(double));
    double *N = (double *)malloc((size_t)C * dv * sizeof(double));
    double *P = (double *)malloc((size_t)C * C * sizeof(double));
    double *Snew = (double *)malloc((size_t)dv * dk * sizeof(double));
    if (state_in) {
        memcpy(S, state_in + ((size_t)b * H + h) * dv * dk,
               (size_t)dv * dk * sizeof(double));
    }
    for (long t0 = 0; t0 < T; t0 += C) {
        const int n = (T - t0 < C) ? (int)(T - t0) : C;
#define KROW(i) (k + tok(b, t0 + (i), h, T, H, dk))
#define QROW(i) (q + tok(b, t0 + (i), h, T, H, dk))
#define VROW(i) (v + tok(b, t0 + (i), h, T, H, dv))
#define BETA(i) (beta[gate(b, t0 + (i), h, T, H)])
#define DECAY(i) (decay[gate(b, t0 + (i), h, T, H)])
        /* decay products */
        for (int i = 0; i < n; ++i) {
            gam[i] = (i == 0 ? 1.0 : gam[i - 1]) * DECAY(i);
            for (int j = 0; j < n; ++j) G[i * C + j] = 0.0;
            G[i * C + i] = 1.0;
            for (int j = i - 1; j >= 0; --j) G[i * C + j] = G[i * C + j + 1] * DECAY(j + 1);
        }
        /* A (strictly lower) and P (lower, diagonal included) */
        for (int i = 0; i < n; ++i) {
            for (int j = 0; j < n; ++j) {
                double kk = 0.0, qk = 0.0;
                for (int e = 0; e < dk; ++e) {
                    kk += KROW(i)[e] * KROW(j)[e];
                    qk += QROW(i)[e] * KROW(j)[e];
                }
                A[i * C + j] = (j < i) ? BETA(i) * G[i * C + j] * kk : 0.0;
                P[i * C + j] = (j <= i) ? G[i * C + j] * qk : 0.0;
            }
        }
        /* Tm = (I + A)^-1 by forward substitution, column by column */
        for (int c = 0; c < n; ++c) {
            for (int i = 0; i < n; ++i) {
                double x = (i == c) ? 1.0 : 0.0;
                for (int j = 0; j < i; ++j) x -= A[i * C + j] * Tm[j * C + c];
                Tm[i * C + c] = x;
            }
        }
        /* W = Tm diag(b gam) K,  U = Tm diag(b) V */
        for (int i = 0; i < n; ++i) {
            for (int e = 0; e < dk; ++e) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += Tm[i * C + j] * BETA(j) * gam[j] * KROW(j)[e];
                W[(size_t)i * dk + e] = acc;
            }
            for (int e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += Tm[i * C + j] * BETA(j) * VROW(j)[e];
                U[(size_t)i * dv + e] = acc;
            }
        }
        /* N = U - W S0^T */
        for (int i = 0; i < n; ++i) {
            for (int e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int f = 0; f < dk; ++f) acc += W[(size_t)i * dk + f] * S[(size_t)e * dk + f];
                N[(size_t)i * dv + e] = U[(size_t)i * dv + e] - acc;
            }
        }
        /* O = (diag(gam) Q S0^T + P N) / sqrt(d_k) */
        for (int i = 0; i < n; ++i) {
            double *ot = out + tok(b, t0 + i, h, T, H, dv);
            for (int e = 0; e < dv; ++e) {
                double inter = 0.0, intra = 0.0;
                for (int f = 0; f < dk; ++f) inter += QROW(i)[f] * S[(size_t)e * dk + f];
                for (int j = 0; j < n; ++j) intra += P[i * C + j] * N[(size_t)j * dv + e];
                ot[e] = (gam[i] * inter + intra) * scale;
            }
        }
        /* S_n = gam_{n-1} S0 + N^T diag(G_{n-1,.}) K */
        for (int e = 0; e < dv; ++e) {
            for (int f = 0; f < dk; ++f) {
                double acc = 0.0;
                for (int j = 0; j < n; ++j) acc += N[(size_t)j * dv + e] * G[(n - 1) * C + j] * KROW(j)[f];
                Snew[(size_t)e * dk + f] = gam[n - 1] * S[(size_t)e * dk + f] + acc;
            }
        }
        memcpy(S, Snew, (size_t)dv * dk * sizeof(double));
#undef KROW
#undef QROW
#undef VROW
#undef BETA
#undef DECAY
    }
    if (state_out) {
        memcpy(state_out + ((size_t)b * H + h) * dv * dk, S,
               (size_t)dv * dk * sizeof(double));
    }
    free(Snew); free(P); free(N); free(U); free(W); free(Tm); free(A);
    free(gam); free(G); free(S);
}

void oracle_chunkwise_f64(int B, long T, int H, int dk, int dv, int C,
                          const double *q, const double *k, const double *v,
                          const double *beta, const double *decay,
                          const double *state_in, double *out, double *state_out)
{
    int bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * H; ++bh) {
        chunk_head_f64(bh / H, bh % H, H, T, dk, dv, C, q, k, v, beta, decay,
                       state_in, out, state_out);
    }
}

/*
 * Tiny brute force.  Each token maps the state affinely:
 *     S_t = S_{t-1} M_t + b_t v_t k_t^T,   M_t = a_t (I - b_t k_t k_t^T),
 * so
 *     S_t = S0 M_1 ... M_t + sum_{s<=t} b_s v_s k_s^T M_{s+1} ... M_t.
 * Every S_t is formed from that sum with explicit d_k x d_k matrix products
 * (O(T^2 d^3)), never from S_{t-1}.  Meant for T <= 32, d <= 16.
 */
void oracle_dense_f64(int B, long T, int H, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      const double *beta, const double *decay,
                      const double *state_in, double *out, double *state_out)
{
    const double scale = 1.0 / sqrt((double)dk);
    double *M = (double *)malloc((size_t)T * dk * dk * sizeof(double));
    double *Pr = (double *)malloc((size_t)dk * dk * sizeof(double));
    double *Tmp = (double *)malloc((size_t)dk * dk * sizeof(double));
    double *St = (double *)malloc((size_t)dv * dk * sizeof(double));
    double *X = (double *)malloc((size_t)dv * dk * sizeof(double));
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            for (long t = 0; t < T; ++t) {
                const double *kt = k + tok(b, t, h, T, H, dk);
                const double bt = beta[gate(b, t, h, T, H)];
                const double at = decay[gate(b, t, h, T, H)];
                double *Mt = M + (size_t)t * dk * dk;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dk; ++j)
                        Mt[i * dk + j] = at * ((i == j ? 1.0 : 0.0) - bt * kt[i] * kt[j]);
            }
            for (long t = 0; t < T; ++t) {
                /* term list: s = -1 stands for the initial state */
                for (size_t e = 0; e < (size_t)dv * dk; ++e) St[e] = 0.0;
                for (long s = -1; s <= t; ++s) {
                    /* Pr = M_{s+1} ... M_t (identity when s == t) */
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dk; ++j) Pr[i * dk + j] = (i == j) ? 1.0 : 0.0;
                    for (long r = s + 1; r <= t; ++r) {
                        const double *Mr = M + (size_t)r * dk * dk;
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dk; ++j) {
                                double acc = 0.0;
                                for (int l = 0; l < dk; ++l) acc += Pr[i * dk + l] * Mr[l * dk + j];
                                Tmp[i * dk + j] = acc;
                            }
                        memcpy(Pr, Tmp, (size_t)dk * dk * sizeof(double));
                    }
                    /* X = the left factor: S0, or b_s v_s k_s^T */
                    if (s < 0) {
                        if (!state_in) continue;
                        memcpy(X, state_in + ((size_t)b * H + h) * dv * dk,
                               (size_t)dv * dk * sizeof(double));
                    } else {
                        const double *ks = k + tok(b, s, h, T, H, dk);
                        const double *vs = v + tok(b, s, h, T, H, dv);
                        const double bs = beta[gate(b, s, h, T, H)];
                        for (int i = 0; i < dv; ++i)
                            for (int j = 0; j < dk; ++j) X[i * dk + j] = bs * vs[i] * ks[j];
                    }
                    for (int i = 0; i < dv; ++i)
                        for (int j = 0; j < dk; ++j) {
                            double acc = 0.0;
                            for (int l = 0; l < dk; ++l) acc += X[i * dk + l] * Pr[l * dk + j];
                            St[i * dk + j] += acc;
                        }
                }
                const double *qt = q + tok(b, t, h, T, H, dk);
                double *ot = out + tok(b, t, h, T, H, dv);
                for (int i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dk; ++j) acc += St[i * dk + j] * qt[j];
                    ot[i] = acc * scale;
                }
            }
            if (state_out) {
                if (T == 0) {
                    for (size_t e = 0; e < (size_t)dv * dk; ++e)
                        St[e] = state_in ? state_in[((size_t)b * H + h) * dv * dk + e] : 0.0;
                }
                memcpy(state_out + ((size_t)b * H + h) * dv * dk, St,
                       (size_t)dv * dk * sizeof(double));
            }
        }
    }
    free(X); free(St); free(Tmp); free(Pr); free(M);
}
