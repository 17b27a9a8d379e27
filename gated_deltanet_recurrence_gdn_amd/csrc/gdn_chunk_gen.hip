// gdn_chunk_gen.hip -- the chunked (UT-transform) form for every supported
// shape: chunk length C in {16, 32, 64, 128}, d_k and d_v in {16, 32, 64, 128},
// fp32, bf16 or FP8 inputs, all arithmetic in fp32 on the vector ALUs.
//
// It computes the same per-chunk quantities as the bf16 MFMA kernel: with
// g_i = sum_{r<=i} log2 a_r over the chunk, gam_i = 2^{g_i} and
// G_ij = 2^{g_i - g_j} (j <= i),
//
//   A  = strict_lower(diag(b) (K K^T .* G)),   Tm = (I + A)^{-1}
//   R  = diag(b) (V - diag(gam) K S0^T),       N  = Tm R
//   O  = (diag(gam) Q S0^T + P N) / sqrt(d_k), P  = lower_incl(Q K^T .* G)
//   S  = gam_{n-1} S0 + N^T diag(G_{n-1,.}) K
//
// which is the sequential recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) +
// b_t v_t k_t^T unrolled over n <= C tokens (the chunkwise form that the sglang
// SANA-WM record's cam_scan_bidi_chunkwise names).  This kernel serves the
// fp32 I/O path, the chunk lengths other than 64, and head dims below 32,
// where fp32 accuracy or generality matters more than speed.
//
// Decomposition: a block of 256 threads owns one (b, h) and a d_v tile of up
// to 16 columns, holds its 16 x d_k slice of S in LDS (fp32) for the whole call
// and walks the head's chunks in order.  Per chunk, K is staged in LDS; Q rows
// are read from global memory (L1/L2 resident: a wave's lanes share rows).
// One C x C LDS buffer holds A in its strict lower triangle while Tm is built
// column by column into its strict upper triangle (transposed: Tm_ij at
// [j][i]), so neither overwrites the other; P later replaces A.  Only the
// n real rows of a final partial chunk are ever touched, so no padding enters
// any product.
//
// q, k and v are addressed by token and batch strides.  With the fused prologue
// (template flag PRO) the staged K rows are divided by max(||k||_2, 1e-12), the
// products with q are scaled by 1 / max(||q||_2, 1e-12), and the gate logits
// become b = sigmoid(x_b) and log2 a = -softplus(x_a) / ln 2 (float64).
//
// Decay numerics: log2 a is taken and accumulated in float64, clamped at -200
// (2^-200 is 0 in fp32, so a = 0 zeroes every factor across that token), and
// only 2^{g_i - g_j} with j <= i is formed, from the float64 difference.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int GT = 256;   // threads per block
constexpr int GDVT = 16;  // d_v columns per block (fewer when d_v < 16)
constexpr int GMAXE = 128 * GDVT / GT;  // (token, column) elements per thread, at most

struct GenParams {
    const void *q, *k, *v;
    long long qk_ts, qk_bs, v_ts, v_bs;  // element strides between tokens / batch elements
    const float *beta, *decay;
    const float *state_in;
    float *state_out;
    void *out;
    float *partial, *partial_rev;
    long long T;
    int B, H, dk, dv, C, dvt;
    int reverse, out_mode, both_dirs;
    float scale;
};

template <int IO>
__device__ __forceinline__ float ld_io(const void *p, size_t i) {
    if constexpr (IO == IO_BF16) {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
    } else if constexpr (IO == IO_FP8) {
        float f[4];
        fp8x4_to_f32(reinterpret_cast<const uint8_t *>(p)[i], f);  // the byte in bits 0-7
        return f[0];
    } else {
        return reinterpret_cast<const float *>(p)[i];
    }
}

template <int IO>
__device__ __forceinline__ void st_io(void *p, size_t i, float x) {
    if constexpr (IO != IO_F32)
        reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)f32_to_bf16_bits(x);
    else
        reinterpret_cast<float *>(p)[i] = x;
}

// Shared-memory footprint in bytes for one block.
__host__ __device__ inline size_t gen_lds_bytes(int C, int dk, int dvt) {
    return (size_t)C * sizeof(double)                       // g
           + (size_t)5 * C * sizeof(float)                  // b, gam, G_{n-1,i}, rk, rq
           + (size_t)C * (dk + 1) * sizeof(float)           // K
           + (size_t)C * (C + 1) * sizeof(float)            // A / Tm / P
           + (size_t)dvt * (dk + 1) * sizeof(float)         // S tile
           + (size_t)C * dvt * sizeof(float);               // R, then N
}

template <int IO, bool PRO>
__global__ __launch_bounds__(GT) void chunk_gen_kernel(GenParams p) {
    extern __shared__ double smem_d[];
    const int C = p.C, dk = p.dk, dvt = p.dvt;
    const int PK = dk + 1, PC = C + 1;
    double *g = smem_d;
    float *bet = reinterpret_cast<float *>(g + C);
    float *gam = bet + C;
    float *wl = gam + C;
    float *rk = wl + C;  // prologue: inverse L2 norms of k_i and q_i
    float *rq = rk + C;
    float *Ks = rq + C;
    float *Bf = Ks + (size_t)C * PK;
    float *Ss = Bf + (size_t)C * PC;
    float *Rs = Ss + (size_t)dvt * PK;

    const int tid = threadIdx.x;
    const int dv0 = blockIdx.x * dvt;
    const int h = blockIdx.y;
    const int dir = (p.both_dirs && (int)blockIdx.z >= p.B) ? 1 : 0;
    const int b = (int)blockIdx.z - dir * p.B;
    const bool rev = (p.reverse ^ dir) != 0;
    const long long T = p.T;
    const int H = p.H, dv = p.dv;
    // Row (b, t, h) of the token-major [B, T, H, *] gates and out; q, k and v
    // rows by their strides.
    auto row = [&](long long t) -> size_t { return ((size_t)b * T + t) * H + h; };
    auto qk_row = [&](long long t) -> size_t { return (size_t)b * p.qk_bs + (size_t)t * p.qk_ts + (size_t)h * dk; };
    auto v_row = [&](long long t) -> size_t { return (size_t)b * p.v_bs + (size_t)t * p.v_ts + (size_t)h * dv; };

    const size_t sbase = ((size_t)(b * H + h) * dv + dv0) * dk;
    for (int idx = tid; idx < dvt * dk; idx += GT) {
        const int e = idx / dk, f = idx - e * dk;
        Ss[e * PK + f] = p.state_in ? p.state_in[sbase + idx] : 0.0f;
    }
    void *out = p.out;
    float *part = dir ? p.partial_rev : p.partial;

    const long long nch = (T + C - 1) / C;
    for (long long c = 0; c < nch; ++c) {
        const int n = (int)((T - c * C) < C ? (T - c * C) : C);
        auto tok = [&](int i) -> long long { return rev ? T - 1 - (c * C + i) : c * C + i; };
        __syncthreads();  // the previous chunk is done with K, A/Tm/P, R/N and S

        for (int idx = tid; idx < n * dk; idx += GT) {
            const int i = idx / dk, f = idx - i * dk;
            Ks[i * PK + f] = ld_io<IO>(p.k, qk_row(tok(i)) + f);
        }
        if (tid < n) {
            const size_t r = row(tok(tid));
            double la;
            if constexpr (PRO) {  // b = sigmoid(x), log2 a = -softplus(x) / ln 2
                const double xb = p.beta[r], xa = p.decay[r];
                bet[tid] = (float)(1.0 / (1.0 + exp(-xb)));
                la = -(fmax(xa, 0.0) + log1p(exp(-fabs(xa)))) * 1.4426950408889634;
            } else {
                bet[tid] = p.beta[r];
                la = log2((double)p.decay[r]);
            }
            if (!(la > -200.0)) la = -200.0;
            g[tid] = la;
        }
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) {
                s += g[i];
                g[i] = s;
            }
        }
        if (PRO && tid < n) {  // q and k of token tid divided by max(||.||_2, 1e-12)
            const size_t qr = qk_row(tok(tid));
            float sk = 0.0f, sq = 0.0f;
            for (int f = 0; f < dk; ++f) {
                const float kf = Ks[tid * PK + f], qf = ld_io<IO>(p.q, qr + f);
                sk = fmaf(kf, kf, sk);
                sq = fmaf(qf, qf, sq);
            }
            rk[tid] = inv_norm(sk);
            rq[tid] = inv_norm(sq);
        }
        __syncthreads();
        if (tid < n) {
            gam[tid] = exp2f((float)g[tid]);
            wl[tid] = exp2f((float)(g[n - 1] - g[tid]));
        }
        if constexpr (PRO) {
            for (int idx = tid; idx < n * dk; idx += GT) {
                const int i = idx / dk, f = idx - i * dk;
                Ks[i * PK + f] *= rk[i];
            }
            __syncthreads();
        }
        // A_ij = b_i (k_i . k_j) G_ij, j < i, into the strict lower triangle.
        for (int idx = tid; idx < n * n; idx += GT) {
            const int i = idx / n, j = idx - i * n;
            if (j < i) {
                float s = 0.0f;
                for (int f = 0; f < dk; ++f) s = fmaf(Ks[i * PK + f], Ks[j * PK + f], s);
                Bf[i * PC + j] = bet[i] * s * exp2f((float)(g[i] - g[j]));
            }
        }
        __syncthreads();
        // Tm = (I + A)^{-1}, column j by thread j:
        //   Tm_ij = -sum_{m=j}^{i-1} A_im Tm_mj,  Tm_jj = 1,  stored at [j][i].
        // Thread j reads only A (lower) and its own column (row j, upper), and
        // writes only row j's upper part, so the columns run without barriers.
        if (tid < n) {
            const int j = tid;
            for (int i = j + 1; i < n; ++i) {
                const float *Ai = Bf + i * PC;
                const float *Tj = Bf + j * PC;
                float s0 = Ai[j], s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
                int m = j + 1;
                for (; m + 3 < i; m += 4) {
                    s0 = fmaf(Ai[m], Tj[m], s0);
                    s1 = fmaf(Ai[m + 1], Tj[m + 1], s1);
                    s2 = fmaf(Ai[m + 2], Tj[m + 2], s2);
                    s3 = fmaf(Ai[m + 3], Tj[m + 3], s3);
                }
                for (; m < i; ++m) s0 = fmaf(Ai[m], Tj[m], s0);
                Bf[j * PC + i] = -((s0 + s1) + (s2 + s3));
            }
        }
        // R = diag(b) (V - diag(gam) K S0^T)
        for (int idx = tid; idx < n * dvt; idx += GT) {
            const int i = idx / dvt, e = idx - i * dvt;
            float x = 0.0f;
            for (int f = 0; f < dk; ++f) x = fmaf(Ks[i * PK + f], Ss[e * PK + f], x);
            const float vv = ld_io<IO>(p.v, v_row(tok(i)) + dv0 + e);
            Rs[i * dvt + e] = bet[i] * (vv - gam[i] * x);
        }
        __syncthreads();
        // N = Tm R (into registers, then over R)
        float nreg[GMAXE];
#pragma unroll
        for (int u = 0; u < GMAXE; ++u) {
            const int idx = tid + u * GT;
            nreg[u] = 0.0f;
            if (idx < n * dvt) {
                const int i = idx / dvt, e = idx - i * dvt;
                float s = Rs[i * dvt + e];
                for (int m = 0; m < i; ++m) s = fmaf(Bf[m * PC + i], Rs[m * dvt + e], s);
                nreg[u] = s;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < GMAXE; ++u) {
            const int idx = tid + u * GT;
            if (idx < n * dvt) Rs[idx] = nreg[u];
        }
        // P_ij = (q_i . k_j) G_ij, j <= i, over A's triangle (A and Tm are done).
        for (int idx = tid; idx < n * n; idx += GT) {
            const int i = idx / n, j = idx - i * n;
            if (j <= i) {
                const size_t qr = qk_row(tok(i));
                float s = 0.0f;
                for (int f = 0; f < dk; ++f) s = fmaf(ld_io<IO>(p.q, qr + f), Ks[j * PK + f], s);
                if constexpr (PRO) s *= rq[i];
                Bf[i * PC + j] = s * exp2f((float)(g[i] - g[j]));
            }
        }
        __syncthreads();
        // O = (diag(gam) Q S0^T + P N) / sqrt(d_k)
        for (int idx = tid; idx < n * dvt; idx += GT) {
            const int i = idx / dvt, e = idx - i * dvt;
            const size_t r = row(tok(i));
            const size_t qr = qk_row(tok(i));
            float y = 0.0f;
            for (int f = 0; f < dk; ++f) y = fmaf(ld_io<IO>(p.q, qr + f), Ss[e * PK + f], y);
            if constexpr (PRO) y *= rq[i];
            float s = gam[i] * y;
            for (int j = 0; j <= i; ++j) s = fmaf(Bf[i * PC + j], Rs[j * dvt + e], s);
            s *= p.scale;
            const size_t o = r * dv + dv0 + e;
            if (p.out_mode == OUT_PARTIAL)
                part[o] = s;
            else
                st_io<IO>(out, o, s);
        }
        __syncthreads();
        // S = gam_{n-1} S0 + N^T diag(G_{n-1,.}) K
        const float gl = gam[n - 1];
        for (int idx = tid; idx < dvt * dk; idx += GT) {
            const int e = idx / dk, f = idx - e * dk;
            float s = 0.0f;
            for (int i = 0; i < n; ++i) s = fmaf(Rs[i * dvt + e] * wl[i], Ks[i * PK + f], s);
            Ss[e * PK + f] = fmaf(gl, Ss[e * PK + f], s);
        }
    }
    __syncthreads();
    if (p.state_out) {
        for (int idx = tid; idx < dvt * dk; idx += GT) {
            const int e = idx / dk, f = idx - e * dk;
            p.state_out[sbase + idx] = Ss[e * PK + f];
        }
    }
}

template <int IO, bool PRO>
hipError_t launch_gen(const GenParams &p, hipStream_t stream) {
    const size_t lds = gen_lds_bytes(p.C, p.dk, p.dvt);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chunk_gen_kernel<IO, PRO>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 grid(p.dv / p.dvt, p.H, p.B * (p.both_dirs ? 2 : 1));
    hipLaunchKernelGGL((chunk_gen_kernel<IO, PRO>), grid, dim3(GT), lds, stream, p);
    return hipGetLastError();
}

template <int IO>
hipError_t launch_gen_io(const GenParams &p, int prologue, hipStream_t stream) {
    return prologue ? launch_gen<IO, true>(p, stream) : launch_gen<IO, false>(p, stream);
}

bool pow2_16_128(int x) { return x == 16 || x == 32 || x == 64 || x == 128; }

}  // namespace

bool chunk_general_supported(int C, int dk, int dv) {
    return pow2_16_128(C) && pow2_16_128(dk) && pow2_16_128(dv) &&
           gen_lds_bytes(C, dk, dv < GDVT ? dv : GDVT) <= 160 * 1024;
}

hipError_t launch_chunk_general(const PassArgs &a, int C, hipStream_t stream) {
    if (!chunk_general_supported(C, a.dk, a.dv)) return hipErrorInvalidValue;
    GenParams p;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.qk_ts = a.qk_ts; p.qk_bs = a.qk_bs; p.v_ts = a.v_ts; p.v_bs = a.v_bs;
    p.beta = a.beta; p.decay = a.decay;
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out;
    p.partial = a.partial; p.partial_rev = a.partial_rev;
    p.T = a.T; p.B = a.B; p.H = a.H; p.dk = a.dk; p.dv = a.dv; p.C = C;
    p.dvt = a.dv < GDVT ? a.dv : GDVT;
    p.reverse = a.reverse; p.out_mode = a.out_mode; p.both_dirs = a.both_dirs;
    p.scale = (float)(1.0 / __builtin_sqrt((double)a.dk));
    switch (a.io) {
        case IO_BF16: return launch_gen_io<IO_BF16>(p, a.prologue, stream);
        case IO_FP8: return launch_gen_io<IO_FP8>(p, a.prologue, stream);
        default: return launch_gen_io<IO_F32>(p, a.prologue, stream);
    }
}

}  // namespace gdn
