// gdn_chunk.hip -- chunked (UT-transform) form of the GDN recurrence on bf16 MFMA.
//
// Within a chunk of C tokens starting from state S0 (d_v x d_k), with
// g_i = sum_{r<=i} log a_r, gam_i = e^{g_i}, G_ij = e^{g_i - g_j} (j <= i):
//
//   A  = strict_lower(diag(b) (K K^T .* G))             C x C
//   Tm = (I + A)^{-1}                                   unit lower triangular
//   R  = diag(b) (V - diag(gam) K S0^T)                 C x d_v
//   N  = Tm R                                           the chunk's corrected writes
//   O  = (diag(gam) Q S0^T + P N) / sqrt(d_k),  P = lower_incl(Q K^T .* G)
//   S  = gam_{C-1} S0 + N^T diag(G_{C-1,.}) K
//
// This is the sequential recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) +
// b_t v_t k_t^T rewritten over a block of tokens (the chunkwise WY/UT form; the
// sglang SANA-WM record names its Triton kernel cam_scan_bidi_chunkwise).  The
// C x C and C x d products are dense contractions and run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Parallel decomposition.  Rows of S are independent, so a block owns one
// (b, h) and a 32-wide tile of d_v and walks the head's chunks in order,
// holding its 32 x d_k slice of S in fp32 accumulator registers for the whole
// call.  The S-independent per-chunk work (Gram products, decay factors, the
// triangular inverse) is recomputed by each of the d_v/32 tiles of a head:
// that costs MFMA time but keeps HBM traffic at one read of q/k (the tiles of
// a head are placed on the same XCD so the repeats hit its L2) and buys the
// CU count the sequential chunk chain needs.
//
// Operand layouts.  A 32x32 MFMA accumulator holds 4 consecutive ROWS per
// lane, so every product is arranged so that its output rows are the K
// dimension of the product that consumes it:
//   K K^T, K Q^T are computed as (keys x queries): A and P land row-major;
//   K S^T, Q S^T  (tokens x d_v): R lands as R^T [d_v][token];
//   N = Tm R      (tokens x d_v): N^T [d_v][token];
//   S^T += K^T N~ (d_k x d_v): the state lands as S [d_v][d_k].
// Only K needs a transposed copy in LDS (for the state update).
//
// Decay numerics: g is accumulated in float64 from log a (a = 0 is clamped to
// log a = -1000, which makes every factor across that token exactly 0 in
// fp32), and only e^{g_i - g_j} for j <= i is ever formed, so nothing
// overflows however strong the decay.
//
// A final chunk shorter than C is padded with k = q = v = 0, b = 0, a = 1,
// which leaves every product exact for the real tokens.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int C = 64;     // chunk length
constexpr int NT = 256;   // threads per block: 4 waves
constexpr int DVT = 32;   // d_v columns per block

struct ChunkParams {
    const uint16_t *q, *k, *v;
    const float *beta, *decay;
    const float *state_in;
    float *state_out;
    void *out;
    float *partial;
    long long T;
    int H, dv, ntile, nblocks;
    int reverse, out_mode, xcd_remap;
    float scale;
};

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t a, const bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t ld8(const uint16_t *p) {
    bf16x8_t r;
    __builtin_memcpy(&r, p, 16);
    return r;
}

// acc += A[arow0 .. +32][k] * B[brow0 .. +32][k]^T over k in [k0, k1), where
// both operands are row-major bf16 with the contraction index contiguous.
__device__ __forceinline__ f32x16_t mma_nt(const uint16_t *A, int lda, int arow0, const uint16_t *B,
                                           int ldb, int brow0, int k0, int k1, f32x16_t acc, int lane) {
    const uint16_t *pa = A + (arow0 + (lane & 31)) * lda + 8 * (lane >> 5);
    const uint16_t *pb = B + (brow0 + (lane & 31)) * ldb + 8 * (lane >> 5);
    for (int k = k0; k < k1; k += 16) acc = mfma(ld8(pa + k), ld8(pb + k), acc);
    return acc;
}

// Row index (within a 32x32 accumulator tile) of element r of lane `lane`.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}

template <bool BF16>
__device__ __forceinline__ void store_elem(void *out, size_t e, float x) {
    if constexpr (BF16)
        reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)f32_to_bf16_bits(x);
    else
        reinterpret_cast<float *>(out)[e] = x;
}

template <int DK>
struct __align__(16) Smem {
    static constexpr int LK = DK + 8;  // padded row length (bf16) of d_k-long rows
    static constexpr int LC = C + 8;   // padded row length (bf16) of C-long rows
    static constexpr int LF = C + 4;   // padded row length (fp32) of C-long rows
    uint16_t Ks[C][LK];     // K, token-major
    uint16_t Qs[C][LK];     // Q, token-major
    uint16_t Kt[DK][LC];    // K^T
    uint16_t Vt[DVT][LC];   // V tile, transposed
    uint16_t Sb[DVT][LK];   // bf16 copy of the state tile, row-major [d_v][d_k]
    float Af[C][LF];        // A (lower part read only)
    float Tf[C][LF];        // (I + A)^-1 in fp32
    uint16_t Tb[C][LC];     // (I + A)^-1 in bf16, zero above the diagonal
    uint16_t Pb[C][LC];     // P, zero above the diagonal
    uint16_t Rt[DVT][LC];   // R^T
    uint16_t Nt[DVT][LC];   // N^T
    uint16_t Nd[DVT][LC];   // (diag(G_{C-1,.}) N)^T
    double g[C];            // cumulative log decay
    float gam[C];           // e^{g_i}
    float glast[C];         // e^{g_{C-1} - g_i}
    float bet[C];
    float dec[C];
    float Y[3][16][16];     // triangular-inverse temporaries
};

template <int DK, bool BF16>
__global__ __launch_bounds__(NT) void chunk_kernel(ChunkParams p) {
    static_assert(DK % 32 == 0, "d_k must be a multiple of 32");
    using SM = Smem<DK>;
    constexpr int LK = SM::LK, LC = SM::LC;
    constexpr int NSB = DK / 32;  // 32-row blocks of S^T (d_k rows)
    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int col = lane & 31;    // accumulator column

    // Block -> (b, h, d_v tile).  With the XCD remap, the ntile blocks of one head
    // get linear ids that differ by multiples of 8, i.e. land on one XCD.
    int L = blockIdx.x;
    int head, tile;
    if (p.xcd_remap) {
        const int xcd = L & 7, slot = L >> 3;
        tile = slot % p.ntile;
        head = (slot / p.ntile) * 8 + xcd;
    } else {
        tile = L % p.ntile;
        head = L / p.ntile;
    }
    const int h = head % p.H;
    const int b = head / p.H;
    const int H = p.H;
    const int dv = p.dv;
    const int dv0 = tile * DVT;
    const long long T = p.T;

    // fp32 state S^T block (d_k rows 32*wid .., d_v cols dv0 + col), waves < NSB.
    f32x16_t st = zero16();
    const size_t sbase = ((size_t)(b * H + h) * dv + dv0 + col) * DK;
    if (wid < NSB) {
        if (p.state_in) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dk = 32 * wid + 8 * r4 + 4 * (lane >> 5);
                const float4 s4 = *reinterpret_cast<const float4 *>(p.state_in + sbase + dk);
                st[4 * r4 + 0] = s4.x; st[4 * r4 + 1] = s4.y; st[4 * r4 + 2] = s4.z; st[4 * r4 + 3] = s4.w;
            }
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int dk = 32 * wid + 8 * r4 + 4 * (lane >> 5);
            uint2 w;
            w.x = pack_bf16x2(st[4 * r4 + 0], st[4 * r4 + 1]);
            w.y = pack_bf16x2(st[4 * r4 + 2], st[4 * r4 + 3]);
            *reinterpret_cast<uint2 *>(&sm.Sb[col][dk]) = w;
        }
    }
    __syncthreads();

    const long long nchunks = (T + C - 1) / C;
    for (long long ci = 0; ci < nchunks; ++ci) {
        const long long s0 = ci * C;  // first sequence index of the chunk
        const int n = (int)((T - s0) < C ? (T - s0) : C);
        auto tok = [&](int j) -> long long { return p.reverse ? T - 1 - (s0 + j) : s0 + j; };

        // ---- P0: stage K, Q, V tile, b, a --------------------------------------
        {
            constexpr int VPR = DK / 8;  // 16-byte vectors per q/k row
#pragma unroll
            for (int i = 0; i < (C * VPR) / NT; ++i) {
                const int vi = tid + i * NT;
                const int j = vi / VPR, seg = vi % VPR;
                uint4 kw = make_uint4(0, 0, 0, 0), qw = make_uint4(0, 0, 0, 0);
                if (j < n) {
                    const size_t e = ((size_t)(b * T + tok(j)) * H + h) * DK + seg * 8;
                    kw = *reinterpret_cast<const uint4 *>(p.k + e);
                    qw = *reinterpret_cast<const uint4 *>(p.q + e);
                }
                *reinterpret_cast<uint4 *>(&sm.Ks[j][seg * 8]) = kw;
                *reinterpret_cast<uint4 *>(&sm.Qs[j][seg * 8]) = qw;
                const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.Kt[seg * 8 + 2 * e][j] = (uint16_t)(kk[e] & 0xffffu);
                    sm.Kt[seg * 8 + 2 * e + 1][j] = (uint16_t)(kk[e] >> 16);
                }
            }
            {
                // V tile: C tokens x 32 d_v = 256 vectors, one per thread.
                const int j = tid >> 2, part = tid & 3;
                uint4 vw = make_uint4(0, 0, 0, 0);
                if (j < n)
                    vw = *reinterpret_cast<const uint4 *>(p.v + ((size_t)(b * T + tok(j)) * H + h) * dv + dv0 + part * 8);
                const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.Vt[part * 8 + 2 * e][j] = (uint16_t)(vv[e] & 0xffffu);
                    sm.Vt[part * 8 + 2 * e + 1][j] = (uint16_t)(vv[e] >> 16);
                }
            }
            if (tid < C) {
                float bb = 0.f, aa = 1.f;
                if (tid < n) {
                    const size_t g = (size_t)(b * T + tok(tid)) * H + h;
                    bb = p.beta[g];
                    aa = p.decay[g];
                }
                sm.bet[tid] = bb;
                sm.dec[tid] = aa;
            }
        }
        __syncthreads();

        // ---- P1: decay factors (wave 0) ------------------------------------------
        if (wid == 0) {
            const float a = sm.dec[lane];
            double x = a > 0.f ? log((double)a) : -1000.0;
            if (x < -1000.0) x = -1000.0;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            sm.g[lane] = x;
            const double glast = __shfl(x, 63, 64);
            sm.gam[lane] = expf((float)x);
            sm.glast[lane] = expf((float)(glast - x));
        }
        __syncthreads();

        // ---- P2: Gram blocks -> A, P;  K S^T -> R;  Q S^T kept for O ------------
        // Tiles are (key block jb, query block ib): A[i][j] and P[i][j] need j <= i.
        f32x16_t xo = zero16();  // waves 2, 3: Q S^T for token block (wid - 2)
        {
            auto gram_to_A = [&](int jb, int ib) {
                f32x16_t acc = mma_nt(&sm.Ks[0][0], LK, 32 * jb, &sm.Ks[0][0], LK, 32 * ib, 0, DK, zero16(), lane);
                const int i = 32 * ib + col;
                const double gi = sm.g[i];
                const float bi = sm.bet[i];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int j0 = 32 * jb + 8 * r4 + 4 * (lane >> 5);
                    float4 o;
                    float *op = &o.x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + e;
                        op[e] = (j < i) ? bi * expf((float)(gi - sm.g[j])) * acc[4 * r4 + e] : 0.f;
                    }
                    *reinterpret_cast<float4 *>(&sm.Af[i][j0]) = o;
                }
            };
            auto gram_to_P = [&](int jb, int ib) {
                f32x16_t acc = mma_nt(&sm.Ks[0][0], LK, 32 * jb, &sm.Qs[0][0], LK, 32 * ib, 0, DK, zero16(), lane);
                const int i = 32 * ib + col;
                const double gi = sm.g[i];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int j0 = 32 * jb + 8 * r4 + 4 * (lane >> 5);
                    float pv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + e;
                        pv[e] = (j <= i) ? expf((float)(gi - sm.g[j])) * acc[4 * r4 + e] : 0.f;
                    }
                    uint2 w;
                    w.x = pack_bf16x2(pv[0], pv[1]);
                    w.y = pack_bf16x2(pv[2], pv[3]);
                    *reinterpret_cast<uint2 *>(&sm.Pb[i][j0]) = w;
                }
            };
            auto ks_to_R = [&](int tb) {
                f32x16_t acc = mma_nt(&sm.Ks[0][0], LK, 32 * tb, &sm.Sb[0][0], LK, 0, 0, DK, zero16(), lane);
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int i0 = 32 * tb + 8 * r4 + 4 * (lane >> 5);
                    const uint2 vw = *reinterpret_cast<const uint2 *>(&sm.Vt[col][i0]);
                    const float vv[4] = {bf16_lo(vw.x), bf16_hi(vw.x), bf16_lo(vw.y), bf16_hi(vw.y)};
                    float rv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = i0 + e;
                        rv[e] = sm.bet[i] * (vv[e] - sm.gam[i] * acc[4 * r4 + e]);
                    }
                    uint2 w;
                    w.x = pack_bf16x2(rv[0], rv[1]);
                    w.y = pack_bf16x2(rv[2], rv[3]);
                    *reinterpret_cast<uint2 *>(&sm.Rt[col][i0]) = w;
                }
            };
            if (wid == 0) {
                gram_to_A(0, 0);
                gram_to_P(0, 0);
                ks_to_R(0);
            } else if (wid == 1) {
                gram_to_A(0, 1);
                gram_to_P(0, 1);
                ks_to_R(1);
            } else {
                const int tb = wid - 2;
                if (wid == 2) gram_to_A(1, 1);
                else gram_to_P(1, 1);
                xo = mma_nt(&sm.Qs[0][0], LK, 32 * tb, &sm.Sb[0][0], LK, 0, 0, DK, zero16(), lane);
#pragma unroll
                for (int r = 0; r < 16; ++r) xo[r] *= sm.gam[32 * tb + acc_row(r, lane)];
            }
            // P[i][j] for the (query block a, key block b) tile is never read: the
            // O product for query block a stops at key 31.
        }
        __syncthreads();

        // ---- P3: Tm = (I + A)^-1 ----------------------------------------------------
        // 16x16 diagonal blocks by forward substitution (one wave each, lane = column),
        // then the off-diagonal blocks by distance from the diagonal:
        // T_rc = -T_rr * sum_{k=c}^{r-1} A_rk T_kc.
        if (lane < 16) {
            const int base = 16 * wid, c = lane;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) s -= sm.Af[base + i][base + j] * x[j];
                x[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.Tf[base + i][base + c] = x[i];
        }
        __syncthreads();
        {
            const int ti = tid >> 4, tj = tid & 15;
            for (int d = 1; d < 4; ++d) {
                const int nb = 4 - d;
                for (int cb = 0; cb < nb; ++cb) {
                    const int rb = cb + d;
                    float y = 0.f;
                    for (int kb = cb; kb < rb; ++kb) {
#pragma unroll
                        for (int m = 0; m < 16; ++m)
                            y += sm.Af[16 * rb + ti][16 * kb + m] * sm.Tf[16 * kb + m][16 * cb + tj];
                    }
                    sm.Y[cb][ti][tj] = y;
                }
                __syncthreads();
                for (int cb = 0; cb < nb; ++cb) {
                    const int rb = cb + d;
                    float t = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) t += sm.Tf[16 * rb + ti][16 * rb + m] * sm.Y[cb][m][tj];
                    sm.Tf[16 * rb + ti][16 * cb + tj] = -t;
                }
                __syncthreads();
            }
        }
        // bf16 copy with zeros above the diagonal.
        for (int idx = tid; idx < C * C / 2; idx += NT) {
            const int i = idx / (C / 2), j = 2 * (idx % (C / 2));
            const float t0 = (j <= i) ? sm.Tf[i][j] : 0.f;
            const float t1 = (j + 1 <= i) ? sm.Tf[i][j + 1] : 0.f;
            *reinterpret_cast<uint32_t *>(&sm.Tb[i][j]) = pack_bf16x2(t0, t1);
        }
        __syncthreads();

        // ---- P4: N = Tm R (waves 0, 1: token block wid) ---------------------------
        if (wid < 2) {
            const f32x16_t acc = mma_nt(&sm.Tb[0][0], LC, 32 * wid, &sm.Rt[0][0], LC, 0, 0, 32 * (wid + 1),
                                        zero16(), lane);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int i0 = 32 * wid + 8 * r4 + 4 * (lane >> 5);
                uint2 w, wd;
                w.x = pack_bf16x2(acc[4 * r4 + 0], acc[4 * r4 + 1]);
                w.y = pack_bf16x2(acc[4 * r4 + 2], acc[4 * r4 + 3]);
                wd.x = pack_bf16x2(sm.glast[i0 + 0] * acc[4 * r4 + 0], sm.glast[i0 + 1] * acc[4 * r4 + 1]);
                wd.y = pack_bf16x2(sm.glast[i0 + 2] * acc[4 * r4 + 2], sm.glast[i0 + 3] * acc[4 * r4 + 3]);
                *reinterpret_cast<uint2 *>(&sm.Nt[col][i0]) = w;
                *reinterpret_cast<uint2 *>(&sm.Nd[col][i0]) = wd;
            }
        }
        __syncthreads();

        // ---- P5: outputs (waves 2, 3) and the state update (waves < NSB) ---------
        if (wid >= 2) {
            const int tb = wid - 2;
            xo = mma_nt(&sm.Pb[0][0], LC, 32 * tb, &sm.Nt[0][0], LC, 0, 0, 32 * (tb + 1), xo, lane);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * tb + acc_row(r, lane);
                if (i < n) {
                    const size_t e = ((size_t)(b * T + tok(i)) * H + h) * dv + dv0 + col;
                    const float o = xo[r] * p.scale;
                    if (p.out_mode == OUT_PARTIAL) p.partial[e] = o;
                    else if (p.out_mode == OUT_COMBINE) store_elem<BF16>(p.out, e, p.partial[e] + o);
                    else store_elem<BF16>(p.out, e, o);
                }
            }
        }
        if (wid < NSB) {
            const float gl = sm.gam[C - 1];
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] *= gl;
            st = mma_nt(&sm.Kt[0][0], LC, 32 * wid, &sm.Nd[0][0], LC, 0, 0, C, st, lane);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int dk = 32 * wid + 8 * r4 + 4 * (lane >> 5);
                uint2 w;
                w.x = pack_bf16x2(st[4 * r4 + 0], st[4 * r4 + 1]);
                w.y = pack_bf16x2(st[4 * r4 + 2], st[4 * r4 + 3]);
                *reinterpret_cast<uint2 *>(&sm.Sb[col][dk]) = w;
            }
        }
        __syncthreads();
    }

    if (p.state_out && wid < NSB) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int dk = 32 * wid + 8 * r4 + 4 * (lane >> 5);
            *reinterpret_cast<float4 *>(p.state_out + sbase + dk) =
                make_float4(st[4 * r4 + 0], st[4 * r4 + 1], st[4 * r4 + 2], st[4 * r4 + 3]);
        }
    }
}

template <int DK>
hipError_t launch_dk(const PassArgs &a, hipStream_t stream) {
    ChunkParams p;
    p.q = static_cast<const uint16_t *>(a.q);
    p.k = static_cast<const uint16_t *>(a.k);
    p.v = static_cast<const uint16_t *>(a.v);
    p.beta = a.beta; p.decay = a.decay;
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out; p.partial = a.partial;
    p.T = a.T; p.H = a.H; p.dv = a.dv;
    p.ntile = a.dv / DVT;
    const int heads = a.B * a.H;
    p.nblocks = heads * p.ntile;
    p.xcd_remap = (heads % 8) == 0;
    p.reverse = a.reverse; p.out_mode = a.out_mode;
    p.scale = (float)(1.0 / __builtin_sqrt((double)DK));
    hipLaunchKernelGGL((chunk_kernel<DK, true>), dim3(p.nblocks), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool chunk_supported(int C_, int dk, int dv, int io_bf16) {
    const bool dims = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
    return C_ == C && dims && io_bf16;
}

hipError_t launch_chunk(const PassArgs &a, int C_, hipStream_t stream) {
    if (!chunk_supported(C_, a.dk, a.dv, a.io_bf16)) return hipErrorInvalidValue;
    switch (a.dk) {
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
