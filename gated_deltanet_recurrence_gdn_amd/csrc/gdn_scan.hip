// gdn_scan.hip -- the sequential (token-by-token) form of the GDN recurrence.
//
// Per token, every row i of the d_v x d_k state evolves on its own:
//     u_i = S_i . k,  p_i = S_i . q,  nu_i = b (v_i - a u_i),
//     S_i <- a S_i + nu_i k,          o_i = (a p_i + nu_i (k . q)) / sqrt(d_k)
// which is S_t = a S (I - b k k^T) + b v k^T, o_t = S_t q / sqrt(d_k) written
// row by row.  Row independence is what the "row-split grid + shared-mem
// state" CUDA kernel of the librediffusion PR #21 page ("What's added") uses;
// here the rows are split over lanes instead:
//
//   * a row of d_k fp32 state values lives in the VGPRs of L = d_k / 8 lanes
//     (8 values per lane) for the whole sequence; the two dot products are
//     8 FMAs per lane plus a DPP reduction inside the L-lane group;
//   * a block holds ROWS = min(256 / L, d_v) rows of one (b, h) and streams
//     the head's tokens through LDS in stages of TB tokens: q/k rows are read
//     from HBM as 16-byte vectors, widened to fp32 once, and the per-token
//     k . q is reduced at staging time; the next stage's loads are in flight
//     in registers while the current stage is computed;
//   * outputs are staged in LDS and written as contiguous row segments.
//
// q, k and v are addressed by token and batch strides, so the same kernel reads
// contiguous [B,T,H,d] tensors or views into a packed projection.  With the fused
// prologue (template flag PRO) the staging step also divides each q and k row by
// max(||.||_2, 1e-12) (a sum over the row's L lanes) and turns the gate logits
// into b = sigmoid(x_b), a = exp(-softplus(x_a)), all in fp32.
//
// State traffic: one read of state_in and one write of state_out per call
// (the review on the same page flags per-step global-memory state traffic in
// its gdn_bidi kernel; here the state never leaves the VGPRs mid-call).
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

constexpr int TB = 32;       // tokens per LDS stage
constexpr int NT = 256;      // max threads per block

struct ScanParams {
    const void *q, *k, *v;
    long long qk_ts, qk_bs, v_ts, v_bs;  // element strides between tokens / batch elements
    const float *beta, *decay;
    const float *state_in;
    float *state_out;
    void *out;
    float *partial, *partial_rev;
    long long T;
    int B, H, dv;
    int reverse, out_mode, both_dirs;
    float scale;
};

template <bool BF16>
struct Chunk8;  // 8 consecutive I/O elements held in registers

template <>
struct Chunk8<true> {
    uint4 w;
    __device__ void load(const void *base, size_t elem) {
        w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
    }
    __device__ void zero() { w = make_uint4(0, 0, 0, 0); }
    __device__ void to_f32(float f[8]) const {
        f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    }
};

template <>
struct Chunk8<false> {
    float4 a, b;
    __device__ void load(const void *base, size_t elem) {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + elem);
        a = p[0];
        b = p[1];
    }
    __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ void to_f32(float f[8]) const {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

template <bool BF16>
__device__ __forceinline__ void store_out(void *out, size_t elem, float x) {
    if constexpr (BF16)
        reinterpret_cast<uint16_t *>(out)[elem] = (uint16_t)f32_to_bf16_bits(x);
    else
        reinterpret_cast<float *>(out)[elem] = x;
}

template <int DK, bool BF16, bool PRO>
__global__ __launch_bounds__(NT) void scan_kernel(ScanParams p) {
    constexpr int E = 8;               // state values per lane
    constexpr int L = DK / E;          // lanes per row
    constexpr int ROWS_MAX = NT / L;
    constexpr int KCH = TB * DK / E;   // 8-element q/k chunks per stage

    __shared__ __align__(16) float kf[TB][DK];
    __shared__ __align__(16) float qf[TB][DK];
    __shared__ float vf[TB][ROWS_MAX];
    __shared__ float of[TB][ROWS_MAX];
    __shared__ float gb[TB], ga[TB], gkq[TB];

    const int nthr = blockDim.x;
    const int rows = nthr / L;
    const int tid = threadIdx.x;
    const int seg = tid % L;           // which 8 of the row's d_k values
    const int rloc = tid / L;          // row within the block
    const int row0 = blockIdx.x * rows;
    const int h = blockIdx.y;
    // grid.z covers (direction, b); the second direction (both_dirs) runs reversed
    // and writes its own fp32 partial.
    const int dir = blockIdx.z >= p.B ? 1 : 0;
    const int b = blockIdx.z - dir * p.B;
    const int reverse = p.reverse ^ dir;
    float *partial = dir ? p.partial_rev : p.partial;
    const int H = p.H;
    const long long T = p.T;
    const int dv = p.dv;

    // q/k chunks this thread stages: chunk c -> token c / L, segment c % L.
    // A block has rows * L >= 16 L = 2 DK threads (d_v >= 16), so at most
    // KCH / (2 DK) = TB / 16 = 2 chunks per thread.
    constexpr int KPT = TB / 16;
    // v chunks: TB * rows / 8 per stage, i.e. TB / (8 L) per thread.
    constexpr int VPT = (TB / E + L - 1) / L;
    const int vch = TB * rows / E;
    const int vpt_tok = rows / E;         // v chunks per token

    // Initial state: this lane's 8 values of row (row0 + rloc).
    float s[E];
    const size_t srow = ((size_t)(b * H + h) * dv + row0 + rloc) * DK + seg * E;
    if (p.state_in) {
        const float4 *sp = reinterpret_cast<const float4 *>(p.state_in + srow);
        const float4 a0 = sp[0], a1 = sp[1];
        s[0] = a0.x; s[1] = a0.y; s[2] = a0.z; s[3] = a0.w;
        s[4] = a1.x; s[5] = a1.y; s[6] = a1.z; s[7] = a1.w;
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = 0.f;
    }

    const long long nst = (T + TB - 1) / TB;
    Chunk8<BF16> kr[KPT], qr[KPT], vr[VPT];
    float br = 0.f, ar = 0.f;

    auto tok_of = [&](long long st, int j) -> long long {
        const long long sidx = st * TB + j;
        return reverse ? T - 1 - sidx : sidx;
    };
    auto issue = [&](long long st) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * nthr;
            if (c < KCH) {
                const int j = c / L;
                if (st * TB + j < T) {
                    const size_t e = (size_t)b * p.qk_bs + (size_t)tok_of(st, j) * p.qk_ts + (size_t)h * DK +
                                     (c % L) * E;
                    kr[i].load(p.k, e);
                    qr[i].load(p.q, e);
                } else {
                    kr[i].zero();
                    qr[i].zero();
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * nthr;
            if (c < vch) {
                const int j = c / vpt_tok;
                const int part = c % vpt_tok;
                if (st * TB + j < T)
                    vr[i].load(p.v, (size_t)b * p.v_bs + (size_t)tok_of(st, j) * p.v_ts + (size_t)h * dv + row0 +
                                        part * E);
                else
                    vr[i].zero();
            }
        }
        if (tid < TB) {
            if (st * TB + tid < T) {
                const size_t g = (size_t)(b * T + tok_of(st, tid)) * H + h;
                br = p.beta[g];
                ar = p.decay[g];
            } else {
                br = 0.f;
                ar = 1.f;
            }
        }
    };
    auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * nthr;
            if (c < KCH) {
                const int j = c / L, sg = c % L;
                float kk[E], qq[E];
                kr[i].to_f32(kk);
                qr[i].to_f32(qq);
                if constexpr (PRO) {  // q / max(||q||, 1e-12), the same for k
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        sk = fmaf(kk[e], kk[e], sk);
                        sq = fmaf(qq[e], qq[e], sq);
                    }
                    const float rk = inv_norm(group_sum<L>(sk)), rq = inv_norm(group_sum<L>(sq));
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        kk[e] *= rk;
                        qq[e] *= rq;
                    }
                }
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    kf[j][sg * E + e] = kk[e];
                    qf[j][sg * E + e] = qq[e];
                    d = fmaf(kk[e], qq[e], d);
                }
                d = group_sum<L>(d);
                if (sg == 0) gkq[j] = d;
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * nthr;
            if (c < vch) {
                const int j = c / vpt_tok;
                const int part = c % vpt_tok;
                float vv[E];
                vr[i].to_f32(vv);
#pragma unroll
                for (int e = 0; e < E; ++e) vf[j][part * E + e] = vv[e];
            }
        }
        if (tid < TB) {
            if constexpr (PRO) {
                gb[tid] = sigmoid_f32(br);
                ga[tid] = decay_from_logit(ar);
            } else {
                gb[tid] = br;
                ga[tid] = ar;
            }
        }
    };

    if (nst > 0) {
        issue(0);
        commit();
        __syncthreads();
    }
    for (long long st = 0; st < nst; ++st) {
        const bool more = st + 1 < nst;
        if (more) issue(st + 1);
        const int nvalid = (int)((T - st * TB) < TB ? (T - st * TB) : TB);
        for (int j = 0; j < nvalid; ++j) {
            const float4 *kp = reinterpret_cast<const float4 *>(&kf[j][seg * E]);
            const float4 *qp = reinterpret_cast<const float4 *>(&qf[j][seg * E]);
            const float4 k0 = kp[0], k1 = kp[1], q0 = qp[0], q1 = qp[1];
            const float kk[E] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
            const float qq[E] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
            float u = 0.f, pq = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                u = fmaf(s[e], kk[e], u);
                pq = fmaf(s[e], qq[e], pq);
            }
            u = group_sum<L>(u);
            pq = group_sum<L>(pq);
            const float a = ga[j], bt = gb[j];
            const float nu = bt * (vf[j][rloc] - a * u);
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] = fmaf(nu, kk[e], a * s[e]);
            if (seg == 0) of[j][rloc] = (a * pq + nu * gkq[j]) * p.scale;
        }
        __syncthreads();
        // Write this stage's outputs: token j, rows [row0, row0 + rows).
        for (int idx = tid; idx < nvalid * rows; idx += nthr) {
            const int j = idx / rows, r = idx % rows;
            const size_t e = ((size_t)(b * T + tok_of(st, j)) * H + h) * dv + row0 + r;
            const float o = of[j][r];
            if (p.out_mode == OUT_PARTIAL) {
                partial[e] = o;
            } else {
                store_out<BF16>(p.out, e, o);
            }
        }
        if (more) commit();
        __syncthreads();
    }

    if (p.state_out) {
        float4 *sp = reinterpret_cast<float4 *>(p.state_out + srow);
        sp[0] = make_float4(s[0], s[1], s[2], s[3]);
        sp[1] = make_float4(s[4], s[5], s[6], s[7]);
    }
}

template <int DK>
hipError_t launch_dk(const PassArgs &a, hipStream_t stream) {
    constexpr int L = DK / 8;
    const int rows = (NT / L) < a.dv ? (NT / L) : a.dv;
    ScanParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.beta = a.beta; p.decay = a.decay;
    p.qk_ts = a.qk_ts; p.qk_bs = a.qk_bs; p.v_ts = a.v_ts; p.v_bs = a.v_bs;
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out;
    p.partial = a.partial; p.partial_rev = a.partial_rev;
    p.T = a.T; p.B = a.B; p.H = a.H; p.dv = a.dv; p.reverse = a.reverse; p.out_mode = a.out_mode;
    p.both_dirs = a.both_dirs;
    p.scale = (float)(1.0 / __builtin_sqrt((double)DK));
    dim3 grid(a.dv / rows, a.H, a.B * (a.both_dirs ? 2 : 1));
    dim3 block(rows * L);
    if (a.io_bf16 && a.prologue)
        hipLaunchKernelGGL((scan_kernel<DK, true, true>), grid, block, 0, stream, p);
    else if (a.io_bf16)
        hipLaunchKernelGGL((scan_kernel<DK, true, false>), grid, block, 0, stream, p);
    else if (a.prologue)
        hipLaunchKernelGGL((scan_kernel<DK, false, true>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((scan_kernel<DK, false, false>), grid, block, 0, stream, p);
    return hipGetLastError();
}

// out = round(partial + partial_rev), 4 elements per thread.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(void *out, const float4 *pa, const float4 *pb, long long n4) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 x = pa[i], y = pb[i];
        const float o0 = x.x + y.x, o1 = x.y + y.y, o2 = x.z + y.z, o3 = x.w + y.w;
        if constexpr (BF16)
            reinterpret_cast<uint2 *>(out)[i] = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        else
            reinterpret_cast<float4 *>(out)[i] = make_float4(o0, o1, o2, o3);
    }
}

}  // namespace

hipError_t launch_scan(const PassArgs &a, hipStream_t stream) {
    switch (a.dk) {
        case 16: return launch_dk<16>(a, stream);
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine(void *out, const float *partial, const float *partial_rev, long long n,
                          int io_bf16, hipStream_t stream) {
    const long long n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    long long nb = (n4 + 255) / 256;
    if (nb > 256 * 64) nb = 256 * 64;
    const float4 *pa = reinterpret_cast<const float4 *>(partial);
    const float4 *pb = reinterpret_cast<const float4 *>(partial_rev);
    if (io_bf16)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)nb), dim3(256), 0, stream, out, pa, pb, n4);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)nb), dim3(256), 0, stream, out, pa, pb, n4);
    return hipGetLastError();
}


}  // namespace gdn
