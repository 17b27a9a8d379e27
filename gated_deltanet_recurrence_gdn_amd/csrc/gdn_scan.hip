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

constexpr int TB = 48;       // tokens per LDS stage (32: +1% at the batched d = 128 shape)
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

template <int IO>
struct Chunk8;  // 8 consecutive input elements held in registers

template <>
struct Chunk8<IO_BF16> {
    uint4 w;
    __device__ void load(const void *base, size_t elem) {
        w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + elem);
    }
    __device__ void to_f32(float f[8]) const {
        f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
        f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
    }
};

template <>
struct Chunk8<IO_FP8> {
    uint2 w;
    __device__ void load(const void *base, size_t elem) {
        w = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(base) + elem);
    }
    __device__ void to_f32(float f[8]) const {
        fp8x4_to_f32(w.x, f);
        fp8x4_to_f32(w.y, f + 4);
    }
};

template <>
struct Chunk8<IO_F32> {
    float4 a, b;
    __device__ void load(const void *base, size_t elem) {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + elem);
        a = p[0];
        b = p[1];
    }
    __device__ void to_f32(float f[8]) const {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

// u and p each summed over the 16 lanes of a DPP row in one shared chain: after
// the first exchange the even lanes hold partial sums of u and the odd lanes
// partial sums of p, and rotations of the row by 2, 4 and 8 finish each parity
// class in every lane.  Returns u in every lane; p is left in the odd lanes.
// The decay products as = a s of the lane's 8 state values, which need nothing
// from the sums, are issued two after each dependent DPP step: they fill the wait
// states that a DPP read of the previous step's result needs (the scheduling
// barriers keep them there), 7.01 -> 6.67 ms at the batched d = 128 shape.
__device__ __forceinline__ float row16_sum2(float u, float &p, bool odd, float a, const float (&s)[8],
                                            float (&as)[8]) {
    // The wave runs at a raised priority from here until its output is stored: the
    // row sums, nu and the update are one dependent chain, and the other wave on
    // the SIMD (in its dot products) then yields the issue slots to it
    // (6.67 -> 6.12 ms at the batched d = 128 shape).
    __builtin_amdgcn_s_setprio(2);
    float t = odd ? p : u;
    const float o = odd ? u : p;
    t += dpp_mov<0xB1>(o);   // quad_perm [1,0,3,2]: the pair's other lane
    as[0] = a * s[0];
    as[1] = a * s[1];
    __builtin_amdgcn_sched_barrier(0);
    t += dpp_mov<0x122>(t);  // row_ror:2
    as[2] = a * s[2];
    as[3] = a * s[3];
    __builtin_amdgcn_sched_barrier(0);
    t += dpp_mov<0x124>(t);  // row_ror:4
    as[4] = a * s[4];
    as[5] = a * s[5];
    __builtin_amdgcn_sched_barrier(0);
    t += dpp_mov<0x128>(t);  // row_ror:8
    as[6] = a * s[6];
    as[7] = a * s[7];
    __builtin_amdgcn_sched_barrier(0);
    p = t;
    return dpp_mov<0xA0>(t);  // quad_perm [0,0,2,2]: the even lane's sum
}

// Eight consecutive outputs (elem a multiple of 8): one 16-byte store of bf16, or two of fp32.
template <int IO>
__device__ __forceinline__ void store_out8(void *out, size_t elem, const float4 &a, const float4 &b) {
    if constexpr (IO != IO_F32) {
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out) + elem) =
            make_uint4(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w));
    } else {
        float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + elem);
        o[0] = a;
        o[1] = b;
    }
}

// A block holds `rows` consecutive state rows of one (b, h).  A row's d_k values
// live in the VGPRs of L = DK / E lanes: lane `seg` of the row holds d_k indices
// 4 (seg + L i) + m (i < E / 4, m < 4), so the row's lanes read one contiguous
// run of LDS per float4 and every row reads the same addresses (a broadcast).
template <int DK, int E, int IO, bool PRO>
__global__ __launch_bounds__(NT) void scan_kernel(ScanParams p) {
    constexpr int L = DK / E;            // lanes per state row
    constexpr int V4 = E / 4;            // float4 of k (and of q) per lane and token
    constexpr int ROWS_MAX = NT / L;
    constexpr int SL = DK / 8;           // staging: lanes per q/k row, 8 elements each
    constexpr int KCH = TB * SL;         // 8-element q/k chunks per stage
    // a block has rows * L >= 16 L threads (d_v >= 16)
    constexpr int KPT = (KCH + 16 * L - 1) / (16 * L);
    constexpr int VPT = (TB / 8 + L - 1) / L;
    // gate loads per thread: a block can have as few as 16 threads (L = 1, d_v = 16)
    constexpr int GPT = (TB + 16 * L - 1) / (16 * L);

    __shared__ __align__(16) float kf[TB][DK];
    __shared__ __align__(16) float qf[TB][DK];
    __shared__ __align__(16) float vf[TB][ROWS_MAX];
    __shared__ __align__(16) float of[TB][ROWS_MAX];
    __shared__ float odump[NT];  // the output writes of the lanes that do not own o
    __shared__ __align__(16) float gt[TB][4];  // a, b, (k . q) / sqrt(d_k) per token

    const int nthr = blockDim.x;
    const int rows = nthr / L;
    const int tid = threadIdx.x;
    const int seg = tid % L;           // which E of the row's d_k values
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
    const int vch = TB * rows / 8;     // 8-element v (and output) chunks per stage
    const int vpt_tok = rows / 8;      // v chunks per token: a power of two (rows is)
    const int lg_vpt = __builtin_ctz((unsigned)vpt_tok);

    // Initial state: this lane's E values of row (row0 + rloc).
    float s[E];
    const size_t srow = ((size_t)(b * H + h) * dv + row0 + rloc) * DK;
#pragma unroll
    for (int i = 0; i < V4; ++i) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.state_in) x = *reinterpret_cast<const float4 *>(p.state_in + srow + 4 * (seg + L * i));
        s[4 * i] = x.x; s[4 * i + 1] = x.y; s[4 * i + 2] = x.z; s[4 * i + 3] = x.w;
    }
    // Wait for the state here, once: the compiler cannot tell through the loops
    // below that this conditional load has landed, and would otherwise wait for
    // every load in flight (the next stage's prefetch) before each stage's tokens.
    __builtin_amdgcn_s_waitcnt(0);

    const long long nst = (T + TB - 1) / TB;
    Chunk8<IO> kr[KPT], qr[KPT], vr[VPT];
    float br[GPT], ar[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        br[i] = 0.f;
        ar[i] = 1.f;
    }

    // Token at walk position sidx, clamped to the last one: the loads are
    // unconditional (past the end they re-read a real token), and commit()
    // turns padding into exact no-ops.
    auto tok_of = [&](long long sidx) -> long long {
        const long long c = sidx < T ? sidx : T - 1;
        return reverse ? T - 1 - c : c;
    };
    auto issue = [&](long long st) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * nthr;
            if (c < KCH) {
                const size_t e = (size_t)b * p.qk_bs + (size_t)tok_of(st * TB + c / SL) * p.qk_ts +
                                 (size_t)h * DK + (c % SL) * 8;
                kr[i].load(p.k, e);
                qr[i].load(p.q, e);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * nthr;
            if (c < vch)
                vr[i].load(p.v, (size_t)b * p.v_bs + (size_t)tok_of(st * TB + (c >> lg_vpt)) * p.v_ts +
                                    (size_t)h * dv + row0 + (c & (vpt_tok - 1)) * 8);
        }
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int j = tid + i * nthr;
            if (j < TB) {
                const size_t g = (size_t)(b * T + tok_of(st * TB + j)) * H + h;
                br[i] = p.beta[g];
                ar[i] = p.decay[g];
            }
        }
    };
    // Registers -> LDS in fp32.  Tokens past T become b = 0, a = 1, q = k = v = 0:
    // then u = 0, nu = 0 and S is left exactly as it was.
    auto commit = [&](long long st) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * nthr;
            if (c < KCH) {
                const int j = c / SL, sg = c % SL;
                const bool real = st * TB + j < T;
                float kk[8], qq[8];
                kr[i].to_f32(kk);
                qr[i].to_f32(qq);
                if (!real) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kk[e] = qq[e] = 0.f;
                }
                if constexpr (PRO) {  // q / max(||q||, 1e-12), the same for k
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        sk = fmaf(kk[e], kk[e], sk);
                        sq = fmaf(qq[e], qq[e], sq);
                    }
                    const float rk = inv_norm(group_sum<SL>(sk)), rq = inv_norm(group_sum<SL>(sq));
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        kk[e] *= rk;
                        qq[e] *= rq;
                    }
                }
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(kk[e], qq[e], d);
                d = group_sum<SL>(d) * p.scale;
#pragma unroll
                for (int e = 0; e < 8; ++e) qq[e] *= p.scale;  // o = S q / sqrt(d_k): the scale rides on q
                *reinterpret_cast<float4 *>(&kf[j][sg * 8]) = make_float4(kk[0], kk[1], kk[2], kk[3]);
                *reinterpret_cast<float4 *>(&kf[j][sg * 8 + 4]) = make_float4(kk[4], kk[5], kk[6], kk[7]);
                *reinterpret_cast<float4 *>(&qf[j][sg * 8]) = make_float4(qq[0], qq[1], qq[2], qq[3]);
                *reinterpret_cast<float4 *>(&qf[j][sg * 8 + 4]) = make_float4(qq[4], qq[5], qq[6], qq[7]);
                if (sg == 0) gt[j][2] = d;
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * nthr;
            if (c < vch) {
                const int j = c >> lg_vpt, part = c & (vpt_tok - 1);
                const bool real = st * TB + j < T;
                float vv[8];
                vr[i].to_f32(vv);
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[e] = real ? vv[e] : 0.f;
                *reinterpret_cast<float4 *>(&vf[j][part * 8]) = make_float4(vv[0], vv[1], vv[2], vv[3]);
                *reinterpret_cast<float4 *>(&vf[j][part * 8 + 4]) = make_float4(vv[4], vv[5], vv[6], vv[7]);
            }
        }
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int j = tid + i * nthr;
            if (j < TB) {
                const bool real = st * TB + j < T;
                float bb = br[i], aa = ar[i];
                if constexpr (PRO) {
                    bb = sigmoid_f32(br[i]);
                    aa = decay_from_logit(ar[i]);
                }
                gt[j][0] = real ? aa : 1.f;
                gt[j][1] = real ? bb : 0.f;
            }
        }
    };

    // One token, with its operands already in registers.
    struct Tok {
        float4 k[V4], q[V4];
        float4 g;  // a, b, (k . q) / sqrt(d_k)
        float v;
    };
    auto ld_tok = [&](int j, Tok &t) {
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            t.k[i] = *reinterpret_cast<const float4 *>(&kf[j][4 * (seg + L * i)]);
            t.q[i] = *reinterpret_cast<const float4 *>(&qf[j][4 * (seg + L * i)]);
        }
        t.g = *reinterpret_cast<const float4 *>(&gt[j][0]);
        t.v = vf[j][rloc];
    };
    const bool odd = (tid & 1) != 0;
    auto step = [&](int j, const Tok &t) {
        // u = S_i . k and p = S_i . q (q carries 1/sqrt(d_k))
        float u, pq;
        float as_[E];  // a S_i, the decayed state
        if constexpr (L == 16) {
            u = 0.f;
            pq = 0.f;
#pragma unroll
            for (int i = 0; i < V4; ++i) {
                const float kk[4] = {t.k[i].x, t.k[i].y, t.k[i].z, t.k[i].w};
                const float qq[4] = {t.q[i].x, t.q[i].y, t.q[i].z, t.q[i].w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    u = fmaf(s[4 * i + m], kk[m], u);
                    pq = fmaf(s[4 * i + m], qq[m], pq);
                }
            }
            u = row16_sum2(u, pq, odd, t.g.x, s, as_);  // pq now on the odd lanes
        } else {
            // two partial sums each (four independent chains)
            float u0 = 0.f, u1 = 0.f, p0 = 0.f, p1 = 0.f;
#pragma unroll
            for (int i = 0; i < V4; ++i) {
                const float kk[4] = {t.k[i].x, t.k[i].y, t.k[i].z, t.k[i].w};
                const float qq[4] = {t.q[i].x, t.q[i].y, t.q[i].z, t.q[i].w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    if (m & 1) {
                        u1 = fmaf(s[4 * i + m], kk[m], u1);
                        p1 = fmaf(s[4 * i + m], qq[m], p1);
                    } else {
                        u0 = fmaf(s[4 * i + m], kk[m], u0);
                        p0 = fmaf(s[4 * i + m], qq[m], p0);
                    }
                }
            }
            // the decay products first (they need nothing from the sums), then the
            // sums at a raised priority, as in the 16-lane path (-2% on the bidirectional
            // scan at the batched d = 128 shape, which takes 16 values per lane)
#pragma unroll
            for (int i = 0; i < E; ++i) as_[i] = t.g.x * s[i];
            __builtin_amdgcn_s_setprio(2);
            u = group_sum<L>(u0 + u1);
            pq = group_sum<L>(p0 + p1);
        }
        const float a = t.g.x, bt = t.g.y, kq = t.g.z;
        const float nu = bt * (t.v - a * u);
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            s[4 * i] = fmaf(nu, t.k[i].x, as_[4 * i]);
            s[4 * i + 1] = fmaf(nu, t.k[i].y, as_[4 * i + 1]);
            s[4 * i + 2] = fmaf(nu, t.k[i].z, as_[4 * i + 2]);
            s[4 * i + 3] = fmaf(nu, t.k[i].w, as_[4 * i + 3]);
        }
        // one lane of the row owns o (q and k . q carry 1/sqrt(d_k)); every lane
        // stores, the others into odump, so that no per-token exec mask is set up
        // and restored around the store (7.01 -> 6.91 ms at the batched d = 128 shape)
        {
            float *dst = seg == (L == 16 ? 1 : 0) ? &of[j][rloc] : &odump[tid];
            *dst = fmaf(a, pq, nu * kq);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    if (nst > 0) {
        issue(0);
        commit(0);
        __syncthreads();
    }
    for (long long st = 0; st < nst; ++st) {
        const bool more = st + 1 < nst;
        if (more) issue(st + 1);
        // every stage runs all TB tokens (padding is a no-op); token j + 2's operands
        // are read from LDS while token j is computed, from three rotating register
        // sets (the reads past the last token wrap to the start of the same stage and
        // are not used; one token ahead instead: +2%).  Fully unrolled, every LDS
        // address is a constant offset from one base: no per-token address arithmetic
        // and no loop branch (7.88 -> 7.02 ms at the batched d = 128 shape).
        Tok tk[3];
        ld_tok(0, tk[0]);
        ld_tok(1, tk[1]);
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            ld_tok((j + 2) % TB, tk[(j + 2) % 3]);
            step(j, tk[j % 3]);
        }
        __syncthreads();
        // Write this stage's outputs: token j, rows [row0, row0 + rows), eight rows
        // per thread in one 16-byte store (one 2-byte store per row before, and
        // scalar LDS stores of v: 5.98 -> 5.70 ms at the batched d = 128 shape).
        const int nvalid = (int)((T - st * TB) < TB ? (T - st * TB) : TB);
        for (int c = tid; c < nvalid * vpt_tok; c += nthr) {
            const int j = c >> lg_vpt, part = c & (vpt_tok - 1);
            const size_t e = ((size_t)(b * T + tok_of(st * TB + j)) * H + h) * dv + row0 + part * 8;
            const float4 o0 = *reinterpret_cast<const float4 *>(&of[j][part * 8]);
            const float4 o1 = *reinterpret_cast<const float4 *>(&of[j][part * 8 + 4]);
            if (p.out_mode == OUT_PARTIAL) {
                reinterpret_cast<float4 *>(partial + e)[0] = o0;
                reinterpret_cast<float4 *>(partial + e)[1] = o1;
            } else {
                store_out8<IO>(p.out, e, o0, o1);
            }
        }
        if (more) commit(st + 1);
        __syncthreads();
    }

    if (p.state_out) {
#pragma unroll
        for (int i = 0; i < V4; ++i)
            *reinterpret_cast<float4 *>(p.state_out + srow + 4 * (seg + L * i)) =
                make_float4(s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
    }
}

template <int DK, int E, int IO, bool PRO>
hipError_t launch_e(const PassArgs &a, const ScanParams &p, hipStream_t stream) {
    constexpr int L = DK / E;
    const int rows = (NT / L) < a.dv ? (NT / L) : a.dv;
    dim3 grid(a.dv / rows, a.H, a.B * (a.both_dirs ? 2 : 1));
    hipLaunchKernelGGL((scan_kernel<DK, E, IO, PRO>), grid, dim3(rows * L), 0, stream, p);
    return hipGetLastError();
}

template <int DK, int E, int IO>
hipError_t launch_dk_io(const PassArgs &a, const ScanParams &p, hipStream_t stream) {
    return a.prologue ? launch_e<DK, E, IO, true>(a, p, stream) : launch_e<DK, E, IO, false>(a, p, stream);
}

template <int DK, int E>
hipError_t launch_dk_e(const PassArgs &a, const ScanParams &p, hipStream_t stream) {
    switch (a.io) {
        case IO_BF16: return launch_dk_io<DK, E, IO_BF16>(a, p, stream);
        case IO_FP8: return launch_dk_io<DK, E, IO_FP8>(a, p, stream);
        default: return launch_dk_io<DK, E, IO_F32>(a, p, stream);
    }
}

// E = 8 state values per lane unless that puts more than two waves on a SIMD (256
// CUs x 4): the second wave hides the latency of each token's dependent chain (dot
// products, cross-lane sums, nu, update), which one wave alone leaves exposed.
// With more work than that, E = 16 halves the cross-lane sums per state value.
template <int DK>
hipError_t launch_dk(const PassArgs &a, hipStream_t stream) {
    ScanParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.beta = a.beta; p.decay = a.decay;
    p.qk_ts = a.qk_ts; p.qk_bs = a.qk_bs; p.v_ts = a.v_ts; p.v_bs = a.v_bs;
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out;
    p.partial = a.partial; p.partial_rev = a.partial_rev;
    p.T = a.T; p.B = a.B; p.H = a.H; p.dv = a.dv; p.reverse = a.reverse; p.out_mode = a.out_mode;
    p.both_dirs = a.both_dirs;
    p.scale = (float)(1.0 / __builtin_sqrt((double)DK));
    const long long waves8 = (long long)a.B * a.H * (a.both_dirs ? 2 : 1) * a.dv * (DK / 8) / 64;
    if (waves8 > 2048) return launch_dk_e<DK, 16>(a, p, stream);
    return launch_dk_e<DK, 8>(a, p, stream);
}

typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// out = round(partial + partial_rev), 4 elements per thread.  Every byte is read
// or written once, so the loads and stores are non-temporal (no cache
// allocation for data that is not used again): 3% of the bidirectional call.
template <bool BF16>
__global__ __launch_bounds__(256) void combine_kernel(void *out, const float4 *pa, const float4 *pb, long long n4) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    const f32x4v_t *va = reinterpret_cast<const f32x4v_t *>(pa);
    const f32x4v_t *vb = reinterpret_cast<const f32x4v_t *>(pb);
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const f32x4v_t x = __builtin_nontemporal_load(va + i), y = __builtin_nontemporal_load(vb + i);
        const f32x4v_t o = x + y;
        if constexpr (BF16) {
            const u32x2v_t w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2v_t *>(out) + i);
        } else {
            __builtin_nontemporal_store(o, reinterpret_cast<f32x4v_t *>(out) + i);
        }
    }
}

// The bidirectional MFMA split's middle rows: out = round(a + b) over the token rows
// [t0, t1) of each batch element, a and b bf16 rows of the two directions (4 values
// per thread).
__global__ __launch_bounds__(256) void combine_rows_kernel(uint16_t *out, const uint2 *pa, const uint2 *pb, int B,
                                                           long long T, long long row4, long long t0, long long t1) {
    const long long per_b = (t1 - t0) * row4;
    const long long n4 = per_b * B;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x; j < n4; j += stride) {
        const long long b = j / per_b;
        const long long i = (b * T + t0) * row4 + (j - b * per_b);
        const uint2 x = pa[i], y = pb[i];
        reinterpret_cast<uint2 *>(out)[i] = make_uint2(pack_bf16x2(bf16_lo(x.x) + bf16_lo(y.x), bf16_hi(x.x) + bf16_hi(y.x)),
                                                       pack_bf16x2(bf16_lo(x.y) + bf16_lo(y.y), bf16_hi(x.y) + bf16_hi(y.y)));
    }
}

}  // namespace

hipError_t launch_combine_rows_bf16(uint16_t *out, const uint16_t *partial, const uint16_t *partial_rev, int B,
                                    long long T, long long row, long long t0, long long t1, hipStream_t stream) {
    if (t1 <= t0 || row % 4) return t1 <= t0 ? hipSuccess : hipErrorInvalidValue;
    const long long n4 = (long long)B * (t1 - t0) * (row / 4);
    long long nb = (n4 + 255) / 256;
    if (nb > 256 * 64) nb = 256 * 64;
    hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)nb), dim3(256), 0, stream, out,
                       reinterpret_cast<const uint2 *>(partial), reinterpret_cast<const uint2 *>(partial_rev), B, T,
                       row / 4, t0, t1);
    return hipGetLastError();
}

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
                          int io, hipStream_t stream) {
    const long long n4 = n / 4;
    if (n4 == 0) return hipSuccess;
    long long nb = (n4 + 255) / 256;
    if (nb > 256 * 64) nb = 256 * 64;
    const float4 *pa = reinterpret_cast<const float4 *>(partial);
    const float4 *pb = reinterpret_cast<const float4 *>(partial_rev);
    if (io != IO_F32)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)nb), dim3(256), 0, stream, out, pa, pb, n4);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)nb), dim3(256), 0, stream, out, pa, pb, n4);
    return hipGetLastError();
}


}  // namespace gdn
