// gdn_seg.hip -- the combine step of the segment-parallel causal form.
//
// The recurrence S_t = S_{t-1} M_t + b_t v_t k_t^T, M_t = a_t (I - b_t k_t k_t^T), is
// affine in the state, so over a segment of tokens starting from S_start:
//   S_t = S_start P_t + S_t^0,   P_t = M_first ... M_t,
//   o_t = S_t q_t / sqrt(d_k) = S_start w_t + o_t^0,   w_t = P_t q_t / sqrt(d_k),
// where S^0, o^0 are the same segment run from a zero state.  The chunk kernel has
// already produced, per segment s > 0: o^0 (bf16 rows), the segment's own final
// state S^0_end (seg_sloc[s]), and, from a run with v = 0 started at the identity,
// w_t (its bf16 outputs) and P_end (its final state, written transposed: seg_phi[s - 1]).
// Segment 0 ran from
// the caller's state, so its outputs are final and seg_sloc[0] is the true state at
// the end of segment 0.  Here:
//   S_start[1] = seg_sloc[0],  S_start[s+1] = S_start[s] P_end[s] + seg_sloc[s],
//   state_out = S_start[nseg-1] P_end[nseg-1] + seg_sloc[nseg-1],
//   out_t = round(o^0_t + S_start[s] w_t) for every token t of segments s > 0,
// all on bf16 MFMA in one launch (seg_combine_kernel).  Each fp32 state operand is
// split into a bf16 high part and the bf16 rounding of the rest (~2^-16 relative):
// three products per step of the chain, two per correction, whose w is bf16 already.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct SegParams {
    const float *sloc;   // [nseg][B,H,dv,dk]
    const float *phi;    // [nseg-1][B,H,dk,dk], each transition transposed
    float *state_out;    // [B,H,dv,dk] or nullptr
    const uint16_t *w;     // [B,T,H,dk] bf16
    const uint16_t *part;  // [B,T,H,dv] bf16
    uint16_t *out;       // [B,T,H,dv] bf16
    long long T;
    int B, H, dv, nseg, seg_len;
};

__device__ __forceinline__ f32x4_t mfma16k32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t lds16(const uint16_t *p) {
    bf16x8_t r;
    __builtin_memcpy(&r, p, 16);
    return r;
}
__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu); }
// x as a bf16 high part (round to nearest even) and the bf16 rounding of the rest:
// hi + lo carries x to about 2^-16 relative.
__device__ __forceinline__ void split1(float x, uint16_t &hi, uint16_t &lo) {
    hi = bf16_bits(x);
    lo = bf16_bits(x - __uint_as_float((uint32_t)hi << 16));
}
// Eight fp32 values as high and low bf16 operand halves.
__device__ __forceinline__ void split8(const float4 &x0, const float4 &x1, bf16x8_t &hi, bf16x8_t &lo) {
    const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        l[e] = pack_bf16x2(v[2 * e] - bf16_lo(h[e]), v[2 * e + 1] - bf16_hi(h[e]));
    }
    __builtin_memcpy(&hi, h, 16);
    __builtin_memcpy(&lo, l, 16);
}
// a b on bf16 MFMA from split operands: a_hi b_hi + a_hi b_lo + a_lo b_hi.
__device__ __forceinline__ f32x4_t mfma_split(bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl, f32x4_t c) {
    c = mfma16k32(ah, bh, c);
    c = mfma16k32(ah, bl, c);
    return mfma16k32(al, bh, c);
}

// 16x16x32 products: A operand lane (16 g + r) = row r, k 8 g .. 8 g + 7 of a 32-wide
// k step; B operand lane (16 g + r) = column r, the same k; accumulator lane
// (16 g + r) = rows 4 g .. 4 g + 3 of column r.

// One launch, block (b h, y).  Rows y < (nseg - 1) per_seg correct the outputs of a run
// of up to CORR_CHUNKS chunks of segment s = 1 + y / per_seg; the last row (present when
// state_out is asked for) forms state_out.  Each block first forms the state it needs
// by the chain S <- S P_end[s'] + S^0_end[s'] from S^0_end[0] (s - 1 steps for a
// correction block, nseg - 1 for the state block; blocks of one segment repeat the same
// steps rather than wait on each other), then:
//   correction block: O^T (columns x tokens) = S_start W^T for each 16-token group
//     (wave w takes groups w and w + 4) and each 16-column group of d_v; the A operand is
//     the state's rows (high and low part) from LDS, the B operand 16 bytes of the lane's
//     token row of W straight from memory; the accumulator lane (16 g + r) holds columns
//     4 g .. 4 g + 3 of token r: out = round(o^0 + O), one 8-byte load and one 8-byte
//     store.
//   state block: writes the chain's final state, fp32, to state_out.
constexpr int CORR_CHUNKS = 2;  // runs of 1 or 4 chunks measured 1-8% slower on the short workloads

template <int DK, int DV>
struct CombSmem {
    static constexpr int P = DK + 8;
    uint16_t sh[DV][P], sl[DV][P];  // the state's rows, split bf16 (A operand)
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_combine_kernel(SegParams p) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    CombSmem<DK, DV> &sm = *reinterpret_cast<CombSmem<DK, DV> *>(lds_raw);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int head = blockIdx.x;  // b * H + h
    const int b = head / p.H, h = head % p.H;
    const int per_seg = (p.seg_len + CORR_CHUNKS - 1) / CORR_CHUNKS;
    const int ncorr = (p.nseg - 1) * per_seg;
    const bool state_blk = (int)blockIdx.y >= ncorr;
    const int seg = state_blk ? p.nseg : 1 + (int)blockIdx.y / per_seg;
    const long long n = (p.T + 63) / 64;
    long long c_begin = 0, c_end = 0;
    if (!state_blk) {
        c_begin = (long long)seg * p.seg_len + CORR_CHUNKS * ((int)blockIdx.y % per_seg);
        c_end = c_begin + CORR_CHUNKS;
        if (c_end > (long long)(seg + 1) * p.seg_len) c_end = (long long)(seg + 1) * p.seg_len;
        if (c_end > n) c_end = n;
        if (c_begin >= c_end) return;  // past the last chunk: the whole block leaves
    }
    constexpr int NKS = DK / 32;
    const size_t sstride = (size_t)p.B * p.H * DV * DK;
    const size_t pstride = (size_t)p.B * p.H * DK * DK;

    // the chain over segments 1 .. seg - 1; wave w owns the 16x16 tiles i = w + 4 j of
    // the d_v x d_k state.  The identity runs wrote each transition transposed, so the
    // B operand (column j of the transition, 8 consecutive k) is a row segment of it,
    // loaded straight into registers.  The tiles are taken one column group of the
    // transition at a time, and each group's columns are loaded while the previous
    // group's products run, so that one group's operands are live.  Each step's
    // S^0_end tiles are loaded into the accumulators, which the products add to; with
    // at most 4 tiles per wave, where registers allow, they are loaded a step ahead.
    constexpr int NCG = DK / 16;                 // column groups of the state
    constexpr int NTW = (DV / 16) * NCG / 4;     // tiles per wave
    constexpr int NCW = NCG > 4 ? NCG / 4 : 1;   // distinct column groups per wave: (w + 4 jj) % NCG
    f32x4_t acc[NTW];
    float4 v[2 * NKS];
    auto load_phi = [&](int s1, int jj) {  // column group (w + 4 jj) % NCG of step s1's transition
        const float *row = p.phi + (s1 - 1) * pstride + (size_t)head * DK * DK +
                           (size_t)(16 * ((wid + 4 * jj) % NCG) + r16) * DK + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            v[2 * ks] = *reinterpret_cast<const float4 *>(row + 32 * ks);
            v[2 * ks + 1] = *reinterpret_cast<const float4 *>(row + 32 * ks + 4);
        }
    };
    auto load_tiles = [&](int s1, f32x4_t (&dst)[NTW]) {  // dst = this wave's tiles of S^0_end[s1]
        const float *src = p.sloc + s1 * sstride + (size_t)head * DV * DK;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int i = wid + 4 * j, rg = i / NCG, cg = i % NCG;
#pragma unroll
            for (int m = 0; m < 4; ++m) dst[j][m] = src[(size_t)(16 * rg + 4 * g4 + m) * DK + 16 * cg + r16];
        }
    };
    constexpr bool AHEAD = NTW <= 4;
    f32x4_t nxt[AHEAD ? NTW : 1];
    if (seg > 1) {
        load_phi(1, 0);
        load_tiles(1, acc);
        if constexpr (AHEAD)
            if (seg > 2) load_tiles(2, nxt);
    }
    // S^0_end[0], the true state at the end of segment 0, split into LDS
    {
        const float *src = p.sloc + (size_t)head * DV * DK;
        constexpr int NST = (DV * DK / 8 + 255) / 256;  // 8-value runs per thread
        constexpr int BATCH = NST < 4 ? NST : 4;          // of which this many are in flight
#pragma unroll
        for (int i0 = 0; i0 < NST; i0 += BATCH) {
            float4 sv[2 * BATCH];
#pragma unroll
            for (int it = 0; it < BATCH; ++it) {
                const int i = threadIdx.x + 256 * (i0 + it);
                if (i < DV * DK / 8) {
                    sv[2 * it] = *reinterpret_cast<const float4 *>(src + 8 * (size_t)i);
                    sv[2 * it + 1] = *reinterpret_cast<const float4 *>(src + 8 * (size_t)i + 4);
                }
            }
#pragma unroll
            for (int it = 0; it < BATCH; ++it) {
                const int i = threadIdx.x + 256 * (i0 + it);
                if (i < DV * DK / 8) {
                    const int c = (8 * i) / DK, k0 = (8 * i) % DK;
                    bf16x8_t h8, l8;
                    split8(sv[2 * it], sv[2 * it + 1], h8, l8);
                    *reinterpret_cast<bf16x8_t *>(&sm.sh[c][k0]) = h8;
                    *reinterpret_cast<bf16x8_t *>(&sm.sl[c][k0]) = l8;
                }
            }
        }
    }

    for (int s1 = 1; s1 < seg; ++s1) {
        __syncthreads();  // the state is staged
#pragma unroll
        for (int jj = 0; jj < NCW; ++jj) {
            bf16x8_t bh[NKS], bl[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) split8(v[2 * ks], v[2 * ks + 1], bh[ks], bl[ks]);
            if (jj + 1 < NCW) load_phi(s1, jj + 1);
            else if (s1 + 1 < seg) load_phi(s1 + 1, 0);
#pragma unroll
            for (int j = jj; j < NTW; j += NCW) {
                const int rg = (wid + 4 * j) / NCG;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int k0 = 32 * ks + 8 * g4;
                    acc[j] = mfma_split(lds16(&sm.sh[16 * rg + r16][k0]), lds16(&sm.sl[16 * rg + r16][k0]), bh[ks],
                                        bl[ks], acc[j]);
                }
            }
        }
        __syncthreads();  // every read of the staged state is done
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int i = wid + 4 * j, rg = i / NCG, cg = i % NCG;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                uint16_t hh, ll;
                split1(acc[j][m], hh, ll);
                sm.sh[16 * rg + 4 * g4 + m][16 * cg + r16] = hh;
                sm.sl[16 * rg + 4 * g4 + m][16 * cg + r16] = ll;
            }
        }
        if (s1 + 1 < seg) {
            if constexpr (AHEAD) {
#pragma unroll
                for (int j = 0; j < NTW; ++j) acc[j] = nxt[j];
                if (s1 + 2 < seg) load_tiles(s1 + 2, nxt);
            } else {
                load_tiles(s1 + 1, acc);
            }
        }
    }
    if (state_blk) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int i = wid + 4 * j, rg = i / NCG, cg = i % NCG;
#pragma unroll
            for (int m = 0; m < 4; ++m)
                p.state_out[((size_t)head * DV + 16 * rg + 4 * g4 + m) * DK + 16 * cg + r16] = acc[j][m];
        }
        return;
    }
    __syncthreads();  // the segment's start state is staged

    const long long t_begin = 64 * c_begin;
    const long long t_end = 64 * c_end < p.T ? 64 * c_end : p.T;
    const int ngroups = (int)((t_end - t_begin + 15) / 16);
    constexpr int NVG = DV / 16;  // column groups of out
    auto load = [&](int grp, bf16x8_t (&w)[NKS], uint2 (&z)[NVG]) {
        long long t = t_begin + 16 * grp + r16;
        if (t >= p.T) t = p.T - 1;  // loads stay in bounds; stores only below t_end
        const uint16_t *row = p.w + (((size_t)b * p.T + t) * p.H + h) * DK + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) w[ks] = *reinterpret_cast<const bf16x8_t *>(row + 32 * ks);
        const uint16_t *zr = p.part + (((size_t)b * p.T + t) * p.H + h) * DV + 4 * g4;
#pragma unroll
        for (int cg = 0; cg < NVG; ++cg) z[cg] = *reinterpret_cast<const uint2 *>(zr + 16 * cg);
    };
    // wave w corrects token groups w and w + 4 together: each A operand read from LDS
    // serves both groups' products, and no operand is held across groups
    static_assert(CORR_CHUNKS == 2, "the groups of a correction block are two per wave");
    if (wid >= ngroups) return;
    bf16x8_t w0[NKS], w1[NKS];
    uint2 z0[NVG], z1[NVG];
    load(wid, w0, z0);
    load(wid + 4, w1, z1);  // clamped rows when past the end: products unused
    const long long t0 = t_begin + 16 * wid + r16, t1 = t0 + 64;
    uint16_t *orow0 = p.out + (((size_t)b * p.T + (t0 < p.T ? t0 : p.T - 1)) * p.H + h) * DV + 4 * g4;
    uint16_t *orow1 = p.out + (((size_t)b * p.T + (t1 < p.T ? t1 : p.T - 1)) * p.H + h) * DV + 4 * g4;
#pragma unroll
    for (int cg = 0; cg < NVG; ++cg) {
        f32x4_t d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int k0 = 32 * ks + 8 * g4;
            const bf16x8_t ah = lds16(&sm.sh[16 * cg + r16][k0]), al = lds16(&sm.sl[16 * cg + r16][k0]);
            d0 = mfma16k32(ah, w0[ks], d0);
            d1 = mfma16k32(ah, w1[ks], d1);
            d0 = mfma16k32(al, w0[ks], d0);
            d1 = mfma16k32(al, w1[ks], d1);
        }
        if (t0 < t_end)
            *reinterpret_cast<uint2 *>(orow0 + 16 * cg) =
                make_uint2(pack_bf16x2(bf16_lo(z0[cg].x) + d0[0], bf16_hi(z0[cg].x) + d0[1]),
                           pack_bf16x2(bf16_lo(z0[cg].y) + d0[2], bf16_hi(z0[cg].y) + d0[3]));
        if (t1 < t_end)
            *reinterpret_cast<uint2 *>(orow1 + 16 * cg) =
                make_uint2(pack_bf16x2(bf16_lo(z1[cg].x) + d1[0], bf16_hi(z1[cg].x) + d1[1]),
                           pack_bf16x2(bf16_lo(z1[cg].y) + d1[2], bf16_hi(z1[cg].y) + d1[3]));
    }
}

template <int DK, int DV>
hipError_t launch_seg_dv(const PassArgs &a, hipStream_t stream) {
    SegParams p;
    p.sloc = a.seg_sloc;
    p.phi = a.seg_phi;
    p.state_out = a.state_out;
    p.w = static_cast<const uint16_t *>(a.seg_w);
    p.part = static_cast<const uint16_t *>(a.seg_partial);
    p.out = static_cast<uint16_t *>(a.out);
    p.T = a.T;
    p.B = a.B; p.H = a.H; p.dv = DV; p.nseg = a.nseg; p.seg_len = a.seg_len;
    const int per_seg = (a.seg_len + CORR_CHUNKS - 1) / CORR_CHUNKS;
    const long long ny = (long long)(a.nseg - 1) * per_seg + (a.state_out ? 1 : 0);
    if (ny <= 0 || ny > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL((seg_combine_kernel<DK, DV>), dim3(a.B * a.H, (unsigned)ny), dim3(256),
                       sizeof(CombSmem<DK, DV>), stream, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_seg_dk(const PassArgs &a, hipStream_t stream) {
    switch (a.dv) {
        case 32: return launch_seg_dv<DK, 32>(a, stream);
        case 64: return launch_seg_dv<DK, 64>(a, stream);
        case 128: return launch_seg_dv<DK, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_seg_combine(const PassArgs &a, hipStream_t stream) {
    if (a.nseg < 2 || a.seg_len < 1 || a.io == IO_F32) return hipErrorInvalidValue;
    switch (a.dk) {
        case 32: return launch_seg_dk<32>(a, stream);
        case 64: return launch_seg_dk<64>(a, stream);
        case 128: return launch_seg_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
