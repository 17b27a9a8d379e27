// gdn_chunk.hip -- chunked (UT-transform) form of the GDN recurrence on bf16 MFMA.
//
// Within a chunk of C tokens starting from state S0 (d_v x d_k), with
// g_i = sum_{r<=i} log2 a_r, gam_i = 2^{g_i}, G_ij = 2^{g_i - g_j} (j <= i):
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
// sglang SANA-WM record names its Triton kernel cam_scan_bidi_chunkwise).  Every
// C x C and C x d product runs on MFMA (bf16 operands, fp32 accumulation).
//
// Parallel decomposition.  Rows of S are independent, so a block owns one
// (b, h) and a 32-wide tile of d_v and walks the head's chunks in order.  The
// S-independent per-chunk work (decay factors, Gram products, the triangular
// inverse) is recomputed by each d_v tile of a head: that costs MFMA time, not
// HBM traffic, because the tiles of a head are placed on one XCD and share q/k
// through its L2, and it buys the CU count the sequential chunk chain needs.
//
// Roles.  Eight waves; waves w and w + 4 share a SIMD, and the pairs are chosen
// to even out the SIMDs' work.  One workgroup barrier per chunk period.  In
// period c:
//   wave 0     the state chain of chunk c, alone on its SIMD.  S^T (d_k x 32)
//              lives in fp32 MFMA accumulators for the whole call; X = K S^T,
//              R, N = Tm R and the update S^T = gam_{C-1} S^T + K^T N~ hand their
//              results from one product to the next in registers: a 32x32
//              accumulator becomes the next product's bf16 operand with one
//              v_permlane32_swap per two rows (the 32x32x16 A and B operands
//              share one lane layout), so the chain has no barrier and no LDS
//              round trip of its own.  It publishes bf16 copies of S (for the
//              next period's outputs) and of N (behind an LDS flag, for this
//              period's outputs).
//   waves 6, 3 outputs of chunk c, one 32-token half each: P of the half's query
//              rows in registers (formed while the chain works on N), then
//              O^T = gam .* (S Q^T) + N^T P^T, written as 8-byte row segments.
//   waves 1, 2, 5  chunk c+1: K rows 0-31, K rows 32-63 and Q rows 0-31
//              (HBM -> registers -> LDS); the diagonal 32x32 blocks of A and their
//              16x16 diagonal Tm blocks (fp32 substitution in registers) from the
//              K waves' own rows, the off-diagonal block A(1,0), and the other Tm
//              blocks by 16x16x16 MFMA, with LDS counters as their only syncs.
//   wave 4     Q rows 32-63 of chunk c+1 into LDS (memory operations only,
//              beside the chain).
//   wave 7     gate vectors of chunk c+2: float64 prefix sum of log2 a (DPP
//              within 16-lane rows, then the row carries), 2^g, b 2^g,
//              2^{g_last - g}, b, and the factors of the off-diagonal 32x32
//              block; b_t v_t of chunk c+1 (fp32, d_v-major) for R.
// Global loads run two periods ahead (K/Q/V of chunk c+3, gates of c+4, in
// alternating register sets), so their latency hides behind two periods; a
// register set is refilled right after it has been stored to LDS, and no
// product reads it, so no wait on an in-flight load lands inside a period.
//
// Decay numerics: log2 a is accumulated in float64 (log2 a is clamped at
// -200, and 2^-200 is 0 in fp32, so a = 0 makes every factor across that token
// exactly 0), and only 2^{g_i - g_j} for j <= i is ever formed, so nothing
// overflows however strong the decay.  A final chunk of n < C tokens is padded
// with rows that re-read token n-1 (finite values, no out-of-bounds access)
// and get b = 0, a = 1: their corrected writes N are exactly 0 and the decay of
// the real rows is unchanged, so every product is exact for the real tokens;
// padded outputs are not stored.
#include "gdn_common.h"
#include "gdn_launch.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;     // chunk length
constexpr int NT = 512;   // threads per block: 8 waves
constexpr int DVT = 32;   // d_v columns per block
constexpr int LC = C + 8; // padded bf16 row pitch of C-long rows
constexpr int SPIN_LIMIT = 1 << 20;  // bound on any LDS-flag wait (never reached in a correct run)

struct ChunkParams {
    const uint16_t *q, *k, *v;
    const float *beta, *decay;
    const float *state_in;
    float *state_out;
    void *out;
    float *partial, *partial_rev;
    long long T;
    int H, dv, ntile, nblk_dir;
    int reverse, out_mode, xcd_remap, both_dirs;
    float scale;
};

template <int DK>
struct __align__(16) Smem {
    static constexpr int LK = DK + 8;  // padded bf16 row pitch of d_k-long rows
    uint16_t Ks[2][C][LK];   // K, token-major (chunk parity)
    uint16_t Qs[2][C][LK];   // Q, token-major
    float bVt[2][DVT][C + 4];  // b_t v_t of the d_v tile, fp32, [d_v][token]
    uint16_t Sb[2][DVT][LK]; // bf16 state tile at the start of a chunk, [d_v][d_k]
    uint16_t Nt[DVT][LC];    // N^T of the current chunk
    uint16_t Tb[2][C][LC];   // Tm, row-major, zero above the diagonal
    uint16_t Ab[C][LC];      // A (its off-diagonal 16x16 blocks are read)
    float g[3][C];           // cumulative log2 decay (summed in float64), chunk mod 3
    float bet[3][C];         // b (0 on padding)
    float gam[3][C];         // 2^{g_i}
    float bg[3][C];          // b_i 2^{g_i}
    float glast[3][C];       // 2^{g_{C-1} - g_i}
    float xf[3][C];          // 2^{g_31 - g_j} (j < 32), 2^{g_i - g_31} (i >= 32): both <= 1
    int nflag;               // chunks whose N^T has been published
    int kctr;                // K row blocks stored (one arrival per K wave and period)
    int tctr;                // A blocks and diagonal Tm blocks ready (three arrivals per period)
    int stuck;               // set once any wait ran out; later waits return at once
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t lds16(const uint16_t *p) {
    bf16x8_t r;
    __builtin_memcpy(&r, p, 16);
    return r;
}
__device__ __forceinline__ s16x4_t lds8(const uint16_t *p) {
    s16x4_t r;
    __builtin_memcpy(&r, p, 8);
    return r;
}
// Transposed LDS read: within each 16-lane group, result lane i slot s is the
// element at position i%4 of the 4 addressed by lane 4s + i/4.
__device__ __forceinline__ s16x4_t lds_tr(const uint16_t *p) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p));
}
__device__ __forceinline__ bf16x8_t join(s16x4_t a, s16x4_t b) {
    bf16x8_t r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char *>(&r) + 8, &b, 8);
    return r;
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ s16x4_t pack4s(float a, float b, float c, float d) {
    const uint2 u = pack4(a, b, c, d);
    s16x4_t r;
    __builtin_memcpy(&r, &u, 8);
    return r;
}
__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int r = 0; r < 16; ++r) z[r] = 0.f;
    return z;
}
__device__ __forceinline__ f32x4_t zero4() {
    f32x4_t z;
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = 0.f;
    return z;
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A 32x32x16 accumulator holds row 8q + 4h + m of its column (lane % 32) in
// register 4q + m of lane half h = lane / 32.  The A and B operands of the same
// instruction hold, in lane half h, the 8 consecutive k-rows 8h .. 8h + 7 of
// row/column lane % 32.  So the rows 16 KK .. 16 KK + 15 of an accumulator
// become one k-step of an operand (rows as k, the accumulator's columns as the
// operand's rows/columns) by exchanging 4 rows between the lane halves:
// v_permlane32_swap swaps the upper half of its first operand with the lower
// half of its second.
// x = rows 16KK + 4h + 0..3 and y = rows 16KK + 8 + 4h + 0..3, already packed to bf16.
__device__ __forceinline__ bf16x8_t packed_to_op(uint2 x, uint2 y) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
    const uint4 w = make_uint4(s0[0], s1[0], s0[1], s1[1]);
    bf16x8_t r;
    __builtin_memcpy(&r, &w, 16);
    return r;
}
template <int KK>
__device__ __forceinline__ bf16x8_t acc_to_op(const f32x16_t &a) {
    return packed_to_op(make_uint2(pack_bf16x2(a[8 * KK + 0], a[8 * KK + 1]), pack_bf16x2(a[8 * KK + 2], a[8 * KK + 3])),
                        make_uint2(pack_bf16x2(a[8 * KK + 4], a[8 * KK + 5]), pack_bf16x2(a[8 * KK + 6], a[8 * KK + 7])));
}

// Off-diagonal blocks of block column CB of Tm = (I + A)^{-1}, walking down:
//   T_rc = -T_rr * sum_{k=c}^{r-1} A_rk T_kc   (16x16 blocks, bf16 16x16x16 MFMA).
// The diagonal blocks are already in Tb; the column's blocks are passed from one
// product to the next in registers (accumulator layout == B-operand layout).
// All A and T_rr operands are read before any block is written.
template <int CB>
__device__ __forceinline__ void tm_column(uint16_t (*Tb)[LC], const uint16_t (*Ab)[LC], int l16, int g16) {
    s16x4_t tcol[4];
    s16x4_t aop[4][4];  // aop[rb][kb] = A_rb,kb for CB <= kb < rb
    s16x4_t top[4];     // top[rb] = T_rb,rb
    tcol[CB] = lds_tr(&Tb[16 * CB + 4 * g16 + (l16 >> 2)][16 * CB + 4 * (l16 & 3)]);
#pragma unroll
    for (int rb = CB + 1; rb < 4; ++rb) {
        top[rb] = lds8(&Tb[16 * rb + l16][16 * rb + 4 * g16]);
#pragma unroll
        for (int kb = CB; kb < rb; ++kb) aop[rb][kb] = lds8(&Ab[16 * rb + l16][16 * kb + 4 * g16]);
    }
    f32x4_t tout[4];
#pragma unroll
    for (int rb = CB + 1; rb < 4; ++rb) {
        f32x4_t y = zero4();
#pragma unroll
        for (int kb = CB; kb < rb; ++kb) y = mfma16(aop[rb][kb], tcol[kb], y);
        const f32x4_t t = mfma16(top[rb], pack4s(y[0], y[1], y[2], y[3]), zero4());
        tcol[rb] = pack4s(-t[0], -t[1], -t[2], -t[3]);
        tout[rb] = t;
    }
#pragma unroll
    for (int rb = CB + 1; rb < 4; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) Tb[16 * rb + 4 * g16 + r][16 * CB + l16] = (uint16_t)f32_to_bf16_bits(-tout[rb][r]);
}

// Bounded waits on LDS counters.  In a correct run every wait ends within a
// chunk period; the bound (and the sticky `stuck` flag, which makes every later
// wait return at once) only guarantees that the kernel always terminates.
__device__ __forceinline__ void wait_at_least(int *ctr, int target, int *stuck) {
    for (int i = 0; i < SPIN_LIMIT; ++i) {
        if (__hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
        if (__hip_atomic_load(stuck, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) return;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(stuck, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void publish(int *ctr, int value, int lane) {
    // release: this wave's earlier LDS writes are complete before the counter moves
    if (lane == 0) __hip_atomic_store(ctr, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void arrive(int *ctr, int lane) {
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Per-block constants: base pointers already offset to (b, token 0, h), token
// strides in elements, and the chunk walk.
struct Ctx {
    const uint16_t *q, *k, *v;  // v offset to the block's d_v tile
    const float *beta, *decay;
    long long T;
    int nchunks;
    int rs;   // q/k elements between consecutive tokens: H * d_k
    int rsv;  // v/out elements between consecutive tokens: H * d_v
    int H;    // gate elements between consecutive tokens
    int reverse;
    __device__ bool has(int c) const { return c >= 0 && c < nchunks; }
    __device__ int ntok(int c) const {
        const long long r = T - (long long)c * C;
        return r < C ? (int)r : C;
    }
    __device__ long long tok(int c, int j) const {
        const long long s = (long long)c * C + j;
        return reverse ? T - 1 - s : s;
    }
    // token j of chunk c, with rows past the end of a short final chunk clamped
    // to its last token (loads stay in bounds and read finite data)
    __device__ long long tok_clamped(int c, int j) const {
        const int nt = ntok(c);
        return tok(c, j < nt ? j : nt - 1);
    }
};

// One wave's 32-row block of K or Q (rows 32 (role & 1) .. + 31 of K for roles
// 0-1, of Q for roles 2-3), loaded row-coalesced: DK / 8 lanes per row, each
// with 8 consecutive columns, 512 / DK rows per load instruction, so every load
// reads whole rows and touches only the cache lines those rows span.
template <int DK>
struct RowBlock {
    static constexpr int LPR = DK / 8;         // lanes per row
    static constexpr int RPL = 64 / LPR;       // rows per load
    static constexpr int NLD = 32 / RPL;       // loads per 32 rows
    bf16x8_t r[NLD];
};

// Loads are unconditional: rows past the end of a final short chunk re-read
// token n-1 (finite data; those tokens carry b = 0 and a = 1, so every product
// they enter is multiplied by 0 or never stored).  Conditional loads into
// zeroed registers would make the compiler wait for all earlier loads.
template <int DK>
__device__ __forceinline__ RowBlock<DK> load_block(const Ctx &x, int c, int role, int lane) {
    using RB = RowBlock<DK>;
    RB d;
    const uint16_t *base = (role < 2) ? x.k : x.q;
    const int r0 = 32 * (role & 1) + lane / RB::LPR;
    const int col = 8 * (lane % RB::LPR);
#pragma unroll
    for (int s = 0; s < RB::NLD; ++s)
        d.r[s] = *reinterpret_cast<const bf16x8_t *>(base + (size_t)x.tok_clamped(c, r0 + RB::RPL * s) * x.rs + col);
    return d;
}

// The same block into a token-major [C][LK] LDS buffer.
template <int DK>
__device__ __forceinline__ void store_block(uint16_t (*dst)[DK + 8], const RowBlock<DK> &blk, int role, int lane) {
    using RB = RowBlock<DK>;
    const int r0 = 32 * (role & 1) + lane / RB::LPR;
    const int col = 8 * (lane % RB::LPR);
#pragma unroll
    for (int s = 0; s < RB::NLD; ++s) *reinterpret_cast<bf16x8_t *>(&dst[r0 + RB::RPL * s][col]) = blk.r[s];
}

// ---- wave 0: the state chain ------------------------------------------------
template <int DK, bool BF16>
struct Chain {
    static constexpr int NKS = DK / 16;  // k-steps over d_k
    static constexpr int NSB = DK / 32;  // 32-row blocks of S^T
    f32x16_t sacc[NSB];                  // S^T: d_k rows 32*rb + .., d_v column lane % 32
    bf16x8_t sop[NKS];                   // bf16 S^T as the B operand of X = K S^T

    __device__ __forceinline__ void publish_state(Smem<DK> &sm, int slot, int lane) {
        const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int rb = 0; rb < NSB; ++rb) {
            uint2 w[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                w[q] = pack4(sacc[rb][4 * q], sacc[rb][4 * q + 1], sacc[rb][4 * q + 2], sacc[rb][4 * q + 3]);
                *reinterpret_cast<uint2 *>(&sm.Sb[slot][l32][32 * rb + 8 * q + 4 * hi]) = w[q];
            }
            sop[2 * rb] = packed_to_op(w[0], w[1]);
            sop[2 * rb + 1] = packed_to_op(w[2], w[3]);
        }
    }

    __device__ __forceinline__ void init(const ChunkParams &p, Smem<DK> &sm, size_t sbase, int lane) {
        const int hi = lane >> 5;
#pragma unroll
        for (int rb = 0; rb < NSB; ++rb) {
            sacc[rb] = zero16();
            if (p.state_in) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 s4 = *reinterpret_cast<const float4 *>(p.state_in + sbase + 32 * rb + 8 * q + 4 * hi);
                    sacc[rb][4 * q + 0] = s4.x; sacc[rb][4 * q + 1] = s4.y;
                    sacc[rb][4 * q + 2] = s4.z; sacc[rb][4 * q + 3] = s4.w;
                }
            }
        }
        publish_state(sm, 0, lane);
    }

    __device__ __forceinline__ void step(Smem<DK> &sm, int c, int lane) {
        const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
        const int s2 = c & 1, s3 = c % 3;
        // X = K S^T  (tokens x d_v), two 32-token blocks
        f32x16_t xacc[2] = {zero16(), zero16()};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            xacc[0] = mfma32(lds16(&sm.Ks[s2][l32][16 * s + 8 * hi]), sop[s], xacc[0]);
            xacc[1] = mfma32(lds16(&sm.Ks[s2][32 + l32][16 * s + 8 * hi]), sop[s], xacc[1]);
        }
        // R = diag(b) V - diag(b gam) X, then as the B operand of N = Tm R
        bf16x8_t rop[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i0 = 32 * i + 8 * q + 4 * hi;
                const float4 bv = *reinterpret_cast<const float4 *>(&sm.bVt[s2][l32][i0]);
                const float4 bgm = *reinterpret_cast<const float4 *>(&sm.bg[s3][i0]);
                xacc[i][4 * q + 0] = fmaf(-bgm.x, xacc[i][4 * q + 0], bv.x);
                xacc[i][4 * q + 1] = fmaf(-bgm.y, xacc[i][4 * q + 1], bv.y);
                xacc[i][4 * q + 2] = fmaf(-bgm.z, xacc[i][4 * q + 2], bv.z);
                xacc[i][4 * q + 3] = fmaf(-bgm.w, xacc[i][4 * q + 3], bv.w);
            }
            rop[2 * i] = acc_to_op<0>(xacc[i]);
            rop[2 * i + 1] = acc_to_op<1>(xacc[i]);
        }
        // N = Tm R; Tm is lower triangular: token block i needs keys < 32 (i + 1)
        f32x16_t nacc[2] = {zero16(), zero16()};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < 2) nacc[0] = mfma32(lds16(&sm.Tb[s2][l32][16 * t + 8 * hi]), rop[t], nacc[0]);
            nacc[1] = mfma32(lds16(&sm.Tb[s2][32 + l32][16 * t + 8 * hi]), rop[t], nacc[1]);
        }
        // publish N^T for the output waves
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2 *>(&sm.Nt[l32][32 * i + 8 * q + 4 * hi]) =
                    pack4(nacc[i][4 * q], nacc[i][4 * q + 1], nacc[i][4 * q + 2], nacc[i][4 * q + 3]);
        publish(&sm.nflag, c + 1, lane);
        // N~ = diag(G_{C-1,.}) N as the B operand of the update
        bf16x8_t nop[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 gl = *reinterpret_cast<const float4 *>(&sm.glast[s3][32 * i + 8 * q + 4 * hi]);
                nacc[i][4 * q + 0] *= gl.x; nacc[i][4 * q + 1] *= gl.y;
                nacc[i][4 * q + 2] *= gl.z; nacc[i][4 * q + 3] *= gl.w;
            }
            nop[2 * i] = acc_to_op<0>(nacc[i]);
            nop[2 * i + 1] = acc_to_op<1>(nacc[i]);
        }
        // S^T <- gam_{C-1} S^T + K^T N~  (K^T read transposed from the token-major K)
        const float gl = sm.gam[s3][C - 1];
#pragma unroll
        for (int rb = 0; rb < NSB; ++rb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[rb][r] *= gl;
            const int dcol = 32 * rb + 16 * (g16 & 1) + 4 * (l16 & 3);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int t0 = 16 * t + 8 * hi + (l16 >> 2);
                const bf16x8_t a = join(lds_tr(&sm.Ks[s2][t0][dcol]), lds_tr(&sm.Ks[s2][t0 + 4][dcol]));
                sacc[rb] = mfma32(a, nop[t], sacc[rb]);
            }
        }
        publish_state(sm, (c + 1) & 1, lane);
    }

    __device__ __forceinline__ void finish(const ChunkParams &p, size_t sbase, int lane) {
        const int hi = lane >> 5;
        if (!p.state_out) return;
#pragma unroll
        for (int rb = 0; rb < NSB; ++rb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<float4 *>(p.state_out + sbase + 32 * rb + 8 * q + 4 * hi) =
                    make_float4(sacc[rb][4 * q], sacc[rb][4 * q + 1], sacc[rb][4 * q + 2], sacc[rb][4 * q + 3]);
    }
};

// ---- outputs of one 32-token half (query block TB) -----------------------------
// P of the half's query rows is formed here, in registers, from K and Q in LDS
// while the chain is still working on N:
//   TB = 0: P(0,0) = K_a Q_a^T                    (keys 0-31)
//   TB = 1: P(1,0) = K_a Q_b^T, P(1,1) = K_b Q_b^T  (keys 0-63)
// as (keys x queries) accumulators, whose rows become the k-steps of the
// B operand of O^T += N^T P^T.  The same Q operand feeds (S Q^T)^T.
template <int DK>
__device__ __forceinline__ void p_diag_epilogue(const Smem<DK> &sm, int s3, f32x16_t &acc, int b, int lane) {
    // diagonal block b: element (key j, query i) times 2^{g_i - g_j}, kept for j <= i
    const int l32 = lane & 31, hi = lane >> 5;
    const float *gg = sm.g[s3];
    const int i = 32 * b + l32;
    const float gi = gg[i];
    float4 gj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gj[q] = *reinterpret_cast<const float4 *>(&gg[32 * b + 8 * q + 4 * hi]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j0 = 32 * b + 8 * q + 4 * hi;
        const float gjv[4] = {gj[q].x, gj[q].y, gj[q].z, gj[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float val = acc[4 * q + e] * exp2_fast(gi - gjv[e]);
            acc[4 * q + e] = (j0 + e <= i) ? val : 0.f;
        }
    }
}

template <int DK>
__device__ __forceinline__ void cross_scale(const Smem<DK> &sm, int s3, f32x16_t &acc, float si, int lane) {
    // keys 0-31 x queries 32-63: G_ij = 2^{g_i - g_31} 2^{g_31 - g_j}; si carries
    // the query factor (and b_i for A)
    const int hi = lane >> 5;
    float4 fj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) fj[q] = *reinterpret_cast<const float4 *>(&sm.xf[s3][8 * q + 4 * hi]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[4 * q + 0] *= fj[q].x * si;
        acc[4 * q + 1] *= fj[q].y * si;
        acc[4 * q + 2] *= fj[q].z * si;
        acc[4 * q + 3] *= fj[q].w * si;
    }
}

template <int DK, bool BF16, int TB>
__device__ __forceinline__ void output_step(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int c, int lane,
                                            void *out_b, float *part_b) {
    constexpr int NKS = DK / 16;
    const int l32 = lane & 31, hi = lane >> 5;
    const int s2 = c & 1, s3 = c % 3;
    const uint16_t *qrow = &sm.Qs[s2][32 * TB + l32][8 * hi];
    const uint16_t *ka = &sm.Ks[s2][l32][8 * hi];
    const uint16_t *kb = &sm.Ks[s2][32 + l32][8 * hi];
    const uint16_t *srow = &sm.Sb[s2][l32][8 * hi];
    f32x16_t acc = zero16(), p0 = zero16(), p1 = zero16();
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const bf16x8_t q = lds16(qrow + 16 * s);
        acc = mfma32(lds16(srow + 16 * s), q, acc);
        p0 = mfma32(lds16(ka + 16 * s), q, p0);
        if constexpr (TB == 1) p1 = mfma32(lds16(kb + 16 * s), q, p1);
    }
    // (S Q^T)^T scaled by gam of the query column
    const int i = 32 * TB + l32;
    const float gq = sm.gam[s3][i];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] *= gq;
    // P^T as B operands, k-step t = keys 16 t .. 16 t + 15
    bf16x8_t pop[4];
    if constexpr (TB == 0) {
        p_diag_epilogue(sm, s3, p0, 0, lane);
        pop[0] = acc_to_op<0>(p0);
        pop[1] = acc_to_op<1>(p0);
    } else {
        cross_scale(sm, s3, p0, sm.xf[s3][i], lane);
        p_diag_epilogue(sm, s3, p1, 1, lane);
        pop[0] = acc_to_op<0>(p0);
        pop[1] = acc_to_op<1>(p0);
        pop[2] = acc_to_op<0>(p1);
        pop[3] = acc_to_op<1>(p1);
    }
    // + N^T P^T once the chain has published N^T
    wait_at_least(&sm.nflag, c + 1, &sm.stuck);
#pragma unroll
    for (int t = 0; t < 2 * (TB + 1); ++t) acc = mfma32(lds16(&sm.Nt[l32][16 * t + 8 * hi]), pop[t], acc);
    if (i < x.ntok(c)) {
        const size_t e0 = (size_t)x.tok(c, i) * x.rsv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const size_t e = e0 + 8 * q + 4 * hi;
            const float o0 = acc[4 * q] * p.scale, o1 = acc[4 * q + 1] * p.scale;
            const float o2 = acc[4 * q + 2] * p.scale, o3 = acc[4 * q + 3] * p.scale;
            if (p.out_mode == OUT_PARTIAL) {
                *reinterpret_cast<float4 *>(part_b + e) = make_float4(o0, o1, o2, o3);
            } else {
                if constexpr (BF16)
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out_b) + e) = pack4(o0, o1, o2, o3);
                else
                    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out_b) + e) = make_float4(o0, o1, o2, o3);
            }
        }
    }
}

// ---- wave 4: V tiles and gate vectors ----------------------------------------
struct GateRegs {
    float b, a;
};

// The chunk's V tile (64 tokens x 32 d_v), row-coalesced: in w[s], lane l holds
// token 16 s + l / 4, d_v columns 8 (l % 4) .. + 7.
struct VRow {
    u32x4_t w[4];
};
__device__ __forceinline__ VRow load_v(const Ctx &x, int c, int lane) {
    VRow d;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        d.w[s] = *reinterpret_cast<const u32x4_t *>(x.v + (size_t)x.tok_clamped(c, 16 * s + (lane >> 2)) * x.rsv +
                                                    8 * (lane & 3));
    return d;
}
__device__ __forceinline__ void load_gates(const Ctx &x, int c, int lane, GateRegs &g) {
    if (!x.has(c)) return;  // uniform
    const size_t o = (size_t)x.tok_clamped(c, lane) * x.H;
    g.b = x.beta[o];
    g.a = x.decay[o];
}

// Float64 helpers for the gate prefix sum (64 lanes, lane = token).
template <int CTRL>
__device__ __forceinline__ double dpp_shr_f64(double x) {  // row_shr:k, 0 shifted in
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, 0xF, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double lane_value(double x, int l) {
    const uint64_t u = __double_as_longlong(x);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), l);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane row
// (DPP row_shr 1, 2, 4, 8), then the row totals carried across rows.
__device__ __forceinline__ double prefix_sum64(int lane, double x) {
    x += dpp_shr_f64<0x111>(x);
    x += dpp_shr_f64<0x112>(x);
    x += dpp_shr_f64<0x114>(x);
    x += dpp_shr_f64<0x118>(x);
    const double t0 = lane_value(x, 15), t2 = lane_value(x, 47);
    if ((lane & 16) != 0) x += (lane < 32) ? t0 : t2;  // rows 1 and 3
    const double t01 = lane_value(x, 31);
    if (lane >= 32) x += t01;  // rows 2 and 3
    return x;
}

template <int DK>
__device__ __forceinline__ void gates_compute(const Ctx &x, Smem<DK> &sm, int c, int lane, const GateRegs &gr) {
    const bool real = lane < x.ntok(c);
    const float a = real ? gr.a : 1.f;
    float l2 = __builtin_amdgcn_logf(a);  // log2
    if (!(l2 > -200.0f)) l2 = -200.0f;    // a = 0: 2^-200 is 0 in fp32
    const double xs = prefix_sum64(lane, (double)l2);
    const double xl = lane_value(xs, 63);
    const double x31 = lane_value(xs, 31);
    const int s3 = c % 3;
    sm.xf[s3][lane] = exp2_fast((float)(lane < 32 ? x31 - xs : xs - x31));
    sm.g[s3][lane] = (float)xs;
    const float gm = exp2_fast((float)xs);
    sm.gam[s3][lane] = gm;
    sm.bg[s3][lane] = real ? gr.b * gm : 0.f;
    sm.glast[s3][lane] = exp2_fast((float)(xl - xs));
    sm.bet[s3][lane] = real ? gr.b : 0.f;
}

// ---- waves 1, 2, 5, 6: preparation of the next chunk --------------------------
// role 0: K rows 0-31 (K_a), 1: K rows 32-63 (K_b), 2: Q rows 0-31, 3: Q rows 32-63.
// Gram products as (keys x queries):
//   role 0: A(0,0) = K_a K_a^T      role 1: A(1,1) = K_b K_b^T
//   role 2: A(1,0) = K_a K_b^T, P(0,0) = K_a Q_a^T
//   role 3: P(1,0) = K_a Q_b^T, P(1,1) = K_b Q_b^T
// A(1,0) = b_i (k_i . k_j) G_ij for keys j in 0-31 and queries i in 32-63 (every
// j < i), from its Gram accumulator, with the separable cross-block factors;
// written as bf16 to Ab (all of its 16x16 blocks are off-diagonal blocks of A).
template <int DK>
__device__ __forceinline__ void a_cross_block(Smem<DK> &sm, int cp, f32x16_t acc, int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    const int s3 = cp % 3;
    const int i = 32 + l32;
    cross_scale(sm, s3, acc, sm.xf[s3][i] * sm.bet[s3][i], lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2 *>(&sm.Ab[i][8 * q + 4 * hi]) =
            pack4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// y += a_J * b, where a_J is lane J's value of a within each 16-lane row: one
// v_fmac_f32 with a DPP row_newbcast source (register arithmetic only; no
// memory access).  A DPP source read needs two wait states after a VALU write
// of that register; the caller issues them once, after the last write of every
// register it will broadcast from (fmac_dpp_fence).
template <int J>
__device__ __forceinline__ void fmac_row_bcast(float &y, float a, float b) {
    asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(y)
                 : "v"(a), "v"(b), "n"(J));
}
// Two wait states that every register in a[0..14] has been written before.
__device__ __forceinline__ void fmac_dpp_fence(const float (&a)[16]) {
    asm volatile("s_nop 1" ::"v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
                 "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]));
}

// A diagonal 32x32 block kk of A, from its Gram accumulator acc = K_kk K_kk^T
// (keys x queries), and the two diagonal 16x16 blocks of Tm inside it.
//   * epilogue: A_ij = b_i (k_i . k_j) 2^{g_i - g_j} for j < i, else 0;
//     the off-diagonal 16x16 block (rows 16-31, cols 0-15) goes to Ab for the
//     block-column products;
//   * the lane halves exchange 8 keys (v_permlane32_swap) so that lane i of
//     half 0 holds A[i][0..15] and lane i of half 1 holds A[i][16..31]: lanes
//     0-15 then own the rows of diagonal block 0, lanes 48-63 those of block 1,
//     each 16-lane row one block;
//   * row r of (I + A_bb)^{-1} solves (I + A_bb)^T y = e_r by backward
//     substitution, right-looking (once y_j is known, y_m -= A[j][m] y_j for
//     m < j), with row j of A taken from lane j of the 16-lane row by a DPP
//     broadcast folded into the FMA: no LDS traffic and no waits on it.
template <int DK>
__device__ __forceinline__ void a_diag_block(Smem<DK> &sm, int cp, const f32x16_t &acc, int kk, int lane) {
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15;
    const int s3 = cp % 3, s2 = cp & 1;
    const float *gg = sm.g[s3];
    const int i = 32 * kk + l32;
    const float gi = gg[i];
    const float bi = sm.bet[s3][i];
    float4 gj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gj[q] = *reinterpret_cast<const float4 *>(&gg[32 * kk + 8 * q + 4 * hi]);
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j0 = 32 * kk + 8 * q + 4 * hi;
        const float gjv[4] = {gj[q].x, gj[q].y, gj[q].z, gj[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float val = acc[4 * q + e] * exp2_fast(gi - gjv[e]);
            v[4 * q + e] = (j0 + e < i) ? bi * val : 0.f;
        }
    }
    if (l32 >= 16) {  // rows 16-31, keys 0-15: the off-diagonal 16x16 block
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<uint2 *>(&sm.Ab[i][32 * kk + 8 * q + 4 * hi]) =
                pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
    // half 0: keys 0-3 (q0), 8-11 (q1), 16-19 (q2), 24-27 (q3); half 1: +4.
    // Swap q2 of half 0 with q0 of half 1, q3 of half 0 with q1 of half 1.
    float a[16];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[e]), __float_as_uint(v[8 + e]), false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[4 + e]), __float_as_uint(v[12 + e]), false, false);
        a[e] = __uint_as_float(s02[0]);       // keys 0-3 (half 0) / 16-19 (half 1)
        a[4 + e] = __uint_as_float(s02[1]);   // keys 4-7 / 20-23
        a[8 + e] = __uint_as_float(s13[0]);   // keys 8-11 / 24-27
        a[12 + e] = __uint_as_float(s13[1]);  // keys 12-15 / 28-31
    }
    float y[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) y[m] = (m == l16) ? 1.f : 0.f;
    // level J updates y[J-1] first: the next level starts from it
#define GDN_SUBST_STEP(J)                                                         \
    {                                                                             \
        const float nyj = -y[J];                                                  \
        _Pragma("unroll") for (int m = J - 1; m >= 0; --m) fmac_row_bcast<J>(y[m], a[m], nyj); \
    }
    fmac_dpp_fence(a);
    GDN_SUBST_STEP(15) GDN_SUBST_STEP(14) GDN_SUBST_STEP(13) GDN_SUBST_STEP(12)
    GDN_SUBST_STEP(11) GDN_SUBST_STEP(10) GDN_SUBST_STEP(9) GDN_SUBST_STEP(8)
    GDN_SUBST_STEP(7) GDN_SUBST_STEP(6) GDN_SUBST_STEP(5) GDN_SUBST_STEP(4)
    GDN_SUBST_STEP(3) GDN_SUBST_STEP(2) GDN_SUBST_STEP(1)
#undef GDN_SUBST_STEP
    const bool blk0 = lane < 16, blk1 = lane >= 48;
    if (blk0 || blk1) {
        const int kb = 2 * kk + (blk1 ? 1 : 0);
        uint16_t *row = &sm.Tb[s2][16 * kb + l16][16 * kb];
        *reinterpret_cast<uint4 *>(row) = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                                     pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
        *reinterpret_cast<uint4 *>(row + 8) = make_uint4(pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]),
                                                         pack_bf16x2(y[12], y[13]), pack_bf16x2(y[14], y[15]));
        if (blk0) {  // zero block right of the diagonal inside the 32-row block
            *reinterpret_cast<uint4 *>(row + 16) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(row + 24) = make_uint4(0, 0, 0, 0);
        }
    }
}

// Preparation of chunk cp = it + 1 in period it.
//   role 0: K rows 0-31 (K_a): A(0,0), its diagonal Tm blocks, Tm block column 0
//   role 1: K rows 32-63 (K_b): A(1,1), its diagonal Tm blocks, Tm block column 1
//   role 2: Q rows 0-31 (Q_a): A(1,0) = K_a K_b^T, Tm block column 2
template <int DK>
__device__ __forceinline__ void prep_step(const Ctx &x, Smem<DK> &sm, int it, int role, int lane, int np,
                                          RowBlock<DK> &blk) {
    constexpr int NKS = DK / 16;
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
    const int cp = it + 1;
    const bool valid = x.has(cp);
    const int s2 = cp & 1;
    // 1. this wave's row block of chunk cp -> LDS; the registers then take the
    //    loads of chunk it + 3 at once (two periods to land), and every product
    //    below reads its operands from LDS, so nothing here waits on them
    if (valid) store_block<DK>(role < 2 ? sm.Ks[s2] : sm.Qs[s2], blk, role, lane);
    if (x.has(it + 3)) blk = load_block<DK>(x, it + 3, role, lane);
    const uint16_t *ka = &sm.Ks[s2][l32][8 * hi];       // K rows 0-31
    const uint16_t *kb = &sm.Ks[s2][32 + l32][8 * hi];  // K rows 32-63
    if (role < 2) {
        arrive(&sm.kctr, lane);
        // 2a. K_kk K_kk^T (this wave's own rows, just stored) -> A's diagonal 32x32
        //     block and the diagonal 16x16 blocks of Tm; needs no other wave's data
        if (valid) {
            const uint16_t *kk = role == 0 ? ka : kb;
            f32x16_t g0 = zero16();
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                const bf16x8_t r = lds16(kk + 16 * s);
                g0 = mfma32(r, r, g0);
            }
            a_diag_block(sm, cp, g0, role, lane);
        }
    } else {
        // 2b. A(1,0) = K_a K_b^T, once both K blocks are in LDS
        wait_at_least(&sm.kctr, 2 * np, &sm.stuck);
        if (valid) {
            f32x16_t g0 = zero16();
#pragma unroll
            for (int s = 0; s < NKS; ++s) g0 = mfma32(lds16(ka + 16 * s), lds16(kb + 16 * s), g0);
            a_cross_block(sm, cp, g0, lane);
        }
    }
    // 3. off-diagonal blocks of Tm, one block column per wave, once every wave's
    //    diagonal blocks and A blocks are in LDS
    arrive(&sm.tctr, lane);
    wait_at_least(&sm.tctr, 3 * np, &sm.stuck);
    if (valid) {
        if (role == 0) tm_column<0>(sm.Tb[s2], sm.Ab, l16, g16);
        else if (role == 1) tm_column<1>(sm.Tb[s2], sm.Ab, l16, g16);
        else tm_column<2>(sm.Tb[s2], sm.Ab, l16, g16);
    }
}

template <int DK, bool BF16>
__global__ __launch_bounds__(NT) void chunk_kernel(ChunkParams p) {
    static_assert(DK % 32 == 0 && DK <= 128, "d_k must be 32, 64 or 128");
    __shared__ Smem<DK> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

    // Block -> (direction, b, h, d_v tile).  Blocks are dispatched round-robin over
    // the 8 XCDs (linear id mod 8); with the remap, the blocks on one XCD take
    // consecutive (head, tile) indices, so the d_v tiles of a head share an L2.
    int L = blockIdx.x;
    int dir = 0;
    if (p.both_dirs && L >= p.nblk_dir) {
        dir = 1;
        L -= p.nblk_dir;
    }
    const int v = p.xcd_remap ? (L & 7) * (p.nblk_dir >> 3) + (L >> 3) : L;
    const int tile = v % p.ntile;
    const int head = v / p.ntile;
    const int h = head % p.H;
    const int b = head / p.H;
    const int dv0 = tile * DVT;

    Ctx x;
    x.T = p.T;
    x.nchunks = (int)((p.T + C - 1) / C);
    x.rs = p.H * DK;
    x.rsv = p.H * p.dv;
    x.H = p.H;
    x.reverse = p.reverse ^ dir;
    const size_t tok0 = (size_t)b * p.T * p.H + h;  // (b, token 0, h) in [B, T, H]
    x.q = p.q + tok0 * DK;
    x.k = p.k + tok0 * DK;
    x.v = p.v + tok0 * p.dv + dv0;
    x.beta = p.beta + tok0;
    x.decay = p.decay + tok0;
    const int n = x.nchunks;

    if (tid == 0) {
        sm.nflag = 0;
        sm.kctr = 0;
        sm.tctr = 0;
        sm.stuck = 0;
    }

    // Roles by wave (waves w and w + 4 share a SIMD): 0 chain and 4 the Q_b
    // loader beside it (memory operations only); 1 and 5: preparation roles 0
    // and 2; 2 and 6: preparation role 1 and the outputs of tokens 0-31; 3 and
    // 7: the outputs of tokens 32-63 and the gate vectors with b v.  Every role walks the same periods it = -2 .. n-1
    // (two per loop trip, so that register sets alternate at compile time) with
    // one barrier each.
    void *out_b = BF16 ? (void *)(reinterpret_cast<uint16_t *>(p.out) + tok0 * p.dv + dv0)
                       : (void *)(reinterpret_cast<float *>(p.out) + tok0 * p.dv + dv0);
    float *part = dir ? p.partial_rev : p.partial;
    float *part_b = part ? part + tok0 * p.dv + dv0 : nullptr;
    if (wid == 0) {
        const size_t sbase = ((size_t)(b * p.H + h) * p.dv + dv0 + (lane & 31)) * DK;
        Chain<DK, BF16> ch;
        ch.init(p, sm, sbase, lane);
        __syncthreads();
        for (int it = -2; it < n; it += 2) {
            if (it >= 0) ch.step(sm, it, lane);
            __syncthreads();
            if (it + 1 >= 0 && it + 1 < n) ch.step(sm, it + 1, lane);
            __syncthreads();
        }
        ch.finish(p, sbase, lane);
    } else if (wid == 6) {
        __syncthreads();
        for (int it = -2; it < n; it += 2) {
            if (it >= 0) output_step<DK, BF16, 0>(x, sm, p, it, lane, out_b, part_b);
            __syncthreads();
            if (it + 1 >= 0 && it + 1 < n) output_step<DK, BF16, 0>(x, sm, p, it + 1, lane, out_b, part_b);
            __syncthreads();
        }
    } else if (wid == 3) {
        __syncthreads();
        for (int it = -2; it < n; it += 2) {
            if (it >= 0) output_step<DK, BF16, 1>(x, sm, p, it, lane, out_b, part_b);
            __syncthreads();
            if (it + 1 >= 0 && it + 1 < n) output_step<DK, BF16, 1>(x, sm, p, it + 1, lane, out_b, part_b);
            __syncthreads();
        }
    } else if (wid == 4) {
        // Q rows 32-63 of chunk c are stored in period c-1 from register set c&1
        // (loaded in period c-3).  Memory operations only, beside the chain.
        RowBlock<DK> qA, qB;
        if (x.has(0)) qA = load_block<DK>(x, 0, 3, lane);
        auto store_q = [&](int c, const RowBlock<DK> &q) { store_block<DK>(sm.Qs[c & 1], q, 3, lane); };
        __syncthreads();
        for (int it = -2; it < n; it += 2) {
            if (x.has(it + 1)) store_q(it + 1, qB);
            if (x.has(it + 3)) qB = load_block<DK>(x, it + 3, 3, lane);
            __syncthreads();
            if (x.has(it + 2)) store_q(it + 2, qA);
            if (x.has(it + 4)) qA = load_block<DK>(x, it + 4, 3, lane);
            __syncthreads();
        }
    } else if (wid == 7) {
        // Gates of chunk c are computed in period c-2 from register set c&1
        // (loaded in period c-4); b_t v_t of chunk c is stored in period c-1 from
        // V register set c&1 (loaded in period c-3), with b_t from the gate slot.
        GateRegs gA{0.f, 1.f}, gB{0.f, 1.f};
        VRow vA, vB;
        if (x.has(0)) vA = load_v(x, 0, lane);
        load_gates(x, 0, lane, gA);
        load_gates(x, 1, lane, gB);
        auto store_bv = [&](int c, const VRow &v) {
            const int d0 = 8 * (lane & 3);
#pragma unroll
            for (int s_ = 0; s_ < 4; ++s_) {
                const int t = 16 * s_ + (lane >> 2);
                const float bt = sm.bet[c % 3][t];
                float *col = &sm.bVt[c & 1][d0][t];
                const uint32_t w4[4] = {v.w[s_].x, v.w[s_].y, v.w[s_].z, v.w[s_].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    col[(2 * e) * (C + 4)] = bt * bf16_lo(w4[e]);
                    col[(2 * e + 1) * (C + 4)] = bt * bf16_hi(w4[e]);
                }
            }
        };
        __syncthreads();
        for (int it = -2; it < n; it += 2) {
            if (x.has(it + 1)) store_bv(it + 1, vB);
            if (x.has(it + 3)) vB = load_v(x, it + 3, lane);
            if (x.has(it + 2)) gates_compute(x, sm, it + 2, lane, gA);
            load_gates(x, it + 4, lane, gA);
            __syncthreads();
            if (x.has(it + 2)) store_bv(it + 2, vA);
            if (x.has(it + 4)) vA = load_v(x, it + 4, lane);
            if (x.has(it + 3)) gates_compute(x, sm, it + 3, lane, gB);
            load_gates(x, it + 5, lane, gB);
            __syncthreads();
        }
    } else {
        const int role = (wid == 1) ? 0 : (wid == 2) ? 1 : 2;
        RowBlock<DK> rA, rB;  // row blocks of even / odd chunks
        if (x.has(0)) rA = load_block<DK>(x, 0, role, lane);
        __syncthreads();
        int np = 0;  // periods walked so far (sync targets)
        for (int it = -2; it < n; it += 2) {
            prep_step<DK>(x, sm, it, role, lane, ++np, rB);      // prepares chunk it+1 (odd)
            __syncthreads();
            prep_step<DK>(x, sm, it + 1, role, lane, ++np, rA);  // prepares chunk it+2 (even)
            __syncthreads();
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
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out;
    p.partial = a.partial; p.partial_rev = a.partial_rev;
    p.T = a.T; p.H = a.H; p.dv = a.dv;
    p.ntile = a.dv / DVT;
    p.nblk_dir = a.B * a.H * p.ntile;
    p.xcd_remap = (p.nblk_dir % 8) == 0;
    p.reverse = a.reverse; p.out_mode = a.out_mode; p.both_dirs = a.both_dirs;
    p.scale = (float)(1.0 / __builtin_sqrt((double)DK));
    const int nblk = p.nblk_dir * (a.both_dirs ? 2 : 1);
    hipLaunchKernelGGL((chunk_kernel<DK, true>), dim3(nblk), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(int C_, int dk, int dv, int io_bf16) {
    const bool dims = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
    return C_ == C && dims && io_bf16;
}

hipError_t launch_chunk_mfma(const PassArgs &a, int C_, hipStream_t stream) {
    if (!chunk_mfma_supported(C_, a.dk, a.dv, a.io_bf16)) return hipErrorInvalidValue;
    switch (a.dk) {
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
