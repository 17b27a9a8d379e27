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
// (b, h) and a 32-wide tile of d_v and walks the head's chunks in order, with
// its 32 x d_k slice of S in fp32 accumulator registers for the whole call.
// The S-independent per-chunk work (decay factors, Gram products, the
// triangular inverse) is recomputed by each d_v tile of a head: that costs MFMA
// time but keeps HBM traffic at one read of q/k per head (the tiles of a head
// are placed on one XCD so the repeats hit its L2) and buys the CU count the
// sequential chunk chain needs.
//
// Software pipeline.  Iteration c runs the state chain of chunk c and prepares
// chunk c+1, in three barrier-separated phases:
//   phase 1: X = [K;Q] S^T (8 MFMA per wave), R = diag(b)(V - diag(gam) K S^T);
//            off-diagonal blocks of Tm for chunk c; decay factors of chunk c+1;
//            global loads for chunk c+2 issued
//   phase 2: N = Tm R;  Gram products K K^T, K Q^T of chunk c+1 -> A, P
//   phase 3: O = diag(gam) Q S^T + P N (stored);  S update;  16x16 diagonal
//            blocks of Tm for chunk c+1;  chunk c+2 staged into LDS
// Each wave owns one 32-token row block of K or Q (wave 0: K rows 0-31, 1: K
// rows 32-63, 2: Q rows 0-31, 3: Q rows 32-63), loaded from HBM straight into
// registers in MFMA operand layout and prefetched two chunks ahead; the same
// registers serve the Gram products of chunk c+1 and the state products of
// chunk c+1.  K is also kept token-major in LDS (three chunk buffers) and read
// transposed with ds_read_b64_tr_b16 where a product contracts over tokens.
//
// Operand layouts.  A 32x32 MFMA accumulator holds 4 consecutive rows per
// lane, so products are oriented so that accumulator rows are the contraction
// index of the consumer, or the output is contiguous in memory:
//   K K^T, K Q^T as (keys x queries): A and P land row-major;
//   K S^T (tokens x d_v): R lands as R^T [d_v][token];
//   N = Tm R (tokens x d_v): N^T [d_v][token];
//   O^T = S Q^T + N^T P^T (d_v x tokens): 4 consecutive d_v per lane -> 8-byte stores;
//   S^T += K^T N~ (d_k x d_v): the state lands as S [d_v][d_k] for the next X.
// For the 16x16x16 MFMA the accumulator layout equals the B-operand layout, so
// the triangular-inverse chains pass blocks from one product to the next in
// registers.
//
// Triangular inverse.  Tm's four 16x16 diagonal blocks are inverted in fp32
// on the VALU (one row per lane, backward substitution on (I + A)^T); the
// off-diagonal blocks follow block column by block column,
//   T_rc = -T_rr * sum_{k=c}^{r-1} A_rk T_kc,
// on 16x16x16 bf16 MFMA, one block column per wave.
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

constexpr int C = 64;     // chunk length
constexpr int NT = 512;   // threads per block: 4 chain waves + 4 preparation waves
constexpr int DVT = 32;   // d_v columns per block
constexpr int LC = C + 8; // padded bf16 row pitch of C-long rows
constexpr int LV = DVT + 8;

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
    uint16_t Ks[3][C][LK];   // K, token-major, three chunk buffers
    uint16_t Qs[2][C][LK];   // Q, token-major, two chunk buffers
    uint16_t Vs[C][LV];      // V tile of the next chunk, token-major
    uint16_t Sb[DVT][LK];    // bf16 copy of the state tile, [d_v][d_k]
    uint16_t Rt[DVT][LC];    // R^T
    uint16_t Nt[DVT][LC];    // N^T
    uint16_t Nd[DVT][LC];    // (diag(G_{C-1,.}) N)^T
    uint16_t Pb[2][C][LC];   // P, row-major, zero above the diagonal
    uint16_t Tb[C][LC];      // Tm, row-major, zero above the diagonal
    uint16_t Ab[C][LC];      // A (its off-diagonal 16x16 blocks are read)
    float Ad[4][16][20];     // A's diagonal 16x16 blocks, row-major, fp32
    float g[2][C];           // cumulative log2 decay (summed in float64)
    float gam[2][C];         // 2^{g_i}
    float glast[2][C];       // 2^{g_{C-1} - g_i}
    float bet[2][C];
    float rawdec[C], rawbet[C];
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

// Off-diagonal blocks of block column CB of Tm = (I + A)^{-1}, walking down:
//   T_rc = -T_rr * sum_{k=c}^{r-1} A_rk T_kc   (16x16 blocks, bf16 16x16x16 MFMA).
// The diagonal blocks are already in Tb; the column's blocks are passed from one
// product to the next in registers (accumulator layout == B-operand layout).
template <int CB>
__device__ __forceinline__ void tm_column(uint16_t (*Tb)[LC], const uint16_t (*Ab)[LC], int l16, int g16) {
    s16x4_t tcol[4];
    tcol[CB] = lds_tr(&Tb[16 * CB + 4 * g16 + (l16 >> 2)][16 * CB + 4 * (l16 & 3)]);
#pragma unroll
    for (int rb = CB + 1; rb < 4; ++rb) {
        f32x4_t y = zero4();
#pragma unroll
        for (int kb = CB; kb < rb; ++kb) y = mfma16(lds8(&Ab[16 * rb + l16][16 * kb + 4 * g16]), tcol[kb], y);
        const f32x4_t t = mfma16(lds8(&Tb[16 * rb + l16][16 * rb + 4 * g16]), pack4s(y[0], y[1], y[2], y[3]), zero4());
        tcol[rb] = pack4s(-t[0], -t[1], -t[2], -t[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) Tb[16 * rb + 4 * g16 + r][16 * CB + l16] = (uint16_t)f32_to_bf16_bits(-t[r]);
    }
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
    __device__ int ntok(int c) const {
        const long long r = T - (long long)c * C;
        return r < C ? (int)r : C;
    }
    __device__ long long tok(int c, int j) const {
        const long long s = (long long)c * C + j;
        return reverse ? T - 1 - s : s;
    }
};

// Loads are unconditional: rows past the end of a final short chunk re-read
// token n-1 (finite data; those tokens carry b = 0 and a = 1, so every product
// they enter is multiplied by 0 or never stored).  Conditional loads into
// zeroed registers would make the compiler wait for all earlier loads.
template <int DK>
__device__ __forceinline__ void load_block(const Ctx &x, int c, int role, int lane, bf16x8_t *dst) {
    if (c >= x.nchunks) return;  // uniform
    const int nt = x.ntok(c);
    const int r = 32 * (role & 1) + (lane & 31);
    const uint16_t *src = ((role < 2) ? x.k : x.q) + (size_t)x.tok(c, r < nt ? r : nt - 1) * x.rs + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < DK / 16; ++s) {
        const uint4 w = *reinterpret_cast<const uint4 *>(src + 16 * s);
        __builtin_memcpy(&dst[s], &w, 16);
    }
}

// ---- state chain: waves 0-3 -------------------------------------------------
template <int DK, bool BF16>
__device__ __forceinline__ void chain_loop(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int wid,
                                           int lane, void *out_b, float *part_b, size_t sbase) {
    constexpr int NKS = DK / 16;
    constexpr int NSB = DK / 32;
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g16 = lane >> 4;

    f32x16_t sacc = zero16();  // S^T block: d_k rows 32*wid.., d_v cols l32 (waves < NSB)
    if (wid < NSB) {
        if (p.state_in) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const float4 s4 = *reinterpret_cast<const float4 *>(p.state_in + sbase + 32 * wid + 8 * rb + 4 * hi);
                sacc[4 * rb + 0] = s4.x; sacc[4 * rb + 1] = s4.y; sacc[4 * rb + 2] = s4.z; sacc[4 * rb + 3] = s4.w;
            }
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<uint2 *>(&sm.Sb[l32][32 * wid + 8 * rb + 4 * hi]) =
                pack4(sacc[4 * rb], sacc[4 * rb + 1], sacc[4 * rb + 2], sacc[4 * rb + 3]);
    }
    __syncthreads();

    for (int c = -1; c < x.nchunks; ++c) {
        const bool chain = c >= 0;
        const int cb = (c + 3) & 1;  // gate/P buffer of chunk c
        // ===== phase 1: X = [K;Q] S^T, R ===================================
        // this wave's row block of chunk c (K rows for waves 0-1, Q rows for 2-3)
        const uint16_t *blk = (wid < 2) ? &sm.Ks[c < 0 ? 0 : c % 3][32 * (wid & 1) + l32][8 * hi]
                                        : &sm.Qs[c & 1][32 * (wid & 1) + l32][8 * hi];
        f32x16_t xacc = zero16();
        if (chain) {
            if (wid < 2) {
                // K S^T (tokens x d_v), then R = diag(b)(V - diag(gam) K S^T) -> R^T
#pragma unroll
                for (int s = 0; s < NKS; ++s) xacc = mfma32(lds16(blk + 16 * s), lds16(&sm.Sb[l32][16 * s + 8 * hi]), xacc);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int i0 = 32 * wid + 8 * rb + 4 * hi;
                    const s16x4_t vv = lds_tr(&sm.Vs[i0 + (l16 >> 2)][16 * (g16 & 1) + 4 * (l16 & 3)]);
                    uint2 vu;
                    __builtin_memcpy(&vu, &vv, 8);
                    const float4 bt = *reinterpret_cast<const float4 *>(&sm.bet[cb][i0]);
                    const float4 gm = *reinterpret_cast<const float4 *>(&sm.gam[cb][i0]);
                    const float r0 = bt.x * (bf16_lo(vu.x) - gm.x * xacc[4 * rb + 0]);
                    const float r1 = bt.y * (bf16_hi(vu.x) - gm.y * xacc[4 * rb + 1]);
                    const float r2 = bt.z * (bf16_lo(vu.y) - gm.z * xacc[4 * rb + 2]);
                    const float r3 = bt.w * (bf16_hi(vu.y) - gm.w * xacc[4 * rb + 3]);
                    *reinterpret_cast<uint2 *>(&sm.Rt[l32][i0]) = pack4(r0, r1, r2, r3);
                }
            } else {
                // (Q S^T)^T (d_v x tokens), scaled by gam of the token column
#pragma unroll
                for (int s = 0; s < NKS; ++s) xacc = mfma32(lds16(&sm.Sb[l32][16 * s + 8 * hi]), lds16(blk + 16 * s), xacc);
                const float gq = sm.gam[cb][32 * (wid - 2) + l32];
#pragma unroll
                for (int r = 0; r < 16; ++r) xacc[r] *= gq;
            }
        }
        __syncthreads();
        // ===== phase 2: N = Tm R ==============================================
        if (chain && wid < 2) {
            f32x16_t nacc = zero16();  // token block wid; Tm lower triangular: keys < 32*(wid+1)
#pragma unroll
            for (int k = 0; k < 64; k += 16) {
                if (k >= 32 * (wid + 1)) break;
                nacc = mfma32(lds16(&sm.Tb[32 * wid + l32][k + 8 * hi]), lds16(&sm.Rt[l32][k + 8 * hi]), nacc);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int i0 = 32 * wid + 8 * rb + 4 * hi;
                const float4 gl = *reinterpret_cast<const float4 *>(&sm.glast[cb][i0]);
                *reinterpret_cast<uint2 *>(&sm.Nt[l32][i0]) =
                    pack4(nacc[4 * rb], nacc[4 * rb + 1], nacc[4 * rb + 2], nacc[4 * rb + 3]);
                *reinterpret_cast<uint2 *>(&sm.Nd[l32][i0]) =
                    pack4(gl.x * nacc[4 * rb], gl.y * nacc[4 * rb + 1], gl.z * nacc[4 * rb + 2], gl.w * nacc[4 * rb + 3]);
            }
        }
        __syncthreads();
        // ===== phase 3: outputs, state update =================================
        if (chain) {
            if (wid >= 2) {
                // O^T = gam (Q S^T)^T + N^T P^T for query block tb, keys < 32*(tb+1)
                const int tb = wid - 2;
#pragma unroll
                for (int k = 0; k < 64; k += 16) {
                    if (k >= 32 * (tb + 1)) break;
                    xacc = mfma32(lds16(&sm.Nt[l32][k + 8 * hi]), lds16(&sm.Pb[cb][32 * tb + l32][k + 8 * hi]), xacc);
                }
                const int i = 32 * tb + l32;
                if (i < x.ntok(c)) {
                    const size_t e0 = (size_t)x.tok(c, i) * x.rsv;
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        const size_t e = e0 + 8 * rb + 4 * hi;
                        float o0 = xacc[4 * rb] * p.scale, o1 = xacc[4 * rb + 1] * p.scale;
                        float o2 = xacc[4 * rb + 2] * p.scale, o3 = xacc[4 * rb + 3] * p.scale;
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
            if (wid < NSB) {
                // S^T <- gam_{C-1} S^T + K^T N~  (K^T read transposed from the token-major K)
                const float gl = sm.gam[cb][C - 1];
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[r] *= gl;
                const int kb3 = c % 3;
                const int dcol = 32 * wid + 16 * (g16 & 1) + 4 * (l16 & 3);
#pragma unroll
                for (int t = 0; t < 64; t += 16) {
                    const int t0 = t + 8 * hi + (l16 >> 2);
                    const bf16x8_t a = join(lds_tr(&sm.Ks[kb3][t0][dcol]), lds_tr(&sm.Ks[kb3][t0 + 4][dcol]));
                    sacc = mfma32(a, lds16(&sm.Nd[l32][t + 8 * hi]), sacc);
                }
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    *reinterpret_cast<uint2 *>(&sm.Sb[l32][32 * wid + 8 * rb + 4 * hi]) =
                        pack4(sacc[4 * rb], sacc[4 * rb + 1], sacc[4 * rb + 2], sacc[4 * rb + 3]);
            }
        }
        __syncthreads();
    }

    if (p.state_out && wid < NSB) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            *reinterpret_cast<float4 *>(p.state_out + sbase + 32 * wid + 8 * rb + 4 * hi) =
                make_float4(sacc[4 * rb], sacc[4 * rb + 1], sacc[4 * rb + 2], sacc[4 * rb + 3]);
    }
}

// ---- preparation: waves 4-7 (role = wid - 4) ---------------------------------
template <int DK>
__device__ __forceinline__ void prep_loop(const Ctx &x, Smem<DK> &sm, int role, int lane) {
    constexpr int NKS = DK / 16;
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
    const int ptid = 64 * role + lane;
    const int v_tok = ptid >> 2, v_part = ptid & 3;  // V tile: 64 tokens x 4 16-byte vectors

    auto store_block = [&](int c, const bf16x8_t *src) {
        uint16_t *row = (role < 2) ? &sm.Ks[c % 3][32 * (role & 1) + l32][8 * hi] : &sm.Qs[c & 1][32 * (role & 1) + l32][8 * hi];
#pragma unroll
        for (int s = 0; s < NKS; ++s) __builtin_memcpy(row + 16 * s, &src[s], 16);
    };
    auto load_v = [&](int c, uint4 &w) {
        if (c >= x.nchunks) return;  // uniform
        const int nt = x.ntok(c);
        w = *reinterpret_cast<const uint4 *>(x.v + (size_t)x.tok(c, v_tok < nt ? v_tok : nt - 1) * x.rsv + 8 * v_part);
    };
    // gates of chunk c (role 0, lane = token); padding gets b = 0, a = 1 when stored
    auto load_gates = [&](int c, float &bb, float &aa, bool &ok) {
        ok = false;
        if (c >= x.nchunks) return;  // uniform
        const int nt = x.ntok(c);
        ok = lane < nt;
        const size_t g = (size_t)x.tok(c, ok ? lane : nt - 1) * x.H;
        bb = x.beta[g];
        aa = x.decay[g];
    };

    bf16x8_t rcur[NKS], rnext[NKS];  // this wave's row block of chunk c+1, and of chunk c+2
    uint4 vpf = make_uint4(0, 0, 0, 0);
    float bpf = 0.f, apf = 1.f;
    bool gpf = false;
    if (x.nchunks > 0) {
        load_block<DK>(x, 0, role, lane, rcur);
        if (role == 0) load_gates(0, bpf, apf, gpf);
        store_block(0, rcur);
        if (role == 0) {
            sm.rawbet[lane] = gpf ? bpf : 0.f;
            sm.rawdec[lane] = gpf ? apf : 1.f;
        }
    }
    __syncthreads();

    for (int c = -1; c < x.nchunks; ++c) {
        const bool prep = c + 1 < x.nchunks;
        const int nb = c & 1;  // gate/P buffer of chunk c+1 (== (c + 4) & 1)
        f32x16_t g0 = zero16(), g1 = zero16();
        // ===== phase 1: later chunks' loads; Tm of chunk c; Gram products of c+1
        load_block<DK>(x, c + 2, role, lane, rnext);
        load_v(c + 1, vpf);
        if (role == 0) load_gates(c + 2, bpf, apf, gpf);
        if (c >= 0) {  // off-diagonal 16x16 blocks of Tm for chunk c: block column `role`
            if (role == 0) tm_column<0>(sm.Tb, sm.Ab, l16, g16);
            else if (role == 1) tm_column<1>(sm.Tb, sm.Ab, l16, g16);
            else if (role == 2) tm_column<2>(sm.Tb, sm.Ab, l16, g16);
        }
        if (prep) {
            if (role == 3) {
                // decay factors of chunk c+1: g = cumulative log2 a (summed in float64)
                const float a = sm.rawdec[lane];
                float l2 = __builtin_amdgcn_logf(a);  // log2
                if (!(l2 > -200.0f)) l2 = -200.0f;    // a = 0: 2^-200 is 0 in fp32
                double xs = (double)l2;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const double y = __shfl_up(xs, off, 64);
                    if (lane >= off) xs += y;
                }
                const double xl = __shfl(xs, 63, 64);
                sm.g[nb][lane] = (float)xs;
                sm.gam[nb][lane] = exp2_fast((float)xs);
                sm.glast[nb][lane] = exp2_fast((float)(xl - xs));
                sm.bet[nb][lane] = sm.rawbet[lane];
            }
            // Gram products of chunk c+1, computed as (keys x queries):
            //   role 0: K_a K_a^T          role 1: K_b K_b^T
            //   role 2: K_a Q_a^T, K_a K_b^T   role 3: K_a Q_b^T, K_b Q_b^T
            const int kb3 = (c + 1) % 3;
            if (role < 2) {
#pragma unroll
                for (int s = 0; s < NKS; ++s) g0 = mfma32(rcur[s], rcur[s], g0);
            } else if (role == 2) {
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const int ko = 16 * s + 8 * hi;
                    const bf16x8_t ka = lds16(&sm.Ks[kb3][l32][ko]);
                    g0 = mfma32(ka, rcur[s], g0);
                    g1 = mfma32(ka, lds16(&sm.Ks[kb3][32 + l32][ko]), g1);
                }
            } else {
#pragma unroll
                for (int s = 0; s < NKS; ++s) {
                    const int ko = 16 * s + 8 * hi;
                    g0 = mfma32(lds16(&sm.Ks[kb3][l32][ko]), rcur[s], g0);
                    g1 = mfma32(lds16(&sm.Ks[kb3][32 + l32][ko]), rcur[s], g1);
                }
            }
        }
        __syncthreads();
        // ===== phase 2: Gram epilogues of chunk c+1 -> A, P ===================
        if (prep) {
            // element (key j, query i); factor 2^{g_i - g_j} for j <= i
            const float *gg = sm.g[nb];
            auto epi = [&](const f32x16_t &acc, int jb, int ib, bool is_k) {
                const int i = 32 * ib + l32;
                const float gi = gg[i];
                const float bi = sm.bet[nb][i];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int j0 = 32 * jb + 8 * rb + 4 * hi;
                    const float4 gj = *reinterpret_cast<const float4 *>(&gg[j0]);
                    const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
                    float v4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int j = j0 + e;
                        const float val = acc[4 * rb + e] * exp2_fast(gi - gjv[e]);
                        v4[e] = is_k ? ((j < i) ? bi * val : 0.f) : ((j <= i) ? val : 0.f);
                    }
                    if (!is_k) {
                        *reinterpret_cast<uint2 *>(&sm.Pb[nb][i][j0]) = pack4(v4[0], v4[1], v4[2], v4[3]);
                    } else if ((i >> 4) == (j0 >> 4)) {
                        *reinterpret_cast<float4 *>(&sm.Ad[i >> 4][i & 15][j0 & 15]) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                    } else if ((i >> 4) > (j0 >> 4)) {
                        *reinterpret_cast<uint2 *>(&sm.Ab[i][j0]) = pack4(v4[0], v4[1], v4[2], v4[3]);
                    }
                }
            };
            if (role == 0) {
                epi(g0, 0, 0, true);
            } else if (role == 1) {
                epi(g0, 1, 1, true);
            } else if (role == 2) {
                epi(g0, 0, 0, false);
                epi(g1, 0, 1, true);
            } else {
                epi(g0, 0, 1, false);
                epi(g1, 1, 1, false);
            }
        }
        __syncthreads();
        // ===== phase 3: diagonal blocks of Tm for chunk c+1; staging ==========
        if (prep && role < 2 && g16 < 2) {
            // lane l16 of half g16 owns row l16 of block 2*role + g16.  Row i of
            // (I + A_kk)^{-1} solves (I + A_kk)^T y = e_i; backward substitution,
            // right-looking: once y_j is known, y_m -= A[j][m] y_j for every m < j.
            const int kb = 2 * role + g16;
            const int i = l16;
            float y[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) y[m] = (m == i) ? 1.f : 0.f;
#pragma unroll
            for (int j = 15; j >= 1; --j) {
                const float *arow = &sm.Ad[kb][j][0];  // A[j][m], m < j
                float av[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    if (4 * q4 >= j) break;
                    const float4 f = *reinterpret_cast<const float4 *>(arow + 4 * q4);
                    av[4 * q4] = f.x; av[4 * q4 + 1] = f.y; av[4 * q4 + 2] = f.z; av[4 * q4 + 3] = f.w;
                }
#pragma unroll
                for (int m = 0; m < j; ++m) y[m] -= av[m] * y[j];
            }
            uint16_t *row = &sm.Tb[16 * kb + i][16 * kb];
            const uint4 w0 = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                        pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            const uint4 w1 = make_uint4(pack_bf16x2(y[8], y[9]), pack_bf16x2(y[10], y[11]),
                                        pack_bf16x2(y[12], y[13]), pack_bf16x2(y[14], y[15]));
            *reinterpret_cast<uint4 *>(row) = w0;
            *reinterpret_cast<uint4 *>(row + 8) = w1;
            if ((kb & 1) == 0) {  // zero block right of the diagonal inside the 32-row block
                *reinterpret_cast<uint4 *>(row + 16) = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(row + 24) = make_uint4(0, 0, 0, 0);
            }
        }
        // stage chunk c+2 (row blocks), chunk c+1's V tile and chunk c+2's gates
        if (c + 2 < x.nchunks) store_block(c + 2, rnext);
        if (prep) *reinterpret_cast<uint4 *>(&sm.Vs[v_tok][8 * v_part]) = vpf;
        if (role == 0 && c + 2 < x.nchunks) {
            sm.rawbet[lane] = gpf ? bpf : 0.f;
            sm.rawdec[lane] = gpf ? apf : 1.f;
        }
#pragma unroll
        for (int s = 0; s < NKS; ++s) rcur[s] = rnext[s];
        __syncthreads();
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

    if (wid < 4) {
        void *out_b = BF16 ? (void *)(reinterpret_cast<uint16_t *>(p.out) + tok0 * p.dv + dv0)
                           : (void *)(reinterpret_cast<float *>(p.out) + tok0 * p.dv + dv0);
        float *part = dir ? p.partial_rev : p.partial;
        float *part_b = part ? part + tok0 * p.dv + dv0 : nullptr;
        const size_t sbase = ((size_t)(b * p.H + h) * p.dv + dv0 + (lane & 31)) * DK;
        chain_loop<DK, BF16>(x, sm, p, wid, lane, out_b, part_b, sbase);
    } else {
        prep_loop<DK>(x, sm, wid - 4, lane);
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
