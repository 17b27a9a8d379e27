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
// Two kernels per call.
//
// tm_kernel (throughput): Tm depends only on K and the gates, so it is formed
// once per (direction, b, h, chunk) -- one block each, all chunks in parallel --
// and written as bf16 in exactly the register order in which the state chain
// uses it as an MFMA operand (5 KiB per chunk), with the chunk's gate records
// (b and log2 a of each token, and 1/||k|| with the prologue: 512 bytes or 1 KiB,
// so that chunk_kernel reads its
// gates in one coalesced load instead of two loads whose lanes all fall on
// different cache lines).  That costs extra HBM traffic
// (K read again, Tm written and read back) and takes the Gram products, the
// decay epilogues and the triangular inverse off the sequential path, where
// every d_v tile of a head would otherwise redo them.
//
// chunk_kernel (sequential over chunks): rows of S are independent, so a block
// owns one (b, h) and a 32-wide tile of d_v and walks the head's chunks in
// order.  The tiles of a head are placed on one XCD and share q/k/Tm through its
// L2.  Eight waves with fixed roles; waves w and w + 4 share a SIMD (w < 4, the
// compute wave, at a raised wave priority); one workgroup barrier per chunk
// period.  In period c:
//   waves 0, 1  the state chain of chunk c, 16 d_v columns each.  S^T (d_k x 16)
//               lives in fp32 accumulators of 16x16x32 MFMAs for the whole call.
//               X = K S^T, R, N = Tm R and S^T = gam_{C-1} S^T + K^T N~ hand their
//               results from one product to the next in registers with no lane
//               exchange: a 16x16 accumulator holds rows 4(l/16) .. +3 of column
//               l % 16, and two of them side by side are one k-step of a B
//               operand if the k index is permuted (slots 0-3 = rows 4g .. 4g+3 of
//               the first block, slots 4-7 = the same rows of the second); the A
//               operand is read from LDS under the same permutation.  Each publishes its columns of N and a bf16 copy
//               of its S columns for the outputs in double-buffered LDS slots
//               (read after the period's barrier).
//   waves 2, 3  outputs, query blocks {0, 3} and {1, 2} (16 queries each, the
//               same work): in period c, gam .* (S Q^T) and P of chunk c in
//               registers; in period c+1, + N^T P^T, staged through a
//               wave-private LDS tile and stored as whole 64-byte row segments.
//   waves 4, 5  K and Q of chunk c+1 (HBM -> registers -> LDS), loaded in
//               period c-2 (two register sets alternate).
//   wave 6      gate vectors of chunk c+2 from the chunk's gate records (b,
//               log2 a and, with the prologue, 1/||k|| per token, written contiguously by tm_kernel
//               from the strided [B, T, H] gates): float64 prefix sum of log2 a
//               (DPP within 16-lane rows, then the row carries), 2^g, b 2^g,
//               2^{g_last - g}, b.  It also stages chunk c+1's Tm operands
//               (HBM -> registers -> LDS, loaded in period c-2), so the chain
//               never waits on a global load (0.861 -> 0.832 ms per call), and,
//               in the second launch of the bidirectional split, the other
//               direction's outputs of chunk c.
//   wave 7      b_t v_t of chunk c+1 (fp32, d_v-major) for R.
//
// Fused input prologue (template flag PRO): q, k, v are read in place from a
// packed token-major projection (token and batch strides), the gate inputs are
// logits (b = sigmoid(x_b), log2 a = -softplus(x_a) / ln 2, applied by tm_kernel
// as it reads them), and q, k are L2-normalised without touching the bf16
// operands: tm_kernel forms each token's 1 / ||k|| from the K rows it loads and
// folds it into A's row and column factors (and puts it in the gate record, from
// which chunk_kernel folds it into the per-token factors of R, the state update
// and P); the output waves
// form 1 / ||q|| from the Q operands they hold (v_dot2 and two lane swaps) and
// apply it with the 1/sqrt(d_k)
// scale.  Only per-token factors change, so without the prologue every factor is
// bit for bit the plain one.
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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int C = 64;     // chunk length
constexpr int NT = 512;   // threads per block of the chunk kernel: 8 waves
constexpr int DVT = 32;   // d_v columns per block
constexpr int LC = C + 8; // padded bf16 row pitch of C-long rows

// Tm in chain operand order: operand o = (token block nb, k-step ks) of N = Tm R
// for (nb, ks) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1) -- the blocks above the
// diagonal are zero and never stored.  Lane l of operand o holds
// Tm[16 nb + l%16][32 ks + 4 (l/16) + 0..3] and Tm[16 nb + l%16][32 ks + 16 + 4 (l/16) + 0..3].
// In memory (inverse pass -> gate wave) operands 0 and 3, whose second halves lie
// above the diagonal, keep their first halves only (8 bytes per lane): 5 KiB per
// chunk; the LDS slot holds the full operands.
constexpr int TM_OPS = 6;
constexpr int TM_LDS_ELEMS = TM_OPS * 64 * 8;  // bf16 per chunk in LDS
constexpr int TM_ELEMS = 4 * 64 * 8 + 2 * 64 * 4;  // bf16 per chunk in memory
__host__ __device__ constexpr bool tm_half(int o) { return o == 0 || o == 3; }
__host__ __device__ constexpr int tm_off(int o) {  // element offset of operand o in memory
    return o == 0 ? 0 : o == 1 ? 256 : o == 2 ? 768 : o == 3 ? 1280 : o == 4 ? 1536 : 2048;
}
static_assert(tm_off(5) + 64 * 8 == TM_ELEMS, "operand layout");
__host__ __device__ constexpr int tm_op(int nb, int ks) { return nb < 2 ? nb : 2 + 2 * (nb - 2) + ks; }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16k32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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
__device__ __forceinline__ s16x4_t pack4s(const f32x4_t &v) { return pack4s(v[0], v[1], v[2], v[3]); }
__device__ __forceinline__ bf16x8_t join_u2(uint2 a, uint2 b) {
    const uint4 w = make_uint4(a.x, a.y, b.x, b.y);
    bf16x8_t r;
    __builtin_memcpy(&r, &w, 16);
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

// Per-block constants: base pointers already offset to (b, token 0, h), token
// strides in elements, and the chunk walk.
struct Ctx {
    const char *q, *k, *v;      // bytes; v offset to the block's d_v tile
    const float *beta, *decay;
    const void *grec;           // the head's gate records, C per chunk: float4 (b, log2 a, 1/||k||, 0)
                                // with the prologue, else float2 (b, log2 a)
    long long T;
    int nchunks;
    int c0 = 0, c1 = 0;  // the chunks this launch walks: [c0, c1) (chunk_kernel)
    int rs;   // q/k bytes between consecutive tokens (H * d_k elements when contiguous)
    int rsv;  // v bytes between consecutive tokens (H * d_v elements when contiguous)
    int rso;  // out elements between consecutive tokens: H * d_v
    int H;    // gate elements between consecutive tokens
    int reverse;
    __device__ bool has(int c) const { return c >= c0 && c < c1; }
    // c clamped into [c0, c1 - 1]: the prefetches are unconditional, so past the end
    // of the range they re-read its last chunk
    __device__ int clamp(int c) const { return c < c1 ? c : c1 - 1; }
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

// Row j of chunk c of a token-major tensor with `stride` bytes per token: one
// 64-bit base per chunk, then a 32-bit signed offset per row (clamped to the
// chunk's last token as in Ctx::tok_clamped).
struct ChunkRows {
    const char *base;  // token 0 of the chunk
    int step;          // +stride, or -stride when walking backwards
    int last;          // ntok - 1
    __device__ const char *row(int j) const { return base + (long long)((j < last ? j : last) * step); }
};
__device__ __forceinline__ ChunkRows chunk_rows(const Ctx &x, const char *p, int c, int stride) {
    ChunkRows r;
    r.base = p + x.tok(c, 0) * stride;
    r.step = x.reverse ? -stride : stride;
    r.last = x.ntok(c) - 1;
    return r;
}

// ---- gate vectors (one lane per token of the chunk) ----------------------------
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

// The chunk's gate vectors, lane = token.  Both kernels compute them with this
// one function, so they agree bit for bit.
//
// With the fused prologue, q and k enter only through per-token factors:
// q^_i = rq_i q_i and k^_j = rk_j k_j (rq, rk the inverse L2 norms), so
//   A_ij = (b_i rk_i) 2^{g_i - gk_j} (k_i . k_j),   gk_j = g_j - log2 rk_j,
//   R    = diag(b) V - diag(b gam rk) K S0^T,
//   S    = gam_{C-1} S0 + N^T diag(2^{g_{C-1} - gk}) K,
//   O_i  = rq_i (gam_i (Q S0^T)_i + sum_j 2^{g_i - gk_j} (q_i . k_j) N_j)  (times 1/sqrt(d_k)),
// and the bf16 operands stay the inputs as given.  rk comes from the inverse
// pass (which reads K anyway); rq is formed by the output waves from the Q
// operands they hold.  Without the prologue rk = 1 and gk = g.
struct GateVals {
    float g;      // cumulative log2 decay g_i (summed in float64)
    float gk;     // g_j - log2 rk_j: key-side exponent of A and P
    float bet;    // b (0 on padding)
    float bk;     // b_i rk_i: row factor of A (0 on padding)
    float gam;    // 2^{g_i}
    float bg;     // b_i 2^{g_i} rk_i
    float glast;  // 2^{g_{C-1} - gk_i}
    float xf;     // 2^{g_31 - gk_j} (j < 32), 2^{g_i - g_31} (i >= 32): both <= 1 for unit rk
};
// b_t and log2 a_t of one token from the gate inputs (values, or logits with
// the prologue); log2 a is clamped at -200 (a = 0: 2^-200 is 0 in fp32).
template <bool PRO>
__device__ __forceinline__ void gate_in(float xb, float xa, float &b, float &l2a) {
    if constexpr (PRO) {
        b = sigmoid_f32(xb);
        l2a = log2_decay_from_logit(xa);
    } else {
        b = xb;
        l2a = __builtin_amdgcn_logf(xa);  // log2
    }
    if (!(l2a > -200.0f)) l2a = -200.0f;
}
// From b_t and log2 a_t (gate_in) and the inverse k norm of every token.
template <bool PRO>
__device__ __forceinline__ GateVals gate_values(int lane, int ntok, float b, float l2, float rk) {
    const bool real = lane < ntok;
    if (!real) l2 = 0.0f;  // padding: a = 1
    const double xs = prefix_sum64(lane, (double)l2);
    const double xl = lane_value(xs, 63);
    const double x31 = lane_value(xs, 31);
    double xk = xs;
    if constexpr (PRO) xk = xs - (double)__builtin_amdgcn_logf(rk);
    GateVals r;
    r.xf = exp2_fast((float)(lane < 32 ? x31 - xk : xs - x31));
    r.g = (float)xs;
    r.gk = (float)xk;
    r.gam = exp2_fast((float)xs);
    r.bg = real ? b * r.gam * rk : 0.f;
    r.glast = exp2_fast((float)(xl - xk));
    r.bet = real ? b : 0.f;
    r.bk = real ? b * rk : 0.f;
    return r;
}

// =============================================================================
// tm_kernel: Tm = (I + A)^{-1} of every chunk, in chain operand order.
// =============================================================================
struct TmParams {
    const char *k;
    const float *beta, *decay;
    uint16_t *tm;     // [dirs][B][H][nchunks][TM_ELEMS]
    void *grec;       // [dirs][B][H][nchunks][C] gate records: float4 (b, log2 a, 1/||k||, 0) with
                      // the prologue, else float2 (b, log2 a)
    long long T;
    long long qk_ts, qk_bs;
    int B, H, nchunks, reverse;
    int c0, nc;       // the chunks of this launch: [c0, c0 + nc)
    int nblk, xcd_remap;  // the launch's block count; 1: blocks remapped so each XCD takes a contiguous range
};

// K is dead once the Gram products are in registers, so Tm and A reuse its
// space (a barrier separates the last read of K from the first write of Tm / A).
template <int DK>
struct __align__(16) TmSmem {
    union {
        uint16_t Ks[C][DK + 8];  // K, token-major
        struct {
            uint16_t Tb[C][LC];  // Tm, row-major, zero above the diagonal
            uint16_t Ab[C][LC];  // A (its off-diagonal 16x16 blocks are read)
        };
    };
    float g[C], gk[C], bk[C], xf[C];  // GateVals
    float rk[C];                     // prologue: inverse L2 norms of k_t
};

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
//   * epilogue: A_ij = b_i rk_i (k_i . k_j) 2^{g_i - gk_j} for j < i, else 0
//     (rk = 1 and gk = g without the prologue);
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
__device__ __forceinline__ void a_diag_block(TmSmem<DK> &sm, const f32x16_t &acc, int kk, int lane) {
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15;
    const int i = 32 * kk + l32;
    const float gi = sm.g[i];
    const float bi = sm.bk[i];
    float4 gj[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gj[q] = *reinterpret_cast<const float4 *>(&sm.gk[32 * kk + 8 * q + 4 * hi]);
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
        uint16_t *row = &sm.Tb[16 * kb + l16][16 * kb];
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

// A(1,0) = b_i rk_i (k_i . k_j) 2^{g_i - gk_j} for keys j in 0-31 and queries i
// in 32-63 (every j < i), from its Gram accumulator K_a K_b^T (keys x queries),
// with the separable factors 2^{g_i - g_31} 2^{g_31 - gk_j}; written as bf16 to
// Ab (all of its 16x16 blocks are off-diagonal blocks of A).
template <int DK>
__device__ __forceinline__ void a_cross_block(TmSmem<DK> &sm, const f32x16_t &acc, int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
    const int i = 32 + l32;
    const float si = sm.xf[i] * sm.bk[i];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 fj = *reinterpret_cast<const float4 *>(&sm.xf[8 * q + 4 * hi]);
        *reinterpret_cast<uint2 *>(&sm.Ab[i][8 * q + 4 * hi]) =
            pack4(acc[4 * q] * (fj.x * si), acc[4 * q + 1] * (fj.y * si), acc[4 * q + 2] * (fj.z * si),
                  acc[4 * q + 3] * (fj.w * si));
    }
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

// Sum of squares of 8 bf16 values (two per word).
__device__ __forceinline__ float sumsq8(const u32x4_t &w) {
    const uint32_t u[4] = {w[0], w[1], w[2], w[3]};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(u[e]), hi = bf16_hi(u[e]);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}

// Columns of a row that one 16-byte load holds: 8 bf16 or 16 FP8 values.
template <int IO>
__host__ __device__ constexpr int seg_cols() { return IO == IO_FP8 ? 16 : 8; }

// One 16-byte row segment as loaded, widened to bf16 and stored at dst
// (seg_cols<IO>() bf16 values); returns the sum of their squares if asked.
template <int IO, bool SUMSQ>
__device__ __forceinline__ float put_seg(uint16_t *dst, const u32x4_t &w) {
    if constexpr (IO == IO_FP8) {
        const uint2 a = fp8x4_to_bf16x4(w[0]), b = fp8x4_to_bf16x4(w[1]);
        const uint2 c = fp8x4_to_bf16x4(w[2]), d = fp8x4_to_bf16x4(w[3]);
        const u32x4_t lo = {a.x, a.y, b.x, b.y}, hi = {c.x, c.y, d.x, d.y};
        *reinterpret_cast<u32x4_t *>(dst) = lo;
        *reinterpret_cast<u32x4_t *>(dst + 8) = hi;
        return SUMSQ ? sumsq8(lo) + sumsq8(hi) : 0.f;
    } else {
        *reinterpret_cast<u32x4_t *>(dst) = w;
        return SUMSQ ? sumsq8(w) : 0.f;
    }
}

// One block (4 waves) per (direction, b, h, chunk); up to 8 blocks per CU.
template <int DK, int IO, bool PRO>
__global__ __launch_bounds__(256, 8) void tm_kernel(TmParams p) {
    __shared__ TmSmem<DK> sm;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Head fastest: blocks that run together read the same tokens of all heads,
    // which lie next to each other in the token-major K and the [B, T, H] gates.
    // Blocks are dispatched round-robin over the 8 XCDs (linear id mod 8); with the
    // remap each XCD takes a contiguous range of that order, so the gate lines that
    // the heads of a chunk share are fetched into one XCD's L2, not into eight.
    long long L = p.xcd_remap ? (long long)(blockIdx.x & 7) * (p.nblk >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    const int h = (int)(L % p.H);
    L /= p.H;
    const int c = p.c0 + (int)(L % p.nc);
    L /= p.nc;
    const int b = (int)(L % p.B);
    const int dir = (int)(L / p.B);

    constexpr int ES = io_in_bytes(IO);
    Ctx x;
    x.T = p.T;
    x.nchunks = p.nchunks;
    x.c0 = 0;
    x.c1 = p.nchunks;
    x.rs = (int)(p.qk_ts * ES);
    x.rsv = 0;
    x.rso = 0;
    x.H = p.H;
    x.reverse = p.reverse ^ dir;
    const size_t gtok0 = (size_t)b * p.T * p.H + h;  // (b, token 0, h) of the [B, T, H] gates
    x.q = nullptr;
    x.v = nullptr;
    x.k = p.k + ((size_t)b * p.qk_bs + (size_t)h * DK) * ES;
    x.beta = p.beta + gtok0;
    x.decay = p.decay + gtok0;
    x.grec = nullptr;

    // 1. The chunk's K rows into LDS as bf16, row-coalesced (16 bytes per lane,
    //    DK / seg_cols lanes per row, block-wide passes).  With the prologue the
    //    same lanes form every row's inverse L2 norm (a sum over the row's lanes).
    //    Wave 3 reads the gate inputs.
    float xb = 0.f, xa = 1.f;
    if (wid == 3) {
        const size_t o = (size_t)x.tok_clamped(c, lane) * x.H;
        xb = x.beta[o];
        xa = x.decay[o];
    }
    {
        constexpr int SC = seg_cols<IO>(), LPR = DK / SC, RPB = 256 / LPR, NP = (C + RPB - 1) / RPB;
        const int r0 = threadIdx.x / LPR, seg = threadIdx.x % LPR;
        u32x4_t r[NP];
#pragma unroll
        for (int s = 0; s < NP; ++s)
            if (r0 + RPB * s < C)
                r[s] = *reinterpret_cast<const u32x4_t *>(x.k + (size_t)x.tok_clamped(c, r0 + RPB * s) * x.rs + 16 * seg);
#pragma unroll
        for (int s = 0; s < NP; ++s) {
            const int row = r0 + RPB * s;
            if (row < C) {
                const float sk = put_seg<IO, PRO>(&sm.Ks[row][SC * seg], r[s]);
                if constexpr (PRO) {
                    const float t = group_sum<LPR>(sk);
                    if (seg == 0) sm.rk[row] = inv_norm(t);
                }
            }
        }
    }
    __syncthreads();

    // 2. the Gram products of the diagonal 32x32 blocks of A (waves 0, 1) and of
    //    the off-diagonal block A(1,0) (wave 2), then the epilogues with their
    //    diagonal 16x16 Tm blocks
    constexpr int NKS = DK / 16;
    const int l32 = lane & 31, hi = lane >> 5, l16 = lane & 15, g16 = lane >> 4;
    const uint16_t *ka = &sm.Ks[l32][8 * hi];
    const uint16_t *kb = &sm.Ks[32 + l32][8 * hi];
    f32x16_t g0 = zero16();
    if (wid < 2) {
        const uint16_t *kk = wid == 0 ? ka : kb;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const bf16x8_t r = lds16(kk + 16 * s);
            g0 = mfma32(r, r, g0);
        }
    } else if (wid == 2) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) g0 = mfma32(lds16(ka + 16 * s), lds16(kb + 16 * s), g0);
    } else {
        // wave 3: the gate vectors (the prologue's factors need every row's norm)
        const float rk = PRO ? sm.rk[lane] : 1.f;
        float bt, l2;
        gate_in<PRO>(xb, xa, bt, l2);
        const GateVals gv = gate_values<PRO>(lane, x.ntok(c), bt, l2, rk);
        sm.g[lane] = gv.g;
        sm.gk[lane] = gv.gk;
        sm.bk[lane] = gv.bk;
        sm.xf[lane] = gv.xf;
        // the chunk's gate record, one 16-byte entry per token, contiguous for chunk_kernel
        const size_t gi = ((size_t)((dir * p.B + b) * p.H + h) * p.nchunks + c) * C + lane;
        if constexpr (PRO) static_cast<float4 *>(p.grec)[gi] = make_float4(bt, l2, rk, 0.f);
        else static_cast<float2 *>(p.grec)[gi] = make_float2(bt, l2);
    }
    __syncthreads();  // K is read; Tm and A overwrite it
    if (wid < 2) a_diag_block(sm, g0, wid, lane);
    else if (wid == 2) a_cross_block(sm, g0, lane);
    __syncthreads();

    // 3. the off-diagonal 16x16 blocks of Tm, one block column per wave
    if (wid == 0) tm_column<0>(sm.Tb, sm.Ab, l16, g16);
    else if (wid == 1) tm_column<1>(sm.Tb, sm.Ab, l16, g16);
    else if (wid == 2) tm_column<2>(sm.Tb, sm.Ab, l16, g16);
    __syncthreads();

    // 4. the six operand blocks, one 16-byte store per lane (8 bytes for operands 0
    //    and 3, whose second halves are zero)
    uint16_t *dst = p.tm + ((size_t)((dir * p.B + b) * p.H + h) * p.nchunks + c) * TM_ELEMS;
    for (int o = wid; o < TM_OPS; o += 4) {
        const int nb = o < 2 ? o : 2 + (o - 2) / 2;
        const int ks = o < 2 ? 0 : (o - 2) & 1;
        const uint16_t *row = &sm.Tb[16 * nb + l16][32 * ks + 4 * g16];
        const uint2 lo = *reinterpret_cast<const uint2 *>(row);
        if (tm_half(o)) {
            *reinterpret_cast<uint2 *>(dst + tm_off(o) + (size_t)lane * 4) = lo;
        } else {
            const uint2 up = *reinterpret_cast<const uint2 *>(row + 16);
            *reinterpret_cast<uint4 *>(dst + tm_off(o) + (size_t)lane * 8) = make_uint4(lo.x, lo.y, up.x, up.y);
        }
    }
}

// =============================================================================
// chunk_kernel: the chunks of a head in order.
// =============================================================================
struct ChunkParams {
    const char *q, *k, *v;
    long long qk_ts, qk_bs, v_ts, v_bs;  // element strides between tokens / batch elements
    const void *grec;                    // gate records written by tm_kernel
    const float *state_in;
    float *state_out;
    void *out;
    float *partial, *partial_rev;
    const uint16_t *tm;
    long long T;
    long long state_dir_stride;  // elements between the two directions' states (both_dirs)
    int B, H, dv, ntile, nblk_dir;
    int reverse, out_mode, xcd_remap, both_dirs;
    int c0, c1;                  // the chunks of this launch: [c0, c1)
    float scale;
    // SWEEP_SEG only: block row y walks segment s = seg_base + y, chunks
    // [s seg_len, min(n, (s + 1) seg_len)); its state_out is y seg_state_stride
    // elements further on.  seg_zero_start: segments s > 0 start from zero (else
    // every segment starts from state_in).  seg0_store: segment 0 stores out, the
    // others store bf16 rows into seg_out (else every run stores into seg_out).
    int seg_len, seg_base, seg_zero_start, seg0_store;
    long long seg_state_stride;
    int seg_rows;  // block rows (y) this parameter set covers; the launch's other rows use the second set
    int state_out_t;  // state_out written transposed ([d_k][d_v] per head)
    void *seg_out;    // SWEEP_SEG: bf16 [B,T,H,d_v] rows of every run but segment 0's own
};

template <int DK>
struct __align__(16) Smem {
    // Row pitch of K, Q and S: reads of one 16-byte segment per lane from 16
    // consecutive rows (and the chain's transposed reads of K) spread over the banks.
    static constexpr int LKK = DK + 16;
    uint16_t Ks[2][C][LKK];  // K, token-major (chunk parity)
    uint16_t Qs[2][C][LKK];  // Q, token-major
    float bVt[2][DVT][C + 4];  // b_t v_t of the d_v tile, fp32, [d_v][bv_slot(d_v, token)]
    uint16_t Sb[2][DVT][LKK];  // bf16 state tile at the start of a chunk, [d_v][d_k]
    uint16_t Nt[2][DVT][LC];  // N^T (chunk parity), keys in sdk order
    float g[3][C];           // gate vectors, chunk mod 3 (GateVals)
    float gk[3][C];
    float bet[3][C];
    float gam[3][C];
    float bg[3][C];
    float glast[3][C];
    // Output staging, one 16-query tile per output wave and query block.  The
    // pitch of 36 floats keeps both the writes (16-byte columns of 16 rows) and the
    // row-major reads free of bank conflicts.
    static constexpr int LOT = DVT + 4;
    float Ot[4][16][LOT];
    // Tm of a chunk in the chain's operand order (chunk parity), staged by the gate wave
    uint16_t Tms[2][TM_LDS_ELEMS];
};

// OUT_ADD_PARTIAL only: the other direction's outputs of a chunk's tokens, widened
// to fp32 (chunk parity), staged by the gate wave, in dynamic LDS that only
// launches of that mode request.
constexpr int LPT = DVT + 4;
typedef float PartTile[C][LPT];
constexpr size_t PART_LDS_BYTES = 2 * sizeof(PartTile);
__device__ __forceinline__ PartTile *part_tiles() {
    extern __shared__ __align__(16) float dyn_lds[];
    return reinterpret_cast<PartTile *>(dyn_lds);
}

// Column d of bVt holds token t at position t + 16 (d / 8), mod 64: the four
// 8-column groups that one store instruction writes then start on different
// banks, and runs of 4 aligned tokens stay aligned.
__device__ __forceinline__ int bv_slot(int d, int t) { return (t + 16 * (d >> 3)) & 63; }

// ---- waves 0, 1: the state chain, 16 d_v columns each ------------------------
// Lane l = 16 g + r.  A 16x16 accumulator block holds rows 4g .. 4g + 3 of column
// r.  Two blocks side by side form one k-step of a B operand with the k index
// permuted: slot s < 4 is row 4g + s of the first block, slot s >= 4 row
// 4g + s - 4 of the second.  The matching A operand row r holds, in lane group
// g, columns 4g .. 4g + 3 of the first 16 and of the second 16 of its 32.
//
// The d_k axis of S is stored permuted the same way in reverse: row 4g + m of
// S^T block db (32-wide group kd = db / 2, h = db % 2) is d_k index
// 32 kd + 8 g + 4 h + m, so that the eight d_k of one k-step of X = K S^T are
// consecutive and the A operand is a single 16-byte read of a K row.
__device__ __forceinline__ int sdk(int db, int g4) { return 32 * (db >> 1) + 8 * g4 + 4 * (db & 1); }
struct TmOps {
    bf16x8_t o[TM_OPS];
};

template <int DK>
struct Chain16 {
    static constexpr int NKS = DK / 32;  // k-steps of X over d_k
    static constexpr int NDB = DK / 16;  // 16-row blocks of S^T
    f32x4_t sacc[NDB];                   // S^T rows 16 db + 4g + 0..3, column r
    bf16x8_t sop[NKS];                   // bf16 S^T as the B operand of X = K S^T

    __device__ __forceinline__ void publish_state(Smem<DK> &sm, int slot, int col, int g4) {
        uint2 w[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            w[db] = pack4(sacc[db][0], sacc[db][1], sacc[db][2], sacc[db][3]);
            *reinterpret_cast<uint2 *>(&sm.Sb[slot][col][sdk(db, g4)]) = w[db];
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) sop[ks] = join_u2(w[2 * ks], w[2 * ks + 1]);
    }

    __device__ __forceinline__ void init(const ChunkParams &p, Smem<DK> &sm, size_t sbase, int col, int g4, int c0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            sacc[db] = zero4();
            if (p.state_in) {
                const float4 s4 = *reinterpret_cast<const float4 *>(p.state_in + sbase + sdk(db, g4));
                sacc[db][0] = s4.x; sacc[db][1] = s4.y; sacc[db][2] = s4.z; sacc[db][3] = s4.w;
            }
        }
        publish_state(sm, c0 & 1, col, g4);  // the slot of the launch's first chunk
    }

    // K^T as the A operands of the update: row r of block db is d_k
    // sdk(db, r / 4) + r % 4, tokens 32 ks + 4g + (0..3, 16..19), read transposed
    // from the token-major K (lane 4s + j of a 16-lane group addresses token
    // 4g + s, columns sdk(db, j) .. + 3).  They do not depend on N, so they are
    // read before N is formed.
    struct KtOps {
        bf16x8_t o[2 * NDB];
    };
    __device__ __forceinline__ KtOps load_kt(const Smem<DK> &sm, int s2, int lane) const {
        constexpr int LK = Smem<DK>::LKK;
        const int g4 = lane >> 4, r16 = lane & 15;
        const uint16_t *kt = &sm.Ks[s2][4 * g4 + (r16 >> 2)][8 * (r16 & 3)];
        KtOps k;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const uint16_t *p0 = kt + 32 * (db >> 1) + 4 * (db & 1);
            k.o[2 * db] = join(lds_tr(p0), lds_tr(p0 + 16 * LK));
            k.o[2 * db + 1] = join(lds_tr(p0 + 32 * LK), lds_tr(p0 + 48 * LK));
        }
        return k;
    }

    // First half of chunk c: X, R, N, and S scaled by the chunk's decay; this
    // wave's columns of N^T published; the K^T operands read.
    __device__ __forceinline__ void step_n(Smem<DK> &sm, int c, int lane, int col, const TmOps &tm,
                                           f32x4_t (&nacc)[4], KtOps &kt) {
        const int g4 = lane >> 4, r16 = lane & 15;
        const int s2 = c & 1, s3 = c % 3;
        // X = K S^T, four 16-token blocks; k-step ks = d_k 32 ks + 8 g .. + 7
        f32x4_t xacc[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                xacc[tb] = mfma16k32(lds16(&sm.Ks[s2][16 * tb + r16][32 * ks + 8 * g4]), sop[ks], xacc[tb]);
        }
        // the decay of S over the chunk, off the X -> N -> S path
        const float gl = sm.gam[s3][C - 1];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int m = 0; m < 4; ++m) sacc[db][m] *= gl;
        // R = diag(b) V - diag(b gam) X
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const float4 bv = *reinterpret_cast<const float4 *>(&sm.bVt[s2][col][bv_slot(col, 16 * tb + 4 * g4)]);
            const float4 bgm = *reinterpret_cast<const float4 *>(&sm.bg[s3][16 * tb + 4 * g4]);
            xacc[tb][0] = fmaf(-bgm.x, xacc[tb][0], bv.x);
            xacc[tb][1] = fmaf(-bgm.y, xacc[tb][1], bv.y);
            xacc[tb][2] = fmaf(-bgm.z, xacc[tb][2], bv.z);
            xacc[tb][3] = fmaf(-bgm.w, xacc[tb][3], bv.w);
        }
        const bf16x8_t rop0 = join(pack4s(xacc[0]), pack4s(xacc[1]));
        const bf16x8_t rop1 = join(pack4s(xacc[2]), pack4s(xacc[3]));
        kt = load_kt(sm, s2, lane);
        // N = Tm R (Tm lower triangular: token blocks 0, 1 need keys 0-31 only)
        nacc[0] = mfma16k32(tm.o[tm_op(0, 0)], rop0, zero4());
        nacc[1] = mfma16k32(tm.o[tm_op(1, 0)], rop0, zero4());
        nacc[2] = mfma16k32(tm.o[tm_op(2, 0)], rop0, zero4());
        nacc[3] = mfma16k32(tm.o[tm_op(3, 0)], rop0, zero4());
        nacc[2] = mfma16k32(tm.o[tm_op(2, 1)], rop1, nacc[2]);
        nacc[3] = mfma16k32(tm.o[tm_op(3, 1)], rop1, nacc[3]);
        // publish this wave's columns of N^T for the output waves, keys in the
        // permuted order of the state's d_k (sdk)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
            *reinterpret_cast<uint2 *>(&sm.Nt[s2][col][sdk(nb, g4)]) =
                pack4(nacc[nb][0], nacc[nb][1], nacc[nb][2], nacc[nb][3]);
    }

    // Second half: S^T <- (gam_{C-1} S^T) + K^T N~, N~ = diag(G_{C-1,.}) N.
    __device__ __forceinline__ void step_s(Smem<DK> &sm, int c, int lane, int col, f32x4_t (&nacc)[4],
                                           const KtOps &kt) {
        const int g4 = lane >> 4;
        const int s3 = c % 3;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const float4 gl = *reinterpret_cast<const float4 *>(&sm.glast[s3][16 * nb + 4 * g4]);
            nacc[nb][0] *= gl.x; nacc[nb][1] *= gl.y; nacc[nb][2] *= gl.z; nacc[nb][3] *= gl.w;
        }
        const bf16x8_t nop0 = join(pack4s(nacc[0]), pack4s(nacc[1]));
        const bf16x8_t nop1 = join(pack4s(nacc[2]), pack4s(nacc[3]));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            sacc[db] = mfma16k32(kt.o[2 * db], nop0, sacc[db]);
            sacc[db] = mfma16k32(kt.o[2 * db + 1], nop1, sacc[db]);
        }
        publish_state(sm, (c + 1) & 1, col, g4);
    }

    __device__ __forceinline__ void finish(const ChunkParams &p, size_t sbase, int g4) {
        if (!p.state_out) return;
        if (p.state_out_t) {
            // transposed: element (row r, column j) of the head's d_v x d_k state goes to
            // column r of row j (d_v = d_k for the runs that ask for it)
            const size_t head = sbase / ((size_t)p.dv * DK);
            const int r = (int)(sbase / DK - head * p.dv);
            float *dst = p.state_out + head * p.dv * DK + r;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int m = 0; m < 4; ++m) dst[(size_t)(sdk(db, g4) + m) * p.dv] = sacc[db][m];
            return;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<float4 *>(p.state_out + sbase + sdk(db, g4)) =
                make_float4(sacc[db][0], sacc[db][1], sacc[db][2], sacc[db][3]);
    }
};

// Tm operands of chunk c from its LDS slot.
__device__ __forceinline__ TmOps lds_tm(const uint16_t *slot, int lane) {
    TmOps t;
#pragma unroll
    for (int o = 0; o < TM_OPS; ++o) t.o[o] = lds16(slot + (size_t)o * 512 + (size_t)lane * 8);
    return t;
}
// Tm operands of chunk c as stored in memory (operands 0 and 3 halved), loaded by
// the gate wave (clamped into range: the load is unconditional and its result
// unused past the last chunk) and written to the LDS slot in full.
struct TmMem {
    uint2 h[2];  // operands 0 and 3
    uint4 f[4];  // operands 1, 2, 4, 5
};
__device__ __forceinline__ void store_tm(uint16_t *slot, const TmMem &t, int lane) {
#pragma unroll
    for (int o = 0; o < TM_OPS; ++o) {
        const int i = o < 3 ? o - 1 : o - 2;
        const uint4 v = tm_half(o) ? make_uint4(t.h[o == 3].x, t.h[o == 3].y, 0u, 0u) : t.f[i];
        *reinterpret_cast<uint4 *>(slot + (size_t)o * 512 + (size_t)lane * 8) = v;
    }
}
__device__ __forceinline__ TmMem load_tm(const uint16_t *tm_head, int c, int n, int lane) {
    const int cc = c < n ? c : n - 1;  // n: one past the last chunk of the launch
    const uint16_t *src = tm_head + (size_t)cc * TM_ELEMS;
    TmMem t;
#pragma unroll
    for (int o = 0; o < TM_OPS; ++o) {
        if (tm_half(o)) t.h[o == 3] = *reinterpret_cast<const uint2 *>(src + tm_off(o) + (size_t)lane * 4);
        else t.f[o < 3 ? o - 1 : o - 2] = *reinterpret_cast<const uint4 *>(src + tm_off(o) + (size_t)lane * 8);
    }
    return t;
}

// ---- waves 2, 3: outputs of chunk c ------------------------------------------
// For a block of 16 queries q: O^T (d_v x queries) = gam .* (S Q_q^T) + N^T P_q^T,
// with P_q^T (keys x queries) = K Q_q^T .* G for keys j <= query i, as 16x16x32
// products: S Q^T and K Q^T read rows of S, K and Q with 8 consecutive d_k per
// lane (one 16-byte read); N^T P^T takes two P accumulator blocks side by side as
// its B operand (the permuted k order of the chain) and N^T, whose keys the
// chain stores in the matching order, as its A operand.  Query blocks {0, 3} and
// {1, 2} need five key blocks each, so the two waves do the same work.
// With the prologue, rq is set to this lane's query's inverse L2 norm.  The lane
// holds d_k / 4 values of its query r in the Q operands (the other lanes of the
// query are r + 16, r + 32, r + 48): it sums their squares with v_dot2_f32_bf16
// (bf16 products are exact in fp32), adds the partner lanes' sums with
// v_permlane16_swap and v_permlane32_swap, and takes v_rsq_f32 of max(sum,
// 1e-24), which is 1 / max(||q||, 1e-12) to within an ulp.  These are short VALU
// chains: the first version formed diag(Q Q^T) with four chained MFMAs and read
// it back through ds_bpermute, which cost 8% of the call.
template <int DK, bool PRO>
__device__ __forceinline__ void out_products(const Smem<DK> &sm, int s2, int s3, int q, int lane,
                                             const bf16x8_t (&sa)[2][DK / 32], f32x4_t (&o)[2], f32x4_t (&pk)[4],
                                             float &rq) {
    constexpr int NKS = DK / 32;
    const int g4 = lane >> 4, r16 = lane & 15;
    bf16x8_t qo[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qo[ks] = lds16(&sm.Qs[s2][16 * q + r16][32 * ks + 8 * g4]);
    if constexpr (PRO) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4_t w;
            __builtin_memcpy(&w, &qo[ks], 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t we = w[e];
                bf16x2_t x;
                __builtin_memcpy(&x, &we, 4);
                if (e & 1) d1 = __builtin_amdgcn_fdot2_f32_bf16(x, x, d1, false);
                else d0 = __builtin_amdgcn_fdot2_f32_bf16(x, x, d0, false);
            }
        }
        float d = d0 + d1;
        const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d), __float_as_uint(d), false, false);
        d = __uint_as_float(x16[0]) + __uint_as_float(x16[1]);  // lanes l and l ^ 16
        const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(d), __float_as_uint(d), false, false);
        d = __uint_as_float(x32[0]) + __uint_as_float(x32[1]);  // and l ^ 32: all four lanes of query r16
        rq = __builtin_amdgcn_rsqf(fmaxf(d, 1e-24f));
    }
    o[0] = zero4();
    o[1] = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) pk[kb] = zero4();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        o[0] = mfma16k32(sa[0][ks], qo[ks], o[0]);
        o[1] = mfma16k32(sa[1][ks], qo[ks], o[1]);
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (kb > q) break;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            pk[kb] = mfma16k32(lds16(&sm.Ks[s2][16 * kb + r16][32 * ks + 8 * g4]), qo[ks], pk[kb]);
    }
    // gam of the query column on S Q^T; 2^{g_i - gk_j} and the causal mask on
    // P^T (gk = g without the prologue)
    const int qi = 16 * q + r16;
    const float gq = sm.gam[s3][qi];
    const float gi = sm.g[s3][qi];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        o[0][m] *= gq;
        o[1][m] *= gq;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        if (kb > q) break;
        const float4 gj = *reinterpret_cast<const float4 *>(&sm.gk[s3][16 * kb + 4 * g4]);
        const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float v = pk[kb][m] * exp2_fast(gi - gjv[m]);
            pk[kb][m] = (kb < q || 4 * g4 + m <= r16) ? v : 0.f;
        }
    }
}

template <int DK>
__device__ __forceinline__ void out_pn(const Smem<DK> &sm, int slot, int q, int lane, f32x4_t (&o)[2],
                                       const f32x4_t (&pk)[4]) {
    const int g4 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (2 * t > q) break;
        const bf16x8_t b = join(pack4s(pk[2 * t]), 2 * t + 1 <= q ? pack4s(pk[2 * t + 1]) : pack4s(zero4()));
        o[0] = mfma16k32(lds16(&sm.Nt[slot][r16][32 * t + 8 * g4]), b, o[0]);
        o[1] = mfma16k32(lds16(&sm.Nt[slot][16 + r16][32 * t + 8 * g4]), b, o[1]);
    }
}

// Stores of a 16-query block.  In the accumulators lane (g, r) holds query r,
// columns 4g .. 4g + 3 and 16 + 4g .. + 3, so 16 consecutive lanes address 16
// different output rows and every lane of a store instruction touches its own
// 64-byte segment.  The block goes through a wave-private LDS tile instead and is
// read back row-major, so that the lanes of one store instruction write whole
// 64-byte row segments (4 lanes per row for bf16 out, 8 per row for the fp32
// partials): a quarter of the address work of the per-lane stores.
__device__ __forceinline__ void wave_lds_sync() {
    // ds instructions of one wave execute in order; this only keeps the compiler
    // from moving the reads above the writes of other lanes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int DK, bool PRO, bool ADD>
__device__ __forceinline__ void out_store(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int c, int q,
                                          int slot, int lane, const f32x4_t (&o)[2], float rq, void *out_b,
                                          float *part_b) {
    const int g4 = lane >> 4, r16 = lane & 15;
    const float sc = PRO ? p.scale * rq : p.scale;
    float(*tile)[Smem<DK>::LOT] = sm.Ot[slot];
#pragma unroll
    for (int dvb = 0; dvb < 2; ++dvb)
        *reinterpret_cast<float4 *>(&tile[r16][16 * dvb + 4 * g4]) =
            make_float4(o[dvb][0] * sc, o[dvb][1] * sc, o[dvb][2] * sc, o[dvb][3] * sc);
    wave_lds_sync();
    const int n = x.ntok(c);
    if (p.out_mode == OUT_PARTIAL) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = (lane >> 3) + 8 * i, col = 4 * (lane & 7);
            const float4 v = *reinterpret_cast<const float4 *>(&tile[row][col]);
            // non-temporal: the combine reads each partial once, much later
            if (16 * q + row < n)
                __builtin_nontemporal_store(u32x4_t{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                                    __float_as_uint(v.w)},
                                            reinterpret_cast<u32x4_t *>(part_b + (size_t)x.tok(c, 16 * q + row) * x.rso +
                                                                        col));
        }
    } else {
        const int row = lane >> 2, col = 8 * (lane & 3);
        float4 a = *reinterpret_cast<const float4 *>(&tile[row][col]);
        float4 b = *reinterpret_cast<const float4 *>(&tile[row][col + 4]);
        if (16 * q + row < n) {
            if constexpr (ADD) {
                // the other direction's fp32 output of this token (written by the
                // previous launch, staged in LDS): the sum is rounded once
                const PartTile &pt = part_tiles()[c & 1];
                const float4 u = *reinterpret_cast<const float4 *>(&pt[16 * q + row][col]);
                const float4 w = *reinterpret_cast<const float4 *>(&pt[16 * q + row][col + 4]);
                a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
                b.x += w.x; b.y += w.y; b.z += w.z; b.w += w.w;
            }
            const uint2 lo = pack4(a.x, a.y, a.z, a.w), hi = pack4(b.x, b.y, b.z, b.w);
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out_b) + (size_t)x.tok(c, 16 * q + row) * x.rso +
                                       col) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }
}

// Wave W of the two output waves: query blocks {0, 3} (W = 0) or {1, 2} (W = 1).
// The products of chunk c are formed in period c and held in registers; N^T P^T
// and the stores follow at the start of period c + 1, when N^T of chunk c is in
// its LDS slot (written by the chain in period c, visible after the barrier).
struct OutRegs {
    f32x4_t oa[2], ob[2], pa[4], pb[4];
    float ra = 1.f, rb = 1.f;  // prologue: inverse q norms of the lane's query in blocks QA, QB
};

template <int DK, int W, bool PRO>
__device__ __forceinline__ void out_products_step(Smem<DK> &sm, int c, int lane, OutRegs &r) {
    constexpr int NKS = DK / 32;
    constexpr int QA = W ? 1 : 0, QB = W ? 2 : 3;
    const int g4 = lane >> 4, r16 = lane & 15;
    const int s2 = c & 1, s3 = c % 3;
    bf16x8_t sa[2][NKS];  // rows of S (two 16-column blocks of d_v) as A operands
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        sa[0][ks] = lds16(&sm.Sb[s2][r16][32 * ks + 8 * g4]);
        sa[1][ks] = lds16(&sm.Sb[s2][16 + r16][32 * ks + 8 * g4]);
    }
    out_products<DK, PRO>(sm, s2, s3, QA, lane, sa, r.oa, r.pa, r.ra);
    out_products<DK, PRO>(sm, s2, s3, QB, lane, sa, r.ob, r.pb, r.rb);
}

template <int DK, int W, bool PRO, bool ADD>
__device__ __forceinline__ void out_finish_step(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int c,
                                                int lane, OutRegs &r, void *out_b, float *part_b) {
    constexpr int QA = W ? 1 : 0, QB = W ? 2 : 3;
    out_pn(sm, c & 1, QA, lane, r.oa, r.pa);
    out_pn(sm, c & 1, QB, lane, r.ob, r.pb);
    out_store<DK, PRO, ADD>(x, sm, p, c, QA, 2 * W, lane, r.oa, r.ra, out_b, part_b);
    out_store<DK, PRO, ADD>(x, sm, p, c, QB, 2 * W + 1, lane, r.ob, r.rb, out_b, part_b);
}

// Period c of an output wave: finish chunk c - 1, then the products of chunk c.
template <int DK, int W, bool PRO, bool ADD>
__device__ __forceinline__ void output_period(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int c, int lane,
                                              OutRegs &r, void *out_b, float *part_b) {
    const bool fin = x.has(c - 1), run = x.has(c);
    if (fin && run) {
        out_finish_step<DK, W, PRO, ADD>(x, sm, p, c - 1, lane, r, out_b, part_b);
        out_products_step<DK, W, PRO>(sm, c, lane, r);
    } else if (run) {
        out_products_step<DK, W, PRO>(sm, c, lane, r);
    } else if (fin) {
        out_finish_step<DK, W, PRO, ADD>(x, sm, p, c - 1, lane, r, out_b, part_b);
    }
}

// The output waves' walk over the launch's periods.
template <int DK, int W, bool PRO, bool ADD>
__device__ __forceinline__ void output_role(const Ctx &x, Smem<DK> &sm, const ChunkParams &p, int lane,
                                            void *out_b, float *part_b) {
    OutRegs r;
    __syncthreads();
    for (int it = x.c0 - 2; it < x.c1 + 1; it += 2) {
        output_period<DK, W, PRO, ADD>(x, sm, p, it, lane, r, out_b, part_b);
        __syncthreads();
        output_period<DK, W, PRO, ADD>(x, sm, p, it + 1, lane, r, out_b, part_b);
        __syncthreads();
    }
}

// ---- waves 4, 5: K and Q of a chunk, row-coalesced -----------------------------
// 16 bytes per lane (8 bf16 or 16 FP8 columns), DK / seg_cols lanes per row, so
// every load instruction reads whole rows; stored to LDS as bf16.
template <int DK, int IO>
struct Rows64 {
    static constexpr int LPR = DK / seg_cols<IO>();  // lanes per row
    static constexpr int RPL = 64 / LPR;             // rows per load
    static constexpr int NLD = C / RPL;              // loads per chunk
    u32x4_t r[NLD];
};

// Loads are unconditional per lane: rows past the end of a final short chunk
// re-read token n-1 (finite data; those tokens carry b = 0 and a = 1, so every
// product they enter is multiplied by 0 or never stored).
template <int DK, int IO>
__device__ __forceinline__ Rows64<DK, IO> load_rows(const char *base, const Ctx &x, int c, int lane) {
    using RB = Rows64<DK, IO>;
    RB d;
    const ChunkRows cr = chunk_rows(x, base, c, x.rs);
    const int r0 = lane / RB::LPR;
    const int off = 16 * (lane % RB::LPR);
#pragma unroll
    for (int s = 0; s < RB::NLD; ++s) d.r[s] = *reinterpret_cast<const u32x4_t *>(cr.row(r0 + RB::RPL * s) + off);
    return d;
}
template <int DK, int PITCH, int IO>
__device__ __forceinline__ void store_rows(uint16_t (*dst)[PITCH], const Rows64<DK, IO> &blk, int lane) {
    using RB = Rows64<DK, IO>;
    const int r0 = lane / RB::LPR;
    const int col = seg_cols<IO>() * (lane % RB::LPR);
#pragma unroll
    for (int s = 0; s < RB::NLD; ++s) put_seg<IO, false>(&dst[r0 + RB::RPL * s][col], blk.r[s]);
}

// ---- waves 6, 7: gate vectors; V tiles -----------------------------------------
struct GateRegs {
    float4 r;  // the token's gate record from tm_kernel: b, log2 a, 1/||k|| (1 without the prologue)
};

// The chunk's V tile (64 tokens x 32 d_v), row-coalesced: in w[s], lane l holds
// token 16 s + l / 4, d_v columns 8 (l % 4) .. + 7 (16 bytes of bf16 or 8 of FP8).
template <int IO>
struct VRow {
    u32x4_t w[4];  // bf16: 8 columns; FP8: 8 columns in w[s][0..1]
};
template <int IO>
__device__ __forceinline__ VRow<IO> load_v(const Ctx &x, int c, int lane) {
    VRow<IO> d;
    const ChunkRows cr = chunk_rows(x, x.v, c, x.rsv);
    constexpr int SEG = 8 * io_in_bytes(IO);  // bytes of 8 columns
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const char *src = cr.row(16 * s + (lane >> 2)) + SEG * (lane & 3);
        if constexpr (IO == IO_FP8) {
            const u32x2_t u = *reinterpret_cast<const u32x2_t *>(src);
            d.w[s] = u32x4_t{u[0], u[1], 0u, 0u};
        } else {
            d.w[s] = *reinterpret_cast<const u32x4_t *>(src);
        }
    }
    return d;
}
// One record per lane from a contiguous run per chunk (1 KiB with the prologue, else
// 512 bytes; the strided [B, T, H] gates were read, activated and clamped by
// tm_kernel).  Unconditional (c is clamped into range by the caller), so that the
// count of loads in flight is the same on every path.
template <bool PRO>
__device__ __forceinline__ void load_gates(const Ctx &x, int c, int lane, GateRegs &g) {
    const size_t i = (size_t)c * C + lane;
    if constexpr (PRO) {
        g.r = static_cast<const float4 *>(x.grec)[i];
    } else {
        const float2 v = static_cast<const float2 *>(x.grec)[i];
        g.r = make_float4(v.x, v.y, 1.f, 0.f);
    }
}

// The other direction's outputs of a chunk's tokens for this block's 32 d_v columns,
// bf16 rows written by the first launch: lane l holds row 8 s + l / 8, columns
// 4 (l % 8) .. + 3 (rows past the end of a short final chunk re-read its last token;
// they are never used).  Widened to fp32 when staged.
struct PartRows {
    uint2 r[8];
};
__device__ __forceinline__ PartRows load_part(const Ctx &x, const uint16_t *other_b, int c, int lane) {
    PartRows d;
    const int nt = x.ntok(c);
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_) {
        const int j = 8 * s_ + (lane >> 3);
        const uint16_t *src = other_b + (size_t)x.tok(c, j < nt ? j : nt - 1) * x.rso + 4 * (lane & 7);
        d.r[s_] = *reinterpret_cast<const uint2 *>(src);
    }
    return d;
}
__device__ __forceinline__ void store_part(int c, const PartRows &d, int lane) {
    PartTile &pt = part_tiles()[c & 1];
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_)
        *reinterpret_cast<float4 *>(&pt[8 * s_ + (lane >> 3)][4 * (lane & 7)]) =
            make_float4(bf16_lo(d.r[s_].x), bf16_hi(d.r[s_].x), bf16_lo(d.r[s_].y), bf16_hi(d.r[s_].y));
}

template <int DK, bool PRO>
__device__ __forceinline__ void gates_store(const Ctx &x, Smem<DK> &sm, int c, int lane, const GateRegs &gr) {
    const GateVals v = gate_values<PRO>(lane, x.ntok(c), gr.r.x, gr.r.y, gr.r.z);
    const int s3 = c % 3;
    sm.g[s3][lane] = v.g;
    sm.gk[s3][lane] = v.gk;
    sm.bet[s3][lane] = v.bet;
    sm.gam[s3][lane] = v.gam;
    sm.bg[s3][lane] = v.bg;
    sm.glast[s3][lane] = v.glast;
}

template <int DK, int IO>
__device__ __forceinline__ void store_bv(Smem<DK> &sm, int c, const VRow<IO> &v, int lane) {
    const int d0 = 8 * (lane & 3);
#pragma unroll
    for (int s_ = 0; s_ < 4; ++s_) {
        const int t = 16 * s_ + (lane >> 2);
        const float bt = sm.bet[c % 3][t];
        float *col = &sm.bVt[c & 1][d0][bv_slot(d0, t)];
        float vv[8];
        if constexpr (IO == IO_FP8) {
            fp8x4_to_f32(v.w[s_][0], vv);
            fp8x4_to_f32(v.w[s_][1], vv + 4);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vv[2 * e] = bf16_lo(v.w[s_][e]);
                vv[2 * e + 1] = bf16_hi(v.w[s_][e]);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) col[e * (C + 4)] = bt * vv[e];
    }
}

// SWEEP_ALL: one launch walks every chunk.  SWEEP_FIRST / SWEEP_SECOND: the first
// ([0, c1)) and second ([c0, n), out_mode OUT_ADD_PARTIAL) launches of the
// bidirectional form's split sweep.  SWEEP_SEG: the token segments of the
// segment-parallel causal form, one per block row.
enum Sweep : int { SWEEP_ALL = 0, SWEEP_FIRST = 1, SWEEP_SECOND = 2, SWEEP_SEG = 3 };
template <int DK, int IO, bool PRO, int SW>
__global__ __launch_bounds__(NT) void chunk_kernel(ChunkParams p_arg, ChunkParams p_alt) {
    constexpr bool ADD = SW == SWEEP_SECOND;
    ChunkParams p = p_arg;
    int seg = 0;
    if constexpr (SW == SWEEP_SEG) {
        // block rows [0, seg_rows) use the first parameter set, the rest the second (the
        // identity runs); a set with fewer blocks per row leaves the surplus at once
        int y = (int)blockIdx.y;
        if (y >= p_arg.seg_rows) {
            p = p_alt;
            y -= p_arg.seg_rows;
        }
        if ((int)blockIdx.x >= p.nblk_dir) return;
        seg = p.seg_base + y;
        if (p.state_out) p.state_out += (size_t)y * p.seg_state_stride;
        if (p.seg_zero_start && seg > 0) p.state_in = nullptr;
        if (!(p.seg0_store && seg == 0)) p.out = p.seg_out;
        p.out_mode = OUT_STORE;
    }
    constexpr int ES = io_in_bytes(IO);
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
    x.c0 = SW == SWEEP_SECOND || SW == SWEEP_FIRST ? p.c0 : SW == SWEEP_SEG ? seg * p.seg_len : 0;
    x.c1 = SW == SWEEP_FIRST ? p.c1 : x.nchunks;
    if constexpr (SW == SWEEP_SEG) x.c1 = min(x.nchunks, x.c0 + p.seg_len);
    x.rs = (int)(p.qk_ts * ES);
    x.rsv = (int)(p.v_ts * ES);
    x.rso = p.H * p.dv;
    x.H = p.H;
    x.reverse = p.reverse ^ dir;
    const size_t tok0 = (size_t)b * p.T * p.H + h;  // (b, token 0, h) of the [B, T, H] gates and out rows
    const size_t qk0 = ((size_t)b * p.qk_bs + (size_t)h * DK) * ES;
    x.q = p.q + qk0;
    x.k = p.k + qk0;
    x.v = p.v + ((size_t)b * p.v_bs + (size_t)h * p.dv + dv0) * ES;
    x.beta = x.decay = nullptr;  // the gates arrive as tm_kernel's records (x.grec)
    const int n = x.nchunks;
    {
        const size_t g0 = (size_t)((dir * p.B + b) * p.H + h) * n * C;
        x.grec = PRO ? static_cast<const void *>(static_cast<const float4 *>(p.grec) + g0)
                     : static_cast<const void *>(static_cast<const float2 *>(p.grec) + g0);
    }

    // Every role walks the same periods it = c0 - 2 .. c1 (the last one finishes
    // the outputs of chunk c1 - 1), two per loop trip so that register sets
    // alternate at compile time, with one barrier each.
    const int c0 = x.c0, c1 = x.c1;
    // out is bf16 for every input type this kernel takes.  The first launch of the
    // bidirectional split stores each direction's outputs the same way, as bf16 rows of
    // that direction's partial buffer, which the second launch reads back.
    void *out_b = reinterpret_cast<uint16_t *>(p.out) + tok0 * p.dv + dv0;
    if constexpr (SW == SWEEP_FIRST)
        out_b = reinterpret_cast<uint16_t *>(dir ? p.partial_rev : p.partial) + tok0 * p.dv + dv0;
    float *part = dir ? p.partial_rev : p.partial;
    float *part_b = part ? part + tok0 * p.dv + dv0 : nullptr;
    // OUT_ADD_PARTIAL: the other direction's bf16 rows
    const uint16_t *other = reinterpret_cast<const uint16_t *>(dir ? p.partial : p.partial_rev);
    const uint16_t *other_b = other ? other + tok0 * p.dv + dv0 : nullptr;
    // The chain and output waves run at a raised priority: each SIMD pairs one of them
    // with a memory wave, and the compute wave then takes the issue slots first
    // (bit-identical; 0.817 -> 0.804 ms per call at the batched d = 128 shape; the
    // memory waves raised instead made it 9% slower).
    if (wid < 4) __builtin_amdgcn_s_setprio(2);
    if (wid < 2) {
        // The chain reads chunk c's Tm operands from the LDS slot the gate wave
        // filled in period c-1, so it never waits on a global load.
        const int g4 = lane >> 4;
        const int col = 16 * wid + (lane & 15);
        size_t sbase = ((size_t)(b * p.H + h) * p.dv + dv0 + col) * DK;
        if constexpr (SW == SWEEP_FIRST || SW == SWEEP_SECOND) sbase += (size_t)dir * p.state_dir_stride;
        Chain16<DK> ch;
        ch.init(p, sm, sbase, col, g4, c0);
        __syncthreads();
        f32x4_t nacc[4];
        typename Chain16<DK>::KtOps kt;
        for (int it = c0 - 2; it < c1 + 1; it += 2) {
            const bool run0 = x.has(it), run1 = x.has(it + 1);
            if (run0) {
                const TmOps t = lds_tm(sm.Tms[it & 1], lane);
                ch.step_n(sm, it, lane, col, t, nacc, kt);
                ch.step_s(sm, it, lane, col, nacc, kt);
            }
            __syncthreads();
            if (run1) {
                const TmOps t = lds_tm(sm.Tms[(it + 1) & 1], lane);
                ch.step_n(sm, it + 1, lane, col, t, nacc, kt);
                ch.step_s(sm, it + 1, lane, col, nacc, kt);
            }
            __syncthreads();
        }
        ch.finish(p, sbase, g4);
    } else if (wid == 2) {
        output_role<DK, 0, PRO, ADD>(x, sm, p, lane, out_b, part_b);
    } else if (wid == 3) {
        output_role<DK, 1, PRO, ADD>(x, sm, p, lane, out_b, part_b);
    } else if (wid < 6) {
        // K (wave 4) or Q (wave 5) of chunk c is stored in period c-1 from register
        // set c&1, loaded in period c-3.  Memory operations only.  The loads are
        // unconditional (past the last chunk they re-read it), so that the count
        // of loads in flight is the same on every path and the wait before a store
        // covers only the loads of the chunk being stored.
        const bool is_k = wid == 4;
        const char *base = is_k ? x.k : x.q;
        auto store = [&](int c, const Rows64<DK, IO> &r) {
            if (is_k) store_rows<DK, Smem<DK>::LKK, IO>(sm.Ks[c & 1], r, lane);
            else store_rows<DK, Smem<DK>::LKK, IO>(sm.Qs[c & 1], r, lane);
        };
        Rows64<DK, IO> rA, rB;
        rA = load_rows<DK, IO>(base, x, c0, lane);
        __syncthreads();
        for (int it = c0 - 2; it < c1 + 1; it += 2) {
            if (x.has(it + 1)) store(it + 1, rB);
            rB = load_rows<DK, IO>(base, x, x.clamp(it + 3), lane);
            __syncthreads();
            if (x.has(it + 2)) store(it + 2, rA);
            rA = load_rows<DK, IO>(base, x, x.clamp(it + 4), lane);
            __syncthreads();
        }
    } else if (wid == 6) {
        // Gates of chunk c are computed in period c-2 from register set c&1
        // (loaded in period c-4).  With OUT_ADD_PARTIAL this wave also stages the
        // other direction's outputs of chunk c into LDS in period c (loaded in
        // period c-2), for the output waves' stores of chunk c in period c+1.
        GateRegs gA, gB;
        load_gates<PRO>(x, c0, lane, gA);
        load_gates<PRO>(x, x.clamp(c0 + 1), lane, gB);
        PartRows pA, pB;
        // Tm of chunk c is stored in period c-1 from register set c&1, loaded in period c-3
        const uint16_t *tm_head = p.tm + (size_t)((dir * p.B + b) * p.H + h) * n * TM_ELEMS;
        TmMem mA = load_tm(tm_head, c0, c1, lane), mB;
        __syncthreads();
        for (int it = c0 - 2; it < c1 + 1; it += 2) {
            if (x.has(it + 1)) store_tm(sm.Tms[(it + 1) & 1], mB, lane);
            mB = load_tm(tm_head, it + 3, c1, lane);
            if (x.has(it + 2)) gates_store<DK, PRO>(x, sm, it + 2, lane, gA);
            load_gates<PRO>(x, x.clamp(it + 4), lane, gA);
            if constexpr (ADD) {
                if (x.has(it)) store_part(it, pA, lane);
                pA = load_part(x, other_b, x.clamp(it + 2), lane);
            }
            __syncthreads();
            if (x.has(it + 2)) store_tm(sm.Tms[(it + 2) & 1], mA, lane);
            mA = load_tm(tm_head, it + 4, c1, lane);
            if (x.has(it + 3)) gates_store<DK, PRO>(x, sm, it + 3, lane, gB);
            load_gates<PRO>(x, x.clamp(it + 5), lane, gB);
            if constexpr (ADD) {
                if (x.has(it + 1)) store_part(it + 1, pB, lane);
                pB = load_part(x, other_b, x.clamp(it + 3), lane);
            }
            __syncthreads();
        }
    } else {
        // b_t v_t of chunk c is stored in period c-1 from V register set c&1
        // (loaded in period c-3, unconditionally as for K and Q), with b_t from
        // the gate slot of chunk c.
        VRow<IO> vA, vB;
        vA = load_v<IO>(x, c0, lane);
        __syncthreads();
        for (int it = c0 - 2; it < c1 + 1; it += 2) {
            if (x.has(it + 1)) store_bv<DK, IO>(sm, it + 1, vB, lane);
            vB = load_v<IO>(x, x.clamp(it + 3), lane);
            __syncthreads();
            if (x.has(it + 2)) store_bv<DK, IO>(sm, it + 2, vA, lane);
            vA = load_v<IO>(x, x.clamp(it + 4), lane);
            __syncthreads();
        }
    }
}

template <int DK, int IO, bool PRO>
hipError_t launch_dk(const PassArgs &a, hipStream_t stream) {
    const int nchunks = (int)((a.T + C - 1) / C);
    const int dirs = a.both_dirs ? 2 : 1;
    const long long ntm = (long long)dirs * a.B * a.H * nchunks;
    if (!a.tm || ntm > a.tm_chunks || ntm > 0x7fffffffLL) return hipErrorInvalidValue;
    // The gate records follow the Tm blocks of the handle's whole capacity.
    void *grec = a.tm + (size_t)a.tm_chunks * TM_ELEMS;

    TmParams t;
    t.k = static_cast<const char *>(a.k);
    t.beta = a.beta; t.decay = a.decay;
    t.tm = a.tm;
    t.grec = grec;
    t.T = a.T; t.qk_ts = a.qk_ts; t.qk_bs = a.qk_bs;
    t.B = a.B; t.H = a.H; t.nchunks = nchunks; t.reverse = a.reverse;
    // The bidirectional split's second launch needs the inverses of chunks [n1, n)
    // only after the first launch, which leaves CUs idle when B H is small: given a
    // side stream, those inverses are formed there, beside the first launch.
    const int n1 = (nchunks + 1) / 2;
    const bool side = a.both_dirs && a.bidi_state && a.side_stream && n1 < nchunks;
    // With the side stream, the first half is walked in two launches, [0, q) and
    // [q, n1), so that only the inverses of [0, q) precede the first: those of [q, n1)
    // and of the second half are formed on the side stream, in that order, beside it.
    const int q = side && a.ev_join_mid && n1 >= 16 ? (n1 + 1) / 2 : n1;
    auto set_range = [&](int c0, int nc) {
        t.c0 = c0;
        t.nc = nc;
        t.nblk = dirs * a.B * a.H * nc;
        t.xcd_remap = t.nblk % 8 == 0;
    };
    set_range(0, side ? q : nchunks);
    hipLaunchKernelGGL((tm_kernel<DK, IO, PRO>), dim3((unsigned)t.nblk), dim3(256), 0, stream, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipStream_t s2 = static_cast<hipStream_t>(a.side_stream);
    hipEvent_t fork = static_cast<hipEvent_t>(a.ev_fork), join = static_cast<hipEvent_t>(a.ev_join);
    hipEvent_t join_mid = static_cast<hipEvent_t>(a.ev_join_mid);
    if (side) {
        if ((e = hipEventRecord(fork, stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(s2, fork, 0)) != hipSuccess) return e;
        if (q < n1) {
            set_range(q, n1 - q);
            hipLaunchKernelGGL((tm_kernel<DK, IO, PRO>), dim3((unsigned)t.nblk), dim3(256), 0, s2, t);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if ((e = hipEventRecord(join_mid, s2)) != hipSuccess) return e;
        }
        set_range(n1, nchunks - n1);
        hipLaunchKernelGGL((tm_kernel<DK, IO, PRO>), dim3((unsigned)t.nblk), dim3(256), 0, s2, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = hipEventRecord(join, s2)) != hipSuccess) return e;
    }

    ChunkParams p;
    p.q = static_cast<const char *>(a.q);
    p.k = static_cast<const char *>(a.k);
    p.v = static_cast<const char *>(a.v);
    p.qk_ts = a.qk_ts; p.qk_bs = a.qk_bs; p.v_ts = a.v_ts; p.v_bs = a.v_bs;
    p.grec = grec;
    p.state_in = a.state_in; p.state_out = a.state_out; p.out = a.out;
    p.partial = a.partial; p.partial_rev = a.partial_rev;
    p.tm = a.tm;
    p.T = a.T; p.B = a.B; p.H = a.H; p.dv = a.dv;
    p.state_dir_stride = 0;
    p.ntile = a.dv / DVT;
    p.nblk_dir = a.B * a.H * p.ntile;
    p.xcd_remap = (p.nblk_dir % 8) == 0;
    p.reverse = a.reverse; p.out_mode = a.out_mode; p.both_dirs = a.both_dirs;
    p.c0 = 0; p.c1 = nchunks;
    p.scale = (float)(1.0 / __builtin_sqrt((double)DK));
    p.state_out_t = 0;
    p.seg_out = nullptr;
    const int nblk = p.nblk_dir * dirs;
    if (!a.both_dirs && a.nseg > 1) {
        // Segment-parallel causal form, one launch with a block row per segment run.
        // Rows 0 .. nseg-1: segment 0 from state_in, storing out; segments 1 .. nseg-1
        // from zero, storing bf16 rows o^0.  Rows nseg .. 2 nseg-2: segments 1 .. nseg-1
        // again, from the identity with v = 0 (d_v = d_k): row i of that run's state is
        // e_i^T times the product of the segment's per-token transitions, so its
        // outputs are w_t = (that product up to t) q_t / sqrt(d_k) and its final state
        // is the segment's transition.  A small combine then forms the true start
        // states and corrects the later segments' outputs.
        if (!a.seg_partial || !a.seg_w || !a.seg_sloc || !a.seg_phi || !a.seg_eye || !a.seg_vzero ||
            (long long)a.seg_len * (a.nseg - 1) >= nchunks)
            return hipErrorInvalidValue;
        ChunkParams pi = p;
        pi.v = static_cast<const char *>(a.seg_vzero);
        pi.v_ts = 0; pi.v_bs = 0;
        pi.dv = DK;
        pi.ntile = DK / DVT;
        pi.nblk_dir = a.B * a.H * pi.ntile;
        pi.xcd_remap = (pi.nblk_dir % 8) == 0;
        pi.state_in = a.seg_eye;
        pi.state_out = a.seg_phi;
        pi.out = nullptr;
        pi.partial = nullptr;
        pi.seg_out = a.seg_w;
        pi.seg_len = a.seg_len; pi.seg_base = 1; pi.seg_zero_start = 0; pi.seg0_store = 0;
        pi.seg_state_stride = (long long)a.B * a.H * DK * DK;
        pi.seg_rows = a.nseg - 1;
        pi.state_out_t = 1;  // the transitions, transposed: the combine reads their columns as rows

        p.state_out = a.seg_sloc;
        p.seg_out = a.seg_partial;
        p.seg_len = a.seg_len; p.seg_base = 0; p.seg_zero_start = 1; p.seg0_store = 1;
        p.seg_state_stride = (long long)a.B * a.H * a.dv * DK;
        p.seg_rows = a.nseg;
        const int gx = nblk > pi.nblk_dir ? nblk : pi.nblk_dir;
        hipLaunchKernelGGL((chunk_kernel<DK, IO, PRO, SWEEP_SEG>), dim3(gx, 2 * a.nseg - 1), dim3(NT), 0, stream,
                           p, pi);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        return launch_seg_combine(a, stream);
    }
    if (!(a.both_dirs && a.bidi_state)) {
        hipLaunchKernelGGL((chunk_kernel<DK, IO, PRO, SWEEP_ALL>), dim3(nblk), dim3(NT), 0, stream, p, p);
        return hipGetLastError();
    }
    // Bidirectional form in two launches.  The first walks chunks [0, n1) of both
    // directions (the forward one tokens [0, 64 n1), the reverse one the last 64 n1
    // tokens), writes its outputs as bf16 rows of the partial buffers and keeps each
    // direction's fp32 state; the second
    // walks chunks [n1, n) from those states, and each direction adds the other's
    // partial of the same token -- written by the first launch -- before rounding
    // out once.  Tokens both first halves covered (at most 64, in the middle) are
    // combined by a small row-range pass.
    p.state_dir_stride = (long long)a.B * a.H * a.dv * DK;
    p.state_in = nullptr;
    p.state_out = a.bidi_state;
    p.out_mode = OUT_STORE;  // into the direction's partial buffer (see the kernel)
    p.c0 = 0; p.c1 = q;
    hipLaunchKernelGGL((chunk_kernel<DK, IO, PRO, SWEEP_FIRST>), dim3(nblk), dim3(NT), 0, stream, p, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (q < n1) {
        // resume from the fp32 states in place: each block reads its own columns at
        // its start and writes them at its end
        if ((e = hipStreamWaitEvent(stream, join_mid, 0)) != hipSuccess) return e;
        p.state_in = a.bidi_state;
        p.c0 = q; p.c1 = n1;
        hipLaunchKernelGGL((chunk_kernel<DK, IO, PRO, SWEEP_FIRST>), dim3(nblk), dim3(NT), 0, stream, p, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (n1 < nchunks) {
        if (side && (e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return e;
        p.state_in = a.bidi_state;
        p.state_out = nullptr;
        p.out_mode = OUT_ADD_PARTIAL;
        p.c0 = n1; p.c1 = nchunks;
        hipLaunchKernelGGL((chunk_kernel<DK, IO, PRO, SWEEP_SECOND>), dim3(nblk), dim3(NT), PART_LDS_BYTES, stream,
                           p, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const long long half = (long long)C * n1;
    const long long t0 = a.T - half > 0 ? a.T - half : 0, t1 = half < a.T ? half : a.T;
    return launch_combine_rows_bf16(static_cast<uint16_t *>(a.out), reinterpret_cast<const uint16_t *>(a.partial),
                                    reinterpret_cast<const uint16_t *>(a.partial_rev), a.B, a.T,
                                    (long long)a.H * a.dv, t0, t1, stream);
}

template <int DK>
hipError_t launch_dk(const PassArgs &a, hipStream_t stream) {
    if (a.io == IO_FP8) return a.prologue ? launch_dk<DK, IO_FP8, true>(a, stream) : launch_dk<DK, IO_FP8, false>(a, stream);
    return a.prologue ? launch_dk<DK, IO_BF16, true>(a, stream) : launch_dk<DK, IO_BF16, false>(a, stream);
}

}  // namespace

bool chunk_mfma_supported(int C_, int dk, int dv, int io) {
    const bool dims = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
    return C_ == C && dims && (io == IO_BF16 || io == IO_FP8);
}

size_t chunk_mfma_tm_bytes(long long chunks) {
    return (size_t)chunks * (TM_ELEMS * sizeof(uint16_t) + C * sizeof(float4));
}

hipError_t launch_chunk_mfma(const PassArgs &a, int C_, hipStream_t stream) {
    if (!chunk_mfma_supported(C_, a.dk, a.dv, a.io)) return hipErrorInvalidValue;
    switch (a.dk) {
        case 32: return launch_dk<32>(a, stream);
        case 64: return launch_dk<64>(a, stream);
        case 128: return launch_dk<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
