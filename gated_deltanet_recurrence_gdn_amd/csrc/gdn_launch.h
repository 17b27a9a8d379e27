// gdn_launch.h -- internal interface between the C-ABI layer and the kernels.
// Not installed; callers use include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace gdn {

// Element type of q, k, v.  out is fp32 for IO_F32 and bf16 otherwise.
enum IoType : int {
    IO_F32 = 0,   // fp32
    IO_BF16 = 1,  // bf16
    IO_FP8 = 2,   // OCP FP8 E4M3 (widened exactly to bf16 / fp32 at load)
};
__host__ __device__ constexpr int io_in_bytes(int io) { return io == IO_F32 ? 4 : io == IO_BF16 ? 2 : 1; }
__host__ __device__ constexpr int io_out_bytes(int io) { return io == IO_F32 ? 4 : 2; }

// What a pass does with the per-token outputs o_t.
enum OutMode : int {
    OUT_STORE = 0,    // out[t] = round(o_t) in the I/O dtype
    OUT_PARTIAL = 1,  // partial[t] = o_t in fp32 (one direction of the bidirectional form)
    OUT_ADD_PARTIAL = 2,  // out[t] = round(o_t + the other direction's partial[t]) (bidirectional)
};

// One pass of the recurrence over a whole call, all (b, h) pairs.
struct PassArgs {
    // q, k, v: head h of token t of batch element b starts at element
    // b * qk_bs + t * qk_ts + h * dk of q and k (b * v_bs + t * v_ts + h * dv of
    // v): contiguous [B,T,H,d] tensors, or views into a packed projection.
    const void *q;          // io dtype
    const void *k;
    const void *v;
    long long qk_ts, qk_bs; // q and k: elements between tokens / batch elements
    long long v_ts, v_bs;   // v: the same
    const float *beta;      // [B,T,H]: b_t (prologue: its logit)
    const float *decay;     // [B,T,H]: a_t (prologue: its logit)
    int prologue;           // 1: q, k are L2-normalised per token and head, and
                            //    b = sigmoid(beta), a = exp(-softplus(decay))
    const float *state_in;  // [B,H,dv,dk] or nullptr (zeros)
    float *state_out;       // [B,H,dv,dk] or nullptr; may equal state_in
    void *out;              // [B,T,H,dv] fp32 or bf16 (OUT_STORE), see IoType
    float *partial;         // [B,T,H,dv] fp32 (OUT_PARTIAL); bf16 rows in the MFMA kernel's bidi split
    float *partial_rev;     // [B,T,H,dv] the same for the reverse direction (both_dirs)
    int B, H, dk, dv;
    long long T;
    int io;                 // IoType of q, k, v
    int reverse;            // 1: walk tokens T-1 .. 0
    int out_mode;           // OutMode
    int both_dirs;          // 1: one launch runs both directions (OUT_PARTIAL into
                            //    partial and partial_rev), from zero state
    uint16_t *tm;           // MFMA kernel only: the per-chunk scratch of the handle
    long long tm_chunks;    // chunk capacity of tm (directions x B x H x chunks)
    float *bidi_state;      // MFMA kernel, both_dirs: [2][B,H,dv,dk] fp32 scratch; when set, the
                            // bidirectional form is two launches split at the middle chunk and
                            // writes out itself (no separate combine)
    void *side_stream;      // optional (with bidi_state): a hipStream_t on which the inverses of
    void *ev_fork;          // the second half are formed beside the first launch, ordered by
    void *ev_join;          // these two hipEvent_t (fork: stream -> side, join: side -> stream)
    void *ev_join_mid;      // optional third hipEvent_t: with it the first half runs as two launches
                            // and the inverses of its second part are formed on the side stream
                            // too, joined back by this event before that part
    // Segment-parallel causal form (MFMA kernel, causal, nseg > 1):
    // the call's chunks are cut into nseg segments of seg_len chunks.  Segment 0 runs
    // from state_in and writes out; every later segment runs from zero into
    // seg_partial, and in the same launch the same segment runs from the identity with v = 0
    // (seg_w: its outputs w_t, seg_phi: its final state, the segment's transition);
    // then the true start states follow segment by segment and each later token's
    // output is corrected by S_start w_t.
    int nseg, seg_len;
    void *seg_partial;      // [B,T,H,dv] bf16
    void *seg_w;            // [B,T,H,dk] bf16
    float *seg_sloc;        // [nseg][B,H,dv,dk] fp32: final states from each segment's own start
    float *seg_phi;         // [nseg-1][B,H,dk,dk] fp32: transitions of segments 1 .. nseg-1, transposed
    const float *seg_eye;   // [B,H,dk,dk] fp32 identity matrices
    const void *seg_vzero;  // H * max(dk, dv) zeros of the input type (v of the identity runs)
};

// Token-major contiguous strides for q, k [B,T,H,dk] and v [B,T,H,dv].
inline void contiguous_strides(PassArgs &a) {
    a.qk_ts = (long long)a.H * a.dk;
    a.qk_bs = a.T * a.qk_ts;
    a.v_ts = (long long)a.H * a.dv;
    a.v_bs = a.T * a.v_ts;
}

// Sequential per-token scan (the chunk_len = 1 form).
hipError_t launch_scan(const PassArgs &a, hipStream_t stream);

// Chunked (UT-transform) form, bf16 MFMA kernel: C = 64, bf16 or FP8 inputs,
// d_k, d_v in {32, 64, 128}.
// It needs PassArgs::tm: chunk_mfma_tm_bytes(n) bytes hold the triangular
// inverses of n chunks (one per direction, b, h and chunk) and their tokens'
// gate records.
bool chunk_mfma_supported(int C, int dk, int dv, int io);
size_t chunk_mfma_tm_bytes(long long chunks);
hipError_t launch_chunk_mfma(const PassArgs &a, int C, hipStream_t stream);

// Chunked form, general fp32 kernel: C, d_k, d_v in {16, 32, 64, 128}, every
// IoType.
bool chunk_general_supported(int C, int dk, int dv);
hipError_t launch_chunk_general(const PassArgs &a, int C, hipStream_t stream);

// out[e] = round(partial[e] + partial_rev[e]) over n elements (n % 4 == 0), out
// in fp32 for IO_F32 and bf16 otherwise.
hipError_t launch_combine(void *out, const float *partial, const float *partial_rev, long long n,
                          int io, hipStream_t stream);
// out = round(partial + partial_rev) over the token rows [t0, t1) of every batch
// element of [B, T, row] tensors (row % 4 == 0), all three bf16: the middle rows of the
// bidirectional MFMA split, whose first launch stores bf16 partial rows.
hipError_t launch_combine_rows_bf16(uint16_t *out, const uint16_t *partial, const uint16_t *partial_rev, int B,
                                    long long T, long long row, long long t0, long long t1, hipStream_t stream);

// Segment-parallel causal form, after the sweeps: state_out and, for every token of
// segments > 0, out = round(seg_partial + S_start w_t), with each segment's true start
// state S_start formed from the segment states and transitions (one launch).
hipError_t launch_seg_combine(const PassArgs &a, hipStream_t stream);

// The fixed device array behind gdn_forward_noalloc (gdn_static.hip): its size,
// and its device address on `device` (resolved on the first call for that device,
// with the device made current for it; *is_gfx950 is false, and *ptr NULL, for a
// device of another architecture).
constexpr size_t STATIC_SCRATCH_BYTES = 64ull << 20;
hipError_t static_scratch(int device, void **ptr, bool *is_gfx950);

// Chunked form with chunk length C: the MFMA kernel where it applies, else the
// general one.  hipErrorInvalidValue for a (C, dk, dv, dtype) neither covers.
inline bool chunk_supported(int C, int dk, int dv, int io) {
    return chunk_mfma_supported(C, dk, dv, io) || chunk_general_supported(C, dk, dv);
}
inline hipError_t launch_chunk(const PassArgs &a, int C, hipStream_t stream) {
    if (a.T <= 0) return hipErrorInvalidValue;  // the chunked kernels read at least one token
    // Block counts of the chunked grids (at most two directions x B x H x d_v) are ints.
    if (2LL * a.B * a.H * a.dv > 0x7fffffffLL) return hipErrorInvalidValue;
    if (chunk_mfma_supported(C, a.dk, a.dv, a.io)) return launch_chunk_mfma(a, C, stream);
    return launch_chunk_general(a, C, stream);
}

}  // namespace gdn
