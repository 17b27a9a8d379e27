// gdn_launch.h -- internal interface between the C-ABI layer and the kernels.
// Not installed; callers use include/gdn.h.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// What a pass does with the per-token outputs o_t.
enum OutMode : int {
    OUT_STORE = 0,    // out[t] = round(o_t) in the I/O dtype
    OUT_PARTIAL = 1,  // partial[t] = o_t in fp32 (one direction of the bidirectional form)
};

// One pass of the recurrence over a whole call, all (b, h) pairs.
struct PassArgs {
    const void *q;          // [B,T,H,dk] io dtype
    const void *k;          // [B,T,H,dk]
    const void *v;          // [B,T,H,dv]
    const float *beta;      // [B,T,H]
    const float *decay;     // [B,T,H]
    const float *state_in;  // [B,H,dv,dk] or nullptr (zeros)
    float *state_out;       // [B,H,dv,dk] or nullptr; may equal state_in
    void *out;              // [B,T,H,dv] io dtype (OUT_STORE)
    float *partial;         // [B,T,H,dv] fp32 (OUT_PARTIAL)
    float *partial_rev;     // [B,T,H,dv] fp32, reverse direction's partial (both_dirs)
    int B, H, dk, dv;
    long long T;
    int io_bf16;            // 1: bf16 I/O, 0: fp32 I/O
    int reverse;            // 1: walk tokens T-1 .. 0
    int out_mode;           // OutMode
    int both_dirs;          // 1: one launch runs both directions (OUT_PARTIAL into
                            //    partial and partial_rev), from zero state
};

// Sequential per-token scan (the chunk_len = 1 form).
hipError_t launch_scan(const PassArgs &a, hipStream_t stream);

// Chunked (UT-transform) form with chunk length C.  Returns
// hipErrorInvalidValue for a (C, dk, dv, dtype) it has no kernel for.
hipError_t launch_chunk(const PassArgs &a, int C, hipStream_t stream);

// out[e] = round(partial[e] + partial_rev[e]) over n elements (n % 4 == 0).
hipError_t launch_combine(void *out, const float *partial, const float *partial_rev, long long n,
                          int io_bf16, hipStream_t stream);

// Whether launch_chunk has a kernel for this shape.
bool chunk_supported(int C, int dk, int dv, int io_bf16);

}  // namespace gdn
