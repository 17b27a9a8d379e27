/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated-Delta-Net recurrence library.
 *
 * The operation.  Per batch element b and head h, independently, over tokens
 * t = 0 .. T-1 with a d_v x d_k fp32 state S:
 *
 *     S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     o_t = S_t q_t / sqrt(d_k)
 *
 * This is the GDN (Gated-Delta-Net) linear-attention recurrence of the SANA
 * video DiTs: the librediffusion PR #21 page ("feat(sana): in-tree
 * SANA-Streaming V2V DiT (GDN linear-attention) + C-API", section "What's
 * added") ships it as a CUDA kernel behind a C API, and the sglang SANA-WM
 * record (errors.standardbeagle.com page, field sourceCode) names its inputs
 * q, k, v, beta, decay.  The state carried from call to call is the "causal
 * linear attention KV cache" of the diffusers LongSANA PR page (section
 * "PR feature"); the bidirectional form is the full-sequence SANA-WM variant
 * of the FlashDreams "SANA-WM" page (section "Bidirectional variant").  The
 * pages do not print the update; the formula above is the gated delta rule.
 *
 * gdn_forward and gdn_forward_bidi take q and k as given, and beta (b_t) and
 * decay (a_t) as plain values in [0, 1], one per token and head -- not logits,
 * not log-decays.  gdn_forward_packed and gdn_forward_bidi_packed instead read
 * q, k and v straight from a packed projection and apply the input prologue
 * inside the kernels (see there).
 *
 * Layouts.  Every tensor pointer is a DEVICE pointer to a contiguous,
 * row-major array on the handle's device:
 *     q, k       [B, T, H, d_k]   io_dtype
 *     v          [B, T, H, d_v]   io_dtype
 *     out        [B, T, H, d_v]   fp32 (GDN_F32) or bf16 (GDN_BF16, GDN_FP8)
 *     beta,decay [B, T, H]        float32
 *     state      [B, H, d_v, d_k] float32  (row i is output channel i: o = S q)
 * q, k, v, out and the states must be 16-byte aligned; beta and decay 4-byte.
 * FP8 inputs are one byte per element, so their rows are 16-byte multiples too.
 *
 * Ownership.  The caller owns every tensor and the stream.  The library owns
 * the handle and its device scratch, allocated once in gdn_create and freed in
 * gdn_free: the two fp32 partials and two fp32 states of gdn_forward_bidi
 * (GDN_FLAG_BIDI; with them, on handles the MFMA kernel serves, a second
 * stream of default priority and three events, see gdn_forward_bidi), and, on
 * handles the bf16 MFMA chunked kernel can serve (bf16 or FP8 inputs, d_k and
 * d_v >= 32), the per-chunk triangular inverses of that kernel and each
 * token's gate record (b, log2 a and, for the packed entry points, the inverse
 * k norm): 6 KiB per direction, b, h and 64-token chunk up to max_T.  The
 * forward calls allocate nothing, never
 * synchronise and never copy between host and device: they validate, enqueue
 * kernels on the given stream and return.  Device faults surface at the
 * caller's next synchronisation, as with any HIP launch.  A handle must be
 * used by one host thread at a time, and its calls must not overlap on the
 * device, since they share the handle's scratch: enqueue them on one stream,
 * or order streams with events.  Separate handles are independent and may run
 * concurrently on different streams.
 *
 * Errors.  Every call returns GDN_OK (0) or a negative gdn_status; nothing is
 * thrown across this boundary and no call silently falls back to another
 * algorithm.  Validation happens before any launch, so a rejected call leaves
 * out and state_out untouched.  gdn_last_error() describes the last failure.
 */
#ifndef GDN_H
#define GDN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gdn_ctx *gdn_handle; /* opaque; hides every HIP type */

typedef enum {
    GDN_OK = 0,
    GDN_ERR_ARG = -1,         /* NULL pointer, bad size, T > max_T, ...        */
    GDN_ERR_UNSUPPORTED = -2, /* d_k/d_v not in {16,32,64,128}, dtype, chunk_len */
    GDN_ERR_ALIGN = -3,       /* pointer alignment (see Layouts)               */
    GDN_ERR_ALIAS = -4,       /* an output overlaps an input or another output */
    GDN_ERR_DEVICE = -5,      /* no such device, not gfx950, HIP runtime error  */
    GDN_ERR_OOM = -6,         /* scratch allocation failed in gdn_create        */
    GDN_ERR_LAUNCH = -7       /* kernel launch was rejected                     */
} gdn_status;

/* Element type of q, k, v (and qkv).  out is fp32 for GDN_F32 and bf16 for the
 * others; beta, decay and the state are always fp32.  GDN_FP8 is OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN =
 * S.1111.111), widened exactly to bf16 / fp32 inside the kernels: halving the
 * bytes of q, k and v; the FlashDreams SANA-WM page (section "Developer Details",
 * the precision bullet) lists FP8 inference beside the bf16 default.  Its
 * arithmetic is that of the bf16 path. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1, GDN_FP8 = 2 } gdn_dtype;

/* Request the scratch that gdn_forward_bidi needs: 2 * B * max_T * H * d_v fp32
 * partial outputs and 2 * B * H * d_v * d_k fp32 states. */
#define GDN_FLAG_BIDI 1u

/* Segment-parallel causal form, for calls whose heads leave most of the device's
 * CUs idle (streaming calls of a few thousand tokens, few heads).  On the bf16 MFMA
 * chunked path (chunk_len 64, bf16 or FP8 inputs, d_k and d_v >= 32) a causal call
 * of at least 16 chunks is cut into up to 8 token segments of whole chunks that run
 * concurrently: segment 0 from state_in, each later one from zero and, beside it,
 * from the identity with v = 0, which gives the segment's transition; a combine
 * then forms each segment's true start state and adds its contribution to the
 * outputs (the recurrence is affine in the state; the later segments' own outputs
 * and the identity runs' outputs pass through bf16 rows, and the correction
 * products run on bf16 MFMA with the fp32 states split in two bf16 parts).  The
 * segment count is the largest whose blocks fit on the device at once.  Results
 * stay within the stated tolerances, but are not bit-identical to one sweep, nor
 * across different splits of a sequence into calls.  Costs per handle: bf16
 * [B, max_T, H, d_v + d_k] plus fp32 8 d_v x d_k states and 8 d_k x d_k matrices
 * per (b, h).  Without this flag every call is one sweep. */
#define GDN_FLAG_SEGMENTS 2u

typedef struct {
    int device;        /* HIP device ordinal; -1 = dry run (validate only, no GPU) */
    int B, H;          /* batch (1 .. 32767) and heads (>= 1, H * max(d_k, d_v)   *
                        * at most 2^24 / 3)                                     */
    int d_k, d_v;      /* head dims, each in {16, 32, 64, 128}                    */
    int io_dtype;      /* gdn_dtype of q, k, v (out: fp32 or bf16, see gdn_dtype) */
    long long max_T;   /* largest T any call on this handle will pass, >= 0       */
    unsigned flags;    /* GDN_FLAG_* bits                                         */
} gdn_config;

/*
 * Create a handle.  On success *out_h holds it and GDN_OK is returned.  On
 * failure *out_h is set to NULL, a negative status is returned and one line
 * is printed to stderr (gdn_last_error(NULL) repeats it).  device = -1 gives
 * a dry-run handle: every call is fully validated and then returns GDN_OK
 * without touching a GPU.
 */
int gdn_create(const gdn_config *cfg, gdn_handle *out_h);

/*
 * Causal recurrence over T tokens (0 <= T <= max_T), starting from state_in
 * and leaving the final state in state_out.
 *   state_in   NULL = zero initial state; never written unless it is state_out.
 *   state_out  NULL = final state discarded; may equal state_in (in-place carry).
 *   chunk_len  1 = sequential scan; 16, 32, 64 or 128 = chunked (UT-transform)
 *              form with chunks of that many tokens; 0 = default (64).  Others
 *              return GDN_ERR_UNSUPPORTED.  bf16 or FP8 inputs with chunk_len 64
 *              and d_k, d_v >= 32 run on bf16 MFMA with fp32 accumulation;
 *              every other chunked request (fp32 I/O, other chunk lengths,
 *              d = 16) runs a kernel that computes in fp32 throughout.
 *   hip_stream a hipStream_t (NULL = the null stream of the handle's device).
 * Streaming: calling with consecutive token ranges and state_out of one call
 * as state_in of the next reproduces a single call over the whole range.
 * With chunk_len = 1 the result is bit-identical to the single call; with the
 * chunked form it is bit-identical when every call but the last is a multiple
 * of chunk_len long, and equal within rounding otherwise.
 * T = 0 is valid: state_out receives state_in (or zeros); out is untouched.
 */
int gdn_forward(gdn_handle h, const void *q, const void *k, const void *v,
                const float *beta, const float *decay,
                const float *state_in, float *state_out, void *out,
                long long T, int chunk_len, void *hip_stream);

/*
 * Bidirectional form over one full sequence:
 *     out = fwd(x; S = 0) + R(fwd(R x; S = 0)),
 * R reversing the token axis; token t is counted by both directions.  The two
 * directions' outputs are summed in fp32 and rounded once to io_dtype; on the
 * bf16 MFMA path the term a direction produced in its first half of the sweep is
 * kept as a bf16 row until the other direction adds to it.  The reverse pass
 * places its chunk grid from token T-1 downwards and both directions are treated
 * alike, so reversing the inputs reverses the output exactly.  Needs a handle
 * created with GDN_FLAG_BIDI.  No state is read or returned.  On the bf16 MFMA
 * path the call also enqueues up to two kernels on a stream the handle owns
 * (created with GDN_FLAG_BIDI, default priority), forked from and joined back
 * into hip_stream by events: work enqueued on hip_stream after the call still
 * runs after all of it, and the call can be captured into a HIP graph.
 */
int gdn_forward_bidi(gdn_handle h, const void *q, const void *k, const void *v,
                     const float *beta, const float *decay, void *out,
                     long long T, int chunk_len, void *hip_stream);

/*
 * Fused input prologue.  The same forms as gdn_forward / gdn_forward_bidi
 * (same handle, state, out, T, chunk_len and stream rules), with the inputs
 * taken from a packed token-major projection and prepared in the kernels:
 *
 *   qkv    io_dtype; element j of token t of batch element b is
 *          qkv[b * batch_stride + t * token_stride + j], with
 *            q of head h at j = h d_k + (0 .. d_k-1),
 *            k of head h at j = H d_k + h d_k + (0 .. d_k-1),
 *            v of head h at j = 2 H d_k + h d_v + (0 .. d_v-1)
 *          -- the [N, 3C] layout (C = H d) whose split into q, k, v the
 *          librediffusion PR #21 page's review moves onto the GPU (suggestion
 *          "k_split_qkv"), here read in place by the recurrence kernels.
 *   token_stride, batch_stride   in elements; token_stride >= 2 H d_k + H d_v,
 *          batch_stride >= 0, both multiples of 16 bytes; qkv 16-byte aligned.
 *   beta_logit, decay_logit      [B, T, H] float32 logits x_b, x_a.
 *
 * Per token and head the kernels use
 *     q <- q / max(||q||_2, 1e-12),  k <- k / max(||k||_2, 1e-12),
 *     b_t = sigmoid(x_b) = 1 / (1 + e^{-x_b}),
 *     a_t = exp(-softplus(x_a)) = 1 / (1 + e^{x_a}),
 * computed in fp32 from the inputs as given (the chunked bf16 / FP8 kernel takes
 * 1 / max(||q||, 1e-12) with the hardware reciprocal square root, to within an
 * ulp; the sglang SANA-WM record widens
 * q, k, v with .float().contiguous() in a separate pass before its scan; here
 * nothing is materialised).  out (contiguous [B, T, H, d_v]) and state_out
 * must not overlap the byte range qkv spans.  Errors as for gdn_forward, plus
 * GDN_ERR_ARG for a token_stride below the packed row, GDN_ERR_ALIGN for a
 * stride that is not a multiple of 16 bytes and GDN_ERR_UNSUPPORTED for a
 * token_stride above 2^24 elements.
 */
int gdn_forward_packed(gdn_handle h, const void *qkv, long long token_stride,
                       long long batch_stride, const float *beta_logit,
                       const float *decay_logit, const float *state_in,
                       float *state_out, void *out, long long T, int chunk_len,
                       void *hip_stream);

/* Bidirectional form with the fused prologue (needs GDN_FLAG_BIDI). */
int gdn_forward_bidi_packed(gdn_handle h, const void *qkv, long long token_stride,
                            long long batch_stride, const float *beta_logit,
                            const float *decay_logit, void *out, long long T,
                            int chunk_len, void *hip_stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  gdn_forward's causal
 * form (same arguments, layouts, state, chunk_len and stream rules), with no
 * handle: *cfg is a configuration as for gdn_create (flags must be 0; max_T is
 * not used).  The call allocates nothing, on the device or the host.  The
 * scratch of the bf16 / FP8 MFMA chunked kernel (chunk_len 64, d_k, d_v >= 32:
 * 6 KiB per b, h and 64-token chunk) is one fixed 64 MiB device array inside the
 * library, one per GPU, held until the process ends; a call whose
 * B * H * ceil(T / 64) exceeds 10,922 chunks is refused with
 * GDN_ERR_UNSUPPORTED before anything is launched (B = 1, H = 20 allows
 * T <= 34,944).  The other paths (scan, fp32 chunked kernel) need no scratch.
 * Every call on one GPU shares that GPU's array: calls that may overlap on the
 * device (streams not ordered by events) race and give wrong results.  The
 * first call on a device resolves the array's address and checks the device
 * (hipGetSymbolAddress, hipGetDeviceProperties): make it outside graph capture.
 * Errors as for gdn_forward, GDN_ERR_DEVICE for a device that is not a gfx950;
 * the message is read with gdn_last_error(NULL).  device = -1 validates only.
 */
int gdn_forward_noalloc(const gdn_config *cfg, const void *q, const void *k,
                        const void *v, const float *beta, const float *decay,
                        const float *state_in, float *state_out, void *out,
                        long long T, int chunk_len, void *hip_stream);

/* Release the handle and its scratch.  NULL is a no-op. */
void gdn_free(gdn_handle h);

/* Message of the last failed call on h (NULL: last gdn_create failure on
 * this thread).  Never NULL; "" when there was none.  Valid until the next
 * call on the same handle. */
const char *gdn_last_error(gdn_handle h);

/* Library version, "major.minor.patch". */
const char *gdn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
