// gdn_api.cpp -- the C ABI (include/gdn.h): handle lifetime, validation,
// dispatch to the HIP kernels on the caller's stream.
//
// The create/forward/free handle pattern, a NULL handle plus one stderr line on
// a failed create, and building the object completely before publishing the
// handle follow the librediffusion PR #21 page (sections "What's added" and the
// review of librediffusion_sana_create).  An unavailable path is an error,
// never a silent fallback (the sglang SANA-WM record raises when a forced GDN
// backend fails its prechecks).
#include "gdn.h"
#include "gdn_launch.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>
#include <new>

// Messages live in fixed buffers, so no call but gdn_create allocates host memory.
constexpr size_t ERR_LEN = 512;

struct gdn_ctx {
    gdn_config cfg{};
    char err[ERR_LEN] = {0};
    float *scratch = nullptr;  // bidirectional form: two fp32 [B, max_T, H, d_v] partials, then
                               // two fp32 [B, H, d_v, d_k] states (the MFMA kernel's split sweep)
    size_t scratch_bytes = 0;
    uint16_t *tm = nullptr;    // per-chunk triangular inverses of the MFMA chunked kernel
    long long tm_chunks = 0;   // their capacity: directions x B x H x ceil(max_T / 64)
    // bidirectional MFMA path: a second stream (default priority) and three events, so that
    // most inverses are formed beside the first sweep launches
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_join_mid = nullptr;
    // segment-parallel causal form (GDN_FLAG_SEGMENTS on a handle the MFMA kernel serves):
    // one allocation holding the buffers gdn::PassArgs describes, and the CU count that
    // bounds the segment count
    float *seg = nullptr;
    int ncu = 0;
};

namespace {
// At most this many segments per call, each of at least SEG_MIN_CHUNKS 64-token chunks.
constexpr int SEG_MAX = 8;
constexpr int SEG_MIN_CHUNKS = 8;
// Offsets, in floats, of the segment buffers inside gdn_ctx::seg: the bf16 rows
// (partial outputs and w, two values per float slot; d_v and d_k are even), then the
// fp32 states, transitions and identities, then the zero row of v, sized in floats
// too.
struct SegLayout {
    size_t partial, w, sloc, phi, eye, vzero, total;
};
SegLayout seg_layout(const gdn_config &c) {
    SegLayout l;
    const size_t tok = (size_t)c.B * (size_t)c.max_T * c.H;
    const size_t st = (size_t)c.B * c.H * c.d_v * c.d_k, tr = (size_t)c.B * c.H * c.d_k * c.d_k;
    l.partial = 0;
    l.w = l.partial + tok * c.d_v / 2;
    l.sloc = l.w + tok * c.d_k / 2;
    l.phi = l.sloc + SEG_MAX * st;
    l.eye = l.phi + (SEG_MAX - 1) * tr;
    l.vzero = l.eye + tr;
    l.total = l.vzero + (size_t)c.H * (c.d_k > c.d_v ? c.d_k : c.d_v);
    return l;
}
}  // namespace

static_assert((int)GDN_F32 == (int)gdn::IO_F32 && (int)GDN_BF16 == (int)gdn::IO_BF16 &&
                  (int)GDN_FP8 == (int)gdn::IO_FP8,
              "gdn_dtype values are the kernels' IoType values");

namespace {

// Last failure of gdn_create, or of a call that takes no handle, on this thread.
thread_local char g_create_err[ERR_LEN];

int set_err(char *dst, int code, const char *fmt, va_list ap) {
    vsnprintf(dst, ERR_LEN, fmt, ap);
    return code;
}

int fail(gdn_ctx *h, int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    set_err(h->err, code, fmt, ap);
    va_end(ap);
    return code;
}

int fail_create(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    set_err(g_create_err, code, fmt, ap);
    va_end(ap);
    fprintf(stderr, "gdn_create failed: %s\n", g_create_err);
    return code;
}

bool valid_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(const Range &a, const Range &b) {
    return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

Range rng(const char *name, const void *p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

// Checks that p is device memory of `device` (not host memory, which would
// fault on the GPU).  Skipped for dry-run handles.
int check_device_ptr(gdn_ctx *h, const char *name, const void *p) {
    if (!p || h->cfg.device < 0) return GDN_OK;
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, GDN_ERR_ARG, "%s: not a HIP allocation (%s)", name, hipGetErrorString(e));
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(h, GDN_ERR_ARG, "%s: not device memory", name);
    if (attr.device != h->cfg.device)
        return fail(h, GDN_ERR_ARG, "%s: lives on device %d, handle is on device %d", name,
                    attr.device, h->cfg.device);
    return GDN_OK;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

// Largest token stride (elements) of q, k, v: the kernels address up to 64
// tokens of a chunk with 32-bit offsets from the chunk's first token.
constexpr long long MAX_TOKEN_STRIDE = 1LL << 24;
constexpr int MAX_B = 32767;  // (directions x B) <= 65535

// The token inputs of one call: contiguous [B,T,H,d] tensors, or views into a
// packed qkv projection with the prologue applied in the kernels.
struct Inputs {
    const void *q, *k, *v;
    long long qk_ts, qk_bs, v_ts, v_bs;  // elements between tokens / batch elements
    const float *beta, *decay;           // values, or logits (prologue)
    int prologue;
    Range in[5];                         // the byte ranges read, for the aliasing check
    int n_in;
    const void *dev_ptrs[5];             // distinct device pointers to check
    const char *dev_names[5];
    int n_dev;
};

int check_gate_ptrs(gdn_ctx *h, const float *beta, const float *decay, const char *nb, const char *nd) {
    if (reinterpret_cast<uintptr_t>(beta) % 4 || reinterpret_cast<uintptr_t>(decay) % 4)
        return fail(h, GDN_ERR_ALIGN, "%s/%s are not 4-byte aligned", nb, nd);
    return GDN_OK;
}

// Plain inputs: q, k [B,T,H,d_k], v [B,T,H,d_v], beta and decay [B,T,H] values.
int prepare_plain(gdn_ctx *h, const void *q, const void *k, const void *v, const float *beta,
                  const float *decay, const void *out, long long T, Inputs *in, size_t *out_bytes) {
    const gdn_config &c = h->cfg;
    if (T < 0) return fail(h, GDN_ERR_ARG, "T = %lld is negative", T);
    if (T > c.max_T) return fail(h, GDN_ERR_ARG, "T = %lld exceeds max_T = %lld", T, c.max_T);
    const size_t es = gdn::io_in_bytes(c.io_dtype);
    const size_t tok = (size_t)c.B * (size_t)T * (size_t)c.H;
    const size_t qk_bytes = tok * c.d_k * es, v_bytes = tok * c.d_v * es, g_bytes = tok * sizeof(float);
    *out_bytes = tok * c.d_v * gdn::io_out_bytes(c.io_dtype);
    *in = Inputs{};
    in->q = q; in->k = k; in->v = v; in->beta = beta; in->decay = decay; in->prologue = 0;
    in->qk_ts = (long long)c.H * c.d_k; in->qk_bs = T * in->qk_ts;
    in->v_ts = (long long)c.H * c.d_v; in->v_bs = T * in->v_ts;
    if (T == 0) return GDN_OK;
    if (!q || !k || !v || !beta || !decay || !out)
        return fail(h, GDN_ERR_ARG, "q, k, v, beta, decay and out must be non-NULL when T > 0");
    const void *a16[] = {q, k, v, out};
    const char *n16[] = {"q", "k", "v", "out"};
    for (int i = 0; i < 4; ++i)
        if (reinterpret_cast<uintptr_t>(a16[i]) % 16)
            return fail(h, GDN_ERR_ALIGN, "%s is not 16-byte aligned", n16[i]);
    int st = check_gate_ptrs(h, beta, decay, "beta", "decay");
    if (st) return st;
    in->in[0] = rng("q", q, qk_bytes);
    in->in[1] = rng("k", k, qk_bytes);
    in->in[2] = rng("v", v, v_bytes);
    in->in[3] = rng("beta", beta, g_bytes);
    in->in[4] = rng("decay", decay, g_bytes);
    in->n_in = 5;
    const void *dp[] = {q, k, v, beta, decay};
    const char *dn[] = {"q", "k", "v", "beta", "decay"};
    for (int i = 0; i < 5; ++i) {
        in->dev_ptrs[i] = dp[i];
        in->dev_names[i] = dn[i];
    }
    in->n_dev = 5;
    return GDN_OK;
}

// Packed inputs: element j of token t of batch element b at
// qkv[b * batch_stride + t * token_stride + j], q at j in [0, H d_k), k at
// [H d_k, 2 H d_k), v at [2 H d_k, 2 H d_k + H d_v); beta and decay are logits.
int prepare_packed(gdn_ctx *h, const void *qkv, long long token_stride, long long batch_stride,
                   const float *beta_logit, const float *decay_logit, const void *out, long long T,
                   Inputs *in, size_t *out_bytes) {
    const gdn_config &c = h->cfg;
    if (T < 0) return fail(h, GDN_ERR_ARG, "T = %lld is negative", T);
    if (T > c.max_T) return fail(h, GDN_ERR_ARG, "T = %lld exceeds max_T = %lld", T, c.max_T);
    const long long row = 2LL * c.H * c.d_k + (long long)c.H * c.d_v;
    if (token_stride < row)
        return fail(h, GDN_ERR_ARG, "token_stride = %lld is below the packed row of %lld elements (2 H d_k + H d_v)",
                    token_stride, row);
    if (batch_stride < 0) return fail(h, GDN_ERR_ARG, "batch_stride = %lld is negative", batch_stride);
    if (token_stride > MAX_TOKEN_STRIDE)
        return fail(h, GDN_ERR_UNSUPPORTED, "token_stride = %lld exceeds %lld elements", token_stride,
                    MAX_TOKEN_STRIDE);
    const size_t es = gdn::io_in_bytes(c.io_dtype);
    if ((token_stride * (long long)es) % 16 || (batch_stride * (long long)es) % 16)
        return fail(h, GDN_ERR_ALIGN, "token_stride and batch_stride must be multiples of 16 bytes (%zu elements)",
                    16 / es);
    const size_t tok = (size_t)c.B * (size_t)T * (size_t)c.H;
    const size_t g_bytes = tok * sizeof(float);
    *out_bytes = tok * c.d_v * gdn::io_out_bytes(c.io_dtype);
    *in = Inputs{};
    const char *base = static_cast<const char *>(qkv);
    in->q = qkv;
    in->k = base ? base + (size_t)c.H * c.d_k * es : nullptr;
    in->v = base ? base + 2 * (size_t)c.H * c.d_k * es : nullptr;
    in->qk_ts = in->v_ts = token_stride;
    in->qk_bs = in->v_bs = batch_stride;
    in->beta = beta_logit; in->decay = decay_logit; in->prologue = 1;
    if (T == 0) return GDN_OK;
    if (!qkv || !beta_logit || !decay_logit || !out)
        return fail(h, GDN_ERR_ARG, "qkv, beta_logit, decay_logit and out must be non-NULL when T > 0");
    if (reinterpret_cast<uintptr_t>(qkv) % 16) return fail(h, GDN_ERR_ALIGN, "qkv is not 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(out) % 16) return fail(h, GDN_ERR_ALIGN, "out is not 16-byte aligned");
    int st = check_gate_ptrs(h, beta_logit, decay_logit, "beta_logit", "decay_logit");
    if (st) return st;
    const double ext = ((double)(c.B - 1) * batch_stride + (double)(T - 1) * token_stride + row) * es;
    if (ext > 9.0e18) return fail(h, GDN_ERR_ARG, "the qkv extent is too large");
    const size_t qkv_bytes = (size_t)((c.B - 1) * batch_stride + (T - 1) * token_stride + row) * es;
    in->in[0] = rng("qkv", qkv, qkv_bytes);
    in->in[1] = rng("beta_logit", beta_logit, g_bytes);
    in->in[2] = rng("decay_logit", decay_logit, g_bytes);
    in->n_in = 3;
    const void *dp[] = {qkv, beta_logit, decay_logit};
    const char *dn[] = {"qkv", "beta_logit", "decay_logit"};
    for (int i = 0; i < 3; ++i) {
        in->dev_ptrs[i] = dp[i];
        in->dev_names[i] = dn[i];
    }
    in->n_dev = 3;
    return GDN_OK;
}

int check_aliasing(gdn_ctx *h, const Range *outs, int n_out, const Range *ins, int n_in,
                   const void *state_in, const void *state_out) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(h, GDN_ERR_ALIAS, "%s overlaps %s", outs[i].name, outs[j].name);
        for (int j = 0; j < n_in; ++j) {
            if (overlap(outs[i], ins[j])) {
                const bool inplace_state = state_out && state_in == state_out &&
                                           outs[i].lo == reinterpret_cast<uintptr_t>(state_out) &&
                                           ins[j].lo == reinterpret_cast<uintptr_t>(state_in);
                if (!inplace_state)
                    return fail(h, GDN_ERR_ALIAS, "%s overlaps input %s", outs[i].name, ins[j].name);
            }
        }
    }
    return GDN_OK;
}

int launch_status(gdn_ctx *h, hipError_t e, const char *what) {
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(h, GDN_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    }
    return GDN_OK;
}

int resolve_chunk(gdn_ctx *h, int chunk_len, int *C) {
    if (chunk_len == 0) chunk_len = 64;
    if (chunk_len == 1) {
        *C = 1;
        return GDN_OK;
    }
    if (!gdn::chunk_supported(chunk_len, h->cfg.d_k, h->cfg.d_v, h->cfg.io_dtype))
        return fail(h, GDN_ERR_UNSUPPORTED,
                    "chunk_len = %d is not supported for d_k = %d, d_v = %d, io_dtype = %d "
                    "(use 1 for the sequential scan, 16, 32, 64 or 128 (0 = 64) for the chunked form)",
                    chunk_len, h->cfg.d_k, h->cfg.d_v, h->cfg.io_dtype);
    *C = chunk_len;
    return GDN_OK;
}

// The checks of a configuration that need no device: shapes, dtype, flags (any
// bit outside `allowed` is refused), sizes.  Returns a status; the message goes to err.
int check_config(const gdn_config &c, unsigned allowed, char *err) {
    auto bad = [err](int code, const char *fmt, ...) {
        va_list ap;
        va_start(ap, fmt);
        set_err(err, code, fmt, ap);
        va_end(ap);
        return code;
    };
    if (c.B < 1 || c.H < 1) return bad(GDN_ERR_ARG, "B = %d and H = %d must be >= 1", c.B, c.H);
    // The scan and the general chunked kernel index (direction, b) by the grid's z
    // dimension, at most 65535: two directions per b on bidirectional handles.
    if (c.B > MAX_B) return bad(GDN_ERR_UNSUPPORTED, "B = %d is too large (at most %d)", c.B, MAX_B);
    if (!valid_dim(c.d_k) || !valid_dim(c.d_v))
        return bad(GDN_ERR_UNSUPPORTED, "d_k = %d, d_v = %d: each must be 16, 32, 64 or 128", c.d_k, c.d_v);
    if (c.io_dtype != GDN_F32 && c.io_dtype != GDN_BF16 && c.io_dtype != GDN_FP8)
        return bad(GDN_ERR_UNSUPPORTED, "io_dtype = %d is not GDN_F32, GDN_BF16 or GDN_FP8", c.io_dtype);
    if (c.max_T < 0) return bad(GDN_ERR_ARG, "max_T = %lld is negative", c.max_T);
    if (c.device < -1) return bad(GDN_ERR_ARG, "device = %d", c.device);
    if (c.flags & ~allowed) return bad(GDN_ERR_ARG, "unknown or unsupported flags 0x%x", c.flags);
    if ((long long)c.H * (c.d_k > c.d_v ? c.d_k : c.d_v) > MAX_TOKEN_STRIDE / 3)
        return bad(GDN_ERR_UNSUPPORTED, "H = %d is too large (H * max(d_k, d_v) * 3 must be <= %lld)", c.H,
                   MAX_TOKEN_STRIDE);
    // Element count guard: B*T*H*d must fit comfortably in 64-bit byte offsets.
    const double elems = (double)c.B * (double)c.max_T * (double)c.H * 128.0 * 4.0;
    if (elems > 9.0e18) return bad(GDN_ERR_ARG, "B*max_T*H is too large");
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_version(void) { return "0.2.0"; }

int gdn_create(const gdn_config *cfg, gdn_handle *out_h) {
    if (out_h) *out_h = nullptr;
    if (!cfg || !out_h) return fail_create(GDN_ERR_ARG, "cfg and out_h must be non-NULL");
    const gdn_config c = *cfg;
    if (int st = check_config(c, GDN_FLAG_BIDI | GDN_FLAG_SEGMENTS, g_create_err)) {
        fprintf(stderr, "gdn_create failed: %s\n", g_create_err);
        return st;
    }

    size_t scratch_bytes = 0;
    if (c.flags & GDN_FLAG_BIDI)
        scratch_bytes = 2 * (size_t)c.B * (size_t)c.max_T * c.H * c.d_v * sizeof(float) +
                        2 * (size_t)c.B * c.H * c.d_v * c.d_k * sizeof(float);
    // The MFMA chunked kernel (bf16 or FP8 inputs, chunk 64, d_k and d_v >= 32) forms each
    // chunk's triangular inverse in a pass of its own and reads it back.
    long long tm_chunks = 0;
    if (gdn::chunk_mfma_supported(64, c.d_k, c.d_v, c.io_dtype))
        tm_chunks = ((c.flags & GDN_FLAG_BIDI) ? 2LL : 1LL) * c.B * c.H * ((c.max_T + 63) / 64);
    const size_t tm_bytes = gdn::chunk_mfma_tm_bytes(tm_chunks);

    float *scratch = nullptr;
    uint16_t *tm = nullptr;
    float *seg = nullptr;
    int ncu = 0;
    if (c.device >= 0) {
        int n = 0;
        hipError_t e = hipGetDeviceCount(&n);
        if (e != hipSuccess || n == 0) {
            (void)hipGetLastError();
            return fail_create(GDN_ERR_DEVICE, "no HIP device available (%s)",
                               e != hipSuccess ? hipGetErrorString(e) : "0 devices");
        }
        if (c.device >= n) return fail_create(GDN_ERR_DEVICE, "device %d does not exist (%d devices)", c.device, n);
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, c.device);
        if (e != hipSuccess) return fail_create(GDN_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail_create(GDN_ERR_DEVICE, "device %d is %s; this library is built for gfx950",
                               c.device, prop.gcnArchName);
        ncu = prop.multiProcessorCount;
        if (scratch_bytes) {
            DeviceGuard g(c.device);
            e = hipMalloc(reinterpret_cast<void **>(&scratch), scratch_bytes);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return fail_create(GDN_ERR_OOM, "hipMalloc(%zu bytes) for the bidirectional partials: %s",
                                   scratch_bytes, hipGetErrorString(e));
            }
        }
        if (tm_bytes) {
            DeviceGuard g(c.device);
            e = hipMalloc(reinterpret_cast<void **>(&tm), tm_bytes);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                if (scratch) (void)hipFree(scratch);
                return fail_create(GDN_ERR_OOM, "hipMalloc(%zu bytes) for the per-chunk inverses: %s", tm_bytes,
                                   hipGetErrorString(e));
            }
        }
        // The segment buffers, only where two segments fit on the device at once; the
        // identity matrices and the zero row are written here, once.
        const long long bm = (long long)c.B * c.H * (c.d_v / 32), bi = (long long)c.B * c.H * (c.d_k / 32);
        if ((c.flags & GDN_FLAG_SEGMENTS) && tm_bytes && 2 * bm + bi <= ncu) {
            DeviceGuard g(c.device);
            const SegLayout l = seg_layout(c);
            e = hipMalloc(reinterpret_cast<void **>(&seg), l.total * sizeof(float));
            if (e == hipSuccess) {
                std::vector<float> host(l.total - l.eye, 0.0f);
                const size_t n_rows = (size_t)c.B * c.H * c.d_k;  // row r of matrix r / d_k: 1 at column r % d_k
                for (size_t r = 0; r < n_rows; ++r) host[r * c.d_k + r % c.d_k] = 1.0f;
                e = hipMemcpy(seg + l.eye, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice);
            }
            if (e != hipSuccess) {
                (void)hipGetLastError();
                if (seg) (void)hipFree(seg);
                if (tm) (void)hipFree(tm);
                if (scratch) (void)hipFree(scratch);
                return fail_create(GDN_ERR_OOM, "the segment buffers (%zu bytes): %s", l.total * sizeof(float),
                                   hipGetErrorString(e));
            }
        }
    }
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_join_mid = nullptr;
    if (c.device >= 0 && (c.flags & GDN_FLAG_BIDI) && tm_chunks > 0) {
        DeviceGuard g(c.device);
        hipError_t e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_join, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&ev_join_mid, hipEventDisableTiming);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            if (ev_join) (void)hipEventDestroy(ev_join);
            if (ev_fork) (void)hipEventDestroy(ev_fork);
            if (side) (void)hipStreamDestroy(side);
            if (seg) (void)hipFree(seg);
            if (scratch) (void)hipFree(scratch);
            if (tm) (void)hipFree(tm);
            return fail_create(GDN_ERR_DEVICE, "creating the bidirectional side stream: %s", hipGetErrorString(e));
        }
    }
    gdn_ctx *h = new (std::nothrow) gdn_ctx;
    if (!h) {
        if (ev_join_mid) (void)hipEventDestroy(ev_join_mid);
        if (ev_join) (void)hipEventDestroy(ev_join);
        if (ev_fork) (void)hipEventDestroy(ev_fork);
        if (side) (void)hipStreamDestroy(side);
        if (seg) (void)hipFree(seg);
        if (scratch) (void)hipFree(scratch);
        if (tm) (void)hipFree(tm);
        return fail_create(GDN_ERR_OOM, "out of host memory");
    }
    h->cfg = c;
    h->scratch = scratch;
    h->scratch_bytes = scratch_bytes;
    h->tm = tm;
    h->tm_chunks = tm ? tm_chunks : 0;
    h->side = side;
    h->ev_fork = ev_fork;
    h->ev_join = ev_join;
    h->ev_join_mid = ev_join_mid;
    h->seg = seg;
    h->ncu = ncu;
    *out_h = h;
    g_create_err[0] = 0;
    return GDN_OK;
}

void gdn_free(gdn_handle h) {
    if (!h) return;
    if (h->scratch || h->tm || h->side || h->seg) {
        DeviceGuard g(h->cfg.device);
        if (h->seg) (void)hipFree(h->seg);
        if (h->ev_join_mid) (void)hipEventDestroy(h->ev_join_mid);
        if (h->ev_join) (void)hipEventDestroy(h->ev_join);
        if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
        if (h->side) (void)hipStreamDestroy(h->side);
        if (h->scratch) (void)hipFree(h->scratch);
        if (h->tm) (void)hipFree(h->tm);
    }
    delete h;
}

const char *gdn_last_error(gdn_handle h) { return h ? h->err : g_create_err; }

}  // extern "C"

namespace {

// Segment-parallel causal form: the largest segment count whose blocks (each
// segment's d_v tiles, and each later segment's identity run over d_k tiles) fit on
// the device's CUs at once, with segments of at least SEG_MIN_CHUNKS chunks.  Leaves
// a.nseg = 0 (one sweep) when fewer than two segments fit.
void set_segments(const gdn_ctx *h, gdn::PassArgs &a) {
    const gdn_config &c = h->cfg;
    const long long n = (a.T + 63) / 64;
    const long long bm = (long long)c.B * c.H * (c.d_v / 32), bi = (long long)c.B * c.H * (c.d_k / 32);
    int p = 1;
    for (int q = 2; q <= SEG_MAX; ++q)
        if (q * bm + (q - 1) * bi <= h->ncu && n / q >= SEG_MIN_CHUNKS) p = q;
    if (p < 2) return;
    const int len = (int)((n + p - 1) / p);
    const int nseg = (int)((n + len - 1) / len);  // no empty segment
    // the combine's grid rows: (nseg - 1) runs of 2 chunks per segment, plus one
    if (nseg < 2 || (long long)(nseg - 1) * ((len + 1) / 2) + 1 > 65535) return;
    const SegLayout l = seg_layout(c);
    a.nseg = nseg;
    a.seg_len = len;
    a.seg_partial = h->seg + l.partial;
    a.seg_w = h->seg + l.w;
    a.seg_sloc = h->seg + l.sloc;
    a.seg_phi = h->seg + l.phi;
    a.seg_eye = h->seg + l.eye;
    a.seg_vzero = h->seg + l.vzero;
}

gdn::PassArgs pass_args(const gdn_ctx *h, const Inputs &in, long long T) {
    const gdn_config &c = h->cfg;
    gdn::PassArgs a{};
    a.q = in.q; a.k = in.k; a.v = in.v;
    a.qk_ts = in.qk_ts; a.qk_bs = in.qk_bs; a.v_ts = in.v_ts; a.v_bs = in.v_bs;
    a.beta = in.beta; a.decay = in.decay; a.prologue = in.prologue;
    a.B = c.B; a.H = c.H; a.dk = c.d_k; a.dv = c.d_v; a.T = T;
    a.io = c.io_dtype;  // gdn_dtype and gdn::IoType share their values
    a.tm = h->tm; a.tm_chunks = h->tm_chunks;
    return a;
}

int run_forward(gdn_ctx *h, const Inputs &in, const float *state_in, float *state_out, void *out,
                size_t out_bytes, long long T, int chunk_len, void *hip_stream) {
    const gdn_config &c = h->cfg;
    int st, C = 0;
    if ((st = resolve_chunk(h, chunk_len, &C))) return st;
    const size_t s_bytes = (size_t)c.B * c.H * c.d_v * c.d_k * sizeof(float);
    if ((state_in && reinterpret_cast<uintptr_t>(state_in) % 16) ||
        (state_out && reinterpret_cast<uintptr_t>(state_out) % 16))
        return fail(h, GDN_ERR_ALIGN, "state_in/state_out are not 16-byte aligned");
    const bool tok = T > 0;
    Range outs[2];
    int n_out = 0;
    if (tok) outs[n_out++] = rng("out", out, out_bytes);
    if (state_out) outs[n_out++] = rng("state_out", state_out, s_bytes);
    Range ins[6];
    int n_in = 0;
    if (tok)
        for (int i = 0; i < in.n_in; ++i) ins[n_in++] = in.in[i];
    if (state_in) ins[n_in++] = rng("state_in", state_in, s_bytes);
    if ((st = check_aliasing(h, outs, n_out, ins, n_in, state_in, state_out))) return st;
    if (c.device < 0) return GDN_OK;  // dry run: validated, nothing launched

    if (tok) {
        for (int i = 0; i < in.n_dev; ++i)
            if ((st = check_device_ptr(h, in.dev_names[i], in.dev_ptrs[i]))) return st;
        if ((st = check_device_ptr(h, "out", out))) return st;
    }
    if ((st = check_device_ptr(h, "state_in", state_in))) return st;
    if ((st = check_device_ptr(h, "state_out", state_out))) return st;
    if (!tok && !state_out) return GDN_OK;  // nothing to compute or write

    DeviceGuard g(c.device);
    gdn::PassArgs a = pass_args(h, in, T);
    a.state_in = state_in; a.state_out = state_out; a.out = out; a.partial = nullptr;
    a.reverse = 0; a.out_mode = gdn::OUT_STORE;
    if (h->seg && tok && C != 1 && gdn::chunk_mfma_supported(C, c.d_k, c.d_v, c.io_dtype)) set_segments(h, a);
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    // With no tokens only the state is written (state_in copied, or zeros).  The
    // scan kernel does exactly that for every shape and input type without reading
    // q, k, v or the gates; the chunked kernels need at least one token.
    const bool scan = C == 1 || !tok;
    hipError_t e = scan ? gdn::launch_scan(a, s) : gdn::launch_chunk(a, C, s);
    return launch_status(h, e, scan ? "scan" : "chunked");
}

int run_bidi(gdn_ctx *h, const Inputs &in, void *out, size_t out_bytes, long long T, int chunk_len,
             void *hip_stream) {
    const gdn_config &c = h->cfg;
    int st, C = 0;
    if ((st = resolve_chunk(h, chunk_len, &C))) return st;
    if (T == 0) return GDN_OK;
    Range outs[1] = {rng("out", out, out_bytes)};
    if ((st = check_aliasing(h, outs, 1, in.in, in.n_in, nullptr, nullptr))) return st;
    if (c.device < 0) return GDN_OK;
    for (int i = 0; i < in.n_dev; ++i)
        if ((st = check_device_ptr(h, in.dev_names[i], in.dev_ptrs[i]))) return st;
    if ((st = check_device_ptr(h, "out", out))) return st;

    DeviceGuard g(c.device);
    gdn::PassArgs a = pass_args(h, in, T);
    const size_t n_out = (size_t)c.B * (size_t)T * c.H * c.d_v;
    a.state_in = nullptr; a.state_out = nullptr; a.out = out;
    a.partial = h->scratch;
    a.partial_rev = h->scratch + (size_t)c.B * (size_t)c.max_T * c.H * c.d_v;
    hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
    // Both directions run concurrently (the reverse direction walks the tokens from
    // T-1 down, chunk grid anchored there), and out = round(forward + reverse): one
    // rounding, and fp32 addition is commutative, so reversing the inputs reverses
    // the output exactly.  The MFMA chunked kernel splits its sweeps at the middle
    // chunk, keeps the first half's outputs as bf16 rows and adds the other
    // direction's output itself; the other kernels write both fp32 partials in one
    // launch and a combine pass adds them.
    a.reverse = 0;
    a.both_dirs = 1;
    a.out_mode = gdn::OUT_PARTIAL;
    const bool split = C != 1 && gdn::chunk_mfma_supported(C, c.d_k, c.d_v, c.io_dtype);
    if (split) {
        a.bidi_state = a.partial_rev + (size_t)c.B * (size_t)c.max_T * c.H * c.d_v;
        a.side_stream = h->side;
        a.ev_fork = h->ev_fork;
        a.ev_join = h->ev_join;
        a.ev_join_mid = h->ev_join_mid;
    }
    hipError_t e = (C == 1) ? gdn::launch_scan(a, s) : gdn::launch_chunk(a, C, s);
    if ((st = launch_status(h, e, "bidirectional pass"))) return st;
    if (split) return GDN_OK;
    e = gdn::launch_combine(out, a.partial, a.partial_rev, (long long)n_out, a.io, s);
    return launch_status(h, e, "bidirectional combine");
}

int need_bidi(gdn_ctx *h, const char *fn) {
    if (!(h->cfg.flags & GDN_FLAG_BIDI))
        return fail(h, GDN_ERR_ARG, "%s needs a handle created with GDN_FLAG_BIDI", fn);
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_forward(gdn_handle h, const void *q, const void *k, const void *v, const float *beta,
                const float *decay, const float *state_in, float *state_out, void *out, long long T,
                int chunk_len, void *hip_stream) {
    if (!h) {
        snprintf(g_create_err, ERR_LEN, "gdn_forward: NULL handle");
        return GDN_ERR_ARG;
    }
    h->err[0] = 0;
    Inputs in;
    size_t out_bytes;
    int st = prepare_plain(h, q, k, v, beta, decay, out, T, &in, &out_bytes);
    if (st) return st;
    return run_forward(h, in, state_in, state_out, out, out_bytes, T, chunk_len, hip_stream);
}

int gdn_forward_packed(gdn_handle h, const void *qkv, long long token_stride, long long batch_stride,
                       const float *beta_logit, const float *decay_logit, const float *state_in,
                       float *state_out, void *out, long long T, int chunk_len, void *hip_stream) {
    if (!h) {
        snprintf(g_create_err, ERR_LEN, "gdn_forward_packed: NULL handle");
        return GDN_ERR_ARG;
    }
    h->err[0] = 0;
    Inputs in;
    size_t out_bytes;
    int st = prepare_packed(h, qkv, token_stride, batch_stride, beta_logit, decay_logit, out, T, &in, &out_bytes);
    if (st) return st;
    return run_forward(h, in, state_in, state_out, out, out_bytes, T, chunk_len, hip_stream);
}

int gdn_forward_bidi(gdn_handle h, const void *q, const void *k, const void *v, const float *beta,
                     const float *decay, void *out, long long T, int chunk_len, void *hip_stream) {
    if (!h) {
        snprintf(g_create_err, ERR_LEN, "gdn_forward_bidi: NULL handle");
        return GDN_ERR_ARG;
    }
    h->err[0] = 0;
    int st = need_bidi(h, "gdn_forward_bidi");
    if (st) return st;
    Inputs in;
    size_t out_bytes;
    if ((st = prepare_plain(h, q, k, v, beta, decay, out, T, &in, &out_bytes))) return st;
    return run_bidi(h, in, out, out_bytes, T, chunk_len, hip_stream);
}

int gdn_forward_bidi_packed(gdn_handle h, const void *qkv, long long token_stride, long long batch_stride,
                            const float *beta_logit, const float *decay_logit, void *out, long long T,
                            int chunk_len, void *hip_stream) {
    if (!h) {
        snprintf(g_create_err, ERR_LEN, "gdn_forward_bidi_packed: NULL handle");
        return GDN_ERR_ARG;
    }
    h->err[0] = 0;
    int st = need_bidi(h, "gdn_forward_bidi_packed");
    if (st) return st;
    Inputs in;
    size_t out_bytes;
    if ((st = prepare_packed(h, qkv, token_stride, batch_stride, beta_logit, decay_logit, out, T, &in,
                             &out_bytes)))
        return st;
    return run_bidi(h, in, out, out_bytes, T, chunk_len, hip_stream);
}

// No handle and no allocation: the configuration comes with the call and the
// MFMA chunked kernel's per-chunk scratch is the fixed device array of
// gdn_static.hip.  Messages go to the thread's handle-less buffer
// (gdn_last_error(NULL)).
int gdn_forward_noalloc(const gdn_config *cfg, const void *q, const void *k, const void *v, const float *beta,
                        const float *decay, const float *state_in, float *state_out, void *out, long long T,
                        int chunk_len, void *hip_stream) {
    if (!cfg) {
        snprintf(g_create_err, ERR_LEN, "gdn_forward_noalloc: cfg must be non-NULL");
        return GDN_ERR_ARG;
    }
    gdn_ctx ctx;
    ctx.cfg = *cfg;
    ctx.cfg.max_T = T < 0 ? 0 : T;  // the limit is the fixed scratch, checked below
    g_create_err[0] = 0;
    int st = check_config(ctx.cfg, 0u, g_create_err);
    if (st) return st;
    const gdn_config &c = ctx.cfg;
    const int C = chunk_len == 0 ? 64 : chunk_len;
    const long long per_chunk = (long long)gdn::chunk_mfma_tm_bytes(1);
    const long long capacity = (long long)gdn::STATIC_SCRATCH_BYTES / per_chunk;
    if (T > 0 && C != 1 && gdn::chunk_mfma_supported(C, c.d_k, c.d_v, c.io_dtype)) {
        const long long need = (long long)c.B * c.H * ((T + 63) / 64);
        if (need > capacity) {
            snprintf(g_create_err, ERR_LEN,
                     "gdn_forward_noalloc: B * H * ceil(T / 64) = %lld chunks need %lld bytes of scratch; the fixed "
                     "array holds %zu bytes (%lld chunks): split the call over tokens or heads, or use gdn_forward",
                     need, need * per_chunk, gdn::STATIC_SCRATCH_BYTES, capacity);
            return GDN_ERR_UNSUPPORTED;
        }
    }
    if (c.device >= 0) {
        void *ptr = nullptr;
        bool gfx950 = false;
        const hipError_t e = gdn::static_scratch(c.device, &ptr, &gfx950);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            snprintf(g_create_err, ERR_LEN, "gdn_forward_noalloc: device %d: %s", c.device, hipGetErrorString(e));
            return GDN_ERR_DEVICE;
        }
        if (!gfx950) {
            snprintf(g_create_err, ERR_LEN, "gdn_forward_noalloc: device %d is not a gfx950", c.device);
            return GDN_ERR_DEVICE;
        }
        ctx.tm = static_cast<uint16_t *>(ptr);
        ctx.tm_chunks = capacity;
    }
    Inputs in;
    size_t out_bytes;
    st = prepare_plain(&ctx, q, k, v, beta, decay, out, T, &in, &out_bytes);
    if (!st) st = run_forward(&ctx, in, state_in, state_out, out, out_bytes, T, chunk_len, hip_stream);
    if (st) snprintf(g_create_err, ERR_LEN, "%s", ctx.err);
    return st;
}

}  // extern "C"
