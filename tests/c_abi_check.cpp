// The C ABI used from C++ with no Python or torch in the process: device buffers
// from hipMalloc, inputs from a fixed pseudo-random sequence, and two closed forms
// that hold at any length, checked on the host for the scan, the fp32 chunked
// kernel and the bf16 MFMA chunked kernel:
//   a = 0 at every token:  o_t = b_t (k_t . q_t) v_t / sqrt(d_k),  S_T = b_T v_T k_T^T
//   b = 0, a = 1:          o_t = S_0 q_t / sqrt(d_k),  state_out == state_in bit for bit
// plus the error path (an unsupported chunk length, a host pointer).  Exit status 0
// and a final "ok" line when every case passes.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn.h"

namespace {

uint32_t g_rng = 12345u;
float uniform() {  // in [-1, 1)
    g_rng = g_rng * 1664525u + 1013904223u;
    return (float)((g_rng >> 8) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
}
uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
    uint32_t u;
    std::memcpy(&u, &x, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
float from_bf16(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return x;
}
double rel_l2(const std::vector<double> &got, const std::vector<double> &want) {
    double num = 0, den = 0;
    for (size_t i = 0; i < got.size(); ++i) {
        num += (got[i] - want[i]) * (got[i] - want[i]);
        den += want[i] * want[i];
    }
    return std::sqrt(num / (den > 0 ? den : 1));
}

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        const hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                       \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

// One (input type, chunk length) case of both closed forms.  Returns 0 on success.
int run_case(int io, int chunk) {
    const int B = 1, H = 2, dk = 64, dv = 64;
    const long long T = 130;
    const size_t nqk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv, ng = (size_t)B * T * H;
    const size_t ns = (size_t)B * H * dv * dk;
    const bool bf16 = io == GDN_BF16;
    const size_t es = bf16 ? 2 : 4;
    const double tol = bf16 ? 1e-2 : 1e-5;

    // inputs as the device will see them (bf16-rounded for bf16), kept in fp32 here
    std::vector<float> q(nqk), k(nqk), v(nv), beta(ng), s0(ns);
    for (auto &x : q) x = uniform();
    for (auto &x : k) x = uniform();
    for (auto &x : v) x = uniform();
    for (auto &x : beta) x = 0.5f + 0.4f * uniform();
    for (auto &x : s0) x = 0.3f * uniform();
    std::vector<uint16_t> qh(nqk), kh(nqk), vh(nv);
    if (bf16) {
        for (size_t i = 0; i < nqk; ++i) {
            qh[i] = to_bf16(q[i]);
            q[i] = from_bf16(qh[i]);
            kh[i] = to_bf16(k[i]);
            k[i] = from_bf16(kh[i]);
        }
        for (size_t i = 0; i < nv; ++i) {
            vh[i] = to_bf16(v[i]);
            v[i] = from_bf16(vh[i]);
        }
    }
    const std::vector<float> zeros(ng, 0.0f), ones(ng, 1.0f);

    gdn_config cfg{};
    cfg.device = 0;
    cfg.B = B;
    cfg.H = H;
    cfg.d_k = dk;
    cfg.d_v = dv;
    cfg.io_dtype = io;
    cfg.max_T = T;
    gdn_handle h = nullptr;
    if (gdn_create(&cfg, &h) != GDN_OK) {
        std::fprintf(stderr, "gdn_create: %s\n", gdn_last_error(nullptr));
        return 1;
    }
    void *dq, *dk_, *dv_, *dout;
    float *dbeta, *ddecay, *ds0, *dst;
    CHECK_HIP(hipMalloc(&dq, nqk * es));
    CHECK_HIP(hipMalloc(&dk_, nqk * es));
    CHECK_HIP(hipMalloc(&dv_, nv * es));
    CHECK_HIP(hipMalloc(&dout, nv * es));
    CHECK_HIP(hipMalloc(&dbeta, ng * 4));
    CHECK_HIP(hipMalloc(&ddecay, ng * 4));
    CHECK_HIP(hipMalloc(&ds0, ns * 4));
    CHECK_HIP(hipMalloc(&dst, ns * 4));
    CHECK_HIP(hipMemcpy(dq, bf16 ? (const void *)qh.data() : q.data(), nqk * es, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk_, bf16 ? (const void *)kh.data() : k.data(), nqk * es, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv_, bf16 ? (const void *)vh.data() : v.data(), nv * es, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ds0, s0.data(), ns * 4, hipMemcpyHostToDevice));

    auto read_out = [&](std::vector<double> &o) -> int {
        o.resize(nv);
        if (bf16) {
            std::vector<uint16_t> oh(nv);
            if (hipMemcpy(oh.data(), dout, nv * 2, hipMemcpyDeviceToHost) != hipSuccess) return 1;
            for (size_t i = 0; i < nv; ++i) o[i] = from_bf16(oh[i]);
        } else {
            std::vector<float> of(nv);
            if (hipMemcpy(of.data(), dout, nv * 4, hipMemcpyDeviceToHost) != hipSuccess) return 1;
            for (size_t i = 0; i < nv; ++i) o[i] = of[i];
        }
        return 0;
    };
    const double scale = 1.0 / std::sqrt((double)dk);
    int fails = 0;

    // a = 0 at every token
    CHECK_HIP(hipMemcpy(dbeta, beta.data(), ng * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ddecay, zeros.data(), ng * 4, hipMemcpyHostToDevice));
    int st = gdn_forward(h, dq, dk_, dv_, dbeta, ddecay, ds0, dst, dout, T, chunk, nullptr);
    CHECK_HIP(hipDeviceSynchronize());
    if (st != GDN_OK) {
        std::fprintf(stderr, "gdn_forward: %s\n", gdn_last_error(h));
        return 1;
    }
    std::vector<double> o, want(nv), sgot(ns), swant(ns);
    if (read_out(o)) return 1;
    for (long long t = 0; t < T; ++t)
        for (int hh = 0; hh < H; ++hh) {
            const size_t r = (size_t)t * H + hh;
            double kq = 0;
            for (int i = 0; i < dk; ++i) kq += (double)k[r * dk + i] * q[r * dk + i];
            for (int i = 0; i < dv; ++i) want[r * dv + i] = beta[r] * kq * v[r * dv + i] * scale;
        }
    {
        std::vector<float> sf(ns);
        CHECK_HIP(hipMemcpy(sf.data(), dst, ns * 4, hipMemcpyDeviceToHost));
        for (int hh = 0; hh < H; ++hh) {
            const size_t r = (size_t)(T - 1) * H + hh;
            for (int i = 0; i < dv; ++i)
                for (int j = 0; j < dk; ++j) {
                    const size_t e = ((size_t)hh * dv + i) * dk + j;
                    sgot[e] = sf[e];
                    swant[e] = (double)beta[r] * v[r * dv + i] * k[r * dk + j];
                }
        }
    }
    const double r1 = rel_l2(o, want), r2 = rel_l2(sgot, swant);
    std::printf("io=%d chunk=%d a=0: rel-L2 out %.3e state %.3e\n", io, chunk, r1, r2);
    fails += !(r1 <= tol && r2 <= tol);

    // b = 0, a = 1 from s0
    CHECK_HIP(hipMemcpy(dbeta, zeros.data(), ng * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(ddecay, ones.data(), ng * 4, hipMemcpyHostToDevice));
    st = gdn_forward(h, dq, dk_, dv_, dbeta, ddecay, ds0, dst, dout, T, chunk, nullptr);
    CHECK_HIP(hipDeviceSynchronize());
    if (st != GDN_OK) {
        std::fprintf(stderr, "gdn_forward: %s\n", gdn_last_error(h));
        return 1;
    }
    if (read_out(o)) return 1;
    for (long long t = 0; t < T; ++t)
        for (int hh = 0; hh < H; ++hh) {
            const size_t r = (size_t)t * H + hh;
            for (int i = 0; i < dv; ++i) {
                double acc = 0;
                for (int j = 0; j < dk; ++j) acc += (double)s0[((size_t)hh * dv + i) * dk + j] * q[r * dk + j];
                want[r * dv + i] = acc * scale;
            }
        }
    std::vector<float> sf(ns);
    CHECK_HIP(hipMemcpy(sf.data(), dst, ns * 4, hipMemcpyDeviceToHost));
    const bool kept = std::memcmp(sf.data(), s0.data(), ns * 4) == 0;
    const double r3 = rel_l2(o, want);
    std::printf("io=%d chunk=%d b=0,a=1: rel-L2 out %.3e, state kept bit for bit: %s\n", io, chunk, r3,
                kept ? "yes" : "no");
    fails += !(r3 <= tol && kept);

    CHECK_HIP(hipFree(dq));
    CHECK_HIP(hipFree(dk_));
    CHECK_HIP(hipFree(dv_));
    CHECK_HIP(hipFree(dout));
    CHECK_HIP(hipFree(dbeta));
    CHECK_HIP(hipFree(ddecay));
    CHECK_HIP(hipFree(ds0));
    CHECK_HIP(hipFree(dst));
    gdn_free(h);
    return fails;
}

// Rejected calls: status codes and a message, nothing launched.
int run_errors() {
    gdn_config cfg{};
    cfg.device = 0;
    cfg.B = 1;
    cfg.H = 1;
    cfg.d_k = 16;
    cfg.d_v = 16;
    cfg.io_dtype = GDN_F32;
    cfg.max_T = 8;
    gdn_handle h = nullptr;
    if (gdn_create(&cfg, &h) != GDN_OK) return 1;
    void *d;
    CHECK_HIP(hipMalloc(&d, 4096));
    float *df = static_cast<float *>(d);
    int fails = 0;
    const int s1 = gdn_forward(h, d, d, d, df, df, nullptr, nullptr, df + 512, 8, 7, nullptr);
    std::printf("chunk_len 7: status %d (%s)\n", s1, gdn_last_error(h));
    fails += !(s1 == GDN_ERR_UNSUPPORTED && std::strlen(gdn_last_error(h)) > 0);
    std::vector<float> host(256, 0.0f);
    const int s2 = gdn_forward(h, host.data(), d, d, df, df, nullptr, nullptr, df + 512, 8, 1, nullptr);
    std::printf("host q: status %d (%s)\n", s2, gdn_last_error(h));
    fails += !(s2 == GDN_ERR_ARG);
    CHECK_HIP(hipFree(d));
    gdn_free(h);
    return fails;
}

}  // namespace

int main() {
    std::printf("%s\n", gdn_version());
    int fails = 0;
    const int cases[][2] = {{GDN_F32, 1}, {GDN_F32, 32}, {GDN_BF16, 64}, {GDN_BF16, 1}};
    for (const auto &c : cases) fails += run_case(c[0], c[1]);
    fails += run_errors();
    if (fails) {
        std::printf("c-abi check FAILED: %d\n", fails);
        return 1;
    }
    std::printf("c-abi check ok\n");
    return 0;
}
