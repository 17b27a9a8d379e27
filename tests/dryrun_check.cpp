// The C ABI's host-side validation with no GPU: dry-run handles (device = -1)
// and gdn_forward_noalloc's dry run check every argument and launch nothing, so
// the pointers here are fake, well-separated addresses that are never
// dereferenced.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code (the library's C-ABI layer is compiled into this program), so an
// out-of-range access, overflow or leak in the validation fails the run.  Exit
// status 0 and a final "dry-run check ok" line when every case gives the
// expected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "gdn.h"

namespace {

int g_fail = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond);  \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

const uintptr_t BASE = 1ull << 40, GiB = 1ull << 30;
void *addr(int i, uintptr_t off = 0) { return reinterpret_cast<void *>(BASE + (uintptr_t)i * GiB + off); }
float *faddr(int i, uintptr_t off = 0) { return static_cast<float *>(addr(i, off)); }

gdn_config cfg(int B, int H, int dk, int dv, int io, long long max_T, unsigned flags, int device = -1) {
    gdn_config c;
    c.device = device;
    c.B = B;
    c.H = H;
    c.d_k = dk;
    c.d_v = dv;
    c.io_dtype = io;
    c.max_T = max_T;
    c.flags = flags;
    return c;
}

int fwd(gdn_handle h, long long T, int chunk, void *q = addr(0), void *out = addr(7), float *s_in = faddr(5),
        float *s_out = faddr(6)) {
    return gdn_forward(h, q, addr(1), addr(2), faddr(3), faddr(4), s_in, s_out, out, T, chunk, nullptr);
}

void causal_cases() {
    gdn_handle h = nullptr;
    gdn_config c = cfg(2, 3, 64, 32, GDN_BF16, 1000, GDN_FLAG_BIDI);
    EXPECT(gdn_create(&c, &h) == GDN_OK && h);
    for (int chunk : {0, 1, 16, 32, 64, 128}) EXPECT(fwd(h, 1000, chunk) == GDN_OK);
    EXPECT(fwd(h, 0, 64, nullptr, nullptr) == GDN_OK);  // T = 0 may pass NULL tokens and out
    EXPECT(fwd(h, 100, 64, addr(0), addr(7), faddr(5), faddr(5)) == GDN_OK);  // in-place state
    EXPECT(fwd(h, 100, 64, addr(0), addr(7), nullptr, nullptr) == GDN_OK);
    EXPECT(fwd(h, -1, 64) == GDN_ERR_ARG);
    EXPECT(fwd(h, 1001, 64) == GDN_ERR_ARG);
    EXPECT(fwd(h, 100, 3) == GDN_ERR_UNSUPPORTED);
    EXPECT(fwd(h, 100, 256) == GDN_ERR_UNSUPPORTED);
    EXPECT(fwd(h, 100, 64, addr(0, 2)) == GDN_ERR_ALIGN);
    EXPECT(fwd(h, 100, 64, nullptr) == GDN_ERR_ARG);
    EXPECT(fwd(h, 100, 64, addr(0), addr(0)) == GDN_ERR_ALIAS);                    // out == q
    EXPECT(fwd(h, 100, 64, addr(0), addr(7), faddr(5), faddr(5, 16)) == GDN_ERR_ALIAS);  // partial overlap
    EXPECT(fwd(h, 100, 64, addr(0), addr(7), faddr(5), faddr(7, 64)) == GDN_ERR_ALIAS);  // state_out in out
    EXPECT(std::strlen(gdn_last_error(h)) > 0);
    // bidirectional
    EXPECT(gdn_forward_bidi(h, addr(0), addr(1), addr(2), faddr(3), faddr(4), addr(7), 999, 64, nullptr) == GDN_OK);
    EXPECT(gdn_forward_bidi(h, addr(0), addr(1), addr(2), faddr(3), faddr(4), addr(1), 999, 64, nullptr) ==
           GDN_ERR_ALIAS);
    // packed prologue: row = 2 H d_k + H d_v = 480 elements
    EXPECT(gdn_forward_packed(h, addr(0), 480, 480 * 1000, faddr(3), faddr(4), nullptr, faddr(6), addr(7), 1000, 64,
                              nullptr) == GDN_OK);
    EXPECT(gdn_forward_packed(h, addr(0), 479, 0, faddr(3), faddr(4), nullptr, nullptr, addr(7), 10, 64, nullptr) ==
           GDN_ERR_ARG);
    EXPECT(gdn_forward_packed(h, addr(0), 484, 0, faddr(3), faddr(4), nullptr, nullptr, addr(7), 10, 64, nullptr) ==
           GDN_ERR_ALIGN);
    EXPECT(gdn_forward_packed(h, addr(0), 1ll << 25, 0, faddr(3), faddr(4), nullptr, nullptr, addr(7), 10, 64,
                              nullptr) == GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_forward_bidi_packed(h, addr(0), 480, 0, faddr(3), faddr(4), addr(7), 1000, 1, nullptr) == GDN_OK);
    gdn_free(h);

    gdn_config c2 = cfg(1, 2, 16, 16, GDN_F32, 10, 0);
    EXPECT(gdn_create(&c2, &h) == GDN_OK);
    EXPECT(gdn_forward_bidi(h, addr(0), addr(1), addr(2), faddr(3), faddr(4), addr(7), 10, 1, nullptr) ==
           GDN_ERR_ARG);  // no GDN_FLAG_BIDI
    gdn_free(h);
}

void create_cases() {
    gdn_handle h = reinterpret_cast<gdn_handle>(addr(9));
    gdn_config bad[] = {cfg(0, 1, 16, 16, GDN_F32, 10, 0),      cfg(1, 0, 16, 16, GDN_F32, 10, 0),
                        cfg(40000, 1, 16, 16, GDN_F32, 10, 0),  cfg(1, 1, 48, 16, GDN_F32, 10, 0),
                        cfg(1, 1, 16, 256, GDN_F32, 10, 0),     cfg(1, 1, 16, 16, 7, 10, 0),
                        cfg(1, 1, 16, 16, GDN_F32, -1, 0),      cfg(1, 1, 16, 16, GDN_F32, 10, 8),
                        cfg(1, 1 << 20, 128, 128, GDN_F32, 10, 0), cfg(1, 1, 16, 16, GDN_F32, 1ll << 60, 0)};
    for (const gdn_config &b : bad) {
        EXPECT(gdn_create(&b, &h) < 0);
        EXPECT(h == nullptr);
        EXPECT(std::strlen(gdn_last_error(nullptr)) > 0);
        h = reinterpret_cast<gdn_handle>(addr(9));
    }
    EXPECT(gdn_create(nullptr, &h) == GDN_ERR_ARG);
    gdn_config ok = cfg(1, 1, 16, 16, GDN_F32, 10, 0);
    EXPECT(gdn_create(&ok, nullptr) == GDN_ERR_ARG);
    gdn_free(nullptr);
    EXPECT(gdn_forward(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1,
                       nullptr) == GDN_ERR_ARG);
    EXPECT(std::strlen(gdn_version()) >= 5);
}

void noalloc_cases() {
    gdn_config c = cfg(2, 3, 64, 32, GDN_BF16, 0, 0);
    auto na = [&](const gdn_config &cc, long long T, int chunk, void *out = addr(7)) {
        return gdn_forward_noalloc(&cc, addr(0), addr(1), addr(2), faddr(3), faddr(4), faddr(5), faddr(6), out, T,
                                   chunk, nullptr);
    };
    EXPECT(na(c, 1000, 64) == GDN_OK);
    EXPECT(na(c, 1000, 1) == GDN_OK);
    EXPECT(na(c, 1000, 7) == GDN_ERR_UNSUPPORTED);
    EXPECT(na(c, 1000, 64, addr(0)) == GDN_ERR_ALIAS);
    gdn_config big = cfg(1, 20, 128, 128, GDN_BF16, 0, 0);
    // the fixed array holds 10,922 chunk records: 20 heads x 546 chunks fit, 547 do not
    EXPECT(na(big, 34944, 64) == GDN_OK);
    EXPECT(na(big, 34945, 64) == GDN_ERR_UNSUPPORTED);
    EXPECT(std::strstr(gdn_last_error(nullptr), "scratch") != nullptr);
    EXPECT(na(big, 100000, 1) == GDN_OK);
    gdn_config bidi = cfg(1, 2, 64, 64, GDN_BF16, 0, GDN_FLAG_BIDI);
    EXPECT(na(bidi, 10, 64) == GDN_ERR_ARG);
    EXPECT(gdn_forward_noalloc(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1,
                               nullptr) == GDN_ERR_ARG);
}

}  // namespace

int main() {
    causal_cases();
    create_cases();
    noalloc_cases();
    if (g_fail) {
        std::printf("dry-run check: %d failure(s)\n", g_fail);
        return 1;
    }
    std::printf("dry-run check ok\n");
    return 0;
}
