// Exercises the host-side argument validation of every libspecverify entry
// point: each call below must be refused (or be a no-op) before any launch,
// so nothing here needs a GPU.  Built from the library's sources as host
// code only, with AddressSanitizer and UndefinedBehaviorSanitizer, by
// tests/test_sanitizers.py.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>

#include "spec_verify.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int rc_ = (call);                                                         \
        if (rc_ != (want)) {                                                            \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (int)(want)); \
            g_fail = 1;                                                                 \
        }                                                                               \
    } while (0)

int main() {
    // fake device pointers: never dereferenced, every call is refused first
    alignas(16) static char buf[4096];
    void* p = buf;
    const float* fp = reinterpret_cast<const float*>(buf);
    const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
    int32_t* op = reinterpret_cast<int32_t*>(buf);
    float* ofp = reinterpret_cast<float*>(buf);
    const int INV = SPEC_ERR_INVALID_ARG, WS = SPEC_ERR_WORKSPACE;

    // spec_accept / spec_accept_noalloc
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, -1, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 256, 10, 0, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 0, 0, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, 7, fp, ip, ip, 2, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 10, 0, -1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 10, 0, __builtin_nanf(""), 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, nullptr, ip, ip, 2, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 10, ((int64_t)1 << 32) - 1, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, p, 16, nullptr), WS);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 2, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, buf + 1, 4000, nullptr), WS);
    EXPECT(spec_accept(p, SPEC_F32, fp, ip, ip, 0, 2, 10, 0, 1.f, 1, 0, op, op, ofp, op, nullptr, 0, nullptr), SPEC_OK);
    EXPECT(spec_accept_noalloc(p, SPEC_F32, fp, ip, ip, 2048, 5, 151936, 0, 0.6f, 1, 0, op, op, ofp, op, nullptr), WS);
    EXPECT(spec_accept_noalloc(p, SPEC_BF16, fp, ip, ip, -3, 5, 100, 0, 0.6f, 1, 0, op, op, ofp, op, nullptr), INV);
    EXPECT(spec_accept_noalloc(p, SPEC_BF16, fp, ip, ip, 0, 5, 100, 0, 0.6f, 1, 0, op, op, ofp, op, nullptr), SPEC_OK);
    if (spec_accept_workspace_bytes(64, 7, 128256) == 0) g_fail = 1;
    if (spec_accept_workspace_bytes(-1, 7, 128256) != 0) g_fail = 1;

    // spec_accept_sampled
    EXPECT(spec_accept_sampled(p, p, SPEC_BF16, ip, ip, 2, 2, 10, 0, 0.f, 1.f, 0.9f, 0.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept_sampled(p, p, SPEC_BF16, ip, ip, 2, 2, 10, 0, 1.f, 1.f, 1.5f, 0.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept_sampled(p, p, SPEC_BF16, ip, ip, 2, 2, 10, 0, 1.f, 1.f, 0.9f, 1.f, 1, 0, op, op, ofp, op, p, 4096, nullptr), INV);
    EXPECT(spec_accept_sampled(p, p, SPEC_BF16, ip, ip, 2, 2, 10, 0, 1.f, 1.f, 0.9f, 0.1f, 1, 0, op, op, ofp, op, p, 8, nullptr), WS);
    EXPECT(spec_accept_sampled(p, p, SPEC_BF16, ip, ip, 0, 2, 10, 0, 1.f, 1.f, 0.9f, 0.1f, 1, 0, op, op, ofp, op, nullptr, 0, nullptr), SPEC_OK);

    // spec_verify_linear
    EXPECT(spec_verify_linear(p, p, p, SPEC_F32, 4, 12, 64, nullptr, 0, nullptr), INV);   // N % 8
    EXPECT(spec_verify_linear(p, p, p, SPEC_F32, 4, 16, 60, nullptr, 0, nullptr), INV);   // K % 8
    EXPECT(spec_verify_linear(p, p, p, 9, 4, 16, 64, nullptr, 0, nullptr), INV);
    EXPECT(spec_verify_linear(buf + 2, p, p, SPEC_F32, 4, 16, 64, nullptr, 0, nullptr), INV);
    EXPECT(spec_verify_linear(p, p, p, SPEC_F32, 0, 16, 64, nullptr, 0, nullptr), SPEC_OK);
    EXPECT(spec_verify_linear(p, p, p, SPEC_F32, -1, 16, 64, nullptr, 0, nullptr), INV);

    // spec_pack_weight / spec_verify_linear_packed
    EXPECT((int)spec_packed_weight_bytes(96, 16), 0);                                          // K % 64
    EXPECT((int)spec_packed_weight_bytes(128, 33), 4 * 2 * 2048);
    EXPECT(spec_pack_weight(p, p, 96, 16, nullptr), INV);
    EXPECT(spec_pack_weight(p, p, 64, 0, nullptr), INV);
    EXPECT(spec_pack_weight(p, buf + 2, 64, 16, nullptr), INV);
    EXPECT(spec_verify_linear_packed(p, p, p, SPEC_F32, 4, 16, 96, nullptr, 0, nullptr), INV);  // K % 64
    EXPECT(spec_verify_linear_packed(p, p, p, 9, 4, 16, 64, nullptr, 0, nullptr), INV);
    EXPECT(spec_verify_linear_packed(buf + 2, p, p, SPEC_F32, 4, 16, 64, nullptr, 0, nullptr), INV);
    EXPECT(spec_verify_linear_packed(p, p, p, SPEC_F32, 0, 16, 64, nullptr, 0, nullptr), SPEC_OK);
    EXPECT(spec_verify_linear_packed(p, p, p, SPEC_F32, -1, 16, 64, nullptr, 0, nullptr), INV);

    // spec_verify_attention
    EXPECT(spec_verify_attention(p, p, p, ip, ip, 2, 3, 32, 8, 100, 64, 0.1f, p, SPEC_F32, op, p, 4096, nullptr), INV);
    EXPECT(spec_verify_attention(p, p, p, ip, ip, 2, 3, 32, 5, 100, 128, 0.1f, p, SPEC_F32, op, p, 4096, nullptr), INV);
    EXPECT(spec_verify_attention(p, p, p, ip, ip, 2, 8, 32, 8, 100, 128, 0.1f, p, SPEC_F32, op, p, 4096, nullptr), INV);

    // spec_adapt
    uint64_t tel[SPEC_ADAPT_TELEMETRY_WORDS];
    EXPECT(spec_adapt(ip, ip, 4, 40, p, tel, op, 1, 4, 8, SPEC_ADAPT_THRESHOLD, 0.35, 0.0, nullptr), INV);
    EXPECT(spec_adapt(ip, ip, 4, 4, p, tel, op, 3, 2, 8, SPEC_ADAPT_THRESHOLD, 0.35, 0.0, nullptr), INV);
    EXPECT(spec_adapt(ip, ip, 4, 4, p, tel, op, 1, 4, 17, SPEC_ADAPT_THRESHOLD, 0.35, 0.0, nullptr), INV);
    EXPECT(spec_adapt(ip, ip, 4, 4, p, tel, op, 1, 4, 8, 5, 0.35, 0.0, nullptr), INV);

    EXPECT(spec_debug_set_wait_bound(-2), INV);
    EXPECT(spec_debug_set_wait_bound(0), SPEC_OK);
    if (!g_fail) printf("sanitized host validation: all checks passed\n");
    return g_fail;
}
