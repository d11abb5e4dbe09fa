// abi_driver.cpp -- drives the host-side validation of libkdnscan (argument
// checks, plans, workspace and echo-size queries, status strings) through the
// C ABI with no GPU work: every call here returns before any kernel launch or
// HIP memory call.  Built by the sanitizer test with the host code of the
// ABI translation unit under AddressSanitizer and UndefinedBehaviorSanitizer;
// output arrays are exactly sized heap blocks, so a write past what the
// header promises aborts the run.  Exit status 0 means every call returned
// the status the header documents.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/kdnscan.h"

namespace {

int g_fail = 0;
void expect(const char* what, int got, int want) {
    if (got != want) {
        std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        g_fail = 1;
    }
}

// stand-in device addresses: never dereferenced by a query or a rejected call
const void* const FAKE = reinterpret_cast<const void*>(uintptr_t{0x10000});
const void* const MIS = reinterpret_cast<const void*>(uintptr_t{0x10002});   // misaligned
float* F(const void* p) { return const_cast<float*>(static_cast<const float*>(p)); }

int diag_query(int64_t B, int64_t H, int64_t T, int64_t dk, int64_t dv, kdn_scan_opts* opts,
               size_t* need, float I_prior = 1.0f, const void* q = FAKE, const void* o = FAKE) {
    return kdn_diag_scan_fwd_ex(B, H, T, dk, dv, KDN_BF16, q, FAKE, FAKE, FAKE, FAKE, F(FAKE), I_prior,
                                nullptr, nullptr, F(o), nullptr, nullptr, opts, nullptr, need, nullptr);
}

void plans() {
    const int64_t Ts[] = {0, 1, 15, 16, 17, 601, 2048, 16384, 65537};
    const int64_t dims[] = {16, 32, 64, 128};
    for (int64_t T : Ts)
        for (int64_t dv : dims)
            for (int32_t S : {0, 1, 2, 3, 5, 64, 1000}) {
                int32_t chunk = 0, segs = 0, R = 0;
                expect("plan", kdn_diag_plan(2, 16, T, 128, dv, S, &chunk, &segs, &R, nullptr, 0), KDN_OK);
                // bounds into an exactly sized array, then one entry short
                std::vector<int64_t> b(static_cast<size_t>(segs) + 1);
                expect("plan bounds", kdn_diag_plan(2, 16, T, 128, dv, S, nullptr, nullptr, nullptr, b.data(), segs), KDN_OK);
                if (b.front() != 0 || b.back() != T) { std::fprintf(stderr, "plan bounds ends\n"); g_fail = 1; }
                for (size_t i = 1; i < b.size(); ++i)
                    if (b[i] < b[i - 1]) { std::fprintf(stderr, "plan bounds order\n"); g_fail = 1; }
                if (segs > 1) {
                    std::vector<int64_t> small(static_cast<size_t>(segs) - 1);
                    expect("plan short", kdn_diag_plan(2, 16, T, 128, dv, S, nullptr, nullptr, nullptr,
                                                       small.data(), segs - 2), KDN_EINVAL);
                }
            }
    expect("plan B<0", kdn_diag_plan(-1, 1, 1, 64, 64, 0, nullptr, nullptr, nullptr, nullptr, 0), KDN_EINVAL);
    expect("plan S<0", kdn_diag_plan(1, 1, 1, 64, 64, -2, nullptr, nullptr, nullptr, nullptr, 0), KDN_EINVAL);
    expect("plan dk", kdn_diag_plan(1, 1, 1, 48, 64, 0, nullptr, nullptr, nullptr, nullptr, 0), KDN_EUNSUPPORTED);
    expect("plan huge", kdn_diag_plan(1, 1, int64_t{1} << 40, 64, 64, 0, nullptr, nullptr, nullptr, nullptr, 0), KDN_EINVAL);
}

void diag_queries() {
    for (int64_t T : {int64_t{0}, int64_t{1}, int64_t{100}, int64_t{16384}})
        for (int32_t S : {0, 1, 4}) {
            kdn_scan_opts o{};
            o.segments = S;
            o.echo_capacity = 0;
            size_t need = 0;
            expect("fwd query", diag_query(2, 16, T, 128, 128, &o, &need), KDN_OK);
            if (T > 0 && need < 16u * 2 * 16 * static_cast<size_t>(T)) { std::fprintf(stderr, "fwd need\n"); g_fail = 1; }
            if (o.echo_words < 0 || o.echo_words % KDN_ECHO_WORDS) { std::fprintf(stderr, "echo words\n"); g_fail = 1; }
        }
    size_t need = 0;
    expect("fwd null opts", diag_query(1, 2, 50, 64, 64, nullptr, &need), KDN_OK);
    expect("fwd B<0", diag_query(-1, 2, 50, 64, 64, nullptr, &need), KDN_EINVAL);
    expect("fwd dk", diag_query(1, 2, 50, 24, 64, nullptr, &need), KDN_EUNSUPPORTED);
    expect("fwd dv", diag_query(1, 2, 50, 64, 256, nullptr, &need), KDN_EUNSUPPORTED);
    expect("fwd prior 0", diag_query(1, 2, 50, 64, 64, nullptr, &need, 0.0f), KDN_EINVAL);
    expect("fwd prior nan", diag_query(1, 2, 50, 64, 64, nullptr, &need, std::nanf("")), KDN_EINVAL);
    expect("fwd prior inf", diag_query(1, 2, 50, 64, 64, nullptr, &need, INFINITY), KDN_EINVAL);
    expect("fwd q null", diag_query(1, 2, 50, 64, 64, nullptr, &need, 1.0f, nullptr), KDN_EINVAL);
    expect("fwd q misaligned", diag_query(1, 2, 50, 64, 64, nullptr, &need, 1.0f, MIS), KDN_EINVAL);
    expect("fwd o null", diag_query(1, 2, 50, 64, 64, nullptr, &need, 1.0f, FAKE, nullptr), KDN_EINVAL);
    expect("fwd T 2^31", diag_query(1, 1, int64_t{1} << 31, 64, 64, nullptr, &need), KDN_EINVAL);
    expect("fwd B huge", diag_query(int64_t{1} << 23, 16, 1 << 20, 128, 128, nullptr, &need), KDN_EINVAL);
    kdn_scan_opts bad{};
    bad.segments = -1;
    expect("opts segments", diag_query(1, 2, 50, 64, 64, &bad, &need), KDN_EINVAL);
    bad = kdn_scan_opts{};
    bad.bounds_echo = reinterpret_cast<int64_t*>(uintptr_t{0x10004});
    bad.echo_capacity = 8;
    expect("opts echo align", diag_query(1, 2, 50, 64, 64, &bad, &need), KDN_EINVAL);
    bad = kdn_scan_opts{};
    bad.echo_capacity = -3;
    expect("opts echo cap", diag_query(1, 2, 50, 64, 64, &bad, &need), KDN_EINVAL);
    // a workspace that is too small, and none at all
    size_t small = 8;
    expect("fwd small ws", kdn_diag_scan_fwd(2, 16, 16384, 128, 128, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                             F(FAKE), 1.0f, nullptr, nullptr, F(FAKE), nullptr, nullptr,
                                             const_cast<void*>(FAKE), &small, nullptr), KDN_EWORKSPACE);
    expect("fwd no ws", kdn_diag_scan_fwd(2, 16, 16384, 128, 128, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          F(FAKE), 1.0f, nullptr, nullptr, F(FAKE), nullptr, nullptr,
                                          nullptr, nullptr, nullptr), KDN_EWORKSPACE);
    // the no-allocation entry rejects bad arguments before touching the device
    expect("noalloc B<0", kdn_diag_scan_fwd_noalloc(-1, 2, 50, 64, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                    F(FAKE), 1.0f, nullptr, nullptr, F(FAKE), nullptr, nullptr,
                                                    nullptr), KDN_EINVAL);
    expect("noalloc dk", kdn_diag_scan_fwd_noalloc(1, 2, 50, 40, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                   F(FAKE), 1.0f, nullptr, nullptr, F(FAKE), nullptr, nullptr,
                                                   nullptr), KDN_EUNSUPPORTED);
}

void other_queries() {
    size_t need = 0;
    kdn_scan_opts o{};
    o.segments = 2;
    expect("varlen segments", kdn_diag_scan_varlen_fwd_ex(2, 2, 50, 64, 64, KDN_BF16,
                                                          static_cast<const int64_t*>(FAKE), FAKE, FAKE, FAKE,
                                                          FAKE, FAKE, F(FAKE), 1.0f, nullptr, nullptr, F(FAKE),
                                                          nullptr, nullptr, &o, nullptr, &need, nullptr), KDN_EINVAL);
    expect("varlen query", kdn_diag_scan_varlen_fwd(7, 16, 4000, 128, 128, KDN_BF16,
                                                    static_cast<const int64_t*>(FAKE), FAKE, FAKE, FAKE, FAKE,
                                                    FAKE, F(FAKE), 1.0f, nullptr, nullptr, F(FAKE), nullptr,
                                                    nullptr, nullptr, &need, nullptr), KDN_OK);
    for (int32_t S : {0, 1, 3}) {
        kdn_scan_opts m{};
        m.segments = S;
        expect("mobius query", kdn_mobius_precision_scan_ex(1, 4, 5000, F(FAKE), F(FAKE), F(FAKE), nullptr, F(FAKE),
                                                            64, 64, F(FAKE), F(FAKE), F(FAKE), nullptr, F(FAKE),
                                                            nullptr, &m, nullptr, &need, nullptr), KDN_OK);
    }
    expect("mobius dk", kdn_mobius_precision_scan(1, 4, 50, F(FAKE), F(FAKE), F(FAKE), nullptr, F(FAKE), 48, 64,
                                                  F(FAKE), F(FAKE), F(FAKE), nullptr, F(FAKE), nullptr, nullptr,
                                                  &need, nullptr), KDN_EUNSUPPORTED);
    expect("mobius a null", kdn_mobius_precision_scan(1, 4, 50, nullptr, F(FAKE), F(FAKE), nullptr, F(FAKE), 0, 0,
                                                      nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                      &need, nullptr), KDN_EINVAL);
    float* const fk = F(FAKE);
    expect("bwd query", kdn_diag_scan_bwd(8, 16, 2048, 128, 128, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, 1.0f,
                                          nullptr, nullptr, fk, nullptr, nullptr, fk, fk, fk, fk, fk, fk, nullptr,
                                          nullptr, nullptr, nullptr, &need, nullptr), KDN_OK);
    expect("bwd dk", kdn_diag_scan_bwd(1, 2, 64, 32, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, 1.0f,
                                       nullptr, nullptr, fk, nullptr, nullptr, fk, fk, fk, fk, fk, fk, nullptr,
                                       nullptr, nullptr, nullptr, &need, nullptr), KDN_EUNSUPPORTED);
    expect("bwd d_o null", kdn_diag_scan_bwd(1, 2, 64, 64, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, 1.0f,
                                             nullptr, nullptr, nullptr, nullptr, nullptr, fk, fk, fk, fk, fk, fk,
                                             nullptr, nullptr, nullptr, nullptr, &need, nullptr), KDN_EINVAL);
    // the gradient with a segment request (long rows) and over packed batches,
    // split and whole, and the packed plan query
    for (int32_t S : {0, 1, 4, 64}) {
        kdn_scan_opts m{};
        m.segments = S;
        expect("bwd_ex query", kdn_diag_scan_bwd_ex(2, 16, 16384, 128, 128, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                    fk, 1.0f, nullptr, nullptr, fk, nullptr, nullptr, fk, fk, fk, fk,
                                                    fk, fk, nullptr, nullptr, nullptr, &m, nullptr, &need, nullptr),
               KDN_OK);
    }
    {
        kdn_scan_opts m{};
        int64_t echo[8];
        m.bounds_echo = echo;
        m.echo_capacity = 8;
        expect("bwd_ex echo", kdn_diag_scan_bwd_ex(1, 2, 64, 64, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, 1.0f,
                                                   nullptr, nullptr, fk, nullptr, nullptr, fk, fk, fk, fk, fk, fk,
                                                   nullptr, nullptr, nullptr, &m, nullptr, &need, nullptr),
               KDN_EINVAL);
    }
    for (int64_t T : {int64_t(40), int64_t(16384)}) {
        expect("varlen bwd query", kdn_diag_scan_varlen_bwd(64, 16, T, 128, 128, KDN_BF16,
                                                            static_cast<const int64_t*>(FAKE), FAKE, FAKE, FAKE,
                                                            FAKE, FAKE, fk, 1.0f, nullptr, nullptr, fk, nullptr,
                                                            nullptr, fk, fk, fk, fk, fk, fk, fk, nullptr, nullptr,
                                                            nullptr, &need, nullptr), KDN_OK);
    }
    {
        int64_t seg = -1, items = -1, comps = -1;
        int32_t R = -1;
        expect("varlen plan", kdn_diag_varlen_plan(64, 16, 16384, 128, 128, 0, &seg, &R, &items, &comps), KDN_OK);
        if (seg != 2048 || items != 72 || comps != 8 || R < 1) {
            std::fprintf(stderr, "varlen plan values\n");
            g_fail = 1;
        }
        expect("varlen plan request", kdn_diag_varlen_plan(64, 16, 16384, 128, 128, 2, nullptr, nullptr, nullptr,
                                                           nullptr), KDN_EINVAL);
    }
    expect("decode dk", kdn_decode_step(1, 2, 8, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, 1.0f, fk, fk, fk,
                                        nullptr), KDN_EUNSUPPORTED);
    expect("decode prior", kdn_decode_step(1, 2, 64, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, fk, -1.0f, fk, fk,
                                           fk, nullptr), KDN_EINVAL);
    expect("noise B<0", kdn_diag_noise_scan_fwd(-1, 2, 64, 64, 64, KDN_BF16, FAKE, FAKE, FAKE, FAKE, fk, fk,
                                                nullptr, nullptr, fk, nullptr, nullptr, nullptr), KDN_EINVAL);
    for (int s = -12; s <= 12; ++s)
        if (kdn_status_string(s) == nullptr) { std::fprintf(stderr, "status string\n"); g_fail = 1; }
}

}  // namespace

int main() {
    plans();
    diag_queries();
    other_queries();
    if (g_fail) return 1;
    std::printf("host validation sanitizer run: ok\n");
    return 0;
}
