// Host-only driver of the C++ packer for an AddressSanitizer + UndefinedBehavior-
// Sanitizer build (g++ -fsanitize=address,undefined, with packer.cpp): packs every
// format on ragged shapes, special values and keep fractions, reads the sections
// and statistics back, validates, corrupts a copy of a section to exercise the
// validator's failure paths, and checks every argument error.  Exit status 0 and
// no sanitizer report is the pass condition; the numbers themselves are checked
// against the oracle by the Python tests.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "mbd.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (%s)\n", what, mbd_last_error());
        ++failures;
    }
}

uint16_t bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

std::vector<uint16_t> weights(int64_t M, int64_t K, uint32_t seed, bool specials) {
    std::mt19937 rng(seed);
    std::student_t_distribution<float> t4(4.f);
    std::vector<uint16_t> w(size_t(M * K));
    for (auto& v : w) v = bf16(t4(rng) * 0.02f);
    if (specials && M * K >= 256) {
        for (int k = 0; k < 128; ++k) w[size_t(k)] = 0;              // an all-zero block
        w[200] = 0x0001; w[201] = 0x8001; w[202] = 0x8000;            // subnormals, -0
    }
    return w;
}

void roundtrip(int32_t fmt, const std::vector<uint16_t>& w, int64_t M, int64_t K, const float* norm,
               const mbd_pack_params* pp) {
    mbd_packed* h = nullptr;
    const mbd_status s = mbd_pack(fmt, w.data(), M, K, norm, pp, &h);
    expect(s == MBD_OK && h, "pack");
    if (s != MBD_OK) return;
    int32_t n = 0;
    expect(mbd_packed_sections(h, nullptr, 0, &n) == MBD_OK && n > 0, "section count");
    std::vector<mbd_section> secs(static_cast<size_t>(n));
    expect(mbd_packed_sections(h, secs.data(), n, &n) == MBD_OK, "sections");
    uint64_t sum = 0;
    for (const auto& sec : secs) {                                    // touch every padded byte
        const uint8_t* p = static_cast<const uint8_t*>(sec.data);
        for (uint64_t i = 0; i < sec.padded_bytes; ++i) sum += p[i];
        expect(sec.padded_bytes >= sec.bytes + 256 && sec.padded_bytes % 256 == 0, "padding");
    }
    mbd_stats st;
    expect(mbd_packed_stats(h, &st) == MBD_OK && st.M == M && st.K == K && std::isfinite(st.bpw), "stats");
    expect(mbd_validate(h) == MBD_OK, "validate");
    // flip the first meaningful word of section 0: the validator may accept or
    // reject it, but must stay inside the buffers
    if (secs[0].bytes >= 4) {
        uint32_t* p0 = static_cast<uint32_t*>(const_cast<void*>(secs[0].data));
        const uint32_t old = p0[0];
        p0[0] = ~old;
        (void)mbd_validate(h);
        p0[0] = old;
        expect(mbd_validate(h) == MBD_OK, "validate after restore");
    }
    if (sum == 0xFFFFFFFFFFFFFFFFull) std::puts("");                  // keep the reads
    mbd_packed_free(h);
}

}  // namespace

int main() {
    const int64_t shapes[][2] = {{1, 128}, {3, 384}, {17, 256}, {33, 1152}, {5, 4096 + 128}, {2, 8192}};
    for (const auto& sh : shapes) {
        const int64_t M = sh[0], K = sh[1];
        const auto w = weights(M, K, uint32_t(M * 131 + K), true);
        std::vector<float> norm(static_cast<size_t>(K));
        std::mt19937 rng{uint32_t(K)};
        std::lognormal_distribution<float> ln(0.f, 1.f);
        for (auto& v : norm) v = ln(rng);
        for (int32_t fmt : {MBD_TERNARY_B128, MBD_INT4_G128, MBD_TERNARY_SKIP, MBD_MX32}) roundtrip(fmt, w, M, K, nullptr, nullptr);
        const int32_t keeps[][2] = {{3, 10}, {1, 1}, {0, 1}, {1, 2}};
        for (const auto& kp : keeps) {
            mbd_pack_params pp{kp[0], kp[1], 1};
            roundtrip(MBD_CASSANDRA, w, M, K, norm.data(), &pp);
            roundtrip(MBD_CASSANDRA_MX, w, M, K, norm.data(), &pp);
        }
    }
    {   // stacked experts
        const auto w = weights(4 * 40, 256, 7, false);
        mbd_pack_params pp{3, 10, 4};
        roundtrip(MBD_TERNARY_B128, w, 160, 256, nullptr, &pp);
        roundtrip(MBD_INT4_G128, w, 160, 256, nullptr, &pp);
    }
    {   // argument and range errors
        const auto w = weights(4, 256, 9, false);
        std::vector<float> norm(256, 1.f);
        mbd_packed* h = nullptr;
        expect(mbd_pack(MBD_INT4_G128, nullptr, 4, 256, nullptr, nullptr, &h) == MBD_EINVAL, "null w");
        expect(mbd_pack(99, w.data(), 4, 256, nullptr, nullptr, &h) == MBD_EINVAL, "bad fmt");
        expect(mbd_pack(MBD_INT4_G128, w.data(), 4, 200, nullptr, nullptr, &h) == MBD_ESHAPE, "bad K");
        expect(mbd_pack(MBD_CASSANDRA, w.data(), 4, 256, nullptr, nullptr, &h) == MBD_EINVAL, "no norms");
        auto bad = w;
        bad[7] = 0x7F80;                                              // +Inf
        expect(mbd_pack(MBD_INT4_G128, bad.data(), 4, 256, nullptr, nullptr, &h) == MBD_ERANGE, "inf");
        norm[3] = -1.f;
        expect(mbd_pack(MBD_CASSANDRA, w.data(), 4, 256, norm.data(), nullptr, &h) == MBD_ERANGE, "negative norm");
        expect(mbd_packed_sections(nullptr, nullptr, 0, nullptr) == MBD_EINVAL, "sections null");
        expect(mbd_validate(nullptr) == MBD_EINVAL, "validate null");
        mbd_packed_free(nullptr);
        for (int s = 0; s < 9; ++s) expect(mbd_status_str(s) != nullptr, "status string");
    }
    if (failures) std::fprintf(stderr, "%d failures\n", failures);
    else std::puts("packer driver: all checks passed");
    return failures ? 1 : 0;
}
