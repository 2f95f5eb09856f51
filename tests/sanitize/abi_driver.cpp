// Host-only driver of the library's C ABI for an AddressSanitizer + Undefined-
// BehaviorSanitizer build: the HIP sources compiled for the host only, their host
// passes instrumented, linked with packer.cpp.  Every call here fails validation
// before any device work (the pointers are fake and never dereferenced), so it
// runs without a GPU and exercises the argument checks, the error reporting and
// the size arithmetic of every entry point.  Exit status 0 and no sanitizer
// report is the pass condition.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mbd.h"

namespace {

int failures = 0;

void expect(mbd_status got, mbd_status want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "FAILED: %s: status %d, expected %d (%s)\n", what, int(got), int(want), mbd_last_error());
        ++failures;
    }
}

void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

mbd_dweights desc(int32_t fmt, int64_t M, int64_t K, int32_t n_sym = 0, uintptr_t ptr = 0x1000, int64_t n_mats = 1) {
    mbd_dweights d;
    std::memset(&d, 0, sizeof d);
    d.fmt = fmt;
    d.M = M;
    d.K = K;
    d.n_sym = n_sym;
    d.n_mats = n_mats;
    for (int i = 0; i < MBD_MAX_SECTIONS; ++i) d.sec[i] = fake(ptr);
    return d;
}

const uint16_t* X16 = static_cast<const uint16_t*>(fake(0x10000));
float* Y16 = static_cast<float*>(fake(0x10000));
const int32_t* R16 = static_cast<const int32_t*>(fake(0x10000));

void status_strings() {
    for (int s = 0; s < 8; ++s)
        if (!mbd_status_str(s) || !*mbd_status_str(s)) ++failures;
    if (std::strcmp(mbd_status_str(99), "unknown status") != 0) ++failures;
}

void gemv_errors() {
    mbd_dweights d = desc(MBD_INT4_G128, 16, 256);
    expect(mbd_gemv(nullptr, X16, 1, Y16, nullptr), MBD_EINVAL, "gemv NULL weights");
    expect(mbd_gemv(&d, nullptr, 1, Y16, nullptr), MBD_EINVAL, "gemv NULL x");
    expect(mbd_gemv(&d, X16, 0, Y16, nullptr), MBD_ESHAPE, "gemv B = 0");
    expect(mbd_gemv(&d, X16, 17, Y16, nullptr), MBD_ESHAPE, "gemv B = 17");
    d.K = 200;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_ESHAPE, "gemv K % 128");
    d = desc(MBD_INT4_G128, 16, 256);
    d.fmt = 42;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EINVAL, "gemv unknown format");
    d = desc(MBD_INT4_G128, 16, 256, 0, 0x10004);
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EALIGN, "gemv misaligned codes");
    d = desc(MBD_MX32, 16, 48);
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_ESHAPE, "gemv MX32 K = 48");
    const int32_t fmts[2] = {MBD_INT4_G128, MBD_TERNARY_B128};
    const int64_t rows[2] = {int64_t(1) << 20, int64_t(1) << 21};
    for (int f = 0; f < 2; ++f)
        for (int B : {1, 8}) {
            d = desc(fmts[f], rows[f], 8192);
            expect(mbd_gemv(&d, X16, B, Y16, nullptr), MBD_ESHAPE, "gemv codes of 4 GiB");
        }
    // batch 5..16 addresses the activations with 32-bit element offsets
    for (int f = 0; f < 2; ++f) {
        d = desc(fmts[f], 16, int64_t(1) << 28);
        expect(mbd_gemv(&d, X16, 16, Y16, nullptr), MBD_ESHAPE, "gemv activations of 2^32 elements");
    }
    d = desc(MBD_INT4_G128, 16, 256);
    expect(mbd_dequant(&d, nullptr, nullptr), MBD_EINVAL, "dequant NULL output");
    expect(mbd_dequant(&d, static_cast<float*>(fake(0x10004)), nullptr), MBD_EALIGN, "dequant misaligned output");
}

void skip_errors() {
    mbd_dweights d = desc(MBD_TERNARY_SKIP, 16, 256, 0, 0x10000);
    d.n_mats = 2;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EINVAL, "skip: one matrix only");
    d.n_mats = 1;
    d.sec[3] = nullptr;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EINVAL, "skip: tile_base missing");
    expect(mbd_dequant(&d, Y16, nullptr), MBD_EINVAL, "skip dequant: tile_base missing");
    d.sec[3] = fake(0x10000);
    d.sec[2] = fake(0x10002);
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EALIGN, "skip: slabs misaligned");
    d.sec[2] = fake(0x10000);
    d.K = 128 * 4097;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_ESHAPE, "skip: 16-bit in-tile offset");
    d.K = 200;
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_ESHAPE, "skip: K % 128");
}

void cassandra_errors() {
    mbd_dweights d = desc(MBD_CASSANDRA_MX, 16, 256, 0, 0x10000);
    expect(mbd_gemv(&d, X16, 1, Y16, nullptr), MBD_EINVAL, "Cassandra-2 data in mbd_gemv");
    expect(mbd_spec_gemv(&d, X16, 17, Y16, nullptr), MBD_ESHAPE, "Cassandra-2 spec GEMV B = 17");
    d.sec[4] = nullptr;
    expect(mbd_spec_gemv(&d, X16, 1, Y16, nullptr), MBD_EINVAL, "Cassandra-2 kprefix missing");
    uint16_t* out = static_cast<uint16_t*>(fake(0x10000));
    expect(mbd_spec_decode(&d, out, nullptr), MBD_EINVAL, "Cassandra-2 decode kprefix missing");
    d.sec[4] = fake(0x10008);
    expect(mbd_spec_gemv(&d, X16, 1, Y16, nullptr), MBD_EALIGN, "Cassandra-2 kprefix misaligned");
    d.sec[4] = fake(0x10000);
    d.K = 200;
    expect(mbd_spec_decode(&d, out, nullptr), MBD_ESHAPE, "Cassandra-2 decode K % 128");

    d = desc(MBD_CASSANDRA, 16, 256);
    d.n_kept = 5;
    expect(mbd_spec_decode(&d, out, nullptr), MBD_EINVAL, "kept values without a codebook");
    d.n_sym = 300;
    expect(mbd_spec_decode(&d, out, nullptr), MBD_EINVAL, "codebook of 300 symbols");
    d.n_sym = 12;
    d.sec[2] = nullptr;
    expect(mbd_spec_decode(&d, out, nullptr), MBD_EINVAL, "unary stream missing");
    d.sec[2] = fake(0x10000);
    expect(mbd_spec_gemv(&d, X16, 20, Y16, nullptr), MBD_ESHAPE, "spec GEMV B = 20");
    d.sec[7] = nullptr;
    expect(mbd_verify_restore(&d, out, nullptr), MBD_EINVAL, "verification data missing");
    d = desc(MBD_CASSANDRA, 16, 1536, 12);
    expect(mbd_gemv(&d, X16, 16, Y16, nullptr), MBD_ESHAPE, "verify GEMM K % 4096");
}

void encoder_errors() {
    uint64_t n = 0;
    expect(mbd_encode_workspace_bytes(0, &n), MBD_ESHAPE, "encode workspace M = 0");
    expect(mbd_encode_workspace_bytes(8, &n), MBD_OK, "encode workspace M = 8");
    if (n < 64) ++failures;
    mbd_encode_plan_t plan;
    std::memset(&plan, 0, sizeof plan);
    const float* nrm = static_cast<const float*>(fake(0x10000));
    void* ws = fake(0x10000);
    expect(mbd_encode_plan(nullptr, nrm, 8, 256, 3, 10, ws, n, &plan, nullptr), MBD_EINVAL, "plan NULL w");
    expect(mbd_encode_plan(X16, nrm, 8, 200, 3, 10, ws, n, &plan, nullptr), MBD_ESHAPE, "plan K % 128");
    expect(mbd_encode_plan(X16, nrm, 8, 256, 3, 10, ws, 16, &plan, nullptr), MBD_EINVAL, "plan workspace too small");
    expect(mbd_encode_plan(X16, nrm, 8, 256, 3, 10, fake(0x10008), n, &plan, nullptr), MBD_EALIGN, "plan misaligned workspace");
    expect(mbd_encode_plan(X16, nrm, 8, 256, 3, 10, ws, n, nullptr, nullptr), MBD_EINVAL, "plan NULL plan");
    void* secs[8];
    for (auto& s : secs) s = fake(0x10000);
    plan.n_kept = 8 * 76 + 1;
    plan.n_tiles = 1;
    expect(mbd_encode_cassandra(X16, nrm, 8, 256, 3, 10, &plan, secs, ws, n, nullptr), MBD_EINVAL, "plan of another shape");
    plan.n_kept = 8 * 76;
    secs[2] = nullptr;
    expect(mbd_encode_cassandra(X16, nrm, 8, 256, 3, 10, &plan, secs, ws, n, nullptr), MBD_EINVAL, "unary buffer missing");
    secs[2] = fake(0x10008);
    expect(mbd_encode_cassandra(X16, nrm, 8, 256, 3, 10, &plan, secs, ws, n, nullptr), MBD_EALIGN, "unary buffer misaligned");
}

void moe_errors() {
    mbd_dweights e = desc(MBD_TERNARY_B128, 64, 256, 0, 0x1000, 8);
    uint64_t need = 0;
    expect(mbd_moe_workspace_bytes(8, 2, 4, &need), MBD_OK, "moe workspace");
    if (need == 0) ++failures;
    expect(mbd_moe_workspace_bytes(0, 2, 4, &need), MBD_ESHAPE, "moe workspace, no experts");
    expect(mbd_moe_workspace_bytes(8, 2, 4, &need), MBD_OK, "moe workspace again");
    void* ws = fake(0x10000);
    expect(mbd_moe_gemv(&e, R16, 2, 4, X16, 0, Y16, ws, 1, nullptr), MBD_EINVAL, "moe workspace too small");
    e.fmt = MBD_CASSANDRA;
    expect(mbd_moe_gemv(&e, R16, 2, 4, X16, 0, Y16, ws, need, nullptr), MBD_EINVAL, "moe Cassandra experts");
    e = desc(MBD_TERNARY_SKIP, 64, 256);
    expect(mbd_moe_gemv(&e, R16, 1, 1, X16, 0, Y16, ws, 1 << 20, nullptr), MBD_EINVAL, "moe skip-format experts");
    e = desc(MBD_TERNARY_B128, 64, 256, 0, 0x1000, 64);
    expect(mbd_moe_gemv_noalloc(nullptr, R16, 2, 4, X16, 0, Y16, nullptr), MBD_EINVAL, "noalloc NULL experts");
    expect(mbd_moe_gemv_noalloc(&e, nullptr, 2, 4, X16, 0, Y16, nullptr), MBD_EINVAL, "noalloc NULL route");
    expect(mbd_moe_gemv_noalloc(&e, R16, 8192, 8, X16, 0, Y16, nullptr), MBD_ESHAPE, "noalloc route beyond the scratch");
    expect(mbd_moe_gemv_noalloc(&e, R16, 2, 0, X16, 0, Y16, nullptr), MBD_ESHAPE, "noalloc k = 0");
    mbd_dweights big = desc(MBD_INT4_G128, int64_t(1) << 20, 8192, 0, 0x1000, 2);
    expect(mbd_moe_gemv_noalloc(&big, R16, 1, 2, X16, 0, Y16, nullptr), MBD_ESHAPE, "noalloc codes of 4 GiB");
    expect(mbd_moe_gemv(&big, R16, 1, 2, X16, 0, Y16, ws, 1 << 20, nullptr), MBD_ESHAPE, "moe codes of 4 GiB");
    mbd_dweights wide = desc(MBD_TERNARY_B128, 1, int64_t(1) << 30, 0, 0x1000, 2);
    expect(mbd_moe_gemv(&wide, R16, 2, 2, X16, 1, Y16, ws, 1 << 20, nullptr), MBD_ESHAPE, "moe activations of 2^32 elements");
    expect(mbd_moe_gemv_noalloc(&wide, R16, 2, 2, X16, 1, Y16, nullptr), MBD_ESHAPE, "noalloc activations of 2^32 elements");
}

void probe_errors() {
    uint32_t* sink = static_cast<uint32_t*>(fake(0x10000));
    expect(mbd_probe_stream_read(nullptr, 1024, sink, 4, 256, nullptr), MBD_EINVAL, "probe NULL src");
    expect(mbd_probe_stream_read(fake(0x10008), 1024, sink, 4, 256, nullptr), MBD_EALIGN, "probe misaligned src");
    expect(mbd_probe_stream_read(fake(0x10000), 1000, sink, 4, 256, nullptr), MBD_EALIGN, "probe bytes % 16");
    expect(mbd_probe_stream_read(fake(0x10000), 1024, sink, 4, 100, nullptr), MBD_ESHAPE, "probe threads % 64");
    expect(mbd_probe_stream_read(fake(0x10000), 1024, sink, 0, 256, nullptr), MBD_ESHAPE, "probe no blocks");
}

void pack_errors() {
    std::vector<uint16_t> w(4 * 128, 0);
    mbd_packed* h = nullptr;
    expect(mbd_pack(MBD_INT4_G128, nullptr, 4, 128, nullptr, nullptr, &h), MBD_EINVAL, "pack NULL w");
    expect(mbd_pack(99, w.data(), 4, 128, nullptr, nullptr, &h), MBD_EINVAL, "pack unknown format");
    expect(mbd_pack(MBD_INT4_G128, w.data(), 4, 100, nullptr, nullptr, &h), MBD_ESHAPE, "pack K % 128");
    expect(mbd_pack(MBD_CASSANDRA, w.data(), 4, 128, nullptr, nullptr, &h), MBD_EINVAL, "pack Cassandra without norms");
    expect(mbd_pack(MBD_INT4_G128, w.data(), 4, 128, nullptr, nullptr, &h), MBD_OK, "pack INT4");
    if (h) mbd_packed_free(h);
}

}  // namespace

int main() {
    status_strings();
    pack_errors();
    gemv_errors();
    skip_errors();
    cassandra_errors();
    encoder_errors();
    moe_errors();
    probe_errors();
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
