// Internal declarations shared by the packer (host C++) and the HIP launchers.
#pragma once

#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/mbd.h"

namespace mbd {

// Per-thread message of the last failing call; set() returns the status so that
// `return fail(MBD_ESHAPE, "...")` reads naturally.
mbd_status fail(mbd_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

constexpr int64_t kTile = 4096;       // Cassandra flat tile (elements)
constexpr int kMantHiBits = 3;        // Cassandra kept mantissa high bits
constexpr uint64_t kPadAlign = 256;   // section padding granularity

inline uint64_t padded_size(uint64_t bytes) {
    return ((bytes + kPadAlign - 1) / kPadAlign) * kPadAlign + kPadAlign;
}

struct Section {
    const char* name;
    std::vector<uint8_t> buf;   // padded_size(bytes) bytes, zero padded
    uint64_t bytes = 0;
    void resize(uint64_t b) { bytes = b; buf.assign(padded_size(b), 0); }
    template <class T> T* as() { return reinterpret_cast<T*>(buf.data()); }
    template <class T> const T* as() const { return reinterpret_cast<const T*>(buf.data()); }
};

}  // namespace mbd

struct mbd_packed {
    int32_t fmt = 0;
    int64_t M = 0, K = 0;
    int32_t n_sym = 0;
    int64_t n_kept = 0;
    int64_t unary_bits = 0;
    int64_t n_tiles = 0;
    int32_t keep_num = 3, keep_den = 10;
    double zero_fraction = 0.0;
    std::vector<mbd::Section> sec;
};
