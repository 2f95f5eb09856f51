// Offline CPU packer for the three compressed weight layouts, the MX-32 variant
// and ternary with all-zero blocks left out, plus the status / error plumbing of
// the C ABI.
//
// Ternary: [Bonsai2] 1.2 (absmean block 128), 3.4 / 5.5 (all-zero block -> scale 1,
//          flagged, its codes not stored).
// INT4:    [GPT54-INT4] 3.2 (group 128, scale max|w|/7, codes in [-7, 7]).
// Cassandra: [Cassandra] 3.2 (Wanda pruning + bitmap, mantissa truncation,
//          speculation + verification = original), 3.3 (unary exponent ranks, MX).
// The section layouts are documented in include/mbd.h.
#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdarg>
#include <cstring>
#include <new>
#include <numeric>
#include <thread>

#include "mbd_internal.h"

namespace mbd {

static thread_local std::string g_last_error;

mbd_status fail(mbd_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

namespace {

// bf16 bits -> exact double (bf16 is the high half of an IEEE binary32).
inline double bf16_to_double(uint16_t b) {
    uint32_t u = uint32_t(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return double(f);
}

inline bool bf16_nonfinite(uint16_t b) { return ((b >> 7) & 0xFF) == 0xFF; }

// IEEE binary16 round-to-nearest-even of an exact double.
inline uint16_t fp16_rne(double v) {
    uint16_t sign = std::signbit(v) ? 0x8000 : 0;
    double a = std::fabs(v);
    if (a == 0.0) return sign;
    int e;
    std::frexp(a, &e);
    e -= 1;                                   // 2^e <= a < 2^(e+1)
    if (e < -14) {                            // subnormal: quantum 2^-24
        double m = std::nearbyint(std::ldexp(a, 24));
        return uint16_t(sign | uint16_t(m));  // m == 1024 is the smallest normal
    }
    double m = std::nearbyint(std::ldexp(a, 10 - e));   // in [1024, 2048]
    if (m == 2048.0) { e += 1; m = 1024.0; }
    int biased = e + 15;
    if (biased >= 31) return uint16_t(sign | 0x7C00);
    return uint16_t(sign | (biased << 10) | (int(m) - 1024));
}

inline double fp16_to_double(uint16_t h) {
    int E = (h >> 10) & 0x1F, M = h & 0x3FF;
    double v = E ? std::ldexp(double(1024 + M), E - 25) : std::ldexp(double(M), -24);
    return (h & 0x8000) ? -v : v;
}

struct RoundNearest {   // the packer's arithmetic assumes round-to-nearest-even
    int saved;
    RoundNearest() : saved(std::fegetround()) { std::fesetround(FE_TONEAREST); }
    ~RoundNearest() { std::fesetround(saved); }
};

unsigned n_workers(int64_t rows) {
    unsigned hc = std::max(1u, std::thread::hardware_concurrency());
    return unsigned(std::max<int64_t>(1, std::min<int64_t>(std::min(hc, 16u), rows / 64)));
}

template <class F>
void parallel_rows(int64_t M, F&& f) {
    unsigned nw = n_workers(M);
    if (nw <= 1) { f(int64_t(0), M); return; }
    std::vector<std::thread> th;
    int64_t per = (M + nw - 1) / nw;
    for (unsigned i = 0; i < nw; ++i) {
        int64_t r0 = i * per, r1 = std::min<int64_t>(M, r0 + per);
        if (r0 >= r1) break;
        th.emplace_back([&f, r0, r1] { RoundNearest rn; f(r0, r1); });
    }
    for (auto& t : th) t.join();
}

// ------------------------------------------------------------------ ternary / INT4

// Word offset of word wd (0 .. 128/cpw - 1) of group g of row m in the
// tile-interleaved code order, for a stack of matrices of Mm rows each.
int64_t code_word_offset(bool ternary, int64_t m, int64_t g, int wd, int64_t Mm, int64_t K) {
    const int64_t mat = m / Mm, r = m - mat * Mm, t0 = r & ~int64_t(15);
    const int64_t R = std::min<int64_t>(16, Mm - t0), mi = r - t0;
    const int64_t wpr = K / (ternary ? 16 : 8);                 // words per row
    const int64_t base = (mat * Mm + t0) * wpr;
    if (!ternary) return base + g * 16 * R + ((wd >> 2) * R + mi) * 4 + (wd & 3);
    const int64_t P = (K / 128) / 2;                            // full block pairs
    const int kq = wd >> 1, j = wd & 1;
    if (g < 2 * P) return base + (g >> 1) * 16 * R + (kq * R + mi) * 4 + (g & 1) * 2 + j;
    return base + P * 16 * R + (kq * R + mi) * 2 + j;
}

mbd_status pack_block_quant(mbd_packed* h, const uint16_t* w, bool ternary, int64_t n_mats) {
    const int64_t M = h->M, K = h->K, G = K / 128, Mm = M / n_mats;
    const int cpw = ternary ? 16 : 8, bits = ternary ? 2 : 4;
    h->sec.resize(2);
    h->sec[0].name = "codes";
    h->sec[0].resize(uint64_t(M) * (K / cpw) * 4);
    h->sec[1].name = "scales";
    h->sec[1].resize(uint64_t(M) * G * 2);
    uint32_t* codes = h->sec[0].as<uint32_t>();
    uint16_t* scales = h->sec[1].as<uint16_t>();
    std::vector<int64_t> zeros(M, 0);
    std::vector<int> bad(M, 0);   // 1: non-finite input, 2: scale overflow

    parallel_rows(M, [&](int64_t r0, int64_t r1) {
        double v[128];
        for (int64_t m = r0; m < r1; ++m) {
            for (int64_t g = 0; g < G; ++g) {
                const uint16_t* src = w + m * K + g * 128;
                double acc = 0.0;
                for (int i = 0; i < 128; ++i) {
                    if (bf16_nonfinite(src[i])) { bad[m] = 1; return; }
                    v[i] = bf16_to_double(src[i]);
                    acc = ternary ? acc + std::fabs(v[i]) : std::max(acc, std::fabs(v[i]));
                }
                double stat = ternary ? acc / 128.0 : acc / 7.0;
                uint16_t s = fp16_rne(stat);
                if ((s & 0x7FFF) == 0x7C00) { bad[m] = 2; return; }
                bool zero = (acc == 0.0) || (s == 0);
                if (zero) s = 0x3C00;
                scales[m * G + g] = s;
                double sv = fp16_to_double(s);
                const int qmax = ternary ? 1 : 7, off = ternary ? 1 : 8;
                for (int wd = 0; wd < 128 / cpw; ++wd) {
                    uint32_t word = 0;
                    // element j of the word: evens in the low half, odds in the high half
                    for (int j = 0; j < cpw; ++j) {
                        int q = 0;
                        if (!zero) {
                            double r = std::nearbyint(v[wd * cpw + j] / sv);
                            q = int(std::max<double>(-qmax, std::min<double>(qmax, r)));
                        }
                        zeros[m] += (q == 0);
                        word |= uint32_t(q + off) << (bits * (j >> 1) + ((j & 1) ? 16 : 0));
                    }
                    codes[code_word_offset(ternary, m, g, wd, Mm, K)] = word;
                }
            }
        }
    });
    for (int64_t m = 0; m < M; ++m) {
        if (bad[m] == 1) return fail(MBD_ERANGE, "bf16 Inf/NaN in row %lld", (long long)m);
        if (bad[m] == 2) return fail(MBD_ERANGE, "fp16 scale overflow in row %lld", (long long)m);
    }
    int64_t z = std::accumulate(zeros.begin(), zeros.end(), int64_t(0));
    h->zero_fraction = double(z) / double(M * K);
    return MBD_OK;
}

// Ternary with all-zero blocks left out ([Bonsai2] 3.4, 5.5): the dense packing
// first, then every block whose 8 words are all code 1 (q = 0) is dropped and the
// rest re-laid per (16-row tile, block column): its stored blocks ranked by tile
// row, unit (rank, quarter) of 8 bytes at quarter * stored + rank.
mbd_status pack_ternary_skip(mbd_packed* h, const uint16_t* w) {
    const int64_t M = h->M, K = h->K, G = K / 128, tiles = (M + 15) / 16;
    if (16 * G > 65536) return fail(MBD_ESHAPE, "K=%lld too large for the 16-bit in-tile block offset", (long long)K);
    mbd_status s = pack_block_quant(h, w, true, 1);
    if (s != MBD_OK) return s;
    Section dense = std::move(h->sec[0]);
    const uint32_t* dc = dense.as<uint32_t>();
    h->sec.resize(4);
    h->sec[2].name = "slabs";
    h->sec[2].resize(uint64_t(tiles) * G * 4);
    h->sec[3].name = "tile_base";
    h->sec[3].resize(uint64_t(tiles + 1) * 4);
    uint32_t* slabs = h->sec[2].as<uint32_t>();
    uint32_t* base = h->sec[3].as<uint32_t>();
    auto word = [&](int64_t m, int64_t g, int wd) { return dc[code_word_offset(true, m, g, wd, M, K)]; };
    int64_t total = 0;
    for (int64_t t = 0; t < tiles; ++t) {
        const int64_t r0 = 16 * t, R = std::min<int64_t>(16, M - r0);
        base[t] = uint32_t(total);
        uint32_t in_tile = 0;
        for (int64_t g = 0; g < G; ++g) {
            uint32_t mask = 0;
            for (int64_t mi = 0; mi < R; ++mi) {
                bool zero = true;
                for (int wd = 0; wd < 8; ++wd) zero = zero && word(r0 + mi, g, wd) == 0x55555555u;
                if (!zero) mask |= 1u << mi;
            }
            slabs[t * G + g] = mask | (in_tile << 16);
            in_tile += uint32_t(__builtin_popcount(mask));
        }
        total += in_tile;
        if (total > int64_t(UINT32_MAX)) return fail(MBD_ESHAPE, "too many stored blocks");
    }
    base[tiles] = uint32_t(total);
    h->sec[0].name = "codes";
    h->sec[0].resize(uint64_t(total) * 32);
    uint32_t* codes = h->sec[0].as<uint32_t>();
    for (int64_t t = 0; t < tiles; ++t) {
        const int64_t r0 = 16 * t, R = std::min<int64_t>(16, M - r0);
        for (int64_t g = 0; g < G; ++g) {
            const uint32_t sw = slabs[t * G + g], mask = sw & 0xFFFFu;
            const int nz = __builtin_popcount(mask);
            uint32_t* dst = codes + (int64_t(base[t]) + (sw >> 16)) * 8;
            int r = 0;
            for (int64_t mi = 0; mi < R; ++mi) {
                if (!((mask >> mi) & 1)) continue;
                for (int kq = 0; kq < 4; ++kq)
                    for (int j = 0; j < 2; ++j) dst[(kq * nz + r) * 2 + j] = word(r0 + mi, g, 2 * kq + j);
                ++r;
            }
        }
    }
    return MBD_OK;
}

// ------------------------------------------------------------------ Cassandra

// Wanda keep bitmap ([Cassandra] 3.2): per row the floor(K * keep) highest
// |w| * norm, ties to the lower k; also rejects non-finite inputs.
mbd_status wanda_bitmap(const mbd_packed* h, const uint16_t* w, const float* norm, std::vector<uint32_t>& bitmap) {
    const int64_t M = h->M, K = h->K, N = M * K;
    const int64_t nk_row = (K * h->keep_num) / h->keep_den;
    for (int64_t k = 0; k < K; ++k)
        if (!std::isfinite(norm[k]) || norm[k] < 0.f)
            return fail(MBD_ERANGE, "act_norm[%lld] is negative or not finite", (long long)k);
    for (int64_t f = 0; f < N; ++f)
        if (bf16_nonfinite(w[f])) return fail(MBD_ERANGE, "bf16 Inf/NaN at flat index %lld", (long long)f);
    bitmap.assign((N + 31) / 32, 0);
    parallel_rows(M, [&](int64_t r0, int64_t r1) {
        std::vector<double> score(K);
        std::vector<int32_t> idx(K);
        for (int64_t m = r0; m < r1; ++m) {
            for (int64_t k = 0; k < K; ++k) {
                score[k] = std::fabs(bf16_to_double(w[m * K + k])) * double(norm[k]);
                idx[k] = int32_t(k);
            }
            auto better = [&](int32_t a, int32_t b) {
                return score[a] > score[b] || (score[a] == score[b] && a < b);
            };
            if (nk_row > 0 && nk_row < K)
                std::nth_element(idx.begin(), idx.begin() + nk_row, idx.end(), better);
            for (int64_t i = 0; i < nk_row; ++i) {
                int64_t f = m * K + idx[i];
                // rows may share a bitmap word: set bits atomically per word
                __atomic_fetch_or(&bitmap[f >> 5], 1u << (f & 31), __ATOMIC_RELAXED);
            }
        }
    });
    return MBD_OK;
}

mbd_status pack_cassandra(mbd_packed* h, const uint16_t* w, const float* norm) {
    const int64_t N = h->M * h->K;
    // 1. Wanda keep bitmap.
    std::vector<uint32_t> bitmap;
    mbd_status st = wanda_bitmap(h, w, norm, bitmap);
    if (st != MBD_OK) return st;
    const int64_t nbw = int64_t(bitmap.size());

    // 2. Exponent histogram of kept values -> codebook by (-count, exponent).
    int64_t hist[256] = {0};
    int64_t nk = 0;
    for (int64_t f = 0; f < N; ++f)
        if ((bitmap[f >> 5] >> (f & 31)) & 1) { hist[(w[f] >> 7) & 0xFF]++; nk++; }
    std::vector<int> syms;
    for (int e = 0; e < 256; ++e) if (hist[e]) syms.push_back(e);
    std::sort(syms.begin(), syms.end(), [&](int a, int b) {
        return hist[a] > hist[b] || (hist[a] == hist[b] && a < b);
    });
    int rank_of[256];
    std::fill(rank_of, rank_of + 256, -1);
    for (size_t r = 0; r < syms.size(); ++r) rank_of[syms[r]] = int(r);
    int64_t ubits = 0;
    for (int e = 0; e < 256; ++e) if (hist[e]) ubits += hist[e] * (rank_of[e] + 1);

    const int64_t T = (N + kTile - 1) / kTile;
    h->n_kept = nk;
    h->n_sym = int32_t(syms.size());
    h->unary_bits = ubits;
    h->n_tiles = T;
    h->sec.resize(8);
    const char* names[8] = {"bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix",
                            "lo_nib", "pruned"};
    for (int i = 0; i < 8; ++i) h->sec[i].name = names[i];
    h->sec[0].resize(uint64_t(nbw) * 4);
    h->sec[1].resize(uint64_t((nk + 7) / 8) * 4);
    h->sec[2].resize(uint64_t((ubits + 31) / 32) * 4);
    h->sec[3].resize(syms.size());
    h->sec[4].resize(uint64_t(T + 1) * 8);
    h->sec[5].resize(uint64_t(T + 1) * 4);
    h->sec[6].resize(uint64_t((nk + 7) / 8) * 4);
    h->sec[7].resize(uint64_t(N - nk) * 2);
    std::memcpy(h->sec[0].buf.data(), bitmap.data(), nbw * 4);
    for (size_t r = 0; r < syms.size(); ++r) h->sec[3].buf[r] = uint8_t(syms[r]);
    uint32_t* spec = h->sec[1].as<uint32_t>();
    uint32_t* unary = h->sec[2].as<uint32_t>();
    uint64_t* bitoff = h->sec[4].as<uint64_t>();
    uint32_t* kprefix = h->sec[5].as<uint32_t>();
    uint32_t* lo = h->sec[6].as<uint32_t>();
    uint16_t* pruned = h->sec[7].as<uint16_t>();

    // 3. Split fields, write the unary stream and the tile table in flat order.
    int64_t j = 0, p = 0, pos = 0;
    for (int64_t f = 0; f < N; ++f) {
        if ((f % kTile) == 0) { bitoff[f / kTile] = uint64_t(pos); kprefix[f / kTile] = uint32_t(j); }
        uint16_t b = w[f];
        if ((bitmap[f >> 5] >> (f & 31)) & 1) {
            uint32_t S = b >> 15, E = (b >> 7) & 0xFF, Mn = b & 0x7F;
            uint32_t sn = (S << 3) | (Mn >> (7 - kMantHiBits));
            uint32_t ln = Mn & ((1u << (7 - kMantHiBits)) - 1);
            spec[j >> 3] |= sn << (4 * (j & 7));
            lo[j >> 3] |= ln << (4 * (j & 7));
            pos += rank_of[E];
            unary[pos >> 5] |= 1u << (pos & 31);
            pos += 1;
            ++j;
        } else {
            pruned[p++] = b;
        }
    }
    bitoff[T] = uint64_t(pos);
    kprefix[T] = uint32_t(j);
    return MBD_OK;
}

// ------------------------------------------------------------------ MX-32

mbd_status pack_mx32(mbd_packed* h, const uint16_t* w) {
    const int64_t M = h->M, K = h->K, G = K / 32;
    for (int64_t f = 0; f < M * K; ++f)
        if (bf16_nonfinite(w[f])) return fail(MBD_ERANGE, "bf16 Inf/NaN at flat index %lld", (long long)f);
    h->sec.resize(3);
    h->sec[0].name = "mx_exp";
    h->sec[0].resize(uint64_t(M * G));
    h->sec[1].name = "mx_sign";
    h->sec[1].resize(uint64_t(M * G) * 4);
    h->sec[2].name = "mx_mag";
    h->sec[2].resize(uint64_t(M * K));
    uint8_t* xe = h->sec[0].as<uint8_t>();
    uint32_t* sg = h->sec[1].as<uint32_t>();
    uint8_t* mag = h->sec[2].as<uint8_t>();
    for (int64_t gi = 0; gi < M * G; ++gi) {
        const uint16_t* src = w + gi * 32;
        int X = 1;
        for (int i = 0; i < 32; ++i) X = std::max(X, std::max(int((src[i] >> 7) & 0xFF), 1));
        uint32_t s = 0;
        for (int i = 0; i < 32; ++i) {
            int E = (src[i] >> 7) & 0xFF, Mn = src[i] & 0x7F;
            int ep = std::max(E, 1), sig = E ? (128 | Mn) : Mn, d = X - ep;
            mag[gi * 32 + i] = uint8_t(d >= 8 ? 0 : (sig >> d));
            s |= uint32_t(src[i] >> 15) << i;
        }
        xe[gi] = uint8_t(X);
        sg[gi] = s;
    }
    return MBD_OK;
}

// Cassandra-2 speculation data ([Cassandra] 3.3): the kept values of the same
// Wanda bitmap, in groups of 32 consecutive kept values sharing their largest
// effective exponent X = max(max(E, 1)); each keeps sign and the 4-bit
// significand (implicit one + 3 high mantissa bits) shifted right by X - e'.
mbd_status pack_cassandra_mx(mbd_packed* h, const uint16_t* w, const float* norm) {
    const int64_t N = h->M * h->K;
    std::vector<uint32_t> bitmap;
    mbd_status st = wanda_bitmap(h, w, norm, bitmap);
    if (st != MBD_OK) return st;
    int64_t nk = 0;
    for (uint32_t b : bitmap) nk += __builtin_popcount(b);
    const int64_t T = (N + kTile - 1) / kTile, ng = (nk + 31) / 32;
    h->n_kept = nk;
    h->n_tiles = T;
    h->sec.resize(5);
    const char* names[5] = {"bitmap", "mx_nib", "mx_sign", "mx_exp", "kprefix"};
    for (int i = 0; i < 5; ++i) h->sec[i].name = names[i];
    h->sec[0].resize(uint64_t(bitmap.size()) * 4);
    h->sec[1].resize(uint64_t((nk + 7) / 8) * 4);
    h->sec[2].resize(uint64_t(ng) * 4);
    h->sec[3].resize(uint64_t(ng));
    h->sec[4].resize(uint64_t(T + 1) * 4);
    std::memcpy(h->sec[0].buf.data(), bitmap.data(), bitmap.size() * 4);
    uint32_t* nib = h->sec[1].as<uint32_t>();
    uint32_t* sign = h->sec[2].as<uint32_t>();
    uint8_t* xexp = h->sec[3].as<uint8_t>();
    uint32_t* kprefix = h->sec[4].as<uint32_t>();
    uint16_t grp[32];
    int gn = 0;
    int64_t j = 0;
    auto flush = [&]() {
        const int64_t g = (j - gn) / 32;
        int X = 1;
        for (int i = 0; i < gn; ++i) X = std::max(X, std::max(int((grp[i] >> 7) & 0xFF), 1));
        for (int i = 0; i < gn; ++i) {
            const uint32_t b = grp[i], E = (b >> 7) & 0xFF, H = (b & 0x7F) >> (7 - kMantHiBits);
            const int d = X - std::max(int(E), 1);
            const uint32_t sig = E ? 8u + H : H, mag = d >= 4 ? 0u : sig >> d;
            const int64_t idx = 32 * g + i;
            nib[idx >> 3] |= mag << (4 * (idx & 7));
            sign[g] |= (b >> 15) << i;
        }
        xexp[g] = uint8_t(X);
        gn = 0;
    };
    for (int64_t f = 0; f < N; ++f) {
        if ((f % kTile) == 0) kprefix[f / kTile] = uint32_t(j);
        if ((bitmap[f >> 5] >> (f & 31)) & 1) {
            grp[gn++] = w[f];
            ++j;
            if (gn == 32) flush();
        }
    }
    if (gn) flush();
    kprefix[T] = uint32_t(j);
    return MBD_OK;
}

// ------------------------------------------------------------------ validation

mbd_status validate(const mbd_packed* h) {
    const int64_t M = h->M, K = h->K, N = M * K;
    if (h->fmt == MBD_TERNARY_B128 || h->fmt == MBD_INT4_G128) {
        bool ter = h->fmt == MBD_TERNARY_B128;
        const uint32_t* c = h->sec[0].as<uint32_t>();
        int64_t nw = int64_t(h->sec[0].bytes / 4);
        for (int64_t i = 0; i < nw; ++i) {
            uint32_t v = c[i];
            if (ter) {
                // a 2-bit field equal to 3 has both bits set
                if (v & (v >> 1) & 0x55555555u) return fail(MBD_EFORMAT, "ternary code 3 in word %lld", (long long)i);
            } else {
                for (int j = 0; j < 8; ++j)
                    if (((v >> (4 * j)) & 15) == 0) return fail(MBD_EFORMAT, "int4 code 0 in word %lld", (long long)i);
            }
        }
        const uint16_t* s = h->sec[1].as<uint16_t>();
        for (int64_t i = 0; i < M * (K / 128); ++i)
            if ((s[i] & 0x7C00) == 0x7C00) return fail(MBD_EFORMAT, "non-finite scale %lld", (long long)i);
        return MBD_OK;
    }
    if (h->fmt == MBD_TERNARY_SKIP) {
        const int64_t G = K / 128, tiles = (M + 15) / 16;
        const uint32_t* c = h->sec[0].as<uint32_t>();
        const uint32_t* sl = h->sec[2].as<uint32_t>();
        const uint32_t* base = h->sec[3].as<uint32_t>();
        for (int64_t i = 0; i < int64_t(h->sec[0].bytes / 4); ++i)
            if (c[i] & (c[i] >> 1) & 0x55555555u) return fail(MBD_EFORMAT, "ternary code 3 in word %lld", (long long)i);
        if (base[0] != 0) return fail(MBD_EFORMAT, "tile_base[0] != 0");
        for (int64_t t = 0; t < tiles; ++t) {
            const int64_t R = std::min<int64_t>(16, M - 16 * t);
            uint32_t in_tile = 0;
            for (int64_t g = 0; g < G; ++g) {
                const uint32_t sw = sl[t * G + g], mask = sw & 0xFFFFu;
                if ((mask >> R) || (sw >> 16) != in_tile) return fail(MBD_EFORMAT, "bad slab word (tile %lld, block %lld)", (long long)t, (long long)g);
                in_tile += uint32_t(__builtin_popcount(mask));
            }
            if (uint64_t(base[t + 1]) != uint64_t(base[t]) + in_tile) return fail(MBD_EFORMAT, "bad tile_base at tile %lld", (long long)t);
        }
        if (uint64_t(base[tiles]) * 32 != h->sec[0].bytes) return fail(MBD_EFORMAT, "codes size does not match the stored blocks");
        const uint16_t* s = h->sec[1].as<uint16_t>();
        for (int64_t i = 0; i < M * G; ++i)
            if ((s[i] & 0x7C00) == 0x7C00) return fail(MBD_EFORMAT, "non-finite scale %lld", (long long)i);
        return MBD_OK;
    }
    if (h->fmt == MBD_CASSANDRA_MX) {
        const uint32_t* bm = h->sec[0].as<uint32_t>();
        const uint8_t* xe = h->sec[3].as<uint8_t>();
        const uint32_t* kp = h->sec[4].as<uint32_t>();
        const int64_t nk_row = (K * h->keep_num) / h->keep_den;
        for (int64_t m = 0; m < M; ++m) {
            int64_t c = 0;
            for (int64_t k = 0; k < K; ++k) { int64_t f = m * K + k; c += (bm[f >> 5] >> (f & 31)) & 1; }
            if (c != nk_row) return fail(MBD_EFORMAT, "row %lld keeps %lld, expected %lld", (long long)m, (long long)c, (long long)nk_row);
        }
        int64_t j = 0;
        for (int64_t t = 0; t < h->n_tiles; ++t) {
            if (int64_t(kp[t]) != j) return fail(MBD_EFORMAT, "kprefix mismatch at tile %lld", (long long)t);
            for (int64_t f = t * kTile; f < std::min(N, (t + 1) * kTile); ++f) j += (bm[f >> 5] >> (f & 31)) & 1;
        }
        if (int64_t(kp[h->n_tiles]) != j || j != h->n_kept) return fail(MBD_EFORMAT, "kprefix sentinel mismatch");
        for (int64_t g = 0; g < (h->n_kept + 31) / 32; ++g)
            if (xe[g] == 0 || xe[g] == 255) return fail(MBD_EFORMAT, "bad shared exponent in group %lld", (long long)g);
        return MBD_OK;
    }
    if (h->fmt == MBD_MX32) {
        const uint8_t* xe = h->sec[0].as<uint8_t>();
        for (int64_t i = 0; i < M * (K / 32); ++i)
            if (xe[i] == 0 || xe[i] == 255) return fail(MBD_EFORMAT, "bad shared exponent %lld", (long long)i);
        return MBD_OK;
    }
    // Cassandra
    const uint32_t* bm = h->sec[0].as<uint32_t>();
    const uint32_t* un = h->sec[2].as<uint32_t>();
    const uint64_t* bo = h->sec[4].as<uint64_t>();
    const uint32_t* kp = h->sec[5].as<uint32_t>();
    const int64_t nk_row = (K * h->keep_num) / h->keep_den;
    for (int64_t m = 0; m < M; ++m) {
        int64_t c = 0;
        for (int64_t k = 0; k < K; ++k) { int64_t f = m * K + k; c += (bm[f >> 5] >> (f & 31)) & 1; }
        if (c != nk_row) return fail(MBD_EFORMAT, "row %lld keeps %lld, expected %lld", (long long)m, (long long)c, (long long)nk_row);
    }
    if (N % 32) {
        uint32_t tail = bm[N >> 5] >> (N & 31);
        if (tail) return fail(MBD_EFORMAT, "bitmap bits set past the last element");
    }
    int64_t bit = 0;
    for (int64_t t = 0; t < h->n_tiles; ++t) {
        int64_t a = t * kTile, b = std::min(N, a + kTile), c = 0;
        for (int64_t f = a; f < b; ++f) c += (bm[f >> 5] >> (f & 31)) & 1;
        if (int64_t(kp[t + 1]) - int64_t(kp[t]) != c) return fail(MBD_EFORMAT, "kprefix mismatch at tile %lld", (long long)t);
        if (int64_t(bo[t]) != bit) return fail(MBD_EFORMAT, "bitoff mismatch at tile %lld", (long long)t);
        // walk c codewords; each rank must be < n_sym
        for (int64_t i = 0; i < c; ++i) {
            int64_t r = 0;
            while (bit < h->unary_bits && !((un[bit >> 5] >> (bit & 31)) & 1)) { ++bit; ++r; }
            if (bit >= h->unary_bits) return fail(MBD_EFORMAT, "unary stream ends early in tile %lld", (long long)t);
            if (r >= h->n_sym) return fail(MBD_EFORMAT, "unary rank %lld outside the codebook", (long long)r);
            ++bit;
        }
    }
    if (int64_t(kp[h->n_tiles]) != h->n_kept || int64_t(bo[h->n_tiles]) != h->unary_bits || bit != h->unary_bits)
        return fail(MBD_EFORMAT, "tile table sentinel mismatch");
    return MBD_OK;
}

}  // namespace
}  // namespace mbd

using namespace mbd;

extern "C" {

const char* mbd_status_str(mbd_status s) {
    switch (s) {
        case MBD_OK: return "ok";
        case MBD_EINVAL: return "invalid argument";
        case MBD_ESHAPE: return "unsupported shape";
        case MBD_EALIGN: return "misaligned pointer";
        case MBD_ERANGE: return "value out of range";
        case MBD_EFORMAT: return "inconsistent packed data";
        case MBD_EHIP: return "HIP error";
        case MBD_ENOMEM: return "out of host memory";
        default: return "unknown status";
    }
}

const char* mbd_last_error(void) { return g_last_error.c_str(); }

mbd_status mbd_pack(int32_t fmt, const uint16_t* w, int64_t M, int64_t K, const float* act_norm,
                    const mbd_pack_params* params, mbd_packed** out) {
    if (!out) return fail(MBD_EINVAL, "out is NULL");
    *out = nullptr;
    if (!w) return fail(MBD_EINVAL, "w_bf16_host is NULL");
    if (fmt < MBD_TERNARY_B128 || fmt > MBD_CASSANDRA_MX) return fail(MBD_EINVAL, "unknown format %d", fmt);
    const bool cas = fmt == MBD_CASSANDRA || fmt == MBD_CASSANDRA_MX;
    if (M < 1 || K < 1) return fail(MBD_ESHAPE, "M and K must be positive");
    int64_t kmul = fmt == MBD_MX32 ? 32 : 128;
    if (K % kmul) return fail(MBD_ESHAPE, "K=%lld is not a multiple of %lld", (long long)K, (long long)kmul);
    if (cas && !act_norm) return fail(MBD_EINVAL, "Cassandra packing needs act_norm_host");
    int32_t kn = 3, kd = 10;
    int64_t nm = 1;
    if (params) { kn = params->keep_num; kd = params->keep_den; nm = params->n_mats ? params->n_mats : 1; }
    if (nm < 1 || M % nm) return fail(MBD_EINVAL, "n_mats=%lld does not divide M=%lld", (long long)nm, (long long)M);
    if (nm > 1 && fmt != MBD_TERNARY_B128 && fmt != MBD_INT4_G128) return fail(MBD_EINVAL, "n_mats > 1 needs TERNARY or INT4");
    if (cas && (kd < 1 || kn < 0 || kn > kd)) return fail(MBD_EINVAL, "keep fraction %d/%d", kn, kd);
    if (cas && M * K > int64_t(UINT32_MAX)) return fail(MBD_ESHAPE, "M*K exceeds the 32-bit kept prefix");
    mbd_packed* h = nullptr;
    try {
        h = new mbd_packed();
        h->fmt = fmt; h->M = M; h->K = K; h->keep_num = kn; h->keep_den = kd;
        RoundNearest rn;
        mbd_status s;
        switch (fmt) {
            case MBD_TERNARY_B128: s = pack_block_quant(h, w, true, nm); break;
            case MBD_INT4_G128: s = pack_block_quant(h, w, false, nm); break;
            case MBD_CASSANDRA: s = pack_cassandra(h, w, act_norm); break;
            case MBD_TERNARY_SKIP: s = pack_ternary_skip(h, w); break;
            case MBD_CASSANDRA_MX: s = pack_cassandra_mx(h, w, act_norm); break;
            default: s = pack_mx32(h, w); break;
        }
        if (s != MBD_OK) { delete h; return s; }
    } catch (const std::bad_alloc&) {
        delete h;
        return fail(MBD_ENOMEM, "host allocation failed while packing");
    }
    *out = h;
    return MBD_OK;
}

mbd_status mbd_packed_sections(const mbd_packed* h, mbd_section* arr, int32_t cap, int32_t* n) {
    if (!h || !n) return fail(MBD_EINVAL, "NULL argument");
    *n = int32_t(h->sec.size());
    if (cap > 0 && !arr) return fail(MBD_EINVAL, "arr is NULL");
    for (int32_t i = 0; i < std::min<int32_t>(cap, *n); ++i)
        arr[i] = mbd_section{h->sec[i].name, h->sec[i].buf.data(), h->sec[i].bytes, uint64_t(h->sec[i].buf.size())};
    return MBD_OK;
}

mbd_status mbd_packed_stats(const mbd_packed* h, mbd_stats* o) {
    if (!h || !o) return fail(MBD_EINVAL, "NULL argument");
    std::memset(o, 0, sizeof *o);
    o->fmt = h->fmt; o->M = h->M; o->K = h->K; o->n_sym = h->n_sym; o->n_kept = h->n_kept;
    o->unary_bits = h->unary_bits; o->n_tiles = h->n_tiles; o->zero_fraction = h->zero_fraction;
    double n = double(h->M) * double(h->K), total = 0;
    for (auto& s : h->sec) total += double(s.bytes) * 8;
    o->bpw = total / n;
    if (h->fmt == MBD_CASSANDRA_MX) o->spec_bpw = o->bpw;   // speculation data only
    if (h->fmt == MBD_CASSANDRA) {
        double spec = 0;
        for (int i = 0; i < 6; ++i) spec += double(h->sec[i].bytes) * 8;
        o->spec_bpw = spec / n;
        o->unary_avg_bits = h->n_kept ? double(h->unary_bits) / double(h->n_kept) : 0.0;
        // entropy from the codebook-rank histogram recomputed off the stream
        std::vector<int64_t> cnt(h->n_sym, 0);
        const uint32_t* un = h->sec[2].as<uint32_t>();
        int64_t r = 0;
        for (int64_t b = 0; b < h->unary_bits; ++b) {
            if ((un[b >> 5] >> (b & 31)) & 1) { if (r < h->n_sym) cnt[r]++; r = 0; } else ++r;
        }
        double H = 0;
        for (auto c : cnt) if (c) { double p = double(c) / double(h->n_kept); H -= p * std::log2(p); }
        o->exp_entropy_bits = H;
    }
    return MBD_OK;
}

mbd_status mbd_validate(const mbd_packed* h) {
    if (!h) return fail(MBD_EINVAL, "NULL handle");
    return validate(h);
}

void mbd_packed_free(mbd_packed* h) { delete h; }

}  // extern "C"
