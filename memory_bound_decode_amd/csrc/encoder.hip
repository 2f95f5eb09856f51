// Cassandra encoder on the device ([Cassandra] 3.2 value pruning, mantissa
// split; 3.3 frequency-ranked unary exponent code; 3.5 the online encoder the
// paper builds in hardware): the MBD_CASSANDRA sections of a bf16 weight already
// in device memory, bit-identical to the CPU packer.
//
// One workgroup per row for the row-local steps; the rows are independent except
// for the exponent histogram (integer atomics, so the counts do not depend on
// timing) and the row offsets of the unary stream (one exclusive scan).
//
//   plan:   clear -> select (Wanda top-k per row, histogram of kept exponents)
//           -> codebook (ranks by (-count, exponent), totals) -> host reads totals
//   encode: clear -> select (writes the bitmap) -> codebook -> row bits
//           -> row offsets -> write (nibbles, pruned values, unary bits, tile table)
//
// A thread of a row owns a run of whole bitmap words (32 columns each), so the
// row's elements are visited in column order thread by thread, and block scans
// give each thread its first kept index, pruned index and unary bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>

#include "hip_check.h"
#include "mbd_internal.h"

namespace mbd {
namespace enc {

constexpr int TILE = 4096;
constexpr int NT = 256;                 // threads per row workgroup
constexpr int MANT_LO_BITS = 7 - kMantHiBits;

// Workspace: header, histogram, rank table, per-row unary bits (then offsets).
struct Header {
    uint32_t n_sym;
    uint32_t bad;                       // bit 0: non-finite weight, bit 1: bad norm
    uint64_t unary_bits;
};
constexpr size_t WS_HIST = 64, WS_RANK = WS_HIST + 256 * 4, WS_ROWS = WS_RANK + 256 * 4;

struct EncArgs {
    const uint16_t* w;
    const float* norm;
    int64_t M, K;
    int32_t nk;                         // kept values per row
    Header* hdr;
    uint32_t* hist;                     // [256]
    uint32_t* rank_of;                  // [256]
    uint64_t* rows;                     // [M] unary bits per row, then exclusive offsets
    // sections (encode only)
    uint32_t* bitmap;
    uint32_t* spec_nib;
    uint32_t* unary;
    uint8_t* codebook;
    uint64_t* bitoff;
    uint32_t* kprefix;
    uint32_t* lo_nib;
    uint16_t* pruned;
};

// Wanda score |w| * norm as an exact, order-preserving 64-bit integer: |w| =
// ws 2^wx (8-bit significand), norm = ns 2^nx (24-bit), so the product's
// significand P = ws ns fits 32 bits; normalised to bit 31 it sits below a
// biased exponent.  A zero score is key 0.
__device__ __forceinline__ uint64_t score_key(uint16_t wb, float nrm) {
    const uint32_t we = (wb >> 7) & 0xFFu, wm = wb & 0x7Fu;
    const uint32_t nb = __float_as_uint(nrm), ne = (nb >> 23) & 0xFFu, nm = nb & 0x7FFFFFu;
    const uint32_t ws = we ? 128u + wm : wm, ns = ne ? (1u << 23) + nm : nm;
    uint32_t P = ws * ns;                                    // < 2^32
    if (P == 0u) return 0ull;
    const int lz = __clz(int(P));
    P <<= lz;
    const int X = int(we ? we : 1u) - 134 + int(ne ? ne : 1u) - 150 - lz + 400;   // in [87, 1024)
    return (uint64_t(uint32_t(X)) << 32) | P;
}

template <class T>
__device__ T block_excl_scan(T v, T* tmp, T* total) {
    const int t = threadIdx.x;
    tmp[t] = v;
    __syncthreads();
    for (int o = 1; o < blockDim.x; o <<= 1) {
        const T u = t >= o ? tmp[t - o] : T(0);
        __syncthreads();
        tmp[t] += u;
        __syncthreads();
    }
    const T incl = tmp[t];
    if (total) *total = tmp[blockDim.x - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(256) void enc_clear_kernel(Header* hdr, uint32_t* hist) {
    const int t = threadIdx.x;
    hist[t] = 0u;
    if (t == 0) { hdr->n_sym = 0u; hdr->bad = 0u; hdr->unary_bits = 0ull; }
}

// Zero n 32-bit words (the streams written with atomic ors, and their padding).
__global__ __launch_bounds__(256) void enc_zero_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x)
        p[i] = 0u;
}

// A 32-bit key that never inverts the exact order: the exact key's top bits
// (for scores a > b, key32(a) >= key32(b); key32(a) > key32(b) implies a > b).
__device__ __forceinline__ uint32_t score_key32(uint16_t wb, float nrm) {
    return uint32_t(score_key(wb, nrm) >> 10);
}

constexpr int NS = 512;                 // threads per row in the selection

// Sum of v over the workgroup (NS threads); `slot` alternates between calls so
// that one barrier per call suffices.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t (*part)[NS / 64], int slot) {
    // 16-lane row sums with DPP moves (no LDS round trips), then the four rows'
    // sums from lanes 0, 16, 32, 48
    v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
    v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
    v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x141, 0xF, 0xF, true));   // row_half_mirror
    v += uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x140, 0xF, 0xF, true));   // row_mirror
    v = uint32_t(__builtin_amdgcn_readlane(int(v), 0)) + uint32_t(__builtin_amdgcn_readlane(int(v), 16)) +
        uint32_t(__builtin_amdgcn_readlane(int(v), 32)) + uint32_t(__builtin_amdgcn_readlane(int(v), 48));
    if ((threadIdx.x & 63) == 0) part[slot][threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < NS / 64; ++i) s += part[slot][i];
    return s;
}

// Per row: the nk largest scores, ties to the lower column ([Cassandra] 3.2).
// The threshold is built bit by bit from the top, each bit kept when enough keys
// reach it (a count per bit, no per-element atomics): first on the 32-bit keys,
// which settles every column whose key differs from the threshold's, then on the
// exact 64-bit keys of the columns that share the threshold's 32-bit key; a block
// scan in column order keeps the first of the exact ties.  A thread owns WPT
// bitmap words (32 WPT columns) and holds their 32-bit keys in registers (WPT = 0:
// any width, keys recomputed from memory).  Adds the kept exponents to the
// histogram; WRITE also stores the row's bitmap words.
template <bool WRITE, int WPT>
__global__ __launch_bounds__(NS) void enc_select_kernel(EncArgs a) {
    __shared__ uint32_t lhist[256];
    __shared__ uint32_t part[2][NS / 64];
    __shared__ uint32_t scan[NS];
    constexpr int CPT = WPT > 0 ? 32 * WPT : 1;
    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int K = int(a.K), nwords = K / 32;
    const int wpt = WPT > 0 ? WPT : (nwords + NS - 1) / NS;
    const int w0 = min(nwords, t * wpt), w1 = min(nwords, w0 + wpt);
    const int c0 = 32 * w0, c1 = 32 * w1;
    const uint16_t* wr = a.w + r * a.K;
    if (t < 256) lhist[t] = 0u;
    uint32_t kk[CPT];
    if constexpr (WPT > 0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) kk[i] = c0 + i < c1 ? score_key32(wr[c0 + i], a.norm[c0 + i]) : 0u;
    }
    // f(i, key32) for the thread's columns c0 + i in order (register keys are
    // indexed only from fully unrolled loops)
    auto each = [&](auto&& f) __attribute__((always_inline)) {
        if constexpr (WPT > 0) {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                if (c0 + i < c1) f(i, kk[i]);
        } else {
            for (int i = 0; i < c1 - c0; ++i) f(i, score_key32(wr[c0 + i], a.norm[c0 + i]));
        }
    };
    auto key64 = [&](int i) { return score_key(wr[c0 + i], a.norm[c0 + i]); };
    // input checks (reported through the header)
    for (int c = c0; c < c1; ++c) {
        if (((wr[c] >> 7) & 0xFF) == 0xFF) atomicOr(&a.hdr->bad, 1u);
        if (r == 0 && !(a.norm[c] >= 0.f && a.norm[c] <= 3.402823466e38f)) atomicOr(&a.hdr->bad, 2u);
    }
    const bool all = a.nk >= K, none = a.nk <= 0;
    int slot = 0;
    uint32_t T32 = 0, rem = 0;
    uint64_t T64 = 0;
    bool exact = false;                  // the tie set needs the 64-bit keys
    if (!all && !none) {
        const uint32_t nk = uint32_t(a.nk);
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T32 | (1u << bit);
            uint32_t n = 0;
            each([&](int, uint32_t k) { n += k >= cand; });
            if (block_sum(n, part, slot) >= nk) T32 = cand;
            slot ^= 1;
        }
        uint32_t gt = 0, eq = 0;
        each([&](int, uint32_t k) {
            gt += k > T32;
            eq += k == T32;
        });
        const uint32_t need = nk - block_sum(gt, part, slot);
        slot ^= 1;
        const uint32_t neq = block_sum(eq, part, slot);
        slot ^= 1;
        rem = need;
        if (neq > need) {                                // order the tie set exactly
            exact = true;
            for (int bit = 41; bit >= 0; --bit) {        // keys are below 2^42
                const uint64_t cand = T64 | (1ull << bit);
                uint32_t n = 0;
                each([&](int i, uint32_t k) { n += k == T32 && key64(i) >= cand; });
                if (block_sum(n, part, slot) >= need) T64 = cand;
                slot ^= 1;
            }
            uint32_t g64 = 0;
            each([&](int i, uint32_t k) { g64 += k == T32 && key64(i) > T64; });
            rem = need - block_sum(g64, part, slot);
            slot ^= 1;
        }
    }
    // keep: key32 > T32; key32 == T32 and (no exact step, or key64 > T64, or
    // key64 == T64 among the first `rem` such columns in column order)
    uint32_t tie = 0;
    if (!all && !none) each([&](int i, uint32_t k) { tie += k == T32 && (!exact || key64(i) == T64); });
    uint32_t e = block_excl_scan<uint32_t>(tie, scan, nullptr);
    uint32_t cur = 0;
    each([&](int i, uint32_t k) {
        bool keep = all;
        if (!all && !none) {
            if (k > T32) {
                keep = true;
            } else if (k == T32) {
                if (!exact) {
                    keep = e++ < rem;
                } else {
                    const uint64_t k64 = key64(i);
                    keep = k64 > T64 || (k64 == T64 && e++ < rem);
                }
            }
        }
        if (keep) {
            cur |= 1u << (i & 31);
            atomicAdd(&lhist[(wr[c0 + i] >> 7) & 0xFF], 1u);
        }
        if ((i & 31) == 31) {                            // c1 - c0 is whole words
            if constexpr (WRITE) a.bitmap[(r * a.K) / 32 + w0 + (i >> 5)] = cur;
            cur = 0;
        }
    });
    __syncthreads();
    if (t < 256 && lhist[t]) atomicAdd(&a.hist[t], lhist[t]);
}

// Codebook: present exponents ranked by (-count, exponent); totals to the header.
__global__ __launch_bounds__(256) void enc_codebook_kernel(EncArgs a, int write_cb) {
    __shared__ uint32_t c[256];
    __shared__ uint64_t bits[256];
    const int e = threadIdx.x;
    c[e] = a.hist[e];
    __syncthreads();
    uint32_t rank = 0, present = 0;
    for (int f = 0; f < 256; ++f) {
        present += c[f] > 0;
        rank += c[f] > 0 && (c[f] > c[e] || (c[f] == c[e] && f < e));
    }
    a.rank_of[e] = c[e] ? rank : 0u;
    if (c[e] && write_cb) a.codebook[rank] = uint8_t(e);
    bits[e] = uint64_t(c[e]) * (rank + 1);
    __syncthreads();
    if (e == 0) {
        uint64_t s = 0;
        for (int f = 0; f < 256; ++f) s += bits[f];
        a.hdr->n_sym = present;
        a.hdr->unary_bits = s;
    }
}

// Unary bits of each row's kept values.
__global__ __launch_bounds__(NT) void enc_rowbits_kernel(EncArgs a) {
    __shared__ uint64_t scan[NT];
    __shared__ uint32_t rk[256];
    const int t = threadIdx.x;
    rk[t] = a.rank_of[t];
    __syncthreads();
    const int64_t r = blockIdx.x;
    // The row's sum does not depend on the order, so thread t takes the 8-value
    // chunks t, t + NT, ...: one 16-byte load of the row (consecutive threads,
    // consecutive chunks) and the chunk's bitmap byte (bit i = value 8c + i).
    // Rows start 16-byte aligned (w is, and K is a multiple of 128).
    const int nch = int(a.K / 8);
    const uint4* wr = reinterpret_cast<const uint4*>(a.w + r * a.K);
    const uint8_t* bm = reinterpret_cast<const uint8_t*>(a.bitmap + (r * a.K) / 32);
    uint64_t b = 0;
    for (int c = t; c < nch; c += NT) {
        const uint32_t m = bm[c];
        const uint4 v = wr[c];
        const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((m >> i) & 1u) b += rk[(e[i >> 1] >> (16 * (i & 1) + 7)) & 0xFFu] + 1;
    }
    uint64_t total;
    block_excl_scan<uint64_t>(b, scan, &total);
    if (t == 0) a.rows[r] = total;
}

// Exclusive offsets of the rows' unary bits (one workgroup, rows in chunks).
__global__ __launch_bounds__(1024) void enc_rowscan_kernel(EncArgs a) {
    __shared__ uint64_t scan[1024];
    __shared__ uint64_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < a.M; base += blockDim.x) {
        const int64_t r = base + threadIdx.x;
        const uint64_t v = r < a.M ? a.rows[r] : 0ull;
        uint64_t total;
        const uint64_t ex = block_excl_scan<uint64_t>(v, scan, &total);
        if (r < a.M) a.rows[r] = carry + ex;
        __syncthreads();
        if (threadIdx.x == 0) carry += total;
        __syncthreads();
    }
}

// Words of a stream that one thread fills in order: a word wholly inside the
// thread's range is stored, a word it shares with a neighbour is or'ed in (the
// stream starts zeroed).
struct WordSink {
    uint32_t* p;
    uint64_t lo, hi;        // the thread's bit range [lo, hi)
    uint64_t cap;           // words in the buffer
    uint64_t idx = ~0ull;
    uint32_t cur = 0;
    __device__ __forceinline__ void flush() {
        if (idx == ~0ull || idx >= cap) return;
        const bool whole = idx * 32 >= lo && idx * 32 + 32 <= hi;
        if (whole) p[idx] = cur;
        else if (cur) atomicOr(&p[idx], cur);
    }
    __device__ __forceinline__ void put(uint64_t bit, uint32_t v) {   // v placed at bit (within one word)
        const uint64_t w = bit >> 5;
        if (w != idx) {
            flush();
            idx = w;
            cur = 0;
        }
        cur |= v << (bit & 31);
    }
};

// The streams of one row: kept values' nibbles and unary codes in kept order,
// pruned values raw, and the tile-table entries of tiles that start in the row.
// NS threads; a thread owns WPT bitmap words (32 WPT columns), read as 16-byte
// loads into registers (WPT = 0: any width, read element by element).  Unary
// writes stay below cap_words (the caller's buffer), also if w changed between
// the plan and this call.
template <int WPT>
__global__ __launch_bounds__(NS) void enc_write_kernel(EncArgs a, int64_t T, uint64_t total_bits, uint64_t cap_words) {
    __shared__ uint32_t scan32[NS];
    __shared__ uint64_t scan64[NS];
    __shared__ uint32_t rk[256];
    constexpr int CPT = WPT > 0 ? 32 * WPT : 2;
    const int t = threadIdx.x;
    if (t < 256) rk[t] = a.rank_of[t];
    __syncthreads();
    const int64_t r = blockIdx.x, K = a.K;
    const int nwords = int(K / 32), wpt = WPT > 0 ? WPT : (nwords + NS - 1) / NS;
    const int w0 = min(nwords, t * wpt), w1 = min(nwords, w0 + wpt);
    const int c0 = 32 * w0, c1 = 32 * w1;
    const uint16_t* wr = a.w + r * K;
    const uint32_t* bm = a.bitmap + (r * K) / 32;
    uint32_t wv[CPT / 2], bw[WPT > 0 ? WPT : 1];
    if constexpr (WPT > 0) {
        // words past the thread's last (the row's last thread may own fewer) read as 0
#pragma unroll
        for (int q = 0; q < WPT; ++q) {
            const bool own = w0 + q < w1;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint4 v = own ? *reinterpret_cast<const uint4*>(wr + c0 + 32 * q + 8 * h) : make_uint4(0, 0, 0, 0);
                wv[16 * q + 4 * h] = v.x; wv[16 * q + 4 * h + 1] = v.y;
                wv[16 * q + 4 * h + 2] = v.z; wv[16 * q + 4 * h + 3] = v.w;
            }
            bw[q] = own ? bm[w0 + q] : 0u;
        }
    }
    // f(i, w bits, kept) for the thread's columns c0 + i in order
    auto each = [&](auto&& f) __attribute__((always_inline)) {
        if constexpr (WPT > 0) {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
                if (c0 + i < c1) f(i, uint16_t(wv[i >> 1] >> (16 * (i & 1))), ((bw[i >> 5] >> (i & 31)) & 1u) != 0u);
        } else {
            for (int i = 0; i < c1 - c0; ++i) f(i, wr[c0 + i], ((bm[w0 + (i >> 5)] >> (i & 31)) & 1u) != 0u);
        }
    };
    uint32_t kc = 0;
    uint64_t bc = 0;
    each([&](int, uint16_t v, bool kept) {
        if (kept) {
            ++kc;
            bc += rk[(v >> 7) & 0xFF] + 1;
        }
    });
    uint32_t j = block_excl_scan<uint32_t>(kc, scan32, nullptr);      // kept before, in the row
    uint64_t bit = a.rows[r] + block_excl_scan<uint64_t>(bc, scan64, nullptr);
    if (r == a.M - 1 && t == 0) {                                      // sentinel
        a.kprefix[T] = uint32_t(a.M * int64_t(a.nk));
        a.bitoff[T] = total_bits;
    }
    if (c0 >= c1) return;
    const int64_t kbase = r * int64_t(a.nk), pbase = r * (K - a.nk);
    const uint64_t g0 = uint64_t(kbase + j), nib_words = (uint64_t(a.M) * a.nk + 7) / 8;
    WordSink sn{a.spec_nib, 4 * g0, 4 * (g0 + kc), nib_words};
    WordSink ln{a.lo_nib, 4 * g0, 4 * (g0 + kc), nib_words};
    WordSink un{a.unary, bit, bit + bc, cap_words};
    each([&](int i, uint16_t v, bool kept) {
        const int64_t c = c0 + i, f = r * K + c;
        if (f % TILE == 0) {                                           // a tile starts here
            a.kprefix[f / TILE] = uint32_t(kbase + j);
            a.bitoff[f / TILE] = bit;
        }
        if (kept) {
            const uint64_t g = uint64_t(kbase + j);
            const uint32_t S = v >> 15, E = (v >> 7) & 0xFF, Mn = v & 0x7F;
            sn.put(4 * g, (S << 3) | (Mn >> MANT_LO_BITS));
            ln.put(4 * g, Mn & ((1u << MANT_LO_BITS) - 1));
            const uint64_t end = bit + rk[E];                         // rank zeros, then the one
            un.put(end, 1u);
            bit = end + 1;
            ++j;
        } else {
            a.pruned[pbase + (c - j)] = v;
        }
    });
    sn.flush();
    ln.flush();
    un.flush();
}

}  // namespace enc
}  // namespace mbd

using namespace mbd;
using namespace mbd::enc;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

mbd_status enc_args(const uint16_t* w, const float* norm, int64_t M, int64_t K, int32_t kn, int32_t kd, void* ws,
                    uint64_t ws_bytes, EncArgs* a) {
    if (!w || !norm || !ws) return fail(MBD_EINVAL, "NULL argument");
    if (M < 1 || K < 128 || K % 128) return fail(MBD_ESHAPE, "the encoder needs M >= 1 and K a positive multiple of 128");
    if (M * K > int64_t(UINT32_MAX)) return fail(MBD_ESHAPE, "M*K exceeds the 32-bit kept prefix");
    if (M > INT32_MAX) return fail(MBD_ESHAPE, "too many rows");
    if (kd < 1 || kn < 0 || kn > kd) return fail(MBD_EINVAL, "keep fraction %d/%d", kn, kd);
    uint64_t need = 0;
    mbd_encode_workspace_bytes(M, &need);
    if (ws_bytes < need) return fail(MBD_EINVAL, "workspace of %llu bytes, need %llu", (unsigned long long)ws_bytes,
                                     (unsigned long long)need);
    if (!aligned16(w) || !aligned16(ws) || (reinterpret_cast<uintptr_t>(norm) & 3))
        return fail(MBD_EALIGN, "w and ws must be 16-byte, act_norm 4-byte aligned");
    std::memset(a, 0, sizeof *a);
    char* base = static_cast<char*>(ws);
    a->w = w; a->norm = norm; a->M = M; a->K = K;
    a->nk = int32_t((K * kn) / kd);
    a->hdr = reinterpret_cast<Header*>(base);
    a->hist = reinterpret_cast<uint32_t*>(base + WS_HIST);
    a->rank_of = reinterpret_cast<uint32_t*>(base + WS_RANK);
    a->rows = reinterpret_cast<uint64_t*>(base + WS_ROWS);
    return MBD_OK;
}

uint64_t padded(uint64_t b) { return padded_size(b); }

// Selection with the keys in registers for rows up to 4 words a thread.
template <bool WRITE>
mbd_status launch_select(const EncArgs& a, hipStream_t st) {
    const int64_t wpt = (a.K / 32 + NS - 1) / NS;
    const dim3 g(unsigned(a.M)), b(NS);
    if (wpt <= 1) hipLaunchKernelGGL((enc_select_kernel<WRITE, 1>), g, b, 0, st, a);
    else if (wpt <= 2) hipLaunchKernelGGL((enc_select_kernel<WRITE, 2>), g, b, 0, st, a);
    else if (wpt <= 4) hipLaunchKernelGGL((enc_select_kernel<WRITE, 4>), g, b, 0, st, a);
    else hipLaunchKernelGGL((enc_select_kernel<WRITE, 0>), g, b, 0, st, a);
    return hip_check("encoder selection launch");
}

}  // namespace

extern "C" {

mbd_status mbd_encode_workspace_bytes(int64_t M, uint64_t* bytes) {
    if (!bytes) return fail(MBD_EINVAL, "bytes is NULL");
    if (M < 1) return fail(MBD_ESHAPE, "M must be positive");
    *bytes = WS_ROWS + uint64_t(M) * 8;
    return MBD_OK;
}

mbd_status mbd_encode_plan(const uint16_t* w, const float* act_norm, int64_t M, int64_t K, int32_t keep_num,
                           int32_t keep_den, void* ws, uint64_t ws_bytes, mbd_encode_plan_t* plan, void* stream) {
    hip_clear();
    if (!plan) return fail(MBD_EINVAL, "plan is NULL");
    EncArgs a;
    mbd_status s = enc_args(w, act_norm, M, K, keep_num, keep_den, ws, ws_bytes, &a);
    if (s != MBD_OK) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(enc_clear_kernel, dim3(1), dim3(256), 0, st, a.hdr, a.hist);
    if ((s = launch_select<false>(a, st)) != MBD_OK) return s;
    hipLaunchKernelGGL(enc_codebook_kernel, dim3(1), dim3(256), 0, st, a, 0);
    if ((s = hip_check("encoder plan launch")) != MBD_OK) return s;
    Header h;
    if (hipMemcpyAsync(&h, a.hdr, sizeof h, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return hip_check("encoder plan read-back");
    if (h.bad & 1u) return fail(MBD_ERANGE, "bf16 Inf/NaN in w");
    if (h.bad & 2u) return fail(MBD_ERANGE, "act_norm has a negative or non-finite entry");
    const int64_t N = M * K, nk = M * int64_t(a.nk), T = (N + TILE - 1) / TILE;
    std::memset(plan, 0, sizeof *plan);
    plan->n_kept = nk;
    plan->n_sym = int32_t(h.n_sym);
    plan->unary_bits = int64_t(h.unary_bits);
    plan->n_tiles = T;
    const uint64_t b[8] = {uint64_t((N + 31) / 32) * 4, uint64_t((nk + 7) / 8) * 4, (h.unary_bits + 31) / 32 * 4,
                           uint64_t(h.n_sym),          uint64_t(T + 1) * 8,       uint64_t(T + 1) * 4,
                           uint64_t((nk + 7) / 8) * 4, uint64_t(N - nk) * 2};
    for (int i = 0; i < 8; ++i) {
        plan->bytes[i] = b[i];
        plan->padded_bytes[i] = padded(b[i]);
    }
    return MBD_OK;
}

mbd_status mbd_encode_cassandra(const uint16_t* w, const float* act_norm, int64_t M, int64_t K, int32_t keep_num,
                                int32_t keep_den, const mbd_encode_plan_t* plan, void* const* sec, void* ws,
                                uint64_t ws_bytes, void* stream) {
    hip_clear();
    if (!plan || !sec) return fail(MBD_EINVAL, "NULL argument");
    EncArgs a;
    mbd_status s = enc_args(w, act_norm, M, K, keep_num, keep_den, ws, ws_bytes, &a);
    if (s != MBD_OK) return s;
    for (int i = 0; i < 8; ++i) {
        if (!sec[i]) return fail(MBD_EINVAL, "section %d is NULL", i);
        if (!aligned16(sec[i])) return fail(MBD_EALIGN, "section %d is not 16-byte aligned", i);
    }
    const int64_t N = M * K, T = (N + TILE - 1) / TILE;
    if (plan->n_kept != M * int64_t(a.nk) || plan->n_tiles != T)
        return fail(MBD_EINVAL, "plan does not match the shape and keep fraction");
    a.bitmap = static_cast<uint32_t*>(sec[0]);
    a.spec_nib = static_cast<uint32_t*>(sec[1]);
    a.unary = static_cast<uint32_t*>(sec[2]);
    a.codebook = static_cast<uint8_t*>(sec[3]);
    a.bitoff = static_cast<uint64_t*>(sec[4]);
    a.kprefix = static_cast<uint32_t*>(sec[5]);
    a.lo_nib = static_cast<uint32_t*>(sec[6]);
    a.pruned = static_cast<uint16_t*>(sec[7]);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // every section's padding is zeroed, and the streams written with atomic ors
    // entirely; the other sections' meaningful bytes are all written below
    for (int i = 0; i < 8; ++i) {
        const bool whole = i == 1 || i == 2 || i == 6;
        const uint64_t from = whole ? 0 : (plan->bytes[i] / 4) * 4;
        const int64_t words = int64_t((plan->padded_bytes[i] - from) / 4);
        hipLaunchKernelGGL(enc_zero_kernel, dim3(unsigned(std::min<int64_t>(1024, (words + 255) / 256 + 1))), dim3(256),
                           0, st, reinterpret_cast<uint32_t*>(static_cast<char*>(sec[i]) + from), words);
    }
    hipLaunchKernelGGL(enc_clear_kernel, dim3(1), dim3(256), 0, st, a.hdr, a.hist);
    if ((s = launch_select<true>(a, st)) != MBD_OK) return s;
    hipLaunchKernelGGL(enc_codebook_kernel, dim3(1), dim3(256), 0, st, a, 1);
    hipLaunchKernelGGL(enc_rowbits_kernel, dim3(unsigned(M)), dim3(NT), 0, st, a);
    hipLaunchKernelGGL(enc_rowscan_kernel, dim3(1), dim3(1024), 0, st, a);
    {
        const int64_t wpt = (K / 32 + NS - 1) / NS;
        const dim3 g(static_cast<unsigned>(M)), b(NS);
        const uint64_t ub = uint64_t(plan->unary_bits), cap = plan->padded_bytes[2] / 4;
        if (wpt <= 1) hipLaunchKernelGGL((enc_write_kernel<1>), g, b, 0, st, a, T, ub, cap);
        else if (wpt <= 2) hipLaunchKernelGGL((enc_write_kernel<2>), g, b, 0, st, a, T, ub, cap);
        else hipLaunchKernelGGL((enc_write_kernel<0>), g, b, 0, st, a, T, ub, cap);
    }
    return hip_check("encoder launch");
}

}  // extern "C"
