// Cassandra bit-split bf16 weights on gfx950 ([Cassandra] 3.2, 3.3, 3.5) and the
// MX-32 shared-exponent variant ([Cassandra] 3.3, Cassandra-2).
//
// One wave decodes one 4096-element tile.  The tile table (unary bit offset and
// kept prefix per tile) makes tiles independent, the software analogue of the
// paper's chunked decoder that carries boundary state between chunks:
//
//   A. unary -> kept values.  Lanes take consecutive 32-bit words of the tile's
//      unary stream; a wave prefix sum of the per-word one counts gives each
//      word's first codeword index and a wave max-scan gives the position of the
//      previous codeword end (the carried boundary state).  Each one bit closes a
//      codeword whose rank is the zero run before it; rank -> exponent through the
//      codebook in LDS, and the kept value (S, E, mantissa high bits, plus the low
//      nibble when restoring) is written to LDS in kept order.
//   B. bitmap -> dense.  Lane l owns elements [64l, 64l+64) of the tile (two
//      bitmap words); a wave prefix sum of their popcounts gives its first kept
//      index, and walking its 64 bits picks either the next kept value or the
//      next pruned value (restore: staged raw bits; draft: +0.0).  The 64
//      results stay in registers as 32 bf16 pairs.
//
// Consumers: dense store (draft decode / restore), dot2 against x (draft GEMV),
// or an LDS row block of 16 rows feeding v_mfma_f32_16x16x32_bf16 (verify GEMM,
// restore fused so the bf16 weight never goes to HBM).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "hip_check.h"
#include "mbd_internal.h"

namespace mbd {
namespace cas {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int TILE = 4096;
constexpr int ROW_STRIDE = 4168;   // u16 entries per LDS tile buffer (2084 dwords = 4 mod 32 banks)

struct CasArgs {
    const uint32_t* bitmap;
    const uint32_t* spec_nib;
    const uint32_t* unary;
    const uint8_t* codebook;
    const uint64_t* bitoff;
    const uint32_t* kprefix;
    const uint32_t* lo_nib;
    const uint16_t* pruned;
    int64_t M, K, N, T;
    int n_sym;
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int wave_incl_add(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (l >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_max(int v) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (l >= o) v = max(v, t);
    }
    return v;
}

// Rolling window over a packed nibble stream starting at nibble index n.
struct NibWin {
    uint64_t cur;
    uint32_t w2, w3, w4;
    int avail;
    __device__ __forceinline__ void init(const uint32_t* __restrict__ s, int64_t n) {
        const uint32_t* p = s + (n >> 3);
        const uint32_t w0 = p[0], w1 = p[1];
        w2 = p[2]; w3 = p[3]; w4 = p[4];
        const int sh = int(n & 7);
        cur = ((uint64_t(w1) << 32) | w0) >> (4 * sh);
        avail = 16 - sh;
    }
    __device__ __forceinline__ uint32_t next() {
        const uint32_t v = uint32_t(cur) & 15u;
        cur >>= 4;
        if (--avail == 8) {
            cur |= uint64_t(w2) << 32;
            w2 = w3; w3 = w4; avail = 16;
        }
        return v;
    }
};

// Decode tile t (tl elements) with one wave.  `buf` is this wave's LDS tile
// buffer (ROW_STRIDE u16 entries, 16-byte aligned), `cb` the codebook in LDS.
// On return pairs[i] holds elements 64*lane + 2i (low half) and 2i+1 (high half).
template <bool RESTORE>
__device__ __forceinline__ void decode_tile(const CasArgs& a, int64_t t, int tl, uint16_t* __restrict__ buf,
                                            const uint8_t* __restrict__ cb, uint32_t (&pairs)[32]) {
    const int lane = lane_id();
    const int64_t kp0 = a.kprefix[t], kp1 = a.kprefix[t + 1];
    const int64_t bo0 = int64_t(a.bitoff[t]), bo1 = int64_t(a.bitoff[t + 1]);
    const int nk = int(kp1 - kp0);
    const int np = tl - nk;
    const int64_t f0 = t * TILE;

    // bitmap words of this lane's 64 elements (zero past the end of the matrix)
    const int64_t wi = t * (TILE / 32) + 2 * lane;
    const int64_t nwords = (a.N + 31) >> 5;
    const uint32_t bw0 = wi < nwords ? a.bitmap[wi] : 0u;
    const uint32_t bw1 = wi + 1 < nwords ? a.bitmap[wi + 1] : 0u;

    // restore: stage this tile's pruned values at buf[o .. o+np)
    int o = 0, kreg = 0;
    if constexpr (RESTORE) {
        const int64_t pb = f0 - kp0;
        const int64_t a0 = pb & ~int64_t(7);
        o = int(pb - a0);
        const int units = (o + np + 7) >> 3;
        const uint4* src = reinterpret_cast<const uint4*>(a.pruned + a0);
        uint4* dst = reinterpret_cast<uint4*>(buf);
        for (int u = lane; u < units; u += 64) dst[u] = src[u];
        kreg = o + np;
    }

    // ---- phase A: unary codewords -> kept values in buf[kreg + j]
    const int64_t wstart = bo0 >> 5, wend = (bo1 + 31) >> 5;
    int jb = 0;
    int prev = -1;                               // last codeword end, relative to bo0
    for (int64_t wb = wstart; wb < wend; wb += 64) {
        const int64_t w = wb + lane;
        uint32_t word = w < wend ? a.unary[w] : 0u;
        const int64_t rel = w * 32 - bo0;        // stream position of bit 0 of this word, relative
        if (rel < 0) word &= ~0u << int(-rel);
        const int64_t lim = (bo1 - bo0) - rel;   // bits of this word inside the tile
        if (lim < 32) word &= lim <= 0 ? 0u : ((1u << int(lim)) - 1u);
        const int ones = __popc(word);
        const int incl = wave_incl_add(ones);
        const int total = __shfl(incl, 63, 64);
        const int last = ones ? int(rel) + 31 - __clz(word) : -1;
        const int lmax = wave_incl_max(last);
        int p = __shfl_up(lmax, 1, 64);
        if (lane == 0) p = -1;
        p = max(p, prev);
        int j = jb + incl - ones;
        NibWin sw, lw;
        sw.init(a.spec_nib, kp0 + j);
        if constexpr (RESTORE) lw.init(a.lo_nib, kp0 + j);
        while (word) {
            const int b = __ffs(word) - 1;
            const int pos = int(rel) + b;
            int rank = pos - p - 1;
            rank = min(rank, 255);
            const uint32_t E = cb[rank];
            const uint32_t sn = sw.next();
            uint32_t v = ((sn >> 3) << 15) | (E << 7) | ((sn & 7u) << 4);
            if constexpr (RESTORE) v |= lw.next();
            buf[kreg + j] = uint16_t(v);
            p = pos;
            ++j;
            word &= word - 1;
        }
        jb += total;
        prev = max(prev, __shfl(lmax, 63, 64));
    }
    wave_sync_lds();

    // ---- phase B: walk this lane's 64 bitmap bits
    const int cnt = __popc(bw0) + __popc(bw1);
    const int P = wave_incl_add(cnt) - cnt;
    const int kb = kreg + P;
    const int qb = o + 64 * lane - P;
    int ki = 0;
#pragma unroll
    for (int e = 0; e < 64; e += 2) {
        uint32_t v2 = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ee = e + h;
            const uint32_t bit = ((ee < 32 ? bw0 : bw1) >> (ee & 31)) & 1u;
            const uint32_t vk = buf[kb + ki];
            uint32_t v;
            if constexpr (RESTORE) {
                const uint32_t vp = buf[qb + ee - ki];
                v = bit ? vk : vp;
            } else {
                v = bit ? vk : 0u;
            }
            ki += int(bit);
            v2 |= v << (16 * h);
        }
        pairs[e >> 1] = v2;
    }
    (void)np;
}

// ------------------------------------------------------------------ draft GEMV, any shape

// Dense-walk fallback for K < 4096 or batches above 2.  Block = R consecutive rows
// (flat range [r0*K, (r0+R)*K)); its waves take the overlapping tiles round robin.
// Lane partials are reduced per (row, batch).
template <int BMAX, int R>
__global__ __launch_bounds__(256) void spec_gemv_kernel(CasArgs a, const uint16_t* __restrict__ x, int B,
                                                        float* __restrict__ y) {
    __shared__ __attribute__((aligned(16))) uint16_t bufs[4][ROW_STRIDE];
    __shared__ uint8_t cb[256];
    __shared__ float red[4][R][BMAX];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb[i] = i < a.n_sym ? a.codebook[i] : 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = lane_id(), nw = blockDim.x >> 6;
    const int64_t K = a.K;
    const int64_t r0 = int64_t(blockIdx.x) * R;
    const int64_t fa = r0 * K, fb = min<int64_t>(a.M, r0 + R) * K;
    const int64_t t0 = fa / TILE, t1 = (fb - 1) / TILE;
    float acc[R][BMAX];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[r][b] = 0.f;
    for (int64_t t = t0 + wave; t <= t1; t += nw) {
        const int tl = int(min<int64_t>(TILE, a.N - t * TILE));
        uint32_t pairs[32];
        decode_tile<false>(a, t, tl, bufs[wave], cb, pairs);
        const int64_t f = t * TILE + 64 * lane;
        if (f >= fa && f < fb) {
            const int64_t row = f / K;
            const int rr = int(row - r0);
            const int64_t col = f - row * K;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                if (b < B) {
                    const uint4* xs = reinterpret_cast<const uint4*>(x + b * K + col);
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint4 xv = xs[i];
                        s0 = dot2(pairs[4 * i], xv.x, s0);
                        s1 = dot2(pairs[4 * i + 1], xv.y, s1);
                        s0 = dot2(pairs[4 * i + 2], xv.z, s0);
                        s1 = dot2(pairs[4 * i + 3], xv.w, s1);
                    }
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        if (r == rr) acc[r][b] += s0 + s1;
                }
            }
        }
        wave_sync_lds();   // buffer reuse by the next tile of this wave
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            float v = acc[r][b];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][r][b] = v;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < R * BMAX; i += blockDim.x) {
        const int r = i / BMAX, b = i - r * BMAX;
        const int64_t row = r0 + r;
        if (b < B && row < a.M) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) s += red[w][r][b];
            y[b * a.M + row] = s;
        }
    }
}

// ------------------------------------------------------------------ kept-domain decode
//
// The decoders below give every lane of a wave an equal share of a tile's kept
// values (or of its pruned values) instead of an equal share of its positions,
// so no lane walks the 70% of positions it has nothing to do for:
//
//   * staging: the tile's unary words and bitmap words go to the wave's LDS area
//     with exclusive prefix counts of their one bits;
//   * start: a lane's first kept index j0 is located in the unary stream (end of
//     codeword j0 - 1) and in the bitmap (position of kept j0) by binary search
//     over those prefix counts and a select inside the word;
//   * walk: per kept value, the next one bit of the unary stream gives the rank
//     (zero run length), the next set bit of the bitmap gives the position, and
//     the spec nibble comes from a register window aligned once per 24 values.
//
// Tiles whose unary stream spans more than 128 words (over 4096 code bits, far
// above the ~2.9 bits per kept value of an entropy-ranked codebook) take the same
// walk with the words read from memory and a linear start search.

constexpr int STAGE_UW = 128;   // unary words staged per wave
// Tile flags from the staging (wave-uniform): a cursor's loop over empty words
// runs only in tiles that have such a word (codewords end within the next word and
// bitmap words hold both kinds of bit almost always).
constexpr uint32_t GAP_UNARY = 1;  // a unary word without a one bit, or the words are not staged
constexpr uint32_t GAP_EMPTY = 2;  // a bitmap word without a kept position
constexpr uint32_t GAP_FULL = 4;   // a bitmap word without a pruned position
constexpr int NIB_CHUNK = 32;   // kept values per aligned nibble window (128 bits)
constexpr int GRP = 4;          // kept values decoded before their LDS reads are issued
constexpr int PRU_CHUNK = 32;   // pruned values per aligned register window

struct WaveArea {
    uint32_t uw[STAGE_UW];      // unary words of the tile, bits outside it cleared
    uint32_t bw[TILE / 32];     // bitmap words of the tile
    uint16_t up[STAGE_UW];      // one bits before each unary word
    uint16_t bp[TILE / 64];     // kept values before each 64-position pair of words
};

struct TileHdr {
    int64_t f0;      // first flat element
    int64_t kp0;     // kept values before the tile
    int64_t bo0, bo1;  // unary bit range
    int64_t ws;      // first unary word touched
    int tl;          // elements in the tile
    int nk;          // kept values in the tile
    int nuw;         // unary words touched
};

__device__ __forceinline__ TileHdr tile_hdr(const CasArgs& a, int64_t t) {
    TileHdr h;
    h.f0 = t * TILE;
    h.tl = int(min<int64_t>(TILE, a.N - h.f0));
    h.kp0 = a.kprefix[t];
    h.nk = int(int64_t(a.kprefix[t + 1]) - h.kp0);
    h.bo0 = int64_t(a.bitoff[t]);
    h.bo1 = int64_t(a.bitoff[t + 1]);
    h.ws = h.bo0 >> 5;
    h.nuw = int(((h.bo1 + 31) >> 5) - h.ws);
    return h;
}

// Word k of the tile's unary window with the bits of neighbouring tiles cleared.
__device__ __forceinline__ uint32_t unary_word(const CasArgs& a, const TileHdr& h, int k) {
    const int64_t w = h.ws + k;
    uint32_t v = a.unary[w];
    const int64_t b0 = w * 32;
    if (b0 < h.bo0) v &= ~0u << int(h.bo0 - b0);
    const int64_t lim = h.bo1 - b0;
    if (lim < 32) v &= lim <= 0 ? 0u : ((1u << int(lim)) - 1u);
    return v;
}

// Position of the r-th (from 0) set bit of w; w has more than r set bits.
__device__ __forceinline__ int select32(uint32_t w, int r) {
    int pos = 0;
#pragma unroll
    for (int half = 16; half; half >>= 1) {
        const int c = __popc(w & ((1u << half) - 1u));
        if (r >= c) {
            r -= c;
            w >>= half;
            pos += half;
        }
    }
    return pos;
}

// Cursor over the tile's unary codewords.  GAPS: the tile may hold a staged word
// without a one bit (a codeword longer than 32 bits), so a refill may loop.
template <bool FAST, bool GAPS = true>
struct UnaryCursor {
    int k;          // current word
    uint32_t cw;    // its unconsumed bits
    int q;          // position of the last one bit consumed (window relative)
    uint32_t nx;    // FAST: word k + 1, read one refill ahead
    __device__ __forceinline__ uint32_t word(const CasArgs& a, const TileHdr& h, const WaveArea& W, int i) const {
        if constexpr (FAST) return W.uw[i];
        else return unary_word(a, h, i);
    }
    // position at codeword j0 (the first j0 codewords consumed)
    __device__ __forceinline__ void start(const CasArgs& a, const TileHdr& h, const WaveArea& W, int j0) {
        const int target = j0 - 1;      // the one bit that ends codeword j0 - 1
        int kk = 0, base = 0;
        if (j0 > 0) {
            if constexpr (FAST) {
#pragma unroll
                for (int s = 64; s; s >>= 1)
                    if (kk + s < h.nuw && int(W.up[kk + s]) <= target) kk += s;
                base = W.up[kk];
            } else {
                for (;;) {
                    const int c = __popc(word(a, h, W, kk));
                    if (base + c > target) break;
                    base += c;
                    ++kk;
                }
            }
        }
        const uint32_t w = word(a, h, W, kk);
        const int b = j0 > 0 ? select32(w, target - base) : int(h.bo0 & 31) - 1;
        k = kk;
        q = 32 * kk + b;
        cw = j0 > 0 ? w & ~((2u << b) - 1u) : w;
        if constexpr (FAST) nx = W.uw[k + 1];
    }
    // rank of the next codeword
    __device__ __forceinline__ int next(const CasArgs& a, const TileHdr& h, const WaveArea& W) {
        if constexpr (FAST) {
            // branch-free refill from the word read ahead; a further empty word
            // (a codeword longer than 32 bits) takes the loop, in tiles flagged at
            // staging only
            const bool e = cw == 0;
            cw = e ? nx : cw;
            k += e;
            if constexpr (GAPS)
                while (cw == 0) cw = word(a, h, W, ++k);
            nx = W.uw[k + 1];
        } else {
            while (cw == 0) cw = word(a, h, W, ++k);
        }
        const int pos = 32 * k + __builtin_ctz(cw);
        const int rank = pos - q - 1;
        q = pos;
        cw &= cw - 1u;
        return rank;
    }
};

// Cursor over set bits (kept positions) or clear bits (pruned positions) of the
// tile's bitmap.  GAPS: the tile may hold a word without a bit of the walked kind.
template <bool ZEROS, bool GAPS = true>
struct BitCursor {
    int k;
    uint32_t cw;
    uint32_t nx;    // word k + 1, read one refill ahead
    __device__ __forceinline__ uint32_t word(const WaveArea& W, int i) const {
        return ZEROS ? ~W.bw[i] : W.bw[i];
    }
    // position at the j0-th (from 0) set (or clear) bit
    __device__ __forceinline__ void start(const WaveArea& W, int j0) {
        int p = 0;
#pragma unroll
        for (int s = 32; s; s >>= 1) {
            const int c = ZEROS ? 64 * (p + s) - int(W.bp[p + s]) : int(W.bp[p + s]);
            if (c <= j0) p += s;
        }
        int r = j0 - (ZEROS ? 64 * p - int(W.bp[p]) : int(W.bp[p]));
        uint32_t w = word(W, 2 * p);
        k = 2 * p;
        const int c = __popc(w);
        if (r >= c) {
            r -= c;
            k = 2 * p + 1;
            w = word(W, k);
        }
        cw = w & (~0u << select32(w, r));
        nx = word(W, k + 1);
    }
    __device__ __forceinline__ int next(const WaveArea& W) {
        const bool e = cw == 0;              // branch-free refill; a further empty word loops
        cw = e ? nx : cw;
        k += e;
        if constexpr (GAPS)
            while (cw == 0) cw = word(W, ++k);
        nx = word(W, k + 1);
        const int pos = 32 * k + __builtin_ctz(cw);
        cw &= cw - 1u;
        return pos;
    }
};

// Nibble windows: the 5 words holding nibbles [n, n + 32) of a packed stream,
// loaded early, then funnel-shifted so that nibble n + i sits at bits 4i.
__device__ __forceinline__ void nib_load(const uint32_t* __restrict__ s, int64_t n, uint32_t (&raw)[5]) {
    const uint32_t* p = s + (n >> 3);
#pragma unroll
    for (int i = 0; i < 5; ++i) raw[i] = p[i];
}

__device__ __forceinline__ void nib_align(const uint32_t (&raw)[5], int64_t n, uint32_t (&win)[4]) {
    const uint32_t sh = uint32_t(4 * (n & 7));
#pragma unroll
    for (int i = 0; i < 4; ++i) win[i] = __builtin_amdgcn_alignbit(raw[i + 1], raw[i], sh);
}

// Walk kept values [j0, j0 + cnt) of the tile in kept order, GRP at a time:
// sink.stage(u, rank, spec_nib, lo_nib) for each value of the group (u = its
// slot), sink.skip(u) for slots past the lane's count, then sink.commit().  The
// first nibble windows (nibble kp0 + j0) come preloaded.
template <bool FAST, bool LO, bool GAPS, class Sink>
__device__ __forceinline__ void walk_kept(const CasArgs& a, const TileHdr& h, const WaveArea& W, int j0, int cnt,
                                          const uint32_t (&sraw)[5], const uint32_t (&lraw)[5], Sink& sink) {
    if (cnt <= 0) return;
    UnaryCursor<FAST, GAPS> uc;
    uc.start(a, h, W, j0);
    uint32_t sw[4], lw[4];
    const int64_t n0 = h.kp0 + j0;
    nib_align(sraw, n0, sw);
    if constexpr (LO) nib_align(lraw, n0, lw);
    for (int base = 0; base < cnt; base += NIB_CHUNK) {
        if (base > 0) {
            uint32_t r[5];
            nib_load(a.spec_nib, n0 + base, r);
            nib_align(r, n0 + base, sw);
            if constexpr (LO) {
                nib_load(a.lo_nib, n0 + base, r);
                nib_align(r, n0 + base, lw);
            }
        }
        const int rem = cnt - base;
#pragma unroll
        for (int g = 0; g < NIB_CHUNK / GRP; ++g) {
            if (GRP * g < rem) {
#pragma unroll
                for (int u = 0; u < GRP; ++u) {
                    const int i = GRP * g + u;
                    if constexpr (FAST && !GAPS && Sink::kDrop) {
                        // loop-free cursors: a lane past its share (at most GRP - 1
                        // steps, the group guard stops it) steps on, at most one
                        // word a step inside its staging area, and drops the slot
                        const int rank = uc.next(a, h, W);
                        sink.stage(u, rank, (sw[i / 8] >> (4 * (i % 8))) & 15u,
                                   LO ? (lw[i / 8] >> (4 * (i % 8))) & 15u : 0u);
                        sink.drop(u, i >= rem);
                    } else if (i < rem) {
                        const int rank = uc.next(a, h, W);
                        sink.stage(u, rank, (sw[i / 8] >> (4 * (i % 8))) & 15u,
                                   LO ? (lw[i / 8] >> (4 * (i % 8))) & 15u : 0u);
                    } else {
                        sink.skip(u);
                    }
                }
                sink.commit();
            }
        }
    }
}

// Even share of n items over the 64 lanes: [first, first + count).
__device__ __forceinline__ void lane_share(int n, int lanes, int l, int& first, int& count) {
    const int c = (n + lanes - 1) / lanes;
    first = l * c;
    count = max(0, min(c, n - first));
}

// Pruned values [p0, p0 + cnt) of the tile (raw bf16), PRU_CHUNK at a time:
// emit(pos, value).  The first chunk's words come preloaded (pru_load at e0);
// each later chunk's are loaded while the one before is walked.
constexpr int PRU_WORDS = PRU_CHUNK / 2 + 1;

// 16 of the 17 words come in four 16-byte loads: global multi-dword loads need
// only dword alignment, and one wide load per lane touches far fewer cache lines
// per instruction than 16 single-word loads at the lanes' strides.
typedef uint32_t u32x4_dw_t __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ void pru_load(const CasArgs& a, int64_t e, uint32_t (&raw)[PRU_WORDS]) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.pruned) + (e >> 1);
    static_assert(PRU_WORDS == 17, "four 16-byte loads and one word");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4_dw_t v = *reinterpret_cast<const u32x4_dw_t*>(src + 4 * i);
        raw[4 * i] = v.x; raw[4 * i + 1] = v.y; raw[4 * i + 2] = v.z; raw[4 * i + 3] = v.w;
    }
    raw[16] = src[16];
}

template <bool GAPS, class Emit>
__device__ __forceinline__ void walk_pruned(const CasArgs& a, const TileHdr& h, const WaveArea& W, int p0, int cnt,
                                            const uint32_t (&raw0)[PRU_WORDS], Emit&& emit) {
    if (cnt <= 0) return;
    BitCursor<true, GAPS> zc;
    zc.start(W, p0);
    const int64_t e0 = (h.f0 - h.kp0) + p0;          // pruned stream index of the first value
    uint32_t raw[PRU_WORDS], nxt[PRU_WORDS];
#pragma unroll
    for (int i = 0; i < PRU_WORDS; ++i) raw[i] = raw0[i];
    for (int base = 0; base < cnt; base += PRU_CHUNK) {
        const int64_t e = e0 + base;
        if (base > 0) {
#pragma unroll
            for (int i = 0; i < PRU_WORDS; ++i) raw[i] = nxt[i];
        }
        // the next chunk's words load while this one is walked
        if (base + PRU_CHUNK < cnt) pru_load(a, e + PRU_CHUNK, nxt);
        const uint32_t sh = uint32_t(16 * (e & 1));
        uint32_t v[PRU_CHUNK / 2];
#pragma unroll
        for (int i = 0; i < PRU_CHUNK / 2; ++i) v[i] = __builtin_amdgcn_alignbit(raw[i + 1], raw[i], sh);
        const int rem = cnt - base;
#pragma unroll
        for (int i = 0; i < PRU_CHUNK; ++i) {
            if (i < rem) {
                const int pos = zc.next(W);
                emit(pos, (v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
            }
        }
    }
}

// bf16 bits of a kept value from its codebook exponent and nibbles.
__device__ __forceinline__ uint32_t kept_bits(uint32_t E, uint32_t sn, uint32_t lo) {
    return ((sn & 8u) << 12) | (E << 7) | ((sn & 7u) << 4) | lo;
}

// ---- software pipeline: a tile's global loads are issued one tile ahead.

// Tile-table entries of up to 64 tiles, lane i holding those of the i-th.
struct HdrVec {
    uint32_t kp0, kp1;
    uint64_t bo0, bo1;
};

__device__ __forceinline__ HdrVec hdr_load(const CasArgs& a, int64_t t) {
    HdrVec v;
    v.kp0 = a.kprefix[t];
    v.kp1 = a.kprefix[t + 1];
    v.bo0 = a.bitoff[t];
    v.bo1 = a.bitoff[t + 1];
    return v;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int i) {
    const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), i);
    const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(v >> 32), i);
    return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ TileHdr hdr_get(const CasArgs& a, const HdrVec& v, int i, int64_t t) {
    TileHdr h;
    h.f0 = t * TILE;
    h.tl = int(min<int64_t>(TILE, a.N - h.f0));
    h.kp0 = __builtin_amdgcn_readlane(v.kp0, i);
    h.nk = int(__builtin_amdgcn_readlane(v.kp1, i) - uint32_t(h.kp0));
    h.bo0 = int64_t(readlane64(v.bo0, i));
    h.bo1 = int64_t(readlane64(v.bo1, i));
    h.ws = h.bo0 >> 5;
    h.nuw = int(((h.bo1 + 31) >> 5) - h.ws);
    return h;
}

// A tile's header and the raw words its lanes need first.  Every load is
// unconditional (indices clamped), so the number in flight is static.
struct TileWords {
    TileHdr h;
    int64_t t;
    int j0, cnt;
    uint32_t u0, u1, b0, b1;
    uint32_t sraw[5];
};

__device__ __forceinline__ void tile_issue(const CasArgs& a, const TileHdr& h, int64_t t, TileWords& tw) {
    const int lane = lane_id();
    tw.h = h;
    tw.t = t;
    lane_share(h.nk, 64, lane, tw.j0, tw.cnt);
    nib_load(a.spec_nib, h.kp0 + tw.j0, tw.sraw);
    const int64_t ulast = max<int64_t>(0, h.ws + h.nuw - 1);
    tw.u0 = a.unary[min<int64_t>(h.ws + lane, ulast)];
    tw.u1 = a.unary[min<int64_t>(h.ws + 64 + lane, ulast)];
    const int64_t nwords = (a.N + 31) >> 5;
    const int64_t wi = t * (TILE / 32) + 2 * lane;
    tw.b0 = a.bitmap[min<int64_t>(wi, nwords - 1)];
    tw.b1 = a.bitmap[min<int64_t>(wi + 1, nwords - 1)];
}

// Stage the tile's bitmap (and, when it fits, its unary words) with prefix
// counts, from the words tile_issue loaded.
__device__ __forceinline__ uint32_t tile_stage(const CasArgs& a, const TileWords& tw, WaveArea& W) {
    const int lane = lane_id();
    const TileHdr& h = tw.h;
    uint32_t gaps = GAP_UNARY;
    if (h.nuw <= STAGE_UW) {
        auto mask = [&](uint32_t v, int k) {
            const int64_t b0 = (h.ws + k) * 32;
            if (b0 < h.bo0) v &= ~0u << int(h.bo0 - b0);
            const int64_t lim = h.bo1 - b0;
            if (lim < 32) v &= lim <= 0 ? 0u : ((1u << int(lim)) - 1u);
            return v;
        };
        const uint32_t u0 = lane < h.nuw ? mask(tw.u0, lane) : 0u;
        const uint32_t u1 = lane + 64 < h.nuw ? mask(tw.u1, lane + 64) : 0u;
        const int c0 = __popc(u0), c1 = __popc(u1);
        const int inc = wave_incl_add(c0 | (c1 << 16));
        const int tot0 = __shfl(inc, 63, 64) & 0xFFFF;
        W.uw[lane] = u0;
        W.uw[lane + 64] = u1;
        const bool zu = (lane < h.nuw && u0 == 0u) || (lane + 64 < h.nuw && u1 == 0u);
        gaps = __ballot(zu) ? GAP_UNARY : 0u;
        W.up[lane] = uint16_t((inc & 0xFFFF) - c0);
        W.up[lane + 64] = uint16_t(tot0 + (inc >> 16) - c1);
    }
    const int64_t wi = tw.t * (TILE / 32) + 2 * lane;
    const int64_t nwords = (a.N + 31) >> 5;
    const uint32_t b0 = wi < nwords ? tw.b0 : 0u;
    const uint32_t b1 = wi + 1 < nwords ? tw.b1 : 0u;
    W.bw[2 * lane] = b0;
    W.bw[2 * lane + 1] = b1;
    const int pc = __popc(b0) + __popc(b1);
    W.bp[lane] = uint16_t(wave_incl_add(pc) - pc);
    if (__ballot(b0 == 0u || b1 == 0u)) gaps |= GAP_EMPTY;
    if (__ballot(b0 == ~0u || b1 == ~0u)) gaps |= GAP_FULL;
    wave_sync_lds();
    return gaps;
}

// ------------------------------------------------------------------ sinks

// Kept values scattered as bf16 bits into an LDS tile.
template <bool GAPS>
struct ScatterSink {
    static constexpr bool kDrop = true;     // the walk may stage past the share and drop (measured faster)
    BitCursor<false, GAPS> kc;
    const WaveArea* W;
    const uint8_t* cb;
    uint16_t* d;
    int pos[GRP], rk[GRP];
    uint32_t nib[GRP];
    __device__ __forceinline__ void stage(int u, int rank, uint32_t sn, uint32_t lo) {
        pos[u] = kc.next(*W);
        rk[u] = min(rank, 255);
        nib[u] = sn | (lo << 4);
    }
    __device__ __forceinline__ void skip(int u) {
        pos[u] = -1;
        rk[u] = 0;
        nib[u] = 0;
    }
    // a staged slot past the lane's share: nothing is written
    __device__ __forceinline__ void drop(int u, bool past) {
        pos[u] = past ? -1 : pos[u];
        rk[u] = past ? 0 : rk[u];
    }
    __device__ __forceinline__ void commit() {
        uint32_t E[GRP];
#pragma unroll
        for (int u = 0; u < GRP; ++u) E[u] = cb[rk[u]];
#pragma unroll
        for (int u = 0; u < GRP; ++u)
            if (pos[u] >= 0) d[pos[u]] = uint16_t(kept_bits(E[u], nib[u] & 15u, nib[u] >> 4));
    }
};

// Kept values times activations (batch 1 or 2), into one accumulator per row, or,
// when the tile meets two rows (SPLIT), kept index < jb into accA and the rest
// into accB.  Slots past the lane's count read the LUT's zero entry.
template <int BMAX, bool SPLIT, bool GAPS>
struct DotSink {
    static constexpr bool kDrop = false;    // guarded per value (staging past the share measured slower)
    BitCursor<false, GAPS> kc;
    const WaveArea* W;
    const float* lut;
    const uint16_t* xs;
    int K, colbase, nlast, zero, j, jb;
    int idx[GRP], col[GRP];
    bool inA[GRP];
    float accA[BMAX], accB[BMAX];
    __device__ __forceinline__ void stage(int u, int rank, uint32_t sn, uint32_t) {
        // activation column: position in the tile relative to the start of its row
        col[u] = colbase + kc.next(*W);
        if constexpr (SPLIT) {
            inA[u] = j < jb;
            if (!inA[u]) col[u] -= K;
        }
        idx[u] = (min(rank, nlast) << 4) | int(sn);
        ++j;
    }
    __device__ __forceinline__ void skip(int u) {
        col[u] = 0;
        idx[u] = zero;
        if constexpr (SPLIT) inA[u] = true;
        ++j;
    }
    // a staged slot past the lane's share: weight 0.0 times a real activation
    __device__ __forceinline__ void drop(int u, bool past) {
        col[u] = past ? 0 : col[u];
        idx[u] = past ? zero : idx[u];
    }
    __device__ __forceinline__ void commit() {
        float w[GRP], xv[GRP][BMAX];
#pragma unroll
        for (int u = 0; u < GRP; ++u) {
            w[u] = lut[idx[u]];
#pragma unroll
            for (int b = 0; b < BMAX; ++b) xv[u][b] = __uint_as_float(uint32_t(xs[b * K + col[u]]) << 16);
        }
#pragma unroll
        for (int u = 0; u < GRP; ++u)
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                if constexpr (SPLIT) {
                    const float pA = fmaf(w[u], xv[u][b], accA[b]), pB = fmaf(w[u], xv[u][b], accB[b]);
                    accA[b] = inA[u] ? pA : accA[b];
                    accB[b] = inA[u] ? accB[b] : pB;
                } else {
                    accA[b] = fmaf(w[u], xv[u][b], accA[b]);
                }
            }
    }
};

// ------------------------------------------------------------------ dense decode

constexpr int DD_WAVES = 4;

// Restore (RESTORE) or draft decode of a tile whose header, bitmap and unary
// words and first spec nibble window were loaded ahead by tile_issue (the verify
// GEMM issues the next tile's loads before its MFMA phase).  The draft decode
// scatters kept values only: pruned positions keep what the tile held.
template <bool RESTORE = true>
__device__ __forceinline__ void decode_tile_issued(const CasArgs& a, const TileWords& tw, WaveArea& W,
                                                   const uint8_t* cb, uint16_t* d) {
    const TileHdr& h = tw.h;
    uint32_t lraw[5];
    if constexpr (RESTORE) nib_load(a.lo_nib, h.kp0 + tw.j0, lraw);
    // a tile without empty words (nearly all) takes the walks without their loops
    // over empty words; the flag is wave-uniform
    const uint32_t gaps = tile_stage(a, tw, W);
    auto body = [&](auto g) __attribute__((always_inline)) {
        constexpr bool G = decltype(g)::value;
        ScatterSink<G> sk;
        sk.W = &W;
        sk.cb = cb;
        sk.d = d;
        if (tw.cnt > 0) sk.kc.start(W, tw.j0);
        if (h.nuw <= STAGE_UW) walk_kept<true, RESTORE, G>(a, h, W, tw.j0, tw.cnt, tw.sraw, lraw, sk);
        else walk_kept<false, RESTORE, G>(a, h, W, tw.j0, tw.cnt, tw.sraw, lraw, sk);
        if constexpr (RESTORE) {
            int p0, pc;
            lane_share(h.tl - h.nk, 64, lane_id(), p0, pc);
            uint32_t praw[PRU_WORDS];
            pru_load(a, (h.f0 - h.kp0) + p0, praw);
            walk_pruned<G>(a, h, W, p0, pc, praw, [&](int pos, uint32_t v) { d[pos] = uint16_t(v); });
        }
    };
    if (gaps) body(std::true_type{});
    else body(std::false_type{});
}

// Kept values (and, when restoring, pruned values) of a tile are scattered into
// the wave's LDS tile, then written out 16 bytes a lane; a wave takes two tiles.
template <bool RESTORE>
__global__ __launch_bounds__(64 * DD_WAVES) void decode_dense_kernel(CasArgs a, uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t dense[DD_WAVES][TILE];
    __shared__ WaveArea areas[DD_WAVES];
    __shared__ uint8_t cb[256];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb[i] = i < a.n_sym ? a.codebook[i] : 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = lane_id();
    uint16_t* d = dense[wave];
    auto write_out = [&](int64_t t) {
        wave_sync_lds();
        const int tl = int(min<int64_t>(TILE, a.N - t * TILE));
        uint4* o = reinterpret_cast<uint4*>(out + t * TILE);
        for (int g = lane; g < tl / 8; g += 64) o[g] = *reinterpret_cast<const uint4*>(d + 8 * g);
    };
    // two tiles per wave, DD_WAVES apart: both tiles' header, bitmap, unary and
    // first nibble words are issued up front, so the second tile's arrive while
    // the first is decoded (more tiles per wave measured slower)
    auto clear = [&]() {
        if constexpr (!RESTORE) {
            uint4* d4 = reinterpret_cast<uint4*>(d) + lane;       // pruned positions read +0.0
#pragma unroll
            for (int i = 0; i < 8; ++i) d4[64 * i] = make_uint4(0, 0, 0, 0);   // lane-contiguous: no bank conflicts
        }
    };
    const int64_t t0 = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 2 * DD_WAVES + wave);
    const int64_t t1 = t0 + DD_WAVES;
    if (t0 >= a.T) return;
    TileWords w0, w1;
    tile_issue(a, tile_hdr(a, t0), t0, w0);
    const int64_t t1c = min<int64_t>(t1, a.T - 1);
    tile_issue(a, tile_hdr(a, t1c), t1c, w1);
    clear();
    decode_tile_issued<RESTORE>(a, w0, areas[wave], cb, d);
    write_out(t0);
    if (t1 >= a.T) return;
    wave_sync_lds();                                        // the tile is read out before it is overwritten
    clear();
    decode_tile_issued<RESTORE>(a, w1, areas[wave], cb, d);
    write_out(t1);
}

// ------------------------------------------------------------------ draft GEMV (kept domain)

// Block = R consecutive rows, NW waves taking the overlapping tiles round robin.
// Needs K >= 4096 (a tile meets at most two rows).  Lanes share the tile's kept
// values evenly; a lane whose values straddle the row boundary keeps two sums.
// The two row sums are reduced across the wave and added to the wave's own
// partial row sums in LDS, which are summed in wave order at the end.
template <int BMAX>
__global__ __launch_bounds__(1024) void spec_gemv_kept_kernel(CasArgs a, const uint16_t* __restrict__ x, int B,
                                                              float* __restrict__ y, int R) {
    extern __shared__ __attribute__((aligned(16))) uint4 sl4[];
    const int nw = blockDim.x >> 6, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = int(a.K);
    const int nsym = max(1, a.n_sym), nlut = nsym * 16;                  // entry nlut holds 0.0
    uint16_t* xs = reinterpret_cast<uint16_t*>(sl4);                     // [BMAX][K]
    WaveArea* areas = reinterpret_cast<WaveArea*>(xs + BMAX * K);        // [nw]
    float* red = reinterpret_cast<float*>(areas + nw);                   // [nw][R][BMAX]
    float* lutf = red + nw * R * BMAX;                                   // [nsym][16] + zero
    for (int i = threadIdx.x; i <= nlut; i += blockDim.x) {
        const int rank = i >> 4;
        const uint32_t E = rank < a.n_sym ? a.codebook[rank] : 0u;
        lutf[i] = i == nlut ? 0.f : __uint_as_float(kept_bits(E, uint32_t(i & 15), 0u) << 16);
    }
    for (int i = threadIdx.x; i < B * K / 8; i += blockDim.x)
        reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
    for (int i = threadIdx.x; i < nw * R * BMAX; i += blockDim.x) red[i] = 0.f;
    __syncthreads();
    const int64_t r0 = int64_t(blockIdx.x) * R, r1 = min<int64_t>(a.M, r0 + R);
    const int64_t t_a = (r0 * K) / TILE, t_b = (r1 * K - 1) / TILE;
    WaveArea& W = areas[wave];
    float* wred = red + wave * R * BMAX;
    const int64_t tw0 = t_a + wave;
    const int ntiles = t_b >= tw0 ? int((t_b - tw0) / nw) + 1 : 0;
    HdrVec hv;
    // loads of tile i (clamped to the last tile) into dst
    // (tile-table entries of the wave's first 64 tiles sit in hv; later ones, only
    // for rows longer than 64 * 16 tiles, come through scalar loads)
    auto issue_at = [&](int i, TileWords& dst) {
        i = min(i, ntiles - 1);
        const int64_t tn = tw0 + int64_t(i) * nw;
        tile_issue(a, i < 64 ? hdr_get(a, hv, i, tn) : tile_hdr(a, tn), tn, dst);
    };
    // inlined: as a call, the tile buffers would pass through the stack
    auto process = [&](const TileWords& cur) __attribute__((always_inline)) {
        const TileHdr h = cur.h;
        const int j0 = cur.j0, cnt = cur.cnt;
        const uint32_t gaps = tile_stage(a, cur, W);
        const int64_t row_a = h.f0 / K;
        const int bnd = int(min<int64_t>(h.tl, (row_a + 1) * K - h.f0));   // first position of the next row
        int jb = h.nk;                                                      // kept values before bnd
        if (bnd < h.tl) {
            const int p = bnd >> 6, rem = bnd & 63;
            const uint32_t lo = W.bw[2 * p], hi = W.bw[2 * p + 1];
            jb = int(W.bp[p]) + (rem >= 32 ? __popc(lo) + __popc(hi & ((1u << (rem - 32)) - 1u))
                                            : __popc(lo & ((1u << rem) - 1u)));
        }
        float vA[BMAX], vB[BMAX];
        auto run = [&](auto split, auto g) {
            constexpr bool SPLIT = decltype(split)::value, G = decltype(g)::value;
            DotSink<BMAX, SPLIT, G> sk;
            sk.W = &W;
            sk.lut = lutf;
            sk.xs = xs;
            sk.K = K;
            sk.colbase = int(h.f0 - row_a * K);
            sk.nlast = nsym - 1;
            sk.zero = nlut;
            sk.j = j0;
            sk.jb = jb;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) sk.accA[b] = sk.accB[b] = 0.f;
            if (cnt > 0) sk.kc.start(W, j0);
            uint32_t none[5];
            if (h.nuw <= STAGE_UW) walk_kept<true, false, G>(a, h, W, j0, cnt, cur.sraw, none, sk);
            else walk_kept<false, false, G>(a, h, W, j0, cnt, cur.sraw, none, sk);
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                vA[b] = sk.accA[b];
                vB[b] = SPLIT ? sk.accB[b] : 0.f;
            }
        };
        // a tile without empty words (nearly all) takes the walk without its loops
        // over empty words; the flag is wave-uniform
        if (gaps) {
            if (bnd < h.tl) run(std::true_type{}, std::true_type{});
            else run(std::false_type{}, std::true_type{});
        } else {
            if (bnd < h.tl) run(std::true_type{}, std::false_type{});
            else run(std::false_type{}, std::false_type{});
        }
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                vA[b] += __shfl_xor(vA[b], off, 64);
                vB[b] += __shfl_xor(vB[b], off, 64);
            }
            if (lane == 0) {
                if (row_a >= r0 && row_a < r1) wred[int(row_a - r0) * BMAX + b] += vA[b];
                if (bnd < h.tl && row_a + 1 >= r0 && row_a + 1 < r1) wred[int(row_a + 1 - r0) * BMAX + b] += vB[b];
            }
        }
    };
    // two tile buffers, so a buffer is never copied while its loads are in flight
    TileWords ta, tb;
    if (ntiles > 0) {
        hv = hdr_load(a, tw0 + int64_t(min(lane, ntiles - 1)) * nw);
        issue_at(0, ta);
    }
    for (int it = 0; it < ntiles; it += 2) {
        issue_at(it + 1, tb);
        process(ta);
        issue_at(it + 2, ta);
        if (it + 1 < ntiles) process(tb);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * BMAX; i += blockDim.x) {
        const int r = i / BMAX, b = i - r * BMAX;
        if (b < B && r0 + r < r1) {
            float s = 0.f;
            for (int w = 0; w < nw; ++w) s += red[(w * R + r) * BMAX + b];
            y[int64_t(b) * a.M + r0 + r] = s;
        }
    }
}

// ------------------------------------------------------------------ verify GEMM (fused restore + MFMA)

// Block = 16 rows x all K (K % 4096 == 0), one wave per row.  Per 4096-column
// slab each wave restores its row's tile straight into the block's LDS rows
// (kept and pruned values scattered to their positions), then the 16 waves split
// the slab's 128 MFMA k-steps; the waves' partial 16x16 tiles are summed at the end.
constexpr int VG_WAVES = 16;
constexpr int VROW = 4104;   // u16 per LDS row: 2052 dwords, 4 (mod 32) banks apart

__global__ __launch_bounds__(64 * VG_WAVES) void verify_gemm_kernel(CasArgs a, const uint16_t* __restrict__ x, int B,
                                                                   float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint4 vl4[];
    uint16_t* rows = reinterpret_cast<uint16_t*>(vl4);                        // [16][VROW]
    WaveArea* areas = reinterpret_cast<WaveArea*>(rows + 16 * VROW);          // [VG_WAVES]
    uint8_t* cb = reinterpret_cast<uint8_t*>(areas + VG_WAVES);               // [256]
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb[i] = i < a.n_sym ? a.codebook[i] : 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int64_t K = a.K, tpr = K / TILE;
    const int64_t r0 = int64_t(blockIdx.x) * 16, row = r0 + wave;
    const int n = lane & 15, kq = lane >> 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // the next tile's words load during this tile's MFMA phase
    TileWords tw;
    const bool live = row < a.M;                     // rows past M are not decoded
    if (live) tile_issue(a, tile_hdr(a, row * tpr), row * tpr, tw);
    for (int64_t kt = 0; kt < tpr; ++kt) {
        // this wave's activations for its 8 k-steps, loaded ahead of the decode
        uint4 bv[8];
        const uint16_t* xrow = x + int64_t(n) * K + kt * TILE;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = (wave * 8 + s) * 32 + kq * 8;
            bv[s] = n < B ? *reinterpret_cast<const uint4*>(xrow + k) : make_uint4(0, 0, 0, 0);
        }
        // rows past M are not decoded: the outputs they feed are never stored
        if (live) {
            decode_tile_issued(a, tw, areas[wave], cb, rows + wave * VROW);
            const int64_t tn = row * tpr + min<int64_t>(kt + 1, tpr - 1);
            tile_issue(a, tile_hdr(a, tn), tn, tw);
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int k = (wave * 8 + s) * 32 + kq * 8;
            const uint4 av = *reinterpret_cast<const uint4*>(rows + n * VROW + k);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                          __builtin_bit_cast(bf16x8_t, bv[s]), acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // C[row = 4*kq + j][col = n] of this wave's partial
    float* red = reinterpret_cast<float*>(vl4);
    float* rw = red + (wave * 64 + lane) * 4;
    rw[0] = acc[0]; rw[1] = acc[1]; rw[2] = acc[2]; rw[3] = acc[3];
    __syncthreads();
    if (wave == 0) {
        float s[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < VG_WAVES; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] += red[(w * 64 + lane) * 4 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = r0 + 4 * kq + j;
            if (n < B && r < a.M) y[int64_t(n) * a.M + r] = s[j];
        }
    }
}

// ------------------------------------------------------------------ MX-32 GEMM

struct MxArgs {
    const uint8_t* exp;
    const uint32_t* sign;
    const uint8_t* mag;
    int64_t M, K;
};

// Eight MX elements (bytes of m8, sign bits sgn8 bit i = element i) -> bf16x8
// holding (-1)^s * mag * 2^(X-134): the product of an 8-bit integer and a power of
// two is exact in fp32 and keeps at most 8 significant bits, so its top 16 bits
// are the exact bf16.
__device__ __forceinline__ uint4 mx_to_bf16x8(uint2 m8, float scale, uint32_t sgn8) {
    uint32_t out[4];
    const uint32_t mw[2] = {m8.x, m8.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = mw[i >> 1];
        const int b0 = (i & 1) * 2;
        const float f0 = float((w >> (8 * b0)) & 0xFFu) * scale;
        const float f1 = float((w >> (8 * (b0 + 1))) & 0xFFu) * scale;
        // sign bits 2i, 2i+1 -> bits 15, 31 of the packed pair
        const uint32_t s2 = (sgn8 >> (2 * i)) & 3u;
        const uint32_t sm = ((s2 << 15) | (s2 << 30)) & 0x80008000u;
        out[i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u) | sm;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Block = 32 rows (two 16-row MFMA tiles) x all K, one block per CU.  K is
// walked in rounds of MX_SLAB columns, one 128-column chunk per wave: chunk c by
// wave c % MX_WAVES.  In a chunk, lane (n, q) = (lane % 16, lane / 16) holds the
// 32-element MX group q of row n of each tile (32 bytes of magnitudes, its
// exponent and sign word); the MFMA k slots of sub-step s take the group's
// elements 8s..8s+7, and batch row n's same 32 columns come from LDS.  The
// block stages each round's activation slab (all 16 batch rows) in LDS with
// lane-contiguous 16-byte loads, double-buffered: read by each wave straight
// from global memory, every activation load touched 32 cache lines for 1 KB and
// cost as much time as the weights.  The next round's weights and slab are
// loaded while the current chunk is computed.  Partial tiles are summed across
// the waves at the end.
constexpr int MX_WAVES = 16;
constexpr int MX_SLAB = MX_WAVES * 128;             // activation columns per round
constexpr int MX_XROW = MX_SLAB + 8;                // u16 per staged row: rows 4 banks apart
constexpr size_t MX_LDS = size_t(2) * 16 * MX_XROW * 2;
static_assert(MX_SLAB / 8 * 16 == 4 * 64 * MX_WAVES, "a slab is four 16-byte pieces per thread");
static_assert(MX_LDS >= sizeof(float) * MX_WAVES * 2 * 64 * 4, "the partial tiles reuse the slab buffers");

struct MxChunk {
    uint4 ma0, ma1, mb0, mb1;   // magnitudes, tiles A and B
    uint32_t ea, eb, sa, sb;    // exponents, sign words
};

__global__ __launch_bounds__(64 * MX_WAVES) void mx_gemm_kernel(MxArgs a, const uint16_t* __restrict__ x, int B,
                                                               float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint4 mxl4[];
    uint16_t* xs = reinterpret_cast<uint16_t*>(mxl4);           // [2][16][MX_XROW]
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int n = lane & 15, q = lane >> 4;
    const int64_t K = a.K, G = K / 32;
    const int64_t r0 = int64_t(blockIdx.x) * 32;
    const int64_t rA = min<int64_t>(r0 + n, a.M - 1), rB = min<int64_t>(r0 + 16 + n, a.M - 1);
    const int nchunks = int((K + 127) / 128);
    const int nrounds = int((K + MX_SLAB - 1) / MX_SLAB);
    auto load = [&](int c, MxChunk& d) {
        // the group's columns; a chunk past K (only when K % 128 != 0) reloads group 0
        int64_t g = int64_t(c) * 4 + q;
        if (g >= G) g = 0;
        const uint4* pa = reinterpret_cast<const uint4*>(a.mag + rA * K + g * 32);
        const uint4* pb = reinterpret_cast<const uint4*>(a.mag + rB * K + g * 32);
        d.ma0 = pa[0]; d.ma1 = pa[1];
        d.mb0 = pb[0]; d.mb1 = pb[1];
        d.ea = a.exp[rA * G + g];
        d.eb = a.exp[rB * G + g];
        d.sa = a.sign[rA * G + g];
        d.sb = a.sign[rB * G + g];
    };
    // slab r: piece p = threadIdx.x + 1024 i is batch row p / 256, columns
    // r MX_SLAB + 8 (p % 256) + [0, 8); rows past B and columns past K read zero
    auto x_issue = [&](int r, uint4 (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = int(threadIdx.x) + 64 * MX_WAVES * i, row = p >> 8;
            const int64_t col = int64_t(r) * MX_SLAB + 8 * (p & 255);
            v[i] = row < B && col < K ? *reinterpret_cast<const uint4*>(x + row * K + col) : make_uint4(0, 0, 0, 0);
        }
    };
    auto x_store = [&](int buf, const uint4 (&v)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = int(threadIdx.x) + 64 * MX_WAVES * i, row = p >> 8;
            *reinterpret_cast<uint4*>(xs + (buf * 16 + row) * MX_XROW + 8 * (p & 255)) = v[i];
        }
    };
    f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c, const MxChunk& d, int buf) {
        const bool live = int64_t(c) * 4 + q < G;    // group past K: contributes nothing
        const float sa = live ? __builtin_ldexpf(1.f, int(d.ea) - 134) : 0.f;
        const float sb = live ? __builtin_ldexpf(1.f, int(d.eb) - 134) : 0.f;
        const uint2 ma[4] = {make_uint2(d.ma0.x, d.ma0.y), make_uint2(d.ma0.z, d.ma0.w),
                             make_uint2(d.ma1.x, d.ma1.y), make_uint2(d.ma1.z, d.ma1.w)};
        const uint2 mb[4] = {make_uint2(d.mb0.x, d.mb0.y), make_uint2(d.mb0.z, d.mb0.w),
                             make_uint2(d.mb1.x, d.mb1.y), make_uint2(d.mb1.z, d.mb1.w)};
        const uint16_t* xb = xs + (buf * 16 + n) * MX_XROW + wave * 128 + q * 32;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 bv = *reinterpret_cast<const uint4*>(xb + 8 * s);
            const uint4 av = mx_to_bf16x8(ma[s], sa, (d.sa >> (8 * s)) & 0xFFu);
            const uint4 aw = mx_to_bf16x8(mb[s], sb, (d.sb >> (8 * s)) & 0xFFu);
            accA = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                           __builtin_bit_cast(bf16x8_t, bv), accA, 0, 0, 0);
            accB = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw),
                                                           __builtin_bit_cast(bf16x8_t, bv), accB, 0, 0, 0);
        }
    };
    // Round r reads slab buffer r % 2 and weight buffer r % 2; the barrier that
    // ends a round orders its slab reads before the next round's slab stores into
    // the other buffer.  The scheduling fences keep each round's loads issued
    // before its compute (left to itself the compiler sinks them below it).
    MxChunk c0, c1;
    uint4 xr[4];
    x_issue(0, xr);
    load(min(wave, nchunks - 1), c0);
    x_store(0, xr);
    __syncthreads();
    for (int r = 0; r < nrounds; r += 2) {
        const bool more = r + 1 < nrounds;             // block-uniform
        if (more) x_issue(r + 1, xr);
        load(min(MX_WAVES * (r + 1) + wave, nchunks - 1), c1);
        __builtin_amdgcn_sched_barrier(0);
        if (MX_WAVES * r + wave < nchunks) compute(MX_WAVES * r + wave, c0, 0);
        if (more) x_store(1, xr);
        __syncthreads();
        if (!more) break;
        const bool more2 = r + 2 < nrounds;
        if (more2) x_issue(r + 2, xr);
        load(min(MX_WAVES * (r + 2) + wave, nchunks - 1), c0);
        __builtin_amdgcn_sched_barrier(0);
        if (MX_WAVES * (r + 1) + wave < nchunks) compute(MX_WAVES * (r + 1) + wave, c1, 1);
        if (more2) x_store(0, xr);
        __syncthreads();
    }
    // the slab buffers are free after the last barrier
    float* red = reinterpret_cast<float*>(mxl4);      // [MX_WAVES][2][64][4]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        red[((wave * 2 + 0) * 64 + lane) * 4 + j] = accA[j];
        red[((wave * 2 + 1) * 64 + lane) * 4 + j] = accB[j];
    }
    __syncthreads();
    // C[row = 4q + j][col = n]; waves 0 and 1 sum tiles A and B
    if (wave < 2) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < MX_WAVES; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] += red[((w * 2 + wave) * 64 + lane) * 4 + j];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = r0 + 16 * wave + 4 * q + j;
            if (n < B && r < a.M) y[int64_t(n) * a.M + r] = s4[j];
        }
    }
}

__global__ __launch_bounds__(256) void mx_dequant_kernel(MxArgs a, float* __restrict__ out) {
    const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (g >= a.M * (a.K / 32)) return;
    const int ex = int(a.exp[g]) - 134;
    const uint32_t sg = a.sign[g];
    const uint4* m = reinterpret_cast<const uint4*>(a.mag + g * 32);
    float4* o = reinterpret_cast<float4*>(out + g * 32);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint4 mv = m[q];
        const uint32_t w[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float4 v;
            float* vp = reinterpret_cast<float*>(&v);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int e = q * 16 + i * 4 + b;
                const float f = __builtin_ldexpf(float((w[i] >> (8 * b)) & 0xFFu), ex);
                vp[b] = ((sg >> e) & 1u) ? -f : f;
            }
            o[q * 4 + i] = v;
        }
    }
}

// ------------------------------------------------------------------ Cassandra-2 draft (MX-32 exponent code)
//
// [Cassandra] 3.3, Cassandra-2: the kept values' exponents are not coded one by
// one; 32 consecutive kept values share the largest exponent X and keep a 4-bit
// magnitude, so kept value j is (-1)^S mag 2^(X - 130) with no stream to parse.
// A lane owns 64 positions of a 4096-element tile (two bitmap words, never across
// a row since K % 128 == 0); a wave prefix sum of their popcounts gives its first
// kept index, and it walks its set bits, reading kept values j, j + 1, ... with
// the nibble word (8 values) and the group's sign word and exponent (32 values)
// cached in registers.

struct MxSpecArgs {
    const uint32_t* bitmap;
    const uint32_t* nib;
    const uint32_t* sign;
    const uint8_t* xexp;
    const uint32_t* kprefix;
    int64_t M, K, N, T;
};

// Draft GEMV.  Block = R consecutive rows, its waves taking the tiles that meet
// them round robin (a tile shared with the next block is walked by both, each
// keeping its own rows).  Per tile every lane has one row; the lanes of a row
// are consecutive, a segmented shuffle sum leaves the row's sum in its first
// lane, which adds it to the wave's row total in LDS; the waves' totals are
// summed in wave order at the end.  XL: activations staged in LDS.
//
// Software pipeline: a tile's bitmap words are loaded two tiles ahead, and its
// lanes' nibble, sign and exponent words (all a lane's up to 64 kept values can
// need: 9 nibble words, 3 groups) one tile ahead, so the walk itself never waits
// for memory.  In the walk the words move through register queues.
struct MxLane {
    uint32_t w0, w1;            // bitmap words of the lane's 64 positions
    uint32_t j0;                // first kept index
    uint32_t q[9], sg[3];       // nibble words from j0 / 8, sign words from j0 / 32
    uint32_t xe;                // exponents of groups j0 / 32 .. + 2 (bytes 0..2)
};

__device__ __forceinline__ void mx_bitmap(const MxSpecArgs& a, int64_t t, MxLane& L) {
    const uint32_t f = uint32_t(t * TILE) + 64u * uint32_t(lane_id());
    const bool live = int64_t(f) < a.N;
    const uint32_t wi = live ? f >> 5 : 0u;
    const uint32_t v0 = a.bitmap[wi], v1 = a.bitmap[wi + 1];
    L.w0 = live ? v0 : 0u;
    L.w1 = live ? v1 : 0u;
}

typedef uint32_t mx_u32x4_dw_t __attribute__((ext_vector_type(4), aligned(4)));

// Kept index of the lane's first value and the loads of its words.  Every load
// is unconditional: indices past the data stay inside the sections' padding.
__device__ __forceinline__ void mx_prep(const MxSpecArgs& a, int64_t t, MxLane& L) {
    const int pc = __popc(L.w0) + __popc(L.w1);
    L.j0 = a.kprefix[t] + uint32_t(wave_incl_add(pc) - pc);
    const uint32_t* np = a.nib + (L.j0 >> 3);
    const mx_u32x4_dw_t n0 = *reinterpret_cast<const mx_u32x4_dw_t*>(np);
    const mx_u32x4_dw_t n1 = *reinterpret_cast<const mx_u32x4_dw_t*>(np + 4);
    L.q[0] = n0.x; L.q[1] = n0.y; L.q[2] = n0.z; L.q[3] = n0.w;
    L.q[4] = n1.x; L.q[5] = n1.y; L.q[6] = n1.z; L.q[7] = n1.w;
    L.q[8] = np[8];
    const uint32_t g = L.j0 >> 5;
    L.sg[0] = a.sign[g]; L.sg[1] = a.sign[g + 1]; L.sg[2] = a.sign[g + 2];
    L.xe = uint32_t(a.xexp[g]) | (uint32_t(a.xexp[g + 1]) << 8) | (uint32_t(a.xexp[g + 2]) << 16);
}

template <int BMAX, bool XL>
__global__ __launch_bounds__(1024) void mx_spec_gemv_kernel(MxSpecArgs a, const uint16_t* __restrict__ x, int B,
                                                            float* __restrict__ y, int R) {
    extern __shared__ __attribute__((aligned(16))) uint4 sm4[];
    const int nw = blockDim.x >> 6, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t K = uint32_t(a.K);
    uint16_t* xs = reinterpret_cast<uint16_t*>(sm4);                          // [BMAX][K]
    float* red = reinterpret_cast<float*>(xs + (XL ? BMAX * int64_t(K) : 0)); // [nw][R][BMAX]
    if constexpr (XL)
        for (int i = threadIdx.x; i < int(uint32_t(B) * K / 8); i += blockDim.x)
            reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
    for (int i = threadIdx.x; i < nw * R * BMAX; i += blockDim.x) red[i] = 0.f;
    __syncthreads();
    const uint16_t* xv = XL ? xs : x;
    const int64_t r0 = int64_t(blockIdx.x) * R, r1 = min<int64_t>(a.M, r0 + R);
    const int64_t t_a = (r0 * K) / TILE, t_b = (r1 * K - 1) / TILE;
    float* wred = red + wave * R * BMAX;
    const int64_t tw0 = t_a + wave;
    const int ntiles = t_b >= tw0 ? int((t_b - tw0) / nw) + 1 : 0;
    auto tile_of = [&](int i) { return tw0 + int64_t(min(i, ntiles - 1)) * nw; };

    auto walk = [&](int64_t t, const MxLane& L) {
        const uint32_t f = uint32_t(t * TILE) + 64u * uint32_t(lane);   // N <= 2^32
        const bool live = int64_t(f) < a.N;
        const uint32_t row = f / K, col0 = f - row * K;
        const bool mine = live && int64_t(row) >= r0 && int64_t(row) < r1;
        float acc[BMAX];
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[b] = 0.f;
        if (mine) {
            uint64_t mm = uint64_t(L.w0) | (uint64_t(L.w1) << 32);
            uint32_t q0 = L.q[0] >> (4 * (L.j0 & 7)), q1 = L.q[1], q2 = L.q[2], q3 = L.q[3], q4 = L.q[4],
                     q5 = L.q[5], q6 = L.q[6], q7 = L.q[7], q8 = L.q[8];
            uint32_t s0 = L.sg[0] >> (L.j0 & 31), s1 = L.sg[1], s2 = L.sg[2], xe = L.xe;
            int ni = int(L.j0 & 7), si = int(L.j0 & 31);
            float scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
            const uint16_t* xc = xv + col0;
            while (mm) {
                const int p = __builtin_ctzll(mm);
                mm &= mm - 1;
                float v = float(q0 & 15u) * scale;               // exact: <= 4 significant bits
                v = (s0 & 1u) ? -v : v;
#pragma unroll
                for (int b = 0; b < BMAX; ++b)
                    if (b < B) acc[b] = fmaf(v, __uint_as_float(uint32_t(xc[b * K + p]) << 16), acc[b]);
                q0 >>= 4;
                s0 >>= 1;
                if (++ni == 8) {
                    ni = 0;
                    q0 = q1; q1 = q2; q2 = q3; q3 = q4; q4 = q5; q5 = q6; q6 = q7; q7 = q8;
                }
                if (++si == 32) {
                    si = 0;
                    s0 = s1; s1 = s2;
                    xe >>= 8;
                    scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
                }
            }
        }
        // segmented suffix sums over the lanes of each row (rows are contiguous
        // lane ranges): afterwards the first lane of a row holds the row's sum
        const int rid = int(row);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int orow = __shfl_down(rid, off, 64);
            const bool add = lane + off < 64 && orow == rid;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                const float o = __shfl_down(acc[b], off, 64);
                acc[b] = add ? acc[b] + o : acc[b];
            }
        }
        const int prow = __shfl_up(rid, 1, 64);
        if (mine && (lane == 0 || prow != rid)) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) wred[int(row - r0) * BMAX + b] += acc[b];
        }
    };

    // two lane buffers: tile i walks from one while tile i + 1's words load into
    // the other (a buffer is never copied while its loads are in flight)
    MxLane la, lb;
    if (ntiles > 0) {
        mx_bitmap(a, tile_of(0), la);
        mx_bitmap(a, tile_of(1), lb);
        mx_prep(a, tile_of(0), la);
    }
    for (int i = 0; i < ntiles; i += 2) {
        mx_prep(a, tile_of(i + 1), lb);
        walk(tile_of(i), la);
        mx_bitmap(a, tile_of(i + 2), la);
        mx_prep(a, tile_of(i + 2), la);
        if (i + 1 < ntiles) walk(tile_of(i + 1), lb);
        mx_bitmap(a, tile_of(i + 3), lb);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * BMAX; i += blockDim.x) {
        const int r = i / BMAX, b = i - r * BMAX;
        if (b < B && r0 + r < r1) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[(w * R + r) * BMAX + b];
            y[int64_t(b) * a.M + r0 + r] = sum;
        }
    }
}

// Kept-domain draft GEMV (K >= 4096, batch <= 2, activations in LDS): every lane
// takes an even share of the tile's kept values (c = ceil(kept / 64) consecutive
// ones), finds the first one's position with the bitmap cursor over the tile's
// staged bitmap words, and walks on, so no lane idles while another walks a
// dense stretch.  A tile meets at most two rows, so a lane keeps two sums.  A
// tile's table entries, bitmap words and the lane's nibble, sign and exponent
// words are loaded one tile ahead.
struct MxKept {
    uint32_t kp0, nk;           // the tile's first kept index and kept count
    uint32_t first;             // the lane's first kept value, tile relative
    int cnt;                    // its count
    uint32_t b0, b1;            // bitmap words 2 lane, 2 lane + 1 of the tile
    uint32_t q[9], sg[3], xe;   // as MxLane, from kept index kp0 + first
};

__device__ __forceinline__ void mx_kept_issue(const MxSpecArgs& a, int64_t t, MxKept& L) {
    const int lane = lane_id();
    L.kp0 = a.kprefix[t];
    L.nk = a.kprefix[t + 1] - L.kp0;
    int first, cnt;
    lane_share(int(L.nk), 64, lane, first, cnt);
    L.first = uint32_t(first);
    L.cnt = cnt;
    const int64_t nwords = (a.N + 31) >> 5, wi = t * (TILE / 32) + 2 * lane;
    const uint32_t v0 = a.bitmap[min<int64_t>(wi, nwords - 1)], v1 = a.bitmap[min<int64_t>(wi + 1, nwords - 1)];
    L.b0 = wi < nwords ? v0 : 0u;
    L.b1 = wi + 1 < nwords ? v1 : 0u;
    const uint32_t j0 = L.kp0 + L.first;                 // at most 63 values past the stream
    const uint32_t* np = a.nib + (j0 >> 3);
    const mx_u32x4_dw_t n0 = *reinterpret_cast<const mx_u32x4_dw_t*>(np);
    const mx_u32x4_dw_t n1 = *reinterpret_cast<const mx_u32x4_dw_t*>(np + 4);
    L.q[0] = n0.x; L.q[1] = n0.y; L.q[2] = n0.z; L.q[3] = n0.w;
    L.q[4] = n1.x; L.q[5] = n1.y; L.q[6] = n1.z; L.q[7] = n1.w;
    L.q[8] = np[8];
    const uint32_t g = j0 >> 5;
    L.sg[0] = a.sign[g]; L.sg[1] = a.sign[g + 1]; L.sg[2] = a.sign[g + 2];
    L.xe = uint32_t(a.xexp[g]) | (uint32_t(a.xexp[g + 1]) << 8) | (uint32_t(a.xexp[g + 2]) << 16);
}

// Draft weights: two tiles per wave (both tiles' loads issued up front).  Lanes
// take even shares of a tile's kept values, find their positions with the bitmap
// cursor and scatter the bf16 values into the wave's zeroed LDS tile, which is
// then written out 16 bytes a lane.
constexpr int MXD_WAVES = 4;

__global__ __launch_bounds__(64 * MXD_WAVES) void mx_spec_decode_kernel(MxSpecArgs a, uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t dense[MXD_WAVES][TILE];
    __shared__ WaveArea areas[MXD_WAVES];
    const int wave = int(threadIdx.x >> 6), lane = lane_id();
    uint16_t* d = dense[wave];
    WaveArea& W = areas[wave];
    auto decode = [&](int64_t t, const MxKept& L) {
        uint4* d4 = reinterpret_cast<uint4*>(d) + lane;       // pruned positions read +0.0
#pragma unroll
        for (int i = 0; i < 8; ++i) d4[64 * i] = make_uint4(0, 0, 0, 0);   // lane-contiguous: no bank conflicts
        W.bw[2 * lane] = L.b0;
        W.bw[2 * lane + 1] = L.b1;
        const int pc = __popc(L.b0) + __popc(L.b1);
        W.bp[lane] = uint16_t(wave_incl_add(pc) - pc);
        // a tile without a bitmap word free of kept positions (nearly all) walks
        // with the cursor compiled without its loop over empty words
        const bool gaps = __ballot(L.b0 == 0u || L.b1 == 0u) != 0;
        wave_sync_lds();
        auto scatter = [&](auto g) __attribute__((always_inline)) {
            BitCursor<false, decltype(g)::value> kc;
            kc.start(W, int(L.first));
            const uint32_t j0 = L.kp0 + L.first;
            uint32_t q0 = L.q[0] >> (4 * (j0 & 7)), q1 = L.q[1], q2 = L.q[2], q3 = L.q[3], q4 = L.q[4],
                     q5 = L.q[5], q6 = L.q[6], q7 = L.q[7], q8 = L.q[8];
            uint32_t s0 = L.sg[0] >> (j0 & 31), s1 = L.sg[1], s2 = L.sg[2], xe = L.xe;
            int ni = int(j0 & 7), si = int(j0 & 31);
            float scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
            for (int v = 0; v < L.cnt; ++v) {
                const int pos = kc.next(W);
                float w = float(q0 & 15u) * scale;               // exact: <= 4 significant bits
                w = (s0 & 1u) ? -w : w;
                d[pos] = uint16_t(__float_as_uint(w) >> 16);
                q0 >>= 4;
                s0 >>= 1;
                if (++ni == 8) {
                    ni = 0;
                    q0 = q1; q1 = q2; q2 = q3; q3 = q4; q4 = q5; q5 = q6; q6 = q7; q7 = q8;
                }
                if (++si == 32) {
                    si = 0;
                    s0 = s1; s1 = s2;
                    xe >>= 8;
                    scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
                }
            }
        };
        if (L.cnt > 0) {
            if (gaps) scatter(std::true_type{});
            else scatter(std::false_type{});
        }
        wave_sync_lds();
        const int tl = int(min<int64_t>(TILE, a.N - t * TILE));
        uint4* o = reinterpret_cast<uint4*>(out + t * TILE);
        for (int g = lane; g < tl / 8; g += 64) o[g] = *reinterpret_cast<const uint4*>(d + 8 * g);
    };
    const int64_t t0 = __builtin_amdgcn_readfirstlane(int(blockIdx.x) * 2 * MXD_WAVES + wave);
    const int64_t t1 = t0 + MXD_WAVES;
    if (t0 >= a.T) return;
    MxKept l0, l1;
    mx_kept_issue(a, t0, l0);
    mx_kept_issue(a, min<int64_t>(t1, a.T - 1), l1);
    decode(t0, l0);
    if (t1 >= a.T) return;
    wave_sync_lds();                                         // the tile is read out before it is overwritten
    decode(t1, l1);
}

template <int BMAX>
__global__ __launch_bounds__(1024) void mx_spec_gemv_kept_kernel(MxSpecArgs a, const uint16_t* __restrict__ x, int B,
                                                                 float* __restrict__ y, int R) {
    extern __shared__ __attribute__((aligned(16))) uint4 sm4[];
    const int nw = blockDim.x >> 6, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = int(a.K);
    uint16_t* xs = reinterpret_cast<uint16_t*>(sm4);                     // [BMAX][K]
    WaveArea* areas = reinterpret_cast<WaveArea*>(xs + BMAX * K);        // [nw]
    float* red = reinterpret_cast<float*>(areas + nw);                   // [nw][R][BMAX]
    for (int i = threadIdx.x; i < B * K / 8; i += blockDim.x)
        reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(x)[i];
    for (int i = threadIdx.x; i < nw * R * BMAX; i += blockDim.x) red[i] = 0.f;
    __syncthreads();
    const int64_t r0 = int64_t(blockIdx.x) * R, r1 = min<int64_t>(a.M, r0 + R);
    const int64_t t_a = (r0 * K) / TILE, t_b = (r1 * K - 1) / TILE;
    WaveArea& W = areas[wave];
    float* wred = red + wave * R * BMAX;
    const int64_t tw0 = t_a + wave;
    const int ntiles = t_b >= tw0 ? int((t_b - tw0) / nw) + 1 : 0;
    auto tile_of = [&](int i) { return tw0 + int64_t(min(i, ntiles - 1)) * nw; };

    auto walk = [&](int64_t t, const MxKept& L) {
        // stage the tile's bitmap words with exclusive prefix counts per word pair
        W.bw[2 * lane] = L.b0;
        W.bw[2 * lane + 1] = L.b1;
        const int pc = __popc(L.b0) + __popc(L.b1);
        W.bp[lane] = uint16_t(wave_incl_add(pc) - pc);
        const bool gaps = __ballot(L.b0 == 0u || L.b1 == 0u) != 0;   // as in the draft decode
        wave_sync_lds();
        const int64_t f0 = t * TILE;
        const int tl = int(min<int64_t>(TILE, a.N - f0));
        const int64_t row_a = f0 / K;
        const int bnd = int(min<int64_t>(tl, (row_a + 1) * K - f0));   // first position of the next row
        const int colbase = int(f0 - row_a * K);
        float accA[BMAX], accB[BMAX];
#pragma unroll
        for (int b = 0; b < BMAX; ++b) accA[b] = accB[b] = 0.f;
        auto dot = [&](auto g) __attribute__((always_inline)) {
            BitCursor<false, decltype(g)::value> kc;
            kc.start(W, int(L.first));
            const uint32_t j0 = L.kp0 + L.first;
            uint32_t q0 = L.q[0] >> (4 * (j0 & 7)), q1 = L.q[1], q2 = L.q[2], q3 = L.q[3], q4 = L.q[4],
                     q5 = L.q[5], q6 = L.q[6], q7 = L.q[7], q8 = L.q[8];
            uint32_t s0 = L.sg[0] >> (j0 & 31), s1 = L.sg[1], s2 = L.sg[2], xe = L.xe;
            int ni = int(j0 & 7), si = int(j0 & 31);
            float scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
            for (int v = 0; v < L.cnt; ++v) {
                const int pos = kc.next(W);
                float w = float(q0 & 15u) * scale;               // exact: <= 4 significant bits
                w = (s0 & 1u) ? -w : w;
                const bool inA = pos < bnd;
                const int col = colbase + pos - (inA ? 0 : K);
#pragma unroll
                for (int b = 0; b < BMAX; ++b) {
                    if (b < B) {
                        const float xv = __uint_as_float(uint32_t(xs[b * K + col]) << 16);
                        const float pA = fmaf(w, xv, accA[b]), pB = fmaf(w, xv, accB[b]);
                        accA[b] = inA ? pA : accA[b];
                        accB[b] = inA ? accB[b] : pB;
                    }
                }
                q0 >>= 4;
                s0 >>= 1;
                if (++ni == 8) {
                    ni = 0;
                    q0 = q1; q1 = q2; q2 = q3; q3 = q4; q4 = q5; q5 = q6; q6 = q7; q7 = q8;
                }
                if (++si == 32) {
                    si = 0;
                    s0 = s1; s1 = s2;
                    xe >>= 8;
                    scale = ldexpf(1.f, int(xe & 0xFFu) - 130);
                }
            }
        };
        if (L.cnt > 0) {
            if (gaps) dot(std::true_type{});
            else dot(std::false_type{});
        }
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                accA[b] += __shfl_xor(accA[b], off, 64);
                accB[b] += __shfl_xor(accB[b], off, 64);
            }
            if (lane == 0) {
                if (row_a >= r0 && row_a < r1) wred[int(row_a - r0) * BMAX + b] += accA[b];
                if (bnd < tl && row_a + 1 >= r0 && row_a + 1 < r1) wred[int(row_a + 1 - r0) * BMAX + b] += accB[b];
            }
        }
        wave_sync_lds();                                 // the staged words are rewritten next tile
    };

    MxKept la, lb;
    if (ntiles > 0) mx_kept_issue(a, tile_of(0), la);
    for (int i = 0; i < ntiles; i += 2) {
        mx_kept_issue(a, tile_of(i + 1), lb);
        walk(tile_of(i), la);
        mx_kept_issue(a, tile_of(i + 2), la);
        if (i + 1 < ntiles) walk(tile_of(i + 1), lb);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < R * BMAX; i += blockDim.x) {
        const int r = i / BMAX, b = i - r * BMAX;
        if (b < B && r0 + r < r1) {
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += red[(w * R + r) * BMAX + b];
            y[int64_t(b) * a.M + r0 + r] = sum;
        }
    }
}

}  // namespace cas
}  // namespace mbd

// ------------------------------------------------------------------ host side

using namespace mbd;
using namespace mbd::cas;

namespace {

#ifndef MBD_SPEC_KW
#define MBD_SPEC_KW 16        // kept-domain draft GEMV: waves per block
#endif
#ifndef MBD_SPEC_KR
#define MBD_SPEC_KR 16        // kept-domain draft GEMV: rows per block
#endif

inline bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

mbd_status cas_args(const mbd_dweights* w, bool need_verify, CasArgs* a) {
    if (!w) return fail(MBD_EINVAL, "NULL descriptor");
    if (w->fmt != MBD_CASSANDRA) return fail(MBD_EINVAL, "descriptor is not MBD_CASSANDRA");
    if (w->M < 0 || w->K < 128 || w->K % 128) return fail(MBD_ESHAPE, "Cassandra needs K a positive multiple of 128");
    if (w->n_sym < 0 || w->n_sym > 256) return fail(MBD_EINVAL, "n_sym=%d outside [0, 256]", w->n_sym);
    if (w->n_sym == 0 && w->M > 0 && w->n_kept > 0) return fail(MBD_EINVAL, "n_sym=0 with kept values");
    const int last = need_verify ? 8 : 6;
    for (int i = 0; i < last; ++i) {
        if (!w->sec[i]) return fail(MBD_EINVAL, "section %d is NULL", i);
        if (!aligned(w->sec[i], 16)) return fail(MBD_EALIGN, "section %d is not 16-byte aligned", i);
    }
    a->bitmap = static_cast<const uint32_t*>(w->sec[0]);
    a->spec_nib = static_cast<const uint32_t*>(w->sec[1]);
    a->unary = static_cast<const uint32_t*>(w->sec[2]);
    a->codebook = static_cast<const uint8_t*>(w->sec[3]);
    a->bitoff = static_cast<const uint64_t*>(w->sec[4]);
    a->kprefix = static_cast<const uint32_t*>(w->sec[5]);
    a->lo_nib = static_cast<const uint32_t*>(w->sec[6]);
    a->pruned = static_cast<const uint16_t*>(w->sec[7]);
    a->M = w->M;
    a->K = w->K;
    a->N = w->M * w->K;
    a->T = (a->N + TILE - 1) / TILE;
    a->n_sym = w->n_sym;
    return MBD_OK;
}

int round_batch(int B) {
    int b = 1;
    while (b < B) b <<= 1;
    return b;
}

mbd_status decode_dense(const mbd_dweights* w, uint16_t* out, hipStream_t st, bool restore) {
    CasArgs a;
    mbd_status s = cas_args(w, restore, &a);
    if (s != MBD_OK) return s;
    if (!out) return fail(MBD_EINVAL, "output is NULL");
    if (!aligned(out, 16)) return fail(MBD_EALIGN, "output must be 16-byte aligned");
    if (a.N == 0) return MBD_OK;
    const int per_block = 2 * DD_WAVES;                                 // tiles per block
    const unsigned blocks = unsigned((a.T + per_block - 1) / per_block);
    if (restore)
        hipLaunchKernelGGL(decode_dense_kernel<true>, dim3(blocks), dim3(64 * DD_WAVES), 0, st, a, out);
    else
        hipLaunchKernelGGL(decode_dense_kernel<false>, dim3(blocks), dim3(64 * DD_WAVES), 0, st, a, out);
    return hip_check(restore ? "restore launch" : "spec decode launch");
}

mbd_status mx_spec_args(const mbd_dweights* w, MxSpecArgs* a) {
    if (!w) return fail(MBD_EINVAL, "NULL descriptor");
    if (w->M < 0 || w->K < 128 || w->K % 128) return fail(MBD_ESHAPE, "Cassandra needs K a positive multiple of 128");
    if (w->M * w->K > int64_t(UINT32_MAX)) return fail(MBD_ESHAPE, "M*K exceeds the 32-bit kept prefix");
    for (int i = 0; i < 5; ++i) {
        if (!w->sec[i]) return fail(MBD_EINVAL, "section %d is NULL", i);
        if (!aligned(w->sec[i], 16)) return fail(MBD_EALIGN, "section %d is not 16-byte aligned", i);
    }
    a->bitmap = static_cast<const uint32_t*>(w->sec[0]);
    a->nib = static_cast<const uint32_t*>(w->sec[1]);
    a->sign = static_cast<const uint32_t*>(w->sec[2]);
    a->xexp = static_cast<const uint8_t*>(w->sec[3]);
    a->kprefix = static_cast<const uint32_t*>(w->sec[4]);
    a->M = w->M;
    a->K = w->K;
    a->N = w->M * w->K;
    a->T = (a->N + TILE - 1) / TILE;
    return MBD_OK;
}

mbd_status mx_spec_decode(const mbd_dweights* w, uint16_t* out, hipStream_t st) {
    MxSpecArgs a;
    mbd_status s = mx_spec_args(w, &a);
    if (s != MBD_OK) return s;
    if (!out) return fail(MBD_EINVAL, "output is NULL");
    if (!aligned(out, 16)) return fail(MBD_EALIGN, "output must be 16-byte aligned");
    if (a.N == 0) return MBD_OK;
    hipLaunchKernelGGL(mx_spec_decode_kernel, dim3(unsigned((a.T + 2 * MXD_WAVES - 1) / (2 * MXD_WAVES))), dim3(64 * MXD_WAVES),
                       0, st, a, out);
    return hip_check("spec decode launch");
}

// Rows per block: about 32 tiles a block; waves: up to 16, one per tile.
// Activations go to LDS when they fit in 64 KB.
mbd_status mx_spec_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st) {
    MxSpecArgs a;
    mbd_status s = mx_spec_args(w, &a);
    if (s != MBD_OK) return s;
    if (!x || !y) return fail(MBD_EINVAL, "NULL argument");
    if (B < 1 || B > 16) return fail(MBD_ESHAPE, "B=%d outside [1, 16]", B);
    if (!aligned(x, 16) || !aligned(y, 4)) return fail(MBD_EALIGN, "x must be 16-byte and y 4-byte aligned");
    if (a.M == 0) return MBD_OK;
    const int bmax = round_batch(B);
    if (a.K >= TILE && bmax <= 2) {
        // kept-domain walk: a tile meets at most two rows
        constexpr int KW = MBD_SPEC_KW, KR = MBD_SPEC_KR;
        const size_t kl = size_t(bmax) * a.K * 2 + KW * sizeof(WaveArea) + size_t(KW) * KR * bmax * 4;
        if (kl <= 150 * 1024) {
            static std::atomic<int> d1{0}, d2{0};
            const void* kern = bmax == 1 ? reinterpret_cast<const void*>(mx_spec_gemv_kept_kernel<1>)
                                         : reinterpret_cast<const void*>(mx_spec_gemv_kept_kernel<2>);
            if ((s = lds_limit(kern, bmax == 1 ? d1 : d2, kl, "draft GEMV")) != MBD_OK) return s;
            const unsigned blocks = unsigned((a.M + KR - 1) / KR);
            if (bmax == 1)
                hipLaunchKernelGGL(mx_spec_gemv_kept_kernel<1>, dim3(blocks), dim3(64 * KW), kl, st, a, x, B, y, KR);
            else
                hipLaunchKernelGGL(mx_spec_gemv_kept_kernel<2>, dim3(blocks), dim3(64 * KW), kl, st, a, x, B, y, KR);
            return hip_check("spec GEMV launch");
        }
    }
    const bool xl = int64_t(bmax) * a.K * 2 <= 64 * 1024;
    int R = int(std::max<int64_t>(1, std::min<int64_t>(64, (32 * TILE) / a.K))), nw = 1;
    size_t lds = 0;
    for (;; R /= 2) {                                   // fewer rows until the LDS fits
        const int64_t tiles = (int64_t(R) * a.K + TILE - 1) / TILE + 1;
        nw = int(std::min<int64_t>(16, tiles));
        lds = (xl ? size_t(bmax) * a.K * 2 : 0) + size_t(nw) * R * bmax * 4;
        if (lds <= 150 * 1024 || R == 1) break;
    }
    const unsigned blocks = unsigned((a.M + R - 1) / R);
#define MBD_MXS_CASE(BM, XL)                                                                                     \
    if (bmax == BM && xl == XL) {                                                                                \
        static std::atomic<int> done{0};                                                                         \
        const void* kern = reinterpret_cast<const void*>(mx_spec_gemv_kernel<BM, XL>);                           \
        if ((s = lds_limit(kern, done, lds, "draft GEMV")) != MBD_OK) return s;                                  \
        hipLaunchKernelGGL((mx_spec_gemv_kernel<BM, XL>), dim3(blocks), dim3(64 * nw), lds, st, a, x, B, y, R);  \
        return hip_check("spec GEMV launch");                                                                    \
    }
    MBD_MXS_CASE(1, true) MBD_MXS_CASE(2, true) MBD_MXS_CASE(4, true) MBD_MXS_CASE(8, true) MBD_MXS_CASE(16, true)
    MBD_MXS_CASE(1, false) MBD_MXS_CASE(2, false) MBD_MXS_CASE(4, false) MBD_MXS_CASE(8, false) MBD_MXS_CASE(16, false)
#undef MBD_MXS_CASE
    return fail(MBD_EINVAL, "no draft GEMV variant");
}

}  // namespace

mbd_status mbd_gemv_cassandra(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st) {
    CasArgs a;
    mbd_status s = cas_args(w, true, &a);
    if (s != MBD_OK) return s;
    if (a.K % TILE) return fail(MBD_ESHAPE, "the fused verify GEMM needs K %% 4096 == 0 (K=%lld)", (long long)a.K);
    if (a.M == 0) return MBD_OK;
    const size_t lds = size_t(16) * VROW * 2 + size_t(VG_WAVES) * sizeof(WaveArea) + 256;
    static std::atomic<int> lds_done{0};
    if ((s = lds_limit(reinterpret_cast<const void*>(verify_gemm_kernel), lds_done, lds, "verify GEMM")) != MBD_OK)
        return s;
    const unsigned blocks = unsigned((a.M + 15) / 16);
    hipLaunchKernelGGL(verify_gemm_kernel, dim3(blocks), dim3(64 * VG_WAVES), lds, st, a, x, B, y);
    return hip_check("verify GEMM launch");
}

mbd_status mbd_gemv_mx32(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st) {
    if (w->K < 32 || w->K % 32 || w->M < 0) return fail(MBD_ESHAPE, "MX32 needs K a positive multiple of 32");
    for (int i = 0; i < 3; ++i)
        if (!w->sec[i]) return fail(MBD_EINVAL, "section %d is NULL", i);
    if (!aligned(w->sec[1], 4) || !aligned(w->sec[2], 16)) return fail(MBD_EALIGN, "MX sections misaligned");
    if (w->M == 0) return MBD_OK;
    MxArgs a{static_cast<const uint8_t*>(w->sec[0]), static_cast<const uint32_t*>(w->sec[1]),
             static_cast<const uint8_t*>(w->sec[2]), w->M, w->K};
    static std::atomic<int> lds_done{0};
    mbd_status s = lds_limit(reinterpret_cast<const void*>(mx_gemm_kernel), lds_done, MX_LDS, "MX GEMM");
    if (s != MBD_OK) return s;
    const unsigned blocks = unsigned((w->M + 31) / 32);
    hipLaunchKernelGGL(mx_gemm_kernel, dim3(blocks), dim3(64 * MX_WAVES), MX_LDS, st, a, x, B, y);
    return hip_check("MX GEMM launch");
}

mbd_status mbd_dequant_mx32(const mbd_dweights* w, float* out, hipStream_t st) {
    if (w->K < 32 || w->K % 32 || w->M < 0) return fail(MBD_ESHAPE, "MX32 needs K a positive multiple of 32");
    for (int i = 0; i < 3; ++i)
        if (!w->sec[i]) return fail(MBD_EINVAL, "section %d is NULL", i);
    if (!aligned(w->sec[1], 4) || !aligned(w->sec[2], 16)) return fail(MBD_EALIGN, "MX sections misaligned");
    if (w->M == 0) return MBD_OK;
    MxArgs a{static_cast<const uint8_t*>(w->sec[0]), static_cast<const uint32_t*>(w->sec[1]),
             static_cast<const uint8_t*>(w->sec[2]), w->M, w->K};
    const int64_t groups = w->M * (w->K / 32);
    hipLaunchKernelGGL(mx_dequant_kernel, dim3(unsigned((groups + 255) / 256)), dim3(256), 0, st, a, out);
    return hip_check("MX dequant launch");
}

extern "C" {

mbd_status mbd_spec_decode(const mbd_dweights* w, uint16_t* w_spec, void* stream) {
    hip_clear();
    if (w && w->fmt == MBD_CASSANDRA_MX) return mx_spec_decode(w, w_spec, reinterpret_cast<hipStream_t>(stream));
    return decode_dense(w, w_spec, reinterpret_cast<hipStream_t>(stream), false);
}

mbd_status mbd_verify_restore(const mbd_dweights* w, uint16_t* w_out, void* stream) {
    hip_clear();
    return decode_dense(w, w_out, reinterpret_cast<hipStream_t>(stream), true);
}

mbd_status mbd_spec_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, void* stream) {
    hip_clear();
    if (w && w->fmt == MBD_CASSANDRA_MX) return mx_spec_gemv(w, x, B, y, reinterpret_cast<hipStream_t>(stream));
    CasArgs a;
    mbd_status s = cas_args(w, false, &a);
    if (s != MBD_OK) return s;
    if (!x || !y) return fail(MBD_EINVAL, "NULL argument");
    if (B < 1 || B > 16) return fail(MBD_ESHAPE, "B=%d outside [1, 16]", B);
    if (!aligned(x, 16) || !aligned(y, 4)) return fail(MBD_EALIGN, "x must be 16-byte and y 4-byte aligned");
    if (a.M == 0) return MBD_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int bmax = round_batch(B);
    // kept-domain kernel: K >= 4096 (a tile meets at most two rows), batch <= 2,
    // activations staged in LDS
    constexpr int KW = MBD_SPEC_KW, KR = MBD_SPEC_KR;
    const size_t kl = size_t(bmax) * a.K * 2 + KW * sizeof(WaveArea) + size_t(KW) * KR * bmax * 4 +
                      (size_t(std::max(1, a.n_sym)) * 16 + 1) * 4;
    if (a.K >= TILE && bmax <= 2 && kl <= 160 * 1024) {
        static std::atomic<int> done1{0}, done2{0};
        const void* kern = bmax == 1 ? reinterpret_cast<const void*>(spec_gemv_kept_kernel<1>)
                                     : reinterpret_cast<const void*>(spec_gemv_kept_kernel<2>);
        if ((s = lds_limit(kern, bmax == 1 ? done1 : done2, kl, "draft GEMV")) != MBD_OK) return s;
        const unsigned blocks = unsigned((a.M + KR - 1) / KR);
        if (bmax == 1)
            hipLaunchKernelGGL(spec_gemv_kept_kernel<1>, dim3(blocks), dim3(64 * KW), kl, st, a, x, B, y, KR);
        else
            hipLaunchKernelGGL(spec_gemv_kept_kernel<2>, dim3(blocks), dim3(64 * KW), kl, st, a, x, B, y, KR);
        return hip_check("spec GEMV launch");
    }
    // rows per block: smallest R in {1, 2, 4} whose flat range is whole tiles
    int R = 1;
    if ((a.K % TILE) != 0) R = ((2 * a.K) % TILE == 0) ? 2 : 4;
    if (bmax > 4 && R > 2) R = 2;
    const int64_t fa_tiles = (int64_t(R) * a.K + TILE - 1) / TILE + 1;
    const int nw = int(std::min<int64_t>(4, fa_tiles));
    const unsigned blocks = unsigned((a.M + R - 1) / R);
#define MBD_SPEC_CASE(BM, RR)                                                                          \
    if (bmax == BM && R == RR) {                                                                       \
        hipLaunchKernelGGL((spec_gemv_kernel<BM, RR>), dim3(blocks), dim3(64 * nw), 0, st, a, x, B, y); \
        return hip_check("spec GEMV launch");                                                          \
    }
    MBD_SPEC_CASE(1, 1) MBD_SPEC_CASE(1, 2) MBD_SPEC_CASE(1, 4)
    MBD_SPEC_CASE(2, 1) MBD_SPEC_CASE(2, 2) MBD_SPEC_CASE(2, 4)
    MBD_SPEC_CASE(4, 1) MBD_SPEC_CASE(4, 2) MBD_SPEC_CASE(4, 4)
    MBD_SPEC_CASE(8, 1) MBD_SPEC_CASE(8, 2)
    MBD_SPEC_CASE(16, 1) MBD_SPEC_CASE(16, 2)
#undef MBD_SPEC_CASE
    return fail(MBD_EINVAL, "no spec GEMV variant");
}

}  // extern "C"
