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

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// ------------------------------------------------------------------ dense decode

template <bool RESTORE>
__global__ __launch_bounds__(256) void decode_dense_kernel(CasArgs a, uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint16_t bufs[4][ROW_STRIDE];
    __shared__ uint8_t cb[256];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb[i] = i < a.n_sym ? a.codebook[i] : 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int64_t t = int64_t(blockIdx.x) * 4 + wave;
    if (t >= a.T) return;
    const int tl = int(min<int64_t>(TILE, a.N - t * TILE));
    uint32_t pairs[32];
    decode_tile<RESTORE>(a, t, tl, bufs[wave], cb, pairs);
    if (64 * lane < tl) {
        uint4* dst = reinterpret_cast<uint4*>(out + t * TILE + 64 * lane);
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = make_uint4(pairs[4 * i], pairs[4 * i + 1], pairs[4 * i + 2], pairs[4 * i + 3]);
    }
}

// ------------------------------------------------------------------ draft GEMV

// Block = R consecutive rows (flat range [r0*K, (r0+R)*K)); its waves take the
// overlapping tiles round robin.  Lane partials are reduced per (row, batch).
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

// ------------------------------------------------------------------ verify GEMM (fused restore + MFMA)

// Block = 16 rows x all K (K % 4096 == 0), 8 waves.  Per 4096-column slab each
// wave restores two of the 16 row tiles into LDS, then the waves split the slab's
// 128 MFMA k-steps; partial 16x16 tiles are summed across waves at the end.
constexpr int VG_WAVES = 8;

__global__ __launch_bounds__(512) void verify_gemm_kernel(CasArgs a, const uint16_t* __restrict__ x, int B,
                                                          float* __restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint16_t vlds[];
    uint16_t* rows = vlds;                                              // [16][ROW_STRIDE]
    uint8_t* cb = reinterpret_cast<uint8_t*>(vlds + 16 * ROW_STRIDE);  // [256]
    float* red = reinterpret_cast<float*>(cb + 256);                    // [VG_WAVES][64][4]
    for (int i = threadIdx.x; i < 256; i += blockDim.x) cb[i] = i < a.n_sym ? a.codebook[i] : 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int64_t K = a.K, tpr = K / TILE;
    const int64_t r0 = int64_t(blockIdx.x) * 16;
    const int n = lane & 15, kq = lane >> 4;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t kt = 0; kt < tpr; ++kt) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = wave * 2 + rr;
            uint16_t* buf = rows + r * ROW_STRIDE;
            const int64_t row = r0 + r;
            uint32_t pairs[32];
            if (row < a.M) {
                decode_tile<true>(a, row * tpr + kt, TILE, buf, cb, pairs);
            } else {
#pragma unroll
                for (int i = 0; i < 32; ++i) pairs[i] = 0u;
            }
            wave_sync_lds();
            uint4* dst = reinterpret_cast<uint4*>(buf + 64 * lane);
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = make_uint4(pairs[4 * i], pairs[4 * i + 1], pairs[4 * i + 2], pairs[4 * i + 3]);
        }
        __syncthreads();
        // this wave's 16 k-steps of 32 columns
        const uint16_t* xrow = x + int64_t(n) * K + kt * TILE;
        const bool xv = n < B;
#pragma unroll 4
        for (int s = 0; s < 16; ++s) {
            const int k = (wave * 16 + s) * 32 + kq * 8;
            const uint4 av = *reinterpret_cast<const uint4*>(rows + n * ROW_STRIDE + k);
            uint4 bv = make_uint4(0, 0, 0, 0);
            if (xv) bv = *reinterpret_cast<const uint4*>(xrow + k);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                          __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // C[row = 4*kq + j][col = n] of this wave's partial
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
            const int64_t row = r0 + 4 * kq + j;
            if (n < B && row < a.M) y[int64_t(n) * a.M + row] = s[j];
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

// Eight MX elements (one lane's MFMA operand) -> bf16x8: mag * 2^(X-134), sign.
__device__ __forceinline__ uint4 mx_to_bf16x8(uint2 m8, uint32_t X, uint32_t sgn8) {
    uint32_t out[4];
    const uint32_t mw[2] = {m8.x, m8.y};
    const int ex = int(X) - 134;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = mw[i >> 1];
        const int b0 = (i & 1) * 2;
        const float f0 = __builtin_ldexpf(float((w >> (8 * b0)) & 0xFFu), ex);
        const float f1 = __builtin_ldexpf(float((w >> (8 * (b0 + 1))) & 0xFFu), ex);
        uint32_t v = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
        v |= ((sgn8 >> (2 * i)) & 1u) << 15;
        v |= ((sgn8 >> (2 * i + 1)) & 1u) << 31;
        out[i] = v;
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Block = 16 rows, 4 waves splitting K in 32-column steps; MFMA bf16 16x16x32.
__global__ __launch_bounds__(256) void mx_gemm_kernel(MxArgs a, const uint16_t* __restrict__ x, int B,
                                                      float* __restrict__ y) {
    __shared__ float red[4][64][4];
    const int wave = threadIdx.x >> 6, lane = lane_id();
    const int n = lane & 15, kq = lane >> 4;
    const int64_t r0 = int64_t(blockIdx.x) * 16;
    const int64_t row = min<int64_t>(r0 + n, a.M - 1);
    const int64_t G = a.K / 32, steps = G;
    const bool xv = n < B;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow = x + int64_t(n) * a.K;
    for (int64_t s = wave; s < steps; s += 4) {
        const int64_t g = row * G + s;
        const uint32_t X = a.exp[g];
        const uint32_t sg = (a.sign[g] >> (8 * kq)) & 0xFFu;
        const uint2 m8 = *reinterpret_cast<const uint2*>(a.mag + row * a.K + s * 32 + kq * 8);
        const uint4 av = mx_to_bf16x8(m8, X, sg);
        uint4 bv = make_uint4(0, 0, 0, 0);
        if (xv) bv = *reinterpret_cast<const uint4*>(xrow + s * 32 + kq * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                      acc, 0, 0, 0);
    }
    red[wave][lane][0] = acc[0]; red[wave][lane][1] = acc[1]; red[wave][lane][2] = acc[2]; red[wave][lane][3] = acc[3];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float s = red[0][lane][j] + red[1][lane][j] + red[2][lane][j] + red[3][lane][j];
            const int64_t r = r0 + 4 * kq + j;
            if (n < B && r < a.M) y[int64_t(n) * a.M + r] = s;
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

}  // namespace cas
}  // namespace mbd

// ------------------------------------------------------------------ host side

using namespace mbd;
using namespace mbd::cas;

namespace {

inline bool aligned(const void* p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) & (al - 1)) == 0; }

mbd_status hip_check(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MBD_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MBD_OK;
}

mbd_status cas_args(const mbd_dweights* w, bool need_verify, CasArgs* a) {
    if (!w) return fail(MBD_EINVAL, "NULL descriptor");
    if (w->fmt != MBD_CASSANDRA) return fail(MBD_EINVAL, "descriptor is not MBD_CASSANDRA");
    if (w->M < 0 || w->K < 128 || w->K % 128) return fail(MBD_ESHAPE, "Cassandra needs K a positive multiple of 128");
    if (w->n_sym < 1 || w->n_sym > 256) return fail(MBD_EINVAL, "n_sym=%d outside [1, 256]", w->n_sym);
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
    const unsigned blocks = unsigned((a.T + 3) / 4);
    if (restore)
        hipLaunchKernelGGL(decode_dense_kernel<true>, dim3(blocks), dim3(256), 0, st, a, out);
    else
        hipLaunchKernelGGL(decode_dense_kernel<false>, dim3(blocks), dim3(256), 0, st, a, out);
    return hip_check(restore ? "restore launch" : "spec decode launch");
}

}  // namespace

mbd_status mbd_gemv_cassandra(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st) {
    CasArgs a;
    mbd_status s = cas_args(w, true, &a);
    if (s != MBD_OK) return s;
    if (a.K % TILE) return fail(MBD_ESHAPE, "the fused verify GEMM needs K %% 4096 == 0 (K=%lld)", (long long)a.K);
    if (a.M == 0) return MBD_OK;
    const size_t lds = size_t(16) * ROW_STRIDE * 2 + 256 + size_t(VG_WAVES) * 64 * 4 * 4;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(verify_gemm_kernel),
                                hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
            return fail(MBD_EHIP, "cannot raise the verify GEMM LDS limit to %zu bytes", lds);
        attr_set = true;
    }
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
    const unsigned blocks = unsigned((w->M + 15) / 16);
    hipLaunchKernelGGL(mx_gemm_kernel, dim3(blocks), dim3(256), 0, st, a, x, B, y);
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
    return decode_dense(w, w_spec, reinterpret_cast<hipStream_t>(stream), false);
}

mbd_status mbd_verify_restore(const mbd_dweights* w, uint16_t* w_out, void* stream) {
    return decode_dense(w, w_out, reinterpret_cast<hipStream_t>(stream), true);
}

mbd_status mbd_spec_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, void* stream) {
    CasArgs a;
    mbd_status s = cas_args(w, false, &a);
    if (s != MBD_OK) return s;
    if (!x || !y) return fail(MBD_EINVAL, "NULL argument");
    if (B < 1 || B > 16) return fail(MBD_ESHAPE, "B=%d outside [1, 16]", B);
    if (!aligned(x, 16) || !aligned(y, 4)) return fail(MBD_EALIGN, "x must be 16-byte and y 4-byte aligned");
    if (a.M == 0) return MBD_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // rows per block: smallest R in {1, 2, 4} whose flat range is whole tiles
    int R = 1;
    if ((a.K % TILE) != 0) R = ((2 * a.K) % TILE == 0) ? 2 : 4;
    const int bmax = round_batch(B);
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
