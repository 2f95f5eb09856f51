// Fused dequant-GEMV / skinny GEMM for block-ternary ([Bonsai2] 1.2) and INT4
// group-128 ([GPT54-INT4] 3.2) weights on gfx950, the grouped expert GEMV, and
// the dense dequant kernels.
//
// Decode time is set by the weight bytes ([Bolt], background), so the kernel is
// built around one coalesced 16-byte load per lane per "chunk" of packed codes
// (64 ternary or 32 INT4 weights), decoded in registers with two-operation
// shift/and-or sequences into bf16 pairs and consumed by v_dot2c_f32_bf16.
//
// Code -> bf16 trick: OR-ing a small field c into the mantissa of 0x4300 (128.0)
// gives the exact bf16 value 128 + c * 2^p for a field at mantissa bit p.  A
// dot2 against pre-arranged activation pairs therefore computes
// sum (128 + c) x; the per-chunk constant sum_k base_k x_k ("bias", shared by
// every row) is subtracted once per chunk and the group scale applied once per
// chunk.  For ternary, fields sit at mantissa bits 0, 2 and 4, so the matching x
// values are pre-scaled by 1, 1/4 and 1/16 when staged, which lets three fields
// be extracted per shift.
//
// Work split: lanes of a wave are grouped G to a row (G = largest power of two
// <= 64 dividing the chunks per row), each lane walks its row's chunks with
// stride G, and every wave covers RPW such row-steps so one x chunk held in
// registers serves RPW rows.  The activations are staged once per workgroup in
// LDS (pair-permuted, plus per-chunk bias), in K slabs when they do not fit.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>

#include "mbd_internal.h"

namespace mbd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even f32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

template <bool TER>
struct Fmt {
    static constexpr int WPC = TER ? 64 : 32;     // weights per 16-byte chunk
    static constexpr int XW = WPC / 2;            // bf16 pair words per chunk
    static constexpr int XQ = XW / 4;             // uint4 per chunk of x pairs
    static constexpr int CPG = 128 / WPC;         // chunks per scale group
};

// Stage the activations of one chunk: pair-permuted (and, for ternary, scaled
// by 1, 1/4, 1/16 per mantissa position class) plus its bias.
template <bool TER>
__device__ __forceinline__ void stage_chunk(const uint16_t* __restrict__ xs, uint4* __restrict__ dst,
                                            int stride_q, float* __restrict__ bias) {
    using F = Fmt<TER>;
    const uint4* src = reinterpret_cast<const uint4*>(xs);
    float b = 0.f;
    if constexpr (TER) {
        // word i covers k = 16i .. 16i+15: pair p = (x[16i+p], x[16i+p+8]), p = 0..7
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 lo = src[2 * i], hi = src[2 * i + 1];
            uint32_t xl[4] = {lo.x, lo.y, lo.z, lo.w}, xh[4] = {hi.x, hi.y, hi.z, hi.w};
            uint32_t pw[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                uint32_t a = (xl[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                uint32_t c = (xh[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                float fa = bf16_to_f32(a), fc = bf16_to_f32(c);
                const int cls = p % 3;                      // 0: x1, 1: x1/4, 2: x1/16
                const float sc = cls == 0 ? 1.f : (cls == 1 ? 0.25f : 0.0625f);
                const float base = cls == 0 ? 129.f : (cls == 1 ? 33.f : 9.f);
                b += base * (fa + fc);
                pw[p] = f32_to_bf16(fa * sc) | (f32_to_bf16(fc * sc) << 16);
            }
            dst[(2 * i) * stride_q] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
            dst[(2 * i + 1) * stride_q] = make_uint4(pw[4], pw[5], pw[6], pw[7]);
        }
    } else {
        // word i covers k = 8i .. 8i+7: pair p = (x[8i+p], x[8i+p+4]), p = 0..3
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 v = src[i];
            uint32_t xv[4] = {v.x, v.y, v.z, v.w};
            uint32_t pw[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t a = (xv[p >> 1] >> (16 * (p & 1))) & 0xFFFFu;
                uint32_t c = (xv[2 + (p >> 1)] >> (16 * (p & 1))) & 0xFFFFu;
                b += bf16_to_f32(a) + bf16_to_f32(c);
                pw[p] = a | (c << 16);
            }
            dst[i * stride_q] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
        }
        b *= 136.f;
    }
    (void)F::XW;
    *bias = b;
}

// Unpack one 16-byte chunk of codes into bf16 pair words (128 + c * 2^p).
template <bool TER>
__device__ __forceinline__ void unpack_chunk(const uint4 w, uint32_t (&p)[Fmt<TER>::XW]) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    constexpr uint32_t MAGIC = 0x43004300u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = wv[i];
        if constexpr (TER) {
            const uint32_t s6 = v >> 6, s12 = v >> 12;
            p[8 * i + 0] = (v & 0x00030003u) | MAGIC;
            p[8 * i + 1] = (v & 0x000C000Cu) | MAGIC;
            p[8 * i + 2] = (v & 0x00300030u) | MAGIC;
            p[8 * i + 3] = (s6 & 0x00030003u) | MAGIC;
            p[8 * i + 4] = (s6 & 0x000C000Cu) | MAGIC;
            p[8 * i + 5] = (s6 & 0x00300030u) | MAGIC;
            p[8 * i + 6] = (s12 & 0x00030003u) | MAGIC;
            p[8 * i + 7] = (s12 & 0x000C000Cu) | MAGIC;
        } else {
            p[4 * i + 0] = (v & 0x000F000Fu) | MAGIC;
            p[4 * i + 1] = ((v >> 4) & 0x000F000Fu) | MAGIC;
            p[4 * i + 2] = ((v >> 8) & 0x000F000Fu) | MAGIC;
            p[4 * i + 3] = ((v >> 12) & 0x000F000Fu) | MAGIC;
        }
    }
}

template <int N>
__device__ __forceinline__ float dot_pairs(const uint32_t (&p)[N], const uint32_t (&x)[N]) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        a0 = dot2(p[i], x[i], a0);
        a1 = dot2(p[i + 1], x[i + 1], a1);
    }
    return a0 + a1;
}

struct BqArgs {
    const uint4* codes;      // [n_mats][M][C] chunks
    const uint16_t* scales;  // [n_mats][M][K/128]
    const uint16_t* x;       // bf16 activations
    float* y;                // fp32 outputs
    int M, K, C, G, SC, B;
    int rows_per_block;
    // expert (grouped) mode
    const int4* jobs;        // {expert, pair_start, n_pairs, 0}
    const int* n_jobs;
    const int* pair_ids;     // pairs sorted by expert: pair id = t*k + slot
    int topk, x_per_pair, row_blocks;
};

// Core: rows [row_base, row_base + rows_per_block) of one matrix, nb <= BMAX batch
// rows whose activations / outputs are given by xrow(b) / yrow(b).
template <bool TER, int BMAX, int RPW, class XRow, class YRow>
__device__ __forceinline__ void bq_core(const BqArgs& a, const uint4* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int row_base, int nb,
                                        XRow xrow, YRow yrow) {
    using F = Fmt<TER>;
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = a.G, RS = 64 / G, C = a.C, K = a.K, M = a.M;
    const int sub = lane & (G - 1), rg = lane / G;
    const int row0 = row_base + wave * (RS * RPW) + rg;
    const int ngroups = K / 128;
    uint4* xl = lds4;                                        // [BMAX][XQ][SC]
    float* bl = reinterpret_cast<float*>(lds4 + BMAX * F::XQ * a.SC);   // [BMAX][SC]

    int rows[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) rows[r] = min(row0 + r * RS, M - 1);

    float acc[RPW][BMAX];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[r][b] = 0.f;

    // first chunk's codes are requested before the activations are staged
    uint4 wc[RPW];
    float sc[RPW];
    auto load = [&](int c, uint4 (&w)[RPW], float (&s)[RPW]) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(codes) + (size_t)rows[r] * C + c);
            w[r] = make_uint4(v.x, v.y, v.z, v.w);
            s[r] = half_bits_to_f32(scales[(size_t)rows[r] * ngroups + c / F::CPG]);
        }
    };
    load(sub, wc, sc);

    for (int c0 = 0; c0 < C; c0 += a.SC) {
        const int scn = min(a.SC, C - c0);
        for (int job = threadIdx.x; job < nb * scn; job += blockDim.x) {
            const int b = job / scn, cc = job - b * scn;
            stage_chunk<TER>(xrow(b) + (size_t)(c0 + cc) * F::WPC, xl + (size_t)b * F::XQ * a.SC + cc,
                             a.SC, bl + b * a.SC + cc);
        }
        __syncthreads();
        for (int cc = sub; cc < scn; cc += G) {
            uint4 wn[RPW];
            float sn[RPW];
            const int cn = c0 + cc + G;
            if (cn < C) load(cn, wn, sn);
            if constexpr (BMAX <= 4) {
                uint32_t xr[BMAX][F::XW];
                float bias[BMAX];
#pragma unroll
                for (int b = 0; b < BMAX; ++b) {
                    if (b < nb) {
#pragma unroll
                        for (int q = 0; q < F::XQ; ++q) {
                            uint4 v = xl[((size_t)b * F::XQ + q) * a.SC + cc];
                            xr[b][4 * q] = v.x; xr[b][4 * q + 1] = v.y; xr[b][4 * q + 2] = v.z; xr[b][4 * q + 3] = v.w;
                        }
                        bias[b] = bl[b * a.SC + cc];
                    }
                }
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    uint32_t p[F::XW];
                    unpack_chunk<TER>(wc[r], p);
#pragma unroll
                    for (int b = 0; b < BMAX; ++b)
                        if (b < nb) acc[r][b] = fmaf(sc[r], dot_pairs(p, xr[b]) - bias[b], acc[r][b]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    uint32_t p[F::XW];
                    unpack_chunk<TER>(wc[r], p);
#pragma unroll
                    for (int b = 0; b < BMAX; ++b) {
                        if (b < nb) {
                            uint32_t xr[F::XW];
#pragma unroll
                            for (int q = 0; q < F::XQ; ++q) {
                                uint4 v = xl[((size_t)b * F::XQ + q) * a.SC + cc];
                                xr[4 * q] = v.x; xr[4 * q + 1] = v.y; xr[4 * q + 2] = v.z; xr[4 * q + 3] = v.w;
                            }
                            acc[r][b] = fmaf(sc[r], dot_pairs(p, xr) - bl[b * a.SC + cc], acc[r][b]);
                        }
                    }
                }
            }
            if (cn < C) {
#pragma unroll
                for (int r = 0; r < RPW; ++r) { wc[r] = wn[r]; sc[r] = sn[r]; }
            }
        }
        __syncthreads();
    }

    // reduce across the G lanes of each row group; lane sub == 0 stores
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            float v = acc[r][b];
            for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
            const int row = row0 + r * RS;
            if (sub == 0 && b < nb && row < M) yrow(b)[row] = v;
        }
    }
}

template <bool TER, int BMAX, int RPW>
__global__ __launch_bounds__(256) void gemv_bq_kernel(BqArgs a) {
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M;
    bq_core<TER, BMAX, RPW>(
        a, a.codes, a.scales, blockIdx.x * a.rows_per_block, a.B,
        [=](int b) { return x + (size_t)b * K; }, [=](int b) { return y + (size_t)b * M; });
}

template <bool TER, int BMAX, int RPW>
__global__ __launch_bounds__(256) void moe_bq_kernel(BqArgs a) {
    const int job = blockIdx.x / a.row_blocks, rb = blockIdx.x - job * a.row_blocks;
    if (job >= *a.n_jobs) return;
    const int4 jd = a.jobs[job];
    const int e = jd.x, start = jd.y, nb = jd.z;
    const int* pids = a.pair_ids + start;
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M, topk = a.topk, xpp = a.x_per_pair;
    const size_t per_codes = (size_t)a.M * a.C, per_scales = (size_t)a.M * (a.K / 128);
    bq_core<TER, BMAX, RPW>(
        a, a.codes + (size_t)e * per_codes, a.scales + (size_t)e * per_scales, rb * a.rows_per_block, nb,
        [=](int b) {
            const int p = pids[b];
            return x + (size_t)(xpp ? p : p / topk) * K;
        },
        [=](int b) { return y + (size_t)pids[b] * M; });
}

// Group (token, slot) pairs by expert: counting sort, then jobs of <= bmax pairs.
// One workgroup; deterministic (pairs keep ascending order within an expert).
__global__ __launch_bounds__(256) void moe_group_kernel(const int* __restrict__ route, int P, int E, int bmax,
                                                        int* __restrict__ counts, int* __restrict__ offsets,
                                                        int* __restrict__ pair_ids, int4* __restrict__ jobs,
                                                        int* __restrict__ n_jobs) {
    __shared__ int s_tot[2];
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = 0;
        for (int p = 0; p < P; ++p) c += (route[p] == e);
        counts[e] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int off = 0, nj = 0;
        for (int e = 0; e < E; ++e) {
            offsets[e] = off;
            for (int s = 0; s < counts[e]; s += bmax) jobs[nj++] = make_int4(e, off + s, min(bmax, counts[e] - s), 0);
            off += counts[e];
        }
        s_tot[0] = nj;
        *n_jobs = nj;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int o = offsets[e];
        for (int p = 0; p < P; ++p)
            if (route[p] == e) pair_ids[o++] = p;
    }
}

// Dense dequant of ternary / INT4: one thread per 16-byte chunk.
template <bool TER>
__global__ __launch_bounds__(256) void dequant_bq_kernel(const uint4* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales, float* __restrict__ out,
                                                         int64_t n_chunks, int C, int K) {
    using F = Fmt<TER>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_chunks) return;
    const int64_t row = i / C, c = i - row * C;
    const float s = half_bits_to_f32(scales[row * (K / 128) + c / F::CPG]);
    const uint4 w = codes[i];
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    float4* o = reinterpret_cast<float4*>(out + row * K + c * F::WPC);
    constexpr int bits = TER ? 2 : 4, per = TER ? 16 : 8, off = TER ? 1 : 8;
    constexpr uint32_t mask = (1u << bits) - 1;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
        for (int j = 0; j < per; j += 4) {
            float4 v;
            v.x = s * (float)((int)((wv[wi] >> (bits * (j + 0))) & mask) - off);
            v.y = s * (float)((int)((wv[wi] >> (bits * (j + 1))) & mask) - off);
            v.z = s * (float)((int)((wv[wi] >> (bits * (j + 2))) & mask) - off);
            v.w = s * (float)((int)((wv[wi] >> (bits * (j + 3))) & mask) - off);
            o[(wi * per + j) / 4] = v;
        }
    }
}

}  // namespace mbd

// ------------------------------------------------------------------ host side

using namespace mbd;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

mbd_status hip_check(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MBD_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MBD_OK;
}

struct BqPlan {
    int C, G, RS, RPW, nw, rows_per_block, SC, blocks;
    size_t lds;
};

BqPlan plan_bq(bool ter, int64_t M, int64_t K, int bmax, int min_blocks) {
    BqPlan p{};
    const int wpc = ter ? 64 : 32, xq = ter ? 8 : 4;
    p.C = int(K / wpc);
    p.G = 64;
    while (p.C % p.G) p.G >>= 1;
    p.RS = 64 / p.G;
    p.RPW = bmax <= 4 ? 4 : 2;
    p.nw = 4;
    auto blocks_for = [&](int nw) {
        int rpb = nw * p.RS * p.RPW;
        return int((M + rpb - 1) / rpb);
    };
    while (p.nw > 1 && blocks_for(p.nw) < min_blocks) p.nw >>= 1;
    p.rows_per_block = p.nw * p.RS * p.RPW;
    p.blocks = blocks_for(p.nw);
    const size_t per_chunk = size_t(bmax) * (xq * 16 + 4);
    int sc = int(std::min<size_t>(p.C, (64 * 1024) / per_chunk));
    sc = std::max(p.G, (sc / p.G) * p.G);
    p.SC = sc;
    p.lds = size_t(bmax) * sc * (xq * 16 + 4);
    return p;
}

template <bool TER>
mbd_status launch_gemv_bq(const BqPlan& pl, BqArgs a, int bmax, hipStream_t st) {
    dim3 grid(pl.blocks), block(64 * pl.nw);
#define MBD_GEMV_CASE(BM, R)                                                                          \
    if (bmax == BM && pl.RPW == R) {                                                                  \
        hipLaunchKernelGGL((gemv_bq_kernel<TER, BM, R>), grid, block, pl.lds, st, a);                 \
        return hip_check("gemv launch");                                                              \
    }
    MBD_GEMV_CASE(1, 4) MBD_GEMV_CASE(2, 4) MBD_GEMV_CASE(4, 4) MBD_GEMV_CASE(8, 2) MBD_GEMV_CASE(16, 2)
#undef MBD_GEMV_CASE
    return fail(MBD_EINVAL, "no gemv variant for batch %d", bmax);
}

template <bool TER>
mbd_status launch_moe_bq(const BqPlan& pl, BqArgs a, int bmax, int grid_blocks, hipStream_t st) {
    dim3 grid(grid_blocks), block(64 * pl.nw);
#define MBD_MOE_CASE(BM, R)                                                                           \
    if (bmax == BM && pl.RPW == R) {                                                                  \
        hipLaunchKernelGGL((moe_bq_kernel<TER, BM, R>), grid, block, pl.lds, st, a);                  \
        return hip_check("moe gemv launch");                                                          \
    }
    MBD_MOE_CASE(1, 4) MBD_MOE_CASE(2, 4) MBD_MOE_CASE(4, 4) MBD_MOE_CASE(8, 2) MBD_MOE_CASE(16, 2)
#undef MBD_MOE_CASE
    return fail(MBD_EINVAL, "no expert gemv variant for batch %d", bmax);
}

int round_batch(int B) {
    int b = 1;
    while (b < B) b <<= 1;
    return b;
}

}  // namespace

// Cassandra / MX32 launchers live in cassandra.hip.
mbd_status mbd_gemv_cassandra(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st);
mbd_status mbd_gemv_mx32(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st);
mbd_status mbd_dequant_mx32(const mbd_dweights* w, float* out, hipStream_t st);

extern "C" {

mbd_status mbd_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, void* stream) {
    if (!w || !x || !y) return fail(MBD_EINVAL, "NULL argument");
    if (B < 1 || B > 16) return fail(MBD_ESHAPE, "B=%d outside [1, 16]", B);
    if (w->M < 0 || w->K < 1) return fail(MBD_ESHAPE, "bad shape M=%lld K=%lld", (long long)w->M, (long long)w->K);
    if (!aligned(x, 16) || !aligned(y, 4)) return fail(MBD_EALIGN, "x must be 16-byte and y 4-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (w->fmt == MBD_CASSANDRA) return mbd_gemv_cassandra(w, x, B, y, st);
    if (w->fmt == MBD_MX32) return mbd_gemv_mx32(w, x, B, y, st);
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128) return fail(MBD_EINVAL, "unknown format %d", w->fmt);
    if (w->K % 128) return fail(MBD_ESHAPE, "K=%lld is not a multiple of 128", (long long)w->K);
    if (w->M > INT32_MAX || w->K > INT32_MAX) return fail(MBD_ESHAPE, "shape too large");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2)) return fail(MBD_EALIGN, "codes must be 16-byte aligned");
    if (w->M == 0) return MBD_OK;
    const bool ter = w->fmt == MBD_TERNARY_B128;
    const int bmax = round_batch(B);
    BqPlan pl = plan_bq(ter, w->M, w->K, bmax, 512);
    BqArgs a{};
    a.codes = static_cast<const uint4*>(w->sec[0]);
    a.scales = static_cast<const uint16_t*>(w->sec[1]);
    a.x = x;
    a.y = y;
    a.M = int(w->M); a.K = int(w->K); a.C = pl.C; a.G = pl.G; a.SC = pl.SC; a.B = B;
    a.rows_per_block = pl.rows_per_block;
    return ter ? launch_gemv_bq<true>(pl, a, bmax, st) : launch_gemv_bq<false>(pl, a, bmax, st);
}

mbd_status mbd_dequant(const mbd_dweights* w, float* out, void* stream) {
    if (!w || !out) return fail(MBD_EINVAL, "NULL argument");
    if (!aligned(out, 16)) return fail(MBD_EALIGN, "w_out must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (w->fmt == MBD_MX32) return mbd_dequant_mx32(w, out, st);
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128)
        return fail(MBD_EINVAL, "dequant supports TERNARY, INT4 and MX32");
    if (w->M < 0 || w->K < 1 || w->K % 128) return fail(MBD_ESHAPE, "bad shape");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2)) return fail(MBD_EALIGN, "codes must be 16-byte aligned");
    if (w->M == 0) return MBD_OK;
    const bool ter = w->fmt == MBD_TERNARY_B128;
    const int C = int(w->K / (ter ? 64 : 32));
    const int64_t n = w->M * C;
    const unsigned blocks = unsigned((n + 255) / 256);
    if (ter)
        hipLaunchKernelGGL((dequant_bq_kernel<true>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint4*>(w->sec[0]), static_cast<const uint16_t*>(w->sec[1]), out, n, C, int(w->K));
    else
        hipLaunchKernelGGL((dequant_bq_kernel<false>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint4*>(w->sec[0]), static_cast<const uint16_t*>(w->sec[1]), out, n, C, int(w->K));
    return hip_check("dequant launch");
}

// Workspace: counts[E] offsets[E] n_jobs[4] pair_ids[P] jobs[max_jobs] (int4).
mbd_status mbd_moe_workspace_bytes(int64_t n_mats, int32_t T, int32_t k, uint64_t* bytes) {
    if (!bytes) return fail(MBD_EINVAL, "bytes is NULL");
    if (n_mats < 1 || n_mats > 65536 || T < 1 || k < 1 || int64_t(T) * k > (1 << 20))
        return fail(MBD_ESHAPE, "bad expert routing shape");
    const int64_t P = int64_t(T) * k;
    const int64_t max_jobs = std::min<int64_t>(n_mats, P) + P;
    uint64_t b = 0;
    b += ((uint64_t(n_mats) * 4 + 15) / 16) * 16 * 2;   // counts, offsets
    b += 16;                                             // n_jobs
    b += ((uint64_t(P) * 4 + 15) / 16) * 16;             // pair ids
    b += uint64_t(max_jobs) * 16;                        // jobs
    *bytes = b;
    return MBD_OK;
}

mbd_status mbd_moe_gemv(const mbd_dweights* w, const int32_t* route, int32_t T, int32_t k, const uint16_t* x,
                        int32_t x_per_pair, float* y, void* ws, uint64_t ws_bytes, void* stream) {
    if (!w || !route || !x || !y || !ws) return fail(MBD_EINVAL, "NULL argument");
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128)
        return fail(MBD_EINVAL, "expert GEMV supports TERNARY and INT4");
    if (w->M < 1 || w->K < 128 || w->K % 128 || w->M > INT32_MAX || w->K > INT32_MAX)
        return fail(MBD_ESHAPE, "bad expert shape");
    uint64_t need = 0;
    mbd_status s = mbd_moe_workspace_bytes(w->n_mats, T, k, &need);
    if (s != MBD_OK) return s;
    if (ws_bytes < need) return fail(MBD_EINVAL, "workspace of %llu bytes, need %llu", (unsigned long long)ws_bytes, (unsigned long long)need);
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(ws, 16) || !aligned(route, 4) ||
        !aligned(w->sec[0], 16) || !aligned(w->sec[1], 2))
        return fail(MBD_EALIGN, "misaligned pointer");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int E = int(w->n_mats), P = T * k;
    const int bmax = std::min(16, round_batch(T));
    const int64_t max_jobs = std::min<int64_t>(E, P) + (P + bmax - 1) / bmax;
    char* base = static_cast<char*>(ws);
    int* counts = reinterpret_cast<int*>(base);
    int* offsets = counts + ((E * 4 + 15) / 16) * 4;
    int* n_jobs = offsets + ((E * 4 + 15) / 16) * 4;
    int* pair_ids = n_jobs + 4;
    int4* jobs = reinterpret_cast<int4*>(pair_ids + ((P * 4 + 15) / 16) * 4);
    hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(256), 0, st, route, P, E, bmax, counts, offsets, pair_ids,
                       jobs, n_jobs);
    if ((s = hip_check("expert grouping launch")) != MBD_OK) return s;
    const bool ter = w->fmt == MBD_TERNARY_B128;
    BqPlan pl = plan_bq(ter, w->M, w->K, bmax, 64);
    BqArgs a{};
    a.codes = static_cast<const uint4*>(w->sec[0]);
    a.scales = static_cast<const uint16_t*>(w->sec[1]);
    a.x = x; a.y = y;
    a.M = int(w->M); a.K = int(w->K); a.C = pl.C; a.G = pl.G; a.SC = pl.SC; a.B = 0;
    a.rows_per_block = pl.rows_per_block;
    a.jobs = jobs; a.n_jobs = n_jobs; a.pair_ids = pair_ids;
    a.topk = k; a.x_per_pair = x_per_pair ? 1 : 0; a.row_blocks = pl.blocks;
    const int64_t grid = max_jobs * pl.blocks;
    if (grid > INT32_MAX) return fail(MBD_ESHAPE, "expert grid too large");
    return ter ? launch_moe_bq<true>(pl, a, bmax, int(grid), st) : launch_moe_bq<false>(pl, a, bmax, int(grid), st);
}

}  // extern "C"
