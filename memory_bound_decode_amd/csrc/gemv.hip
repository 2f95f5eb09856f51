// Fused dequant-GEMV / skinny GEMM for block-ternary ([Bonsai2] 1.2) and INT4
// group-128 ([GPT54-INT4] 3.2) weights on gfx950, the grouped expert GEMV, and
// the dense dequant kernels.
//
// Decode time is set by the weight bytes ([Bolt], background), so the kernel is
// built around one coalesced 16-byte load per lane per "chunk" of packed codes
// (64 ternary or 32 INT4 weights), decoded in registers into bf16 pairs and
// consumed by v_dot2c_f32_bf16.
//
// Code -> bf16: OR-ing a small field c into the mantissa of 0x4300 (bf16 128.0)
// gives the exact bf16 value 128 + c * 2^p for a field at mantissa bit p.  The
// packed layout keeps the even elements of a word in its low half and the odd
// ones in its high half, so one v_and_or_b32 (after a shift) yields the pair
// (w[2t], w[2t+1]) that lines up with the natural activation pair
// (x[2t], x[2t+1]).  A dot2 then accumulates sum (128 + c) x; the per-chunk
// constant sum_k base_k x_k ("bias", shared by every row) is subtracted once
// per chunk and the group scale applied once per chunk.  Ternary fields sit at
// mantissa bits 0, 2 and 4 after a shift by 0, 6 or 12, giving three position
// classes that are accumulated separately and combined with weights 1, 1/4,
// 1/16, so three fields come out of every shift.
//
// Work split: lanes of a wave are grouped G to a row (G = largest power of two
// <= 64 dividing the chunks per row); each lane walks its row's chunks with
// stride G and every wave covers RPW such row-steps.  A ring of PF chunks of
// 16-byte code loads stays in flight per lane.  The activations are staged once
// per workgroup in LDS (raw bf16, quad-interleaved so that neighbouring lanes
// read neighbouring 16-byte words, plus the per-chunk bias), in K slabs when
// they do not fit.  The workgroup barrier waits on LDS traffic only: a plain
// __syncthreads() would also drain every weight load in flight.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <climits>

#include "mbd_internal.h"

namespace mbd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

// Workgroup barrier that waits for this wave's LDS operations only (not for
// vector-memory loads still in flight, unlike __syncthreads()).
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool TER>
struct Fmt {
    static constexpr int WPC = TER ? 64 : 32;     // weights per 16-byte chunk
    static constexpr int XQ = WPC / 8;            // 16-byte words of activations per chunk
    static constexpr int CPG = 128 / WPC;         // chunks per scale group
};

// Stage the activations of one chunk: stage_load issues the 16-byte loads (ahead
// of the weight stream: vector-memory counters retire in issue order),
// stage_store writes them to LDS and the chunk's bias.
template <bool TER>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ xs, uint4 (&raw)[Fmt<TER>::XQ]) {
    const uint4* src = reinterpret_cast<const uint4*>(xs);
#pragma unroll
    for (int i = 0; i < Fmt<TER>::XQ; ++i) raw[i] = src[i];
}

template <bool TER>
__device__ __forceinline__ void stage_store(const uint4 (&raw)[Fmt<TER>::XQ], uint4* __restrict__ dst,
                                            int stride_q, float* __restrict__ bias) {
    float b = 0.f;
#pragma unroll
    for (int q = 0; q < Fmt<TER>::XQ; ++q) {
        dst[q * stride_q] = raw[q];
        const uint32_t v[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float pair = bf16_to_f32(v[j] & 0xFFFFu) + bf16_to_f32(v[j] >> 16);
            if constexpr (TER) {
                // pair p = 4 * (q & 1) + j of the 16-element word q >> 1: class p % 3
                const int cls = (4 * (q & 1) + j) % 3;
                b += (cls == 0 ? 129.f : (cls == 1 ? 33.f : 9.f)) * pair;
            } else {
                b += pair;
            }
        }
    }
    *bias = TER ? b : 136.f * b;
}

// (a & m) | o in one VALU op.  gfx9 VOP3 encodings cannot take a literal, so
// left to itself the compiler splits this into v_and + v_or with literals; the
// masks are kept in VGPRs instead (loaded once per kernel).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// Masks used by the unpackers, held in registers.
struct UnpackConsts {
    uint32_t magic, m2a, m2b, m2c, m4;
    __device__ __forceinline__ void init() {
        magic = 0x43004300u;   // bf16 128.0 in both halves
        m2a = 0x00030003u; m2b = 0x000C000Cu; m2c = 0x00300030u;
        m4 = 0x000F000Fu;
        // an opaque copy keeps them in VGPRs instead of being folded back into literals
        asm volatile("" : "+v"(magic), "+v"(m2a), "+v"(m2b), "+v"(m2c), "+v"(m4));
    }
};

// One 32-bit word of codes -> bf16 pairs.  INT4: pair j = (w[2j], w[2j+1]).
// Ternary: pair p = (w[2p], w[2p+1]) scaled by 1, 4 or 16 for p % 3 = 0, 1, 2.
template <bool TER>
__device__ __forceinline__ void unpack_word(const uint32_t v, uint32_t (&p)[TER ? 8 : 4], const UnpackConsts& k) {
    if constexpr (TER) {
        const uint32_t s6 = v >> 6, s12 = v >> 12;
        p[0] = and_or(v, k.m2a, k.magic);
        p[1] = and_or(v, k.m2b, k.magic);
        p[2] = and_or(v, k.m2c, k.magic);
        p[3] = and_or(s6, k.m2a, k.magic);
        p[4] = and_or(s6, k.m2b, k.magic);
        p[5] = and_or(s6, k.m2c, k.magic);
        p[6] = and_or(s12, k.m2a, k.magic);
        p[7] = and_or(s12, k.m2b, k.magic);
    } else {
        p[0] = and_or(v, k.m4, k.magic);
        p[1] = and_or(v >> 4, k.m4, k.magic);
        p[2] = and_or(v >> 8, k.m4, k.magic);
        p[3] = and_or(v >> 12, k.m4, k.magic);
    }
}

// Dot of one word's pairs with the matching activations (INT4: 4 pairs from one
// 16-byte word; ternary: 8 pairs from two), into class accumulators.
struct Acc3 {
    float a, b, c, d;   // INT4: a, b chains; ternary: a/d class 1, b class 4, c class 16
};

template <bool TER>
__device__ __forceinline__ void dot_word(const uint32_t (&pw)[TER ? 8 : 4], uint4 x0, uint4 x1, Acc3& t) {
    if constexpr (TER) {
        t.a = dot2(pw[0], x0.x, t.a);
        t.b = dot2(pw[1], x0.y, t.b);
        t.c = dot2(pw[2], x0.z, t.c);
        t.d = dot2(pw[3], x0.w, t.d);
        t.b = dot2(pw[4], x1.x, t.b);
        t.c = dot2(pw[5], x1.y, t.c);
        t.a = dot2(pw[6], x1.z, t.a);
        t.b = dot2(pw[7], x1.w, t.b);
    } else {
        (void)x1;
        t.a = dot2(pw[0], x0.x, t.a);
        t.b = dot2(pw[1], x0.y, t.b);
        t.a = dot2(pw[2], x0.z, t.a);
        t.b = dot2(pw[3], x0.w, t.b);
    }
}

template <bool TER>
__device__ __forceinline__ float finish(const Acc3& t) {
    if constexpr (TER) return (t.a + t.d) + 0.25f * t.b + 0.0625f * t.c;
    else return t.a + t.b;
}

// Full chunk (4 code words) against the staged activations of one batch row:
// xq points at quad 0 of the chunk, successive quads are `sq` uint4 apart.
template <bool TER>
__device__ __forceinline__ float chunk_dot(const uint4 w, const uint4* __restrict__ xq, int sq, float bias,
                                           const UnpackConsts& k) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    Acc3 t{-bias, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t pw[TER ? 8 : 4];
        const uint4 x0 = xq[(TER ? 2 * i : i) * sq];
        const uint4 x1 = TER ? xq[(2 * i + 1) * sq] : x0;
        unpack_word<TER>(wv[i], pw, k);
        dot_word<TER>(pw, x0, x1, t);
#if MBD_WORD_FENCE
        __builtin_amdgcn_sched_barrier(0);   // keep one word's pairs live at a time
#endif
    }
    return finish<TER>(t);
}

// Chunk against activations held in registers (one x chunk reused across rows).
template <bool TER>
__device__ __forceinline__ float chunk_dot_xreg(const uint4 w, const uint4 (&xr)[Fmt<TER>::XQ], float bias,
                                                const UnpackConsts& k) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    Acc3 t{-bias, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t pw[TER ? 8 : 4];
        unpack_word<TER>(wv[i], pw, k);
        dot_word<TER>(pw, xr[TER ? 2 * i : i], xr[TER ? 2 * i + 1 : i], t);
    }
    return finish<TER>(t);
}

struct BqArgs {
    const uint4* codes;      // [n_mats][M][C] chunks
    const uint16_t* scales;  // [n_mats][M][K/128]
    const uint16_t* x;       // bf16 activations
    float* y;                // fp32 outputs
    int M, K, C, G, SC, B;
    int gshift;              // log2(G)
    float inv_c;             // 1 / C (division-free staging job split)
    int rows_per_block;      // n_iter * tile_rows
    int tile_rows, n_iter;   // one-slab: the block walks n_iter tiles of tile_rows rows
    // expert (grouped) mode
    const int4* jobs;        // {expert, pair_start, n_pairs, 0}
    const int* n_jobs;
    const int* pair_ids;     // pairs sorted by expert: pair id = t*k + slot
    int topk, x_per_pair, row_blocks;
    const int* route;        // set: group the routes inside the kernel (n_pairs <= kFusedPairs)
    int n_pairs, n_experts;
};

// Scale loads per thread in the one-slab path (rows_per_block * K/128 <= this * threads).
template <int BMAX> struct ScaleLoads { static constexpr int N = BMAX == 1 ? 4 : 16; };

// Load-ring depth and rows per wave-step for each batch bucket.
#ifndef MBD_WORD_FENCE
#define MBD_WORD_FENCE 1
#endif
#ifndef MBD_CODES_NT
#define MBD_CODES_NT 1     // stream the packed codes with non-temporal loads
#endif
#ifndef MBD_B1_RPW
#define MBD_B1_RPW 1
#endif
#ifndef MBD_B1_PF
#define MBD_B1_PF 2
#endif
#ifndef MBD_MAX_WAVES
#define MBD_MAX_WAVES 8       // waves per workgroup (upper bound) for batch 1
#endif
#ifndef MBD_WPE
#define MBD_WPE 4             // INT4 batch-1 target waves per SIMD (caps VGPRs at 512 / MBD_WPE)
#endif
#ifndef MBD_TWPE
#define MBD_TWPE 4            // ternary batch-1 target waves per SIMD
#endif
#ifndef MBD_T1_RPW
#define MBD_T1_RPW 1
#endif
#ifndef MBD_T1_PF
#define MBD_T1_PF 2
#endif
template <bool TER, int BMAX> struct Shape;
template <> struct Shape<false, 1> { static constexpr int RPW = MBD_B1_RPW, PF = MBD_B1_PF; };
template <> struct Shape<true, 1> { static constexpr int RPW = MBD_T1_RPW, PF = MBD_T1_PF; };
#ifndef MBD_BN_WAVES
#define MBD_BN_WAVES 4        // waves per workgroup for batch > 1
#endif
// Batch 1, short rows (one or two chunks per lane): more rows per wave, one load
// each in flight per row, so that a lane still has several loads outstanding and
// the block's staged activations serve more rows.
#ifndef MBD_WIDE_RPW
#define MBD_WIDE_RPW 4
#endif
template <bool TER, int BMAX> struct WideShape { static constexpr int RPW = MBD_WIDE_RPW, PF = 1; };

// Core: rows [row_base, row_base + rows_per_block) of one matrix, nb <= BMAX batch
// rows whose activations / outputs are given by xrow(b) / yrow(b).
template <bool TER, int BMAX, int RPW, int PF, bool ONE_SLAB, class XRow, class YRow>
__device__ __forceinline__ void bq_core(const BqArgs& a, const uint4* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int row_base, int nb,
                                        XRow xrow, YRow yrow) {
    using F = Fmt<TER>;
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // G is a power of two: all per-lane index math is shifts and masks (integer
    // division would sit in front of the first load of every wave)
    const int G = a.G, gs = a.gshift, RS = 64 >> gs, C = a.C, K = a.K, M = a.M, SC = a.SC;
    const int sub = lane & (G - 1), rg = lane >> gs;
    const int row0 = row_base + wave * (RS * RPW) + rg;
    const int ngroups = K >> 7;
    const int nj = C >> gs;              // chunks per lane per row
    const int SJ = SC >> gs;             // chunks per lane per LDS slab (multiple of PF unless one slab)
    uint4* xl = lds4;                                        // [BMAX][XQ][SC]
    float* bl = reinterpret_cast<float*>(lds4 + BMAX * F::XQ * SC);   // [BMAX][SC]
    uint16_t* sl = reinterpret_cast<uint16_t*>(bl + BMAX * SC);       // one-slab: [rows_per_block][ngroups]

    const u32x4_t* rowp[RPW];
    const uint16_t* srow[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int row = min(row0 + r * RS, M - 1);
        rowp[r] = reinterpret_cast<const u32x4_t*>(codes) + (size_t)row * C + sub;
        srow[r] = scales + (size_t)row * ngroups;
    }
    const int TR = a.tile_rows, NI = ONE_SLAB ? a.n_iter : 1;

    float acc[RPW][BMAX];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[r][b] = 0.f;
    UnpackConsts kc;
    kc.init();

    uint4 w[PF][RPW];
    uint32_t s[PF][RPW];     // raw fp16 scale bits: converting at issue time would make the
                             // compiler wait for the load (and, in order, every load before it)
    // Slots past the row's last chunk load a hot, in-bounds dummy (the first
    // activation row) instead of branching: every issue is unconditional, so the
    // count of loads in flight is static and the waits stay exact.
    const u32x4_t* xdummy = reinterpret_cast<const u32x4_t*>(xrow(0)) + (lane & 15);
    auto issue = [&](int j, int p) {
        const bool real = j < nj;
        const int c = sub + G * j;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const u32x4_t* pc = real ? rowp[r] + G * j : xdummy;
#if MBD_CODES_NT
            const u32x4_t v = __builtin_nontemporal_load(pc);
#else
            const u32x4_t v = *pc;
#endif
            w[p][r] = make_uint4(v.x, v.y, v.z, v.w);
            if constexpr (!ONE_SLAB) s[p][r] = real ? srow[r][c / F::CPG] : srow[r][0];
        }
        __builtin_amdgcn_sched_barrier(0);   // each slot's loads stay adjacent, in slot order
    };
    // One-slab walk: items (tile it, chunk j) in order, the ring PF items ahead.
    int iss_it = 0, iss_j = 0;
    auto issue_next = [&](int p) {
        const bool real = iss_it < NI;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int row = min(row0 + iss_it * TR + r * RS, M - 1);
            const u32x4_t* pc = real ? reinterpret_cast<const u32x4_t*>(codes) + (size_t)row * C + sub + G * iss_j
                                     : xdummy;
#if MBD_CODES_NT
            const u32x4_t v = __builtin_nontemporal_load(pc);
#else
            const u32x4_t v = *pc;
#endif
            w[p][r] = make_uint4(v.x, v.y, v.z, v.w);
        }
        if (++iss_j == nj) {
            iss_j = 0;
            ++iss_it;
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Activation loads first, then the first PF chunks of codes, so that waiting
    // for the activations does not wait for the weight stream.
    const int scn0 = min(SC, C);
    const bool one_pass = nb * scn0 <= (int)blockDim.x;
    const int myjob = threadIdx.x;

    const int rloc0 = row0 - row_base;   // this lane's first row inside the block
    int cur_it = 0;   // one-slab: tile being computed
    auto scale = [&](int p, int r, int cc) {
        if constexpr (ONE_SLAB) return half_bits_to_f32(sl[(rloc0 + cur_it * TR + r * RS) * ngroups + (cc / F::CPG)]);
        else return half_bits_to_f32(uint16_t(s[p][r]));
    };
    // reduce across the G lanes of each row group; lane sub == 0 stores
    auto flush = [&](int it) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                float v = acc[r][b];
                for (int off = G >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
                const int row = row0 + it * TR + r * RS;
                if (sub == 0 && b < nb && row < M) yrow(b)[row] = v;
                acc[r][b] = 0.f;
            }
        }
    };
    auto compute = [&](int p, int cc) {
        if constexpr (BMAX == 1 && RPW == 1) {
            acc[0][0] = fmaf(scale(p, 0, cc), chunk_dot<TER>(w[p][0], xl + cc, SC, bl[cc], kc), acc[0][0]);
        } else if constexpr (BMAX == 1) {
            // one read of the chunk's activations from LDS serves all RPW rows
            uint4 xr[F::XQ];
#pragma unroll
            for (int q = 0; q < F::XQ; ++q) xr[q] = xl[q * SC + cc];
            const float bias = bl[cc];
#pragma unroll
            for (int r = 0; r < RPW; ++r)
                acc[r][0] = fmaf(scale(p, r, cc), chunk_dot_xreg<TER>(w[p][r], xr, bias, kc), acc[r][0]);
        } else {
            static_assert(BMAX == 1, "batches above 1 run on the matrix-core kernel");
        }
    };

    if constexpr (ONE_SLAB) {
        // every staging job fits in one pass (the launcher guarantees it)
        // job -> (batch row, chunk) without integer division: (job + 1/2) / C is
        // never within float rounding of an integer for C <= 2^12
        const bool has = myjob < nb * C;
        const int jb = BMAX == 1 ? 0 : int((float(myjob) + 0.5f) * a.inv_c);
        const int jc = myjob - jb * C;
        uint4 xraw[F::XQ];
        // threads without a job load the first chunk again (unconditional issue)
        stage_load<TER>(xrow(has ? jb : 0) + (size_t)(has ? jc : 0) * F::WPC, xraw);
        // the block's fp16 scales: rows_per_block * ngroups contiguous values
        const int nsc = a.rows_per_block * ngroups;
        const int sc_lim = min(M - row_base, a.rows_per_block) * ngroups;   // rows past M are not read
        constexpr int NSL = ScaleLoads<BMAX>::N;
        uint16_t sraw[NSL];
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
            const int e = myjob + i * (int)blockDim.x;
            sraw[i] = scales[(size_t)row_base * ngroups + ((e < nsc && e < sc_lim) ? e : 0)];
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) issue_next(p);
        __builtin_amdgcn_sched_barrier(0);          // keep the weight loads ahead of the staging waits
        if (has) stage_store<TER>(xraw, xl + (size_t)jb * F::XQ * SC + jc, SC, bl + jb * SC + jc);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
            const int e = myjob + i * (int)blockDim.x;
            if (e < nsc) sl[e] = sraw[i];
        }
        barrier_lds();
        const int total = NI * nj;
        int cj = 0;
        for (int f = 0; f < total; f += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                if (f + p < total) {
                    compute(p, sub + G * cj);
                    if (++cj == nj) {
                        flush(cur_it);
                        cj = 0;
                        ++cur_it;
                    }
                }
                issue_next(p);
            }
        }
    } else {
        (void)one_pass;
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p, p);
        for (int js = 0; js < nj; js += SJ) {
            const int c0 = js * G;
            const int scn = min(SC, C - c0);
            for (int job = threadIdx.x; job < nb * scn; job += blockDim.x) {
                const int b = job / scn, cc = job - b * scn;
                uint4 raw[F::XQ];
                stage_load<TER>(xrow(b) + (size_t)(c0 + cc) * F::WPC, raw);
                stage_store<TER>(raw, xl + (size_t)b * F::XQ * SC + cc, SC, bl + b * SC + cc);
            }
            barrier_lds();
            const int je = min(nj, js + SJ);
            for (int j = js; j < je; j += PF) {
#pragma unroll
                for (int p = 0; p < PF; ++p) {
                    const int jj = j + p;
                    if (jj < je) compute(p, sub + G * (jj - js));
                    issue(jj + PF, p);
                }
            }
            barrier_lds();
        }
    }

    if constexpr (!ONE_SLAB) flush(0);
}

#define MBD_BQ_ATTRS(TER, BMAX)                                                     \
    __launch_bounds__(BMAX == 1 ? 1024 : 64 * MBD_BN_WAVES)                         \
    __attribute__((amdgpu_waves_per_eu(BMAX == 1 ? (TER ? MBD_TWPE : MBD_WPE) : 1, 8)))

template <bool TER, int BMAX, int RPW, int PF, bool ONE_SLAB>
__global__ MBD_BQ_ATTRS(TER, BMAX) void gemv_bq_kernel(BqArgs a) {
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M;
    bq_core<TER, BMAX, RPW, PF, ONE_SLAB>(
        a, a.codes, a.scales, blockIdx.x * a.rows_per_block, a.B,
        [=](int b) { return x + (size_t)b * K; }, [=](int b) { return y + (size_t)b * M; });
}

// Routes of up to kFusedPairs (token, slot) pairs are grouped inside the expert
// kernel itself (every block redoes it: cheap only while the route is short);
// up to kSortPairs by one workgroup of moe_group_sort_kernel; longer ones by
// moe_group_kernel.
constexpr int kFusedPairs = 32;
constexpr int kSortPairs = 256;

// Workgroup-wide grouping.  Pairs are ordered by (expert, pair id): a pair's rank
// is the number of pairs with a smaller expert plus the number of earlier pairs
// with the same expert, counted by all threads over segments of the pair list and
// summed with integer LDS atomics, so the order never depends on timing.  A job
// is a run of at most bmax consecutive pairs of one expert.  On return, for each
// rank q: g[5][q] = pair id; g[4][q] = (expert << 5 | pairs) where a job starts
// at q, else -1; g[1][q] = that job's index.
template <int NP>
__device__ void moe_sort_block(const int* __restrict__ route, int P, int E, int bmax, int (&g)[6][NP]) {
    int *ge = g[0], *glo = g[1], *grk = g[2], *gcn = g[3], *ginfo = g[4], *gs = g[5];
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int i = tid; i < P; i += nt) {
        const int e = route[i];
        ge[i] = (e >= 0 && e < E) ? e : INT_MAX;   // ids out of range sort last and form no job
        glo[i] = 0;
        grk[i] = 0;
        gcn[i] = 0;
    }
    __syncthreads();
    const int S = max(1, nt / P), L = (P + S - 1) / S;
    for (int t = tid; t < P * S; t += nt) {
        const int s = t / P, i = t - s * P;
        const int ei = ge[i], u1 = min(P, (s + 1) * L);
        int lo = 0, rk = 0, cn = 0;
        for (int u = s * L; u < u1; ++u) {
            const int eu = ge[u];
            lo += eu < ei;
            cn += eu == ei;
            rk += (eu == ei) & (u < i);
        }
        if (lo) atomicAdd(&glo[i], lo);
        if (rk) atomicAdd(&grk[i], rk);
        if (cn) atomicAdd(&gcn[i], cn);
    }
    __syncthreads();
    for (int i = tid; i < P; i += nt) {
        const int r = grk[i], rank = glo[i] + r;
        gs[rank] = i;
        ginfo[rank] = (ge[i] != INT_MAX && (r & (bmax - 1)) == 0) ? (ge[i] << 5) | min(bmax, gcn[i] - r) : -1;
    }
    __syncthreads();
    for (int i = tid; i < P; i += nt) glo[i] = 0;   // reused: jobs starting before each rank
    __syncthreads();
    for (int t = tid; t < P * S; t += nt) {
        const int s = t / P, q = t - s * P;
        if (ginfo[q] < 0) continue;
        const int u1 = min(q, (s + 1) * L);
        int n = 0;
        for (int u = s * L; u < u1; ++u) n += ginfo[u] >= 0;
        if (n) atomicAdd(&glo[q], n);
    }
    __syncthreads();
}

// One workgroup groups a route of at most kSortPairs pairs into the job table.
__global__ __launch_bounds__(1024) void moe_group_sort_kernel(const int* __restrict__ route, int P, int E, int bmax,
                                                              int* __restrict__ pair_ids, int4* __restrict__ jobs,
                                                              int* __restrict__ n_jobs) {
    __shared__ int g[6][kSortPairs];
    __shared__ int total;
    if (threadIdx.x == 0) total = 0;
    moe_sort_block<kSortPairs>(route, P, E, bmax, g);
    for (int q = threadIdx.x; q < P; q += blockDim.x) {
        pair_ids[q] = g[5][q];
        const int info = g[4][q];
        if (info >= 0) {
            jobs[g[1][q]] = make_int4(info >> 5, q, info & 31, 0);
            atomicAdd(&total, 1);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *n_jobs = total;
}

template <bool TER, int BMAX, int RPW, int PF, bool ONE_SLAB>
__global__ MBD_BQ_ATTRS(TER, BMAX) void moe_bq_kernel(BqArgs a) {
    __shared__ int g[6][kFusedPairs];
    __shared__ int4 gjob;
    const int job = blockIdx.x / a.row_blocks, rb = blockIdx.x - job * a.row_blocks;
    int4 jd;
    const int* pids;
    if (a.route) {
        if (threadIdx.x == 0) gjob = make_int4(-1, 0, 0, 0);
        moe_sort_block<kFusedPairs>(a.route, a.n_pairs, a.n_experts, BMAX, g);
        for (int q = threadIdx.x; q < a.n_pairs; q += blockDim.x)
            if (g[4][q] >= 0 && g[1][q] == job) gjob = make_int4(g[4][q] >> 5, q, g[4][q] & 31, 0);
        __syncthreads();
        jd = gjob;
        if (jd.x < 0) return;
        pids = g[5] + jd.y;
    } else {
        if (job >= *a.n_jobs) return;
        jd = a.jobs[job];
        pids = a.pair_ids + jd.y;
    }
    const int e = jd.x, nb = jd.z;
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M, topk = a.topk, xpp = a.x_per_pair;
    const size_t per_codes = (size_t)a.M * a.C, per_scales = (size_t)a.M * (a.K / 128);
    bq_core<TER, BMAX, RPW, PF, ONE_SLAB>(
        a, a.codes + (size_t)e * per_codes, a.scales + (size_t)e * per_scales, rb * a.rows_per_block, nb,
        [=](int b) {
            const int p = pids[b];
            return x + (size_t)(xpp ? p : p / topk) * K;
        },
        [=](int b) { return y + (size_t)pids[b] * M; });
}

// Group (token, slot) pairs by expert: a wave per expert counts its pairs with
// ballots, one wave scans the counts into pair and job offsets, and the pairs
// are written back in ascending pair order (deterministic), with jobs of at most
// bmax pairs.  Pairs whose expert id is out of range are dropped.
constexpr int kMaxExperts = 4096;

__global__ __launch_bounds__(1024) void moe_group_kernel(const int* __restrict__ route, int P, int E, int bmax,
                                                         int* __restrict__ pair_ids, int4* __restrict__ jobs,
                                                         int* __restrict__ n_jobs) {
    __shared__ int cnt[kMaxExperts], off[kMaxExperts], joff[kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int e = wave; e < E; e += nw) {
        int c = 0;
        for (int p0 = 0; p0 < P; p0 += 64) {
            const int p = p0 + lane;
            c += __popcll(__ballot(p < P && route[p] == e));
        }
        if (lane == 0) cnt[e] = c;
    }
    __syncthreads();
    if (wave == 0) {
        int run = 0, jrun = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + lane;
            const int c = e < E ? cnt[e] : 0, jc = (c + bmax - 1) / bmax;
            int ic = c, ij = jc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int tc = __shfl_up(ic, o, 64), tj = __shfl_up(ij, o, 64);
                if (lane >= o) { ic += tc; ij += tj; }
            }
            if (e < E) { off[e] = run + ic - c; joff[e] = jrun + ij - jc; }
            run += __shfl(ic, 63, 64);
            jrun += __shfl(ij, 63, 64);
        }
        if (lane == 0) *n_jobs = jrun;
    }
    __syncthreads();
    for (int e = wave; e < E; e += nw) {
        int base = off[e];
        for (int p0 = 0; p0 < P; p0 += 64) {
            const int p = p0 + lane;
            const bool hit = p < P && route[p] == e;
            const unsigned long long m = __ballot(hit);
            if (hit) pair_ids[base + __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0))] = p;
            base += __popcll(m);
        }
        const int c = cnt[e], j0 = joff[e], o0 = off[e];
        for (int sidx = lane * bmax; sidx < c; sidx += 64 * bmax)
            jobs[j0 + sidx / bmax] = make_int4(e, o0 + sidx, min(bmax, c - sidx), 0);
    }
}

// ------------------------------------------------------------------ batch >= 2: MFMA

// Batch 2..16 is a skinny GEMM: the codes become bf16 MFMA operands directly.
// A code c of a pair-friendly word, OR'ed into the bf16 pattern of 128, is the
// exact value 128 + c = q + K0 (K0 = 136 for INT4, 129 for ternary), so
// v_mfma_f32_16x16x32_bf16 over one 128-column scale group gives
// sum (q + K0) x; subtracting K0 * sum x and applying the group's fp16 scale
// once per group gives the dequantized dot product.  A block is 32 rows (two
// 16-row tiles) by all of K; its waves take the 128-column groups round robin,
// with the next group's loads in flight while one is computed, and the waves'
// partial tiles are summed at the end.  Lane (n, q) = (lane % 16, lane / 16)
// holds columns [32q, 32q + 32) of the group for weight row n of each tile and
// for batch row n; MFMA sub-step s uses columns 32q + 8s .. + 8 on both operands,
// so every k slot sees the same column on A and B.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int MQ_TILES = 2;
constexpr int MQ_MAXW = 16;
#ifndef MBD_MQ_GPW
#define MBD_MQ_GPW 4          // scale groups per wave (sets the waves per block)
#endif

inline int mq_waves(int64_t K) {
    return int(std::max<int64_t>(1, std::min<int64_t>(MQ_MAXW, (K / 128) / MBD_MQ_GPW)));
}

struct MqGroup {
    uint4 code[MQ_TILES];          // INT4: 4 words (32 codes); ternary: .x, .y (32 codes)
    uint32_t sc[MQ_TILES][2];      // fp16 scales of the lane's 4 output rows, packed in pairs
    uint4 xv[4];                   // 32 activations of batch row n
};

struct MqArgs {
    const uint8_t* codes;   // [n_mats][M][K * bits / 8]
    const uint16_t* scales; // [n_mats][M][K / 128]
    const uint16_t* x;
    float* y;
    int M, K;
    // expert mode
    const int4* jobs;
    const int* n_jobs;
    const int* pair_ids;
    const int* route;       // grouped in the kernel when set (at most kFusedPairs pairs)
    int n_pairs, n_experts, topk, x_per_pair, row_blocks, B;
};

template <bool TER>
__device__ __forceinline__ uint4 mq_unpack(const uint4 c, int s) {
    uint32_t o[4];
    if constexpr (TER) {
        const uint32_t w = (s < 2) ? c.x : c.y;        // 16 codes per word
        const int p0 = 4 * (s & 1);
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = ((w >> (2 * (p0 + p))) & 0x00030003u) | 0x43004300u;
    } else {
        const uint32_t w = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;   // 8 codes per word
#pragma unroll
        for (int p = 0; p < 4; ++p) o[p] = ((w >> (4 * p)) & 0x000F000Fu) | 0x43004300u;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Rows [row_base, row_base + 32) of one matrix; nb <= 16 batch rows whose
// activations / outputs are xrow(b) / yrow(b).
template <bool TER, class XRow, class YRow>
__device__ __forceinline__ void mq_core(const MqArgs& a, const uint8_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int row_base, int nb, XRow xrow,
                                        YRow yrow) {
    constexpr float K0 = TER ? 129.f : 136.f;
    constexpr int BPR = TER ? 4 : 2;                       // elements per byte
    __shared__ float red[MQ_MAXW][MQ_TILES][64][4];
    const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, q = lane >> 4;
    const int K = a.K, M = a.M, ngroups = K >> 7;
    const size_t row_bytes = size_t(K) / BPR;
    int rowc[MQ_TILES];                                    // weight rows this lane loads (clamped)
    int orow[MQ_TILES];                                    // first output row of this lane in each tile
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t) {
        rowc[t] = min(row_base + 16 * t + n, M - 1);
        orow[t] = row_base + 16 * t + 4 * q;
    }
    const bool xlive = n < nb;
    const uint16_t* xr = xrow(xlive ? n : 0);
    auto load = [&](int g, MqGroup& d) {
#pragma unroll
        for (int t = 0; t < MQ_TILES; ++t) {
            const uint8_t* cp = codes + size_t(rowc[t]) * row_bytes + size_t(g) * (128 / BPR) + q * (32 / BPR);
            if constexpr (TER) {
                const uint2 v = *reinterpret_cast<const uint2*>(cp);
                d.code[t] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                d.code[t] = *reinterpret_cast<const uint4*>(cp);
            }
            uint32_t sv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sv[j] = scales[size_t(min(orow[t] + j, M - 1)) * ngroups + g];
            d.sc[t][0] = sv[0] | (sv[1] << 16);
            d.sc[t][1] = sv[2] | (sv[3] << 16);
        }
        const uint4* px = reinterpret_cast<const uint4*>(xr + size_t(g) * 128 + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) d.xv[i] = px[i];
    };
    f32x4_t acc[MQ_TILES];
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Lanes n >= nb carry batch row 0's activations: B column n only reaches
    // output column n, which is not stored.
    auto compute = [&](const MqGroup& d) {
        const uint4* xb = d.xv;
        float sx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sx = dot2(xb[i].x, 0x3F803F80u, sx);
            sx = dot2(xb[i].y, 0x3F803F80u, sx);
            sx = dot2(xb[i].z, 0x3F803F80u, sx);
            sx = dot2(xb[i].w, 0x3F803F80u, sx);
        }
        sx += __shfl_xor(sx, 16, 64);
        sx += __shfl_xor(sx, 32, 64);
        const float bias = K0 * sx;
#pragma unroll
        for (int t = 0; t < MQ_TILES; ++t) {
            f32x4_t cg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, mq_unpack<TER>(d.code[t], s)),
                                                             __builtin_bit_cast(bf16x8_t, xb[s]), cg, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sc = half_bits_to_f32(uint16_t(d.sc[t][j >> 1] >> (16 * (j & 1))));
                acc[t][j] = fmaf(sc, cg[j] - bias, acc[t][j]);
            }
        }
    };
    // two group buffers, so a buffer is never copied while its loads are in flight
    MqGroup g0, g1;
    int g = wave;
    if (g < ngroups) load(g, g0);
    for (; g < ngroups; g += 2 * nw) {
        const int gn = g + nw;
        load(min(gn, ngroups - 1), g1);
        compute(g0);
        load(min(gn + nw, ngroups - 1), g0);
        if (gn < ngroups) compute(g1);
    }
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][t][lane][j] = acc[t][j];
    __syncthreads();
    // C[row = 4q + j][col = n]: wave t (or wave t - nw, ... when there are fewer
    // waves than tiles) sums tile t over the waves
    for (int t = wave; t < MQ_TILES; t += nw) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] += red[w][t][lane][j];
        if (n < nb) {
            float* yr = yrow(n);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = row_base + 16 * t + 4 * q + j;
                if (r < M) yr[r] = s4[j];
            }
        }
    }
}

template <bool TER>
__global__ __launch_bounds__(64 * MQ_MAXW) void gemv_mq_kernel(MqArgs a) {
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M;
    mq_core<TER>(a, a.codes, a.scales, blockIdx.x * 32, a.B, [=](int b) { return x + (size_t)b * K; },
                 [=](int b) { return y + (size_t)b * M; });
}

template <bool TER>
__global__ __launch_bounds__(64 * MQ_MAXW) void moe_mq_kernel(MqArgs a) {
    __shared__ int g[6][kFusedPairs];
    __shared__ int4 gjob;
    const int job = blockIdx.x / a.row_blocks, rb = blockIdx.x - job * a.row_blocks;
    int4 jd;
    const int* pids;
    if (a.route) {
        if (threadIdx.x == 0) gjob = make_int4(-1, 0, 0, 0);
        moe_sort_block<kFusedPairs>(a.route, a.n_pairs, a.n_experts, 16, g);
        for (int qq = threadIdx.x; qq < a.n_pairs; qq += blockDim.x)
            if (g[4][qq] >= 0 && g[1][qq] == job) gjob = make_int4(g[4][qq] >> 5, qq, g[4][qq] & 31, 0);
        __syncthreads();
        jd = gjob;
        if (jd.x < 0) return;
        pids = g[5] + jd.y;
    } else {
        if (job >= *a.n_jobs) return;
        jd = a.jobs[job];
        pids = a.pair_ids + jd.y;
    }
    const int e = jd.x, nb = jd.z;
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M, topk = a.topk, xpp = a.x_per_pair;
    const size_t per_codes = (size_t)M * K / (TER ? 4 : 2), per_scales = (size_t)M * (K / 128);
    mq_core<TER>(
        a, a.codes + (size_t)e * per_codes, a.scales + (size_t)e * per_scales, rb * 32, nb,
        [=](int b) {
            const int p = pids[b];
            return x + (size_t)(xpp ? p : p / topk) * K;
        },
        [=](int b) { return y + (size_t)pids[b] * M; });
}

// Dense dequant of ternary / INT4: one thread per 16-byte chunk.  Element t of a
// word sits at bit (bits * (t / 2)) + (t odd ? 16 : 0).
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
            float e[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = j + u;
                const int sh = bits * (t >> 1) + ((t & 1) ? 16 : 0);
                e[u] = s * (float)((int)((wv[wi] >> sh) & mask) - off);
            }
            o[(wi * per + j) / 4] = make_float4(e[0], e[1], e[2], e[3]);
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

constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950

struct BqPlan {
    int C, G, RS, RPW, PF, nw, rows_per_block, SC, blocks;
    int tile_rows, n_iter;
    size_t lds;
    bool one_slab;   // all activations staged at once, one staging job per thread at most
    bool wide;       // short rows: the many-rows-per-wave shape
};

#ifndef MBD_MAX_TILES
#define MBD_MAX_TILES 2       // row tiles one workgroup walks at most
#endif
#ifndef MBD_MOE_BLOCKS
#define MBD_MOE_BLOCKS 512
#endif

// min_blocks: shrink the workgroup until the grid has at least this many blocks.
// n_mats: matrices the call covers (the grid is n_mats times the plan's blocks).
// In the single-slab kernel a block then walks several row tiles when there are
// more tiles than about one round of resident workgroups, so its staged
// activations serve more rows.
BqPlan plan_bq(bool ter, int64_t M, int64_t K, int bmax, int min_blocks, int prefer_nw = MBD_MAX_WAVES,
               int64_t n_mats = 1) {
    BqPlan p{};
    const int wpc = ter ? 64 : 32, xq = ter ? 8 : 4;   // uint4 of activations per chunk
    p.C = int(K / wpc);
    p.G = 64;
    while (p.C % p.G) p.G >>= 1;
    p.RS = 64 / p.G;
    p.wide = bmax == 1 && p.C / p.G <= 2 && M * n_mats * p.G >= int64_t(2048) * 64 * MBD_WIDE_RPW;
    if (p.wide) {
        p.RPW = MBD_WIDE_RPW; p.PF = 1;
    } else {
        p.RPW = ter ? Shape<true, 1>::RPW : Shape<false, 1>::RPW;
        p.PF = ter ? Shape<true, 1>::PF : Shape<false, 1>::PF;
    }
    p.nw = bmax == 1 ? prefer_nw : MBD_BN_WAVES;
    // batch 1: grow the workgroup (up to 16 waves) when that lets every staging
    // job fit in one pass, i.e. the single-slab kernel
    if (bmax == 1 && p.C > 64 * p.nw && p.C <= 64 * 16) p.nw = 16;
    auto tiles_for = [&](int nw) {
        const int64_t tr = int64_t(nw) * p.RS * p.RPW;
        return (M + tr - 1) / tr;
    };
    while (p.nw > 1 && tiles_for(p.nw) < min_blocks) p.nw >>= 1;
    p.tile_rows = p.nw * p.RS * p.RPW;
    const int64_t tiles = tiles_for(p.nw);
    const size_t per_chunk = size_t(bmax) * (xq * 16 + 4);
    int sc = int(std::min<size_t>(p.C, (64 * 1024) / per_chunk));
    if (sc < p.C) {
        const int unit = p.G * p.PF;   // a partial slab must keep the load ring aligned
        sc = std::max(unit, (sc / unit) * unit);
    }
    p.SC = sc;
    p.lds = size_t(bmax) * sc * (xq * 16 + 4);   // <= 160 KiB: checked by the caller
    const int64_t ngroups = K / 128;
    const int64_t scale_cap = int64_t(bmax == 1 ? ScaleLoads<1>::N : ScaleLoads<2>::N) * 64 * p.nw;
    p.one_slab = sc >= p.C && int64_t(bmax) * p.C <= int64_t(64) * p.nw && p.C <= 4096 &&
                 int64_t(p.tile_rows) * ngroups <= scale_cap;
    p.n_iter = 1;
    if (p.one_slab) {
        // about one round of resident workgroups (waves per CU: 8 per SIMD at
        // batch 1, 4 above), at least min_blocks
        const int64_t waves_per_cu = bmax == 1 ? 32 : 16;
        const int64_t round = std::max<int64_t>(min_blocks, 256 * waves_per_cu / p.nw / std::max<int64_t>(1, n_mats));
        int64_t it = std::max<int64_t>(1, tiles / round);
        it = std::min<int64_t>(it, scale_cap / (int64_t(p.tile_rows) * ngroups));
        it = std::min<int64_t>(it, MBD_MAX_TILES);
        p.n_iter = int(std::max<int64_t>(1, it));
    }
    p.rows_per_block = p.n_iter * p.tile_rows;
    p.blocks = int((M + p.rows_per_block - 1) / p.rows_per_block);
    if (p.one_slab) p.lds += size_t(p.rows_per_block) * ngroups * 2;     // staged scales
    return p;
}

// Batch-1 kernel variants: (rows per wave, ring depth) x single/multi slab.
#define MBD_BQ_DISPATCH(KERNEL, TER, pl, bmax, grid, st, a, what)                                        \
    do {                                                                                                  \
        dim3 blk_(64 * (pl).nw);                                                                          \
        auto go_ = [&](auto kern) {                                                                       \
            hipLaunchKernelGGL(kern, dim3(grid), blk_, (pl).lds, st, a);                                  \
            return hip_check(what);                                                                       \
        };                                                                                                \
        const bool os_ = (pl).one_slab;                                                                   \
        if ((pl).wide) {                                                                                  \
            constexpr int WR = WideShape<TER, 1>::RPW;                                                    \
            return os_ ? go_(KERNEL<TER, 1, WR, 1, true>) : go_(KERNEL<TER, 1, WR, 1, false>);             \
        } else if (bmax == 1) {                                                                           \
            constexpr int R1 = Shape<TER, 1>::RPW, P1 = Shape<TER, 1>::PF;                                \
            return os_ ? go_(KERNEL<TER, 1, R1, P1, true>) : go_(KERNEL<TER, 1, R1, P1, false>);           \
        }                                                                                                 \
        return fail(MBD_EINVAL, "no kernel variant for batch %d", bmax);                                  \
    } while (0)

template <bool TER>
mbd_status launch_gemv_bq(const BqPlan& pl, BqArgs a, int bmax, hipStream_t st) {
    MBD_BQ_DISPATCH(gemv_bq_kernel, TER, pl, bmax, pl.blocks, st, a, "gemv launch");
}

template <bool TER>
mbd_status launch_moe_bq(const BqPlan& pl, BqArgs a, int bmax, int grid_blocks, hipStream_t st) {
    MBD_BQ_DISPATCH(moe_bq_kernel, TER, pl, bmax, grid_blocks, st, a, "expert gemv launch");
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
    if (B >= 2) {
        // skinny GEMM on the matrix cores
        MqArgs m{};
        m.codes = static_cast<const uint8_t*>(w->sec[0]);
        m.scales = static_cast<const uint16_t*>(w->sec[1]);
        m.x = x; m.y = y; m.M = int(w->M); m.K = int(w->K); m.B = B;
        const int nw = mq_waves(w->K);
        const unsigned blocks = unsigned((w->M + 31) / 32);
        if (ter) hipLaunchKernelGGL(gemv_mq_kernel<true>, dim3(blocks), dim3(64 * nw), 0, st, m);
        else hipLaunchKernelGGL(gemv_mq_kernel<false>, dim3(blocks), dim3(64 * nw), 0, st, m);
        return hip_check("batched gemv launch");
    }
    const int bmax = round_batch(B);
    BqPlan pl = plan_bq(ter, w->M, w->K, bmax, 512);
    if (pl.lds > kMaxLds) return fail(MBD_ESHAPE, "activation slab needs %zu bytes of LDS", pl.lds);
    BqArgs a{};
    a.codes = static_cast<const uint4*>(w->sec[0]);
    a.scales = static_cast<const uint16_t*>(w->sec[1]);
    a.x = x;
    a.y = y;
    a.M = int(w->M); a.K = int(w->K); a.C = pl.C; a.G = pl.G; a.SC = pl.SC; a.B = B;
    a.gshift = __builtin_ctz(unsigned(pl.G)); a.inv_c = 1.0f / float(pl.C);
    a.rows_per_block = pl.rows_per_block; a.tile_rows = pl.tile_rows; a.n_iter = pl.n_iter;
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

// Workspace: n_jobs[4] pair_ids[P] (padded to 16 B) jobs[min(E, P) + P] (int4).
mbd_status mbd_moe_workspace_bytes(int64_t n_mats, int32_t T, int32_t k, uint64_t* bytes) {
    if (!bytes) return fail(MBD_EINVAL, "bytes is NULL");
    if (n_mats < 1 || n_mats > kMaxExperts || T < 1 || k < 1 || int64_t(T) * k > (1 << 20))
        return fail(MBD_ESHAPE, "bad expert routing shape (at most %d experts)", kMaxExperts);
    const int64_t P = int64_t(T) * k;
    const int64_t max_jobs = std::min<int64_t>(n_mats, P) + P;
    *bytes = 16 + ((uint64_t(P) * 4 + 15) / 16) * 16 + uint64_t(max_jobs) * 16;
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
    // one token: the batch-1 kernel; more: jobs of up to 16 pairs on the matrix cores
    const bool mq = T >= 2;
    const int bmax = mq ? 16 : 1;
    // sum over experts of ceil(pairs / bmax) <= D + (P - D) / bmax, D = distinct experts
    const int64_t D = std::min<int64_t>(E, P), max_jobs = D + (P - D) / bmax;
    const bool fused = P <= kFusedPairs;
    int* n_jobs = static_cast<int*>(ws);
    int* pair_ids = n_jobs + 4;
    int4* jobs = reinterpret_cast<int4*>(pair_ids + ((P * 4 + 15) / 16) * 4);
    if (!fused) {
        if (P <= kSortPairs)
            hipLaunchKernelGGL(moe_group_sort_kernel, dim3(1), dim3(1024), 0, st, route, P, E, bmax, pair_ids, jobs, n_jobs);
        else
            hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(1024), 0, st, route, P, E, bmax, pair_ids, jobs, n_jobs);
        if ((s = hip_check("expert grouping launch")) != MBD_OK) return s;
    }
    if (mq) {
        MqArgs m{};
        m.codes = static_cast<const uint8_t*>(w->sec[0]);
        m.scales = static_cast<const uint16_t*>(w->sec[1]);
        m.x = x; m.y = y; m.M = int(w->M); m.K = int(w->K);
        m.jobs = jobs; m.n_jobs = n_jobs; m.pair_ids = pair_ids;
        m.route = fused ? route : nullptr;
        m.n_pairs = P; m.n_experts = E; m.topk = k; m.x_per_pair = x_per_pair ? 1 : 0;
        m.row_blocks = int((w->M + 31) / 32);
        const int nw = mq_waves(w->K);
        const int64_t grid = max_jobs * m.row_blocks;
        if (grid > INT32_MAX) return fail(MBD_ESHAPE, "expert grid too large");
        if (w->fmt == MBD_TERNARY_B128)
            hipLaunchKernelGGL(moe_mq_kernel<true>, dim3(unsigned(grid)), dim3(64 * nw), 0, st, m);
        else
            hipLaunchKernelGGL(moe_mq_kernel<false>, dim3(unsigned(grid)), dim3(64 * nw), 0, st, m);
        return hip_check("expert gemv launch");
    }
    const bool ter = w->fmt == MBD_TERNARY_B128;
    // about MBD_MOE_BLOCKS workgroups over the whole call
    const int min_blocks = int(std::max<int64_t>(1, MBD_MOE_BLOCKS / std::max<int64_t>(1, D)));
    BqPlan pl = plan_bq(ter, w->M, w->K, bmax, min_blocks, 16, D);
    if (pl.lds + sizeof(int) * 6 * kFusedPairs + 16 > kMaxLds)
        return fail(MBD_ESHAPE, "activation slab needs %zu bytes of LDS", pl.lds);
    BqArgs a{};
    a.codes = static_cast<const uint4*>(w->sec[0]);
    a.scales = static_cast<const uint16_t*>(w->sec[1]);
    a.x = x; a.y = y;
    a.M = int(w->M); a.K = int(w->K); a.C = pl.C; a.G = pl.G; a.SC = pl.SC; a.B = 0;
    a.gshift = __builtin_ctz(unsigned(pl.G)); a.inv_c = 1.0f / float(pl.C);
    a.rows_per_block = pl.rows_per_block; a.tile_rows = pl.tile_rows; a.n_iter = pl.n_iter;
    a.jobs = jobs; a.n_jobs = n_jobs; a.pair_ids = pair_ids;
    a.topk = k; a.x_per_pair = x_per_pair ? 1 : 0; a.row_blocks = pl.blocks;
    a.route = fused ? route : nullptr;
    a.n_pairs = P; a.n_experts = E;
    const int64_t grid = max_jobs * pl.blocks;
    if (grid > INT32_MAX) return fail(MBD_ESHAPE, "expert grid too large");
    return ter ? launch_moe_bq<true>(pl, a, bmax, int(grid), st) : launch_moe_bq<false>(pl, a, bmax, int(grid), st);
}

}  // extern "C"
