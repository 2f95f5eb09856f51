// Fused dequant-GEMV / skinny GEMM for block-ternary ([Bonsai2] 1.2) and INT4
// group-128 ([GPT54-INT4] 3.2) weights on gfx950, the grouped expert GEMV, and
// the dense dequant kernel.
//
// Decode time is set by the weight bytes ([Bolt], background), and every batch
// size runs on v_mfma_f32_16x16x32_bf16.  Code -> bf16: OR-ing a small field c
// into the mantissa of 0x4300 (bf16 128.0) gives the exact bf16 value
// 128 + c * 2^p for a field at mantissa bit p.  A word keeps its even elements in
// the low half and the odd ones in the high half, so one v_and_or_b32 (after a
// shift) yields an element pair, and four pairs are one lane's MFMA A operand.
// The constant part of the code values ("bias": K0 sum x over a scale group) is
// removed once per group, and the group's fp16 scale applied once per group.
// On a 16-lane SIMD a wave64 VALU op takes 4 clocks, and these kernels are bound
// by VALU issue and latency: a dot2 formulation would add one op per weight pair
// to the unpack (16 wave ops per KB of INT4 codes, 32 per KB of ternary, on top
// of about 60 and 90), while the matrix cores are a separate pipe, so even batch
// 1 uses them and leaves only the unpack on the VALU.
//
// Codes are stored tile-interleaved (include/mbd.h): for each 16-row tile and
// 128-column group (ternary: pair of groups), lane l = 16 kq + m of a wave finds
// the 16 bytes of tile row m, columns 32kq .. +32, at l * 16.  One load
// instruction then reads 1 KB contiguous and lands in A-operand order (lane l
// holds row l % 16, k slots 8 (l / 16) .. +8 of each MFMA step).
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "hip_check.h"
#include "mbd_internal.h"

namespace mbd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

// (a & m) | o, one v_and_or_b32 when m and o sit in VGPRs (UnpackConsts): gfx9
// VOP3 encodings cannot take a literal, so with constant masks the compiler
// splits it into v_and + v_or.  Plain code, not inline asm: the compiler's
// hazard tracking does not see an asm block as a VALU write, and an MFMA that
// reads its result as an A operand too soon reads a stale register.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// Masks used by the unpackers, held in registers.
struct UnpackConsts {
    uint32_t magic, mg1, mg2, m2a, m2b, m2c, m4;
    __device__ __forceinline__ void init() {
        magic = 0x43004300u;   // bf16 128.0 in both halves
        mg1 = 0x42004200u;     // bf16 32.0
        mg2 = 0x41004100u;     // bf16 8.0
        m2a = 0x00030003u; m2b = 0x000C000Cu; m2c = 0x00300030u;
        m4 = 0x000F000Fu;
        // an opaque copy keeps them in VGPRs instead of being folded back into literals
        asm volatile("" : "+v"(magic), "+v"(mg1), "+v"(mg2), "+v"(m2a), "+v"(m2b), "+v"(m2c), "+v"(m4));
    }
};

// A operand of MFMA step s (0..3) from the words of one scale group: INT4 words
// x, y, z, w (step s = word s, 8 codes), ternary words x, y (step s = half s % 2
// of word s / 2).  Ternary pair p of a word is read at mantissa bits 2 (p % 3)
// after a shift by 6 (p / 3), under an exponent that makes the field's unit 1:
// class p % 3 = 0, 1, 2 gives 128 + c, 32 + c, 8 + c (bf16 128, 32, 8 with the
// field at mantissa bits 0, 2, 4), so the activations stay as they are and only
// the constant part differs by class: 129, 33, 9 times x for q = c - 1.
template <bool TER>
__device__ __forceinline__ bf16x8_t code_operand(const uint4 c, int s, const UnpackConsts& k) {
    uint32_t o[4];
    if constexpr (TER) {
        const uint32_t v = (s < 2) ? c.x : c.y;
        const uint32_t s6 = v >> 6, s12 = v >> 12;
        if ((s & 1) == 0) {
            o[0] = and_or(v, k.m2a, k.magic);
            o[1] = and_or(v, k.m2b, k.mg1);
            o[2] = and_or(v, k.m2c, k.mg2);
            o[3] = and_or(s6, k.m2a, k.magic);
        } else {
            o[0] = and_or(s6, k.m2b, k.mg1);
            o[1] = and_or(s6, k.m2c, k.mg2);
            o[2] = and_or(s12, k.m2a, k.magic);
            o[3] = and_or(s12, k.m2b, k.mg1);
        }
    } else {
        const uint32_t v = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
        o[0] = and_or(v, k.m4, k.magic);
        o[1] = and_or(v >> 4, k.m4, k.magic);
        o[2] = and_or(v >> 8, k.m4, k.magic);
        o[3] = and_or(v >> 12, k.m4, k.magic);
    }
    return __builtin_bit_cast(bf16x8_t, make_uint4(o[0], o[1], o[2], o[3]));
}

// Tile-interleaved addressing.  Tile t of a matrix holds rows [16t, 16t + R),
// R = min(16, M - 16t), and starts at byte 16t * row_bytes.  Item i of a tile
// (INT4: group i; ternary: group pair i) starts at i * 64 R, and unit (m, kq) of a
// full item at (kq R + m) * 16; the odd last ternary group is an item of 8-byte
// units at (kq R + m) * 8.
__device__ __forceinline__ uint32_t tile_unit(int m, int kq, int R) { return uint32_t(kq * R + min(m, R - 1)); }

__device__ __forceinline__ float dpp_quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    return v;
}

// Routes of up to kFusedPairs (token, slot) pairs are grouped inside the expert
// kernel itself (every block redoes it: cheap only while the route is short);
// up to kSortPairs by one workgroup of moe_group_sort_kernel; longer ones by
// moe_group_kernel.
constexpr int kFusedPairs = 32;
constexpr int kSortPairs = 256;
// Routes of at most 16 tokens and kExpertPairs pairs over few enough experts run
// one block row per expert, each block listing its expert's pairs itself (no
// grouping at all).
constexpr int kExpertPairs = 256;

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

// ------------------------------------------------------------------ batch 1..4
//
// Few activation rows (batch 1..4).  Column n
// of B holds activation row n (columns past the rows in use repeat the last row
// and are not stored), so one MFMA chain serves every row; with one row only
// column 0 is used, but the multiply-adds still leave the VALU, and the unpack,
// the MFMAs and the scale multiply-adds cost the same for one row as for four.
// A block owns one 16-row tile; its waves take contiguous runs of items (INT4:
// groups; ternary: group pairs), in rounds when K is long.  Each wave stages
// what its own items need in its own LDS area, so no wave waits for another
// before computing:
//   rec[g][kq][t]  80 bytes: activations of row t, columns [128g + 32kq, +32),
//                  and the group's -bias of row t four times, the initial C
//                  values of the group's MFMA chain;
//   sct[g][16]     the tile's fp16 scales of group g.
// bias = sum over the group of (code value - q) x: 136 sum x for INT4 (code value
// q + 136), sum (1 + 128 / 4^class) x for ternary (code value 128 / 4^class + q + 1,
// class 0, 1, 2: 129, 33, 9).  The waves' partial rows meet in LDS at the end.
constexpr int BN_REC = 80;

// Groups one wave stages per round: at most 8, and at most 16 / NB so that the
// staging jobs (16 per group and row) fit four passes of 64 lanes.  INT4 with 4
// rows takes 2: two staging passes keep it at <= 64 VGPRs, so two 16-wave blocks
// share a CU (batch 4, 8192^2: 9.7 us against 11.0 us with 4 groups); ternary,
// whose items are group pairs, keeps 4.
constexpr int bn_max_groups(int NB, bool ter) { return NB >= 4 ? (ter ? 4 : 2) : 8; }
constexpr int bn_group_lds(int NB) { return 4 * NB * BN_REC + 32; }

struct BnArgs {
    const uint8_t* codes;   // tile-interleaved codes of n_mats matrices
    const uint16_t* scales; // [n_mats][M][K / 128]
    const uint32_t* slabs;  // skip format: [tiles][K / 128] stored-row mask | in-tile offset << 16
    const uint32_t* tile_base;   // skip format: [tiles + 1] blocks stored before each tile
    const uint16_t* x;
    float* y;
    int M, K;
    int ipw;                // items per wave per round
    int tiles;              // 16-row tiles per matrix
    int B;                  // activation rows (plain GEMV)
    // expert mode, one token: pair p = slot p, expert route[p]
    const int* route;
    int n_experts, topk, x_per_pair;
};

// Code loads: non-temporal (NT) where a dense matrix streams once, plain where
// that measured faster (expert matrices: T = 1 11.30 -> 10.90 us, T = 8 56.5 ->
// 54.2 us; the 32-row kernel's ternary pairs, whose two 8-byte halves of a unit
// load one group apart: 8192 x 28672 B = 8 26.5 -> 25.0 us).  On the dense
// few-row kernel plain loads were slower (INT4 8192 x 28672 21.1 -> 22.6 us).
template <bool NT, class T>
__device__ __forceinline__ T code_load(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Tile `tile` of one matrix against nb <= NB activation rows xrow(t); output row
// n of the tile goes to yrow(n).  XU: staging passes of 64 lanes.  SK (ternary
// only): the skip format.  An item is still a pair of block columns; lane (m, kq)
// finds its 8 bytes of each through the column's slab word, or, when tile row m's
// block is all-zero and not stored, uses code 1 (q = 0) in every field.  NTL:
// non-temporal code loads.
template <bool TER, bool SK, int PF, int NB, int XU, bool NTL, class XRow, class YRow>
__device__ __forceinline__ void bn_core(const BnArgs& a, const uint8_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int nb, XRow xrow, YRow yrow,
                                        int tile) {
    static_assert(TER || !SK, "the skip format is ternary");
    constexpr int IG = TER ? 2 : 1;                  // groups per item
    constexpr int GLDS = bn_group_lds(NB);
    extern __shared__ uint4 lds4[];
    char* lds = reinterpret_cast<char*>(lds4);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int M = a.M, K = a.K, ngroups = K >> 7;
    const int n_items = IG == 2 ? (ngroups + 1) >> 1 : ngroups;
    const int n_full = TER ? ngroups >> 1 : ngroups;          // items of 16-byte units
    const int m = lane & 15, kq = lane >> 4;
    const int row0 = tile * 16, R = min(16, M - row0);
    const uint8_t* tcodes = SK ? codes + size_t(a.tile_base[tile]) * 32
                               : codes + size_t(row0) * (size_t(K) / (TER ? 4 : 2));
    // skip format: lane l holds the slab word of the round's block column l (sw),
    // the next round's loaded one round ahead (swn)
    const uint32_t* tsl = SK ? a.slabs + size_t(tile) * ngroups : nullptr;
    uint32_t swn = 0;
    if constexpr (SK) swn = tsl[min(IG * wave * a.ipw + lane, ngroups - 1)];
    const uint32_t unit = tile_unit(m, kq, R);
    const int wg = a.ipw * IG;                                // groups a wave stages per round
    char* rec = lds + wave * wg * GLDS;                       // [wg][4][NB][BN_REC]
    uint16_t* sct = reinterpret_cast<uint16_t*>(rec + wg * 4 * NB * BN_REC);   // [wg][16]
    float* red = reinterpret_cast<float*>(lds + nw * wg * GLDS);              // [nw][NB][16]
    const int boff = (kq * NB + min(m, nb - 1)) * BN_REC;    // B column m reads row min(m, nb - 1)
    UnpackConsts kc;
    kc.init();
    float acc[4] = {0.f, 0.f, 0.f, 0.f};

    for (int rb = 0; rb < n_items; rb += nw * a.ipw) {
        const int it0 = rb + wave * a.ipw;
        const int n = min(a.ipw, n_items - it0);
        if (n <= 0) continue;
        const int g0 = it0 * IG, ng = min(n * IG, ngroups - g0);
        const int njobs = 16 * ng * nb;
        const uint32_t sw = swn;
        if constexpr (SK) swn = tsl[min(IG * (rb + nw * a.ipw + wave * a.ipw) + lane, ngroups - 1)];

        // Staging loads first (vector-memory counters retire in issue order, so the
        // staging waits do not wait for the code stream).  Job j = (row t, local
        // group gl, quarter, slice), j = (t ng + gl) 16 + 4 quarter + slice: 8
        // activations, columns 32 quarter + 8 slice .. +8 of the group.  Lanes past
        // the last job redo jobs of the last (row, group), the same values into the
        // same slots.  The same passes load the scale entries e = (local group
        // e / 16, tile row e % 16).
        // at most 8 groups x 16 rows of scales: two passes
        constexpr int SU = XU < 2 ? XU : 2;
        const float inv_ng = NB == 1 ? 0.f : 1.f / float(ng);
        (void)inv_ng;
        uint4 xv[XU];
        int jr[XU], se[SU];                  // jr: record byte offset * 4 + slice
        uint32_t sv[SU];
#pragma unroll
        for (int u = 0; u < XU; ++u) {
            const int j = min(lane + 64 * u, njobs - 16 + (lane & 15));
            if constexpr (NB == 1) {
                // job j = 16 gl + 4 q + sl: columns 8 j .. +8 of the round's groups,
                // record gl 4 + q (80 bytes each), slice sl
                jr[u] = (j >> 2) * (BN_REC * 4) + (j & 3);
                xv[u] = *reinterpret_cast<const uint4*>(xrow(0) + (g0 * 128 + 8 * j));
            } else {
                const int gt = j >> 4;
                const int t = int((float(gt) + 0.5f) * inv_ng);   // gt / ng, exact for gt < 128
                const int gl = gt - t * ng, q = (j >> 2) & 3, sl = j & 3;
                jr[u] = (((gl * 4 + q) * NB + t) * BN_REC) * 4 + sl;
                xv[u] = *reinterpret_cast<const uint4*>(xrow(t) + (g0 + gl) * 128 + q * 32 + sl * 8);
            }
            if (u < SU) {
                se[u] = min(lane + 64 * u, 16 * ng - 1);
                // 32-bit element offset: a matrix's codes stay under 4 GiB (every entry
                // point checks it), so M K / 128 < 2^27
                sv[u] = scales[uint32_t((row0 + min(se[u] & 15, R - 1)) * ngroups + g0 + (se[u] >> 4))];
            }
        }

        // The odd last ternary group has 8-byte units: its 16-byte load takes the
        // unit in the low half and 8 bytes past it, which lie inside the codes
        // section or its padding (a load of one width keeps the waits exact).
        // skip format: bits 2p, 2p + 1 of stf = slot p's two blocks are stored (for
        // this lane's row); rmk[p] = the two blocks' stored-row masks of the tile
        uint4 w[PF];
        uint32_t stf = 0, rmk[PF];
        auto issue = [&](int p, int i) __attribute__((always_inline)) {
            const int it = it0 + i;
            if constexpr (SK) {
                // stored blocks of a column ranked by tile row, unit (rank, kq) at
                // (kq nz + rank) * 8; a lane whose block is not stored reads the
                // column's first unit (in bounds: codes are padded) and drops it.
                // The odd last column's partner is the column itself (not computed).
                uint32_t v[4], stb = 0, rm = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t ws = uint32_t(__builtin_amdgcn_readlane(int(sw), min(2 * i + h, ng - 1)));
                    const uint32_t mask = ws & 0xFFFFu;
                    rm |= mask << (16 * h);
                    const uint32_t nz = uint32_t(__builtin_popcount(mask));
                    const uint32_t rank = uint32_t(__builtin_popcount(mask & ((1u << m) - 1u)));
                    const bool st = (mask >> m) & 1u;
                    const uint32_t off = (ws >> 16) * 32u + (st ? (uint32_t(kq) * nz + rank) * 8u : 0u);
                    const u32x2_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(tcodes + off));
                    v[2 * h] = u.x; v[2 * h + 1] = u.y;
                    stb |= uint32_t(st) << h;
                }
                w[p] = make_uint4(v[0], v[1], v[2], v[3]);
                stf = (stf & ~(3u << (2 * p))) | (stb << (2 * p));
                rmk[p] = rm;
            } else {
                const uint32_t off = (TER && it >= n_full) ? unit * 8 : unit * 16;
                const u32x4_t v = code_load<NTL>(reinterpret_cast<const u32x4_t*>(tcodes + size_t(it) * 64 * R + off));
                w[p] = make_uint4(v.x, v.y, v.z, v.w);
            }
        };
#pragma unroll
        for (int p = 0; p < PF; ++p) issue(p, min(p, n - 1));
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int u = 0; u < XU; ++u) {
            if (64 * u < njobs) {                            // uniform: passes of padding jobs only are skipped
                const int sl = jr[u] & 3;                    // slice: columns 8 sl .. +8 of the quarter
                const uint32_t v4[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
                uint32_t xo[4];
                float part = 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    if constexpr (TER) {
                        // columns 8 sl + 2jj, +1 (a quarter starts on a word boundary): pair
                        // (4 sl + jj) % 8 of a 16-code word, class pair % 3, constant part
                        // 129, 33, 9 (exact in bf16)
                        const int ce = jj % 3, co = (4 + jj) % 3;    // class for an even / odd slice
                        const uint32_t wpair = (sl & 1) ? (co == 0 ? 0x43014301u : co == 1 ? 0x42044204u : 0x41104110u)
                                                        : (ce == 0 ? 0x43014301u : ce == 1 ? 0x42044204u : 0x41104110u);
                        part = dot2(v4[jj], wpair, part);
                        xo[jj] = v4[jj];
                    } else {
                        part = dot2(v4[jj], 0x3F803F80u, part);    // (1.0, 1.0)
                        xo[jj] = v4[jj];
                    }
                }
                // the 16 jobs of a (row, group) are one DPP row: every lane gets the row sum
                part = dpp_quad_sum(part);
                part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0x141, 0xF, 0xF, true));
                part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0x140, 0xF, 0xF, true));
                const float nbias = TER ? -part : -136.f * part;
                char* r = rec + (jr[u] >> 2);
                *reinterpret_cast<uint4*>(r + 16 * sl) = make_uint4(xo[0], xo[1], xo[2], xo[3]);
                *reinterpret_cast<float*>(r + 64 + 4 * sl) = nbias;   // the four slices write the four copies
            }
            if (u < SU && 64 * u < 16 * ng) sct[se[u]] = uint16_t(sv[u]);
        }
        // a wave's LDS operations complete in order: its own stores are visible to
        // all its lanes once they have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

        // rm (skip format): the group's stored-row mask; an all-zero block that is
        // not stored gets scale 0, so that it adds exactly nothing instead of the
        // rounding residue of its offset sums under the stored scale of 1
        auto group = [&](const uint4 gw, int lg, uint32_t rm) __attribute__((always_inline)) {
            const char* r = rec + lg * 4 * NB * BN_REC + boff;
            f32x4_t c = *reinterpret_cast<const f32x4_t*>(r + 64);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(code_operand<TER>(gw, s, kc),
                                                            *reinterpret_cast<const bf16x8_t*>(r + 16 * s), c, 0, 0, 0);
            const uint2 sc = *reinterpret_cast<const uint2*>(sct + lg * 16 + 4 * kq);
            float s4[4] = {half_bits_to_f32(uint16_t(sc.x)), half_bits_to_f32(uint16_t(sc.x >> 16)),
                           half_bits_to_f32(uint16_t(sc.y)), half_bits_to_f32(uint16_t(sc.y >> 16))};
            if constexpr (SK) {
                const uint32_t rq = rm >> (4 * kq);
#pragma unroll
                for (int j = 0; j < 4; ++j) s4[j] = (rq >> j) & 1u ? s4[j] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(s4[j], c[j], acc[j]);
        };
        auto compute = [&](int p, int i) __attribute__((always_inline)) {
            if constexpr (SK) {                          // not stored: code 1 (q = 0) everywhere
                const bool s0 = (stf >> (2 * p)) & 1u, s1 = (stf >> (2 * p + 1)) & 1u;
                group(make_uint4(s0 ? w[p].x : 0x55555555u, s0 ? w[p].y : 0x55555555u, 0u, 0u), i * IG,
                      rmk[p] & 0xFFFFu);
                if (it0 + i < n_full)
                    group(make_uint4(s1 ? w[p].z : 0x55555555u, s1 ? w[p].w : 0x55555555u, 0u, 0u), i * IG + 1,
                          rmk[p] >> 16);
            } else {
                group(w[p], i * IG, 0u);
                if (TER && it0 + i < n_full) group(make_uint4(w[p].z, w[p].w, 0u, 0u), i * IG + 1, 0u);
            }
        };
        int i = 0;
        for (; i + PF < n; i += PF) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                compute(p, i + p);
                issue(p, min(i + p + PF, n - 1));
                __builtin_amdgcn_sched_barrier(0);   // refill each slot as soon as it is consumed
            }
        }
#pragma unroll
        for (int p = 0; p < PF; ++p)
            if (i + p < n) compute(p, i + p);
    }

    // C[row 4kq + jj][column m]: column m < nb is activation row m
    if (m < nb) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) red[(wave * NB + m) * 16 + 4 * kq + jj] = acc[jj];
    }
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * nb; t += blockDim.x) {
        const int on = t >> 4, orow = t & 15;
        if (orow < R) {
            float s = 0.f;
            for (int v = 0; v < nw; ++v) s += red[(v * NB + on) * 16 + orow];
            yrow(on)[row0 + orow] = s;
        }
    }
}

template <bool TER, bool SK, int PF, int NB, int XU>
__global__ __launch_bounds__(1024) void gemv_bn_kernel(BnArgs a) {
    const uint16_t* x = a.x;
    float* y = a.y;
    const int K = a.K, M = a.M;
    bn_core<TER, SK, PF, NB, XU, true>(a, a.codes, a.scales, a.B, [=](int t) { return x + size_t(t) * K; },
                             [=](int n) { return y + size_t(n) * M; }, blockIdx.x);
}

// One token: every (token, slot) pair is a one-row job, block (pair, tile).  With
// one activation row there is nothing to group: the pair's expert is read from the
// route, and pairs whose expert id is out of range write nothing.
template <bool TER, int PF, int XU>
__global__ __launch_bounds__(1024) void moe_b1_kernel(BnArgs a) {
    const int p = blockIdx.x / a.tiles, tile = blockIdx.x - p * a.tiles;
    const int e = a.route[p];
    if (e < 0 || e >= a.n_experts) return;
    const int K = a.K, M = a.M;
    const size_t per_codes = size_t(M) * K / (TER ? 4 : 2), per_scales = size_t(M) * (K / 128);
    const uint16_t* xr = a.x + size_t(a.x_per_pair ? p : p / a.topk) * K;
    float* yr = a.y + size_t(p) * M;
    bn_core<TER, false, PF, 1, XU, false>(a, a.codes + size_t(e) * per_codes, a.scales + size_t(e) * per_scales, 1,
                            [=](int) { return xr; }, [=](int) { return yr; }, tile);
}

// ------------------------------------------------------------------ batch 5..16: MFMA

// Batch 5..16 (and expert jobs of several tokens) is a skinny GEMM: the codes
// become bf16 MFMA operands directly, and the activations are read per group
// straight from memory (no staging).
// A code c of a pair-friendly word, OR'ed into the bf16 pattern of 128, is the
// exact value 128 + c = q + K0 (K0 = 136 for INT4; ternary 129, 33 or 9 by
// position class, see code_operand), so v_mfma_f32_16x16x32_bf16 over one
// 128-column scale group gives sum (q + K0) x; subtracting sum K0 x and applying
// the group's fp16 scale
// once per group gives the dequantized dot product.  A block is 32 rows (two
// 16-row tiles) by all of K; its waves take the 128-column groups round robin,
// with the next group's loads in flight while one is computed, and the waves'
// partial tiles are summed at the end.  Lane (n, q) = (lane % 16, lane / 16)
// holds columns [32q, 32q + 32) of the group for weight row n of each tile (the
// tile-interleaved unit (n, q)) and for batch row n; MFMA sub-step s uses columns
// 32q + 8s .. + 8 on both operands, so every k slot sees the same column on A and
// B.  Ternary waves take group pairs, so that the two 8-byte halves of each
// 16-byte unit are loaded back to back.

#ifndef MBD_MQ_TILES
#define MBD_MQ_TILES 2        // 16-row tiles per block
#endif
constexpr int MQ_TILES = MBD_MQ_TILES;
constexpr int MQ_ROWS = 16 * MQ_TILES;
constexpr int MQ_MAXW = 16;
#ifndef MBD_MQ_GPW
#define MBD_MQ_GPW 8          // expert jobs: scale groups per wave (sets the waves per block; 4, 6, 12 and 16 measured slower)
#endif
#ifndef MBD_MQ_GPW_GEMV
#define MBD_MQ_GPW_GEMV 8     // plain GEMV: longer per-wave pipelines measured faster
#endif

inline int mq_waves(int64_t K, int gpw) {
    return int(std::max<int64_t>(1, std::min<int64_t>(MQ_MAXW, (K / 128) / gpw)));
}

// Few batch rows on the 32-row kernel (activations through LDS) pay only when its
// blocks have 16 waves and there is a block for every one of the 256 CUs (at
// 4096 x 16384, 128 blocks, B = 3 took 13.6 against 10.2 us on the few-row kernel).
inline bool mq_wide(int64_t M, int64_t K) {
    return mq_waves(K, MBD_MQ_GPW_GEMV) >= 16 && (M + MQ_ROWS - 1) / MQ_ROWS >= 256;
}

struct MqGroup {
    uint4 code[MQ_TILES];          // INT4: 4 words (32 codes); ternary: .x, .y (32 codes)
    uint32_t sc[MQ_TILES][4];      // raw fp16 scales of the lane's 4 output rows (global
                                   // path): packing them at issue would wait for the loads
    uint4 xv[4];                   // activation pieces (layout in mq_core)
    int g;                         // the group (scales from LDS)
    uint32_t rm[MQ_TILES];         // skip format: the block column's stored-row mask per tile
};

// Scales staged in LDS per block, [group][MQ_ROWS], while they fit this budget.
constexpr int MQ_SCALE_LDS = 32 * 1024;

// Dynamic LDS of a block: the staged scales when SL, then, for expert jobs, the
// waves' partial tiles sized to the block's nw waves (a short expert matrix runs
// one or a few waves, and a 16-wave array would cap the blocks a CU holds).  The
// plain GEMV keeps a static 16-wave array: with it the compiler schedules the
// INT4 group loads ahead of the MFMAs, measured 8% faster at 8192 x 8192, batch 8.
inline size_t mq_scale_lds(int ngroups, bool sl) { return sl ? size_t(ngroups) * MQ_ROWS * 2 : 0; }
inline size_t mq_lds_bytes(int nw, int ngroups, bool sl) {
    return mq_scale_lds(ngroups, sl) + size_t(nw) * MQ_TILES * 64 * 4 * sizeof(float);
}
// Each wave's activation rows for one group, [16][MQ_XROW] bf16, after the parts
// above: rows 4 banks apart.
constexpr int MQ_XROW = 128 + 8;
inline size_t mq_x_lds(int nw) { return size_t(nw) * 16 * MQ_XROW * 2; }
#ifndef MBD_MQ_DEPTH
#define MBD_MQ_DEPTH 2        // group buffers per wave
#endif
constexpr int MQ_DEPTH = MBD_MQ_DEPTH;

struct MqArgs {
    const uint8_t* codes;   // [n_mats][M][K * bits / 8]
    const uint16_t* scales; // [n_mats][M][K / 128]
    const uint32_t* slabs;  // skip format (see BnArgs)
    const uint32_t* tile_base;
    const uint16_t* x;
    float* y;
    int M, K;
    // expert mode
    const int4* jobs;
    const int* n_jobs;
    const int* pair_ids;
    const int* route;       // grouped in the kernel when set (at most kFusedPairs pairs)
    int n_pairs, n_experts, topk, x_per_pair, row_blocks, B;
    int by_expert;          // block index = expert * row_blocks + row block (route set)
};

// Ternary constant part of step s's k slots (negated, bf16 pairs): slot pair p of
// the step is word pair 4 (s % 2) + p, of class (4 (s % 2) + p) % 3 (the classes
// of code_operand): -129, -33 or -9.
__device__ __forceinline__ uint32_t ter_nk0(int s, int p) {
    const int cl = (4 * (s & 1) + p) % 3;
    return cl == 0 ? 0xC301C301u : cl == 1 ? 0xC204C204u : 0xC110C110u;
}

// Rows [row_base, row_base + MQ_ROWS) of one matrix; nb <= 16 batch rows whose
// activations / outputs are rows xrow(b) of a.x (x + xrow(b) K; the launchers
// keep a.x's rows times K below 2^32) / yrow(b).  SL: the block's fp16 scales are
// staged in LDS once (coalesced row runs) and a lane reads its 4 rows' scales of
// a group with one 8-byte LDS read, instead of 4 global loads per tile and group.
// SK: the ternary skip format; the
// waves take single block columns, and lane j of sw holds the slab word of this
// wave's column j / MQ_TILES in tile j % MQ_TILES (the launcher keeps a wave's
// columns times MQ_TILES within 64).
template <bool TER, bool SK, bool SL, bool DYN_RED, bool XS, class XRow, class YRow>
__device__ __forceinline__ void mq_core(const MqArgs& a, const uint8_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, int row_base, int nb, XRow xrow,
                                        YRow yrow) {
    static_assert(TER || !SK, "the skip format is ternary");
    constexpr int BPR = TER ? 4 : 2;                       // elements per byte
    extern __shared__ __attribute__((aligned(16))) float mq_lds[];
    const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;
    uint16_t* mq_sc = reinterpret_cast<uint16_t*>(mq_lds);                // SL: [ngroups][MQ_ROWS]
    float* red;                                                            // [nw][MQ_TILES][64][4]
    float* after = mq_lds + (SL ? (a.K >> 7) * (MQ_ROWS / 2) : 0);
    if constexpr (DYN_RED) {
        red = after;
        after += nw * MQ_TILES * 64 * 4;
    } else {
        __shared__ float red_s[MQ_MAXW * MQ_TILES * 64 * 4];
        red = red_s;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint16_t* xw = reinterpret_cast<uint16_t*>(after) + wave * 16 * MQ_XROW;   // XS: this wave's activation rows
    const int n = lane & 15, q = lane >> 4;
    const int K = a.K, M = a.M, ngroups = K >> 7;
    const uint32_t row_bytes = uint32_t(K) / BPR;
    const int npairs = ngroups >> 1;                       // ternary: full group pairs
    // Per-lane 32-bit offsets (the group's part of every address is uniform):
    // code bytes of the lane's unit in each tile (a tile past M: the last tile),
    // scale bytes of its 4 output rows (clamped).
    uint32_t coff[MQ_TILES], coff8[MQ_TILES], soff[MQ_TILES][4];
    uint32_t item[MQ_TILES];
    int orow[MQ_TILES];                                    // first output row of this lane in each tile
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t) {
        const int r0 = min(row_base + 16 * t, (M - 1) & ~15);
        const int R = min(16, M - r0);
        const uint32_t u = tile_unit(n, q, R);
        item[t] = 64u * uint32_t(R);
        coff[t] = uint32_t(r0) * row_bytes + u * 16;
        coff8[t] = uint32_t(r0) * row_bytes + u * 8;
        orow[t] = row_base + 16 * t + 4 * q;
#pragma unroll
        for (int j = 0; j < 4; ++j) soff[t][j] = uint32_t(min(orow[t] + j, M - 1)) * uint32_t(2 * ngroups);   // bytes
    }
    auto stage_scales = [&]() __attribute__((always_inline)) {
        if constexpr (SL) {
            for (int i = threadIdx.x; i < ngroups * MQ_ROWS; i += blockDim.x) {
                const int rr = i / ngroups, g = i - rr * ngroups;
                mq_sc[g * MQ_ROWS + rr] = scales[size_t(min(row_base + rr, M - 1)) * ngroups + g];
            }
            __syncthreads();
        }
    };
    // expert jobs issue their first group loads before the scales are staged (MoE
    // T = 8 54.5 -> 53.8 us); for the plain GEMV that order measured 5-7% slower
    if constexpr (!DYN_RED) stage_scales();
    const bool xlive = n < nb;
    // Activations.  MFMA order: lane (n, q) takes batch row n (row 0 past nb),
    // columns 32 q + 8 s + [0, 8) at step s of the group; read that way, one load
    // instruction touches 32 cache lines for 1 KB.  XS: piece i of lane l is 16
    // bytes of batch row 4 i + l / 16 (row 0 past nb) at column 8 (l % 16), so 16
    // lanes read a row's 256 bytes (pieces whose four rows are all past nb are not
    // loaded), and the compute passes them through the wave's LDS rows into MFMA
    // order.  The round trip pays from 12 batch rows, or with 16 waves per block.
    uint32_t xo[4];                                        // XS: element offsets in a.x
    const uint16_t* xr = a.x;                              // !XS: batch row n
    if constexpr (XS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rb = 4 * i + (lane >> 4);
            xo[i] = uint32_t(xrow(rb < nb ? rb : 0)) * uint32_t(K) + 8u * uint32_t(lane & 15);
        }
    } else {
        xr = a.x + size_t(xrow(xlive ? n : 0)) * size_t(K);
    }
    const uint16_t* xq = xw + (xlive ? n : 0) * MQ_XROW + 32 * q;
    // skip format: byte offset of each tile's stored blocks, and the slab words
    uint32_t tbase[MQ_TILES];
    uint32_t sw = 0;
    if constexpr (SK) {
#pragma unroll
        for (int t = 0; t < MQ_TILES; ++t) tbase[t] = a.tile_base[min(row_base + 16 * t, (M - 1) & ~15) >> 4] * 32u;
        const int j = lane / MQ_TILES, tj = lane % MQ_TILES;
        const int tix = min(row_base + 16 * tj, (M - 1) & ~15) >> 4;
        sw = a.slabs[size_t(tix) * ngroups + min(wave + nw * j, ngroups - 1)];
    }
    auto load = [&](int li, int g, MqGroup& d) {
#pragma unroll
        for (int t = 0; t < MQ_TILES; ++t) {
            if constexpr (SK) {
                const uint32_t ws = uint32_t(__builtin_amdgcn_readlane(int(sw), li * MQ_TILES + t));
                const uint32_t mask = ws & 0xFFFFu;
                const uint32_t nz = uint32_t(__builtin_popcount(mask));
                const uint32_t rank = uint32_t(__builtin_popcount(mask & ((1u << n) - 1u)));
                const bool st = (mask >> n) & 1u;
                const uint32_t off = tbase[t] + (ws >> 16) * 32u + (st ? (uint32_t(q) * nz + rank) * 8u : 0u);
                const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(codes + off));
                d.code[t] = make_uint4(v.x, v.y, st ? 1u : 0u, 0u);
                d.rm[t] = mask;
            } else if constexpr (TER) {
                const int h = g >> 1;
                const bool pair = h < npairs;
                const uint8_t* base = codes + (pair ? size_t(h) * item[t] + (g & 1) * 8 : size_t(npairs) * item[t]);
                const u32x2_t v = code_load<false>(reinterpret_cast<const u32x2_t*>(base + (pair ? coff[t] : coff8[t])));
                d.code[t] = make_uint4(v.x, v.y, 0u, 0u);
            } else {
                // codes stream once: non-temporal, so that the activations every block
                // reads stay in L2
                const u32x4_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(codes + size_t(g) * item[t] + coff[t]));
                d.code[t] = make_uint4(v.x, v.y, v.z, v.w);
            }
            if constexpr (!SL) {
                const char* sg = reinterpret_cast<const char*>(scales + g);
#pragma unroll
                for (int j = 0; j < 4; ++j) d.sc[t][j] = *reinterpret_cast<const uint16_t*>(sg + soff[t][j]);
            }
        }
        d.g = g;
        if constexpr (XS) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                d.xv[i] = 4 * i < nb ? *reinterpret_cast<const uint4*>(a.x + (xo[i] + uint32_t(g) * 128u))
                                     : make_uint4(0, 0, 0, 0);
        } else {
            const uint4* px = reinterpret_cast<const uint4*>(xr + size_t(g) * 128 + 32 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i) d.xv[i] = px[i];
        }
    };
    f32x4_t acc[MQ_TILES];
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Lanes n >= nb carry batch row 0's activations: B column n only reaches
    // output column n, which is not stored.
    // -sum K0 x per batch column, on the matrix cores: A = -K0 of each k slot in
    // every row (exact in bf16) against the group's activations puts
    // -sum_k K0_k x[n][k] in every row of column n; each tile's chain starts from it.
    UnpackConsts kc;
    kc.init();
    // A of the constant-part MFMAs: INT4 -136 everywhere; ternary by position class
    // (even / odd steps)
    auto nk_operand = [](int s) __attribute__((always_inline)) {
        if constexpr (TER) {
            return __builtin_bit_cast(bf16x8_t, make_uint4(ter_nk0(s, 0), ter_nk0(s, 1), ter_nk0(s, 2), ter_nk0(s, 3)));
        } else {
            return __builtin_bit_cast(bf16x8_t, make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u));
        }
    };
    const bf16x8_t ak0 = nk_operand(0), ak1 = nk_operand(1);
    auto compute = [&](const MqGroup& d) {
        uint4 xb[4];
        if constexpr (XS) {
            // into MFMA order through the wave's LDS rows (the previous group's
            // reads completed before its MFMAs)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * i < nb) *reinterpret_cast<uint4*>(xw + (4 * i + (lane >> 4)) * MQ_XROW + 8 * (lane & 15)) = d.xv[i];
            wave_sync_lds();
#pragma unroll
            for (int s = 0; s < 4; ++s) xb[s] = *reinterpret_cast<const uint4*>(xq + 8 * s);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) xb[s] = d.xv[s];
        }
        f32x4_t cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s & 1 ? ak1 : ak0, __builtin_bit_cast(bf16x8_t, xb[s]), cb, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < MQ_TILES; ++t) {
            f32x4_t cg = cb;
            uint4 cw = d.code[t];
            if constexpr (SK) {                            // not stored: code 1 (q = 0) everywhere
                if (cw.z == 0u) cw = make_uint4(0x55555555u, 0x55555555u, 0u, 0u);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
                cg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(code_operand<TER>(cw, s, kc),
                                                             __builtin_bit_cast(bf16x8_t, xb[s]), cg, 0, 0, 0);
            uint32_t scr[4];
            if constexpr (SL) {
                const uint2 sv = *reinterpret_cast<const uint2*>(mq_sc + d.g * MQ_ROWS + 16 * t + 4 * q);
                scr[0] = sv.x; scr[1] = sv.x >> 16; scr[2] = sv.y; scr[3] = sv.y >> 16;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) scr[j] = d.sc[t][j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float sc = half_bits_to_f32(uint16_t(scr[j]));
                // skip format: a block not stored adds exactly nothing (scale 0)
                if constexpr (SK) sc = (d.rm[t] >> (4 * q + j)) & 1u ? sc : 0.f;
                acc[t][j] = fmaf(sc, cg[j], acc[t][j]);
            }
        }
    };
    // This wave's groups, in order: INT4 wave, wave + nw, ...; ternary the pairs
    // (2h, 2h + 1) for h = wave, wave + nw, ... (the odd last group alone).
    constexpr bool PAIRS = TER && !SK;
    const int nitems = PAIRS ? (ngroups + 1) >> 1 : ngroups;
    const int mine = wave < nitems ? (nitems - 1 - wave) / nw + 1 : 0;
    const bool odd_tail = PAIRS && (ngroups & 1) && mine > 0 && wave + nw * (mine - 1) == npairs;
    const int cnt = PAIRS ? 2 * mine - (odd_tail ? 1 : 0) : mine;
    auto gidx = [&](int i) { return PAIRS ? 2 * (wave + nw * (i >> 1)) + (i & 1) : wave + nw * i; };
    // MQ_DEPTH group buffers (a buffer is never copied while its loads are in
    // flight): the next MQ_DEPTH - 1 groups' loads are in flight while one is
    // computed; indices past the last group reload the last one
    MqGroup gb[MQ_DEPTH];
    if (cnt > 0) {
#pragma unroll
        for (int p = 0; p < MQ_DEPTH - 1; ++p) load(min(p, cnt - 1), gidx(min(p, cnt - 1)), gb[p]);
    }
    if constexpr (DYN_RED) stage_scales();
    for (int i = 0; i < cnt; i += MQ_DEPTH) {
#pragma unroll
        for (int p = 0; p < MQ_DEPTH; ++p) {
            const int ln = min(i + p + MQ_DEPTH - 1, cnt - 1);
            load(ln, gidx(ln), gb[(p + MQ_DEPTH - 1) % MQ_DEPTH]);
            // the loads go out before this group's compute (left to itself the
            // compiler sinks them below it, and no load overlaps any compute)
            __builtin_amdgcn_sched_barrier(0);
            if (i + p < cnt) compute(gb[p]);
        }
    }
#pragma unroll
    for (int t = 0; t < MQ_TILES; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[((wave * MQ_TILES + t) * 64 + lane) * 4 + j] = acc[t][j];
    __syncthreads();
    // C[row = 4q + j][col = n]: wave t (or wave t - nw, ... when there are fewer
    // waves than tiles) sums tile t over the waves
    for (int t = wave; t < MQ_TILES; t += nw) {
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w)
#pragma unroll
            for (int j = 0; j < 4; ++j) s4[j] += red[((w * MQ_TILES + t) * 64 + lane) * 4 + j];
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

template <bool TER, bool SK, bool SL, bool XS>
__global__ __launch_bounds__(64 * MQ_MAXW) void gemv_mq_kernel(MqArgs a) {
    float* y = a.y;
    const int M = a.M;
    mq_core<TER, SK, SL, false, XS>(a, a.codes, a.scales, blockIdx.x * MQ_ROWS, a.B, [=](int b) { return b; },
                 [=](int b) { return y + (size_t)b * M; });
}

template <bool TER, bool SL>
__global__ __launch_bounds__(64 * MQ_MAXW) void moe_mq_kernel(MqArgs a) {
    __shared__ int g[6][kFusedPairs];
    __shared__ int4 gjob;
    __shared__ int plist[kExpertPairs];
    int e, rb, cnt;
    const int* pids;
    if (a.by_expert) {
        // One expert per block row: wave 0 lists the expert's pairs in ascending
        // order with ballots over the route (no grouping pass); a block with no
        // pair exits.  The launcher takes this mode for at most 16 tokens, so an
        // expert meets at most 16 pairs when each token's ids are distinct.
        e = blockIdx.x / a.row_blocks;
        rb = blockIdx.x - e * a.row_blocks;
        if (threadIdx.x < 64) {
            int c = 0;
            for (int p0 = 0; p0 < a.n_pairs; p0 += 64) {
                const int p = p0 + int(threadIdx.x);
                const bool hit = p < a.n_pairs && a.route[p] == e;
                const unsigned long long m = __ballot(hit);
                if (hit) plist[c + int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0)))] = p;
                c += __popcll(m);
            }
            if (threadIdx.x == 0) gjob = make_int4(c, 0, 0, 0);
        }
        __syncthreads();
        cnt = gjob.x;
        pids = plist;
    } else {
        const int job = blockIdx.x / a.row_blocks;
        rb = blockIdx.x - job * a.row_blocks;
        int4 jd;
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
        e = jd.x;
        cnt = jd.z;
    }
    float* y = a.y;
    const int K = a.K, M = a.M, topk = a.topk, xpp = a.x_per_pair;
    const size_t per_codes = (size_t)M * K / (TER ? 4 : 2), per_scales = (size_t)M * (K / 128);
    if (cnt == 0) return;
    mq_core<TER, false, SL, true, false>(
        a, a.codes + (size_t)e * per_codes, a.scales + (size_t)e * per_scales, rb * MQ_ROWS, min(16, cnt),
        [=](int b) {
            const int p = pids[b];
            return xpp ? p : p / topk;
        },
        [=](int b) { return y + (size_t)pids[b] * M; });
}

// 32 dequantized values q * s of one quarter block from its words (ternary 2,
// INT4 4).  Element t of a word sits at bit (bits * (t / 2)) + (t odd ? 16 : 0).
template <bool TER>
__device__ __forceinline__ void dequant_quarter(const uint32_t* wv, float s, float4* o) {
    constexpr int bits = TER ? 2 : 4, per = TER ? 16 : 8, off = TER ? 1 : 8, nwd = TER ? 2 : 4;
    constexpr uint32_t mask = (1u << bits) - 1;
#pragma unroll
    for (int wi = 0; wi < nwd; ++wi) {
#pragma unroll
        for (int jj = 0; jj < per; jj += 4) {
            float e[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = jj + u;
                const int sh = bits * (t >> 1) + ((t & 1) ? 16 : 0);
                e[u] = s * (float)((int)((wv[wi] >> sh) & mask) - off);
            }
            o[(wi * per + jj) / 4] = make_float4(e[0], e[1], e[2], e[3]);
        }
    }
}

// Dense dequant of ternary / INT4: one thread per (row, group, quarter), 32
// elements.
template <bool TER>
__global__ __launch_bounds__(256) void dequant_bq_kernel(const uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales, float* __restrict__ out,
                                                         int64_t n_units, int M, int K) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_units) return;
    const int ngroups = K >> 7;
    const int kq = int(i & 3);
    const int64_t rg = i >> 2, row = rg / ngroups;
    const int g = int(rg - row * ngroups);
    const int64_t r0 = row & ~int64_t(15);
    const int R = int(M - r0 < 16 ? M - r0 : 16);
    const uint32_t unit = tile_unit(int(row - r0), kq, R);
    const uint8_t* tc = codes + size_t(r0) * (size_t(K) / (TER ? 4 : 2));
    uint32_t wv[4];
    if constexpr (TER) {
        const int P = ngroups >> 1, h = g >> 1;
        const uint2 v = h < P ? *reinterpret_cast<const uint2*>(tc + size_t(h) * 64 * R + unit * 16 + (g & 1) * 8)
                              : *reinterpret_cast<const uint2*>(tc + size_t(P) * 64 * R + unit * 8);
        wv[0] = v.x; wv[1] = v.y;
    } else {
        const uint4 v = *reinterpret_cast<const uint4*>(tc + size_t(g) * 64 * R + unit * 16);
        wv[0] = v.x; wv[1] = v.y; wv[2] = v.z; wv[3] = v.w;
    }
    dequant_quarter<TER>(wv, half_bits_to_f32(scales[row * ngroups + g]),
                         reinterpret_cast<float4*>(out + row * K + g * 128 + kq * 32));
}

// Skip format: as above, with the block found through its slab word; an all-zero
// block (not stored) gives zeros.
__global__ __launch_bounds__(256) void dequant_skip_kernel(const uint8_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint32_t* __restrict__ slabs,
                                                           const uint32_t* __restrict__ tile_base,
                                                           float* __restrict__ out, int64_t n_units, int M, int K) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_units) return;
    const int ngroups = K >> 7;
    const int kq = int(i & 3);
    const int64_t rg = i >> 2, row = rg / ngroups;
    const int g = int(rg - row * ngroups);
    const int64_t tile = row >> 4;
    const int m = int(row & 15);
    const uint32_t ws = slabs[tile * ngroups + g], mask = ws & 0xFFFFu;
    uint32_t wv[2] = {0x55555555u, 0x55555555u};
    if ((mask >> m) & 1u) {
        const uint32_t nz = uint32_t(__builtin_popcount(mask)), rank = uint32_t(__builtin_popcount(mask & ((1u << m) - 1u)));
        const uint2 v = *reinterpret_cast<const uint2*>(codes + (size_t(tile_base[tile]) + (ws >> 16)) * 32 +
                                                        (uint32_t(kq) * nz + rank) * 8);
        wv[0] = v.x; wv[1] = v.y;
    }
    dequant_quarter<true>(wv, half_bits_to_f32(scales[row * ngroups + g]),
                          reinterpret_cast<float4*>(out + row * K + g * 128 + kq * 32));
}

}  // namespace mbd

// ------------------------------------------------------------------ host side

using namespace mbd;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

#ifndef MBD_B1_IPW
#define MBD_B1_IPW 4          // items per wave at least (4 KB of codes), few-row kernel
#endif
#ifndef MBD_B1_WAVES
#define MBD_B1_WAVES 8192     // few-row kernel: waves a call aims for (fewer items per wave below it)
#endif
#ifndef MBD_B1_PF_I4
#define MBD_B1_PF_I4 4        // INT4: items (groups, 1 KB) in flight per wave
#endif
#ifndef MBD_B1_PF_T
#define MBD_B1_PF_T 2         // ternary: items (group pairs, 1 KB) in flight per wave
#endif

struct BnPlan {
    int nb_max;      // NB: activation rows per block
    int ipw, nw;
    int xu;          // staging passes: 16 jobs per staged group and row, over 64 lanes
    size_t lds;
};

// Waves per 16-row tile and items per wave for NB activation rows.  Up to
// MBD_B1_IPW items per wave, fewer while the call (tiles = 16-row tiles over all
// its matrices and jobs) would have under about 8192 waves, more when a tile
// would need over 16 waves; a wave stages at most bn_max_groups(NB, ter) groups per
// round.
BnPlan plan_bn(bool ter, int64_t K, int64_t tiles, int NB) {
    BnPlan p{};
    p.nb_max = NB;
    const int64_t IG = ter ? 2 : 1;
    const int64_t ngroups = K / 128, n_items = ter ? (ngroups + 1) / 2 : ngroups;
    const int64_t max_ipw = std::max<int64_t>(1, bn_max_groups(NB, ter) / IG);
    const int64_t fill = (tiles * n_items + MBD_B1_WAVES - 1) / MBD_B1_WAVES;   // items per wave for the wave target
    int64_t ipw = std::max<int64_t>((n_items + 15) / 16, std::min<int64_t>(MBD_B1_IPW, fill));
    ipw = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(ipw, max_ipw), n_items));
    p.ipw = int(ipw);
    p.nw = int(std::min<int64_t>(16, (n_items + ipw - 1) / ipw));
    const int64_t wg = ipw * IG, jobs = 16 * wg * NB;
    p.xu = jobs <= 64 ? 1 : jobs <= 128 ? 2 : 4;
    p.lds = size_t(p.nw) * size_t(wg) * bn_group_lds(NB) + size_t(p.nw) * NB * 64;
    return p;
}

// The 32-row kernels with lds bytes of dynamic LDS, each kernel's limit raised
// first (the activation rows take up to 68 KiB).
template <bool TER, bool SK, bool SL, bool XS>
mbd_status launch_mq1(unsigned blocks, int nw, size_t lds, hipStream_t st, const MqArgs& m) {
    static std::atomic<int> done{0};
    const mbd_status s = lds_limit(reinterpret_cast<const void*>(gemv_mq_kernel<TER, SK, SL, XS>), done, lds,
                                   "batched GEMV");
    if (s != MBD_OK) return s;
    hipLaunchKernelGGL((gemv_mq_kernel<TER, SK, SL, XS>), dim3(blocks), dim3(64 * nw), lds, st, m);
    return MBD_OK;
}

// Activations staged through LDS (XS) from 12 batch rows, or always with 16 waves
// (measured: INT4 8192 x 8192 B = 16 15.0 -> 12.6 us, B = 8 10.9 -> 11.3; INT4
// 8192 x 28672 B = 8 32.1 -> 27.8 us, B = 4 28.6 -> 26.6 us).
template <bool TER, bool SK, bool SL>
mbd_status launch_mq(unsigned blocks, int nw, size_t lds, hipStream_t st, const MqArgs& m) {
    if (m.B >= 12 || nw >= 16)
        return launch_mq1<TER, SK, SL, true>(blocks, nw, lds + mq_x_lds(nw), st, m);
    return launch_mq1<TER, SK, SL, false>(blocks, nw, lds, st, m);
}

template <bool TER, bool SL>
mbd_status launch_moe_mq(unsigned grid, int nw, size_t lds, hipStream_t st, const MqArgs& m) {
    static std::atomic<int> done{0};
    const mbd_status s = lds_limit(reinterpret_cast<const void*>(moe_mq_kernel<TER, SL>), done, lds, "expert GEMV");
    if (s != MBD_OK) return s;
    hipLaunchKernelGGL((moe_mq_kernel<TER, SL>), dim3(grid), dim3(64 * nw), lds, st, m);
    return MBD_OK;
}

// gemv_bn_kernel for the plan's row count and staging passes, or moe_b1_kernel.
template <bool TER, bool SK, bool MOE>
mbd_status launch_bn(const BnPlan& pl, const BnArgs& a, unsigned grid, hipStream_t st) {
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * pl.nw), pl.lds, st, a);
        return hip_check(MOE ? "expert gemv launch" : "gemv launch");
    };
    // ring depth: INT4 with one row MBD_B1_PF_I4; more rows (more staging
    // registers) and ternary (both formats) MBD_B1_PF_T
    constexpr int PF1 = TER ? MBD_B1_PF_T : MBD_B1_PF_I4, PFN = MBD_B1_PF_T;
    if constexpr (MOE) {
        static_assert(!SK, "the expert GEMV takes the dense formats");
        if (pl.nb_max == 1 && pl.xu == 1) return go(moe_b1_kernel<TER, PF1, 1>);
        if (pl.nb_max == 1 && pl.xu == 2) return go(moe_b1_kernel<TER, PF1, 2>);
    } else {
        switch (pl.nb_max * 8 + pl.xu) {
            case 1 * 8 + 1: return go(gemv_bn_kernel<TER, SK, PF1, 1, 1>);
            case 1 * 8 + 2: return go(gemv_bn_kernel<TER, SK, PF1, 1, 2>);
            case 4 * 8 + 1: return go(gemv_bn_kernel<TER, SK, PFN, 4, 1>);
            case 4 * 8 + 2: return go(gemv_bn_kernel<TER, SK, PFN, 4, 2>);
            case 4 * 8 + 4: return go(gemv_bn_kernel<TER, SK, PFN, 4, 4>);
            default: break;
        }
    }
    return fail(MBD_EINVAL, "no kernel for %d rows and %d staging passes", pl.nb_max, pl.xu);
}

int bn_rows(int B) { return B <= 1 ? 1 : 4; }

// Ternary with all-zero blocks not stored ([Bonsai2] 3.4, 5.5).  Batch 1..4 on
// the staged kernel; 5..16 on the 32-row kernel while a wave's block columns
// times its tiles fit the 64 lanes that hold their slab words (K up to 65536),
// else as several staged launches of up to 4 rows.
mbd_status gemv_skip(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st) {
    if (w->K % 128) return fail(MBD_ESHAPE, "K=%lld is not a multiple of 128", (long long)w->K);
    if (w->K > 524288 || w->M > INT32_MAX) return fail(MBD_ESHAPE, "shape too large for the skip format");
    if (w->n_mats > 1) return fail(MBD_EINVAL, "the skip format holds one matrix");
    if (!w->sec[0] || !w->sec[1] || !w->sec[2] || !w->sec[3]) return fail(MBD_EINVAL, "a section is NULL");
    if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2) || !aligned(w->sec[2], 4) || !aligned(w->sec[3], 4))
        return fail(MBD_EALIGN, "codes must be 16-byte, slabs and tile_base 4-byte aligned");
    if (w->M * w->K / 4 >= (int64_t(1) << 32)) return fail(MBD_ESHAPE, "codes beyond 4 GiB");
    if (w->M == 0) return MBD_OK;
    const int tiles = int((w->M + 15) / 16);
    const int ngroups = int(w->K / 128);
    const int nw_mq = mq_waves(w->K, MBD_MQ_GPW_GEMV);
    // from 2 rows on wide shapes (8192 x 28672: B = 2 28.4 -> 24.5 us, B = 4 30.9 ->
    // 24.5 us against the few-row kernel)
    if ((B > 4 || (B >= 2 && mq_wide(w->M, w->K))) && (ngroups + nw_mq - 1) / nw_mq * MQ_TILES <= 64) {
        if (int64_t(B) * w->K >= (int64_t(1) << 32)) return fail(MBD_ESHAPE, "activations of 2^32 elements or more");
        MqArgs m{};
        m.codes = static_cast<const uint8_t*>(w->sec[0]);
        m.scales = static_cast<const uint16_t*>(w->sec[1]);
        m.slabs = static_cast<const uint32_t*>(w->sec[2]);
        m.tile_base = static_cast<const uint32_t*>(w->sec[3]);
        m.x = x; m.y = y; m.M = int(w->M); m.K = int(w->K); m.B = B;
        const unsigned blocks = unsigned((w->M + MQ_ROWS - 1) / MQ_ROWS);
        const bool sll = size_t(ngroups) * MQ_ROWS * 2 <= size_t(MQ_SCALE_LDS);
        const size_t lds = mq_scale_lds(ngroups, sll);
        const mbd_status s = sll ? launch_mq<true, true, true>(blocks, nw_mq, lds, st, m)
                                 : launch_mq<true, true, false>(blocks, nw_mq, lds, st, m);
        if (s != MBD_OK) return s;
        return hip_check("batched gemv launch");
    }
    for (int b0 = 0; b0 < B; b0 += 4) {
        const int nb = std::min(4, B - b0);
        const BnPlan pl = plan_bn(true, w->K, tiles, bn_rows(nb));
        BnArgs a{};
        a.codes = static_cast<const uint8_t*>(w->sec[0]);
        a.scales = static_cast<const uint16_t*>(w->sec[1]);
        a.slabs = static_cast<const uint32_t*>(w->sec[2]);
        a.tile_base = static_cast<const uint32_t*>(w->sec[3]);
        a.x = x + size_t(b0) * w->K; a.y = y + size_t(b0) * w->M;
        a.M = int(w->M); a.K = int(w->K); a.ipw = pl.ipw; a.tiles = tiles; a.B = nb;
        mbd_status s = launch_bn<true, true, false>(pl, a, unsigned(tiles), st);
        if (s != MBD_OK) return s;
    }
    return MBD_OK;
}

}  // namespace

// Cassandra / MX32 launchers live in cassandra.hip.
mbd_status mbd_gemv_cassandra(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st);
mbd_status mbd_gemv_mx32(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, hipStream_t st);
mbd_status mbd_dequant_mx32(const mbd_dweights* w, float* out, hipStream_t st);

extern "C" {

mbd_status mbd_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y, void* stream) {
    hip_clear();
    if (!w || !x || !y) return fail(MBD_EINVAL, "NULL argument");
    if (B < 1 || B > 16) return fail(MBD_ESHAPE, "B=%d outside [1, 16]", B);
    if (w->M < 0 || w->K < 1) return fail(MBD_ESHAPE, "bad shape M=%lld K=%lld", (long long)w->M, (long long)w->K);
    if (!aligned(x, 16) || !aligned(y, 4)) return fail(MBD_EALIGN, "x must be 16-byte and y 4-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (w->fmt == MBD_CASSANDRA) return mbd_gemv_cassandra(w, x, B, y, st);
    if (w->fmt == MBD_MX32) return mbd_gemv_mx32(w, x, B, y, st);
    if (w->fmt == MBD_TERNARY_SKIP) return gemv_skip(w, x, B, y, st);
    if (w->fmt == MBD_CASSANDRA_MX)
        return fail(MBD_EINVAL, "MBD_CASSANDRA_MX holds speculation data only: use mbd_spec_gemv");
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128) return fail(MBD_EINVAL, "unknown format %d", w->fmt);
    if (w->K % 128) return fail(MBD_ESHAPE, "K=%lld is not a multiple of 128", (long long)w->K);
    if (w->M > INT32_MAX || w->K > INT32_MAX) return fail(MBD_ESHAPE, "shape too large");
    const bool ter = w->fmt == MBD_TERNARY_B128;
    // the kernels address a matrix's codes with 32-bit byte offsets
    if (w->M * (w->K / (ter ? 4 : 2)) >= (int64_t(1) << 32)) return fail(MBD_ESHAPE, "codes beyond 4 GiB");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2)) return fail(MBD_EALIGN, "codes must be 16-byte aligned");
    if (w->M == 0) return MBD_OK;
    if (B > 4 || (B >= (ter ? 3 : 2) && mq_wide(w->M, w->K))) {
        // 5..16 rows: the 32-row kernel with activations read per group (at 8 rows
        // it measured even with the few-row kernel, above that faster); on wide
        // shapes from 2 INT4 or 3 ternary rows (8192 x 28672, against the few-row
        // kernel: INT4 B = 2 27.1 -> 26.1 us, B = 3 29.3 -> 26.1, B = 4 29.9 -> 26.6;
        // ternary B = 3 24.5 -> 23.1, B = 4 26.0 -> 23.6; ternary B = 2 within 1%)
        if (int64_t(B) * w->K >= (int64_t(1) << 32)) return fail(MBD_ESHAPE, "activations of 2^32 elements or more");
        MqArgs m{};
        m.codes = static_cast<const uint8_t*>(w->sec[0]);
        m.scales = static_cast<const uint16_t*>(w->sec[1]);
        m.x = x; m.y = y; m.M = int(w->M); m.K = int(w->K); m.B = B;
        const int nw = mq_waves(w->K, MBD_MQ_GPW_GEMV);
        const unsigned blocks = unsigned((w->M + MQ_ROWS - 1) / MQ_ROWS);
        const bool sll = size_t(w->K / 128) * MQ_ROWS * 2 <= size_t(MQ_SCALE_LDS);
        const size_t lds = mq_scale_lds(int(w->K / 128), sll);
        const mbd_status s = ter && sll ? launch_mq<true, false, true>(blocks, nw, lds, st, m)
                             : ter      ? launch_mq<true, false, false>(blocks, nw, lds, st, m)
                             : sll      ? launch_mq<false, false, true>(blocks, nw, lds, st, m)
                                        : launch_mq<false, false, false>(blocks, nw, lds, st, m);
        if (s != MBD_OK) return s;
        return hip_check("batched gemv launch");
    }
    const int tiles = int((w->M + 15) / 16);
    const BnPlan pl = plan_bn(ter, w->K, tiles, bn_rows(B));
    BnArgs a{};
    a.codes = static_cast<const uint8_t*>(w->sec[0]);
    a.scales = static_cast<const uint16_t*>(w->sec[1]);
    a.x = x; a.y = y; a.M = int(w->M); a.K = int(w->K); a.ipw = pl.ipw;
    a.tiles = tiles; a.B = B;
    return ter ? launch_bn<true, false, false>(pl, a, unsigned(tiles), st)
               : launch_bn<false, false, false>(pl, a, unsigned(tiles), st);
}

mbd_status mbd_dequant(const mbd_dweights* w, float* out, void* stream) {
    hip_clear();
    if (!w || !out) return fail(MBD_EINVAL, "NULL argument");
    if (!aligned(out, 16)) return fail(MBD_EALIGN, "w_out must be 16-byte aligned");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (w->fmt == MBD_MX32) return mbd_dequant_mx32(w, out, st);
    if (w->fmt == MBD_TERNARY_SKIP) {
        if (w->M < 0 || w->K < 1 || w->K % 128 || w->K > 524288 || w->M > INT32_MAX) return fail(MBD_ESHAPE, "bad shape");
        if (w->n_mats > 1) return fail(MBD_EINVAL, "the skip format holds one matrix");
        if (!w->sec[0] || !w->sec[1] || !w->sec[2] || !w->sec[3]) return fail(MBD_EINVAL, "a section is NULL");
        if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2) || !aligned(w->sec[2], 4) || !aligned(w->sec[3], 4))
            return fail(MBD_EALIGN, "misaligned section");
        if (w->M == 0) return MBD_OK;
        const int64_t n = w->M * (w->K / 128) * 4;
        hipLaunchKernelGGL(dequant_skip_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<const uint8_t*>(w->sec[0]), static_cast<const uint16_t*>(w->sec[1]),
                           static_cast<const uint32_t*>(w->sec[2]), static_cast<const uint32_t*>(w->sec[3]), out, n,
                           int(w->M), int(w->K));
        return hip_check("dequant launch");
    }
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128)
        return fail(MBD_EINVAL, "dequant supports TERNARY, TERNARY_SKIP, INT4 and MX32");
    if (w->M < 0 || w->K < 1 || w->K % 128) return fail(MBD_ESHAPE, "bad shape");
    if (w->M > INT32_MAX || w->K > INT32_MAX) return fail(MBD_ESHAPE, "shape too large");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    if (!aligned(w->sec[0], 16) || !aligned(w->sec[1], 2)) return fail(MBD_EALIGN, "codes must be 16-byte aligned");
    if (w->M == 0) return MBD_OK;
    const bool ter = w->fmt == MBD_TERNARY_B128;
    const int64_t n = w->M * (w->K / 128) * 4;
    const unsigned blocks = unsigned((n + 255) / 256);
    if (ter)
        hipLaunchKernelGGL((dequant_bq_kernel<true>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint8_t*>(w->sec[0]), static_cast<const uint16_t*>(w->sec[1]), out, n,
                           int(w->M), int(w->K));
    else
        hipLaunchKernelGGL((dequant_bq_kernel<false>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint8_t*>(w->sec[0]), static_cast<const uint16_t*>(w->sec[1]), out, n,
                           int(w->M), int(w->K));
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

}  // extern "C"

namespace {

// The expert GEMV behind both entry points; ws is device memory of ws_bytes bytes
// (the caller's workspace, or this device's static scratch).
// The expert GEMV's checks of the weights and shape, made before any HIP call.
mbd_status moe_check(const mbd_dweights* w) {
    if (w->fmt != MBD_TERNARY_B128 && w->fmt != MBD_INT4_G128)
        return fail(MBD_EINVAL, "expert GEMV supports TERNARY and INT4");
    if (w->M < 1 || w->K < 128 || w->K % 128 || w->M > INT32_MAX || w->K > INT32_MAX)
        return fail(MBD_ESHAPE, "bad expert shape");
    // the kernels address one matrix's codes and scales with 32-bit offsets
    if (w->M * (w->K / (w->fmt == MBD_TERNARY_B128 ? 4 : 2)) >= (int64_t(1) << 32))
        return fail(MBD_ESHAPE, "expert codes beyond 4 GiB");
    return MBD_OK;
}

// Past one token the 32-row kernel addresses the activation rows with 32-bit
// element offsets.
mbd_status moe_x_check(const mbd_dweights* w, int32_t T, int32_t k, int32_t x_per_pair) {
    if (T > 1 && int64_t(x_per_pair ? int64_t(T) * k : T) * w->K >= (int64_t(1) << 32))
        return fail(MBD_ESHAPE, "activations of 2^32 elements or more");
    return MBD_OK;
}

mbd_status moe_gemv(const mbd_dweights* w, const int32_t* route, int32_t T, int32_t k, const uint16_t* x,
                    int32_t x_per_pair, float* y, void* ws, uint64_t ws_bytes, void* stream) {
    if (!w || !route || !x || !y || !ws) return fail(MBD_EINVAL, "NULL argument");
    mbd_status s = moe_check(w);
    if (s != MBD_OK) return s;
    if ((s = moe_x_check(w, T, k, x_per_pair)) != MBD_OK) return s;
    uint64_t need = 0;
    if ((s = mbd_moe_workspace_bytes(w->n_mats, T, k, &need)) != MBD_OK) return s;
    if (ws_bytes < need) return fail(MBD_EINVAL, "workspace of %llu bytes, need %llu", (unsigned long long)ws_bytes, (unsigned long long)need);
    if (!aligned(x, 16) || !aligned(y, 4) || !aligned(ws, 16) || !aligned(route, 4) ||
        !aligned(w->sec[0], 16) || !aligned(w->sec[1], 2))
        return fail(MBD_EALIGN, "misaligned pointer");
    if (!w->sec[0] || !w->sec[1]) return fail(MBD_EINVAL, "codes/scales section is NULL");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const int E = int(w->n_mats), P = T * k;
    const bool ter = w->fmt == MBD_TERNARY_B128;
    const int tiles = int((w->M + 15) / 16);
    if (T == 1) {
        // one token: every (token, slot) pair is a one-row job, nothing to group
        const BnPlan pl = plan_bn(ter, w->K, int64_t(tiles) * std::min(E, P), 1);
        BnArgs a{};
        a.codes = static_cast<const uint8_t*>(w->sec[0]);
        a.scales = static_cast<const uint16_t*>(w->sec[1]);
        a.x = x; a.y = y; a.M = int(w->M); a.K = int(w->K); a.ipw = pl.ipw;
        a.tiles = tiles;
        a.route = route; a.n_experts = E; a.topk = k; a.x_per_pair = x_per_pair ? 1 : 0;
        const int64_t grid = int64_t(P) * tiles;
        if (grid > INT32_MAX) return fail(MBD_ESHAPE, "expert grid too large");
        return ter ? launch_bn<true, false, true>(pl, a, unsigned(grid), st)
                   : launch_bn<false, false, true>(pl, a, unsigned(grid), st);
    }
    // more tokens: jobs of up to 16 pairs of one expert on the 32-row kernel, which
    // reads the activations per group and needs no staging (jobs of one or two
    // pairs, the common case, measured twice as slow on the few-row kernel)
    constexpr int bmax = 16;
    // sum over experts of ceil(pairs / bmax) <= D + (P - D) / bmax, D = distinct experts
    const int64_t D = std::min<int64_t>(E, P), max_jobs = D + (P - D) / bmax;
    // few experts against the route: a block row per expert (blocks of experts no
    // pair routes to exit at once); else jobs grouped in the kernel or beforehand
    const bool by_expert = T <= 16 && P <= kExpertPairs && E <= 2 * P + 64;
    const bool fused = !by_expert && P <= kFusedPairs;
    int* n_jobs = static_cast<int*>(ws);
    int* pair_ids = n_jobs + 4;
    int4* jobs = reinterpret_cast<int4*>(pair_ids + ((P * 4 + 15) / 16) * 4);
    if (!fused && !by_expert) {
        if (P <= kSortPairs)
            hipLaunchKernelGGL(moe_group_sort_kernel, dim3(1), dim3(1024), 0, st, route, P, E, bmax, pair_ids, jobs, n_jobs);
        else
            hipLaunchKernelGGL(moe_group_kernel, dim3(1), dim3(1024), 0, st, route, P, E, bmax, pair_ids, jobs, n_jobs);
        if ((s = hip_check("expert grouping launch")) != MBD_OK) return s;
    }
    MqArgs m{};
    m.codes = static_cast<const uint8_t*>(w->sec[0]);
    m.scales = static_cast<const uint16_t*>(w->sec[1]);
    m.x = x; m.y = y; m.M = int(w->M); m.K = int(w->K);
    m.jobs = jobs; m.n_jobs = n_jobs; m.pair_ids = pair_ids;
    m.route = (fused || by_expert) ? route : nullptr;
    m.by_expert = by_expert ? 1 : 0;
    m.n_pairs = P; m.n_experts = E; m.topk = k; m.x_per_pair = x_per_pair ? 1 : 0;
    m.row_blocks = int((w->M + MQ_ROWS - 1) / MQ_ROWS);
    const int nw = mq_waves(w->K, MBD_MQ_GPW);
    // scales staged while the block's dynamic LDS stays within 60 KiB (a short
    // expert matrix's few waves keep several blocks per CU)
    const bool sll = mq_lds_bytes(nw, int(w->K / 128), true) <= size_t(60 * 1024);
    const size_t lds = mq_lds_bytes(nw, int(w->K / 128), sll);
    const int64_t grid = (by_expert ? int64_t(E) : max_jobs) * m.row_blocks;
    if (grid > INT32_MAX) return fail(MBD_ESHAPE, "expert grid too large");
    const unsigned g = unsigned(grid);
    const mbd_status ls = ter && sll ? launch_moe_mq<true, true>(g, nw, lds, st, m)
                          : ter      ? launch_moe_mq<true, false>(g, nw, lds, st, m)
                          : sll      ? launch_moe_mq<false, true>(g, nw, lds, st, m)
                                     : launch_moe_mq<false, false>(g, nw, lds, st, m);
    if (ls != MBD_OK) return ls;
    return hip_check("expert gemv launch");
}

}  // namespace

// Device scratch of the allocation-free expert GEMV: the grouping tables (job
// count, pair ids, jobs) that the caller's workspace holds otherwise.  Every device
// the library runs on holds its own copy until the process ends.  Host code never
// uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device.
constexpr uint64_t kMoeScratchBytes = uint64_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// This device's address of `scratch`, looked up on the first call on the device.
mbd_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return hip_check("hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MBD_EHIP, "device %d beyond %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MBD_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return MBD_OK;
}

}  // namespace

extern "C" {

mbd_status mbd_moe_gemv(const mbd_dweights* w, const int32_t* route, int32_t T, int32_t k, const uint16_t* x,
                        int32_t x_per_pair, float* y, void* ws, uint64_t ws_bytes, void* stream) {
    hip_clear();
    return moe_gemv(w, route, T, k, x, x_per_pair, y, ws, ws_bytes, stream);
}

mbd_status mbd_moe_gemv_noalloc(const mbd_dweights* w, const int32_t* route, int32_t T, int32_t k,
                                const uint16_t* x, int32_t x_per_pair, float* y, void* stream) {
    hip_clear();
    if (!w || !route || !x || !y) return fail(MBD_EINVAL, "NULL argument");
    mbd_status s = moe_check(w);
    if (s != MBD_OK) return s;
    if ((s = moe_x_check(w, T, k, x_per_pair)) != MBD_OK) return s;
    uint64_t need = 0;
    if ((s = mbd_moe_workspace_bytes(w->n_mats, T, k, &need)) != MBD_OK) return s;
    if (need > kMoeScratchBytes)
        return fail(MBD_ESHAPE, "route of %d x %d pairs over %lld experts needs %llu bytes of scratch, above the "
                    "library's %llu", T, k, (long long)w->n_mats, (unsigned long long)need,
                    (unsigned long long)kMoeScratchBytes);
    void* ws = nullptr;
    if ((s = scratch_address(&ws)) != MBD_OK) return s;
    return moe_gemv(w, route, T, k, x, x_per_pair, y, ws, kMoeScratchBytes, stream);
}

}  // extern "C"
