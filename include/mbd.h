/*
 * mbd.h -- C ABI of libmbd: weight-only low-bit decode GEMV for MI355X (gfx950).
 *
 * Sources the operations follow (cited by page title and section):
 *   [Bonsai2]    "Ternary Bonsai 2" hands-on walkthrough, 27B model to 6 GB:
 *                section 1.2 (block_ternary absmean quantizer, block 128),
 *                sections 3.4 and 5.5 (all-zero blocks: scale 1, flagged).
 *   [GPT54-INT4] "GPT-5.4 small-model compression in practice", section 3.2
 *                (INT4 group 128: scale = max|w| / 7, codes clamped to [-7, 7]).
 *   [Cassandra]  review of "Cassandra: Enabling Reasoning LLMs at Edge via
 *                Self-Speculative Decoding": 3.1 (bf16 fields), 3.2 (Wanda value
 *                pruning + bitmap, mantissa truncation, speculation + verification
 *                = original bits, draft zero-fill, target restore), 3.3 (unary
 *                exponent code by frequency rank; MX shared exponent), 3.5
 *                (chunked parallel unary decode with carried boundary state).
 *   [Bolt]       "Nemotron 3.5 Bolt teardown", background: decode time is set by
 *                the weight bytes read per token.
 *
 * Conventions shared by every call:
 *   - W is [M][K] row-major (row = output channel, K contiguous).  Activations
 *     x / X are bf16 bit patterns [B][K]; outputs y / Y are fp32 [B][M].
 *   - Pointers named *host* are CPU memory; every other data pointer is device
 *     memory owned by the caller (e.g. a torch tensor).  The library never keeps
 *     a pointer after a call returns and never allocates device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device calls only
 *     enqueue work; they never synchronise.  Argument, shape and alignment errors
 *     are reported synchronously before anything is enqueued; a launch failure
 *     returns MBD_EHIP.
 *   - Kernels trust packed data that mbd_validate() accepted; corrupt device
 *     data gives unspecified (but in-bounds) results.
 *   - Thread-safe and reentrant.  mbd_last_error() is a per-thread message for the
 *     most recent failing call on that thread.  No C++ exception crosses the ABI.
 */
#ifndef MBD_H
#define MBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mbd_status;
#define MBD_OK      0
#define MBD_EINVAL  1   /* null pointer, unknown format, bad parameter        */
#define MBD_ESHAPE  2   /* K % 128 != 0 (K % 32 for MX32), B outside [1, 16] */
#define MBD_EALIGN  3   /* device pointer not aligned as documented           */
#define MBD_ERANGE  4   /* bf16 Inf/NaN in W, or a scale that overflows fp16  */
#define MBD_EFORMAT 5   /* packed sections inconsistent (mbd_validate)        */
#define MBD_EHIP    6   /* HIP launch or runtime error                        */
#define MBD_ENOMEM  7   /* host allocation failed                             */

typedef enum {
    MBD_TERNARY_B128 = 1,   /* [Bonsai2] 1.2: 2-bit codes + fp16 scale per 128      */
    MBD_INT4_G128    = 2,   /* [GPT54-INT4] 3.2: 4-bit codes + fp16 scale per 128   */
    MBD_CASSANDRA    = 3,   /* [Cassandra] 3.2-3.3: bit-split speculation / verify  */
    MBD_MX32         = 4,   /* [Cassandra] 3.3: shared max exponent per 32 values   */
    MBD_TERNARY_SKIP = 5,   /* [Bonsai2] 1.2 + 3.4 / 5.5: ternary, all-zero blocks
                               flagged and not stored                              */
    MBD_CASSANDRA_MX = 6    /* [Cassandra] 3.3 Cassandra-2: speculation data with the
                               kept exponents as MX-32 instead of unary codes      */
} mbd_format;

/* ------------------------------------------------------------------ packing
 * Offline, CPU only.  Section layouts (all little-endian):
 *
 * MBD_TERNARY_B128  (sec 0) "codes"  uint32 [M*K/16]: a word holds 16 consecutive
 *                                    elements of a row, the even ones in the low half
 *                                    and the odd ones in the high half: code q+1 of
 *                                    element t of the word at bit 2*(t/2) (+16 if t
 *                                    is odd); code 3 is never written.  Word order is
 *                                    tile-interleaved (below), blocks taken in pairs
 *                                    (2h, 2h+1): unit (m, kq) of a pair is 16 bytes,
 *                                    2 words of block 2h then 2 of block 2h+1 (columns
 *                                    32kq..+32 of each); an odd last block is stored
 *                                    alone in 8-byte units.
 *                   (sec 1) "scales" fp16 [M][K/128]: fp16(mean|w| of the block),
 *                                    round to nearest even; 1.0 for an all-zero
 *                                    block (whose codes are all q = 0).
 *                   q = clamp(round_half_even(w / scale), -1, 1).
 * MBD_INT4_G128     (sec 0) "codes"  uint32 [M*K/8]: a word holds 8 consecutive
 *                                    elements of a row, evens in the low half, odds
 *                                    in the high half: code q+8 of element t of the
 *                                    word at bit 4*(t/2) (+16 if t is odd); code 0 is
 *                                    never written.  Word order is tile-interleaved
 *                                    (below); unit (m, kq) of group g is 16 bytes,
 *                                    the 4 words of columns 128g + 32kq .. +32.
 *                   (sec 1) "scales" fp16 [M][K/128]: fp16(max|w| / 7); 1.0 for
 *                                    an all-zero group.  q = clamp(rne(w/s), -7, 7).
 *                   Tile-interleaved order: rows in tiles of 16 (the last tile of a
 *                   matrix holds the R <= 16 rows left).  A tile holds its groups
 *                   (ternary: group pairs) in order; each is R*4 units, unit (row m
 *                   of the tile, quarter kq) at index kq*R + m, so that the 64 lanes
 *                   of a wave, lane = 16*kq + m, read one contiguous run.  A stack of
 *                   n_mats matrices (mbd_pack_params.n_mats) is tiled matrix by
 *                   matrix: its sections are the concatenation of each matrix's.
 * MBD_TERNARY_SKIP  The MBD_TERNARY_B128 quantizer and word encoding; a block whose
 *                   codes are all q = 0 ([Bonsai2] 3.4 / 5.5: all-zero, scale 1) is
 *                   flagged and its codes are not stored.  tiles = ceil(M / 16).
 *                   (sec 0) "codes"  uint32: the stored blocks, 32 bytes each, tile
 *                                    by tile, block column g by g; the nz stored
 *                                    blocks of (tile, g), ranked r by tile row, as
 *                                    4*nz units of 8 bytes, unit (r, kq) at index
 *                                    kq*nz + r holding columns 32kq .. +32 (2 words).
 *                   (sec 1) "scales" fp16 [M][K/128], as MBD_TERNARY_B128.
 *                   (sec 2) "slabs"  uint32 [tiles][K/128]: bit m (m < R) set when
 *                                    tile row m's block is stored (clear = the
 *                                    all-zero flag); bits 16-31: blocks stored in
 *                                    this tile before column g.  K <= 524288.
 *                   (sec 3) "tile_base" uint32 [tiles+1]: blocks stored before
 *                                    tile t; the last entry is the total.
 * MBD_CASSANDRA     Wanda keep count floor(K*keep_num/keep_den) per row, score
 *                   |w| * act_norm[k], ties to the lower k; 3 high mantissa bits
 *                   kept; 4096-element flat tiles.  f = m*K + k is the flat index.
 *                   (sec 0) "bitmap"   uint32 [ceil(M*K/32)]: keep bit of f at bit f%32
 *                   (sec 1) "spec_nib" uint32 [ceil(kept/8)]: kept values in flat
 *                                      order, (S<<3)|(M>>4), nibble i at bits 4*(i%8)
 *                   (sec 2) "unary"    uint32: rank r of each kept exponent written as
 *                                      r zeros then a one, LSB-first, kept flat order
 *                   (sec 3) "codebook" uint8 [n_sym]: rank -> exponent, ranks by
 *                                      descending count, ties to the smaller exponent
 *                   (sec 4) "bitoff"   uint64 [T+1]: unary bits before tile t
 *                   (sec 5) "kprefix"  uint32 [T+1]: kept values before tile t
 *                   (sec 6) "lo_nib"   uint32 [ceil(kept/8)]: verification, M & 15
 *                   (sec 7) "pruned"   uint16 [M*K - kept]: verification, raw bits
 *                   Sections 0-5 are the speculation data, 6-7 the verification data.
 * MBD_CASSANDRA_MX  Speculation data only, the MBD_CASSANDRA keep rule and bitmap;
 *                   the kept values in kept flat order form groups of 32 (the last
 *                   may be short).  A kept value (S, E, H = 3 high mantissa bits)
 *                   has significand sig = E ? 8 + H : H and e' = max(E, 1); X is
 *                   the largest e' of its group; mag = sig >> (X - e'), 0 once the
 *                   shift reaches 4.  Draft value (-1)^S * mag * 2^(X - 130), exact
 *                   in bf16 (-0.0 when mag = 0 and S = 1); pruned positions +0.0.
 *                   (sec 0) "bitmap"  as MBD_CASSANDRA
 *                   (sec 1) "mx_nib"  uint32 [ceil(kept/8)]: mag of kept value i at
 *                                     bits 4*(i%8) of word i/8
 *                   (sec 2) "mx_sign" uint32 [ceil(kept/32)]: S of kept value i at
 *                                     bit i%32 of word i/32
 *                   (sec 3) "mx_exp"  uint8 [ceil(kept/32)]: X of each group
 *                   (sec 4) "kprefix" uint32 [T+1]: kept values before tile t
 *                   mbd_spec_decode and mbd_spec_gemv take it; mbd_gemv does not
 *                   (no verification data).
 * MBD_MX32          (sec 0) "mx_exp"  uint8 [M][K/32]: X = max over the group of
 *                                     max(E, 1)
 *                   (sec 1) "mx_sign" uint32 [M][K/32]: bit i = sign of element i
 *                   (sec 2) "mx_mag"  uint8 [M][K]: (E ? 128|M : M) >> (X - max(E,1)),
 *                                     0 when the shift is 8 or more.
 *                   Value = (-1)^S * mag * 2^(X - 134), exact in bf16.
 *
 * Every section buffer is zero padded: `padded_bytes` (a multiple of 256, at least
 * `bytes` + 256) is the size to copy to the device; kernels may read the padding.
 */
typedef struct {
    int32_t keep_num;   /* Cassandra keep fraction numerator   (default 3)  */
    int32_t keep_den;   /* Cassandra keep fraction denominator (default 10) */
    int64_t n_mats;     /* TERNARY / INT4: the M rows are n_mats stacked matrices
                           of M / n_mats rows each (default 1; 0 means 1)   */
} mbd_pack_params;

typedef struct mbd_packed mbd_packed;   /* opaque, owns the host section buffers */

typedef struct {
    const char* name;       /* static string, e.g. "codes"                   */
    const void* data;       /* host pointer owned by the mbd_packed handle   */
    uint64_t bytes;         /* meaningful bytes                              */
    uint64_t padded_bytes;  /* bytes to copy to the device (zero padded)     */
} mbd_section;

typedef struct {
    int32_t fmt;
    int32_t n_sym;          /* Cassandra codebook size                       */
    int64_t M, K;
    int64_t n_kept;         /* Cassandra kept values                         */
    int64_t unary_bits;     /* Cassandra unary stream length in bits         */
    int64_t n_tiles;        /* Cassandra 4096-element tiles                  */
    double bpw;             /* all sections' meaningful bits / (M*K)         */
    double spec_bpw;        /* Cassandra speculation sections (0-5) / (M*K)  */
    double exp_entropy_bits;/* Cassandra: Shannon entropy of kept exponents  */
    double unary_avg_bits;  /* Cassandra: unary bits per kept value          */
    double zero_fraction;   /* ternary: fraction of q == 0                   */
} mbd_stats;

/* Pack a bf16 weight.  w_bf16_host [M][K] and act_norm_host [K] (fp32, Cassandra
 * only, else may be NULL) are borrowed for the call.  params may be NULL (defaults).
 * On success *out is a new handle; free it with mbd_packed_free().
 * Errors: EINVAL (null / unknown fmt / bad params), ESHAPE (M < 1, K < 1 or K not a
 * multiple of 128 (32 for MX32)), ERANGE (Inf/NaN in W, fp16 scale overflow, non-finite
 * or negative act_norm), ENOMEM. */
mbd_status mbd_pack(int32_t fmt, const uint16_t* w_bf16_host, int64_t M, int64_t K,
                    const float* act_norm_host, const mbd_pack_params* params,
                    mbd_packed** out);

/* Copy up to `cap` section descriptors into arr (section order as documented above)
 * and the total count into *n.  Pointers stay valid until mbd_packed_free(h).  The
 * sections are the saved form of a quantized weight: codes and scales stored apart
 * ([GPT54-INT4] 3.2, the weight saved with its scales; [Bonsai2] 3.6, export of the
 * packed model), or the speculation and verification parts ([Cassandra] 3.2: the
 * draft loads the first only, the target both).  cap = 0 only reports *n.
 * Errors: EINVAL (NULL h or n, or arr NULL with cap > 0). */
mbd_status mbd_packed_sections(const mbd_packed* h, mbd_section* arr, int32_t cap, int32_t* n);
/* Format statistics of a handle ([Cassandra] 3.3: exponent entropy of the kept
 * values and average unary code length; bits per weight of all sections and of
 * the speculation sections; [Bonsai2] 1.2: fraction of ternary zeros).
 * Errors: EINVAL (NULL argument). */
mbd_status mbd_packed_stats(const mbd_packed* h, mbd_stats* out);
/* Full CPU consistency check of a handle's sections (codes in range, bitmap row
 * counts, tile table vs unary stream, codebook ranks): the conditions under which
 * the decode of [Cassandra] 3.5 and the dequantization of [Bonsai2] 1.2 and
 * [GPT54-INT4] 3.2 are defined.  EFORMAT on failure, EINVAL for NULL. */
mbd_status mbd_validate(const mbd_packed* h);
/* Releases the handle and its host sections; NULL is a no-op. */
void mbd_packed_free(mbd_packed* h);

/* ------------------------------------------------------------------ device data
 * Raw device pointers to byte copies (padded_bytes) of the packed sections, in the
 * documented section order.  Section base pointers must be 16-byte aligned.
 * n_mats > 1 describes n_mats matrices of identical shape stacked back to back in
 * each section (ternary / INT4 only; used by the expert GEMV). */
#define MBD_MAX_SECTIONS 8
typedef struct {
    int32_t fmt;
    int32_t n_sym;
    int64_t M, K;
    int64_t n_kept;
    int64_t n_mats;
    const void* sec[MBD_MAX_SECTIONS];
} mbd_dweights;

/* Dense dequantized weight w_out fp32 [M][K] (TERNARY, TERNARY_SKIP, INT4, MX32):
 * q*s ([Bonsai2] 1.2, the ternary value is the code times its block scale;
 * [GPT54-INT4] 3.2, the INT4 value is the code times its group scale) or
 * (-1)^S*mag*2^(X-134) ([Cassandra] 3.3, the MX value is the shifted significand at
 * the shared exponent), all exact in fp32.  w_out 16-byte aligned, caller-owned.
 * Errors: EINVAL (NULL, unknown format), ESHAPE, EALIGN, EHIP. */
mbd_status mbd_dequant(const mbd_dweights* w, float* w_out, void* stream);

/* Fused dequant-GEMV / skinny GEMM: y[b][m] = sum_k deq(W)[m][k] * x[b][k] with fp32
 * accumulation ([Bolt] background; [Bonsai2] 1.2; [GPT54-INT4] 3.2).
 * TERNARY and INT4: B in [1, 16].  MX32: B in [1, 16] (MFMA bf16, the Cassandra-2
 * verify GEMM).  CASSANDRA: the target-side verify GEMM over the restored weight
 * (speculation + verification data merged on the fly, [Cassandra] 3.2), B in [1, 16].
 * x: bf16 [B][K], 16-byte aligned.  y: fp32 [B][M], 4-byte aligned.  TERNARY,
 * TERNARY_SKIP and INT4 at B > 4 address the activations with 32-bit element
 * offsets: B·K of 2^32 or more returns MBD_ESHAPE. */
mbd_status mbd_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y,
                    void* stream);

/* Expert GEMV over n_mats stacked TERNARY or INT4 matrices (MoE; [Bolt] routes each
 * token to a subset of experts).  route [T][k] int32 expert ids in [0, n_mats) with
 * distinct ids per token.  x bf16: [T][K] (x_per_pair = 0) or [T][k][K]
 * (x_per_pair = 1).  y fp32 [T][k][M]: y[t][j] = W[route[t][j]] @ x_row.  An
 * expert's weights are read once per group of up to 16 tokens routed to it.  At
 * most 4096 experts (MBD_ESHAPE beyond).  Ids outside [0, n_mats) leave their y
 * rows unwritten; an id repeated within a token is outside this contract (with at
 * most 16 tokens, pairs past an expert's 16th may be left unwritten).  ws: device workspace of at least
 * mbd_moe_workspace_bytes(n_mats, T, k) bytes, 16-byte aligned, contents
 * overwritten.  Calls that share a workspace must not overlap.  With T > 1 the
 * activations are addressed with 32-bit element offsets: x's rows (T, or T·k with
 * x_per_pair) times K of 2^32 or more returns MBD_ESHAPE. */
mbd_status mbd_moe_workspace_bytes(int64_t n_mats, int32_t T, int32_t k, uint64_t* bytes);
mbd_status mbd_moe_gemv(const mbd_dweights* experts, const int32_t* route, int32_t T,
                        int32_t k, const uint16_t* x, int32_t x_per_pair, float* y,
                        void* ws, uint64_t ws_bytes, void* stream);

/* mbd_moe_gemv for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the grouping tables in a static
 * device array of the library (1 MiB per device, held until the process ends; its
 * address is looked up once per device on the first call there).  Routes whose
 * workspace (mbd_moe_workspace_bytes) exceeds 1 MiB return MBD_ESHAPE.  Every call
 * on one device shares that array: calls that overlap on a device race (serialise
 * them on one stream).  No allocation of any kind, host or device. */
mbd_status mbd_moe_gemv_noalloc(const mbd_dweights* experts, const int32_t* route, int32_t T,
                                int32_t k, const uint16_t* x, int32_t x_per_pair, float* y,
                                void* stream);

/* Draft weights from the speculation data only ([Cassandra] 3.2, path b): bf16
 * w_spec [M][K]; kept values get (S<<15)|(E<<7)|(M_hi<<4), pruned values +0.0.
 * Sections 6-7 are not read and may be NULL.  w_spec 16-byte aligned. */
mbd_status mbd_spec_decode(const mbd_dweights* w, uint16_t* w_spec, void* stream);

/* Draft GEMV fused with speculation decode: y = W_spec x, B in [1, 16]. */
mbd_status mbd_spec_gemv(const mbd_dweights* w, const uint16_t* x, int32_t B, float* y,
                         void* stream);

/* Bit-exact original weights from speculation + verification data ([Cassandra]
 * 3.2, path c): bf16 w_out [M][K], 16-byte aligned. */
mbd_status mbd_verify_restore(const mbd_dweights* w, uint16_t* w_out, void* stream);

/* ------------------------------------------------------------------ device encoder
 * [Cassandra] 3.2-3.3 (and 3.5, the online encoder the paper builds in hardware):
 * the eight MBD_CASSANDRA sections of a bf16 weight already in device memory,
 * bit-identical to mbd_pack(MBD_CASSANDRA) with the same keep fraction.
 * w: bf16 [M][K] device, 16-byte aligned; act_norm: fp32 [K] device; K % 128 == 0,
 * M*K < 2^32.  ws: device workspace of mbd_encode_workspace_bytes(M) bytes,
 * 16-byte aligned, shared by both calls (contents overwritten).
 * mbd_encode_plan runs the pruning and the exponent histogram and returns the
 * section sizes; it SYNCHRONISES `stream` to read two totals back, and reports
 * MBD_ERANGE for Inf/NaN in w or a negative / non-finite act_norm entry.
 * mbd_encode_cassandra then writes every section: sec[i] is a device buffer of at
 * least plan->padded_bytes[i] bytes, 16-byte aligned (padding zeroed by the call).
 * It only enqueues work; w and act_norm must be those the plan was made from (the
 * unary stream is cut at the planned size otherwise).  Calls that share a
 * workspace must not overlap. */
typedef struct {
    int64_t n_kept;
    int64_t unary_bits;
    int64_t n_tiles;
    int32_t n_sym;
    int32_t reserved;
    uint64_t bytes[8];         /* meaningful bytes of each section, MBD_CASSANDRA order */
    uint64_t padded_bytes[8];  /* buffer bytes the encode call writes               */
} mbd_encode_plan_t;
mbd_status mbd_encode_workspace_bytes(int64_t M, uint64_t* bytes);
mbd_status mbd_encode_plan(const uint16_t* w, const float* act_norm, int64_t M, int64_t K,
                           int32_t keep_num, int32_t keep_den, void* ws, uint64_t ws_bytes,
                           mbd_encode_plan_t* plan, void* stream);
mbd_status mbd_encode_cassandra(const uint16_t* w, const float* act_norm, int64_t M, int64_t K,
                                int32_t keep_num, int32_t keep_den, const mbd_encode_plan_t* plan,
                                void* const* sec, void* ws, uint64_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ measurement aid
 * Streaming-read probe, not a step of the method: reads `bytes` of device memory at
 * src (16-byte aligned, a multiple of 16) with `blocks` x `threads` threads (threads
 * a multiple of 64, at most 1024), 16-byte non-temporal loads, eight in flight per
 * thread.  The measured rate is the practical ceiling of the weight-streaming kernels
 * ([Bolt] background: a decode step's time is the weight bytes it reads).  sink:
 * device uint32 [blocks], never written in practice (it keeps the loads alive).
 * Errors: EINVAL, EALIGN, ESHAPE, EHIP. */
mbd_status mbd_probe_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t blocks,
                                 int32_t threads, void* stream);

const char* mbd_status_str(mbd_status s);
const char* mbd_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MBD_H */
