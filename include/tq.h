/*
 * tq.h -- C ABI of the TurboQuant hot path for AMD Instinct MI355X (gfx950).
 *
 * The library implements the two quantizers and the scoring paths described by
 * the pages on TurboQuant (arXiv 2504.19874):
 *
 *   Algorithm 1 (TurboQuant_mse): keep the vector norm, rotate by a random
 *     orthogonal matrix Pi, map every rotated coordinate to the nearest
 *     Lloyd-Max centroid of the coordinate law at dimension d, invert the
 *     rotation on decode.  [ai-navigate-news Gemma 4 post, section
 *     "仕組み（技術的）"; AiBoss overview, section "TurboQuantの技術原理"]
 *   Algorithm 2 (TurboQuant_prod): Algorithm 1 at b-1 bits, then the sign
 *     bits of S r for the residual r together with ||r|| -- an unbiased
 *     inner-product estimate.  [same post and section; AIgent Lab explainer,
 *     section "視点1" (QJL)]
 *   Dense records: index bit planes and sign bits packed into bytes, norms and
 *     residual norms ("gammas") as fp16.  [same post, same section]
 *   Attention and inner-product search computed on the packed codes.
 *     [AiBoss overview, sections "TurboQuantの主な機能" and
 *     "TurboQuantの応用事例"]
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns a tq_status (0 = TQ_OK, negative = error) unless
 *   stated otherwise.  Nothing throws across the ABI.  Arguments are checked
 *   on the host before anything is launched; a rejected call launches nothing
 *   and writes nothing.
 * - "device pointer" arguments are caller-owned device memory on the device
 *   that was current when the quantizer was created.  The library never frees
 *   them.  "host pointer" arguments are read (or written) synchronously.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Device work is enqueued on it and the call returns without waiting.
 * - A quantizer is immutable after creation and may be used from several
 *   streams or threads at once.
 * - Record layout (one vector): P planes of d bits, P*d/8 bytes.  Bit j of a
 *   plane lives in byte j/8 at bit position j%8 (equivalently: little-endian
 *   64-bit word j/64, bit j%64).  TQ_MSE with b bits: planes 0..b-1 hold bit p
 *   of the centroid index.  TQ_PROD with b bits: planes 0..b-2 hold the index
 *   of the (b-1)-bit codebook, plane b-1 holds the sign bits of S r
 *   (1 = non-negative).  Norms and gammas are IEEE fp16 bit patterns in
 *   separate uint16 arrays.
 * - Non-finite input values are a precondition violation (codes unspecified).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,     /* bad argument: null, size, alignment, mismatch */
  TQ_ERR_UNSUPPORTED = -2, /* valid request outside what the library implements */
  TQ_ERR_HIP = -3,         /* a HIP runtime call failed; see tq_last_hip_error() */
  TQ_ERR_NOMEM = -4,       /* device or host allocation failed */
  TQ_ERR_WORKSPACE = -5    /* workspace pointer null or smaller than required */
} tq_status;

typedef enum { TQ_MSE = 0, TQ_PROD = 1 } tq_mode;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;
/* Arrangement of a sequence of records in memory.
 *   TQ_LAYOUT_ROWS  : one record after another ([T][code_bytes]).
 *   TQ_LAYOUT_TILE32: token-tiled, bit-transposed: tokens are grouped in tiles
 *     of 32; tile k of a sequence holds planes * d uint32 words, word
 *     [k][p][j] has bit i = bit j of plane p of token 32k + i (bits of tokens
 *     past the sequence length are zero).  The same bits as the row layout,
 *     arranged so that a contraction over tokens reads whole words. */
typedef enum { TQ_LAYOUT_ROWS = 0, TQ_LAYOUT_TILE32 = 1 } tq_layout;

typedef struct tq_quantizer tq_quantizer; /* opaque */

/* Lloyd-Max codebook of the coordinate law at dimension d (host, synchronous).
 * The law is that of one coordinate of a uniform point on the unit sphere
 * S^{d-1}: density proportional to (1-u^2)^((d-3)/2) on [-1, 1], the
 * Beta-shaped law of the AiBoss overview, section "TurboQuantの技術原理".
 * Lloyd-Max (boundaries at midpoints, centroids at conditional means) is
 * iterated to the fp64 floor; the codebook is symmetric.
 *   d:         3 <= d <= 65536
 *   bits:      1 <= bits <= 8
 *   centroids: host, 2^bits doubles, written ascending
 *   bounds:    host, 2^bits - 1 doubles (midpoints), may be NULL
 * Returns TQ_ERR_INVALID on bad d/bits or null centroids. */
int tq_codebook_build(int d, int bits, double *centroids, double *bounds);

/* Create a quantizer for dimension d on the current HIP device.
 *   mode TQ_MSE : 1 <= bits <= 4, s ignored (may be NULL)
 *   mode TQ_PROD: 1 <= bits <= 4, s required.  bits = 1 is the pure sign
 *     (QJL) mode, the 1-bit mode of the AiBoss overview (section
 *     "TurboQuantの主な機能"): Algorithm 1 at 0 bits keeps only the norm (its one
 *     centroid is 0), so the residual is x itself and a record is the sign
 *     plane of S x alone.
 *   d:  multiple of 64, 64 <= d <= 2048
 *   pi: host, d*d floats row-major, the rotation (caller keeps ownership;
 *       it is copied).  The library assumes it is orthogonal to fp32
 *       precision and does not check.
 *   s:  host, d*d floats row-major, the QJL projection with d rows.
 * The codebook (bits for TQ_MSE, bits-1 for TQ_PROD) is built here.
 * On success *out receives the quantizer; destroy it with
 * tq_quantizer_destroy. */
int tq_quantizer_create(tq_quantizer **out, int d, int bits, int mode, const float *pi, const float *s);
void tq_quantizer_destroy(tq_quantizer *q);

/* Shape of a quantizer.  Any output pointer may be NULL.
 *   planes     : bit planes per record
 *   code_bytes : planes * d / 8, bytes of one record in `codes` arrays */
int tq_quantizer_info(const tq_quantizer *q, int *d, int *bits, int *mode, int *planes, size_t *code_bytes);

/* Algorithm 1 encode of n vectors.
 *   x:     device, n rows of d values of type xt, row stride ldx elements
 *          (ldx >= d); TQ_F32, TQ_BF16 or TQ_F16
 *   codes: device, n * code_bytes bytes, 16-byte aligned
 *   norms: device, n fp16 bit patterns: fp16(||x||) round-to-nearest-even,
 *          saturating at 65504
 * Index j of a vector is the number of codebook boundaries t_k with
 * t_k * ||x|| < (Pi x)_j (a value on a boundary goes to the lower cell; the
 * zero vector gets index 2^(b-1) - 1 everywhere).  q must be TQ_MSE.
 * n == 0 is a no-op. */
int tq_encode_mse(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx,
                  uint8_t *codes, uint16_t *norms, void *stream);

/* Algorithm 2 encode of n vectors (q must be TQ_PROD).  As tq_encode_mse with
 * the (b-1)-bit codebook, then r = x - n_hat * Pi^T c[idx], sign plane bit i =
 * [(S r)_i >= 0] and gammas[i] = fp16(||r||).  At b = 1 there is no index
 * plane: r = x, the record is the sign plane of S x, norms and gammas both
 * hold fp16(||x||).
 *   gammas: device, n fp16 bit patterns */
int tq_encode_prod(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx,
                   uint8_t *codes, uint16_t *norms, uint16_t *gammas, void *stream);

/* Encode nseq sequences of T vectors straight into a cache, by q's algorithm
 * (TQ_MSE: Algorithm 1, TQ_PROD: Algorithm 2, with the arithmetic of
 * tq_encode_mse / tq_encode_prod): row s*T + t of x becomes position t0 + t of
 * sequence s.  This is the prompt (prefill) write of the decode cache that
 * tq_attn_decode reads, in either of its layouts, with no separate tiling pass.
 *   x:       device, nseq*T rows of d values of type xt, row stride ldx
 *            elements (16-byte aligned rows)
 *   t0, Tstride: first position written and positions per sequence of the
 *            cache; t0 + T <= Tstride
 *   layout:  TQ_LAYOUT_ROWS: codes = device [nseq][Tstride][code_bytes]
 *            TQ_LAYOUT_TILE32: codes = device uint32 [nseq][ceil(Tstride/32)][planes][d];
 *            t0 must be a multiple of 32; the words that hold positions
 *            t0 .. t0+T-1 are written whole, positions from t0+T to the end of
 *            the last such word as zero bits (a later tq_attn_decode_append
 *            sets them); nseq <= 65535 (else TQ_ERR_UNSUPPORTED)
 *   norms:   device [nseq][Tstride] fp16 bit patterns (positions t0.. written)
 *   gammas:  device [nseq][Tstride], TQ_PROD only (ignored for TQ_MSE)
 * Other positions of the cache are not touched.  TQ_ERR_INVALID for a null
 * argument, a misaligned pointer or row stride, or positions outside the
 * cache.  Head dims 64 and 128 write the cache from the encode kernel itself;
 * other head dims stage the records in memory the call allocates on the stream
 * and then move them into place. */
int tq_encode_cache(const tq_quantizer *q, const void *x, int xt, int64_t nseq, int64_t T, int64_t ldx, int64_t t0,
                    int64_t Tstride, int layout, void *codes, uint16_t *norms, uint16_t *gammas, void *stream);

/* Decode n records to fp32 rows.
 *   TQ_MSE : out = n_hat * Pi^T c[idx]
 *   TQ_PROD: out = n_hat * Pi^T c[idx] + sqrt(pi/2)/d * gamma * S^T (2 bits - 1)
 *   gammas: device, required for TQ_PROD, ignored for TQ_MSE
 *   out:    device, n rows, row stride ldo >= d floats */
int tq_decode(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas,
              int64_t n, float *out, int64_t ldo, void *stream);

/* Inner-product scores of m fp32 queries against n records: est = <q, decode(x)>,
 * computed as n_hat <Pi q, c[idx]> (+ sqrt(pi/2)/d * gamma <S q, s> for TQ_PROD).
 *   queries: device, m rows, stride ldq >= d floats
 *   k == 0 : scores = device [m * n] floats, row-major; idx unused
 *   k >= 1 : per query the k best records by descending score (ties -> lower
 *            record index): scores = device [m * k] floats, idx = device
 *            [m * k] int64.  k <= 64 and k <= n.
 *   ws/ws_bytes: device workspace of at least tq_score_ws_bytes(...) bytes */
int tq_score(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
             const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx,
             void *ws, size_t ws_bytes, void *stream);
size_t tq_score_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k);

/* Rearrange nseq sequences of T row-layout records into TQ_LAYOUT_TILE32.
 *   codes: device [nseq][T][code_bytes] (16-byte aligned)
 *   tiles: device [nseq][ceil(T/32)][planes][d] uint32 (every word written)
 * Bits of token slots T..32*ceil(T/32)-1 are written as zero. */
int tq_tile_records(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, uint32_t *tiles,
                    void *stream);

/* Decode attention of one new query token per sequence against a compressed
 * cache: values through Algorithm 2 (vq, TQ_PROD), keys through Algorithm 1
 * (kq, TQ_MSE), as the ai-navigate-news Gemma 4 post assigns them (section
 * "仕組み（技術的）"), or through Algorithm 2 as well (kq TQ_PROD, unbiased
 * scores).  For batch b and query head h, with g = h / (Hq/Hkv):
 *   s_t = scale * <q[b,h], K~[b,g,t]>  for t < seq_len[b]
 *   out[b,h] = sum_t softmax(s)_t V~[b,g,t]      (zero when seq_len[b] == 0)
 * where K~, V~ are the decodes of the records.
 *   q:       device [B, Hq, d] of type qt (TQ_F32, TQ_BF16 or TQ_F16)
 *   kcodes:  device [B, Hkv, Tstride, kcode_bytes], knorms [B, Hkv, Tstride]
 *   kgammas: device [B, Hkv, Tstride] key residual norms when kq is TQ_PROD;
 *            ignored (may be NULL) when kq is TQ_MSE
 *   vcodes:  device, value records in layout `vlayout`:
 *            TQ_LAYOUT_ROWS   [B, Hkv, Tstride, vcode_bytes]: any d and bit
 *                             widths (one wave per sequence split)
 *            TQ_LAYOUT_TILE32 [B, Hkv, ceil(Tstride/32), planes, d] uint32
 *                             words: the matrix-core kernels, for TQ_MSE keys
 *                             and values with at least one index bit, at
 *                             d = 128 (key bits 1-4, value index bits 1-3),
 *                             d = 256 (key bits 1-3, value index bits 1-3)
 *                             and d = 512 (key bits 1-3, 1-bit value
 *                             indices); other cases TQ_ERR_UNSUPPORTED.
 *                             Head dim 128 with 1-bit value indices, key bits
 *                             1-3 and Tstride a multiple of 8 (16-byte aligned
 *                             arrays) takes the wave-streaming kernel.
 *   vnorms, vgammas: device [B, Hkv, Tstride]
 *   seq_len: device [B] int32, 0 <= seq_len[b] <= Tstride
 *   out:     device [B, Hq, d] fp32
 *   ws:      device workspace of at least tq_attn_decode_ws_bytes(...) bytes
 * kq and vq must share d; Hq % Hkv == 0. */
int tq_attn_decode(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                   int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                   const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                   int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *ws, size_t ws_bytes,
                   void *stream);
size_t tq_attn_decode_ws_bytes(const tq_quantizer *kq, int B, int Hq, int Hkv, int64_t Tstride, int vlayout);

/* Attention of a chunk of M query tokens per sequence against the compressed cache (prefill in
 * chunks), causal: query token m of sequence b sits at position q_pos[b] + m and attends the cached
 * tokens 0 .. q_pos[b] + m, so the chunk's own keys and values must already be in the cache (encode
 * them first with tq_encode_mse / tq_encode_prod).  Long prompts are where the compression pays
 * (techblog-plum explainer, section "注意点・未確認事項": contexts of 4K tokens or less gain little).
 * Keys through Algorithm 1 or 2 (kq), values through Algorithm 2 (vq), scores and outputs as
 * tq_attn_decode for each query token:
 *   q:     device [B, M, Hq, d] of type qt;  out: device [B, M, Hq, d] fp32
 *   q_pos: device [B] int32, q_pos[b] >= 0 and q_pos[b] + M <= Tstride (a query token past Tstride
 *          attends the Tstride cached tokens)
 *   cache arguments as tq_attn_decode, with the same layouts and limits: TQ_LAYOUT_ROWS takes any d
 *          and bit widths (one wave per 16 query rows); TQ_LAYOUT_TILE32 runs the decode kernels
 *          over B * M rows, one per query token (row b m attends tokens 0 .. q_pos[b] + m and reads
 *          the cache row of sequence b), with TQ_MSE keys only
 *   ws:    device workspace of at least tq_attn_prefill_ws_bytes(...) bytes (per layout) */
int tq_attn_prefill(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int M, int Hq,
                    int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                    const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                    int64_t Tstride, const int32_t *q_pos, float scale, float *out, void *ws, size_t ws_bytes,
                    void *stream);
size_t tq_attn_prefill_ws_bytes(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride, int vlayout);

/* One decode step with the new token appended: for every (b, g) the new key k_new[b,g] and value
 * v_new[b,g] are encoded (keys by kq's algorithm, values by Algorithm 2, exactly as tq_encode_mse /
 * tq_encode_prod would) into the cache at position t = seq_len[b], then the step attends as
 * tq_attn_decode over the t + 1 tokens 0..t, the new one included.  This is the step just before
 * the cache is read in a decode loop (the past_key_values update of the ai-navigate-news Gemma 4
 * post, section "セットアップ").  The encode runs inside the step's query preparation, so the step
 * launches the same kernels as tq_attn_decode.
 *   k_new, v_new: device [B, Hkv, d] of type xt (TQ_F32, TQ_BF16 or TQ_F16); d <= 512
 *   kcodes, knorms, kgammas, vcodes, vnorms, vgammas: the cache, as for tq_attn_decode, written at
 *     position seq_len[b] (row records, or one bit of each token-tiled word for TQ_LAYOUT_TILE32)
 *   seq_len: device [B] int32, the tokens already cached; read only: the caller advances it (e.g.
 *     seq_len += 1 on the same stream) before the next step.  A sequence with seq_len[b] >= Tstride
 *     has no room: nothing is written and its attention covers the Tstride cached tokens.
 *   ws, ws_bytes: as tq_attn_decode (tq_attn_decode_ws_bytes with the same Tstride)
 * Returns TQ_ERR_UNSUPPORTED for d > 512, otherwise as tq_attn_decode. */
int tq_attn_decode_append(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                          int Hkv, const void *k_new, const void *v_new, int xt, uint8_t *kcodes, uint16_t *knorms,
                          uint16_t *kgammas, uint8_t *vcodes, uint16_t *vnorms, uint16_t *vgammas, int vlayout,
                          int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *ws,
                          size_t ws_bytes, void *stream);

/* tq_attn_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments and result as tq_attn_decode
 * without ws/ws_bytes: the workspace is a device array of TQ_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU, held until the process ends.  The call allocates nothing; its first call on
 * a device looks up that device's array once.
 *   Returns TQ_ERR_WORKSPACE, launching nothing, when tq_attn_decode_ws_bytes(kq, B, Hq, Hkv,
 *   Tstride, vlayout) exceeds TQ_NOALLOC_SCRATCH_BYTES; TQ_ERR_INVALID when the current device is
 *   not the quantizer's.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other streams or
 * threads) race and must be ordered by the caller.  Nothing in the array needs to start at zero. */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_attn_decode_noalloc(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                           int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                           const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                           int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *stream);

/* Optional per-kernel timing.  When enabled, the library records a pair of
 * HIP events on the launch stream around every kernel it launches (a few
 * microseconds of overhead per launch); disabled by default.
 *   tq_profile_enable(on): on != 0 enables, 0 disables (recorded data kept).
 *   tq_profile_query(name, total_ms, count): waits for the recorded events and
 *     returns the summed elapsed time and number of launches whose name
 *     contains `name` (NULL or "" = all).  Launch names: attn_prep, attn_wave
 *     (the wave-streaming attention kernel), attn_fast (the 4-wave one),
 *     attn_wide (the eight-wave head-dim-512 one), attn_qrot_rows (query
 *     rotation at head dim 512), attn_qrot, attn_split (row records),
 *     attn_combine, encode_mse,
 *     encode_prod, encode_norm, encode_rotate, encode_qjl, decode, score_qrot,
 *     score_prep, score_scan, topk, tile_records.
 *   tq_profile_select(name): while enabled, records only the launches whose
 *     kernel name contains `name` (NULL or "" = all, the default), so a timed
 *     loop can bracket one kernel without events around its neighbours.
 *   tq_profile_reset(): drops all recorded launches.
 * Thread-safe; events are shared by all streams of the process. */
int tq_profile_enable(int on);
int tq_profile_select(const char *name);
int tq_profile_query(const char *name, double *total_ms, int64_t *count);
int tq_profile_reset(void);

/* Human-readable name of a status code (static string). */
const char *tq_status_str(int status);
/* hipError_t of the last HIP failure seen by this thread (0 if none). */
int tq_last_hip_error(void);
/* Library version, e.g. "0.1.0" (static string). */
const char *tq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TQ_H */
