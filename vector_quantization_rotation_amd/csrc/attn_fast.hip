// Fast decode attention on a TurboQuant cache: matrix cores on bit planes.
//
// Method (ai-navigate-news Gemma 4 post, section "仕組み（技術的）"): keys are
// Algorithm-1 records, values Algorithm-2 records; scores use the rotated query
// q' = Pi_K q, values are aggregated in the rotated and sign domains and
// rotated back once per head by the combine kernel.
//
// Kernel design (gfx950):
// * A symmetric b-bit Lloyd-Max codebook is an odd function of the index bits,
//   so with s_p = 2 bit_p - 1 it expands exactly over the odd-size subsets S of
//   the bit planes:  c[idx] = sum_S beta_S prod_{p in S} s_p  (2^(b-1) terms;
//   for b = 3: planes b0, b1, b2 and the parity b0^b1^b2).  Each term is a 0/1
//   bit plane, so <q', c[idx]> = 2 sum_S beta_S <q', bits_S> - c[L-1] sum_j q'_j.
// * Keys: a plane word (32 coordinates) feeds v_mfma_f32_16x16x128_f8f6f4 as
//   four fp4 dwords (x & 0x11111111, x & 0x22222222, x & 0x44444444: nibble
//   values 0.5, 1, 2 times the bit; (x & 0x88888888) | 0x11111111: 0.5 - bit);
//   the query images are four fixed-point e4m3 digits per head (one MFMA row
//   each) carrying the inverse nibble factor (-1 for the sign form, whose
//   constant the prep kernel takes off the score offset), and every digit row's
//   sum is exact (see split_fix4_e4m3).
// * Values: a 0/1 plane word feeds v_mfma_i32_16x16x64_i8 directly:
//   (w & 0x01010101 << k) holds four bits as bytes of value 2^k; the 2^-k is
//   folded into the softmax weights, which are split into signed byte digits,
//   one per MFMA row of a head, so integer accumulation is exact.
// * Keys stay in per-token records (their bits run along the contraction).
//   Values are read from the token-tiled layout (32 tokens per word) so that
//   the contraction over tokens also runs along the word bits.
// * attn_fast_kernel: each work-group of 4 waves owns a (batch, kv-head, head
//   group, sequence chunk) and walks it in 256-token steps: score (key pass),
//   turn the scores into int8 weight digits in LDS, aggregate (value pass);
//   online softmax with a rarely-moving reference maximum.  attn_wave_kernel
//   (head_dim 128, 1-bit value indices): one wave per work-group streams its
//   chunk in 64-token steps through a three-slot LDS ring.
#include <algorithm>
#include <type_traits>

#include <hip/hip_ext.h>

#include "append.cuh"
#include "common.cuh"

namespace tq {

constexpr int FA_THREADS = 256;
constexpr int FA_SUB = 256;     // chunk granularity: 4 waves x 64-token steps
constexpr int FA_GMAX = 4;      // query heads per work-group (16 MFMA rows = 4 heads x 4 splits)

struct FastAttnArgs {
  const int *qimg;          // [units][KP*(D/128)*2][64 lanes][4] int32 query operand images
  const float *qinfo;       // [units][FA_GMAX][2]: 1/S_q, c[L-1]*sum(q')
  const uint8_t *kcodes;    // [B, Hkv, Tstride, kcb]
  const uint16_t *knorms;   // [B, Hkv, Tstride]
  const uint32_t *vtiles;   // [B, Hkv, ntile, VPL, D]
  const uint16_t *vnorms, *vgammas;
  const int32_t *seq_len;
  float *part;              // [B*Hq, nsplit, 2 + 2D]
  int64_t Tstride, ntile;
  int Hq, Hkv, G, nsub, chunk, nsplit;
  int seq_add;              // 1 when the step appended a token at seq_len[b] (it is attended too)
  int kv_div;               // query rows per cache row: row b reads the keys and values of sequence b / kv_div
                            // (1 for decode; M for a prefill chunk of M query tokens, each its own row)
  float scale_log2, vqjl;
  float vbeta[4];           // Walsh coefficients of the value codebook (odd subsets)
  float kbeta[8];           // Walsh coefficients of the key codebook (applied after the MFMA when folded)
};


// With many Walsh planes per 128-coordinate block, keep one query image per block and apply the Walsh
// coefficients to the per-plane results instead, so the images fit in registers
__host__ __device__ constexpr bool fold_beta(int D, int KB) { return walsh_count(KB) * (D / 128) > 4; }
// workspace of the query images in KiB per unit (an fp8 image is 64 lanes x 32 B)
__host__ __device__ constexpr int key_images(int D, int KB) {
  return (fold_beta(D, KB) ? 1 : walsh_count(KB)) * (D / 128) * 2;
}
// waves per SIMD the 4-wave kernel is compiled for (registers without spills): also its resident
// work-groups per CU, one wave per SIMD each
__host__ __device__ constexpr int fa_waves_per_eu(int D, int KB, int VB) {
  return D > 256 ? 1 : D > 128 ? (VB >= 2 ? 1 : 2) : (KB == 4 && VB >= 2 ? 1 : (KB == 4 || VB >= 2) ? 2 : 3);
}

__device__ __forceinline__ float rows16_max(float v) {
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float rows16_sum(float v) {
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// fp4 dword of the sign-form key nibbles: bit 3 of every nibble of x kept as the sign of 0.5, so each
// nibble is worth 0.5 - bit.  With the 0.5 pattern `ones` (0x11111111) in a vector register this is one
// AND-OR (the instruction takes one scalar operand only, here the mask); written in C so that the
// compiler sees a vector instruction and keeps the wait states the matrix core needs before reading it
__device__ __forceinline__ int f4_sign_half(uint32_t x, uint32_t ones) { return (int)((x & 0x88888888u) | ones); }
// 0x11111111 in a vector register, opaque to the compiler so that it stays one
__device__ __forceinline__ uint32_t f4_ones_reg() {
  uint32_t c = 0x11111111u;
  asm volatile("" : "+v"(c));
  return c;
}

// ---------------------------------------------------------------------------
// value B operand: four registers of one tile word for token bits kofs..kofs+3
// of every byte.  Byte values are 2^k'(k) with k' = k except k = 3, 7 -> k - 1
// (the top bit of a byte is shifted down so every byte stays non-negative).
// ---------------------------------------------------------------------------
__device__ __forceinline__ intx4 value_bits(uint32_t w, int kofs) {
  intx4 r;
  r[0] = (int)(w & (0x01010101u << kofs));
  r[1] = (int)(w & (0x02020202u << kofs));
  r[2] = (int)(w & (0x04040404u << kofs));
  r[3] = (int)((w >> 1) & (0x04040404u << kofs));
  return r;
}
// raw buffer descriptor from wave-uniform values (forced into scalar registers)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)imin64(bytes, 0x7FFFFFFF));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0, n,
                                           0x00020000);
}

__device__ __forceinline__ int value_kexp(int kbit) { return ((kbit & 3) == 3) ? kbit - 1 : kbit; }

// prefetch helpers (descriptors by value so they stay in scalar registers)
template <int D, int KB>
__device__ __forceinline__ void fa_load_keys(uint32_t (&kw)[4][KB * (D / 128)], __amdgpu_buffer_rsrc_t rk, int vo,
                                             int so) {
  constexpr int KCB = KB * D / 8;
  so = __builtin_amdgcn_readfirstlane(so);
#pragma unroll
  for (int grp = 0; grp < 4; ++grp)
#pragma unroll
    for (int p = 0; p < KB; ++p)
#pragma unroll
      for (int wb = 0; wb < D / 128; ++wb)
        kw[grp][p * (D / 128) + wb] =
            __builtin_amdgcn_raw_buffer_load_b32(rk, vo + grp * 8 * KCB + p * (D / 8) + wb * 16, so, 0);
}

__device__ __forceinline__ void fa_load_norms(uint32_t &nk, uint32_t &nv, uint32_t &ng, __amdgpu_buffer_rsrc_t rkn,
                                              __amdgpu_buffer_rsrc_t rvn, __amdgpu_buffer_rsrc_t rvg, int vo, int so) {
  so = __builtin_amdgcn_readfirstlane(so);
  nk = __builtin_amdgcn_raw_buffer_load_b16(rkn, vo, so, 0);
  nv = __builtin_amdgcn_raw_buffer_load_b16(rvn, vo, so, 0);
  ng = __builtin_amdgcn_raw_buffer_load_b16(rvg, vo, so, 0);
}

template <int D, int VB>
__device__ __forceinline__ void fa_load_values(uint32_t (&vw)[4][D / 64][VB + 1], __amdgpu_buffer_rsrc_t rv, int vo,
                                               int so) {
  constexpr int VPL = VB + 1;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int st = __builtin_amdgcn_readfirstlane(so + tt * 2 * VPL * D * 4);
#pragma unroll
    for (int c = 0; c < D / 64; ++c)
#pragma unroll
      for (int p = 0; p < VPL; ++p) vw[tt][c][p] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo + (p * D + c * 16) * 4, st, 0);
  }
}

// The integer weight grid has a fixed step relative to the softmax reference, so a token far below
// the reference carries few significant bits.  When every score of a head in a whole step lies more
// than REF_DROP below the reference and the current fold segment is at least the kernel's minimum
// length, the reference moves down to that step's maximum (a fold), so that a long tail behind one
// dominant token is weighed on a grid set by its own scale.  The minimum length adapts: an upward
// move within twice that many steps of a downward one (scores that spread widely rather than a long
// low tail) doubles it, up to the kernel's maximum, so the moves stay rare where they buy nothing.  The reference never goes more than
// REF_SPAN below the highest score of the chunk, m_top (tokens further down weigh below 2^-REF_SPAN of
// that token): every weight is then at most 2^(REF_SPAN + slack) and a running sum over fewer than
// 2^31 tokens stays below 2^80 (fp32 has room to 2^128).
constexpr float REF_DROP = 8.f;
constexpr float REF_SPAN = 48.f;
// reference after a fold for one head: up to the step maximum smax when it exceeds the reference,
// down to it (no lower than m_top - REF_SPAN) when it lies more than REF_DROP below, else unchanged
__device__ __forceinline__ float moved_reference(float m_ref, float smax, float m_top, bool allow_down) {
  float m_new = fmaxf(m_ref, smax);
  if (allow_down && smax < m_ref - REF_DROP) m_new = fminf(m_ref, fmaxf(smax, m_top - REF_SPAN));
  return m_new;
}

constexpr float FA_SLACK = 1.f;     // score headroom above the reference maximum (log2 units)
constexpr float FA_NCAP = 1.25f;   // norm and gamma caps: this times the largest seen
constexpr float FA_HEADROOM = 2.f;  // 2^FA_SLACK
constexpr int FA_MINSEG = 2;        // fold segment length (256-token steps) before a downward move, at first
constexpr int FA_MAXSEG = 32;       // ... and at most
constexpr int FA_FOLDMAX = 512;     // steps between folds at most: the int32 digit sums stay below 2^30

// D: head dim; KB: key index bits; VB: value index bits (Algorithm-2 records hold VB+1 planes)
//
// Work-group = 4 waves over one (batch, kv head, head group, sequence chunk),
// walked in steps of 256 tokens.  In a step wave w scores tokens 64w..64w+63
// (all heads; fp8 x fp4 matrix cores as in the wave-streaming kernel), writes
// their int8 weight digits to LDS, and after a barrier
// aggregates all 256 tokens for its quarter of the value columns.  The next
// step's key words, norms and value words are loaded while the current step
// runs.  Softmax weights are scaled by a reference (running maximum, value norm
// and gamma caps) with headroom: scores may exceed the maximum by FA_SLACK
// (log2 units), the caps are FA_NCAP times the largest norm and gamma seen, and the
// weight scale is divided by 2^FA_SLACK.  The reference moves only when a step
// leaves that headroom; the int32 accumulators are folded into fp32 then.
template <int D, int KB, int VB>
__global__ __launch_bounds__(FA_THREADS) __attribute__((amdgpu_waves_per_eu(fa_waves_per_eu(D, KB, VB)))) void attn_fast_kernel(FastAttnArgs a) {
  constexpr int KP = walsh_count(KB);        // key Walsh planes
  constexpr int VMP = walsh_count(VB);       // value Walsh planes (index part)
  constexpr int VPL = VB + 1;                // stored value planes per tile
  constexpr int KW = D / 32;                 // 32-bit words per key plane
  constexpr int KWL = KB * (D / 128);        // key words per lane per 16-token group
  constexpr bool FOLD = fold_beta(D, KB);    // Walsh coefficients applied after the MFMA
  constexpr int NTW = D / 64;                // value column tiles per wave
  constexpr int KCB = KB * D / 8;            // key record bytes
  constexpr float WMAX = 268435328.f;        // 2^28 - 128: largest fp32 whose top 7-bit digit is 127

  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][4][16][64];  // weight digits [plane][token tile][row][slot]
  __shared__ float s_norm[4][2][64];                                   // per wave: n_V, gamma_V of its tokens
  __shared__ float s_kn[4][64];                                        // per wave: n_K
  __shared__ float s_max[4][FA_GMAX + 2];                              // per wave: score max per head, n_V max, gamma max
  __shared__ float s_merge[4][FA_GMAX][3];                             // per wave and head: l, Ym, Yq
  // per wave: bit 0 a score above the reference's headroom, bit 1 + h head h within REF_DROP of it, bit 5
  // a norm or gamma above its cap
  __shared__ int s_flag[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x, split = blockIdx.y;
  // (batch, kv-head) pairs; units = nbg x head subgroups, the subgroup slowest: the work-groups of one
  // pair's subgroups are nbg ids apart, so they land on the same XCD (work-groups go to the 8 XCDs
  // round-robin by id) and share its L2 when nbg is a multiple of 8
  const int nbg = (int)gridDim.x / a.nsub;
  const int sub = unit / nbg, bg = unit % nbg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = imin32(FA_GMAX, a.G - sub * FA_GMAX);
  // sequence length is wave-uniform: keep it (and everything derived) in scalar registers
  const int64_t T = imin64(imax64(__builtin_amdgcn_readfirstlane(a.seq_len[b]), 0) + a.seq_add, a.Tstride);
  const int64_t seq = (int64_t)(b / a.kv_div) * a.Hkv + g;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = imin64(T, c0 + a.chunk);

  const int hl = lane >> 4;      // head owned by this lane in score / accumulator layouts
  const int ln = lane & 15;      // token (score layout) or column (value layout) within 16
  const int kofs = (hl & 1) * 4; // value operand: token-bit offset of this lane group
  const bool head_ok = hl < gw;

  // query operand: e4m3 fixed-point digit images (4 heads x 4 digit rows), one per 128-coordinate block
  // (FOLD) or per (Walsh plane, block)
  constexpr int NI8 = (FOLD ? 1 : KP) * (D / 128);
  intx8 qa[NI8];
  {
    const intx8 *img = reinterpret_cast<const intx8 *>(a.qimg) + (int64_t)unit * NI8 * 64;
#pragma unroll
    for (int i = 0; i < NI8; ++i) qa[i] = img[i * 64 + lane];
  }
  const float qinv = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 0];
  const float qconst = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 1];

  // rows of heads >= gw stay zero for the whole chunk
  for (int i = tid; i < (int)sizeof(s_w) / 4; i += FA_THREADS) reinterpret_cast<uint32_t *>(&s_w[0][0][0][0])[i] = 0u;

  // buffer descriptors over this sequence (scalar registers); reads past the chunk end return 0
  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.kcodes + seq * a.Tstride * KCB, c1 * KCB);
  const __amdgpu_buffer_rsrc_t rkn = uniform_rsrc(a.knorms + seq * a.Tstride, c1 * 2);
  const __amdgpu_buffer_rsrc_t rvn = uniform_rsrc(a.vnorms + seq * a.Tstride, c1 * 2);
  const __amdgpu_buffer_rsrc_t rvg = uniform_rsrc(a.vgammas + seq * a.Tstride, c1 * 2);
  const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(a.vtiles + seq * a.ntile * VPL * D, ((c1 + 31) >> 5) * VPL * D * 4);
  const int vo_k = (64 * wave + 32 * (ln >> 3) + (ln & 7)) * KCB + hl * 4;  // per-lane, fixed
  const int vo_n = (64 * wave + lane) * 2;
  const int vo_v = ((hl >> 1) * VPL * D + wave * (NTW * 16) + ln) * 4;

  float m_ref = -INFINITY, vn_ref = 0.f, vg_ref = 0.f;  // work-group uniform (m_ref per lane head)
  float m_top = -INFINITY;                              // highest score of the chunk so far (per head)
  int since_fold = 0;
  int down_seg = FA_MINSEG;                             // segment length before a downward move
  int since_down = 1 << 30;                             // steps since the last downward move
  float l_run = 0.f, ym_run = 0.f, yq_run = 0.f;        // this lane's tokens, head hl
  float accf[VMP + 1][NTW];
  intx4 vacc[VMP + 1][NTW];
#pragma unroll
  for (int p = 0; p <= VMP; ++p)
#pragma unroll
    for (int c = 0; c < NTW; ++c) {
      accf[p][c] = 0.f;
      vacc[p][c] = intx4{0, 0, 0, 0};
    }

  // ---- prefetch registers ----
  uint32_t kw[4][KWL];
  uint32_t nk = 0, nv = 0, ng = 0;
  uint32_t vw[4][NTW][VPL];
  if (c0 < c1) {
    fa_load_keys<D, KB>(kw, rk, vo_k, (int)(c0 * KCB));
    fa_load_norms(nk, nv, ng, rkn, rvn, rvg, vo_n, (int)(c0 * 2));
    fa_load_values<D, VB>(vw, rv, vo_v, (int)((c0 >> 5) * VPL * D * 4));
  }
  // token of this wave's 64 scored by (group grp, lane): 32 (ln / 8) + 8 grp + ln % 8, so that a
  // lane's four tokens fill four consecutive bytes of the value operand's contraction slots
  const int tbase = 32 * (ln >> 3) + (ln & 7);
  const int slot = (2 * (ln >> 3) + ((ln & 7) >> 2)) * 16 + (ln & 3) * 4;  // byte offset of grp 0
  const float kscale = __builtin_amdgcn_ldexpf(1.f, -value_kexp(ln & 7));
  const uint32_t f4_ones = f4_ones_reg();
  for (int64_t s0 = c0; s0 < c1; s0 += FA_SUB) {
    const int64_t sn = s0 + FA_SUB;
    const int64_t wbase = s0 + 64 * wave;
    // ---- norms of this wave's tokens (lane = token) ----
    const float fvn = f16_to_f32((uint16_t)nv), fvg = f16_to_f32((uint16_t)ng);
    s_kn[wave][lane] = f16_to_f32((uint16_t)nk);
    s_norm[wave][0][lane] = fvn;
    s_norm[wave][1][lane] = fvg;
    // other lanes of this wave read these below: order the LDS writes before their reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- key pass: 4 groups of 16 tokens, fp8 query digits x fp4 key bits (a key word, coordinates
    // 128 wb + 32 hl + 0..31, becomes four fp4 dwords: nibble n of dword t holds bit b = bit 4 n + t,
    // at nibble bit t for t < 3 and as the sign of 0.5 for t = 3); exact fp32 sums per digit row ----
    float sc[4];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      floatx4 cacc[FOLD ? KP : 1];
#pragma unroll
      for (int p = 0; p < (FOLD ? KP : 1); ++p) cacc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int wb = 0; wb < D / 128; ++wb) {
        uint32_t w[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) w[p] = kw[grp][p * (D / 128) + wb];
        uint32_t wp[KP];
        walsh_planes<KB>(w, wp);
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          const uint32_t x = wp[p];
          intx8 bb;
          bb[0] = (int)(x & 0x11111111u);
          bb[1] = (int)(x & 0x22222222u);
          bb[2] = (int)(x & 0x44444444u);
          bb[3] = f4_sign_half(x, f4_ones);  // +-0.5: 0.5 - bit
          bb[4] = bb[5] = bb[6] = bb[7] = 0;  // an fp4 operand reads four registers only
          const int ai = FOLD ? wb : p * (D / 128) + wb;
          cacc[FOLD ? p : 0] =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ai], bb, cacc[FOLD ? p : 0], 0, 4, 0, 0, 0, 0);
        }
      }
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < (FOLD ? KP : 1); ++p) {  // digit rows: Q_d 2^-E_d = 1, 2^-4, 2^-9, 2^-14
        const float x = cacc[p][0] + (cacc[p][1] * 0.0625f + (cacc[p][2] * (1.f / 512.f) + cacc[p][3] * (1.f / 16384.f)));
        v = FOLD ? fmaf(2.f * a.kbeta[p], x, v) : x;
      }
      sc[grp] = v;
    }
    if (sn < c1) {  // key/norm registers are free now
      fa_load_keys<D, KB>(kw, rk, vo_k, (int)(sn * KCB));
      fa_load_norms(nk, nv, ng, rkn, rvn, rvg, vo_n, (int)(sn * 2));
    }
    const bool over_n = fvn > vn_ref || fvg > vg_ref;
    bool over = false;
    bool near = false;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int tw = tbase + 8 * grp;
      const bool ok = head_ok && (wbase + tw) < c1;
      sc[grp] = ok ? (sc[grp] * qinv - qconst) * s_kn[wave][tw] * a.scale_log2 : -INFINITY;
      over = over || sc[grp] > m_ref + FA_SLACK;
      near = near || sc[grp] >= m_ref - REF_DROP;
    }
    const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0ull;  // every lane votes
    const bool wave_over_n = __builtin_amdgcn_ballot_w64(over_n) != 0ull;
    const uint64_t wave_near = __builtin_amdgcn_ballot_w64(near);
    int flag = (wave_over ? 1 : 0) | (wave_over_n ? 32 : 0);
#pragma unroll
    for (int h = 0; h < FA_GMAX; ++h) flag |= ((wave_near >> (16 * h)) & 0xFFFFull) != 0 ? 2 << h : 0;
    if (lane == 0) s_flag[wave] = flag;
    __syncthreads();  // B1: flags visible; previous step's value pass done everywhere
    const int flags = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
    // a whole step (every token valid) in which some present head has no score within REF_DROP of the
    // reference, once the fold segment is FA_MINSEG steps long: move that reference down
    const bool whole = s0 + FA_SUB <= c1;
    ++since_fold;
    ++since_down;
    const bool low = whole && since_fold >= down_seg && ((flags >> 1) & ((1 << gw) - 1)) != ((1 << gw) - 1);
    if ((flags & 33) || low || since_fold >= FA_FOLDMAX) {
      if ((flags & 1) && since_down <= 2 * down_seg) down_seg = imin32(2 * down_seg, FA_MAXSEG);
      if (low) since_down = 0;
      // ---- rare: move the reference to this step's maxima and fold the int32 accumulators ----
      float smax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      smax = rows16_max(smax);
      const float vnm = wave_max_f32(fvn), vgm = wave_max_f32(fvg);
      if (ln == 0) s_max[wave][hl] = smax;
      if (lane == 0) { s_max[wave][FA_GMAX] = vnm; s_max[wave][FA_GMAX + 1] = vgm; }
      __syncthreads();
      float step_m = -INFINITY, step_vn = 0.f, step_vg = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        step_m = fmaxf(step_m, s_max[wv][hl]);
        step_vn = fmaxf(step_vn, s_max[wv][FA_GMAX]);
        step_vg = fmaxf(step_vg, s_max[wv][FA_GMAX + 1]);
      }
      m_top = fmaxf(m_top, step_m);
      const float m_new = moved_reference(m_ref, step_m, m_top, low);
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
      for (int p = 0; p <= VMP; ++p) {
        const float isc = p < VMP ? im : iq;
#pragma unroll
        for (int c = 0; c < NTW; ++c) {
          const float x = (((float)vacc[p][c][0] * 128.f + (float)vacc[p][c][1]) * 128.f + (float)vacc[p][c][2]) *
                              128.f + (float)vacc[p][c][3];
          accf[p][c] = (accf[p][c] + x * isc) * alpha;
          vacc[p][c] = intx4{0, 0, 0, 0};
        }
      }
      l_run *= alpha;
      ym_run *= alpha;
      yq_run *= alpha;
      m_ref = m_new;
      vn_ref = fmaxf(vn_ref, FA_NCAP * step_vn);
      vg_ref = fmaxf(vg_ref, FA_NCAP * step_vg);
      since_fold = 0;
    }
    // ---- weights: p = 2^(s - m_ref) <= 2^FA_SLACK; p n and p gamma as four 7-bit digits, one dword per digit row ----
    {
      const float sm = vn_ref > 0.f ? WMAX * kscale / (vn_ref * FA_HEADROOM) : 0.f;
      const float sq = vg_ref > 0.f ? WMAX * kscale / (vg_ref * FA_HEADROOM) : 0.f;
      const float ism = sm > 0.f ? 1.f / sm : 0.f, isq = sq > 0.f ? 1.f / sq : 0.f;
      uint32_t dm[4] = {0u, 0u, 0u, 0u}, dq[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int tw = tbase + 8 * grp;
        const float p = exp2f(sc[grp] - m_ref);
        const float wm = p * s_norm[wave][0][tw], wq = p * s_norm[wave][1][tw];
        l_run += p;
        const uint32_t um = __float2uint_rn(wm * sm), uq = __float2uint_rn(wq * sq);
        // value sums from the rounded weights the matrix cores use (see the wave-streaming kernel)
        ym_run = fmaf((float)um, ism, ym_run);
        yq_run = fmaf((float)uq, isq, yq_run);
        dm[0] |= (um >> 21) << (8 * grp);
        dm[1] |= ((um >> 14) & 127u) << (8 * grp);
        dm[2] |= ((um >> 7) & 127u) << (8 * grp);
        dm[3] |= (um & 127u) << (8 * grp);
        dq[0] |= (uq >> 21) << (8 * grp);
        dq[1] |= ((uq >> 14) & 127u) << (8 * grp);
        dq[2] |= ((uq >> 7) & 127u) << (8 * grp);
        dq[3] |= (uq & 127u) << (8 * grp);
      }
      if (head_ok) {
#pragma unroll
        for (int sp = 0; sp < 4; ++sp) {
          *reinterpret_cast<uint32_t *>(&s_w[0][wave][4 * hl + sp][slot]) = dm[sp];
          *reinterpret_cast<uint32_t *>(&s_w[1][wave][4 * hl + sp][slot]) = dq[sp];
        }
      }
    }
    __syncthreads();  // B2: weight digits of all 256 tokens visible
    // ---- value pass: 256 tokens x this wave's D/4 columns ----
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const intx4 wa_m = *reinterpret_cast<const intx4 *>(&s_w[0][tt][ln][16 * hl]);
      const intx4 wa_q = *reinterpret_cast<const intx4 *>(&s_w[1][tt][ln][16 * hl]);
#pragma unroll
      for (int c = 0; c < NTW; ++c) {
        uint32_t wpl[VMP];
        walsh_planes<VB>(vw[tt][c], wpl);
#pragma unroll
        for (int p = 0; p < VMP; ++p)
          vacc[p][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_m, value_bits(wpl[p], kofs), vacc[p][c], 0, 0, 0);
        vacc[VMP][c] =
            __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_q, value_bits(vw[tt][c][VB], kofs), vacc[VMP][c], 0, 0, 0);
      }
    }
    if (sn < c1) fa_load_values<D, VB>(vw, rv, vo_v, (int)((sn >> 5) * VPL * D * 4));
  }
  // ---- final fold, reductions, partial record: m, l, acc_mse[D], acc_qjl[D] ----
  {
    const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
    for (int p = 0; p <= VMP; ++p) {
      const float isc = p < VMP ? im : iq;
#pragma unroll
      for (int c = 0; c < NTW; ++c) {
        const float x = (((float)vacc[p][c][0] * 128.f + (float)vacc[p][c][1]) * 128.f + (float)vacc[p][c][2]) *
                            128.f + (float)vacc[p][c][3];
        accf[p][c] += x * isc;
      }
    }
  }
  l_run = rows16_sum(l_run);
  ym_run = rows16_sum(ym_run);
  yq_run = rows16_sum(yq_run);
  if (ln == 0) {
    s_merge[wave][hl][0] = l_run;
    s_merge[wave][hl][1] = ym_run;
    s_merge[wave][hl][2] = yq_run;
  }
  __syncthreads();
  if (head_ok) {
    float L = 0.f, YM = 0.f, YQ = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      L += s_merge[wv][hl][0];
      YM += s_merge[wv][hl][1];
      YQ += s_merge[wv][hl][2];
    }
    float *dst = a.part + (((int64_t)b * a.Hq + h0 + hl) * a.nsplit + split) * (2 + 2 * (int64_t)D);
    if (wave == 0 && ln == 0) { dst[0] = m_ref; dst[1] = L; }
#pragma unroll
    for (int c = 0; c < NTW; ++c) {
      const int col = (wave * NTW + c) * 16 + ln;
      float am = 0.f;
#pragma unroll
      for (int p = 0; p < VMP; ++p) am += a.vbeta[p] * (2.f * accf[p][c] - YM);
      dst[2 + col] = am;
      dst[2 + D + col] = a.vqjl * (2.f * accf[VMP][c] - YQ);
    }
  }
}

// ---------------------------------------------------------------------------
// Wave-streaming variant for head_dim 128 and 1-bit value indices (2-bit prod
// values): every wave is an independent stream over its own token range, with
// no work-group barrier anywhere in the loop.
//
// * Each 64-token step is staged into a wave-private three-slot LDS ring by
//   direct-to-LDS buffer loads issued two steps ahead (keys as 16-byte
//   plane rows, value tiles as they lie in HBM, the three fp16 arrays), so the
//   bytes in flight do not occupy registers.
// * Scores on the key Walsh planes as in attn_fast_kernel, but on the fp8 x fp4
//   matrix-core form (v_mfma_f32_16x16x128_f8f6f4): the query images are four
//   fixed-point digits per head held as e4m3 (about 20 bits in all, and the
//   sums the matrix cores form are exact), a key word of 32 coordinates becomes four
//   fp4 dwords with one AND each (three for nibble bits 0..2, and one more
//   after a shift for bit 3), so the key bits cost half the vector operations
//   of byte operands.
// * Value weights p n and p gamma become 24-bit integers split into three
//   signed byte digits (the integer XOR 0x808080 reads, byte by byte, as the
//   digit minus 128); row 3 of each head's four MFMA rows is a row of ones
//   that sums the value operand's bytes, which restores the 128 offsets
//   exactly.  The digit bytes of a lane's four tokens are gathered with byte
//   permutes.
// * The value operand shifts each tile word by the lane's 4-token offset so
//   every byte holds 1, 2, 4 or 8; the weights carry the inverse factor.
// * The online softmax reference (maximum, value norm and gamma caps) is per
//   wave and carries headroom: a score may exceed the reference maximum by
//   WV_SLACK (log2 units) and the caps are WV_NCAP times the largest norm and
//   gamma seen, with the weight scale divided by 2^WV_SLACK so the integers stay
//   below 2^23.  The int32 accumulators are folded into fp32 (as non-negative
//   unsigned digit sums, so without cancellation) only when a step leaves that
//   headroom, which after the first step is rare.
// * Software pipelining: a step's key pass (matrix-core work) is issued for the
//   next step before this step's softmax, so its MFMAs do not hold up the
//   vector work that follows; the stage ring refills a slot after its value
//   words are read.
// ---------------------------------------------------------------------------
constexpr int WV_STEP = 64;
constexpr float WV_SLACK = 1.f;           // score headroom above the reference maximum (log2 units)
constexpr float WV_NCAP = 1.25f;          // norm and gamma caps: this times the largest seen
constexpr float WV_HEADROOM = 2.f;        // 2^WV_SLACK
constexpr int WV_RING = 3;                // ring slots: stages s+1 and s+2 are in flight while s is used
constexpr float WV_WMAX = 8388352.f;      // 2^23 - 256: weights are integers below 2^23 (see wv_weight)
constexpr float WV_MAGIC = 8388608.f;     // 2^23
constexpr int WV_MINSEG = 8;              // fold segment length (steps) before a downward move, at first
constexpr int WV_MAXSEG = 128;            // ... and at most

typedef __attribute__((address_space(3))) void lds_void_t;

template <int KB>
struct WaveStage {
  static constexpr int KEYS = KB * 1024;   // [plane][64 token slots][16 B]
  static constexpr int VALS = 2 * 1024;    // [2 tiles][2 planes][128 coords] u32, as stored in HBM
  static constexpr int NORMS = 3 * 256;    // n_K, n_V, gamma_V: [64] fp16 each (+128 B landing zone)
  static constexpr int BYTES = KEYS + VALS + NORMS;
  static constexpr int NLOAD = KB + 2 + 3;  // load instructions per stage
};

// wait until at most n vector-memory loads of this wave are outstanding (loads complete in order)
template <int N>
__device__ __forceinline__ void wv_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// key slot of token t (0..63) in a stage: tokens t and t+32 sit side by side
__device__ __forceinline__ int wv_key_slot(int t) { return 2 * (t & 31) + (t >> 5); }

// direct-to-LDS loads of one stage: keys as 16-byte plane rows, the two value tiles, and the three
// fp16 arrays (lanes 0..31 fetch two tokens each; lanes 32..63 aim past every buffer, so they write
// zeros into the landing zone and fetch nothing).  Reads past the sequence end return zeros and
// touch no memory.
template <int KB>
__device__ __forceinline__ void wv_stage_load(uint8_t *stage, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                              __amdgpu_buffer_rsrc_t rkn, __amdgpu_buffer_rsrc_t rvn,
                                              __amdgpu_buffer_rsrc_t rvg, int lane, int voff_k, int voff_n,
                                              int64_t t0) {
  constexpr int KCB = KB * 16;
  using S = WaveStage<KB>;
  const int sk = __builtin_amdgcn_readfirstlane((int)(t0 * KCB));
#pragma unroll
  for (int p = 0; p < KB; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(stage + p * 1024), 16, voff_k + p * 16, sk, 0, 0);
  const int sv = __builtin_amdgcn_readfirstlane((int)((t0 >> 5) * 1024));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(stage + S::KEYS), 16, lane * 16, sv, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(stage + S::KEYS + 1024), 16, lane * 16 + 1024, sv, 0,
                                           0);
  const int sn = __builtin_amdgcn_readfirstlane((int)(t0 * 2));
  uint8_t *nb = stage + S::KEYS + S::VALS;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rkn, (lds_void_t *)(nb), 4, voff_n, sn, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rvn, (lds_void_t *)(nb + 256), 4, voff_n, sn, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rvg, (lds_void_t *)(nb + 512), 4, voff_n, sn, 0, 0);
}

// w s (0 <= w s < 2^23) rounded to the nearest integer, as the low three bytes of the result, each
// XOR 0x80: fma(w, s, 2^23) lands in [2^23, 2^24), where the fp32 spacing is 1, so its mantissa is the
// rounded integer (round to nearest even); the top byte is never read
__device__ __forceinline__ uint32_t wv_weight(float w, float s) {
  return __float_as_uint(fmaf(w, s, WV_MAGIC)) ^ 0x808080u;
}

// value operand: token bits 4c..4c+3 of every byte (c = lane group parity) as bytes 1, 2, 4, 8
__device__ __forceinline__ intx4 wv_value_bits(uint32_t w, int kofs) {
  const uint32_t x = w >> kofs;
  intx4 r;
  r[0] = (int)(x & 0x01010101u);
  r[1] = (int)(x & 0x02020202u);
  r[2] = (int)(x & 0x04040404u);
  r[3] = (int)(x & 0x08080808u);
  return r;
}

// bytes d of four 24-bit words -> one word per digit (byte g = digit of word g)
__device__ __forceinline__ void wv_digits(const uint32_t (&u)[4], uint32_t (&o)[3]) {
  const uint32_t lo01 = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
  const uint32_t lo23 = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
  const uint32_t hi23 = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
  o[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
}

// folded value of one head's four accumulator rows: digits 1, 2^8, 2^16, and the row of ones (the
// sum of the value operand's bytes) times the digit offset 0x808080.  Each digit row plus 128 times the
// row of ones is the sum of that digit's unsigned bytes (exact as a 32-bit unsigned integer, at most
// 2^31 within a fold), so the three terms added in fp32 are all non-negative: no cancellation
__device__ __forceinline__ float wv_fold(const intx4 &v) {
  const uint32_t o = (uint32_t)v[3] * 128u;
  const float u0 = (float)((uint32_t)v[0] + o), u1 = (float)((uint32_t)v[1] + o), u2 = (float)((uint32_t)v[2] + o);
  return fmaf(65536.f, u2, fmaf(256.f, u1, u0));
}

template <int KB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void attn_wave_kernel(FastAttnArgs a) {
  constexpr int D = 128;
  constexpr int KP = walsh_count(KB);
  constexpr int KCB = KB * D / 8;
  constexpr int NTC = D / 16;  // value column tiles
  using S = WaveStage<KB>;

  // one object per ring slot, so the compiler's waits for the direct-to-LDS loads stay per slot
  __shared__ __attribute__((aligned(16))) uint8_t s_ring0[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring1[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring2[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_w[2][16][64];  // weight digits [kind][row][token k]

  const int lane = threadIdx.x;
  const int hl = lane >> 4, ln = lane & 15;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int nbg = (int)gridDim.x / a.nsub;  // (batch, kv-head) pairs; units = nbg x head subgroups
  const int sub = unit / nbg, bg = unit % nbg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = imin32(FA_GMAX, a.G - sub * FA_GMAX);
  const bool head_ok = hl < gw;
  const int64_t T = imin64(imax64(__builtin_amdgcn_readfirstlane(a.seq_len[b]), 0) + a.seq_add, a.Tstride);
  const int64_t seq = (int64_t)(b / a.kv_div) * a.Hkv + g;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = imin64(T, c0 + a.chunk);
  // steps, padded to whole ring turns (padding steps hold no valid token and add nothing)
  const int nvalid = c0 < c1 ? (int)((c1 - c0 + WV_STEP - 1) / WV_STEP) : 0;
  const int nsteps = (nvalid + WV_RING - 1) / WV_RING * WV_RING;

  // query operand: per key image, 4 heads x 4 e4m3 digits over the 128 coordinates (32 bytes per lane)
  intx8 qa[KP];
  {
    const intx8 *img = reinterpret_cast<const intx8 *>(a.qimg) + (int64_t)unit * KP * 64;
#pragma unroll
    for (int i = 0; i < KP; ++i) qa[i] = img[i * 64 + lane];
  }
  // score in log2 units = (image sum * qinv - qconst) * n_K * scale_log2
  const float qinv2 = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 0] * a.scale_log2;
  const float qconst2 = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 1] * a.scale_log2;

  // digit rows start at zero (rows of absent heads stay so); row 4h+3 of both kinds is all ones
  for (int i = lane; i < 2 * 16 * 16; i += 64) {
    const int row = (i >> 4) & 15;
    reinterpret_cast<uint32_t *>(&s_w[0][0][0])[i] = (row & 3) == 3 ? 0x01010101u : 0u;
  }

  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.kcodes + seq * a.Tstride * KCB, c1 * KCB);
  // the fp16 arrays are fetched a dword (two tokens) at a time: round their ranges up to whole dwords
  // (the stride is a multiple of 8 tokens, so this stays inside the sequence's row)
  const int64_t nbytes = (c1 * 2 + 3) & ~(int64_t)3;
  const __amdgpu_buffer_rsrc_t rkn = uniform_rsrc(a.knorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvn = uniform_rsrc(a.vnorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvg = uniform_rsrc(a.vgammas + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(a.vtiles + seq * a.ntile * 2 * D, ((c1 + 31) >> 5) * 2 * D * 4);
  const int voff_k = (32 * (lane & 1) + (lane >> 1)) * KCB;
  const int voff_n = lane < 32 ? lane * 4 : 0x7FFFFF00;  // past every buffer's end for lanes 32..63

  float m_ref = -INFINITY, vn_ref = 0.f, vg_ref = 0.f;
  float m_top = -INFINITY;  // highest score of the chunk so far (per head)
  float l_run = 0.f, ym_run = 0.f, yq_run = 0.f;
  float accf[2][NTC];
  intx4 vacc[2][NTC];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int c = 0; c < NTC; ++c) {
      accf[k][c] = 0.f;
      vacc[k][c] = intx4{0, 0, 0, 0};
    }

  // this lane's tokens in a step: 32 (ln / 8) + (ln % 8) + 8 grp (grp = 0..3)
  const int tbase = 32 * (ln >> 3) + (ln & 7);
  const int slot = (2 * (ln >> 3) + ((ln & 7) >> 2)) * 16 + (ln & 3) * 4;  // byte of grp 0 in a digit row
  const float kscale = 1.f / (float)(1 << (ln & 3));
  const uint32_t f4_ones = f4_ones_reg();
  const int kofs = 4 * (hl & 1);
  int since_fold = 0;
  int down_seg = WV_MINSEG;   // segment length before a downward move
  int since_down = 1 << 30;   // steps since the last downward move
  float sm_l = 0.f, sq_l = 0.f;  // weight scales WV_WMAX 2^-r / (largest n_V, gamma_V so far)
  float ism_l = 0.f, isq_l = 0.f;  // their inverses (0 while a scale is 0)

  // key pass of one step on the stage in `stk`: its key words as fp4 operands against the query digits,
  // the digit-row sums in cacc (fp32, exact)
  auto key_mfma = [&](const uint8_t *stk, floatx4 (&cacc)[4]) {
    uint32_t kw[4][KB];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int ks = wv_key_slot(tbase + 8 * grp);
#pragma unroll
      for (int p = 0; p < KB; ++p) kw[grp][p] = *reinterpret_cast<const uint32_t *>(stk + p * 1024 + ks * 16 + hl * 4);
    }
    // (the four 16-token groups interleaved, so consecutive MFMAs are independent.  A key word,
    // coordinates 32 hl + 0..31, becomes four fp4 dwords: nibble n of dword t holds bit b = bit 4 n + t,
    // as 0.5 b, b, 2 b for t = 0, 1, 2 (one AND each) and as 0.5 - b for t = 3 (b in the sign, 0.5 set))
    uint32_t wp[4][KP];
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) walsh_planes<KB>(kw[grp], wp[grp]);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) cacc[grp] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const uint32_t x = wp[grp][p];
        intx8 bb;
        bb[0] = (int)(x & 0x11111111u);
        bb[1] = (int)(x & 0x22222222u);
        bb[2] = (int)(x & 0x44444444u);
        bb[3] = f4_sign_half(x, f4_ones);  // +-0.5: 0.5 - bit
        bb[4] = bb[5] = bb[6] = bb[7] = 0;  // an fp4 operand reads four registers only
        cacc[grp] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[p], bb, cacc[grp], 0, 4, 0, 0, 0, 0);
      }
  };
  float sc_next[4] = {0.f, 0.f, 0.f, 0.f};  // image sums of the next step's tokens
  auto digit_sum = [&](const floatx4 (&cacc)[4]) {
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)  // digit rows: Q_d 2^-E_d = 1, 2^-4, 2^-9, 2^-14
      sc_next[grp] = fmaf(fmaf(fmaf(cacc[grp][3], 1.f / 32.f, cacc[grp][2]), 1.f / 32.f, cacc[grp][1]), 0.0625f,
                          cacc[grp][0]);
  };

  // step s on the stage in `st` (a fixed ring slot after inlining): its softmax, then the key pass of step
  // s + 1 (stage in `stn`) and its own value pass back to back on the matrix cores, the next step's scores
  // formed from the key-pass sums at the end.  `whole` (a compile-time flag): all 64 tokens of the step are valid and every head of the
  // group is present, so no token or head is masked
  auto body = [&, rk, rkn, rvn, rvg, rv](auto whole, uint8_t *st, const uint8_t *stn, int s) {
    constexpr bool WHOLE = decltype(whole)::value;
    const int64_t t0 = c0 + (int64_t)s * WV_STEP;
    const uint16_t *nrm = reinterpret_cast<const uint16_t *>(st + S::KEYS + S::VALS);
    // every body issues one stage, so stages s + 1 and s + 2 are the only loads that may still be in
    // flight: stage s + 1 (the next key pass) has landed once no more than one stage is outstanding
    wv_wait_vm<S::NLOAD>();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t hn[3][4];  // fp16 of token tbase + 8 grp in the three arrays (128 halves apart)
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) hn[k][grp] = nrm[128 * k + tbase + 8 * grp];
    // ---- scores relative to the reference, d = s - m_ref, and the reference test ----
    float d[4], fvn[4], fvg[4], mn, mg;
    if constexpr (WHOLE) {
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        d[grp] = fmaf(fmaf(sc_next[grp], qinv2, -qconst2), f16_to_f32((uint16_t)hn[0][grp]), -m_ref);
      // the norms are non-negative fp16 numbers, ordered as their bit patterns
      auto umax = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
      mn = f16_to_f32((uint16_t)umax(umax(hn[1][0], hn[1][1]), umax(hn[1][2], hn[1][3])));
      mg = f16_to_f32((uint16_t)umax(umax(hn[2][0], hn[2][1]), umax(hn[2][2], hn[2][3])));
    } else {
      const int rem = (int)imax64(imin64(c1 - t0, WV_STEP), 0);  // valid tokens in this step
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const bool valid = tbase + 8 * grp < rem;
        const float dv = fmaf(fmaf(sc_next[grp], qinv2, -qconst2), f16_to_f32((uint16_t)hn[0][grp]), -m_ref);
        d[grp] = (head_ok && valid) ? dv : -INFINITY;
        fvn[grp] = valid ? f16_to_f32((uint16_t)hn[1][grp]) : 0.f;
        fvg[grp] = valid ? f16_to_f32((uint16_t)hn[2][grp]) : 0.f;
      }
      mn = fmaxf(fmaxf(fvn[0], fvn[1]), fmaxf(fvn[2], fvn[3]));
      mg = fmaxf(fmaxf(fvg[0], fvg[1]), fmaxf(fvg[2], fvg[3]));
    }
    const float dmax = fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3]));
    const uint64_t up = __builtin_amdgcn_ballot_w64(dmax > WV_SLACK);
    uint64_t over = up | __builtin_amdgcn_ballot_w64(mn > vn_ref) | __builtin_amdgcn_ballot_w64(mg > vg_ref);
    ++since_fold;
    ++since_down;
    bool down = false;
    if constexpr (WHOLE) {
      if (since_fold >= down_seg) {
        // a head (16 lanes) none of whose tokens comes within REF_DROP of the reference
        const uint64_t near = __builtin_amdgcn_ballot_w64(dmax >= -REF_DROP);
        down = (near & 0xFFFFull) == 0 || (near & 0xFFFF0000ull) == 0 || (near & 0xFFFF00000000ull) == 0 ||
               (near >> 48) == 0;
      }
    }
    if (over != 0ull || down || since_fold >= 16384) {
      if (up != 0ull && since_down <= 2 * down_seg) down_seg = imin32(2 * down_seg, WV_MAXSEG);
      if (down) since_down = 0;
      // rare: move the reference to this step's maxima and fold the integer accumulators (the scores
      // are formed again from their parts, n_K read again: d holds +inf while the reference is -inf)
      float sct[4];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        sct[grp] = d[grp] == -INFINITY ? -INFINITY
                                       : fmaf(sc_next[grp], qinv2, -qconst2) * f16_to_f32(nrm[tbase + 8 * grp]);
      const float smax = rows16_max(fmaxf(fmaxf(sct[0], sct[1]), fmaxf(sct[2], sct[3])));
      const float vnm = wave_max_f32(mn);
      const float vgm = wave_max_f32(mg);
      m_top = fmaxf(m_top, smax);
      const float m_new = moved_reference(m_ref, smax, m_top, down);
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      const float im = vn_ref * (WV_HEADROOM / WV_WMAX), iq = vg_ref * (WV_HEADROOM / WV_WMAX);
#pragma unroll
      for (int c = 0; c < NTC; ++c) {
        accf[0][c] = fmaf(wv_fold(vacc[0][c]), im, accf[0][c]) * alpha;
        accf[1][c] = fmaf(wv_fold(vacc[1][c]), iq, accf[1][c]) * alpha;
        vacc[0][c] = intx4{0, 0, 0, 0};
        vacc[1][c] = intx4{0, 0, 0, 0};
      }
      l_run *= alpha;
      ym_run *= alpha;
      yq_run *= alpha;
      m_ref = m_new;
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) d[grp] = sct[grp] - m_new;
      vn_ref = fmaxf(vn_ref, WV_NCAP * vnm);
      vg_ref = fmaxf(vg_ref, WV_NCAP * vgm);
      // p <= 2^WV_SLACK and n <= vn_ref, so p n sm_l <= WV_WMAX
      sm_l = vn_ref > 0.f ? WV_WMAX * kscale / (vn_ref * WV_HEADROOM) : 0.f;
      sq_l = vg_ref > 0.f ? WV_WMAX * kscale / (vg_ref * WV_HEADROOM) : 0.f;
      ism_l = sm_l > 0.f ? 1.f / sm_l : 0.f;
      isq_l = sq_l > 0.f ? 1.f / sq_l : 0.f;
      since_fold = 0;
    }
    // ---- weights: p n and p gamma as integers below 2^23, three signed byte digits per token ----
    {
      uint32_t bm[4], bq[4];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        // p = 2^(s - m_ref) <= 2^WV_SLACK (hardware exp2: results below 2^-126 flush to zero; after a
        // downward move p may exceed 1 only by the same headroom)
        const float p = __builtin_amdgcn_exp2f(d[grp]);
        l_run += p;
        // (whole steps: the fp16 norms enter the products as they are, in mixed-precision FMAs)
        float wm, wq;
        if constexpr (WHOLE) {
          wm = fmaf(p, f16_to_f32((uint16_t)hn[1][grp]), 0.f);
          wq = fmaf(p, f16_to_f32((uint16_t)hn[2][grp]), 0.f);
        } else {
          wm = p * fvn[grp];
          wq = p * fvg[grp];
        }
        bm[grp] = __float_as_uint(fmaf(wm, sm_l, WV_MAGIC));
        bq[grp] = __float_as_uint(fmaf(wq, sq_l, WV_MAGIC));
      }
      // the value sums take the rounded weights the matrix cores use, so a weight that rounds to zero
      // drops out of both terms of 2 acc - Y (an error of zero mean) instead of biasing every column:
      // the four integers (the low 23 bits of 2^23 + w) summed as integers, below 2^25
      ym_run = fmaf((float)(bm[0] + bm[1] + bm[2] + bm[3] - 4u * 0x4B000000u), ism_l, ym_run);
      yq_run = fmaf((float)(bq[0] + bq[1] + bq[2] + bq[3] - 4u * 0x4B000000u), isq_l, yq_run);
      // digit words (byte g = digit of token grp g), each byte XOR 0x80: the signed digit minus 128
      uint32_t dgm[3], dgq[3];
      wv_digits(bm, dgm);
      wv_digits(bq, dgq);
      if (WHOLE || head_ok) {
#pragma unroll
        for (int dd = 0; dd < 3; ++dd) {
          *reinterpret_cast<uint32_t *>(&s_w[0][4 * hl + dd][slot]) = dgm[dd] ^ 0x80808080u;
          *reinterpret_cast<uint32_t *>(&s_w[1][4 * hl + dd][slot]) = dgq[dd] ^ 0x80808080u;
        }
      }
    }
    // ---- the value words (four adjacent columns per read; column tile c of this lane is column
    // 64 (c / 4) + 4 ln + c % 4), the last reads of this slot: then refill it one ring turn ahead ----
    uint4 vw[2][2];  // [plane][column half]
    {
      const uint32_t *vt = reinterpret_cast<const uint32_t *>(st + S::KEYS) + (hl >> 1) * 256 + 4 * ln;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) vw[p][h] = *reinterpret_cast<const uint4 *>(vt + 128 * p + 64 * h);
    }
    // the optimizer takes a direct-to-LDS load for a write of a few bytes only, and could otherwise
    // move these reads below the refill of this slot: every value used after it is an input of a
    // volatile statement here, so its read has returned before the refill is issued (the slot's key
    // words were read, and used, by the previous step's key pass; its fp16 values above)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" ::"v"(vw[p][h].x), "v"(vw[p][h].y), "v"(vw[p][h].z), "v"(vw[p][h].w));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_s_waitcnt((0x3F & 15) | ((0x3F >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    wv_stage_load<KB>(st, rk, rv, rkn, rvn, rvg, lane, voff_k, voff_n, t0 + WV_RING * WV_STEP);
    __builtin_amdgcn_sched_barrier(0);
    // ---- key pass of step s + 1 (fp8 query digits x fp4 key bits), then the value pass of step s: the
    // matrix cores take both in turn while the vector units expand their bits ----
    floatx4 cacc[4];
    key_mfma(stn, cacc);
    // ---- value pass: 64 tokens x 128 columns, both kinds ----
    {
      const intx4 wa_m = *reinterpret_cast<const intx4 *>(&s_w[0][ln][16 * hl]);
      const intx4 wa_q = *reinterpret_cast<const intx4 *>(&s_w[1][ln][16 * hl]);
#pragma unroll
      for (int c = 0; c < NTC; ++c) {
        const uint32_t w0 = vw[0][c >> 2][c & 3], w1 = vw[1][c >> 2][c & 3];
        vacc[0][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_m, wv_value_bits(w0, kofs), vacc[0][c], 0, 0, 0);
        vacc[1][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_q, wv_value_bits(w1, kofs), vacc[1][c], 0, 0, 0);
      }
    }
    // the next step's image sums
    digit_sum(cacc);
  };

  if (nsteps > 0) {
    wv_stage_load<KB>(s_ring0, rk, rv, rkn, rvn, rvg, lane, voff_k, voff_n, c0);
    wv_stage_load<KB>(s_ring1, rk, rv, rkn, rvn, rvg, lane, voff_k, voff_n, c0 + WV_STEP);
    wv_stage_load<KB>(s_ring2, rk, rv, rkn, rvn, rvg, lane, voff_k, voff_n, c0 + 2 * WV_STEP);
    {  // the key pass of step 0, once stage 0 has landed
      wv_wait_vm<2 * S::NLOAD>();
      __builtin_amdgcn_sched_barrier(0);
      floatx4 cacc[4];
      key_mfma(s_ring0, cacc);
      digit_sum(cacc);
    }
    // (the last step's key pass reads the stage after the chunk: zeros, never used).  Whole ring turns
    // of whole steps first, then the rest with masking
    const int nwhole = gw == FA_GMAX && c1 > c0 ? (int)((c1 - c0) / WV_STEP) : 0;
    int s = 0;
    for (; s + WV_RING <= nwhole; s += WV_RING) {
      body(std::true_type{}, s_ring0, s_ring1, s);
      body(std::true_type{}, s_ring1, s_ring2, s + 1);
      body(std::true_type{}, s_ring2, s_ring0, s + 2);
    }
    for (; s < nsteps; s += WV_RING) {
      body(std::false_type{}, s_ring0, s_ring1, s);
      body(std::false_type{}, s_ring1, s_ring2, s + 1);
      body(std::false_type{}, s_ring2, s_ring0, s + 2);
    }
    wv_wait_vm<0>();  // the stages past the chunk have landed before the wave ends
  }
  // ---- final fold and partial record: m, l, acc_mse[D], acc_qjl[D] ----
  {
    const float im = vn_ref * (WV_HEADROOM / WV_WMAX), iq = vg_ref * (WV_HEADROOM / WV_WMAX);
#pragma unroll
    for (int c = 0; c < NTC; ++c) {
      accf[0][c] = fmaf(wv_fold(vacc[0][c]), im, accf[0][c]);
      accf[1][c] = fmaf(wv_fold(vacc[1][c]), iq, accf[1][c]);
    }
  }
  l_run = rows16_sum(l_run);
  ym_run = rows16_sum(ym_run);
  yq_run = rows16_sum(yq_run);
  if (head_ok) {
    float *dst = a.part + (((int64_t)b * a.Hq + h0 + hl) * a.nsplit + split) * (2 + 2 * (int64_t)D);
    if (ln == 0) { dst[0] = m_ref; dst[1] = l_run; }
#pragma unroll
    for (int c = 0; c < NTC; ++c) {
      const int col = 64 * (c >> 2) + 4 * ln + (c & 3);
      dst[2 + col] = a.vbeta[0] * (2.f * accf[0][c] - ym_run);
      dst[2 + D + col] = a.vqjl * (2.f * accf[1][c] - yq_run);
    }
  }
}

// ---------------------------------------------------------------------------
// Head dim 512 with 1-bit value indices (the global-layer shape): a work-group of WD_WAVES (four) waves
// walks steps of 16 tokens per wave (64) of one (batch, KV head, four-head group, chunk).
//
// * Each step is staged in LDS by direct-to-LDS loads issued two steps ahead into a three-slot ring:
//   the step's key records as they lie in HBM, its token-tiled value words per plane and coordinate,
//   and the three fp16 arrays.  Nothing in flight occupies registers, and the ring of a four-wave
//   work-group is small enough (67 KB at 3-bit keys) for two work-groups per CU: the two waves that share
//   a SIMD belong to different work-groups and are not held in step by barriers, so one's vector work
//   overlaps the other's matrix-core work.  Every wave loads an equal share of each stage and waits for
//   its own loads; a work-group barrier then makes the stage visible.
// * Wave w scores tokens 16 w .. 16 w + 15 of the step on the fp8 x fp4 matrix cores, one query image
//   per 128-coordinate block with the key codebook's Walsh coefficients applied to the per-plane sums
//   (at 1-bit keys, one plane, folded into the image), as attn_fast_kernel at this head dim.  Lane
//   group g of block wb carries key word 4 g + wb of a plane, so a lane reads the four blocks' words of
//   a plane as one 16-byte piece of the record; the query images follow the same order.
// * Each lane weighs one (head, token): p n and p gamma as 28-bit integers in four 7-bit digits written
//   to the byte of the value operand's contraction slot that holds the token's bit, then the step's
//   tokens are aggregated by every wave for its 128 value columns on the int8 matrix cores.
// * The softmax reference (running maximum per head, value norm and gamma caps, headroom, downward
//   moves behind a dominant token) is shared by the work-group as in attn_fast_kernel.
// ---------------------------------------------------------------------------
constexpr int WD_D = 512;
constexpr int WD_WAVES = 4;
constexpr int WD_STEP = 16 * WD_WAVES;  // tokens per step: 16 per wave
constexpr int WD_THREADS = 64 * WD_WAVES;
constexpr int WD_TT = WD_STEP / 64;     // 64-token tiles of the value operand per step
constexpr int WD_COLS = WD_D / WD_WAVES;  // value columns per wave
constexpr int WD_NH = WD_COLS / 64;     // 16-byte reads of a value word row per lane (4 columns each)
constexpr int WD_FOLDMAX = 1024; // steps between folds at most: the int32 digit sums stay below 2^31

template <int KB, int STEP = WD_STEP, int WAVES = WD_WAVES>
struct WideStage {
  static constexpr int KCB = KB * WD_D / 8;                    // key record bytes
  static constexpr int KEYS = STEP * KCB;                      // the step's key records
  static constexpr int VALS = (STEP / 32) * 2 * WD_D * 4;      // tile words x two planes x 512 coordinates
  static constexpr int NORMS = 4 * 256;                        // n_K, n_V, gamma_V (256 B each), a landing zone
  static constexpr int BYTES = KEYS + VALS + NORMS;
  static constexpr int KLOADS = KEYS / 1024 / WAVES;           // 1 KiB direct-to-LDS loads per wave
  static constexpr int VLOADS = VALS / 1024 / WAVES;
  static constexpr int NLOAD = KLOADS + VLOADS + 1;            // (+ one fp16 array, or a load of nothing)
  static_assert(KEYS % (1024 * WAVES) == 0 && VALS % (1024 * WAVES) == 0, "stage split");
  static_assert(STEP <= 128, "an fp16 array of a step fits one dword per lane");
};

// this wave's share of the loads of one stage (tokens t0 .. t0 + WD_STEP - 1).  Waves 0..2 fetch the three
// fp16 arrays, a dword (two tokens) per lane into 256-byte regions (lanes past the step's tokens, and the
// other waves, aim past every buffer: zeros into the region's tail or the stage's landing zone, no memory
// touched), so every wave issues the same number of loads, all into the one LDS object of the slot.  Reads
// past the chunk return zeros.
template <int KB, int STEP = WD_STEP, int WAVES = WD_WAVES>
__device__ __forceinline__ void wd_stage_load(uint8_t *stage, __amdgpu_buffer_rsrc_t rk,
                                              __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t rkn,
                                              __amdgpu_buffer_rsrc_t rvn, __amdgpu_buffer_rsrc_t rvg, int wave,
                                              int lane, int64_t t0) {
  using S = WideStage<KB, STEP, WAVES>;
  const int sk = __builtin_amdgcn_readfirstlane((int)(t0 * S::KCB));
#pragma unroll
  for (int i = 0; i < S::KLOADS; ++i) {
    const int e = wave * S::KLOADS + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(stage + e * 1024), 16, lane * 16 + e * 1024, sk, 0, 0);
  }
  const int sv = __builtin_amdgcn_readfirstlane((int)((t0 >> 5) * 2 * WD_D * 4));
#pragma unroll
  for (int i = 0; i < S::VLOADS; ++i) {
    const int e = wave * S::VLOADS + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t *)(stage + S::KEYS + e * 1024), 16, lane * 16 + e * 1024,
                                             sv, 0, 0);
  }
  const int sn = __builtin_amdgcn_readfirstlane((int)(t0 * 2));
  const bool real = wave < 3;
  const __amdgpu_buffer_rsrc_t rn = wave == 0 ? rkn : (wave == 1 ? rvn : rvg);
  const bool fetch = real && lane < STEP / 2;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rn, (lds_void_t *)(stage + S::KEYS + S::VALS + (real ? wave : 3) * 256), 4,
                                           fetch ? lane * 4 : 0x7FFFFF00, real ? sn : 0, 0, 0);
}

// every LDS access of this wave issued before has completed, then a work-group barrier (the
// wavefront-scope fences order the compiler's own LDS accesses around it without making it wait for the
// direct-to-LDS loads still in flight)
__device__ __forceinline__ void wd_barrier() {
  __builtin_amdgcn_s_waitcnt((0x3F & 15) | ((0x3F >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KB>
__global__ __launch_bounds__(WD_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void attn_wide_kernel(FastAttnArgs a) {
  constexpr int D = WD_D;
  constexpr int KP = walsh_count(KB);
  constexpr int NB = D / 128;        // 128-coordinate blocks
  constexpr bool FOLD = fold_beta(D, KB);  // one image per block, Walsh coefficients after the MFMA (2-3-bit keys)
  constexpr int NI8 = (FOLD ? 1 : KP) * NB;  // query images (1-bit keys: one per block, 2 beta folded in)
  constexpr int NTC = 4 * WD_NH;     // value columns of a lane: WD_COLS w + 64 (c / 4) + 4 ln + c % 4
  constexpr float WMAX = 268435328.f;  // 2^28 - 128 (see attn_fast_kernel)
  using S = WideStage<KB>;

  // one object per ring slot, so the compiler's waits for the direct-to-LDS loads stay per slot
  __shared__ __attribute__((aligned(16))) uint8_t s_ring0[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring1[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring2[S::BYTES];
  // weight digits [token tile][row][slot] of p n (s_wm) and p gamma (s_wq), two objects so that the compiler
  // keeps their accesses apart from the loads in flight
  __shared__ __attribute__((aligned(16))) uint8_t s_wm[WD_TT][16][64];
  __shared__ __attribute__((aligned(16))) uint8_t s_wq[WD_TT][16][64];
  __shared__ int s_flag[WD_WAVES];
  __shared__ float s_max[WD_WAVES][FA_GMAX + 2];
  __shared__ float s_merge[WD_WAVES][FA_GMAX][3];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 4, ln = lane & 15;
  const int kofs = (hl & 1) * 4;
  const int unit = blockIdx.x, split = blockIdx.y;
  const int nbg = (int)gridDim.x / a.nsub;
  const int sub = unit / nbg, bg = unit % nbg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = imin32(FA_GMAX, a.G - sub * FA_GMAX);
  const bool head_ok = hl < gw;
  const int64_t T = imin64(imax64(__builtin_amdgcn_readfirstlane(a.seq_len[b]), 0) + a.seq_add, a.Tstride);
  const int64_t seq = (int64_t)(b / a.kv_div) * a.Hkv + g;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = imin64(T, c0 + a.chunk);
  const int nvalid = c0 < c1 ? (int)((c1 - c0 + WD_STEP - 1) / WD_STEP) : 0;
  const int nsteps = (nvalid + 2) / 3 * 3;  // whole ring turns (steps past the chunk hold no valid token)

  intx8 qa[NI8];
  {
    const intx8 *img = reinterpret_cast<const intx8 *>(a.qimg) + (int64_t)unit * NI8 * 64;
#pragma unroll
    for (int i = 0; i < NI8; ++i) qa[i] = img[i * 64 + lane];
  }
  const float qinv2 = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 0] * a.scale_log2;
  const float qconst2 = a.qinfo[((int64_t)unit * FA_GMAX + hl) * 2 + 1] * a.scale_log2;
  for (int i = tid; i < (int)sizeof(s_wm) / 4; i += WD_THREADS) {
    reinterpret_cast<uint32_t *>(&s_wm[0][0][0])[i] = 0u;
    reinterpret_cast<uint32_t *>(&s_wq[0][0][0])[i] = 0u;
  }

  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.kcodes + seq * a.Tstride * S::KCB, c1 * S::KCB);
  const int64_t nbytes = (c1 * 2 + 3) & ~(int64_t)3;
  const __amdgpu_buffer_rsrc_t rkn = uniform_rsrc(a.knorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvn = uniform_rsrc(a.vnorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvg = uniform_rsrc(a.vgammas + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(a.vtiles + seq * a.ntile * 2 * D, ((c1 + 31) >> 5) * 2 * D * 4);

  float m_ref = -INFINITY, vn_ref = 0.f, vg_ref = 0.f, m_top = -INFINITY;
  int since_fold = 0, down_seg = FA_MINSEG, since_down = 1 << 30;
  float sm = 0.f, sq = 0.f, ism = 0.f, isq = 0.f;  // weight scales (set at each fold) and their inverses
  float l_run = 0.f, ym_run = 0.f, yq_run = 0.f;
  float accf[2][NTC];
  intx4 vacc[2][NTC];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int c = 0; c < NTC; ++c) {
      accf[p][c] = 0.f;
      vacc[p][c] = intx4{0, 0, 0, 0};
    }

  // this lane's token in a step and its place in the value operand: token tile tt, contraction slot
  // `slot` (lane group 2 (word) + (bit 2 of the token's bit), byte 4 (bit % 4) + bit / 8), byte value
  // 2^value_kexp(bit % 8), undone by kscale
  const int tw = 16 * wave + ln;
  const int tt = tw >> 6, tau = tw & 63, bitw = tau & 31, r8 = bitw & 7;
  const int slot = 16 * (2 * (tau >> 5) + (r8 >> 2)) + 4 * (r8 & 3) + (bitw >> 3);
  const float kscale = __builtin_amdgcn_ldexpf(1.f, -value_kexp(r8));
  const uint32_t f4_ones = f4_ones_reg();

  auto body = [&, rk, rv, rkn, rvn, rvg](uint8_t *st, uint8_t *stl, int s) {
    const int64_t t0 = c0 + (int64_t)s * WD_STEP;
    // this wave's loads of stage s have landed (stage s + 1 may still be in flight); after the barrier
    // everyone's have, and every wave is done with step s - 1, whose slot the loads of s + 2 take
    wv_wait_vm<S::NLOAD>();
    __builtin_amdgcn_sched_barrier(0);
    wd_barrier();
    // every read of the stage first (its key words, value words and fp16 values into registers), then the
    // loads of step s + 2: no LDS read of a ring slot follows a load in flight
    uint4 kw4[KB];
#pragma unroll
    for (int p = 0; p < KB; ++p) kw4[p] = *reinterpret_cast<const uint4 *>(st + tw * S::KCB + p * (D / 8) + 16 * hl);
    uint4 vw4[WD_TT][2][WD_NH];  // [token tile][plane][half]: 4 columns of this lane group's tile word each
#pragma unroll
    for (int t2 = 0; t2 < WD_TT; ++t2)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int hh = 0; hh < WD_NH; ++hh)
          vw4[t2][p][hh] = *reinterpret_cast<const uint4 *>(
              st + S::KEYS + ((2 * (2 * t2 + (hl >> 1)) + p) * D + WD_COLS * wave + 64 * hh + 4 * ln) * 4);
    const uint16_t *nrm = reinterpret_cast<const uint16_t *>(st + S::KEYS + S::VALS);
    const uint32_t hk = nrm[tw], hv = nrm[128 + tw], hg = nrm[256 + tw];
    __builtin_amdgcn_s_waitcnt((0x3F & 15) | ((0x3F >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0): the reads are done
    __builtin_amdgcn_sched_barrier(0);
    wd_stage_load<KB>(stl, rk, rv, rkn, rvn, rvg, wave, lane, t0 + 2 * WD_STEP);
    __builtin_amdgcn_sched_barrier(0);
    // ---- key pass: token tw against the four heads' query digits ----
    floatx4 cacc[FOLD ? KP : 1];
#pragma unroll
    for (int p = 0; p < (FOLD ? KP : 1); ++p) cacc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
    {
#pragma unroll
      for (int wb = 0; wb < NB; ++wb) {
        uint32_t w[KB];
#pragma unroll
        for (int p = 0; p < KB; ++p) w[p] = wb == 0 ? kw4[p].x : wb == 1 ? kw4[p].y : wb == 2 ? kw4[p].z : kw4[p].w;
        uint32_t wp[KP];
        walsh_planes<KB>(w, wp);
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          const uint32_t x = wp[p];
          intx8 bb;
          bb[0] = (int)(x & 0x11111111u);
          bb[1] = (int)(x & 0x22222222u);
          bb[2] = (int)(x & 0x44444444u);
          bb[3] = f4_sign_half(x, f4_ones);
          bb[4] = bb[5] = bb[6] = bb[7] = 0;
          const int ai = FOLD ? wb : p * NB + wb;
          cacc[FOLD ? p : 0] =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[ai], bb, cacc[FOLD ? p : 0], 0, 4, 0, 0, 0, 0);
        }
      }
    }
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < (FOLD ? KP : 1); ++p) {  // digit rows: Q_d 2^-E_d = 1, 2^-4, 2^-9, 2^-14
      const float x = cacc[p][0] + (cacc[p][1] * 0.0625f + (cacc[p][2] * (1.f / 512.f) + cacc[p][3] * (1.f / 16384.f)));
      v = FOLD ? fmaf(2.f * a.kbeta[p], x, v) : x;
    }
    const bool tvalid = t0 + tw < c1;
    const float fvn = tvalid ? f16_to_f32((uint16_t)hv) : 0.f;
    const float fvg = tvalid ? f16_to_f32((uint16_t)hg) : 0.f;
    float sc = (head_ok && tvalid) ? fmaf(v, qinv2, -qconst2) * f16_to_f32((uint16_t)hk) : -INFINITY;
    // ---- reference test (the work-group's flags) and the weight of (head hl, token tw) against the current
    // reference, p n and p gamma as four 7-bit digits each; one barrier publishes both.  When the flags
    // call for a fold (rare after the first step) the reference moves and the weight is made again. ----
    {
      const bool over = sc > m_ref + FA_SLACK;
      const bool near = sc >= m_ref - REF_DROP;
      const bool over_n = fvn > vn_ref || fvg > vg_ref;
      const bool wave_over = __builtin_amdgcn_ballot_w64(over) != 0ull;
      const bool wave_over_n = __builtin_amdgcn_ballot_w64(over_n) != 0ull;
      const uint64_t wave_near = __builtin_amdgcn_ballot_w64(near);
      int flag = (wave_over ? 1 : 0) | (wave_over_n ? 32 : 0);
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) flag |= ((wave_near >> (16 * h)) & 0xFFFFull) != 0 ? 2 << h : 0;
      if (lane == 0) s_flag[wave] = flag;
    }
    float p;
    uint32_t um, uq;
    auto weigh = [&]() {
      p = sc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc - m_ref);
      um = __float2uint_rn(p * fvn * sm);
      uq = __float2uint_rn(p * fvg * sq);
      if (head_ok) {
        s_wm[tt][4 * hl + 0][slot] = (uint8_t)(um >> 21);
        s_wm[tt][4 * hl + 1][slot] = (uint8_t)((um >> 14) & 127u);
        s_wm[tt][4 * hl + 2][slot] = (uint8_t)((um >> 7) & 127u);
        s_wm[tt][4 * hl + 3][slot] = (uint8_t)(um & 127u);
        s_wq[tt][4 * hl + 0][slot] = (uint8_t)(uq >> 21);
        s_wq[tt][4 * hl + 1][slot] = (uint8_t)((uq >> 14) & 127u);
        s_wq[tt][4 * hl + 2][slot] = (uint8_t)((uq >> 7) & 127u);
        s_wq[tt][4 * hl + 3][slot] = (uint8_t)(uq & 127u);
      }
    };
    weigh();
    wd_barrier();  // flags and weight digits visible
    int flags = 0;
#pragma unroll
    for (int w = 0; w < WD_WAVES; ++w) flags |= s_flag[w];
    const bool whole = t0 + WD_STEP <= c1;
    ++since_fold;
    ++since_down;
    const bool low = whole && since_fold >= down_seg && ((flags >> 1) & ((1 << gw) - 1)) != ((1 << gw) - 1);
    if ((flags & 33) || low || since_fold >= WD_FOLDMAX) {
      if ((flags & 1) && since_down <= 2 * down_seg) down_seg = imin32(2 * down_seg, FA_MAXSEG);
      if (low) since_down = 0;
      // move the reference to this step's maxima and fold the int32 accumulators
      const float smax = rows16_max(sc);
      const float vnm = wave_max_f32(fvn), vgm = wave_max_f32(fvg);
      if (ln == 0) s_max[wave][hl] = smax;
      if (lane == 0) { s_max[wave][FA_GMAX] = vnm; s_max[wave][FA_GMAX + 1] = vgm; }
      wd_barrier();
      float step_m = -INFINITY, step_vn = 0.f, step_vg = 0.f;
#pragma unroll
      for (int w = 0; w < WD_WAVES; ++w) {
        step_m = fmaxf(step_m, s_max[w][hl]);
        step_vn = fmaxf(step_vn, s_max[w][FA_GMAX]);
        step_vg = fmaxf(step_vg, s_max[w][FA_GMAX + 1]);
      }
      m_top = fmaxf(m_top, step_m);
      const float m_new = moved_reference(m_ref, step_m, m_top, low);
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const float isc = pl == 0 ? im : iq;
#pragma unroll
        for (int c = 0; c < NTC; ++c) {
          const float x = (((float)vacc[pl][c][0] * 128.f + (float)vacc[pl][c][1]) * 128.f + (float)vacc[pl][c][2]) *
                              128.f + (float)vacc[pl][c][3];
          accf[pl][c] = (accf[pl][c] + x * isc) * alpha;
          vacc[pl][c] = intx4{0, 0, 0, 0};
        }
      }
      l_run *= alpha;
      ym_run *= alpha;
      yq_run *= alpha;
      m_ref = m_new;
      vn_ref = fmaxf(vn_ref, FA_NCAP * step_vn);
      vg_ref = fmaxf(vg_ref, FA_NCAP * step_vg);
      // p <= 2^FA_SLACK and n <= vn_ref, so p n sm <= WMAX kscale
      sm = vn_ref > 0.f ? WMAX * kscale / (vn_ref * FA_HEADROOM) : 0.f;
      sq = vg_ref > 0.f ? WMAX * kscale / (vg_ref * FA_HEADROOM) : 0.f;
      ism = sm > 0.f ? 1.f / sm : 0.f;
      isq = sq > 0.f ? 1.f / sq : 0.f;
      since_fold = 0;
      weigh();       // against the moved reference
      wd_barrier();  // the new digits visible
    }
    l_run += p;
    ym_run = fmaf((float)um, ism, ym_run);
    yq_run = fmaf((float)uq, isq, yq_run);
    // ---- value pass: the step's tokens x this wave's columns, both kinds ----
    {
#pragma unroll
      for (int t2 = 0; t2 < WD_TT; ++t2) {
        const intx4 wa_m = *reinterpret_cast<const intx4 *>(&s_wm[t2][ln][16 * hl]);
        const intx4 wa_q = *reinterpret_cast<const intx4 *>(&s_wq[t2][ln][16 * hl]);
        uint32_t x0[NTC], x1[NTC];
#pragma unroll
        for (int hh = 0; hh < WD_NH; ++hh) {
          const uint4 w0 = vw4[t2][0][hh], w1 = vw4[t2][1][hh];
          x0[4 * hh] = w0.x; x0[4 * hh + 1] = w0.y; x0[4 * hh + 2] = w0.z; x0[4 * hh + 3] = w0.w;
          x1[4 * hh] = w1.x; x1[4 * hh + 1] = w1.y; x1[4 * hh + 2] = w1.z; x1[4 * hh + 3] = w1.w;
        }
#pragma unroll
        for (int c = 0; c < NTC; ++c) {
          vacc[0][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_m, value_bits(x0[c], kofs), vacc[0][c], 0, 0, 0);
          vacc[1][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_q, value_bits(x1[c], kofs), vacc[1][c], 0, 0, 0);
        }
      }
    }
  };

  if (nsteps > 0) {
    wd_stage_load<KB>(s_ring0, rk, rv, rkn, rvn, rvg, wave, lane, c0);
    wd_stage_load<KB>(s_ring1, rk, rv, rkn, rvn, rvg, wave, lane, c0 + WD_STEP);
    // the query images and offsets (loaded before the stages; loads complete in order) are in registers
    // before the loop, so no wait inside it has to cover them
    wv_wait_vm<2 * S::NLOAD>();
    for (int s = 0; s < nsteps; s += 3) {
      body(s_ring0, s_ring2, s);
      body(s_ring1, s_ring0, s + 1);
      body(s_ring2, s_ring1, s + 2);
    }
    wv_wait_vm<0>();  // the last two stages' loads (past the chunk) have landed before the work-group ends
  }
  // ---- final fold, reductions, partial record: m, l, acc_mse[D], acc_qjl[D] ----
  {
    const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float isc = p == 0 ? im : iq;
#pragma unroll
      for (int c = 0; c < NTC; ++c) {
        const float x = (((float)vacc[p][c][0] * 128.f + (float)vacc[p][c][1]) * 128.f + (float)vacc[p][c][2]) *
                            128.f + (float)vacc[p][c][3];
        accf[p][c] += x * isc;
      }
    }
  }
  l_run = rows16_sum(l_run);
  ym_run = rows16_sum(ym_run);
  yq_run = rows16_sum(yq_run);
  if (ln == 0) {
    s_merge[wave][hl][0] = l_run;
    s_merge[wave][hl][1] = ym_run;
    s_merge[wave][hl][2] = yq_run;
  }
  wd_barrier();
  if (head_ok) {
    float L = 0.f, YM = 0.f, YQ = 0.f;
#pragma unroll
    for (int w = 0; w < WD_WAVES; ++w) {
      L += s_merge[w][hl][0];
      YM += s_merge[w][hl][1];
      YQ += s_merge[w][hl][2];
    }
    float *dst = a.part + (((int64_t)b * a.Hq + h0 + hl) * a.nsplit + split) * (2 + 2 * (int64_t)D);
    if (wave == 0 && ln == 0) { dst[0] = m_ref; dst[1] = L; }
#pragma unroll
    for (int c = 0; c < NTC; ++c) {
      const int col = WD_COLS * wave + 64 * (c >> 2) + 4 * ln + (c & 3);
      dst[2 + col] = a.vbeta[0] * (2.f * accf[0][c] - YM);
      dst[2 + D + col] = a.vqjl * (2.f * accf[1][c] - YQ);
    }
  }
}

// ---------------------------------------------------------------------------
// attn_wide8_kernel<KB>: head dim 512, eight query heads per KV head (the global-layer shape), 1-bit value
// indices.  One work-group of eight waves serves both four-head groups of a (batch, KV head, chunk), so the
// key bits of a token are expanded into fp4 operands once for eight heads and the value bits into int8
// operands once for both groups' weight digits (attn_wide_kernel runs a work-group per head group and
// expands them twice).
// * Steps of 128 tokens, staged by direct-to-LDS loads two steps ahead into a three-slot ring as in
//   attn_wide_kernel (each wave an equal share of every stage).
// * Key pass: wave w scores tokens 16w..16w+15 against both groups' query digits (their images in LDS,
//   two MFMAs per fp4 operand).  Lane (head h, token) holds the scores of head h of group 0 and of group 1.
// * Each lane weighs its token for both heads into the digit rows of the two groups' value operands; the
//   softmax reference is kept per head as in attn_wide_kernel, the norm caps per work-group.
// * Value pass: wave w aggregates the step's 128 tokens for value columns 64w..64w+63, each int8 operand of
//   value bits against both groups' weight digits.
// ---------------------------------------------------------------------------
constexpr int W8_WAVES = 8;
constexpr int W8_STEP = 16 * W8_WAVES;  // tokens per step: 16 per wave
constexpr int W8_THREADS = 64 * W8_WAVES;
constexpr int W8_TT = W8_STEP / 64;     // 64-token tiles of the value operand per step
constexpr int W8_COLS = WD_D / W8_WAVES;  // value columns per wave
constexpr int W8_NTC = W8_COLS / 16;    // value column tiles per wave (4 columns of a lane each)

template <int KB>
__global__ __launch_bounds__(W8_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void attn_wide8_kernel(FastAttnArgs a) {
  constexpr int D = WD_D;
  constexpr int KP = walsh_count(KB);
  constexpr int NB = D / 128;
  constexpr bool FOLD = fold_beta(D, KB);
  constexpr int NI8 = (FOLD ? 1 : KP) * NB;  // query images per head group
  constexpr int NC = FOLD ? KP : 1;          // accumulators of the key pass per group
  constexpr float WMAX = 268435328.f;        // 2^28 - 128 (see attn_fast_kernel)
  using S = WideStage<KB, W8_STEP, W8_WAVES>;
  static_assert(W8_TT == 2 && W8_NTC == 4, "layout below");

  __shared__ __attribute__((aligned(16))) uint8_t s_ring0[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring1[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t s_ring2[S::BYTES];
  // flat arrays indexed in one step: the compiler keeps an LDS access apart from the direct-to-LDS loads in
  // flight only when it can trace the address to its array through a few address computations
  __shared__ __attribute__((aligned(16))) intx4 s_qa[2 * NI8 * 64 * 2];      // [group][image][lane][half]
  __shared__ __attribute__((aligned(16))) uint8_t s_wm[2 * W8_TT * 16 * 64];  // [group][tile][digit row][slot]
  __shared__ __attribute__((aligned(16))) uint8_t s_wq[2 * W8_TT * 16 * 64];
  // the small exchanges in one object (the compiler keeps LDS objects apart from the direct-to-LDS loads in
  // flight only while a kernel has few of them)
  struct Small {
    int flag[W8_WAVES];
    float max[W8_WAVES][2][FA_GMAX];
    float maxn[W8_WAVES][2];
    float merge[W8_WAVES][2][FA_GMAX][3];
  };
  __shared__ Small s_sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 4, ln = lane & 15;
  const int kofs = (hl & 1) * 4;
  const int nbg = (int)gridDim.x, bg = blockIdx.x, split = blockIdx.y;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int64_t T = imin64(imax64(__builtin_amdgcn_readfirstlane(a.seq_len[b]), 0) + a.seq_add, a.Tstride);
  const int64_t seq = (int64_t)(b / a.kv_div) * a.Hkv + g;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = imin64(T, c0 + a.chunk);
  const int nvalid = c0 < c1 ? (int)((c1 - c0 + W8_STEP - 1) / W8_STEP) : 0;
  const int nsteps = (nvalid + 2) / 3 * 3;  // whole ring turns

  // the two head groups' images (units g_sub * nbg + bg of the prep kernel) into LDS, one intx8 a thread
  {
    const int gs = tid >> 8, i = (tid >> 6) & 3, l = tid & 63;
    static_assert(NI8 == 4, "one image per thread and group");
    const intx8 *img = reinterpret_cast<const intx8 *>(a.qimg) + ((int64_t)(gs * nbg + bg) * NI8 + i) * 64;
    const intx8 v = img[l];
    const int o = ((gs * NI8 + i) * 64 + l) * 2;
    s_qa[o] = intx4{v[0], v[1], v[2], v[3]};
    s_qa[o + 1] = intx4{v[4], v[5], v[6], v[7]};
  }
  float qinv2[2], qconst2[2];
#pragma unroll
  for (int gs = 0; gs < 2; ++gs) {
    const int64_t u = (int64_t)gs * nbg + bg;
    qinv2[gs] = a.qinfo[(u * FA_GMAX + hl) * 2 + 0] * a.scale_log2;
    qconst2[gs] = a.qinfo[(u * FA_GMAX + hl) * 2 + 1] * a.scale_log2;
  }

  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.kcodes + seq * a.Tstride * S::KCB, c1 * S::KCB);
  const int64_t nbytes = (c1 * 2 + 3) & ~(int64_t)3;
  const __amdgpu_buffer_rsrc_t rkn = uniform_rsrc(a.knorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvn = uniform_rsrc(a.vnorms + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rvg = uniform_rsrc(a.vgammas + seq * a.Tstride, nbytes);
  const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(a.vtiles + seq * a.ntile * 2 * D, ((c1 + 31) >> 5) * 2 * D * 4);

  // per head (lane's head hl of group 0 and of group 1): reference, top score, running sums
  float m_ref[2] = {-INFINITY, -INFINITY}, m_top[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f}, ym_run[2] = {0.f, 0.f}, yq_run[2] = {0.f, 0.f};
  float vn_ref = 0.f, vg_ref = 0.f;  // norm and gamma caps of the work-group
  int since_fold = 0, down_seg = FA_MINSEG, since_down = 1 << 30;
  float sm = 0.f, sq = 0.f, ism = 0.f, isq = 0.f;
  float accf[2][2][W8_NTC];
  intx4 vacc[2][2][W8_NTC];  // [group][plane][column tile]
#pragma unroll
  for (int gs = 0; gs < 2; ++gs)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < W8_NTC; ++c) {
        accf[gs][p][c] = 0.f;
        vacc[gs][p][c] = intx4{0, 0, 0, 0};
      }

  // this lane's token in a step and its slot in the value operand (as attn_wide_kernel)
  const int tw = 16 * wave + ln;
  const int tt = tw >> 6, tau = tw & 63, bitw = tau & 31, r8 = bitw & 7;
  const int slot = 16 * (2 * (tau >> 5) + (r8 >> 2)) + 4 * (r8 & 3) + (bitw >> 3);
  const float kscale = __builtin_amdgcn_ldexpf(1.f, -value_kexp(r8));
  const uint32_t f4_ones = f4_ones_reg();

  auto body = [&, rk, rv, rkn, rvn, rvg](uint8_t *st, uint8_t *stl, int s) {
    const int64_t t0 = c0 + (int64_t)s * W8_STEP;
    wv_wait_vm<S::NLOAD>();
    __builtin_amdgcn_sched_barrier(0);
    wd_barrier();
    // the stage into registers first, then the loads of step s + 2 into the slot step s - 1 used
    uint4 kw4[KB];
#pragma unroll
    for (int p = 0; p < KB; ++p) kw4[p] = *reinterpret_cast<const uint4 *>(st + tw * S::KCB + p * (D / 8) + 16 * hl);
    uint4 vw4[W8_TT][2];  // [token tile][plane]: 4 columns of this lane group's tile word
#pragma unroll
    for (int t2 = 0; t2 < W8_TT; ++t2)
#pragma unroll
      for (int p = 0; p < 2; ++p)
        vw4[t2][p] = *reinterpret_cast<const uint4 *>(
            st + S::KEYS + ((2 * (2 * t2 + (hl >> 1)) + p) * D + W8_COLS * wave + 4 * ln) * 4);
    const uint16_t *nrm = reinterpret_cast<const uint16_t *>(st + S::KEYS + S::VALS);
    const uint32_t hk = nrm[tw], hv = nrm[128 + tw], hg = nrm[256 + tw];
    // ---- key pass: token tw against both groups' query digits (their images read from LDS before the
    // loads of step s + 2 are issued, so that no LDS read waits for loads in flight) ----
    floatx4 cacc[2][NC];
#pragma unroll
    for (int gs = 0; gs < 2; ++gs)
#pragma unroll
      for (int p = 0; p < NC; ++p) cacc[gs][p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wb = 0; wb < NB; ++wb) {
      uint32_t w[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) w[p] = wb == 0 ? kw4[p].x : wb == 1 ? kw4[p].y : wb == 2 ? kw4[p].z : kw4[p].w;
      uint32_t wp[KP];
      walsh_planes<KB>(w, wp);
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const uint32_t x = wp[p];
        intx8 bb;
        bb[0] = (int)(x & 0x11111111u);
        bb[1] = (int)(x & 0x22222222u);
        bb[2] = (int)(x & 0x44444444u);
        bb[3] = f4_sign_half(x, f4_ones);
        bb[4] = bb[5] = bb[6] = bb[7] = 0;
        const int ai = FOLD ? wb : p * NB + wb;
#pragma unroll
        for (int gs = 0; gs < 2; ++gs) {
          // (read as two 16-byte halves: a 32-byte LDS read is split by the compiler into accesses it can no
          // longer tell from the direct-to-LDS loads in flight)
          const int o = ((gs * NI8 + ai) * 64 + lane) * 2;
          const intx4 q0 = s_qa[o], q1 = s_qa[o + 1];
          const intx8 qv = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          cacc[gs][FOLD ? p : 0] =
              __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qv, bb, cacc[gs][FOLD ? p : 0], 0, 4,
                                                               0, 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt((0x3F & 15) | ((0x3F >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0): the reads are done
    __builtin_amdgcn_sched_barrier(0);
    wd_stage_load<KB, W8_STEP, W8_WAVES>(stl, rk, rv, rkn, rvn, rvg, wave, lane, t0 + 2 * W8_STEP);
    __builtin_amdgcn_sched_barrier(0);
    const bool tvalid = t0 + tw < c1;
    const float fvn = tvalid ? f16_to_f32((uint16_t)hv) : 0.f;
    const float fvg = tvalid ? f16_to_f32((uint16_t)hg) : 0.f;
    const float fkn = f16_to_f32((uint16_t)hk);
    float sc[2];
#pragma unroll
    for (int gs = 0; gs < 2; ++gs) {
      float v = 0.f;
#pragma unroll
      for (int p = 0; p < NC; ++p) {  // digit rows: Q_d 2^-E_d = 1, 2^-4, 2^-9, 2^-14
        const float x = cacc[gs][p][0] +
                        (cacc[gs][p][1] * 0.0625f + (cacc[gs][p][2] * (1.f / 512.f) + cacc[gs][p][3] * (1.f / 16384.f)));
        v = FOLD ? fmaf(2.f * a.kbeta[p], x, v) : x;
      }
      sc[gs] = tvalid ? fmaf(v, qinv2[gs], -qconst2[gs]) * fkn : -INFINITY;
    }
    // ---- reference test (flags of the work-group): bit 0 a score above a reference's headroom, bit 1 + 4 gs
    // + h head h of group gs within REF_DROP of its reference, bit 9 a norm or gamma above its cap ----
    {
      const bool over = sc[0] > m_ref[0] + FA_SLACK || sc[1] > m_ref[1] + FA_SLACK;
      const bool over_n = fvn > vn_ref || fvg > vg_ref;
      const uint64_t near0 = __builtin_amdgcn_ballot_w64(sc[0] >= m_ref[0] - REF_DROP);
      const uint64_t near1 = __builtin_amdgcn_ballot_w64(sc[1] >= m_ref[1] - REF_DROP);
      int flag = (__builtin_amdgcn_ballot_w64(over) != 0ull ? 1 : 0) |
                 (__builtin_amdgcn_ballot_w64(over_n) != 0ull ? 512 : 0);
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) {
        flag |= ((near0 >> (16 * h)) & 0xFFFFull) != 0 ? 2 << h : 0;
        flag |= ((near1 >> (16 * h)) & 0xFFFFull) != 0 ? 32 << h : 0;
      }
      if (lane == 0) s_sm.flag[wave] = flag;
    }
    float pw[2];
    uint32_t um[2], uq[2];
    auto weigh = [&]() {
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        pw[gs] = sc[gs] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[gs] - m_ref[gs]);
        um[gs] = __float2uint_rn(pw[gs] * fvn * sm);
        uq[gs] = __float2uint_rn(pw[gs] * fvg * sq);
        const int o = ((gs * W8_TT + tt) * 16 + 4 * hl) * 64 + slot;
        s_wm[o] = (uint8_t)(um[gs] >> 21);
        s_wm[o + 64] = (uint8_t)((um[gs] >> 14) & 127u);
        s_wm[o + 128] = (uint8_t)((um[gs] >> 7) & 127u);
        s_wm[o + 192] = (uint8_t)(um[gs] & 127u);
        s_wq[o] = (uint8_t)(uq[gs] >> 21);
        s_wq[o + 64] = (uint8_t)((uq[gs] >> 14) & 127u);
        s_wq[o + 128] = (uint8_t)((uq[gs] >> 7) & 127u);
        s_wq[o + 192] = (uint8_t)(uq[gs] & 127u);
      }
    };
    weigh();
    wd_barrier();  // flags and weight digits visible
    int flags = 0;
#pragma unroll
    for (int w = 0; w < W8_WAVES; ++w) flags |= s_sm.flag[w];
    const bool whole = t0 + W8_STEP <= c1;
    ++since_fold;
    ++since_down;
    const bool low = whole && since_fold >= down_seg && ((flags >> 1) & 0xFF) != 0xFF;
    if ((flags & 513) || low || since_fold >= WD_FOLDMAX) {
      if ((flags & 1) && since_down <= 2 * down_seg) down_seg = imin32(2 * down_seg, FA_MAXSEG);
      if (low) since_down = 0;
      // move the references to this step's maxima and fold the int32 accumulators
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const float smax = rows16_max(sc[gs]);
        if (ln == 0) s_sm.max[wave][gs][hl] = smax;
      }
      const float vnm = wave_max_f32(fvn), vgm = wave_max_f32(fvg);
      if (lane == 0) { s_sm.maxn[wave][0] = vnm; s_sm.maxn[wave][1] = vgm; }
      wd_barrier();
      float step_vn = 0.f, step_vg = 0.f;
#pragma unroll
      for (int w = 0; w < W8_WAVES; ++w) {
        step_vn = fmaxf(step_vn, s_sm.maxn[w][0]);
        step_vg = fmaxf(step_vg, s_sm.maxn[w][1]);
      }
      const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        float step_m = -INFINITY;
#pragma unroll
        for (int w = 0; w < W8_WAVES; ++w) step_m = fmaxf(step_m, s_sm.max[w][gs][hl]);
        m_top[gs] = fmaxf(m_top[gs], step_m);
        const float m_new = moved_reference(m_ref[gs], step_m, m_top[gs], low);
        const float alpha = m_ref[gs] == -INFINITY ? 0.f : exp2f(m_ref[gs] - m_new);
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) {
          const float isc = pl == 0 ? im : iq;
#pragma unroll
          for (int c = 0; c < W8_NTC; ++c) {
            const intx4 va = vacc[gs][pl][c];
            const float x = (((float)va[0] * 128.f + (float)va[1]) * 128.f + (float)va[2]) * 128.f + (float)va[3];
            accf[gs][pl][c] = (accf[gs][pl][c] + x * isc) * alpha;
            vacc[gs][pl][c] = intx4{0, 0, 0, 0};
          }
        }
        l_run[gs] *= alpha;
        ym_run[gs] *= alpha;
        yq_run[gs] *= alpha;
        m_ref[gs] = m_new;
      }
      vn_ref = fmaxf(vn_ref, FA_NCAP * step_vn);
      vg_ref = fmaxf(vg_ref, FA_NCAP * step_vg);
      // p <= 2^FA_SLACK and n <= vn_ref, so p n sm <= WMAX kscale
      sm = vn_ref > 0.f ? WMAX * kscale / (vn_ref * FA_HEADROOM) : 0.f;
      sq = vg_ref > 0.f ? WMAX * kscale / (vg_ref * FA_HEADROOM) : 0.f;
      ism = sm > 0.f ? 1.f / sm : 0.f;
      isq = sq > 0.f ? 1.f / sq : 0.f;
      since_fold = 0;
      weigh();       // against the moved references
      wd_barrier();  // the new digits visible
    }
#pragma unroll
    for (int gs = 0; gs < 2; ++gs) {
      l_run[gs] += pw[gs];
      ym_run[gs] = fmaf((float)um[gs], ism, ym_run[gs]);
      yq_run[gs] = fmaf((float)uq[gs], isq, yq_run[gs]);
    }
    // ---- value pass: the step's tokens x this wave's columns, both kinds, both groups ----
#pragma unroll
    for (int t2 = 0; t2 < W8_TT; ++t2) {
      intx4 wa_m[2], wa_q[2];
#pragma unroll
      for (int gs = 0; gs < 2; ++gs) {
        const int o = ((gs * W8_TT + t2) * 16 + ln) * 64 + 16 * hl;
        wa_m[gs] = *reinterpret_cast<const intx4 *>(&s_wm[o]);
        wa_q[gs] = *reinterpret_cast<const intx4 *>(&s_wq[o]);
      }
      const uint4 w0 = vw4[t2][0], w1 = vw4[t2][1];
      const uint32_t x0[W8_NTC] = {w0.x, w0.y, w0.z, w0.w}, x1[W8_NTC] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int c = 0; c < W8_NTC; ++c) {
        const intx4 b0 = value_bits(x0[c], kofs), b1 = value_bits(x1[c], kofs);
#pragma unroll
        for (int gs = 0; gs < 2; ++gs) {
          vacc[gs][0][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_m[gs], b0, vacc[gs][0][c], 0, 0, 0);
          vacc[gs][1][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa_q[gs], b1, vacc[gs][1][c], 0, 0, 0);
        }
      }
    }
  };

  if (nsteps > 0) {
    wd_stage_load<KB, W8_STEP, W8_WAVES>(s_ring0, rk, rv, rkn, rvn, rvg, wave, lane, c0);
    wd_stage_load<KB, W8_STEP, W8_WAVES>(s_ring1, rk, rv, rkn, rvn, rvg, wave, lane, c0 + W8_STEP);
    // the query information (loaded before the stages; loads complete in order) is in registers before the
    // loop, so no wait inside it has to cover it
    wv_wait_vm<2 * S::NLOAD>();
    for (int s = 0; s < nsteps; s += 3) {
      body(s_ring0, s_ring2, s);
      body(s_ring1, s_ring0, s + 1);
      body(s_ring2, s_ring1, s + 2);
    }
    wv_wait_vm<0>();  // the last two stages' loads (past the chunk) have landed before the work-group ends
  } else {
    wv_wait_vm<0>();
    wd_barrier();  // (the images in LDS are not read without steps; the barrier keeps every wave in step)
  }
  // ---- final fold, reductions, partial records: m, l, acc_mse[D], acc_qjl[D] per head ----
  {
    const float im = vn_ref * FA_HEADROOM / WMAX, iq = vg_ref * FA_HEADROOM / WMAX;
#pragma unroll
    for (int gs = 0; gs < 2; ++gs)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const float isc = p == 0 ? im : iq;
#pragma unroll
        for (int c = 0; c < W8_NTC; ++c) {
          const intx4 va = vacc[gs][p][c];
          const float x = (((float)va[0] * 128.f + (float)va[1]) * 128.f + (float)va[2]) * 128.f + (float)va[3];
          accf[gs][p][c] += x * isc;
        }
      }
  }
#pragma unroll
  for (int gs = 0; gs < 2; ++gs) {
    const float L = rows16_sum(l_run[gs]), YM = rows16_sum(ym_run[gs]), YQ = rows16_sum(yq_run[gs]);
    if (ln == 0) {
      s_sm.merge[wave][gs][hl][0] = L;
      s_sm.merge[wave][gs][hl][1] = YM;
      s_sm.merge[wave][gs][hl][2] = YQ;
    }
  }
  wd_barrier();
#pragma unroll
  for (int gs = 0; gs < 2; ++gs) {
    float L = 0.f, YM = 0.f, YQ = 0.f;
#pragma unroll
    for (int w = 0; w < W8_WAVES; ++w) {
      L += s_sm.merge[w][gs][hl][0];
      YM += s_sm.merge[w][gs][hl][1];
      YQ += s_sm.merge[w][gs][hl][2];
    }
    const int h = g * a.G + FA_GMAX * gs + hl;
    float *dst = a.part + (((int64_t)b * a.Hq + h) * a.nsplit + split) * (2 + 2 * (int64_t)D);
    if (wave == 0 && ln == 0) { dst[0] = m_ref[gs]; dst[1] = L; }
#pragma unroll
    for (int c = 0; c < W8_NTC; ++c) {
      const int col = W8_COLS * wave + 4 * ln + c;
      dst[2 + col] = a.vbeta[0] * (2.f * accf[gs][0][c] - YM);
      dst[2 + D + col] = a.vqjl * (2.f * accf[gs][1][c] - YQ);
    }
  }
}

// ---------------------------------------------------------------------------
// query operand images: q' = Pi_K q, Walsh-weighted, as four fixed-point e4m3 digits in the fp8
// operand order, with the inverse of each key nibble's value folded in
// ---------------------------------------------------------------------------
struct PrepArgs {
  const void *q;
  int qt, Hq, Hkv, G, nsub;
  const float *piT;
  float kbeta[8];
  float ctop;
  int *qimg;
  float *qinfo;
  const float *qp_in;  // rotated queries [B * Hq][D] fp32 made by attn_qrot_rows_kernel (null: rotate here)
  AppendArgs app;  // the decode step's new token (app.on): key and value encoded by the work-groups of heads 0
                   // and 1 of subgroup 0
};

// four fixed-point digits of u (|u| <= 224) as e4m3 bytes: u = sum_d k_d Q_d + e with Q_d = 2^(4 - 5 d),
// k_0 in [-14, 14], k_1..k_3 in [-16, 16] and |e| <= 2^-12.  Byte d holds k_d 2^E_d f, E_0 = 4 and E_d = 3
// after (each matrix-core row is its own output, so rows 1..3 are lifted clear of the e4m3 floor; their
// sums are scaled back by Q_d 2^-3), f in {2, 1, 0.5, -1} set by the key nibble's form: every such byte
// is an e4m3 number (at most 4 significant bits, within 4..448 when not 0).  All products of a digit row
// are multiples of half its 2^E_d and at most 16 of them in size, so the fp8 matrix-core sums are exact
// (they keep only about 12 bits below the largest product of a sum, so floating digits would not be).
// Returns the digits' value sum_d k_d Q_d (exact in fp32).
__device__ __forceinline__ float split_fix4_e4m3(float u, float f, uint8_t (&o)[4]) {
  float r = u, v = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float q = __builtin_ldexpf(1.f, 4 - 5 * d);
    const float k = rintf(r / q);
    r = fmaf(-k, q, r);
    v = fmaf(k, q, v);
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(k * (d == 0 ? 16.f : 8.f) * f, 0.f, 0, false);
    o[d] = (uint8_t)(pk & 0xFF);
  }
  return v;
}

// the images and offsets of head h of a unit from its rotated query q' (qp, D floats in LDS), by 256
// threads (tid, their waves wv); red: 4 x 2 floats of LDS for this head's reductions.  Every thread of
// the work-group calls it the same number of times (it holds barriers).
// PERM: the word order of the head-dim-512 kernel, where lane group g of block wb's image holds key word
// 4 g + wb of a plane (so a lane reads the four blocks' words of a plane as one 16-byte piece) instead
// of word 4 wb + g
template <int D, int KB, bool PERM>
__device__ __forceinline__ void prep_images(const PrepArgs &a, int unit, int h, bool present, const float *qp,
                                            float (*red)[2], int tid) {
  constexpr int KP = walsh_count(KB);
  constexpr bool FOLD = fold_beta(D, KB);
  const int wv = tid >> 6, lane = tid & 63;
  // sum q' and max |q'_j|
  {
    float sm = 0.f, mx = 0.f;
    for (int j = tid; j < D; j += 256) {
      sm += qp[j];
      mx = fmaxf(mx, fabsf(qp[j]));
    }
    sm = wave_sum_f32(sm);
    mx = wave_max_f32(mx);
    if (lane == 0) { red[wv][0] = sm; red[wv][1] = mx; }
  }
  __syncthreads();
  const float qsum = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
  float bmax = 0.f;
#pragma unroll
  for (int p = 0; p < KP; ++p) bmax = fmaxf(bmax, fabsf(2.f * a.kbeta[p]));
  if (FOLD) bmax = 1.f;  // the coefficients are applied to the kernel's per-plane results
  const float mxs = fmaxf(fmaxf(red[0][1], red[1][1]), fmaxf(red[2][1], red[3][1])) * bmax;
  const float sq = mxs > 0.f ? 224.f / mxs : 0.f;
  // image ii (FOLD: the 128-coordinate block ii, coefficients applied after the matrix cores; else
  // Walsh plane ii / (D / 128) of block ii % (D / 128), 2 beta folded in), lane (row m = 4 h + digit,
  // k-group g), byte i of its 32: contraction index k = 16 g + i (i < 16) or 64 + 16 g + i - 16; the key
  // operand holds k as nibble k % 32 of lane group k / 32, i.e. nibble position n = k % 8 of dword
  // t = (k % 32) / 8, which carries bit b = bit 4 n + t of the block's key word k / 32 as the value
  // 2^(t - 1) b for t < 3 and 0.5 - b for t = 3 (bit b in the nibble's sign, 0.5 always set): coordinate
  // 128 block + 32 (k / 32) + 4 n + t, scaled by 2^(1 - t), or by -1 for t = 3, whose sums then fall
  // short of the bits' sums by half the digits' values of those coordinates (a constant of the query,
  // taken off the score's offset below).  This work-group writes the 16 lanes of its head (rows 4 h ..
  // 4 h + 3 of the four lane groups) in every image.
  // (a thread takes one word position w of one k-group gg of image ii and writes it for the four digit
  // rows: the four rows' words hold the digits of the same four coordinates)
  constexpr int NI8 = (FOLD ? 1 : KP) * (D / 128);
  for (int e = tid; e < NI8 * 4 * 8; e += 256) {
    const int w = e & 7, gg = (e >> 3) & 3, ii = e >> 5;
    const int wb = ii % (D / 128), p = ii / (D / 128);
    uint32_t word[4] = {0u, 0u, 0u, 0u};
    if (present) {
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int i = 4 * w + bb;
        const int k = i < 16 ? 16 * gg + i : 64 + 16 * gg + (i - 16);
        const int t = (k & 31) >> 3, n = k & 7;
        const int j = (PERM ? 32 * (4 * (k >> 5) + wb) : 128 * wb + 32 * (k >> 5)) + 4 * n + t;
        const float f = t == 0 ? 2.f : t == 1 ? 1.f : t == 2 ? 0.5f : -1.f;
        uint8_t o[4];
        split_fix4_e4m3(fminf(fmaxf((FOLD ? 1.f : 2.f * a.kbeta[p]) * qp[j] * sq, -224.f), 224.f), f, o);
#pragma unroll
        for (int dg = 0; dg < 4; ++dg) word[dg] |= (uint32_t)o[dg] << (8 * bb);
      }
    }
#pragma unroll
    for (int dg = 0; dg < 4; ++dg)
      a.qimg[(((int64_t)unit * NI8 + ii) * 64 + 16 * gg + 4 * h + dg) * 8 + w] = (int)word[dg];
  }
  // half the digit values of the images at coordinates 3 mod 4 (the sign-form nibbles)
  float cs = 0.f;
  if (present) {
    for (int e = tid; e < (FOLD ? 1 : KP) * (D / 4); e += 256) {
      const int p = e / (D / 4), j = 4 * (e % (D / 4)) + 3;
      uint8_t o[4];
      cs += split_fix4_e4m3(fminf(fmaxf((FOLD ? 1.f : 2.f * a.kbeta[p]) * qp[j] * sq, -224.f), 224.f), -1.f, o);
    }
  }
  cs = wave_sum_f32(cs);
  __syncthreads();  // every read of red above is done
  if (lane == 0) red[wv][0] = cs;
  __syncthreads();
  if (tid == 0) {
    float c = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
    if (FOLD) {
      float bs = 0.f;
#pragma unroll
      for (int p = 0; p < KP; ++p) bs += 2.f * a.kbeta[p];
      c *= bs;
    }
    c *= 0.5f;
    const float qinv = (present && sq > 0.f) ? 1.f / sq : 0.f;
    a.qinfo[((int64_t)unit * FA_GMAX + h) * 2 + 0] = qinv;
    a.qinfo[((int64_t)unit * FA_GMAX + h) * 2 + 1] = present ? a.ctop * qsum - c * qinv : 0.f;
  }
}

// rotated queries q' = Pi q (q'_j = sum_k Pi^T[k][j] q_k) of R rows at head dims of 512 and more, into
// q' [R][d] fp32: HB rows per work-group (their q staged in LDS), 32 columns, eight slices of the terms
// added through LDS, so each Pi^T entry read serves HB rows and the d x d matrix is spread over many
// work-groups (a work-group per head would stream the whole matrix through one compute unit); a thread
// loads the 64 matrix entries of a pass at once, so one memory round trip covers them
template <int HB>
__global__ __launch_bounds__(256) void attn_qrot_rows_kernel(const void *q, int qt, int64_t R, int d,
                                                             const float *piT, float *out) {
  extern __shared__ __attribute__((aligned(16))) float qrows[];  // [HB][d]
  __shared__ float red[HB][8][33];
  const int64_t r0 = (int64_t)blockIdx.x * HB;
  const int tid = threadIdx.x, c = tid & 31, sl = tid >> 5;
  // (the element type is uniform: one branch around the whole staging; 16 unconditional loads per thread
  // at a time, at clamped indices, so they are in flight together)
  auto stage = [&](auto conv, auto ptr) {
    const int n = HB * d;
    for (int e0 = 0; e0 < n; e0 += 256 * 16) {
      decltype(conv(ptr[0])) v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = imin32(e0 + 256 * u + tid, n - 1);
        v[u] = conv(ptr[imin64(r0 + e / d, R - 1) * d + e % d]);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (e0 + 256 * u + tid < n) qrows[e0 + 256 * u + tid] = v[u];
    }
  };
  if (qt == TQ_F32) stage([](float x) { return x; }, static_cast<const float *>(q));
  else if (qt == TQ_BF16) stage([](uint16_t x) { return bf16_to_f32(x); }, static_cast<const uint16_t *>(q));
  else stage([](uint16_t x) { return f16_to_f32(x); }, static_cast<const uint16_t *>(q));
  __syncthreads();
  const int j = blockIdx.y * 32 + c;
  constexpr int PER = 64;  // terms per pass: a thread's 64 matrix entries are loaded at once
  float acc[HB];
#pragma unroll
  for (int h = 0; h < HB; ++h) acc[h] = 0.f;
  for (int k0 = sl * PER; k0 < d; k0 += 8 * PER) {  // one pass at head dim 512
    float m[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) m[i] = piT[(int64_t)(k0 + i) * d + j];
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first product
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      const float4 *qv = reinterpret_cast<const float4 *>(qrows + h * d + k0);
      float v = acc[h];
#pragma unroll
      for (int i = 0; i < PER / 4; ++i) {
        const float4 a4 = qv[i];
        v = fmaf(m[4 * i], a4.x, v);
        v = fmaf(m[4 * i + 1], a4.y, v);
        v = fmaf(m[4 * i + 2], a4.z, v);
        v = fmaf(m[4 * i + 3], a4.w, v);
      }
      acc[h] = v;
    }
  }
#pragma unroll
  for (int h = 0; h < HB; ++h) red[h][sl][c] = acc[h];
  __syncthreads();
  if (sl == 0) {
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      float v = acc[h];
#pragma unroll
      for (int t = 1; t < 8; ++t) v += red[h][t][c];
      if (r0 + h < R) out[(r0 + h) * d + j] = v;
    }
  }
}

// images for the fp8 x fp4 matrix-core key passes: one work-group per (unit, head of its group), so the
// four heads' images are made in parallel
template <int D, int KB, bool PERM = false>
__global__ __launch_bounds__(256) void attn_fast_prep_kernel(PrepArgs a) {
  constexpr int KP = walsh_count(KB);
  constexpr bool FOLD = fold_beta(D, KB);
  __shared__ float qs[D];
  __shared__ float qp[D];
  __shared__ float red[4][2];
  const int unit = blockIdx.x, h = blockIdx.y;
  const int nbg = (int)gridDim.x / a.nsub;  // (batch, kv-head) pairs; units = nbg x head subgroups
  const int sub = unit / nbg, bg = unit % nbg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = imin32(FA_GMAX, a.G - sub * FA_GMAX);
  const bool present = h < gw;  // a head past the group's end gets zero images and offsets
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  if (a.app.on && sub == 0 && h < 2) {  // the key by head 0's work-group, the value by head 1's
    __shared__ AppendShared app_sh;
    append_token(a.app, b, g, h, app_sh);
  }
  if (a.qp_in) {  // rotated by attn_qrot_rows_kernel
    for (int j = tid; j < D; j += 256) qp[j] = present ? a.qp_in[((int64_t)b * a.Hq + h0 + h) * D + j] : 0.f;
    __syncthreads();
    prep_images<D, KB, PERM>(a, unit, h, present, qp, red, tid);
    return;
  }
  for (int j = tid; j < D; j += 256) {
    float v = 0.f;
    if (present) {
      const int64_t off = ((int64_t)b * a.Hq + h0 + h) * D + j;
      if (a.qt == TQ_F32) v = static_cast<const float *>(a.q)[off];
      else if (a.qt == TQ_BF16) v = bf16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
      else v = f16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
    }
    qs[j] = v;
  }
  __syncthreads();
  // q'_j = sum_k Pi^T[k][j] q_k: thread (slice, j) sums a slice of k for column j (consecutive threads
  // read consecutive entries of a row of Pi^T; the unrolled loop keeps many independent loads in
  // flight), and the slices are added through LDS
  for (int jc = 0; jc < (D > 256 ? D / 256 : 1); ++jc) {
    constexpr int SL = D >= 256 ? 1 : 256 / D;  // k slices (2 for head_dim 128, else 1)
    const int j = (tid % (D < 256 ? D : 256)) + 256 * jc, sl = D < 256 ? tid / D : 0;
    float acc = 0.f;
    constexpr int KS = D / SL, KU = KS < 64 ? KS : 64;
    for (int k0 = sl * KS; k0 < (sl + 1) * KS; k0 += KU) {
      float pv[KU];  // a whole batch of loads in flight at once
#pragma unroll
      for (int i = 0; i < KU; ++i) pv[i] = a.piT[(int64_t)(k0 + i) * D + j];
#pragma unroll
      for (int i = 0; i < KU; ++i) acc = fmaf(pv[i], qs[k0 + i], acc);
    }
    if (SL > 1) {
      if (sl == 1) qp[j] = acc;
      __syncthreads();
      if (sl == 0) qp[j] += acc;
    } else {
      qp[j] = acc;
    }
  }
  __syncthreads();
  prep_images<D, KB, PERM>(a, unit, h, present, qp, red, tid);
}

// the same for head dims of 256 and more, where one work-group per head would read the whole d x d
// matrix once per head: 1024 threads per unit rotate its four heads' queries together (each entry of
// Pi^T read serves the four), then four groups of 256 threads make one head's images each.  (The
// decode-step append keeps the one-work-group-per-head form.)
template <int D, int KB, bool PERM = false>
__global__ __launch_bounds__(1024) void attn_fast_prep_wide_kernel(PrepArgs a) {
  static_assert(D >= 256 && D <= 1024 && D % 256 == 0, "wide prep: head dims 256 .. 1024");
  constexpr int NT = 1024, SL = NT / D;  // k slices per column
  __shared__ float4 qs[D];                // q of the four heads, [k][head]
  __shared__ float qp[FA_GMAX][D];
  __shared__ float qpart[SL > 1 ? SL - 1 : 1][FA_GMAX][D];
  __shared__ float red[FA_GMAX][4][2];
  const int unit = blockIdx.x;
  const int nbg = (int)gridDim.x / a.nsub;
  const int sub = unit / nbg, bg = unit % nbg;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int h0 = g * a.G + sub * FA_GMAX;
  const int gw = imin32(FA_GMAX, a.G - sub * FA_GMAX);
  const int tid = threadIdx.x;
  for (int e = tid; e < FA_GMAX * D; e += NT) {
    const int h = e / D, j = e % D;
    float v = 0.f;
    if (h < gw) {
      const int64_t off = ((int64_t)b * a.Hq + h0 + h) * D + j;
      if (a.qt == TQ_F32) v = static_cast<const float *>(a.q)[off];
      else if (a.qt == TQ_BF16) v = bf16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
      else v = f16_to_f32(static_cast<const uint16_t *>(a.q)[off]);
    }
    reinterpret_cast<float *>(qs)[4 * j + h] = v;
  }
  __syncthreads();
  // q'_j = sum_k Pi^T[k][j] q_k for the four heads: thread (slice, j) sums a slice of k for column j,
  // 32 loads in flight at a time; the slices are added through LDS
  {
    const int j = tid % D, sl = tid / D;
    constexpr int KS = D / SL, KU = 32;
    float acc[FA_GMAX] = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = sl * KS; k0 < (sl + 1) * KS; k0 += KU) {
      float pv[KU];
#pragma unroll
      for (int i = 0; i < KU; ++i) pv[i] = a.piT[(int64_t)(k0 + i) * D + j];
#pragma unroll
      for (int i = 0; i < KU; ++i) {
        const float4 q4 = qs[k0 + i];
        acc[0] = fmaf(pv[i], q4.x, acc[0]);
        acc[1] = fmaf(pv[i], q4.y, acc[1]);
        acc[2] = fmaf(pv[i], q4.z, acc[2]);
        acc[3] = fmaf(pv[i], q4.w, acc[3]);
      }
    }
    if (sl > 0) {
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) qpart[sl - 1][h][j] = acc[h];
    }
    __syncthreads();
    if (sl == 0) {
#pragma unroll
      for (int h = 0; h < FA_GMAX; ++h) {
        float v = acc[h];
#pragma unroll
        for (int q = 0; q < SL - 1; ++q) v += qpart[q][h][j];
        qp[h][j] = v;
      }
    }
  }
  __syncthreads();
  const int hh = tid >> 8;
  prep_images<D, KB, PERM>(a, unit, hh, hh < gw, qp[hh], red[hh], tid & 255);
}

// ---------------------------------------------------------------------------
// token-tiled layout: word [seq][tile][plane][coord] bit i = plane bit of token 32*tile + i
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void tile_records_kernel(const uint8_t *codes, int64_t cb, int planes, int D,
                                                          int64_t T, int64_t ntile, int64_t toff, int64_t ntile_dst,
                                                          uint32_t *tiles) {
  const int lane = threadIdx.x;
  const int64_t seq = blockIdx.y;
  const int64_t tp = blockIdx.x;  // pair of tiles
  const int64_t t = tp * 64 + lane;
  const uint32_t *rec = reinterpret_cast<const uint32_t *>(codes + (seq * T + t) * cb);
  const int wpp = D / 32;
  for (int wi = 0; wi < planes * wpp; ++wi) {
    const uint32_t w = t < T ? rec[wi] : 0u;
    uint32_t lo = 0, hi = 0;
    for (int i = 0; i < 32; ++i) {
      const unsigned long long m = __ballot((w >> i) & 1u);
      if (lane == i) { lo = (uint32_t)m; hi = (uint32_t)(m >> 32); }
    }
    const int p = wi / wpp, j = (wi % wpp) * 32 + lane;
    if (lane < 32) {
      const int64_t t0 = 2 * tp, t1 = 2 * tp + 1;
      if (t0 < ntile) tiles[((seq * ntile_dst + toff + t0) * planes + p) * D + j] = lo;
      if (t1 < ntile) tiles[((seq * ntile_dst + toff + t1) * planes + p) * D + j] = hi;
    }
  }
}

// rows [nseq][T] into the words of tiles toff .. toff + ceil(T/32) - 1 of sequences of ntile_dst tiles
int run_tile_records_at(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, int64_t toff,
                        int64_t ntile_dst, uint32_t *tiles, hipStream_t st) {
  const int64_t ntile = (T + 31) / 32;
  if (nseq == 0 || ntile == 0) return TQ_OK;
  ProfScope ps("tile_records", st);
  dim3 grid((unsigned)((ntile + 1) / 2), (unsigned)nseq);
  hipLaunchKernelGGL(tile_records_kernel, grid, dim3(64), 0, st, codes, (int64_t)q->code_bytes, q->planes, q->d, T,
                     ntile, toff, ntile_dst, tiles);
  return launch_check();
}

int run_tile_records(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, uint32_t *tiles,
                     hipStream_t st) {
  return run_tile_records_at(q, codes, nseq, T, 0, (T + 31) / 32, tiles, st);
}

// ---------------------------------------------------------------------------
// host dispatch
// ---------------------------------------------------------------------------
// Walsh coefficients beta_S (odd subsets, enumeration order of walsh_planes) of a symmetric codebook
void walsh_coeffs(const double *c, int bits, double *beta) {
  static const int subs[4][8] = {{0x1}, {0x1, 0x2}, {0x1, 0x2, 0x4, 0x7}, {0x1, 0x2, 0x4, 0x8, 0x7, 0xB, 0xD, 0xE}};
  const int L = 1 << bits, n = 1 << (bits - 1);
  for (int s = 0; s < n; ++s) {
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      double sign = 1.0;
      for (int p = 0; p < bits; ++p)
        if (subs[bits - 1][s] >> p & 1) sign *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += c[idx] * sign;
    }
    beta[s] = acc / L;
  }
}

namespace {

struct FastPlan {
  int nsub, nsplit, chunk, nins;
  size_t img_off, info_off, part_off, merge_off, total;
};

FastPlan fast_plan(int D, int KB, int VB, int B, int Hq, int Hkv, int64_t T) {
  FastPlan p{};
  const int G = Hq / Hkv;
  p.nsub = (G + FA_GMAX - 1) / FA_GMAX;
  p.nins = key_images(D, KB);
  const int64_t units = (int64_t)B * Hkv * p.nsub;
  // one chunk per resident work-group: long chunks amortise the per-chunk prologue and partials, and a
  // short sequence still spreads over the chip in chunks of one 256-token step (the local-layer shape,
  // 64 units x 1024 tokens, took 41 us in 1024-token chunks and 25 us in 256-token ones)
  const int64_t slots = (int64_t)device_cus() * fa_waves_per_eu(D, KB, VB);
  const int64_t want = std::max<int64_t>(1, slots / std::max<int64_t>(units, 1));
  int64_t chunk = (T + want - 1) / want;
  chunk = std::max<int64_t>(FA_SUB, (chunk + FA_SUB - 1) / FA_SUB * FA_SUB);
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.img_off = 0;
  p.info_off = al((size_t)units * p.nins * 64 * 16);
  p.part_off = p.info_off + al((size_t)units * FA_GMAX * 2 * 4);
  p.merge_off = p.part_off + al((size_t)B * Hq * p.nsplit * (2 + 2 * (size_t)D) * 4);
  p.total = p.merge_off + (size_t)B * Hq * 2 * (size_t)D * 4;
  return p;
}

// wave-streaming plan: one single-wave work-group per resident slot, each a contiguous token range
struct WavePlan {
  int nsplit, chunk;
  size_t img_off, info_off, part_off, merge_off, total;
};

bool wave_supported(int D, int KB, int VB) { return D == 128 && VB == 1 && KB >= 1 && KB <= 3; }

// resident single-wave work-groups of attn_wave_kernel<KB> on the current device (cached per device)
int wave_slots(int KB) {
  static int cache[64][4] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int &slot = cache[dev][KB];
  if (slot > 0) return slot;
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  hipError_t e = hipErrorInvalidValue;
  if (KB == 1) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wave_kernel<1>, 64, 0);
  if (KB == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wave_kernel<2>, 64, 0);
  if (KB == 3) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wave_kernel<3>, 64, 0);
  if (e != hipSuccess || blocks <= 0) blocks = 8;
  slot = cus * blocks;
  return slot;
}

WavePlan wave_plan(int D, int KB, int B, int Hq, int Hkv, int64_t T) {
  WavePlan p{};
  const int G = Hq / Hkv;
  const int nsub = (G + FA_GMAX - 1) / FA_GMAX;
  const int nins = key_images(D, KB);
  const int64_t units = (int64_t)B * Hkv * nsub;
  const int64_t want = std::max<int64_t>(1, wave_slots(KB) / std::max<int64_t>(units, 1));
  int64_t chunk = (T + want - 1) / want;
  // whole ring turns per wave, so only the last range of a sequence pads
  const int64_t turn = (int64_t)WV_RING * WV_STEP;
  chunk = std::max<int64_t>(turn, (chunk + turn - 1) / turn * turn);
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.img_off = 0;
  p.info_off = al((size_t)units * nins * 64 * 16);
  p.part_off = p.info_off + al((size_t)units * FA_GMAX * 2 * 4);
  p.merge_off = p.part_off + al((size_t)B * Hq * p.nsplit * (2 + 2 * (size_t)D) * 4);
  p.total = p.merge_off + (size_t)B * Hq * 2 * (size_t)D * 4;
  return p;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool wide_supported(int D, int KB, int VB) { return D == WD_D && VB == 1 && KB >= 1 && KB <= 3; }

// resident work-groups of attn_wide_kernel<KB> on the current device (cached per device)
int wide_slots(int KB) {
  static int cache[64][4] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int &slot = cache[dev][KB];
  if (slot > 0) return slot;
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  if (KB == 1) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide_kernel<1>, WD_THREADS, 0);
  if (KB == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide_kernel<2>, WD_THREADS, 0);
  if (KB == 3) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide_kernel<3>, WD_THREADS, 0);
  if (e != hipSuccess || blocks <= 0) blocks = 1;
  slot = device_cus() * blocks;
  return slot;
}

// the head-dim-512 plan: the query images and offsets as fast_plan lays them out, chunks of whole ring
// turns (three steps), one per resident work-group
FastPlan wide_plan(int KB, int B, int Hq, int Hkv, int64_t T) {
  FastPlan p = fast_plan(WD_D, KB, 1, B, Hq, Hkv, T);
  const int64_t units = (int64_t)B * Hkv * p.nsub;
  const int64_t want = std::max<int64_t>(1, wide_slots(KB) / std::max<int64_t>(units, 1));
  const int64_t turn = 3 * (int64_t)WD_STEP;
  int64_t chunk = (T + want - 1) / want;
  chunk = std::max<int64_t>(turn, (chunk + turn - 1) / turn * turn);
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.merge_off = p.part_off + al((size_t)B * Hq * p.nsplit * (2 + 2 * (size_t)WD_D) * 4);
  p.total = p.merge_off + (size_t)B * Hq * 2 * (size_t)WD_D * 4;
  return p;
}

// resident work-groups of attn_wide8_kernel<KB> on the device (cached)
int wide8_slots(int KB) {
  static int cache[64][4] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int &slot = cache[dev][KB];
  if (slot > 0) return slot;
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  if (KB == 1) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide8_kernel<1>, W8_THREADS, 0);
  if (KB == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide8_kernel<2>, W8_THREADS, 0);
  if (KB == 3) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, attn_wide8_kernel<3>, W8_THREADS, 0);
  if (e != hipSuccess || blocks <= 0) blocks = 1;
  slot = device_cus() * blocks;
  return slot;
}

// the eight-head plan: one work-group per (batch, KV head, chunk) serves both head groups; chunks of whole
// ring turns (three 128-token steps), one per resident work-group
FastPlan wide8_plan(int KB, int B, int Hq, int Hkv, int64_t T) {
  FastPlan p = fast_plan(WD_D, KB, 1, B, Hq, Hkv, T);
  const int64_t units = (int64_t)B * Hkv;
  const int64_t want = std::max<int64_t>(1, wide8_slots(KB) / std::max<int64_t>(units, 1));
  const int64_t turn = 3 * (int64_t)W8_STEP;
  int64_t chunk = (T + want - 1) / want;
  chunk = std::max<int64_t>(turn, (chunk + turn - 1) / turn * turn);
  p.chunk = (int)std::min<int64_t>(chunk, 1 << 30);
  p.nsplit = (int)std::max<int64_t>(1, (T + p.chunk - 1) / p.chunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.merge_off = p.part_off + al((size_t)B * Hq * p.nsplit * (2 + 2 * (size_t)WD_D) * 4);
  p.total = p.merge_off + (size_t)B * Hq * 2 * (size_t)WD_D * 4;
  return p;
}

bool fast_supported(int D, int KB, int VB) {
  if (D != 128 && D != 256 && D != 512) return false;
  if (KB < 1 || KB > 4 || VB < 1 || VB > 3) return false;
  return key_images(D, KB) <= 16 && (D < 512 || (VB == 1 && KB <= 3));
}

template <int D, int KB, int VB>
int launch_fast(const FastPlan &fp, const FastAttnArgs &fa, const PrepArgs &pa, int units, hipStream_t st) {
  {
    ProfScope ps("attn_prep", st);
    if constexpr (D >= 256) {
      if (!pa.app.on && !pa.qp_in) hipLaunchKernelGGL((attn_fast_prep_wide_kernel<D, KB>), dim3(units), dim3(1024), 0, st, pa);
      else hipLaunchKernelGGL((attn_fast_prep_kernel<D, KB>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
    } else {
      hipLaunchKernelGGL((attn_fast_prep_kernel<D, KB>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
    }
  }
  int rc = launch_check();
  if (rc != TQ_OK) return rc;
  ProfScope ps("attn_fast", st);
  hipLaunchKernelGGL((attn_fast_kernel<D, KB, VB>), dim3(units, fp.nsplit), dim3(FA_THREADS), 0, st, fa);
  return launch_check();
}

}  // namespace

size_t attn_fast_ws_bytes(int D, int KB, int B, int Hq, int Hkv, int64_t T) {
  size_t n = 0;
  for (int vb = 1; vb <= 3; ++vb) n = std::max(n, fast_plan(D, KB, vb, B, Hq, Hkv, T).total);
  if (wave_supported(D, KB, 1)) n = std::max(n, wave_plan(D, KB, B, Hq, Hkv, T).total);
  if (wide_supported(D, KB, 1)) n = std::max(n, wide_plan(KB, B, Hq, Hkv, T).total);
  if (wide_supported(D, KB, 1) && Hkv > 0 && Hq == 8 * Hkv) n = std::max(n, wide8_plan(KB, B, Hq, Hkv, T).total);
  return n;
}

int attn_combine(const float *part, int BH, int nsplit, int d, const tq_quantizer *vq, float *merged, float *out,
                 hipStream_t st);

int run_attn_fast(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq, int Hkv,
                  const uint8_t *kcodes, const uint16_t *knorms, const uint32_t *vtiles, const uint16_t *vnorms,
                  const uint16_t *vgammas, int64_t Tstride, const int32_t *seq_len, int kv_div, float scale,
                  float *out, void *ws, const AppendArgs *app, hipStream_t st) {
  const int D = kq->d, KB = kq->bits, VB = vq->bmse;
  if (!fast_supported(D, KB, VB)) return TQ_ERR_UNSUPPORTED;
  FastPlan fp = fast_plan(D, KB, VB, B, Hq, Hkv, Tstride);
  // the wave-streaming kernel stages 16-byte pieces: sequence rows of the fp16 arrays must stay aligned
  const bool wave = wave_supported(D, KB, VB) && Tstride % 8 == 0 && aligned16(kcodes) && aligned16(knorms) &&
                    aligned16(vtiles) && aligned16(vnorms) && aligned16(vgammas);
  // head dim 512 with 1-bit value indices: attn_wide_kernel (16-byte staged pieces, int32 stage offsets)
  const bool widek = !wave && wide_supported(D, KB, VB) && Tstride % 8 == 0 && aligned16(kcodes) &&
                     aligned16(knorms) && aligned16(vtiles) && aligned16(vnorms) && aligned16(vgammas) &&
                     Tstride * (int64_t)(KB * D / 8) < (int64_t(1) << 31);
  // eight query heads per KV head: one eight-wave work-group serves both head groups
  const bool wide8 = widek && Hq == 8 * Hkv;
  if (widek) fp = wide8 ? wide8_plan(KB, B, Hq, Hkv, Tstride) : wide_plan(KB, B, Hq, Hkv, Tstride);
  if (wave) {
    const WavePlan wp = wave_plan(D, KB, B, Hq, Hkv, Tstride);
    fp.nsplit = wp.nsplit;
    fp.chunk = wp.chunk;
    fp.img_off = wp.img_off;
    fp.info_off = wp.info_off;
    fp.part_off = wp.part_off;
    fp.merge_off = wp.merge_off;
    fp.total = wp.total;
  }
  const int units = B * Hkv * fp.nsub;
  char *w = static_cast<char *>(ws);
  double kb64[8] = {0}, vb64[4] = {0};
  walsh_coeffs(kq->c64, KB, kb64);
  walsh_coeffs(vq->c64, VB, vb64);
  PrepArgs pa{};
  pa.q = q; pa.qt = qt; pa.Hq = Hq; pa.Hkv = Hkv; pa.G = Hq / Hkv; pa.nsub = fp.nsub; pa.piT = kq->piT;
  for (int i = 0; i < 8; ++i) pa.kbeta[i] = (float)kb64[i];
  pa.ctop = (float)kq->c64[(1 << KB) - 1];
  pa.qimg = reinterpret_cast<int *>(w + fp.img_off);
  pa.qinfo = reinterpret_cast<float *>(w + fp.info_off);
  if (app) pa.app = *app;
  int rc = TQ_ERR_UNSUPPORTED;
  if (D >= 512 && B > 0) {
    // the rotated queries of all B * Hq heads first, spread over many work-groups (into the merge area,
    // which the split merge uses only after the attention kernel)
    float *qp = reinterpret_cast<float *>(w + fp.merge_off);
    {
      ProfScope ps("attn_qrot_rows", st);
      hipLaunchKernelGGL(attn_qrot_rows_kernel<8>, dim3((unsigned)cdiv64((int64_t)B * Hq, 8), (unsigned)(D / 32)),
                         dim3(256), (size_t)8 * D * 4, st, q, qt, (int64_t)B * Hq, D, kq->piT, qp);
    }
    if ((rc = launch_check()) != TQ_OK) return rc;
    pa.qp_in = qp;
  }
  FastAttnArgs fa{};
  fa.qimg = pa.qimg; fa.qinfo = pa.qinfo; fa.kcodes = kcodes; fa.knorms = knorms; fa.vtiles = vtiles;
  fa.vnorms = vnorms; fa.vgammas = vgammas; fa.seq_len = seq_len;
  fa.part = reinterpret_cast<float *>(w + fp.part_off);
  fa.Tstride = Tstride; fa.ntile = (Tstride + 31) / 32;
  fa.Hq = Hq; fa.Hkv = Hkv; fa.G = Hq / Hkv; fa.nsub = fp.nsub; fa.chunk = fp.chunk; fa.nsplit = fp.nsplit;
  fa.seq_add = (app && app->on) ? 1 : 0;
  fa.kv_div = kv_div;
  fa.scale_log2 = scale * 1.4426950408889634f;
  fa.vqjl = vq->qjl_scale;
  for (int i = 0; i < 4; ++i) fa.vbeta[i] = (float)vb64[i];
  for (int i = 0; i < 8; ++i) fa.kbeta[i] = (float)kb64[i];
  if (wave) {
    {
      ProfScope ps("attn_prep", st);
      if (KB == 1) hipLaunchKernelGGL((attn_fast_prep_kernel<128, 1>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
      if (KB == 2) hipLaunchKernelGGL((attn_fast_prep_kernel<128, 2>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
      if (KB == 3) hipLaunchKernelGGL((attn_fast_prep_kernel<128, 3>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
    }
    if ((rc = launch_check()) != TQ_OK) return rc;
    {
      ProfKernel pk("attn_wave");
      const dim3 grid((unsigned)units, (unsigned)fp.nsplit);
      if (KB == 1) hipExtLaunchKernelGGL(attn_wave_kernel<1>, grid, dim3(64), 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 2) hipExtLaunchKernelGGL(attn_wave_kernel<2>, grid, dim3(64), 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 3) hipExtLaunchKernelGGL(attn_wave_kernel<3>, grid, dim3(64), 0, st, pk.start, pk.stop, 0, fa);
    }
    if ((rc = launch_check()) != TQ_OK) return rc;
    return attn_combine(fa.part, B * Hq, fp.nsplit, D, vq, reinterpret_cast<float *>(w + fp.merge_off), out,
                        st);
  }
  if (widek) {
    {
      ProfScope ps("attn_prep", st);
      const bool app_on = app && app->on;
      if (KB == 1) {
        if (app_on || pa.qp_in) hipLaunchKernelGGL((attn_fast_prep_kernel<WD_D, 1, true>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
        else hipLaunchKernelGGL((attn_fast_prep_wide_kernel<WD_D, 1, true>), dim3(units), dim3(1024), 0, st, pa);
      }
      if (KB == 2) {
        if (app_on || pa.qp_in) hipLaunchKernelGGL((attn_fast_prep_kernel<WD_D, 2, true>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
        else hipLaunchKernelGGL((attn_fast_prep_wide_kernel<WD_D, 2, true>), dim3(units), dim3(1024), 0, st, pa);
      }
      if (KB == 3) {
        if (app_on || pa.qp_in) hipLaunchKernelGGL((attn_fast_prep_kernel<WD_D, 3, true>), dim3(units, FA_GMAX), dim3(256), 0, st, pa);
        else hipLaunchKernelGGL((attn_fast_prep_wide_kernel<WD_D, 3, true>), dim3(units), dim3(1024), 0, st, pa);
      }
    }
    if ((rc = launch_check()) != TQ_OK) return rc;
    if (wide8) {
      ProfKernel pk("attn_wide8");
      const dim3 grid((unsigned)(B * Hkv), (unsigned)fp.nsplit), blk(W8_THREADS);
      if (KB == 1) hipExtLaunchKernelGGL(attn_wide8_kernel<1>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 2) hipExtLaunchKernelGGL(attn_wide8_kernel<2>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 3) hipExtLaunchKernelGGL(attn_wide8_kernel<3>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
    } else {
      ProfKernel pk("attn_wide");
      const dim3 grid((unsigned)units, (unsigned)fp.nsplit), blk(WD_THREADS);
      if (KB == 1) hipExtLaunchKernelGGL(attn_wide_kernel<1>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 2) hipExtLaunchKernelGGL(attn_wide_kernel<2>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
      if (KB == 3) hipExtLaunchKernelGGL(attn_wide_kernel<3>, grid, blk, 0, st, pk.start, pk.stop, 0, fa);
    }
    if ((rc = launch_check()) != TQ_OK) return rc;
    return attn_combine(fa.part, B * Hq, fp.nsplit, D, vq, reinterpret_cast<float *>(w + fp.merge_off), out,
                        st);
  }
#define TQ_FAST(DD, KK, VV) \
  if (D == DD && KB == KK && VB == VV) rc = launch_fast<DD, KK, VV>(fp, fa, pa, units, st);
  TQ_FAST(128, 1, 1) TQ_FAST(128, 2, 1) TQ_FAST(128, 3, 1) TQ_FAST(128, 4, 1)
  TQ_FAST(128, 1, 2) TQ_FAST(128, 2, 2) TQ_FAST(128, 3, 2) TQ_FAST(128, 4, 2)
  TQ_FAST(128, 1, 3) TQ_FAST(128, 2, 3) TQ_FAST(128, 3, 3) TQ_FAST(128, 4, 3)
  TQ_FAST(256, 1, 1) TQ_FAST(256, 2, 1) TQ_FAST(256, 3, 1)
  TQ_FAST(256, 1, 2) TQ_FAST(256, 2, 2) TQ_FAST(256, 3, 2)
  TQ_FAST(256, 1, 3) TQ_FAST(256, 2, 3) TQ_FAST(256, 3, 3)
  TQ_FAST(512, 1, 1) TQ_FAST(512, 2, 1) TQ_FAST(512, 3, 1)
#undef TQ_FAST
  if (rc != TQ_OK) return rc;
  return attn_combine(fa.part, B * Hq, fp.nsplit, D, vq, reinterpret_cast<float *>(w + fp.merge_off), out,
                        st);
}

}  // namespace tq
