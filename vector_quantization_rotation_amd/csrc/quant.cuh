// Lloyd-Max cell search shared by the fused encode kernel and the GEMM-path epilogue: the cell index of a
// rotated coordinate (Algorithm 1 on the ai-navigate-news Gemma 4 post, section "仕組み（技術的）": the
// nearest centroid of a scalar codebook, which for sorted centroids is the count of cell boundaries below
// the coordinate) with its bits shifted into bit-plane words.
#pragma once

#include "common.cuh"

namespace tq {

// Lloyd-Max cell index idx = #{k : t_k n < y} of one coordinate, its bits shifted into bit-plane words
// (P[s] = 2 P[s] + bit s, columns visited high to low) and, for Algorithm 2, the centroid c[idx] selected on
// the way.  The codebook of the coordinate law is symmetric (c_{L-1-k} = -c_k, t_{L-2-k} = -t_k, the middle
// boundary 0), so the top bit is the test y > t_{L/2-1} n and the rest come from a binary search of |y| over
// the upper half's boundaries alone: for y above the middle the lower bits are m = #{upper t_k n < |y|}, and
// below it they are L/2 - 1 - m, i.e. m with every bit inverted (the two differ from the full count only
// when |y| equals a boundary exactly, a tie).  The words therefore collect m, and quant_fix_planes inverts
// the lower planes' bits wherever the top plane holds 0 once a word is complete.  Each level compares
// against the one boundary its decided bits leave, the compare mask lives in VCC only, and add-with-carry
// does the shift.
template <int BM, bool CENT>
__device__ __forceinline__ void quant_coord(float y, const float (&T)[(1 << BM) - 1], const float (&C)[1 << BM],
                                            uint32_t (&P)[BM], float &cv) {
  if constexpr (BM == 1) {
    if constexpr (CENT) {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t0]\n\t"
          "v_cndmask_b32_e32 %[cv], %[c0], %[c1], vcc\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [cv] "=&v"(cv)
          : [y] "v"(y), [t0] "v"(T[0]), [c0] "v"(C[0]), [c1] "v"(C[1])
          : "vcc");
    } else {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t0]\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0])
          : [y] "v"(y), [t0] "v"(T[0])
          : "vcc");
    }
  } else if constexpr (BM == 2) {
    if constexpr (CENT) {
      // |c| = c[2 + m]; c[idx] = +|c| above the middle boundary, -|c| = c[1 - m] below it
      float ca;
      asm volatile(
          "v_cmp_gt_f32_e64 vcc, |%[y]|, %[t2]\n\t"
          "v_cndmask_b32_e32 %[ca], %[c2], %[c3], vcc\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_cndmask_b32_e64 %[cv], -%[ca], %[ca], vcc\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [ca] "=&v"(ca), [cv] "=&v"(cv)
          : [y] "v"(y), [t1] "v"(T[1]), [t2] "v"(T[2]), [c2] "v"(C[2]), [c3] "v"(C[3])
          : "vcc");
    } else {
      asm volatile(
          "v_cmp_gt_f32_e64 vcc, |%[y]|, %[t2]\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1])
          : [y] "v"(y), [t1] "v"(T[1]), [t2] "v"(T[2])
          : "vcc");
    }
  } else if constexpr (BM == 3) {
    float th;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t3]\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e64 vcc, |%[y]|, %[t5]\n\t"
        "v_cndmask_b32_e32 %[th], %[t4], %[t6], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e64 vcc, |%[y]|, %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [th] "=&v"(th)
        : [y] "v"(y), [t3] "v"(T[3]), [t4] "v"(T[4]), [t5] "v"(T[5]), [t6] "v"(T[6])
        : "vcc");
    if constexpr (CENT) {
      // |c| = c[4 + m] from the words' new low bits, negated below the middle boundary (c[3 - m])
      const int m = (int)((P[0] & 1u) | ((P[1] & 1u) << 1));
      float v = C[4];
#pragma unroll
      for (int i = 1; i < 4; ++i) v = m == i ? C[4 + i] : v;
      cv = (P[2] & 1u) ? v : -v;
    }
  } else {
    static_assert(BM == 4 && !CENT, "4-bit cells: Algorithm 1 only");
    float th, ua, ub;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t7]\n\t"
        "v_addc_co_u32_e32 %[p3], vcc, %[p3], %[p3], vcc\n\t"
        "v_cmp_gt_f32_e64 vcc, |%[y]|, %[t11]\n\t"
        "v_cndmask_b32_e32 %[th], %[t9], %[t13], vcc\n\t"
        "v_cndmask_b32_e32 %[ua], %[t8], %[t12], vcc\n\t"
        "v_cndmask_b32_e32 %[ub], %[t10], %[t14], vcc\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e64 vcc, |%[y]|, %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[ua], %[ub], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e64 vcc, |%[y]|, %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [p3] "+v"(P[3]), [th] "=&v"(th), [ua] "=&v"(ua),
          [ub] "=&v"(ub)
        : [y] "v"(y), [t7] "v"(T[7]), [t8] "v"(T[8]), [t9] "v"(T[9]), [t10] "v"(T[10]), [t11] "v"(T[11]),
          [t12] "v"(T[12]), [t13] "v"(T[13]), [t14] "v"(T[14])
        : "vcc");
  }
}

// completes plane words built by quant_coord: below the middle boundary (top-plane bit 0) the lower bits
// are inverted, m -> L/2 - 1 - m.  `valid` masks the bit positions that hold coordinates
template <int BM>
__device__ __forceinline__ void quant_fix_planes(uint32_t (&P)[BM], uint32_t valid = 0xFFFFFFFFu) {
  const uint32_t below = ~P[BM - 1] & valid;
#pragma unroll
  for (int p = 0; p < BM - 1; ++p) P[p] ^= below;
}

}  // namespace tq
