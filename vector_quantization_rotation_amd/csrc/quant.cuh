// Lloyd-Max cell search shared by the fused encode kernel and the GEMM-path epilogue: the cell index of a
// rotated coordinate (Algorithm 1 on the ai-navigate-news Gemma 4 post, section "仕組み（技術的）": the
// nearest centroid of a scalar codebook, which for sorted centroids is the count of cell boundaries below
// the coordinate) with its bits shifted into bit-plane words.
#pragma once

#include "common.cuh"

namespace tq {

// Lloyd-Max cell index idx = #{k : t_k n < y} of one coordinate by binary
// search over the scaled boundaries T[k-1] = t_k n (non-decreasing in k), its
// bits shifted into the plane words (P[s] = 2 P[s] + bit s of idx, columns
// visited high to low) and, for Algorithm 2, the centroid c[idx] selected on the
// way.  Each level compares against the one boundary its decided bits leave,
// then narrows every lower level's candidates (and the centroids) by that bit;
// the compare mask lives in VCC only, and add-with-carry does the shift.
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
    float th;
    if constexpr (CENT) {
      float ca, cb;
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_cndmask_b32_e32 %[th], %[t0], %[t2], vcc\n\t"
          "v_cndmask_b32_e32 %[ca], %[c0], %[c2], vcc\n\t"
          "v_cndmask_b32_e32 %[cb], %[c1], %[c3], vcc\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
          "v_cndmask_b32_e32 %[cv], %[ca], %[cb], vcc\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [th] "=&v"(th), [ca] "=&v"(ca), [cb] "=&v"(cb), [cv] "=&v"(cv)
          : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [c0] "v"(C[0]), [c1] "v"(C[1]),
            [c2] "v"(C[2]), [c3] "v"(C[3])
          : "vcc");
    } else {
      asm volatile(
          "v_cmp_gt_f32_e32 vcc, %[y], %[t1]\n\t"
          "v_cndmask_b32_e32 %[th], %[t0], %[t2], vcc\n\t"
          "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
          "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
          "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
          : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [th] "=&v"(th)
          : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2])
          : "vcc");
    }
  } else if constexpr (BM == 3) {
    float th, ta, tb;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t3]\n\t"
        "v_cndmask_b32_e32 %[th], %[t1], %[t5], vcc\n\t"
        "v_cndmask_b32_e32 %[ta], %[t0], %[t4], vcc\n\t"
        "v_cndmask_b32_e32 %[tb], %[t2], %[t6], vcc\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[ta], %[tb], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [th] "=&v"(th), [ta] "=&v"(ta), [tb] "=&v"(tb)
        : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [t3] "v"(T[3]), [t4] "v"(T[4]),
          [t5] "v"(T[5]), [t6] "v"(T[6])
        : "vcc");
    if constexpr (CENT) {
      // c[idx] from the finished words' low bits (idx = 4 b2 + 2 b1 + b0)
      const int idx = (int)((P[0] & 1u) | ((P[1] & 1u) << 1) | ((P[2] & 1u) << 2));
      float v = C[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) v = idx == i ? C[i] : v;
      cv = v;
    }
  } else {
    static_assert(BM == 4 && !CENT, "4-bit cells: Algorithm 1 only");
    float th, u0, u1, w0, w1, w2, w3;
    asm volatile(
        "v_cmp_gt_f32_e32 vcc, %[y], %[t7]\n\t"
        "v_cndmask_b32_e32 %[th], %[t3], %[t11], vcc\n\t"
        "v_cndmask_b32_e32 %[u0], %[t1], %[t9], vcc\n\t"
        "v_cndmask_b32_e32 %[u1], %[t5], %[t13], vcc\n\t"
        "v_cndmask_b32_e32 %[w0], %[t0], %[t8], vcc\n\t"
        "v_cndmask_b32_e32 %[w1], %[t2], %[t10], vcc\n\t"
        "v_cndmask_b32_e32 %[w2], %[t4], %[t12], vcc\n\t"
        "v_cndmask_b32_e32 %[w3], %[t6], %[t14], vcc\n\t"
        "v_addc_co_u32_e32 %[p3], vcc, %[p3], %[p3], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[u0], %[u1], vcc\n\t"
        "v_cndmask_b32_e32 %[w0], %[w0], %[w2], vcc\n\t"
        "v_cndmask_b32_e32 %[w1], %[w1], %[w3], vcc\n\t"
        "v_addc_co_u32_e32 %[p2], vcc, %[p2], %[p2], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_cndmask_b32_e32 %[th], %[w0], %[w1], vcc\n\t"
        "v_addc_co_u32_e32 %[p1], vcc, %[p1], %[p1], vcc\n\t"
        "v_cmp_gt_f32_e32 vcc, %[y], %[th]\n\t"
        "v_addc_co_u32_e32 %[p0], vcc, %[p0], %[p0], vcc"
        : [p0] "+v"(P[0]), [p1] "+v"(P[1]), [p2] "+v"(P[2]), [p3] "+v"(P[3]), [th] "=&v"(th), [u0] "=&v"(u0),
          [u1] "=&v"(u1), [w0] "=&v"(w0), [w1] "=&v"(w1), [w2] "=&v"(w2), [w3] "=&v"(w3)
        : [y] "v"(y), [t0] "v"(T[0]), [t1] "v"(T[1]), [t2] "v"(T[2]), [t3] "v"(T[3]), [t4] "v"(T[4]),
          [t5] "v"(T[5]), [t6] "v"(T[6]), [t7] "v"(T[7]), [t8] "v"(T[8]), [t9] "v"(T[9]), [t10] "v"(T[10]),
          [t11] "v"(T[11]), [t12] "v"(T[12]), [t13] "v"(T[13]), [t14] "v"(T[14])
        : "vcc");
  }
}

}  // namespace tq
