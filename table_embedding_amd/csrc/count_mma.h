// Counts x gradient rows on the matrix cores, exact in every product: the
// contraction that the small-table histogram path of the FBTriton TBE page
// ("Forward"; "Fusion boundaries": the backward reuses the histogram) turns
// the gradient of a row into, grad[h][d] = sum_b C[b][h] * G[b][d] with C
// a bag's count of row h and G its grad_out row (scaled by 1/L_b for a mean
// table before it gets here).
//
// A count of at most 8 significant bits is exact in bfloat16, and an fp32
// value x is the exact sum of three bfloat16 parts: hi = x with the low 16
// bits cleared, mid = the same of x - hi, lo = (x - hi) - mid, which has at
// most 8 significant bits left.  Three v_mfma_f32_16x16x32_bf16 (lo, mid,
// hi) per tile then give the fp32 products without rounding; only the fp32
// accumulation rounds.  (This holds while the parts are normal numbers,
// for |x| >= 2^-100; below that the lo part may be subnormal and its
// truncation drops less than 2^-133.)  Counts wider than 8 bits are cut
// into four 8-bit parts (count & 0xff << 8k, each exact), one such pass per
// part.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l = 16 kq + i holds A
// row i, K elements 8 kq .. 8 kq + 7 (element 2j in the low half of dword
// j) and B column i, the same K elements; the result's lane l holds rows
// 4 kq + r (r = 0..3) of column i.
#pragma once
#include "tbe_common.h"

namespace tbe {

typedef float cm_f4 __attribute__((ext_vector_type(4)));
typedef __bf16 cm_bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t cm_u32x4 __attribute__((ext_vector_type(4)));

// The three bfloat16 parts of x0 and x1, packed as K elements 2j and 2j + 1.
__device__ __forceinline__ void cm_split3(float x0, float x1, uint32_t& hi, uint32_t& mid,
                                          uint32_t& lo) {
  const uint32_t h0 = __float_as_uint(x0) & 0xffff0000u, h1 = __float_as_uint(x1) & 0xffff0000u;
  const float r0 = x0 - __uint_as_float(h0), r1 = x1 - __uint_as_float(h1);
  const uint32_t m0 = __float_as_uint(r0) & 0xffff0000u, m1 = __float_as_uint(r1) & 0xffff0000u;
  const uint32_t l0 = __float_as_uint(r0 - __uint_as_float(m0)),
                 l1 = __float_as_uint(r1 - __uint_as_float(m1));
  hi = (h0 >> 16) | h1;
  mid = (m0 >> 16) | m1;
  lo = (l0 >> 16) | (l1 & 0xffff0000u);
}

// acc[rt][nt] += C^T[rows 16 rt .., the K bags] x G[the K bags, this lane's
// DT column tiles] for row tiles rt < nrt.  cnt is the LDS count matrix
// [row][bag] (row pitch P words; bag k of K step ks is consumed by lane group
// kq = (k % 32) / 8 as element k % 8); gv[ks][e][nt] is the lane's grad_out
// value of bag 32 ks + 8 kq + e, column tile nt.  wide: some count may
// exceed 8 bits.
template <int KSTEPS, int DT, int RT, int P>
__device__ __forceinline__ void cm_counts_x_grad(cm_f4 (&acc)[RT][DT], const uint32_t (*cnt)[P],
                                                 const float (&gv)[KSTEPS][8][DT], uint32_t nrt,
                                                 bool wide, uint32_t i, uint32_t kq) {
  const uint32_t nparts = wide ? 4u : 1u;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    cm_u32x4 bh[DT], bm[DT], bl[DT];
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h, m, l;
        cm_split3(gv[ks][2 * j][nt], gv[ks][2 * j + 1][nt], h, m, l);
        bh[nt][j] = h;
        bm[nt][j] = m;
        bl[nt][j] = l;
      }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if ((uint32_t)rt >= nrt) break;  // uniform
      const uint32_t* crow = &cnt[(uint32_t)rt * 16u + i][32u * (uint32_t)ks + 8u * kq];
      const cm_u32x4 n0 = *reinterpret_cast<const cm_u32x4*>(crow);
      const cm_u32x4 n1 = *reinterpret_cast<const cm_u32x4*>(crow + 4);
      for (uint32_t ap = 0; ap < nparts; ++ap) {
        // (an integer of at most 8 significant bits is exactly the upper
        // half of its fp32)
        const uint32_t mask = wide ? 0xffu << (8u * ap) : 0xffffffffu;
        float c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = (float)((e < 4 ? n0[e & 3] : n1[e & 3]) & mask);
        cm_u32x4 av;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[j] = (__float_as_uint(c[2 * j]) >> 16) | (__float_as_uint(c[2 * j + 1]) & 0xffff0000u);
        const cm_bf16x8 A = __builtin_bit_cast(cm_bf16x8, av);
#pragma unroll
        for (int nt = 0; nt < DT; ++nt) {
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(cm_bf16x8, bl[nt]), acc[rt][nt], 0, 0, 0);
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(cm_bf16x8, bm[nt]), acc[rt][nt], 0, 0, 0);
          acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              A, __builtin_bit_cast(cm_bf16x8, bh[nt]), acc[rt][nt], 0, 0, 0);
        }
      }
    }
  }
}

// The count rows [0, nrows), each count and-ed with `mask` (all bits, or one
// 8-bit part 0xff << 8k of wider counts: at most 8 significant bits either
// way, so exact), as packed bfloat16: cbf[row][w] holds bag 2w in its low
// half and bag 2w + 1 in its high half, the A operand layout below.  The
// workgroup's threads share the rows; the caller synchronizes before cbf is
// read.
template <int K, int P, int PB>
__device__ __forceinline__ void cm_counts_to_bf16(const uint32_t (*cnt)[P], uint32_t (*cbf)[PB],
                                                  uint32_t nrows, uint32_t mask, uint32_t tid,
                                                  uint32_t nthreads) {
  static_assert(K % 8 == 0 && P % 4 == 0 && PB % 4 == 0, "16-byte row pieces");
  constexpr uint32_t kPieces = K / 8;  // 8 counts in, 4 words out
  for (uint32_t x = tid; x < nrows * kPieces; x += nthreads) {
    const uint32_t row = x / kPieces, q = x % kPieces;
    const cm_u32x4 n0 = *reinterpret_cast<const cm_u32x4*>(&cnt[row][8u * q]);
    const cm_u32x4 n1 = *reinterpret_cast<const cm_u32x4*>(&cnt[row][8u * q + 4u]);
    cm_u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float c0 = (float)((j < 2 ? n0[2 * j] : n1[2 * j - 4]) & mask);
      const float c1 = (float)((j < 2 ? n0[2 * j + 1] : n1[2 * j - 3]) & mask);
      o[j] = (__float_as_uint(c0) >> 16) | (__float_as_uint(c1) & 0xffff0000u);
    }
    *reinterpret_cast<cm_u32x4*>(&cbf[row][4u * q]) = o;
  }
}

// As cm_counts_x_grad for counts already packed as bfloat16 by
// cm_counts_to_bf16 (row pitch PB words): each accumulator takes the lo,
// mid and hi products in that order, as there, so the sums are the same bit
// for bit.  Row tiles go four at a time, their products issued part by part
// across the four, so consecutive products never wait for each other's
// accumulator.  (Tiles past nrt in a group have zero operands: their rows
// exist in the accumulators and are not stored.)
template <int KSTEPS, int DT, int RT, int PB>
__device__ __forceinline__ void cm_bf16_x_grad(cm_f4 (&acc)[RT][DT], const uint32_t (*cbf)[PB],
                                               const float (&gv)[KSTEPS][8][DT], uint32_t nrt,
                                               uint32_t i, uint32_t kq) {
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    cm_u32x4 bp[3][DT];  // lo, mid, hi
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h, m, l;
        cm_split3(gv[ks][2 * j][nt], gv[ks][2 * j + 1][nt], h, m, l);
        bp[0][nt][j] = l;
        bp[1][nt][j] = m;
        bp[2][nt][j] = h;
      }
    // row tiles in groups of four: four operands in registers, and twelve
    // products per group of which each waits only for the one four back
    static_assert(RT % 4 == 0, "row tiles in groups of four");
#pragma unroll
    for (int g = 0; g < RT; g += 4) {
      if ((uint32_t)g >= nrt) break;  // uniform
      cm_u32x4 av[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        av[r] = (uint32_t)(g + r) < nrt
                    ? *reinterpret_cast<const cm_u32x4*>(
                          &cbf[(uint32_t)(g + r) * 16u + i][16u * (uint32_t)ks + 4u * kq])
                    : (cm_u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int nt = 0; nt < DT; ++nt)
            acc[g + r][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(cm_bf16x8, av[r]), __builtin_bit_cast(cm_bf16x8, bp[part][nt]),
                acc[g + r][nt], 0, 0, 0);
    }
  }
}

}  // namespace tbe
