// Small-table histogram forward (FBTriton TBE page, "Forward": for one small
// table, count how often each row occurs in a bag, then multiply counts by the
// table on the matrix cores; a program owns 16 bags and counts each bag's first
// 256 indices, the rest go through a plain gather).
//
// gfx950 design: a persistent workgroup keeps the whole table (<= 64 x 128
// fp16) transposed in LDS and loops over groups of 16 bags.  Counts are built
// with LDS integer atomics, converted to fp16 (exact: counts <= 256), and the
// [16 x 64] x [64 x D] product runs on v_mfma_f32_16x16x32_f16 (four waves,
// two 16-column tiles each, two K steps).  The tile is staged through LDS so
// the float32 output leaves as coalesced 16-byte stores.  Still HBM-bound: it
// reads the indices once and writes the output once.
//
// Saved histogram (FBTriton page, "Fusion boundaries": the small-table path
// keeps its histogram for the backward instead of fusing the two): with
// hist_save set, the lookups past a bag's first 256 are counted too, after
// the contraction has used the capped counts, and every bag's exact row
// counts are stored as uint16 (a count never exceeds its bag's length; the
// backward recomputes bags of 65536 lookups or more from their indices), with
// {B, N} in a header so that the backward uses them only for this batch.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kBags = 16;
constexpr int kEMax = 64;
constexpr int kDMax = 128;
constexpr int kCountCap = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void fwd_hist_kernel(FwdArgs a, uint32_t E, uint32_t D,
                                                            int mean) {
  __shared__ __attribute__((aligned(16))) _Float16 wt[kDMax][kEMax + 8];  // table transposed: [column][row]
  __shared__ uint32_t cnt[kBags][kEMax];
  __shared__ float tile[kBags][kDMax + 4];
  __shared__ int64_t boff[kBags + 1];

  const TableDev td = a.tables[0];
  const uint16_t* w = reinterpret_cast<const uint16_t*>(td.w);
  for (uint32_t i = threadIdx.x; i < kDMax * kEMax; i += kThreads) {
    const uint32_t col = i / kEMax, row = i % kEMax;
    uint16_t bits = (row < E && col < D) ? w[(size_t)row * D + col] : (uint16_t)0;
    wt[col][row] = __builtin_bit_cast(_Float16, bits);
  }

  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const int64_t ngroups = (a.B + kBags - 1) / kBags;
  if (a.hist_save && blockIdx.x == 0 && threadIdx.x == 0) {
    a.hist_hdr[0] = (uint32_t)a.B;
    a.hist_hdr[1] = a.n;
  }
  for (int64_t g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t b0 = g * kBags;
    const int nb = (int)((a.B - b0) < kBags ? (a.B - b0) : kBags);
    __syncthreads();  // previous group's tile fully stored; table loaded
    for (uint32_t i = threadIdx.x; i < kBags * kEMax; i += kThreads) (&cnt[0][0])[i] = 0u;
    if (threadIdx.x <= (uint32_t)nb) boff[threadIdx.x] = load_idx(a.offsets, a.itype, b0 + threadIdx.x);
    __syncthreads();

    // histogram of each bag's first kCountCap lookups
    const int64_t p0 = boff[0], p1 = boff[nb];
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kThreads) {
      int bi = 0;
#pragma unroll
      for (int k = 1; k < kBags; ++k) bi += (k < nb && boff[k] <= p) ? 1 : 0;
      if (p - boff[bi] < kCountCap) {
        const uint32_t r = (uint32_t)load_idx(a.indices, a.itype, p);
        if (r < E) atomicAdd(&cnt[bi][r], 1u);
      }
    }
    __syncthreads();

    // counts[16 x 64] (fp16, exact) x table[64 x D] on MFMA, fp32 accumulate
    {
      const uint32_t i = lane & 15, kq = lane >> 4;  // A row / B column, K group
      half8 av[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) av[ks][e] = (_Float16)(float)cnt[i][ks * 32 + kq * 8 + e];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const uint32_t col0 = (wave * 2 + nt) * 16;
        if (col0 >= D) continue;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          half8 bv = *reinterpret_cast<const half8*>(&wt[col0 + i][ks * 32 + kq * 8]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[ks], bv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) tile[kq * 4 + r][col0 + i] = acc[r];
      }
    }
    __syncthreads();

    // lookups past the first kCountCap of a bag: plain gather, one wave per bag,
    // sequential in lookup order (and counted for the saved histogram)
    for (int bi = (int)wave; bi < nb; bi += kThreads / kWave) {
      const int64_t q0 = boff[bi] + kCountCap, q1 = boff[bi + 1];
      for (int64_t q = q0; q < q1; ++q) {
        const uint32_t r = (uint32_t)load_idx(a.indices, a.itype, q);
        if (r >= E) continue;
        for (uint32_t col = lane; col < D; col += kWave) tile[bi][col] += (float)wt[col][r];
        if (a.hist_save && lane == 0) cnt[bi][r] += 1u;  // this wave owns the bag's counts
      }
    }
    __syncthreads();
    if (a.hist_save) {  // the group's exact counts, bag-major
      for (uint32_t e = threadIdx.x; e < (uint32_t)nb * E; e += kThreads) {
        const uint32_t bi = e / E, r = e % E;
        const uint32_t c = cnt[bi][r];
        a.hist_save[(b0 + bi) * (int64_t)E + r] = (uint16_t)(c < 65535u ? c : 65535u);
      }
    }

    // store rows b0 .. b0+nb-1 (mean divides by the bag length)
    const uint32_t q4 = D / 4;
    for (uint32_t e = threadIdx.x; e < (uint32_t)nb * q4; e += kThreads) {
      const uint32_t bi = e / q4, c4 = (e % q4) * 4;
      float4 v = make_float4(tile[bi][c4], tile[bi][c4 + 1], tile[bi][c4 + 2], tile[bi][c4 + 3]);
      const int64_t L = boff[bi + 1] - boff[bi];
      if (mean && L > 0) {
        const float fl = (float)L;
        v.x /= fl; v.y /= fl; v.z /= fl; v.w /= fl;
      }
      *reinterpret_cast<float4*>(a.out + (b0 + bi) * (int64_t)a.dtot + c4) = v;
    }
  }
}

}  // namespace

hipError_t launch_forward_hist(const FwdArgs& a, uint32_t E, uint32_t D, int mean, int grid,
                               hipStream_t s) {
  const int64_t ngroups = (a.B + kBags - 1) / kBags;
  if (ngroups == 0) return hipSuccess;
  const int g = (int)(ngroups < grid ? ngroups : grid);
  TBE_LAUNCH("fwd_hist", fwd_hist_kernel, dim3(g), dim3(kThreads), s, a, E, D, mean);
  return hipGetLastError();
}

}  // namespace tbe
