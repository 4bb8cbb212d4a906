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
constexpr int kCntPitch = kEMax + 4;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Positions of a group's lookups in flight per thread in the counting pass.
constexpr int kPer = 8;

template <typename IT>
__global__ __launch_bounds__(kThreads) void fwd_hist_kernel(FwdArgs a, uint32_t E, uint32_t D,
                                                            int mean) {
  __shared__ __attribute__((aligned(16))) _Float16 wt[kDMax][kEMax + 8];  // table transposed: [column][row]
  // counts; a row pitch of 68 words puts the 16 rows that the product's
  // operand reads take at once in distinct banks (a pitch of 64 put all 16
  // in one)
  __shared__ __attribute__((aligned(16))) uint32_t cnt[kBags][kCntPitch];
  __shared__ __attribute__((aligned(16))) float tile[kBags][kDMax + 4];
  __shared__ uint32_t boff[kBags + 1];  // positions (< 2^31)

  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const uint32_t N = a.n;

  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const int64_t ngroups = (a.B + kBags - 1) / kBags;
  if (a.hist_save && blockIdx.x == 0 && threadIdx.x == 0) {
    a.hist_hdr[0] = (uint32_t)a.B;
    a.hist_hdr[1] = a.n;
  }
  // this workgroup's groups [g_lo, g_hi): consecutive, so that a group's
  // first lookup is the previous group's end
  const int64_t g_lo = ngroups * (int64_t)blockIdx.x / (int64_t)gridDim.x;
  const int64_t g_hi = ngroups * (int64_t)(blockIdx.x + 1) / (int64_t)gridDim.x;
  if (g_lo >= g_hi) return;
  // The first group's boundaries and lookups are issued before the table's
  // load, whose latency they share; those of each next group as soon as the
  // current group's end is known, before its counting, so they arrive
  // meanwhile.  A group's loads: its bag boundaries (bag min(x, nb) for
  // thread x, every index in range) and its first kPer lookups per thread
  // from P0 (positions clamped to the last lookup; those past the group's
  // end are dropped where first used).
  uint32_t P0;
  {
    const int64_t o = (int64_t)O[g_lo * kBags];
    P0 = (uint32_t)(o < 0 ? 0 : (o > (int64_t)N ? (int64_t)N : o));
  }
  int64_t o_next = (int64_t)O[g_lo * kBags + min((int64_t)threadIdx.x,
                                                  min((int64_t)kBags, a.B - g_lo * kBags))];
  IT r[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u)
    r[u] = N > 0 ? I[min(P0 + threadIdx.x + (uint32_t)u * kThreads, N - 1u)] : (IT)0;

  const TableDev td = a.tables[0];
  const uint16_t* w = reinterpret_cast<const uint16_t*>(td.w);
  // the table into LDS, transposed: entries outside [0, E) x [0, D) are zero
  // (a zero count times them must give zero); rows are read as 8-byte
  // pieces of four columns (D is a multiple of 4), all in flight before the
  // first LDS write, when the weights are 8-byte aligned
  for (uint32_t i = threadIdx.x; i < kDMax * kEMax; i += kThreads) {
    const uint32_t col = i / kEMax, row = i % kEMax;
    if (row >= E || col >= D) wt[col][row] = (_Float16)0.f;
  }
  if ((reinterpret_cast<uintptr_t>(w) & 7u) == 0) {
    constexpr int kQuadsPer = kDMax * kEMax / 4 / kThreads;  // 8
    const uint32_t nq = E * D / 4;
    uint2 q[kQuadsPer];
#pragma unroll
    for (int k = 0; k < kQuadsPer; ++k)
      q[k] = reinterpret_cast<const uint2*>(w)[min(threadIdx.x + (uint32_t)k * kThreads, nq - 1u)];
#pragma unroll
    for (int k = 0; k < kQuadsPer; ++k) {
      const uint32_t x = threadIdx.x + (uint32_t)k * kThreads;
      if (x < nq) {
        const uint32_t row = 4u * x / D, col = 4u * x % D;
        wt[col][row] = __builtin_bit_cast(_Float16, (uint16_t)(q[k].x & 0xffffu));
        wt[col + 1][row] = __builtin_bit_cast(_Float16, (uint16_t)(q[k].x >> 16));
        wt[col + 2][row] = __builtin_bit_cast(_Float16, (uint16_t)(q[k].y & 0xffffu));
        wt[col + 3][row] = __builtin_bit_cast(_Float16, (uint16_t)(q[k].y >> 16));
      }
    }
  } else {
    for (uint32_t i = threadIdx.x; i < E * D; i += kThreads) {
      const uint32_t row = i / D, col = i % D;
      wt[col][row] = __builtin_bit_cast(_Float16, w[i]);
    }
  }
  for (int64_t g = g_lo; g < g_hi; ++g) {
    const int64_t b0 = g * kBags;
    const int nb = (int)((a.B - b0) < kBags ? (a.B - b0) : kBags);
    __syncthreads();  // previous group's tile fully stored; table loaded
    for (uint32_t i = threadIdx.x; i < kBags * kCntPitch; i += kThreads) (&cnt[0][0])[i] = 0u;
    if (threadIdx.x <= (uint32_t)kBags)
      boff[threadIdx.x] = (uint32_t)(o_next < 0 ? 0 : (o_next > (int64_t)N ? (int64_t)N : o_next));
    __syncthreads();
    const uint32_t P1 = min(max(boff[nb], P0), N);  // the group's lookups are [P0, P1)

    // the next group's boundaries and first lookups, in flight from here on,
    // through this group's counting, product and stores
    const bool more = g + 1 < g_hi;
    int64_t o_nn = 0;
    IT rn[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) rn[u] = (IT)0;
    if (more) {
      const int64_t nbn = min((int64_t)kBags, a.B - (b0 + kBags));
      o_nn = (int64_t)O[b0 + kBags + min((int64_t)threadIdx.x, nbn)];
      if (N > 0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          rn[u] = I[min(P1 + threadIdx.x + (uint32_t)u * kThreads, N - 1u)];
      }
    }

    // histogram of each bag's first kCountCap lookups: kPer lookups per
    // thread at a time, their bags by a search over the boundaries taken
    // level by level for all of them
    for (uint32_t q0 = P0; q0 < P1; q0 += (uint32_t)(kPer * kThreads)) {
      uint32_t row[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u)  // (an index outside [0, E), by its full value, counts nowhere)
        row[u] = (q0 + threadIdx.x + (uint32_t)u * kThreads < P1 &&
                  (uint64_t)(int64_t)r[u] < (uint64_t)E)
                     ? (uint32_t)r[u]
                     : 0xffffffffu;
      const uint32_t qn = q0 + (uint32_t)(kPer * kThreads);
      if (qn < P1) {
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          r[u] = I[min(qn + threadIdx.x + (uint32_t)u * kThreads, P1 - 1u)];
      }
      uint32_t bi[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) bi[u] = 0u;
#pragma unroll
      for (uint32_t step = (uint32_t)kBags / 2u; step > 0u; step >>= 1) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {  // boff[m] for m >= nb is the group's end
          const uint32_t m = bi[u] + step;
          bi[u] = boff[m] <= q0 + threadIdx.x + (uint32_t)u * kThreads ? m : bi[u];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t p = q0 + threadIdx.x + (uint32_t)u * kThreads;
        if (row[u] < E && p - boff[bi[u]] < (uint32_t)kCountCap) atomicAdd(&cnt[bi[u]][row[u]], 1u);
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
        for (int h = 0; h < 2; ++h) {
          const uint4 c4 = *reinterpret_cast<const uint4*>(&cnt[i][ks * 32 + kq * 8 + 4 * h]);
          av[ks][4 * h] = (_Float16)(float)c4.x;
          av[ks][4 * h + 1] = (_Float16)(float)c4.y;
          av[ks][4 * h + 2] = (_Float16)(float)c4.z;
          av[ks][4 * h + 3] = (_Float16)(float)c4.w;
        }
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
        for (int r4 = 0; r4 < 4; ++r4) tile[kq * 4 + r4][col0 + i] = acc[r4];
      }
    }
    __syncthreads();

    // lookups past the first kCountCap of a bag: plain gather, one wave per bag,
    // sequential in lookup order (and counted for the saved histogram)
    for (int bj = (int)wave; bj < nb; bj += kThreads / kWave) {
      const uint32_t q1 = boff[bj + 1];
      for (uint32_t q = boff[bj] + (uint32_t)kCountCap; q < q1; ++q) {
        const int64_t rr = (int64_t)I[q];
        if ((uint64_t)rr >= (uint64_t)E) continue;
        for (uint32_t col = lane; col < D; col += kWave) tile[bj][col] += (float)wt[col][rr];
        if (a.hist_save && lane == 0) cnt[bj][rr] += 1u;  // this wave owns the bag's counts
      }
    }
    __syncthreads();
    if (a.hist_save) {  // the group's exact counts, bag-major
      for (uint32_t e = threadIdx.x; e < (uint32_t)nb * E; e += kThreads) {
        const uint32_t bj = e / E, rr = e % E;
        const uint32_t c = cnt[bj][rr];
        a.hist_save[(b0 + bj) * (int64_t)E + rr] = (uint16_t)(c < 65535u ? c : 65535u);
      }
    }

    // store rows b0 .. b0+nb-1 (mean divides by the bag length)
    const uint32_t q4 = D / 4;
    for (uint32_t e = threadIdx.x; e < (uint32_t)nb * q4; e += kThreads) {
      const uint32_t bj = e / q4, c4 = (e % q4) * 4;
      float4 v = *reinterpret_cast<const float4*>(&tile[bj][c4]);  // (rows of 528 bytes)
      const int64_t L = (int64_t)boff[bj + 1] - (int64_t)boff[bj];
      if (mean && L > 0) {
        const float fl = (float)L;
        v.x /= fl; v.y /= fl; v.z /= fl; v.w /= fl;
      }
      *reinterpret_cast<float4*>(a.out + (b0 + bj) * (int64_t)a.dtot + c4) = v;
    }
    P0 = P1;
    if (more) {
      o_next = o_nn;
#pragma unroll
      for (int u = 0; u < kPer; ++u) r[u] = rn[u];
    }
  }
}

}  // namespace

hipError_t launch_forward_hist(const FwdArgs& a, uint32_t E, uint32_t D, int mean, int grid,
                               hipStream_t s) {
  const int64_t ngroups = (a.B + kBags - 1) / kBags;
  if (ngroups == 0) return hipSuccess;
  const int g = (int)(ngroups < grid ? ngroups : grid);
  if (a.itype == IT_I32)
    TBE_LAUNCH("fwd_hist", fwd_hist_kernel<int32_t>, dim3(g), dim3(kThreads), s, a, E, D, mean);
  else
    TBE_LAUNCH("fwd_hist", fwd_hist_kernel<int64_t>, dim3(g), dim3(kThreads), s, a, E, D, mean);
  return hipGetLastError();
}

}  // namespace tbe
