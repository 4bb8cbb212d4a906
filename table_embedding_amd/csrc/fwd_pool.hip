// Generic forward gather-pool (FBTriton TBE page, "Forward": each bag gathers
// its indexed rows and pools them; 16-bit weights accumulate in float32 and
// float32 weights in float64; tables are bucketed by next_pow2(D) so narrow
// tables do not idle lanes sized for the widest one, section "Fewer reads and
// synchronizations").
//
// Lane mapping: one subgroup of `lpr` lanes per bag; lane k covers columns
// k*VEC + c*lpr*VEC (c < NC) with 16-byte (VEC elements) row loads, so a row
// of the bucket width is read by consecutive lanes in one coalesced sweep.
//
// Memory-level parallelism: lookups are taken eight at a time.  The eight
// indices are loaded, then the eight rows, then the eight rows are
// accumulated in lookup order; scheduling barriers keep the compiler from
// sinking each row load next to its use, which would leave one row in flight.
// A partial last batch repeats the bag's last index and drops the repeats with
// a select, so the batch has no branches (the repeated row is a cache hit).
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kInFlight = 8;

template <int WD>
struct Acc {
  using T = float;
};
template <>
struct Acc<WD_F32> {
  using T = double;
};

template <int WD, int VEC, int NC, typename IT, bool PSW>
__global__ __launch_bounds__(kThreads) void fwd_pool_kernel(FwdArgs a, BucketSet S) {
  using AT = typename Acc<WD>::T;
  BucketDev bk;
  uint32_t bucket_id, lb, lg;
  set_pick(S, bk, bucket_id, lb, lg);
  const uint32_t lpr = bk.lpr;
  const uint32_t lane_in = threadIdx.x & (lpr - 1);
  const uint64_t sg = ((uint64_t)lb * kThreads + threadIdx.x) >> bk.lpr_log2;
  const uint64_t nbags = (uint64_t)bk.ntables * (uint64_t)a.B;
  if (sg >= nbags) return;
  const uint32_t slot = (uint32_t)(sg / (uint64_t)a.B);
  const int64_t b = (int64_t)(sg - (uint64_t)slot * (uint64_t)a.B);
  const uint32_t t = bk.tables[slot];
  const TableDev td = a.tables[t];
  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const int64_t j = (int64_t)t * a.B + b;
  const int64_t lo = O[j];
  const int64_t hi = O[j + 1];
  const uint32_t D = td.dim;

  AT acc[NC][VEC];
  bool act[NC];
  uint32_t colc[NC], cold[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[c][v] = AT(0);
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
    act[c] = colc[c] < D;
    cold[c] = act[c] ? colc[c] : 0u;  // idle lanes read column 0 and discard it
  }

  // software pipeline: the indices of batch i+1 are loaded while the rows of
  // batch i are in flight, so a batch costs one memory round trip
  int64_t nrow[kInFlight];
  float ns[kInFlight];
  if (lo < hi) {
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int64_t q = lo + k < hi ? lo + k : hi - 1;
      nrow[k] = (int64_t)I[q];
      ns[k] = PSW ? a.psw[q] : 1.0f;
    }
  }
  for (int64_t p = lo; p < hi; p += kInFlight) {
    int64_t row[kInFlight];
    float s[kInFlight];
    bool ok[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      row[k] = nrow[k];
      s[k] = ns[k];
      ok[k] = p + k < hi;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float v[kInFlight][VEC];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) load_w<WD, VEC>(td.w, row[k] * D + cold[c], v[k]);
      if (c == 0) {
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
          const int64_t q = p + kInFlight + k < hi ? p + kInFlight + k : hi - 1;
          nrow[k] = (int64_t)I[q];
          ns[k] = PSW ? a.psw[q] : 1.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[c][e] += ok[k] ? AT(s[k]) * AT(v[k][e]) : AT(0);
    }
  }

  const bool mean = td.pooling == POOL_MEAN && hi > lo;
  const AT L = AT(hi - lo);
  float* orow = a.out + b * (int64_t)a.dtot + td.col;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!act[c]) continue;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = (float)(mean ? acc[c][e] / L : acc[c][e]);
    store_f32<VEC>(orow + colc[c], o);
  }
}

template <int WD, int VEC, int NC, typename IT, bool PSW>
hipError_t launch_t(const FwdArgs& a, const BucketSet& S, hipStream_t s) {
  const uint32_t grid = S.gbeg[S.n];
  if (grid == 0) return hipSuccess;
  TBE_LAUNCH("fwd_pool", (fwd_pool_kernel<WD, VEC, NC, IT, PSW>), dim3(grid), dim3(kThreads), s,
             a, S);
  return hipGetLastError();
}

template <int WD, int VEC, int NC>
hipError_t launch(const FwdArgs& a, const BucketSet& S, hipStream_t s) {
  if (a.itype == IT_I32)
    return a.psw ? launch_t<WD, VEC, NC, int32_t, true>(a, S, s)
                 : launch_t<WD, VEC, NC, int32_t, false>(a, S, s);
  return a.psw ? launch_t<WD, VEC, NC, int64_t, true>(a, S, s)
               : launch_t<WD, VEC, NC, int64_t, false>(a, S, s);
}

}  // namespace

hipError_t launch_forward_set(const FwdArgs& a, const BucketSet& bk, int wd, int vec, int nc,
                              hipStream_t s) {
#define TBE_FWD_CASE(W, V, N) \
  if (wd == W && vec == V && nc == N) return launch<W, V, N>(a, bk, s);
  TBE_FWD_CASE(WD_F32, 4, 1)
  TBE_FWD_CASE(WD_F32, 4, 2)
  TBE_FWD_CASE(WD_F32, 4, 4)
  TBE_FWD_CASE(WD_F16, 4, 1)
  TBE_FWD_CASE(WD_F16, 4, 2)
  TBE_FWD_CASE(WD_F16, 4, 4)
  TBE_FWD_CASE(WD_F16, 8, 1)
  TBE_FWD_CASE(WD_F16, 8, 2)
  TBE_FWD_CASE(WD_BF16, 4, 1)
  TBE_FWD_CASE(WD_BF16, 4, 2)
  TBE_FWD_CASE(WD_BF16, 4, 4)
  TBE_FWD_CASE(WD_BF16, 8, 1)
  TBE_FWD_CASE(WD_BF16, 8, 2)
#undef TBE_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tbe
