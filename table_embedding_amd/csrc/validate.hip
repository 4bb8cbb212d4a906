// Input validation and repair (FBTriton TBE page, "Forward": the kernels do
// not check their inputs; an optional bounds check and offset repair is a
// separate pass whose cost is to be measured).  The contract the other
// kernels assume: O[0] = 0, O[T*B] = N, O non-decreasing, and every index of
// table t's bags in [0, R_t).
//
// Check: one thread per bag checks its offset pair; every index is checked
// once by a flat, coalesced pass over [0, N), its table found from the table
// start offsets (one thread per bag walking its own lookups read the indices
// at 0.45 TB/s on C5).  Every access is clamped, so invalid inputs are read
// safely.  Findings go to the error block with atomics: error bits (OR), the
// number of bad indices (add), the first bag with a finding and the first bad
// position (min).  Repair (only with TBE_VALIDATE_REPAIR, after the check):
// out-of-range indices set to row 0 (bags keep their lengths), then offsets
// clamped into [0, N] with O[0] = 0 and O[T*B] = N.  Non-decreasing order is
// reported, not repaired.
#include "tbe_common.h"

namespace tbe {
namespace {

__global__ __launch_bounds__(kThreads) void validate_clear_kernel(uint32_t* err) {
  if (threadIdx.x < (uint32_t)kValWords)
    err[threadIdx.x] = (threadIdx.x == kValFirstBag || threadIdx.x == kValFirstPos) ? 0xffffffffu
                                                                                    : 0u;
}

// One thread per bag: its offset pair (and bag 0 the start offset, the last
// bag the end offset).
template <typename IT>
__global__ __launch_bounds__(kThreads) void validate_offsets_kernel(ValArgs v, uint32_t* err) {
  const IT* __restrict__ O = reinterpret_cast<const IT*>(v.offsets);
  const uint64_t nbag = (uint64_t)v.T * (uint64_t)v.B;
  const uint64_t j = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t bits = 0;
  if (j == 0 && (int64_t)O[0] != 0) bits |= kValOffsetStart;
  if (j == (nbag > 0 ? nbag - 1 : 0) && (int64_t)O[nbag] != v.N) bits |= kValOffsetEnd;
  if (j < nbag) {
    const int64_t lo = (int64_t)O[j], hi = (int64_t)O[j + 1];
    if (lo > hi) bits |= kValOffsetOrder;
    if (lo < 0 || lo > v.N || hi < 0 || hi > v.N) bits |= kValOffsetRange;
  }
  if (bits) {
    atomicOr(&err[kValBits], bits);
    if (j < nbag) atomicMin(&err[kValFirstBag], (uint32_t)j);
  }
}

// Table of position p: the last table whose first offset (clamped into
// [0, N]) is <= p, by binary search over s_tb (an arbitrary table in [0, T)
// when the table offsets are out of order, which the offset check reports).
__device__ __forceinline__ uint32_t table_of(const uint32_t* s_tb, uint32_t T, uint32_t p) {
  uint32_t lo = 0, hi = T;  // s_tb[lo] <= p < s_tb[hi] when ordered
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) >> 1;
    if (s_tb[mid] <= p) lo = mid; else hi = mid;
  }
  return lo;
}

// Every index once, in one coalesced pass over [0, N): workgroup w takes the
// contiguous positions [w*chunk, (w+1)*chunk), so a thread's positions only
// increase and its table is found once by binary search, then advanced; the
// table offsets and row counts are kept in LDS.  REPAIR: an index out of
// range becomes row 0; else it is counted, and the first bad position and
// its bag (searched among the table's offsets, only for bad positions) are
// recorded.
template <typename IT, bool REPAIR>
__global__ __launch_bounds__(kThreads) void validate_indices_kernel(ValArgs v, uint32_t* err) {
  __shared__ uint32_t s_tb[kMaxTables + 1];
  __shared__ uint32_t s_rows[kMaxTables];
  IT* I = reinterpret_cast<IT*>(v.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(v.offsets);
  const uint32_t T = v.T;
  for (uint32_t t = threadIdx.x; t <= T; t += kThreads) {
    const int64_t o = (int64_t)O[(int64_t)t * v.B];
    s_tb[t] = (uint32_t)(o < 0 ? 0 : (o > v.N ? v.N : o));
    if (t < T) s_rows[t] = v.tables[t].rows;
  }
  __syncthreads();
  uint32_t bad = 0, firstpos = 0xffffffffu, firstbag = 0xffffffffu;
  const uint64_t chunk = ((uint64_t)v.N + gridDim.x - 1) / gridDim.x;
  const uint64_t cb = (uint64_t)blockIdx.x * chunk;
  const uint64_t ce = cb + chunk < (uint64_t)v.N ? cb + chunk : (uint64_t)v.N;
  uint32_t t = cb + threadIdx.x < ce ? table_of(s_tb, T, (uint32_t)(cb + threadIdx.x)) : 0u;
  for (uint64_t p0 = cb + threadIdx.x; p0 < ce; p0 += 4 * kThreads) {
    int64_t r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t p = p0 + (uint64_t)u * kThreads;
      r[u] = p < ce ? (int64_t)I[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t p = p0 + (uint64_t)u * kThreads;
      if (p >= ce) continue;
      while (t + 1 < T && s_tb[t + 1] <= (uint32_t)p) ++t;  // positions only increase
      if (r[u] >= 0 && r[u] < (int64_t)s_rows[t]) continue;
      if (REPAIR) {
        I[p] = (IT)0;
        continue;
      }
      ++bad;
      if (p < firstpos) {
        firstpos = (uint32_t)p;
        // its bag: the last bag of table t whose start offset is <= p
        int64_t lo = (int64_t)t * v.B, hi = lo + v.B;
        while (hi - lo > 1) {
          const int64_t mid = (lo + hi) >> 1;
          if ((int64_t)O[mid] <= (int64_t)p) lo = mid; else hi = mid;
        }
        firstbag = (uint32_t)lo;
      }
    }
  }
  if (bad) {
    atomicOr(&err[kValBits], kValIndexRange);
    atomicAdd(&err[kValBadIndices], bad);
    atomicMin(&err[kValFirstPos], firstpos);
    atomicMin(&err[kValFirstBag], firstbag);
  }
}

template <typename IT>
__global__ __launch_bounds__(kThreads) void validate_clamp_kernel(ValArgs v) {
  IT* O = reinterpret_cast<IT*>(v.offsets);
  const uint64_t nbag = (uint64_t)v.T * (uint64_t)v.B;
  const uint64_t j = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (j > nbag) return;
  const int64_t o = (int64_t)O[j];
  const int64_t c = j == 0 ? 0 : (j == nbag ? v.N : (o < 0 ? 0 : (o > v.N ? v.N : o)));
  if (c != o) O[j] = (IT)c;
}

}  // namespace

hipError_t launch_validate_clear(uint32_t* err, hipStream_t s) {
  TBE_LAUNCH("validate_clear", validate_clear_kernel, dim3(1), dim3(kThreads), s, err);
  return hipGetLastError();
}

hipError_t launch_validate(const ValArgs& v, int itype, uint32_t* err, bool repair,
                           hipStream_t s) {
  const uint64_t nbag = (uint64_t)v.T * (uint64_t)v.B;
  const uint32_t ogrid = (uint32_t)((nbag + 1 + kThreads - 1) / kThreads);
  const uint32_t igrid =
      (uint32_t)std::max<int64_t>(1, std::min<int64_t>(2048, (v.N + 1023) / 1024));
  TBE_LAUNCH("validate_clear", validate_clear_kernel, dim3(1), dim3(kThreads), s, err);
  if (itype == IT_I32) {
    TBE_LAUNCH("validate_check", validate_offsets_kernel<int32_t>, dim3(ogrid), dim3(kThreads),
               s, v, err);
    TBE_LAUNCH("validate_check", (validate_indices_kernel<int32_t, false>), dim3(igrid),
               dim3(kThreads), s, v, err);
    if (repair) {
      TBE_LAUNCH("validate_repair", (validate_indices_kernel<int32_t, true>), dim3(igrid),
                 dim3(kThreads), s, v, err);
      TBE_LAUNCH("validate_repair", validate_clamp_kernel<int32_t>, dim3(ogrid), dim3(kThreads),
                 s, v);
    }
  } else {
    TBE_LAUNCH("validate_check", validate_offsets_kernel<int64_t>, dim3(ogrid), dim3(kThreads),
               s, v, err);
    TBE_LAUNCH("validate_check", (validate_indices_kernel<int64_t, false>), dim3(igrid),
               dim3(kThreads), s, v, err);
    if (repair) {
      TBE_LAUNCH("validate_repair", (validate_indices_kernel<int64_t, true>), dim3(igrid),
                 dim3(kThreads), s, v, err);
      TBE_LAUNCH("validate_repair", validate_clamp_kernel<int64_t>, dim3(ogrid), dim3(kThreads),
                 s, v);
    }
  }
  return hipGetLastError();
}

}  // namespace tbe
