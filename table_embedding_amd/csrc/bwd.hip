// Backward with exact row-wise Adagrad, once per touched row (FBTriton TBE
// page, "Backward": runs with SL < 256 are gathered, accumulated in registers
// and updated by one owner with plain stores; runs with SL >= 256 are cut into
// 256-lookup chunks whose partial sums are stored and then reduced by a second
// kernel, or, in the fused form, each chunk fences its partial and decrements a
// countdown so that only the last chunk updates the row.  Section "Fusion
// boundaries": per-sample weights scale each contribution before grouping and
// the optimizer runs as the epilogue).
//
// Every kernel is persistent over a task list whose length lives in device
// memory (no host readback).  Row updates read the gradient rows of the bags
// that used the row (random 16-byte column slices of grad_out), so the path is
// HBM/L2 bandwidth- and latency-bound; gathers keep four lookups in flight.
//
// Determinism: a long run's gradient is the sum of its chunk partials, chunk
// k folded into subgroup (k mod nsg) in ascending k, subgroups combined in
// ascending order, the square-sum reduced in a fixed tree.  The two-launch
// update and the fused last-chunk update call the same workgroup routine, so
// the two give bit-identical weights.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kGatherInFlight = 4;

// Per-lookup contribution scale S[p] * (1/L if mean) and grad_out row.
__device__ __forceinline__ void lookup_meta(const BwdArgs& a, uint32_t pos, int64_t tB, bool mean,
                                            float& sc, int64_t& b) {
  const uint32_t j = a.bag[pos];
  b = (int64_t)j - tB;
  sc = a.psw ? a.psw[pos] : 1.0f;
  if (mean) {
    const int64_t L = load_idx(a.offsets, a.itype, (int64_t)j + 1) - load_idx(a.offsets, a.itype, j);
    sc = sc / (float)L;
  }
}

// Accumulate lookups [i0, i1) with stride `step` of sorted slots into g.
template <int VEC, int NC>
__device__ __forceinline__ void gather(const BwdArgs& a, const TableDev& td, int64_t tB,
                                       uint32_t i0, uint32_t i1, uint32_t step,
                                       const uint32_t* colc, const bool* act, float (*g)[VEC]) {
  const bool mean = td.pooling == POOL_MEAN;
  const float* gbase = a.grad + td.col;
  uint32_t i = i0;
  for (; i + (kGatherInFlight - 1) * step < i1; i += kGatherInFlight * step) {
    uint32_t pos[kGatherInFlight];
#pragma unroll
    for (int k = 0; k < kGatherInFlight; ++k) pos[k] = a.sorted_pos[i + k * step];
    float sc[kGatherInFlight];
    int64_t b[kGatherInFlight];
#pragma unroll
    for (int k = 0; k < kGatherInFlight; ++k) lookup_meta(a, pos[k], tB, mean, sc[k], b[k]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!act[c]) continue;
      float v[kGatherInFlight][VEC];
#pragma unroll
      for (int k = 0; k < kGatherInFlight; ++k)
        load_f32<VEC>(gbase + b[k] * (int64_t)a.dtot + colc[c], v[k]);
#pragma unroll
      for (int k = 0; k < kGatherInFlight; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) g[c][e] += sc[k] * v[k][e];
    }
  }
  for (; i < i1; i += step) {
    const uint32_t pos = a.sorted_pos[i];
    float sc;
    int64_t b;
    lookup_meta(a, pos, tB, mean, sc, b);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!act[c]) continue;
      float v[VEC];
      load_f32<VEC>(gbase + b * (int64_t)a.dtot + colc[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[c][e] += sc * v[e];
    }
  }
}

// Sanity bounds of list entries (they hold for every list the preprocessing
// writes; a stale or foreign workspace is skipped instead of read out of bounds).
__device__ __forceinline__ bool chunk_ok(const BwdArgs& a, uint4 task) {
  return task.z < a.T && task.x <= a.N && task.y <= a.N - task.x && task.y <= (uint32_t)kChunk &&
         task.w < a.max_long;
}
__device__ __forceinline__ bool long_ok(const BwdArgs& a, uint32_t l) {
  const uint4 t = a.long_task[l];
  if (t.w >= a.T || t.x > a.N || t.y > a.N - t.x || t.z >= a.tables[t.w].rows) return false;
  const uint32_t nch = (t.y + kChunk - 1) / kChunk;
  const uint32_t cb = a.long_cbeg[l];
  return cb <= a.max_chunks && nch <= a.max_chunks - cb;
}

// --------------------------------------------------------------- short runs
// One subgroup of lpr lanes owns a run: gather, Adagrad, plain stores.
template <int WD, int VEC, int NC>
__global__ __launch_bounds__(kThreads) void bwd_short_kernel(BwdArgs a, BucketDev bk,
                                                             uint32_t bucket) {
  const uint32_t lpr = bk.lpr;
  const uint32_t lane_in = threadIdx.x & (lpr - 1);
  const uint32_t nsg_grid = (gridDim.x * kThreads) >> bk.lpr_log2;
  const uint32_t sg = (blockIdx.x * kThreads + threadIdx.x) >> bk.lpr_log2;
  const uint32_t beg = a.counters[kCntBegins + bucket];
  const uint32_t end = min(a.counters[kCntBegins + bucket + 1], a.max_short);
  for (uint32_t s = beg + sg; s < end; s += nsg_grid) {
    const uint4 task = a.short_task[s];  // {start, len, row, table}
    if (task.w >= a.T || task.x > a.N || task.y > a.N - task.x) continue;  // never for valid lists
    const TableDev td = a.tables[task.w];
    if (task.z >= td.rows) continue;
    const uint32_t D = td.dim;
    const int64_t row = task.z;
    uint32_t colc[NC];
    bool act[NC];
    float w[NC][VEC], g[NC][VEC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
      act[c] = colc[c] < D;
      if (act[c]) load_w<WD, VEC>(td.w, row * D + colc[c], w[c]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[c][e] = 0.f;
    }
    const float m0 = td.m[row];
    gather<VEC, NC>(a, td, (int64_t)task.w * a.B, task.x, task.x + task.y, 1u, colc, act, g);
    float sq = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (act[c])
#pragma unroll
        for (int e = 0; e < VEC; ++e) sq += g[c][e] * g[c][e];
    sq = subgroup_sum(sq, lpr);
    const float m = m0 + sq / (float)D;
    if (lane_in == 0) {
      td.m[row] = m;
      if (a.debug_count) atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
    }
    const float den = sqrtf(m) + a.eps;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!act[c]) continue;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = w[c][e] - (a.lr * g[c][e]) / den;
      store_w<WD, VEC>(td.w, row * D + colc[c], o);
    }
  }
}

// ---------------------------------------------------------------- long runs

template <int VEC, int NC>
struct LongSmem {
  float red[kThreads * VEC * NC];  // [nsg][bucket width] per-subgroup sums
  float gsum[kThreads * VEC * NC / 1];
  float wsq[kThreads / kWave];
  uint32_t last;
};

// Chunk partial: the workgroup sums the chunk's <= 256 lookups; subgroup sg
// takes slots start+sg, start+sg+nsg, ...; subgroups are combined in order.
template <int VEC, int NC>
__device__ __forceinline__ void chunk_partial(const BwdArgs& a, const BucketDev& bk, uint4 task,
                                              LongSmem<VEC, NC>& sm) {
  const uint32_t lpr = bk.lpr, lane_in = threadIdx.x & (lpr - 1);
  const uint32_t sg = threadIdx.x >> bk.lpr_log2, nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = lpr * VEC * NC;
  const TableDev td = a.tables[task.z];
  const uint32_t D = td.dim;
  uint32_t colc[NC];
  bool act[NC];
  float g[NC][VEC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
    act[c] = colc[c] < D;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[c][e] = 0.f;
  }
  gather<VEC, NC>(a, td, (int64_t)task.z * a.B, task.x + sg, task.x + task.y, nsg, colc, act, g);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.red[sg * width + colc[c] + e] = g[c][e];
  __syncthreads();
}

// Write the combined chunk partial (ascending subgroup order) to partial[c].
template <int VEC, int NC>
__device__ __forceinline__ void chunk_store(const BwdArgs& a, const BucketDev& bk, uint32_t D,
                                            uint32_t c, LongSmem<VEC, NC>& sm) {
  const uint32_t nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = bk.lpr * VEC * NC;
  float* dst = a.partial + (size_t)c * a.pstride;
  for (uint32_t col = threadIdx.x; col < D; col += kThreads) {
    float s = 0.f;
    for (uint32_t k = 0; k < nsg; ++k) s += sm.red[k * width + col];
    dst[col] = s;
  }
}

// Long-run update: reduce the run's chunk partials, then row-wise Adagrad.
// All 256 threads of the workgroup take part.
template <int WD, int VEC, int NC>
__device__ __forceinline__ void long_update(const BwdArgs& a, const BucketDev& bk, uint32_t l,
                                            LongSmem<VEC, NC>& sm) {
  const uint32_t lpr = bk.lpr, lane_in = threadIdx.x & (lpr - 1);
  const uint32_t sg = threadIdx.x >> bk.lpr_log2, nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = lpr * VEC * NC;
  const uint4 task = a.long_task[l];  // {start, len, row, table}
  const uint32_t cb = a.long_cbeg[l];
  const uint32_t nch = (task.y + kChunk - 1) / kChunk;
  const TableDev td = a.tables[task.w];
  const uint32_t D = td.dim;
  const int64_t row = task.z;
  float g[NC][VEC];
  uint32_t colc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[c][e] = 0.f;
  }
  for (uint32_t k = sg; k < nch; k += nsg) {
    const float* src = a.partial + (size_t)(cb + k) * a.pstride;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (colc[c] >= D) continue;
      float v[VEC];
      load_f32<VEC>(src + colc[c], v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[c][e] += v[e];
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.red[sg * width + colc[c] + e] = g[c][e];
  __syncthreads();
  float sqp = 0.f;
  for (uint32_t col = threadIdx.x; col < D; col += kThreads) {
    float s = 0.f;
    for (uint32_t k = 0; k < nsg; ++k) s += sm.red[k * width + col];
    sm.gsum[col] = s;
    sqp += s * s;
  }
  // fixed-order reduction of the square sum: butterfly in the wave, waves in order
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) sqp += __shfl_xor(sqp, o, kWave);
  if (lane_id() == 0) sm.wsq[threadIdx.x / kWave] = sqp;
  __syncthreads();
  const float sq = ((sm.wsq[0] + sm.wsq[1]) + sm.wsq[2]) + sm.wsq[3];
  const float m = td.m[row] + sq / (float)D;
  const float den = sqrtf(m) + a.eps;
  for (uint32_t col = threadIdx.x * VEC; col < D; col += kThreads * VEC) {
    float w[VEC], o[VEC];
    load_w<WD, VEC>(td.w, row * D + col, w);
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = w[e] - (a.lr * sm.gsum[col + e]) / den;
    store_w<WD, VEC>(td.w, row * D + col, o);
  }
  __syncthreads();  // every thread has read td.m[row] and gsum before they change
  if (threadIdx.x == 0) {
    td.m[row] = m;
    if (a.debug_count) atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
  }
}

template <int WD, int VEC, int NC>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(BwdArgs a, BucketDev bk,
                                                             uint32_t bucket) {
  __shared__ LongSmem<VEC, NC> sm;
  const uint32_t nb1 = a.nb + 1;
  const uint32_t beg = a.counters[kCntBegins + 2 * nb1 + bucket];
  const uint32_t end = min(a.counters[kCntBegins + 2 * nb1 + bucket + 1], a.max_chunks);
  for (uint32_t c = beg + blockIdx.x; c < end; c += gridDim.x) {
    const uint4 task = a.chunk_task[c];  // {start, len, table, long index}
    if (!chunk_ok(a, task)) continue;    // uniform per workgroup; never for valid lists
    chunk_partial<VEC, NC>(a, bk, task, sm);
    chunk_store<VEC, NC>(a, bk, a.tables[task.z].dim, c, sm);
    __syncthreads();
  }
}

template <int WD, int VEC, int NC>
__global__ __launch_bounds__(kThreads) void bwd_long_update_kernel(BwdArgs a, BucketDev bk,
                                                                   uint32_t bucket) {
  __shared__ LongSmem<VEC, NC> sm;
  const uint32_t nb1 = a.nb + 1;
  const uint32_t beg = a.counters[kCntBegins + nb1 + bucket];
  const uint32_t end = min(a.counters[kCntBegins + nb1 + bucket + 1], a.max_long);
  for (uint32_t l = beg + blockIdx.x; l < end; l += gridDim.x) {
    if (!long_ok(a, l)) continue;  // uniform per workgroup; never for valid lists
    long_update<WD, VEC, NC>(a, bk, l, sm);
  }
}

// Fused: each chunk publishes its partial (device-scope release), then counts
// down the run's remaining chunks; the workgroup that takes the count to zero
// acquires and performs the update, then re-arms the countdown.
template <int WD, int VEC, int NC>
__global__ __launch_bounds__(kThreads) void bwd_chunk_fused_kernel(BwdArgs a, BucketDev bk,
                                                                   uint32_t bucket) {
  __shared__ LongSmem<VEC, NC> sm;
  const uint32_t nb1 = a.nb + 1;
  const uint32_t beg = a.counters[kCntBegins + 2 * nb1 + bucket];
  const uint32_t end = min(a.counters[kCntBegins + 2 * nb1 + bucket + 1], a.max_chunks);
  for (uint32_t c = beg + blockIdx.x; c < end; c += gridDim.x) {
    const uint4 task = a.chunk_task[c];  // {start, len, table, long index}
    if (!chunk_ok(a, task) || !long_ok(a, task.w)) continue;  // uniform; never for valid lists
    chunk_partial<VEC, NC>(a, bk, task, sm);
    chunk_store<VEC, NC>(a, bk, a.tables[task.z].dim, c, sm);
    __threadfence();  // this thread's partial stores are visible device-wide
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&a.remaining[task.w], 0xffffffffu,
                                                  __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      sm.last = (old == 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (sm.last) {
      __threadfence();  // acquire: other chunks' partials
      long_update<WD, VEC, NC>(a, bk, task.w, sm);
      if (threadIdx.x == 0) {
        const uint32_t len = a.long_task[task.w].y;
        __hip_atomic_store(&a.remaining[task.w], (len + kChunk - 1) / kChunk, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
  }
}

template <int WD, int VEC, int NC>
hipError_t launch(const BwdArgs& a, const BucketDev& bk, uint32_t bucket, bool fused, int grid,
                  hipStream_t s) {
  TBE_LAUNCH("bwd_short", (bwd_short_kernel<WD, VEC, NC>), dim3(grid), dim3(kThreads), s, a, bk,
             bucket);
  if (fused) {
    TBE_LAUNCH("bwd_chunk_fused", (bwd_chunk_fused_kernel<WD, VEC, NC>), dim3(grid),
               dim3(kThreads), s, a, bk, bucket);
  } else {
    TBE_LAUNCH("bwd_chunk", (bwd_chunk_kernel<WD, VEC, NC>), dim3(grid), dim3(kThreads), s, a,
               bk, bucket);
    TBE_LAUNCH("bwd_long_update", (bwd_long_update_kernel<WD, VEC, NC>), dim3(grid),
               dim3(kThreads), s, a, bk, bucket);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_bucket(const BwdArgs& a, const BucketDev& bk, uint32_t bucket, int wd,
                                  int vec, int nc, bool fused, int grid, hipStream_t s) {
#define TBE_BWD_CASE(W, V, N) \
  if (wd == W && vec == V && nc == N) return launch<W, V, N>(a, bk, bucket, fused, grid, s);
  TBE_BWD_CASE(WD_F32, 4, 1)
  TBE_BWD_CASE(WD_F32, 4, 2)
  TBE_BWD_CASE(WD_F32, 4, 4)
  TBE_BWD_CASE(WD_F16, 4, 1)
  TBE_BWD_CASE(WD_F16, 4, 2)
  TBE_BWD_CASE(WD_F16, 4, 4)
  TBE_BWD_CASE(WD_F16, 8, 1)
  TBE_BWD_CASE(WD_F16, 8, 2)
  TBE_BWD_CASE(WD_BF16, 4, 1)
  TBE_BWD_CASE(WD_BF16, 4, 2)
  TBE_BWD_CASE(WD_BF16, 4, 4)
  TBE_BWD_CASE(WD_BF16, 8, 1)
  TBE_BWD_CASE(WD_BF16, 8, 2)
#undef TBE_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tbe
