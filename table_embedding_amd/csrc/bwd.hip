// Backward with exact row-wise Adagrad, once per touched row (FBTriton TBE
// page, "Backward": a run with SL < 256 is gathered, accumulated and updated by
// one program that owns the row and writes it with plain stores; a run with
// SL >= 256 is cut into 256-lookup chunks whose partial sums are stored and
// reduced by a second kernel, or, in the fused form, each chunk publishes its
// partial and decrements a countdown so that only the last chunk updates the
// row; the pages order the two with a fence, here the partials cross XCDs
// with write-through atomic stores and loads instead, since a gfx950 fence
// flushes a whole L2.  Section "Fusion boundaries": per-sample weights scale
// each contribution before grouping and the optimizer runs as the epilogue).
//
// Programs.  Short runs with SL = 1 are owned, two at a time, by a subgroup of
// `lpr` lanes (one row of the bucket width); short runs with 2 <= SL < 32 by a
// subgroup each; short runs with 32 <= SL < 256 by a whole
// 256-thread workgroup whose subgroups split the lookups; chunks and long-run
// updates by a workgroup.  Every kernel is persistent over a task list whose
// length it reads from device memory (no host readback).
//
// Memory.  Per lookup the kernels read the bag id (and the contribution scale)
// of the sorted lookup with the sorted order, then one 16-byte column slice of
// the bag's grad_out row; eight lookups are kept in flight per lane.  A
// single-lookup task carries its bag, so an SL = 1 run costs one task load,
// then the grad_out row, weight row and momentum in parallel.
//
// Determinism.  Sums run in lookup order inside a subgroup; workgroup sums
// combine subgroups in ascending order; the square sum is reduced in a fixed
// tree.  A long run's gradient is the sum of its chunk partials, chunk k folded
// into subgroup (k mod nsg) in ascending k.  The two-launch update and the
// fused last-chunk update call the same workgroup routine, so the two give
// bit-identical weights.
#include "tbe_common.h"

namespace tbe {
namespace {

// Lookups in flight per lane in the gathers: 8, or 4 where the kernel's
// register use at 8 would cost occupancy that a short launch needs (the host
// picks; see the launchers).
constexpr int kInFlightDeep = 8, kInFlightShallow = 4;
constexpr int kTdCache = 128;  // table descriptors cached in LDS by the tiny-run kernel

// Accumulate sorted slots [i0, i1) with stride `step` into g (this lane's
// columns `cold`, already clamped into the row for idle lanes).  Eight lookups
// per batch: bag ids (and scales), then the eight grad_out slices, then the
// sums in lookup order; scheduling barriers keep the loads of a batch in
// flight together.  A partial batch repeats the last slot and drops the
// repeats with a select (no branches inside the batch).
template <int VEC, int NC, bool SCALE, int kInFlight>
__device__ __forceinline__ void gather_t(const BwdArgs& a, const TableDev& td, int64_t tB,
                                         uint32_t i0, uint32_t i1, uint32_t step,
                                         const uint32_t* cold, float (*g)[VEC]) {
  const float* gbase = a.grad + td.col;
  if (i0 >= i1) return;
  // software pipeline: bag ids of batch i+1 load while the rows of batch i are in flight
  uint32_t nbag[kInFlight];
  float nsc[kInFlight];
#pragma unroll
  for (int k = 0; k < kInFlight; ++k) {
    const uint32_t q0 = i0 + (uint32_t)k * step;
    const uint32_t q = q0 < i1 ? q0 : i1 - 1;
    nbag[k] = a.sorted_bag[q];
    nsc[k] = SCALE ? a.sorted_scale[q] : 1.0f;
  }
  for (uint32_t i = i0; i < i1; i += kInFlight * step) {
    int64_t b[kInFlight];
    float sc[kInFlight];
    bool ok[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      // a bag outside the table's B bags (never, for lists the preprocessing
      // wrote) reads row 0 and is dropped
      const int64_t bk = (int64_t)nbag[k] - tB;
      ok[k] = i + (uint32_t)k * step < i1 && (uint64_t)bk < (uint64_t)a.B;
      b[k] = ok[k] ? bk : 0;
      sc[k] = nsc[k];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float v[kInFlight][VEC];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
        load_f32<VEC>(gbase + b[k] * (int64_t)a.dtot + cold[c], v[k]);
      if (c == 0) {
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
          const uint32_t q0 = i + (uint32_t)(kInFlight + k) * step;
          const uint32_t q = q0 < i1 ? q0 : i1 - 1;
          nbag[k] = a.sorted_bag[q];
          nsc[k] = SCALE ? a.sorted_scale[q] : 1.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) g[c][e] += ok[k] ? sc[k] * v[k][e] : 0.0f;
    }
  }
}

template <int VEC, int NC, int IF>
__device__ __forceinline__ void gather(const BwdArgs& a, const TableDev& td, int64_t tB,
                                       uint32_t i0, uint32_t i1, uint32_t step,
                                       const uint32_t* cold, float (*g)[VEC]) {
  if (a.sorted_scale)
    gather_t<VEC, NC, true, IF>(a, td, tB, i0, i1, step, cold, g);
  else
    gather_t<VEC, NC, false, IF>(a, td, tB, i0, i1, step, cold, g);
}

// Sanity bounds of list entries (they hold for every list the preprocessing
// writes; a stale or foreign workspace is skipped instead of read out of bounds).
__device__ __forceinline__ bool span_ok(const BwdArgs& a, uint32_t start, uint32_t len,
                                        uint32_t t, uint32_t row) {
  return t < a.T && start <= a.N && len <= a.N - start && row < a.tables[t].rows;
}
__device__ __forceinline__ bool chunk_ok(const BwdArgs& a, uint4 task) {
  return task.z < a.T && task.x <= a.N && task.y <= a.N - task.x && task.y <= (uint32_t)kChunk &&
         task.w < a.max_long;
}
__device__ __forceinline__ bool long_ok(const BwdArgs& a, uint32_t l) {
  const uint4 t = a.long_task[l];
  if (!span_ok(a, t.x, t.y, t.w, t.z)) return false;
  const uint32_t nch = (t.y + kChunk - 1) / kChunk;
  const uint32_t cb = a.long_cbeg[l];
  return cb <= a.max_chunks && nch <= a.max_chunks - cb;
}

// A cross-workgroup wait of the preprocessing gave up, so its lists may be
// spoiled: every backward kernel then returns before it writes anything
// (weights, momentum, partials, debug counters all keep their contents).
__device__ __forceinline__ bool prep_failed(const BwdArgs& a) { return *a.prep_err != 0u; }

__device__ __forceinline__ uint32_t list_begin(const BwdArgs& a, int list, uint32_t bucket) {
  return a.counters[kCntBegins + list * (a.nb + 1) + bucket];
}

// Table descriptor: from the LDS copy when the plan has at most kTdCache
// tables (TDL), else from global memory.  A compile-time choice, so the
// compiler never emits a generic (flat) load that would wait on both counters.
template <bool TDL>
__device__ __forceinline__ void load_td_cache(const BwdArgs& a, TableDev* s_td) {
  if (TDL) {
    for (uint32_t i = threadIdx.x; i < a.T; i += kThreads) s_td[i] = a.tables[i];
    __syncthreads();
  }
}
template <bool TDL>
__device__ __forceinline__ TableDev get_td(const BwdArgs& a, const TableDev* s_td, uint32_t t) {
  return TDL ? s_td[t] : a.tables[t];
}

// The update of one row owned by a subgroup (g: this lane's columns; m0:
// the row's momentum, read by the caller for row-wise Adagrad only).
// Row-wise Adagrad: M += mean_d g^2, w -= lr g / (sqrt(M) + eps).  Element-
// wise Adagrad (HugeCTR walkthrough, step 5): A[row][d] += g[d]^2 per column,
// w -= lr g / (sqrt(A) + eps).  SGD: w -= lr g, no state.
template <int WD, int VEC, int NC, bool NT>
__device__ __forceinline__ void subgroup_row_update(const BwdArgs& a, const TableDev& td,
                                                    int64_t row, float m0, const float (*w)[VEC],
                                                    const float (*g)[VEC], const uint32_t* colc,
                                                    uint32_t lpr, uint32_t lane_in, bool store) {
  const uint32_t D = td.dim;
  if (a.opt != OPT_ROWWISE_ADAGRAD) {  // uniform
    if (!store) return;
    if (lane_in == 0 && a.debug_count)
      atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (colc[c] >= D) continue;
      float o[VEC];
      if (a.opt == OPT_ADAGRAD) {
        float acc[VEC];
        load_f32<VEC>(td.m + row * D + colc[c], acc);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          acc[e] += g[c][e] * g[c][e];
          o[e] = w[c][e] - (a.lr * g[c][e]) / (sqrtf(acc[e]) + a.eps);
        }
        store_f32<VEC>(td.m + row * D + colc[c], acc);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = w[c][e] - a.lr * g[c][e];
      }
      store_w<WD, VEC, NT>(td.w, row * D + colc[c], o);
    }
    return;
  }
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
    if (colc[c] < D)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sq += g[c][e] * g[c][e];
  sq = subgroup_sum(sq, lpr);
  if (!store) return;
  const float m = m0 + sq / (float)D;
  if (lane_in == 0) {
    gstore(td.m + row, m);
    if (a.debug_count) atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
  }
  const float den = sqrtf(m) + a.eps;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (colc[c] >= D) continue;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = w[c][e] - (a.lr * g[c][e]) / den;
    store_w<WD, VEC, NT>(td.w, row * D + colc[c], o);
  }
}

// ------------------------------------------------------- single-lookup runs
// Most runs have one lookup.  A subgroup takes P (1 or 2) of them per step:
// the task records (which carry the lookup's bag), then every weight row,
// momentum, grad_out slice and scale of the step is loaded before the first
// use -- one memory round trip per step after the task load.
template <int WD, int VEC, int NC, bool SCALE, bool TDL, bool NT, int P>
__device__ __forceinline__ void single_pair(const BwdArgs& a, const TableDev* s_td, uint4 tk0,
                                            uint4 tk1, bool two, uint32_t lpr,
                                            uint32_t lane_in) {
  static_assert(P == 1 || P == 2, "one or two runs per step");
  uint4 tk[2] = {tk0, tk1};  // {start, row, table, bag}
  TableDev td[P];
  bool ok[P];
  int64_t row[P], b[P];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    // sanity bounds, never false for lists the preprocessing wrote
    const uint32_t t = tk[u].z < a.T ? tk[u].z : 0u;
    td[u] = get_td<TDL>(a, s_td, t);
    const int64_t bb = (int64_t)tk[u].w - (int64_t)t * a.B;
    ok[u] = tk[u].z < a.T && tk[u].x < a.N && tk[u].y < td[u].rows && bb >= 0 && bb < a.B;
    row[u] = ok[u] ? (int64_t)tk[u].y : 0;
    b[u] = ok[u] ? bb : 0;
  }
  uint32_t colc[P][NC], cold[P][NC];
  float w[P][NC][VEC], g[P][NC][VEC], m0[P], sc[P];
  RawW<WD, VEC> wr[P][NC];  // converted after the barrier
#pragma unroll
  for (int u = 0; u < P; ++u) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      colc[u][c] = (lane_in + (uint32_t)c * lpr) * VEC;
      cold[u][c] = colc[u][c] < td[u].dim ? colc[u][c] : 0u;
      load_w_raw<WD, VEC, NT>(td[u].w, row[u] * td[u].dim + cold[u][c], wr[u][c]);
      load_f32<VEC>(a.grad + b[u] * (int64_t)a.dtot + td[u].col + cold[u][c], g[u][c]);
    }
    m0[u] = a.opt == OPT_ROWWISE_ADAGRAD ? gload(td[u].m + row[u]) : 0.f;
    sc[u] = SCALE ? a.sorted_scale[ok[u] ? tk[u].x : 0u] : 1.0f;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < P; ++u)
#pragma unroll
    for (int c = 0; c < NC; ++c) cvt_w<WD, VEC>(wr[u][c], w[u][c]);
#pragma unroll
  for (int u = 0; u < P; ++u) {
    if (SCALE)
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) g[u][c][e] *= sc[u];
    subgroup_row_update<WD, VEC, NC, NT>(a, td[u], row[u], m0[u], w[u], g[u], colc[u], lpr, lane_in,
                                     ok[u] && (u == 0 || two));
  }
}

// In list order: subgroup sg of the launch takes positions sg, sg + nsg, ...
// With streamed rows the next task record loads while the current run's rows
// are in flight, and the one-chunk rows' registers are held to eight waves
// per SIMD (two spill): C5 2994 -> 2874 us per launch; the prefetch at the
// seven waves its registers would otherwise allow, 3032 us.  Wider rows keep
// their registers (held to eight waves they spill 20 to 33).
template <int WD, int VEC, int NC, bool SCALE, bool TDL, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT && NC == 1 ? 8 : 1)))
void bwd_single_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ TableDev s_td[TDL ? kTdCache : 1];
  load_td_cache<TDL>(a, s_td);
  const uint32_t lpr = bk.lpr;
  const uint32_t lane_in = threadIdx.x & (lpr - 1);
  const uint32_t nsg_grid = (lg * kThreads) >> bk.lpr_log2;
  const uint32_t sg = (lb * kThreads + threadIdx.x) >> bk.lpr_log2;
  const uint32_t beg = list_begin(a, 0, bucket);
  const uint32_t end = min(list_begin(a, 0, bucket + 1), a.max_single);
  if constexpr (NT) {
    // Batches whose rows are streamed past the caches: one run per step,
    // measured faster than pairs there (8.4M lookups: 283 -> 249 us; 134M
    // lookups: 3117 -> 2917 us).
    uint32_t s = beg + sg;
    uint4 next = s < end ? a.single_task[s] : make_uint4(0, 0, 0, 0);
    for (; s < end; s += nsg_grid) {
      const uint4 tk = next;
      if (s + nsg_grid < end) next = a.single_task[s + nsg_grid];
      single_pair<WD, VEC, NC, SCALE, TDL, NT, 1>(a, s_td, tk, tk, false, lpr, lane_in);
    }
    return;
  }
  for (uint32_t s = beg + sg; s < end; s += 2 * nsg_grid) {
    const uint32_t s1 = (s + nsg_grid < end) ? s + nsg_grid : s;
    single_pair<WD, VEC, NC, SCALE, TDL, NT, 2>(a, s_td, a.single_task[s], a.single_task[s1],
                                                s1 != s, lpr, lane_in);
  }
}

// ----------------------------------------------------- tiny short runs
// One subgroup of lpr lanes owns a run with 2 <= SL < 32: gather, Adagrad,
// plain stores.  The next task record is prefetched.
template <int WD, int VEC, int NC, bool TDL, int IF, bool NT>
__global__ __launch_bounds__(kThreads) void bwd_tiny_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ TableDev s_td[TDL ? kTdCache : 1];
  load_td_cache<TDL>(a, s_td);
  const uint32_t lpr = bk.lpr;
  const uint32_t lane_in = threadIdx.x & (lpr - 1);
  const uint32_t nsg_grid = (lg * kThreads) >> bk.lpr_log2;
  const uint32_t sg = (lb * kThreads + threadIdx.x) >> bk.lpr_log2;
  const uint32_t beg = list_begin(a, 1, bucket);
  const uint32_t end = min(list_begin(a, 1, bucket + 1), a.max_tiny);
  uint32_t s = beg + sg;
  uint4 next = s < end ? a.tiny_task[s] : make_uint4(0, 0, 0, 0);
  for (; s < end; s += nsg_grid) {
    const uint4 task = next;  // {start, len, row, table}
    if (s + nsg_grid < end) next = a.tiny_task[s + nsg_grid];
    const uint32_t start = task.x, len = task.y, t = task.w;
    // sanity bounds, never false for lists the preprocessing wrote
    if (len == 0 || t >= a.T || start > a.N || len > a.N - start) continue;
    const TableDev td = get_td<TDL>(a, s_td, t);
    if (task.z >= td.rows) continue;
    const int64_t row = task.z;
    uint32_t colc[NC], cold[NC];
    float w[NC][VEC], g[NC][VEC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
      cold[c] = colc[c] < td.dim ? colc[c] : 0u;
      load_w<WD, VEC, NT>(td.w, row * td.dim + cold[c], w[c]);
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[c][e] = 0.f;
    }
    const float m0 = a.opt == OPT_ROWWISE_ADAGRAD ? gload(td.m + row) : 0.f;
    gather<VEC, NC, IF>(a, td, (int64_t)t * a.B, start, start + len, 1u, cold, g);
    subgroup_row_update<WD, VEC, NC, NT>(a, td, row, m0, w, g, colc, lpr, lane_in, true);
  }
}

// ------------------------------------------------------ workgroup routines

template <int VEC, int NC>
struct WgSmem {
  float red[kThreads * VEC * NC];   // [nsg][bucket width] per-subgroup sums
  float gsum[kThreads * VEC * NC];  // the row gradient
  float wsq[kThreads / kWave];
  uint32_t last;
};

// Subgroup sg accumulates sorted slots i0+sg, i0+sg+nsg, ... < i1 into sm.red.
template <int VEC, int NC, int IF>
__device__ __forceinline__ void wg_gather(const BwdArgs& a, const BucketDev& bk,
                                          const TableDev& td, uint32_t t, uint32_t i0,
                                          uint32_t i1, WgSmem<VEC, NC>& sm) {
  const uint32_t lpr = bk.lpr, lane_in = threadIdx.x & (lpr - 1);
  const uint32_t sg = threadIdx.x >> bk.lpr_log2, nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = lpr * VEC * NC;
  const uint32_t D = td.dim;
  uint32_t colc[NC], cold[NC];
  float g[NC][VEC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
    cold[c] = colc[c] < D ? colc[c] : 0u;
#pragma unroll
    for (int e = 0; e < VEC; ++e) g[c][e] = 0.f;
  }
  gather<VEC, NC, IF>(a, td, (int64_t)t * a.B, i0 + sg, i1, nsg, cold, g);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.red[sg * width + colc[c] + e] = g[c][e];
  __syncthreads();
}

// Column sums of sm.red in ascending subgroup order into sm.gsum; returns this
// thread's share of sum_d g[d]^2.
template <int VEC, int NC>
__device__ __forceinline__ float red_to_gsum(const BucketDev& bk, uint32_t D,
                                             WgSmem<VEC, NC>& sm) {
  const uint32_t nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = bk.lpr * VEC * NC;
  float sqp = 0.f;
  for (uint32_t col = threadIdx.x; col < D; col += kThreads) {
    float s = 0.f;
    for (uint32_t k = 0; k < nsg; ++k) s += sm.red[k * width + col];
    sm.gsum[col] = s;
    sqp += s * s;
  }
  return sqp;
}

// The row's weights (this thread's columns threadIdx.x * VEC ..) and
// row-wise momentum, loaded by the workgroup before the gradient is ready, so
// that the update does not wait for them.  Rows are at most kThreads * VEC
// wide (bucket widths up to 1024 with VEC >= 4), so one chunk per thread.
template <int VEC>
struct RowPre {
  float w[VEC];
  float m;
};
template <int WD, int VEC, bool NT>
__device__ __forceinline__ void row_prefetch(const BwdArgs& a, const TableDev& td, int64_t row,
                                             RowPre<VEC>& p) {
  const uint32_t col = threadIdx.x * VEC;
  if (col < td.dim) load_w<WD, VEC, NT>(td.w, row * td.dim + col, p.w);
  p.m = a.opt == OPT_ROWWISE_ADAGRAD ? gload(td.m + row) : 0.f;
}

// The update of one row from sm.gsum, all threads of the workgroup (the
// optimizers of subgroup_row_update).  PRE: the row's weights and momentum
// come from row_prefetch; else they are loaded here.
template <int WD, int VEC, int NC, bool PRE, bool NT>
__device__ __forceinline__ void wg_row_update(const BwdArgs& a, const TableDev& td, int64_t row,
                                              float sqp, WgSmem<VEC, NC>& sm,
                                              const RowPre<VEC>& pre) {
  const uint32_t D = td.dim;
  if (a.opt != OPT_ROWWISE_ADAGRAD) {  // uniform
    __syncthreads();  // sm.gsum, written by every wave, is complete
    for (uint32_t col = threadIdx.x * VEC; col < D; col += kThreads * VEC) {
      float w[VEC], o[VEC];
      if (PRE && col == threadIdx.x * VEC) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) w[e] = pre.w[e];
      } else {
        load_w<WD, VEC, NT>(td.w, row * D + col, w);
      }
      if (a.opt == OPT_ADAGRAD) {
        float acc[VEC];
        load_f32<VEC>(td.m + row * D + col, acc);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float gv = sm.gsum[col + e];
          acc[e] += gv * gv;
          o[e] = w[e] - (a.lr * gv) / (sqrtf(acc[e]) + a.eps);
        }
        store_f32<VEC>(td.m + row * D + col, acc);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = w[e] - a.lr * sm.gsum[col + e];
      }
      store_w<WD, VEC, NT>(td.w, row * D + col, o);
    }
    __syncthreads();  // every thread has read sm before it changes
    if (threadIdx.x == 0 && a.debug_count)
      atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
    return;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) sqp += __shfl_xor(sqp, o, kWave);
  if (lane_id() == 0) sm.wsq[threadIdx.x / kWave] = sqp;
  __syncthreads();
  const float sq = ((sm.wsq[0] + sm.wsq[1]) + sm.wsq[2]) + sm.wsq[3];
  const float m = (PRE ? pre.m : gload(td.m + row)) + sq / (float)D;
  const float den = sqrtf(m) + a.eps;
  for (uint32_t col = threadIdx.x * VEC; col < D; col += kThreads * VEC) {
    float w[VEC], o[VEC];
    if (PRE && col == threadIdx.x * VEC) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) w[e] = pre.w[e];
    } else {
      load_w<WD, VEC, NT>(td.w, row * D + col, w);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = w[e] - (a.lr * sm.gsum[col + e]) / den;
    store_w<WD, VEC, NT>(td.w, row * D + col, o);
  }
  __syncthreads();  // every thread has read td.m[row] and sm before they change
  if (threadIdx.x == 0) {
    gstore(td.m + row, m);
    if (a.debug_count) atomicAdd(&a.debug_count[td.key_base + (uint32_t)row], 1u);
  }
}

// Long-run update: reduce the run's chunk partials, then row-wise Adagrad.
// COH: the partials were written by workgroups of other XCDs during this
// kernel, so they are read with agent-scope atomic loads, which bypass this
// XCD's L2 (the two-launch update reads them after a kernel boundary).
template <int WD, int VEC, int NC, bool COH, bool NT>
__device__ __forceinline__ void long_update(const BwdArgs& a, const BucketDev& bk, uint32_t l,
                                            WgSmem<VEC, NC>& sm) {
  const uint32_t lpr = bk.lpr, lane_in = threadIdx.x & (lpr - 1);
  const uint32_t sg = threadIdx.x >> bk.lpr_log2, nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = lpr * VEC * NC;
  const uint4 task = a.long_task[l];  // {start, len, row, table}
  const uint32_t cb = a.long_cbeg[l];
  const uint32_t nch = (task.y + kChunk - 1) / kChunk;
  const TableDev td = a.tables[task.w];
  const uint32_t D = td.dim;
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
      if (COH) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          v[e] = __hip_atomic_load(src + colc[c] + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        load_f32<VEC>(src + colc[c], v);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) g[c][e] += v[e];
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < VEC; ++e) sm.red[sg * width + colc[c] + e] = g[c][e];
  __syncthreads();
  const float sqp = red_to_gsum<VEC, NC>(bk, D, sm);
  // the row is loaded by the update itself: loaded before the partials, it
  // cost the kernel a wave per SIMD (C5 150 -> 169 us)
  RowPre<VEC> unused;
  wg_row_update<WD, VEC, NC, false, NT>(a, td, (int64_t)task.z, sqp, sm, unused);
}

// Write the combined chunk partial (ascending subgroup order) to partial[c];
// COH: with agent-scope atomic stores, which write through this XCD's L2.
template <int VEC, int NC, bool COH>
__device__ __forceinline__ void chunk_store(const BwdArgs& a, const BucketDev& bk, uint32_t D,
                                            uint32_t c, WgSmem<VEC, NC>& sm) {
  const uint32_t nsg = kThreads >> bk.lpr_log2;
  const uint32_t width = bk.lpr * VEC * NC;
  float* dst = a.partial + (size_t)c * a.pstride;
  for (uint32_t col = threadIdx.x; col < D; col += kThreads) {
    float s = 0.f;
    for (uint32_t k = 0; k < nsg; ++k) s += sm.red[k * width + col];
    if (COH)
      __hip_atomic_store(dst + col, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      dst[col] = s;
  }
}

// ------------------------------------------------------- medium short runs
// One workgroup owns a run with 32 <= SL < 256: its subgroups split the
// lookups, the workgroup combines them in LDS and updates the row.
// Five waves per SIMD: the compiler's own choice for 16-bit rows is 99 VGPRs,
// four waves; at five, f16 rows fit without spills (bf16 spills two).
template <int WD, int VEC, int NC, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NC == 1 ? 5 : 1)))
void bwd_medium_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ WgSmem<VEC, NC> sm;
  const uint32_t beg = list_begin(a, 2, bucket);
  const uint32_t end = min(list_begin(a, 2, bucket + 1), a.max_med);
  for (uint32_t m = beg + lb; m < end; m += lg) {
    const uint4 task = a.med_task[m];  // {start, len, row, table}
    if (!span_ok(a, task.x, task.y, task.w, task.z)) continue;  // uniform; never for valid lists
    const TableDev td = a.tables[task.w];
    RowPre<VEC> pre;
    row_prefetch<WD, VEC, NT>(a, td, (int64_t)task.z, pre);
    wg_gather<VEC, NC, kInFlightShallow>(a, bk, td, task.w, task.x, task.x + task.y, sm);
    const float sqp = red_to_gsum<VEC, NC>(bk, td.dim, sm);
    wg_row_update<WD, VEC, NC, true, NT>(a, td, (int64_t)task.z, sqp, sm, pre);
  }
}

// ---------------------------------------------------------------- long runs

// Chunk positions this workgroup takes.  Workgroups are dispatched to the
// eight XCDs round-robin (workgroup i on XCD i mod 8) and each XCD has its own
// L2.  The chunk list places the chunks of a long run so that position c
// reads grad_out rows of about the (c mod 8)-th eighth of the table's bags
// (see the classification), so the workgroups of XCD x take the positions
// c = x (mod 8) and each XCD's L2 holds one eighth of the grad_out columns
// of the table whose long runs are passing through.  The bucket's workgroups
// come in groups of eight starting at a multiple of eight, so lb mod 8 is the
// workgroup's XCD and lb / 8 its rank among the bucket's workgroups there.
__device__ __forceinline__ void chunk_walk(uint32_t lb, uint32_t lg, uint32_t beg, uint32_t& c,
                                           uint32_t& step) {
  if (lg & 7u) {  // not launched in groups of eight: plain striding
    c = beg + lb;
    step = lg;
    return;
  }
  const uint32_t xcd = lb & 7u, rank = lb >> 3, nx = lg >> 3;
  c = beg + ((xcd - beg) & 7u) + 8u * rank;
  step = 8u * nx;
}

// Chunk order.  The chunks of one table on one XCD read that XCD's eighth of
// the table's grad_out rows.  Walked in list order (run after run) the
// workgroups of an XCD sweep the whole eighth at once, more than its L2 holds;
// ordered by the bag of their first lookup they sweep it front to back, and
// the rows in reach at a time are few.  One workgroup per (table, residue mod
// 8) counting-sorts that class's positions by kChunkBins bins of the first
// bag and writes the permutation chunk_perm (positions of one bin in any
// order: the order changes no result, since a chunk's partial goes to its own
// slot and is summed in chunk order).  Chunk lists are in ascending table
// order inside a bucket, so the table's positions are found by binary search.
constexpr uint32_t kChunkBins = 256;

__global__ __launch_bounds__(kThreads) void chunk_order_kernel(BwdArgs a) {
  if (prep_failed(a)) return;
  __shared__ uint32_t hist[kChunkBins];
  __shared__ uint32_t sh4[4];
  const uint32_t t = blockIdx.x >> 3, x = blockIdx.x & 7u;
  if (t >= a.T) return;
  const uint32_t bucket = a.tables[t].bucket;
  const uint32_t bb = list_begin(a, 4, bucket);
  const uint32_t be = min(list_begin(a, 4, bucket + 1), a.max_chunks);
  auto lower = [&](uint32_t v) {  // first position in [bb, be) whose table is >= v
    uint32_t lo = bb, hi = be;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (a.chunk_task[mid].z < v) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  const uint32_t cs = lower(t), ce = lower(t + 1);
  const uint32_t first = cs + ((x - cs) & 7u);  // first position of residue x
  if (first >= ce) return;
  const uint32_t n = (ce - first + 7u) / 8u;
  const int64_t tB = (int64_t)t * a.B;
  auto bin_of = [&](uint32_t c) {
    const uint32_t st = a.chunk_task[c].x;
    const int64_t j = (st < a.N ? (int64_t)a.sorted_bag[st] : tB) - tB;
    const uint64_t b = (uint64_t)(j < 0 ? 0 : j) * kChunkBins / (uint64_t)(a.B > 0 ? a.B : 1);
    return (uint32_t)(b < kChunkBins ? b : kChunkBins - 1);
  };
  hist[threadIdx.x] = 0u;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) atomicAdd(&hist[bin_of(first + 8u * i)], 1u);
  __syncthreads();
  {  // exclusive scan of the bins (one per thread)
    const uint32_t v = hist[threadIdx.x];
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o, kWave);
      if (lane_id() >= (uint32_t)o) incl += y;
    }
    if (lane_id() == kWave - 1) sh4[threadIdx.x / kWave] = incl;
    __syncthreads();
    uint32_t wbase = 0;
    for (uint32_t w = 0; w < threadIdx.x / kWave; ++w) wbase += sh4[w];
    hist[threadIdx.x] = wbase + incl - v;
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += kThreads) {
    const uint32_t c = first + 8u * i;
    const uint32_t r = atomicAdd(&hist[bin_of(c)], 1u);
    a.chunk_perm[first + 8u * r] = c;
  }
}

// The chunks at the next kThreads positions of a workgroup's walk (c0,
// c0 + cstep, ...; one per thread) that the workgroup updates, listed in walk
// order in LDS: positions past the list, the chunks of the contraction's hot
// rows and malformed entries (never, for lists the preprocessing wrote) are
// dropped.  Tested one at a time, each skipped chunk cost the workgroup its
// own chain of three dependent loads, and at C5 most chunks belong to hot
// rows.  Returns how many were listed; ends with a barrier.
struct ChunkBatch {
  uint32_t cp[kThreads];
  uint4 task[kThreads];
  uint32_t wcnt[kThreads / kWave];
};

template <bool FUSED>
__device__ __forceinline__ uint32_t chunk_batch(const BwdArgs& a, uint64_t c0, uint32_t cstep,
                                                uint32_t beg, uint32_t end, ChunkBatch& cb) {
  const uint64_t cw = c0 + (uint64_t)threadIdx.x * cstep;
  bool take = false;
  uint32_t cp = 0;
  uint4 task = make_uint4(0, 0, 0, 0);
  if (cw < end) {
    cp = a.chunk_perm ? a.chunk_perm[cw] : (uint32_t)cw;  // position of the chunk taken
    if (cp >= beg && cp < end) {
      task = a.chunk_task[cp];  // {start, len, table, long index}
      take = chunk_ok(a, task) && (!FUSED || long_ok(a, task.w)) &&
             !(a.long_flag && a.long_flag[task.w]);  // a hot row: the contraction's
    }
  }
  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  const uint64_t m = __ballot(take);
  if (lane == 0) cb.wcnt[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t base = 0, n = 0;
#pragma unroll
  for (uint32_t w = 0; w < kThreads / kWave; ++w) {
    const uint32_t x = cb.wcnt[w];
    base += w < wave ? x : 0u;
    n += x;
  }
  if (take) {
    const uint32_t i = base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    cb.cp[i] = cp;
    cb.task[i] = task;
  }
  __syncthreads();
  return n;
}

template <int WD, int VEC, int NC, int IF>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ WgSmem<VEC, NC> sm;
  __shared__ ChunkBatch cb;
  const uint32_t beg = list_begin(a, 4, bucket);
  const uint32_t end = min(list_begin(a, 4, bucket + 1), a.max_chunks);
  uint32_t c, cstep;
  chunk_walk(lb, lg, beg, c, cstep);
  for (uint64_t c0 = c; c0 < end; c0 += (uint64_t)kThreads * cstep) {
    const uint32_t n = chunk_batch<false>(a, c0, cstep, beg, end, cb);
    for (uint32_t i = 0; i < n; ++i) {
      const uint32_t cp = cb.cp[i];
      const uint4 task = cb.task[i];
      const TableDev td = a.tables[task.z];
      wg_gather<VEC, NC, IF>(a, bk, td, task.z, task.x, task.x + task.y, sm);
      chunk_store<VEC, NC, false>(a, bk, td.dim, cp, sm);
      __syncthreads();
    }
  }
}

template <int WD, int VEC, int NC, bool NT>
__global__ __launch_bounds__(kThreads) void bwd_long_update_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ WgSmem<VEC, NC> sm;
  const uint32_t beg = list_begin(a, 3, bucket);
  const uint32_t end = min(list_begin(a, 3, bucket + 1), a.max_long);
  for (uint32_t l = beg + lb; l < end; l += lg) {
    if (!long_ok(a, l)) continue;  // uniform per workgroup; never for valid lists
    if (a.long_flag && a.long_flag[l]) continue;  // a hot row: the contraction's
    long_update<WD, VEC, NC, false, NT>(a, bk, l, sm);
  }
}

// Fused: each chunk publishes its partial, then counts down the run's
// remaining chunks; the workgroup that takes the count to zero performs the
// update, then re-arms the countdown.  Each XCD has its own L2, which is not
// coherent with the others, and an agent-scope fence on gfx950 writes back and
// invalidates the whole L2 -- per chunk, that made this path 20-25x slower than
// the two-launch one.  So the partial is written with agent-scope atomic
// stores (write-through to the device-coherent level), every thread waits for
// its stores to complete (s_waitcnt 0), the workgroup meets at a barrier, and
// only then is the countdown decremented (an agent-scope atomic, performed at
// the coherent level); the last workgroup reads the partials with agent-scope
// atomic loads (read from the coherent level, not from a stale cache).  This
// is the release/acquire pair without the whole-cache operations, which only
// serve to publish ordinary cached stores; none is published here.
template <int WD, int VEC, int NC, int IF, bool NT>
__global__ __launch_bounds__(kThreads) void bwd_chunk_fused_kernel(BwdArgs a, BucketSet S) {
  if (prep_failed(a)) return;
  BucketDev bk;
  uint32_t bucket, lb, lg;
  set_pick(S, bk, bucket, lb, lg);
  __shared__ WgSmem<VEC, NC> sm;
  __shared__ ChunkBatch cb;
  const uint32_t beg = list_begin(a, 4, bucket);
  const uint32_t end = min(list_begin(a, 4, bucket + 1), a.max_chunks);
  uint32_t c, cstep;
  chunk_walk(lb, lg, beg, c, cstep);
  for (uint64_t c0 = c; c0 < end; c0 += (uint64_t)kThreads * cstep) {
    const uint32_t nb = chunk_batch<true>(a, c0, cstep, beg, end, cb);
    for (uint32_t bi = 0; bi < nb; ++bi) {
      const uint32_t cp = cb.cp[bi];
      const uint4 task = cb.task[bi];
      const TableDev td = a.tables[task.z];
      wg_gather<VEC, NC, IF>(a, bk, td, task.z, task.x, task.x + task.y, sm);
      chunk_store<VEC, NC, true>(a, bk, td.dim, cp, sm);
      __builtin_amdgcn_s_waitcnt(0);  // this thread's write-through stores have completed
      __syncthreads();
      if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&a.remaining[task.w], 0xffffffffu,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = (old == 1u) ? 1u : 0u;
      }
      __syncthreads();
      if (sm.last) {
        long_update<WD, VEC, NC, true, NT>(a, bk, task.w, sm);
        if (threadIdx.x == 0) {
          const uint32_t len = a.long_task[task.w].y;
          __hip_atomic_store(&a.remaining[task.w], (len + kChunk - 1) / kChunk, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __syncthreads();
    }
  }
}

// Hot rows of the contraction (bwd_dense.hip): one workgroup per (table,
// hot row slot); the row gradient is the sum of the contraction's dense_w
// partials in a fixed order (eight interleaved accumulators over workgroup
// order, combined in a fixed tree), then the optimizer of every row update.
template <int WD>
__global__ __launch_bounds__(kThreads) void dense_update_kernel(BwdArgs a) {
  if (prep_failed(a)) return;
  constexpr int VEC = 4;
  __shared__ WgSmem<VEC, 1> sm;
  const uint32_t t = blockIdx.x / kDenseRows, k = blockIdx.x % kDenseRows;
  if (k >= min(a.dense_cnt[t], (uint32_t)kDenseRows)) return;
  const uint4 task = a.dense_rows[(size_t)t * kDenseRows + k];  // {start, len, row, long index}
  const TableDev td = a.tables[t];
  if (task.z >= td.rows) return;  // never, for rows the selection wrote
  const uint32_t D = td.dim;
  const float* part = a.dense_part + ((size_t)t * kDenseRows + k) * a.dense_w * kDensePitch;
  float sqp = 0.f;
  for (uint32_t col = threadIdx.x; col < D; col += kThreads) {
    // the dense_w partials: eight interleaved accumulators (eight loads in
    // flight), combined in a fixed tree
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint32_t w = 0;
    for (; w + 8u <= a.dense_w; w += 8u) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(size_t)(w + (uint32_t)u) * kDensePitch + col];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[u];
    }
    for (; w < a.dense_w; ++w) acc[0] += part[(size_t)w * kDensePitch + col];
    const float g = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    sm.gsum[col] = g;
    sqp += g * g;
  }
  RowPre<VEC> unused;
  wg_row_update<WD, VEC, 1, false, false>(a, td, (int64_t)task.z, sqp, sm, unused);
}

// Co-resident workgroups of a kernel on the whole device (queried once per
// instantiation).  A persistent grid larger than this would leave its last
// workgroups waiting for earlier ones to retire, a tail.
template <typename K>
uint32_t resident(K kernel, int num_cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  return (uint32_t)per_cu * (uint32_t)num_cus;
}

// Fill S.gbeg: bucket k gets min(need_k, cap / n) workgroups (at least 1);
// with mult = 8 every bucket's count is a multiple of eight (at least eight),
// so each bucket's range starts on an XCD boundary of the round-robin dispatch.
uint32_t set_grid(BucketSet& S, const BwdGrids* g, uint32_t BwdGrids::*field, uint32_t cap,
                  uint32_t mult = 1) {
  uint32_t share = cap / S.n > 0 ? cap / S.n : 1u;
  share = share / mult * mult > 0 ? share / mult * mult : mult;
  S.gbeg[0] = 0;
  for (uint32_t k = 0; k < S.n; ++k) {
    uint32_t need = g[k].*field > 0 ? g[k].*field : 1u;
    need = (need + mult - 1) / mult * mult;
    S.gbeg[k + 1] = S.gbeg[k] + (need < share ? need : share);
  }
  for (uint32_t k = S.n + 1; k <= (uint32_t)kMaxBuckets; ++k) S.gbeg[k] = S.gbeg[S.n];
  return S.gbeg[S.n];
}

// Lookups in flight of the tiny-run and chunk gathers.  Four lift the
// occupancy of both kernels (tiny 136 -> 92 VGPRs, chunk 116 -> 69) and pay
// while the launches are short and latency-bound; on a deep batch the kernels
// already keep the memory system busy and eight cut the round trips per run.
// Measured on MI355X (tiny / chunk, us per step, 8 -> 4 in flight): 2.1 M
// lookups 40.0 -> 34.6 / 21.5 -> 18.4; 17 M lookups 292 -> 233 / 578 -> 463;
// 138 M lookups 2408 -> 2545 / 3685 -> 3848.  Medium runs gather with four
// always (at the same three sizes: 24.8 -> 20.5, 179 -> 146, 1449 -> 1189).
// The split is at kBwdDeepLookups (tbe_common.h).

// Single-lookup runs of a deep batch: the persistent grid at half the
// resident workgroups.  The workgroups sweep the row-sorted list together, so
// the grid size sets how wide a window of weight rows is read and rewritten at
// once; on 64 tables of 5 M rows a window half as wide is faster (MI355X,
// us per launch at 1 / 0.83 / 0.67 / 0.5 / 0.33 / 0.25 of the resident grid:
// 3588 / 3613 / 3212 / 3054 / 3376 / 4236 over two runs), while the short
// launches need every workgroup (2.1 M lookups: 50.4 at 1, 61.2 at 0.5;
// 17 M: 286 at 1, 431 at 0.5).  The other run classes lose with any cap.
constexpr uint32_t kSingleDeepGridDiv = 2;

template <int WD, int VEC, int NC, bool TDL, int IF, bool NT>
void launch_small(const BwdArgs& a, BucketSet S, const BwdGrids* g, int cus, hipStream_t s) {
  const uint32_t div = IF == kInFlightDeep ? kSingleDeepGridDiv : 1u;
  if (a.sorted_scale) {
    static const uint32_t cap = resident(bwd_single_kernel<WD, VEC, NC, true, TDL, NT>, cus);
    const uint32_t grid = set_grid(S, g, &BwdGrids::single, cap / div);
    TBE_LAUNCH("bwd_single", (bwd_single_kernel<WD, VEC, NC, true, TDL, NT>), dim3(grid),
               dim3(kThreads), s, a, S);
  } else {
    static const uint32_t cap = resident(bwd_single_kernel<WD, VEC, NC, false, TDL, NT>, cus);
    const uint32_t grid = set_grid(S, g, &BwdGrids::single, cap / div);
    TBE_LAUNCH("bwd_single", (bwd_single_kernel<WD, VEC, NC, false, TDL, NT>), dim3(grid),
               dim3(kThreads), s, a, S);
  }
  static const uint32_t cap_t = resident(bwd_tiny_kernel<WD, VEC, NC, TDL, IF, NT>, cus);
  const uint32_t grid = set_grid(S, g, &BwdGrids::tiny, cap_t);
  TBE_LAUNCH("bwd_tiny", (bwd_tiny_kernel<WD, VEC, NC, TDL, IF, NT>), dim3(grid), dim3(kThreads),
             s, a, S);
}

template <int WD, int VEC, int NC, int IF, bool NT>
void launch_long(const BwdArgs& a, BucketSet S, const BwdGrids* g, bool fused, int cus,
                 hipStream_t s) {
  uint32_t grid;
  if (fused) {
    static const uint32_t cap_f = resident(bwd_chunk_fused_kernel<WD, VEC, NC, IF, NT>, cus);
    grid = set_grid(S, g, &BwdGrids::chunk, cap_f, 8);
    TBE_LAUNCH("bwd_chunk_fused", (bwd_chunk_fused_kernel<WD, VEC, NC, IF, NT>), dim3(grid),
               dim3(kThreads), s, a, S);
  } else {
    static const uint32_t cap_c = resident(bwd_chunk_kernel<WD, VEC, NC, IF>, cus);
    grid = set_grid(S, g, &BwdGrids::chunk, cap_c, 8);
    TBE_LAUNCH("bwd_chunk", (bwd_chunk_kernel<WD, VEC, NC, IF>), dim3(grid), dim3(kThreads), s,
               a, S);
    static const uint32_t cap_l = resident(bwd_long_update_kernel<WD, VEC, NC, NT>, cus);
    grid = set_grid(S, g, &BwdGrids::longrun, cap_l);
    TBE_LAUNCH("bwd_long_update", (bwd_long_update_kernel<WD, VEC, NC, NT>), dim3(grid),
               dim3(kThreads), s, a, S);
  }
}

template <int WD, int VEC, int NC, int IF, bool NT>
void launch_classes(const BwdArgs& a, BucketSet S, const BwdGrids* g, bool fused, int cus,
                    const hipStream_t* ss) {
  if (a.T <= (uint32_t)kTdCache)
    launch_small<WD, VEC, NC, true, IF, NT>(a, S, g, cus, ss[0]);
  else
    launch_small<WD, VEC, NC, false, IF, NT>(a, S, g, cus, ss[0]);
  static const uint32_t cap_m = resident(bwd_medium_kernel<WD, VEC, NC, NT>, cus);
  const uint32_t grid = set_grid(S, g, &BwdGrids::medium, cap_m);
  TBE_LAUNCH("bwd_medium", (bwd_medium_kernel<WD, VEC, NC, NT>), dim3(grid), dim3(kThreads),
             ss[1], a, S);
  launch_long<WD, VEC, NC, IF, NT>(a, S, g, fused, cus, ss[2]);
}

// Weight rows of the backward read and rewritten with non-temporal accesses
// from kBwdStreamRowsLookups lookups on (tbe_common.h): each touched row is read and written once per
// step, and as ordinary accesses those lines push the grad_out rows that the
// gathers reuse out of the caches.  Measured on MI355X (ms per step, plain /
// non-temporal): 138 M lookups 17.01 / 16.52 (single-lookup runs 3288 ->
// 2842 us), 17 M 2.204 / 2.176, and, with cold caches before each step,
// 2.1 M 0.364 / 0.351 (warm steps back to back, where the next forward
// re-reads the hot rows the backward wrote, had measured 0.338 / 0.339 on
// earlier kernels).

template <int WD, int VEC, int NC>
hipError_t launch(const BwdArgs& a, BucketSet S, const BwdGrids* g, bool fused, int cus,
                  const hipStream_t* ss) {
  static_assert(kBwdDeepLookups >= kBwdStreamRowsLookups, "deep batches stream their rows");
  // (test knobs can move both thresholds; the deep variant always streams)
  if ((int64_t)a.N >= knob_bwd_deep_lookups())
    launch_classes<WD, VEC, NC, kInFlightDeep, true>(a, S, g, fused, cus, ss);
  else if ((int64_t)a.N >= knob_bwd_stream_lookups())
    launch_classes<WD, VEC, NC, kInFlightShallow, true>(a, S, g, fused, cus, ss);
  else
    launch_classes<WD, VEC, NC, kInFlightShallow, false>(a, S, g, fused, cus, ss);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_update(const BwdArgs& a, int wd, hipStream_t s) {
  const dim3 grid(a.T * (uint32_t)kDenseRows), block(kThreads);
  if (wd == WD_F32)
    TBE_LAUNCH("dense_update", dense_update_kernel<WD_F32>, grid, block, s, a);
  else if (wd == WD_F16)
    TBE_LAUNCH("dense_update", dense_update_kernel<WD_F16>, grid, block, s, a);
  else
    TBE_LAUNCH("dense_update", dense_update_kernel<WD_BF16>, grid, block, s, a);
  return hipGetLastError();
}

hipError_t launch_chunk_order(const BwdArgs& a, hipStream_t s) {
  if (a.T == 0 || !a.chunk_perm) return hipSuccess;
  TBE_LAUNCH("chunk_order", chunk_order_kernel, dim3(a.T * 8u), dim3(kThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_backward_set(const BwdArgs& a, BucketSet S, const BwdGrids* g, int wd, int vec,
                               int nc, bool fused, int num_cus, const hipStream_t* s) {
#define TBE_BWD_CASE(W, V, N) \
  if (wd == W && vec == V && nc == N) return launch<W, V, N>(a, S, g, fused, num_cus, s);
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
