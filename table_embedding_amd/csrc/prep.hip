// Backward preprocessing on the device (FBTriton TBE page, "Backward":
// transposition, sorting and run-length encoding regroup "rows a sample used"
// into "samples that used a row"; runs shorter than 256 lookups and longer
// runs take different paths; section "Fewer reads and synchronizations": the
// number of long runs is known only at run time, so task lists are compacted
// on the GPU and later kernels read device-resident counts).  HugeCTR's
// walkthrough prints the same pipeline (sample-id expansion, radix sort by
// row with the end bit trimmed to the vocabulary, run flags + inclusive scan +
// run offsets).
//
// Kernels, in launch order (all 256 threads, no host readback anywhere):
//   transpose      key[p] = key_base[t] + I[p], bag[p] = j, and, with
//                  per-sample weights or a mean table, scale[p] = S[p]*(1/L)
//   radix passes   stable LSD sort by key over bits [0, ceil(log2(sum R))),
//                  8-bit digits, payload = bag id (+ scale): upsweep (LDS digit
//                  histogram per tile) -> scan (one workgroup per digit) ->
//                  downsweep (wave-ballot ranking, LDS reorder, coalesced
//                  scatter).  The payload rides along, so the sorted bag ids
//                  come out of the last pass without a gather.
//   rle_count / rle_scan / rle_write   run heads -> run_start, run_key, U
//   cls_count / cls_scan / cls_write   tiny / medium short-run tasks, long
//                                      tasks, chunk tasks, per-bucket begins,
//                                      fused countdowns
//
// Every tile kernel loads its whole tile (16 values per thread, clamped at the
// ragged end) before it computes, so the loads of a thread are in flight
// together instead of one memory round trip per element.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kItems = kTile / kThreads;  // 16 keys per thread

struct PrepDev {
  const TableDev* tables;
  uint32_t T, nb;
  int64_t B;
  int itype;
  const void* indices;
  const void* offsets;
  const float* psw;
  uint32_t N;
  uint32_t ntiles;
};

// Exclusive scan of one value per thread over the 256-thread workgroup.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh4, uint32_t& total) {
  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= (uint32_t)o) x += y;
  }
  if (lane == kWave - 1) sh4[wave] = x;
  __syncthreads();
  uint32_t wp = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    const uint32_t sw = sh4[w];
    wp += (w < (int)wave) ? sw : 0u;
    total += sw;
  }
  __syncthreads();
  return wp + x - v;
}

// 16 consecutive values a[i0 .. i0+15] (i0 a multiple of 16); entries at or
// past n repeat a[n-1] (n >= 1).  Four 16-byte loads for a full group.
__device__ __forceinline__ void load16(const uint32_t* __restrict__ a, uint64_t i0, uint64_t n,
                                       uint32_t* v) {
  if (i0 + kItems <= n) {
    const uint4* p = reinterpret_cast<const uint4*>(a + i0);
#pragma unroll
    for (int q = 0; q < kItems / 4; ++q) {
      const uint4 x = p[q];
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kItems; ++e) v[e] = a[(i0 + e < n) ? i0 + e : n - 1];
  }
}

// ------------------------------------------------------------ transposition
// 16 lanes per bag write its lookups' keys and bag id with contiguous stores.
// With per-sample weights or mean pooling it also writes the contribution
// scale of each lookup, S[p] * (1/L if mean) (FBTriton page, "Fusion
// boundaries": weights scale each contribution before grouping).
template <typename IT>
__global__ __launch_bounds__(kThreads) void transpose_kernel(PrepDev a, uint32_t* key,
                                                             uint32_t* bag, float* scale) {
  const uint32_t lane16 = threadIdx.x & 15;
  const uint64_t j = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) >> 4;
  if (j >= (uint64_t)a.T * (uint64_t)a.B) return;
  const uint32_t t = (uint32_t)(j / (uint64_t)a.B);
  const TableDev td = a.tables[t];
  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const int64_t lo = O[j];
  const int64_t hi = O[j + 1];
  const bool mean = td.pooling == POOL_MEAN;
  for (int64_t p = lo + lane16; p < hi; p += 16) {
    key[p] = td.key_base + (uint32_t)I[p];
    bag[p] = (uint32_t)j;
    if (scale) {
      const float sp = a.psw ? a.psw[p] : 1.0f;
      scale[p] = mean ? sp / (float)(hi - lo) : sp;
    }
  }
}

// ------------------------------------------------------------- radix sort

__global__ __launch_bounds__(kThreads) void radix_upsweep(const uint32_t* __restrict__ keys,
                                                          uint32_t N, uint32_t shift,
                                                          uint32_t* __restrict__ hist,
                                                          uint32_t ntiles) {
  __shared__ uint32_t h[kThreads / kWave][256];
  const uint32_t wave = threadIdx.x / kWave;
  const uint64_t i0 = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kItems;
  uint32_t k[kItems];
  if (i0 < N) load16(keys, i0, N, k);
  for (uint32_t i = threadIdx.x; i < 4 * 256; i += kThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kItems; ++e)
    if (i0 + e < N) atomicAdd(&h[wave][(k[e] >> shift) & 255u], 1u);
  __syncthreads();
  const uint32_t d = threadIdx.x;
  hist[(size_t)d * ntiles + blockIdx.x] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
}

// One workgroup per digit: exclusive scan of that digit's per-tile counts.
__global__ __launch_bounds__(kThreads) void radix_scan(uint32_t* __restrict__ hist,
                                                       uint32_t ntiles,
                                                       uint32_t* __restrict__ rowtot) {
  __shared__ uint32_t sh4[4];
  uint32_t* row = hist + (size_t)blockIdx.x * ntiles;
  uint32_t running = 0;
  for (uint32_t c = 0; c < ntiles; c += kThreads * 4) {
    uint32_t v[4], s = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = c + threadIdx.x * 4 + e;
      v[e] = i < ntiles ? row[i] : 0u;
      s += v[e];
    }
    uint32_t total;
    uint32_t x = block_excl_scan(s, sh4, total) + running;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = c + threadIdx.x * 4 + e;
      if (i < ntiles) row[i] = x;
      x += v[e];
    }
    running += total;
  }
  if (threadIdx.x == 0) rowtot[blockIdx.x] = running;
}

// Stable scatter of one tile.  Wave w owns the contiguous 1024 keys
// [tile + w*1024, tile + (w+1)*1024); in round r lane l holds key
// tile + w*1024 + r*64 + l, so (wave, round, lane) is the position order and
// ranking by wave-private digit counters keeps the sort stable.  The bag id
// (and the contribution scale, when SC) travel with the key.
template <bool SC>
__global__ __launch_bounds__(kThreads) void radix_downsweep(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin,
    const float* __restrict__ sin, uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
    float* __restrict__ sout, uint32_t N, uint32_t shift, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ rowtot, uint32_t ntiles) {
  __shared__ uint32_t s_key[kTile];
  __shared__ uint32_t s_val[kTile];
  __shared__ float s_sc[SC ? kTile : 1];
  __shared__ uint32_t wcnt[kThreads / kWave][256];
  __shared__ uint32_t gbase[256];
  __shared__ uint32_t lstart[256];
  __shared__ uint32_t sh4[4];

  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  const uint32_t tile = blockIdx.x;
  const uint64_t wbase = (uint64_t)tile * kTile + (uint64_t)wave * (kTile / 4);
  // the whole tile is loaded before any ranking
  uint32_t k[kItems], v[kItems], rk[kItems];
  float sc[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const uint64_t i = wbase + (uint64_t)r * kWave + lane;
    const uint64_t ii = i < N ? i : N - 1;
    k[r] = kin[ii];
    v[r] = vin[ii];
    if (SC) sc[r] = sin[ii];
  }
  __builtin_amdgcn_sched_barrier(0);
  for (uint32_t i = threadIdx.x; i < 4 * 256; i += kThreads) (&wcnt[0][0])[i] = 0u;
  {
    uint32_t total;
    const uint32_t d = threadIdx.x;
    const uint32_t dp = block_excl_scan(rowtot[d], sh4, total);
    gbase[d] = dp + hist[(size_t)d * ntiles + tile];
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const bool valid = wbase + (uint64_t)r * kWave + lane < N;
    const uint32_t d = (k[r] >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kRadixBits; ++bit) {
      const bool on = (d >> bit) & 1u;
      const uint64_t bb = __ballot(on);
      peers &= on ? bb : ~bb;
    }
    const uint32_t before = (uint32_t)__popcll(peers & lt_mask);
    const uint32_t prev = wcnt[wave][d];
    rk[r] = prev + before;
    if (valid && before == 0) wcnt[wave][d] = prev + (uint32_t)__popcll(peers);
  }
  __syncthreads();
  {
    const uint32_t d = threadIdx.x;
    uint32_t run = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      const uint32_t c = wcnt[w][d];
      wcnt[w][d] = run;
      run += c;
    }
    uint32_t total;
    lstart[d] = block_excl_scan(run, sh4, total);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const uint64_t i = wbase + (uint64_t)r * kWave + lane;
    if (i < N) {
      const uint32_t d = (k[r] >> shift) & 255u;
      const uint32_t slot = lstart[d] + wcnt[wave][d] + rk[r];
      if (slot < (uint32_t)kTile) {  // always true for a consistent ranking
        s_key[slot] = k[r];
        s_val[slot] = v[r];
        if (SC) s_sc[slot] = sc[r];
      }
    }
  }
  __syncthreads();
  const uint64_t tbase = (uint64_t)tile * kTile;
  const uint32_t n = (uint32_t)((N - tbase) < (uint64_t)kTile ? (N - tbase) : (uint64_t)kTile);
  for (uint32_t s = threadIdx.x; s < n; s += kThreads) {
    const uint32_t key = s_key[s];
    const uint32_t d = (key >> shift) & 255u;
    const uint32_t dst = gbase[d] + (s - lstart[d]);
    if (dst < N) {  // always true for consistent digit counts
      kout[dst] = key;
      vout[dst] = s_val[s];
      if (SC) sout[dst] = s_sc[s];
    }
  }
}

// --------------------------------------------------- run-length encoding
// Blocked layout: thread h of a tile owns sorted slots [tile + 16h, tile + 16h + 16).

__device__ __forceinline__ uint32_t head_mask(const uint32_t* __restrict__ key, uint64_t i0,
                                              uint32_t N) {
  if (i0 >= N) return 0u;
  uint32_t k[kItems];
  const uint32_t prev0 = i0 == 0 ? 0u : key[i0 - 1];
  load16(key, i0, N, k);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t m = 0;
  uint32_t prev = prev0;
#pragma unroll
  for (int e = 0; e < kItems; ++e) {
    const uint64_t i = i0 + e;
    if (i < N && (i == 0 || k[e] != prev)) m |= 1u << e;
    prev = k[e];
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void rle_count(const uint32_t* __restrict__ key, uint32_t N,
                                                      uint32_t* __restrict__ tile_cnt) {
  __shared__ uint32_t sh4[4];
  const uint64_t i0 = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kItems;
  const uint32_t c = __popc(head_mask(key, i0, N));
  uint32_t total;
  block_excl_scan(c, sh4, total);
  if (threadIdx.x == 0) tile_cnt[blockIdx.x] = total;
}

// Single workgroup: exclusive scan of `rows` rows of `n` counters each (in
// place); row totals to `totals`.
__device__ void scan_rows_single_block(uint32_t* data, uint32_t n, int rows, uint32_t* totals) {
  __shared__ uint32_t sh4[4];
  for (int rr = 0; rr < rows; ++rr) {
    uint32_t* row = data + (size_t)rr * n;
    uint32_t running = 0;
    for (uint32_t c = 0; c < n; c += kThreads * 4) {
      uint32_t v[4], s = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = c + threadIdx.x * 4 + e;
        v[e] = i < n ? row[i] : 0u;
        s += v[e];
      }
      uint32_t total;
      uint32_t x = block_excl_scan(s, sh4, total) + running;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t i = c + threadIdx.x * 4 + e;
        if (i < n) row[i] = x;
        x += v[e];
      }
      running += total;
    }
    totals[rr] = running;
  }
}

__global__ __launch_bounds__(kThreads) void rle_scan(uint32_t* tile_cnt, uint32_t ntiles,
                                                     uint32_t N, uint32_t* counters,
                                                     uint32_t* run_start) {
  uint32_t U;
  scan_rows_single_block(tile_cnt, ntiles, 1, &U);
  if (threadIdx.x == 0) {
    counters[kCntU] = U;
    run_start[U] = N;
  }
}

__global__ __launch_bounds__(kThreads) void rle_write(const uint32_t* __restrict__ key, uint32_t N,
                                                      const uint32_t* __restrict__ tile_base,
                                                      uint32_t* __restrict__ run_start,
                                                      uint32_t* __restrict__ run_key) {
  __shared__ uint32_t sh4[4];
  const uint64_t i0 = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kItems;
  const uint32_t m = head_mask(key, i0, N);
  uint32_t total;
  uint32_t u = tile_base[blockIdx.x] + block_excl_scan(__popc(m), sh4, total);
  if (m == 0u) return;
  uint32_t k[kItems];
  load16(key, i0, N, k);
#pragma unroll
  for (int e = 0; e < kItems; ++e) {
    if (m & (1u << e)) {
      run_start[u] = (uint32_t)(i0 + e);
      run_key[u] = k[e];
      ++u;
    }
  }
}

// ----------------------------------------------------------- classification
// Runs are listed by length: SL < kTinyRun and kTinyRun <= SL < 256 are both
// short runs (one program owns the row and updates it with plain stores); the
// split only picks the program size (a lane subgroup or a whole workgroup).
// SL >= 256 are long runs, cut into chunks of 256.

struct ClsDev {
  const uint32_t* run_start;
  const uint32_t* run_key;
  const uint32_t* sorted_bag;
  uint32_t* counters;
  uint32_t* tile_cls;        // kNumLists rows x ntiles
  uint32_t ntiles;
  uint4* single_task;
  uint4* tiny_task;
  uint4* med_task;
  uint4* long_task;
  uint32_t* long_cbeg;
  uint32_t* remaining;
  uint4* chunk_task;
  const TableDev* tables;
  const uint32_t* order;     // table ids in ascending key_base order
  const uint32_t* bkb;       // nb+1 bucket key bounds
  uint32_t T, nb;
  uint32_t N, max_tiny, max_med, max_long, max_chunks;  // list capacities
};

// per-run counts of the five lists: SL = 1, 2 <= SL < 32, 32 <= SL < 256,
// long runs, chunks
__device__ __forceinline__ void run_class(uint32_t len, uint32_t* c) {
  const bool lg = len >= (uint32_t)kLongRun;
  c[0] = len == 1u ? 1u : 0u;
  c[1] = (len >= 2u && len < (uint32_t)kTinyRun) ? 1u : 0u;
  c[2] = (!lg && len >= (uint32_t)kTinyRun) ? 1u : 0u;
  c[3] = lg ? 1u : 0u;
  c[4] = lg ? (len + kChunk - 1) / kChunk : 0u;
}

// run lengths of runs u0 .. u0+15 (0 past U): run_start has U+1 entries
__device__ __forceinline__ void run_lengths(const uint32_t* __restrict__ run_start, uint64_t u0,
                                            uint32_t U, uint32_t* start, uint32_t* len) {
  uint32_t s[kItems];
  load16(run_start, u0, (uint64_t)U + 1, s);
  const uint32_t last = run_start[(u0 + kItems <= U) ? u0 + kItems : U];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int e = 0; e < kItems; ++e) {
    const uint32_t nxt = e + 1 < kItems ? s[e + 1] : last;
    start[e] = s[e];
    len[e] = (u0 + e < U) ? nxt - s[e] : 0u;
  }
}

__global__ __launch_bounds__(kThreads) void cls_count(ClsDev a) {
  __shared__ uint32_t sh4[4];
  const uint32_t U = a.counters[kCntU];
  const uint64_t u0 = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kItems;
  uint32_t acc[kNumLists] = {0u, 0u, 0u, 0u, 0u};
  if (u0 < U) {
    uint32_t start[kItems], len[kItems];
    run_lengths(a.run_start, u0, U, start, len);
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      uint32_t c[kNumLists];
      run_class(len[e], c);
      const uint32_t in = (u0 + e < U) ? 1u : 0u;
      for (int q = 0; q < kNumLists; ++q) acc[q] += in * c[q];
    }
  }
  for (int q = 0; q < kNumLists; ++q) {
    uint32_t tot;
    block_excl_scan(acc[q], sh4, tot);
    if (threadIdx.x == 0) a.tile_cls[q * a.ntiles + blockIdx.x] = tot;
  }
}

__device__ __forceinline__ uint32_t bucket_of_key(const uint32_t* bkb, uint32_t nb, uint32_t key) {
  uint32_t b = 0;
  for (uint32_t i = 1; i < nb; ++i) b += (bkb[i] <= key) ? 1u : 0u;
  return b;
}

__global__ __launch_bounds__(kThreads) void cls_scan(ClsDev a) {
  __shared__ uint32_t tot[kNumLists];
  uint32_t t4[kNumLists];
  scan_rows_single_block(a.tile_cls, a.ntiles, kNumLists, t4);
  if (threadIdx.x == 0) {
    for (int k = 0; k < kNumLists; ++k) {
      tot[k] = t4[k];
      a.counters[kCntSingle + k] = t4[k];
    }
  }
  __syncthreads();
  // begins of the buckets after the last run's bucket (all of them when U == 0)
  const uint32_t U = a.counters[kCntU];
  const int first = U == 0 ? 0 : (int)bucket_of_key(a.bkb, a.nb, a.run_key[U - 1]) + 1;
  for (int b = first + (int)threadIdx.x; b <= (int)a.nb; b += kThreads) {
    for (int k = 0; k < kNumLists; ++k) a.counters[kCntBegins + k * (a.nb + 1) + b] = tot[k];
  }
}

__global__ __launch_bounds__(kThreads) void cls_write(ClsDev a) {
  __shared__ uint32_t s_kb[kMaxTables];
  __shared__ uint32_t s_ord[kMaxTables];
  __shared__ uint32_t s_bkb[64];
  __shared__ uint32_t sh4[4];
  const uint32_t U = a.counters[kCntU];
  const uint64_t tile0 = (uint64_t)blockIdx.x * kTile;
  if (tile0 >= U) return;  // uniform per workgroup: no barrier is skipped by part of it
  const uint64_t u0 = tile0 + (uint64_t)threadIdx.x * kItems;
  uint32_t start[kItems], len[kItems], key[kItems], bag0[kItems];
  uint32_t keyprev = 0;
  const bool mine = u0 < U;
  if (mine) {
    run_lengths(a.run_start, u0, U, start, len);
    load16(a.run_key, u0, U, key);
    keyprev = u0 == 0 ? 0u : a.run_key[u0 - 1];
#pragma unroll
    for (int e = 0; e < kItems; ++e) bag0[e] = a.sorted_bag[start[e] < a.N ? start[e] : a.N - 1];
  }
  for (uint32_t i = threadIdx.x; i < a.T; i += kThreads) {
    const uint32_t t = a.order[i];
    s_ord[i] = t;
    s_kb[i] = a.tables[t].key_base;
  }
  for (uint32_t i = threadIdx.x; i <= a.nb; i += kThreads) s_bkb[i] = a.bkb[i];

  uint32_t acc[kNumLists] = {0u, 0u, 0u, 0u, 0u};
  if (mine) {
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      uint32_t c[kNumLists];
      run_class(len[e], c);
      const uint32_t in = (u0 + e < U) ? 1u : 0u;
      for (int q = 0; q < kNumLists; ++q) acc[q] += in * c[q];
    }
  }
  uint32_t pos[kNumLists];
  for (int q = 0; q < kNumLists; ++q) {
    uint32_t tot;
    pos[q] = a.tile_cls[q * a.ntiles + blockIdx.x] + block_excl_scan(acc[q], sh4, tot);
  }
  // block_excl_scan ends with a barrier, so the LDS tables above are visible
  if (!mine) return;

  int bprev = u0 == 0 ? -1 : (int)bucket_of_key(s_bkb, a.nb, keyprev);
  for (int e = 0; e < kItems; ++e) {
    if (u0 + e >= U) break;
    const uint32_t k = key[e], ln = len[e], st = start[e];
    // table of the key: last table whose key_base <= key
    uint32_t lo = 0, hi = a.T;  // invariant: s_kb[lo] <= key < s_kb[hi] (s_kb[T] = +inf)
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (s_kb[mid] <= k) lo = mid; else hi = mid;
    }
    const uint32_t t = s_ord[lo];
    const uint32_t row = k - s_kb[lo];
    // bucket begins: this run opens buckets (bucket(prev run), bucket(this run)]
    const int bcur = (int)bucket_of_key(s_bkb, a.nb, k);
    for (int b = bprev + 1; b <= bcur; ++b)
      for (int q = 0; q < kNumLists; ++q) a.counters[kCntBegins + q * (a.nb + 1) + b] = pos[q];
    bprev = bcur;
    if (ln == 1u) {
      // {start, row, table, bag of the lookup}
      if (pos[0] < a.N) a.single_task[pos[0]] = make_uint4(st, row, t, bag0[e]);
      ++pos[0];
    } else if (ln < (uint32_t)kTinyRun) {
      if (pos[1] < a.max_tiny) a.tiny_task[pos[1]] = make_uint4(st, ln, row, t);
      ++pos[1];
    } else if (ln < (uint32_t)kLongRun) {
      if (pos[2] < a.max_med) a.med_task[pos[2]] = make_uint4(st, ln, row, t);
      ++pos[2];
    } else {
      const uint32_t nch = (ln + kChunk - 1) / kChunk;
      const uint32_t pl = pos[3], pc = pos[4];
      if (pl < a.max_long) {
        a.long_task[pl] = make_uint4(st, ln, row, t);
        a.long_cbeg[pl] = pc;
        a.remaining[pl] = nch;
      }
      for (uint32_t q = 0; q < nch && pc + q < a.max_chunks; ++q) {
        const uint32_t cl_len = (ln - q * kChunk) < (uint32_t)kChunk ? (ln - q * kChunk)
                                                                      : (uint32_t)kChunk;
        a.chunk_task[pc + q] = make_uint4(st + q * kChunk, cl_len, t, pl);
      }
      pos[4] += nch;
      ++pos[3];
    }
  }
}

}  // namespace

hipError_t launch_preprocess(const PrepArgs& p, int /*grid_persist*/, hipStream_t s) {
  const WsLayout& L = *p.L;
  if (p.N == 0) return hipSuccess;
  uint8_t* ws = p.ws;
  auto u32p = [&](size_t off) { return reinterpret_cast<uint32_t*>(ws + off); };
  auto f32p = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  PrepDev d{p.tables, p.T, p.nb, p.B, p.itype, p.indices, p.offsets, p.psw, p.N, L.ntiles};
  const bool sc = p.need_scale != 0;

  const uint64_t nbag = (uint64_t)p.T * (uint64_t)p.B;
  const uint64_t tgrid = (nbag * 16 + kThreads - 1) / kThreads;
  if (p.itype == IT_I32)
    TBE_LAUNCH("transpose", transpose_kernel<int32_t>, dim3((uint32_t)tgrid), dim3(kThreads), s,
               d, u32p(L.key_a), u32p(L.val_a), sc ? f32p(L.sc_a) : nullptr);
  else
    TBE_LAUNCH("transpose", transpose_kernel<int64_t>, dim3((uint32_t)tgrid), dim3(kThreads), s,
               d, u32p(L.key_a), u32p(L.val_a), sc ? f32p(L.sc_a) : nullptr);

  // ping-pong a -> b -> a ...; the final buffers are b for an odd pass count
  for (int pass = 0; pass < L.npass; ++pass) {
    const bool ab = (pass % 2) == 0;
    const uint32_t* kin = u32p(ab ? L.key_a : L.key_b);
    const uint32_t* vin = u32p(ab ? L.val_a : L.val_b);
    const float* sin = f32p(ab ? L.sc_a : L.sc_b);
    uint32_t* kout = u32p(ab ? L.key_b : L.key_a);
    uint32_t* vout = u32p(ab ? L.val_b : L.val_a);
    float* sout = f32p(ab ? L.sc_b : L.sc_a);
    const uint32_t shift = (uint32_t)(pass * kRadixBits);
    TBE_LAUNCH("radix_upsweep", radix_upsweep, dim3(L.ntiles), dim3(kThreads), s, kin, p.N,
               shift, u32p(L.hist), L.ntiles);
    TBE_LAUNCH("radix_scan", radix_scan, dim3(256), dim3(kThreads), s, u32p(L.hist), L.ntiles,
               u32p(L.rowtot));
    if (sc)
      TBE_LAUNCH("radix_downsweep", radix_downsweep<true>, dim3(L.ntiles), dim3(kThreads), s,
                 kin, vin, sin, kout, vout, sout, p.N, shift, u32p(L.hist), u32p(L.rowtot),
                 L.ntiles);
    else
      TBE_LAUNCH("radix_downsweep", radix_downsweep<false>, dim3(L.ntiles), dim3(kThreads), s,
                 kin, vin, sin, kout, vout, sout, p.N, shift, u32p(L.hist), u32p(L.rowtot),
                 L.ntiles);
  }
  const uint32_t* skey = u32p(L.final_in_b ? L.key_b : L.key_a);
  const uint32_t* sbag = u32p(L.final_in_b ? L.val_b : L.val_a);
  TBE_LAUNCH("rle_count", rle_count, dim3(L.ntiles), dim3(kThreads), s, skey, p.N,
             u32p(L.tile_cnt));
  TBE_LAUNCH("rle_scan", rle_scan, dim3(1), dim3(kThreads), s, u32p(L.tile_cnt), L.ntiles, p.N,
             u32p(L.counters), u32p(L.run_start));
  TBE_LAUNCH("rle_write", rle_write, dim3(L.ntiles), dim3(kThreads), s, skey, p.N,
             u32p(L.tile_cnt), u32p(L.run_start), u32p(L.run_key));

  ClsDev c{u32p(L.run_start), u32p(L.run_key), sbag, u32p(L.counters),
           u32p(L.tile_cls), L.ntiles,
           reinterpret_cast<uint4*>(ws + L.single_task), reinterpret_cast<uint4*>(ws + L.tiny_task),
           reinterpret_cast<uint4*>(ws + L.med_task),
           reinterpret_cast<uint4*>(ws + L.long_task), u32p(L.long_cbeg), u32p(L.remaining),
           reinterpret_cast<uint4*>(ws + L.chunk_task), p.tables, p.order, p.bucket_key_begin,
           p.T, p.nb, p.N, L.max_tiny, L.max_med, L.max_long, L.max_chunks};
  TBE_LAUNCH("cls_count", cls_count, dim3(L.ntiles), dim3(kThreads), s, c);
  TBE_LAUNCH("cls_scan", cls_scan, dim3(1), dim3(kThreads), s, c);
  TBE_LAUNCH("cls_write", cls_write, dim3(L.ntiles), dim3(kThreads), s, c);
  return hipGetLastError();
}

}  // namespace tbe
