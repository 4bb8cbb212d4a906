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
//   transpose      key[p] = key_base[t] + I[p], bag[p] = j          (bag-parallel)
//   radix passes   stable LSD sort of (key, position), 8-bit digits, bits
//                  [0, ceil(log2(sum R))): upsweep (LDS digit histogram per
//                  4096-key tile) -> scan (one workgroup per digit) ->
//                  downsweep (wave-ballot ranking, LDS reorder, coalesced
//                  scatter).  The first pass generates positions itself.
//   rle_count / rle_scan / rle_write   run heads -> run_start, run_key, U
//   cls_count / cls_scan / cls_write   short tasks, long tasks, chunk tasks,
//                                      per-bucket begins, fused countdowns
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

// ------------------------------------------------------------ transposition
// 16 lanes per bag write its lookups' keys and bag id with contiguous stores.
__global__ __launch_bounds__(kThreads) void transpose_kernel(PrepDev a, uint32_t* key,
                                                             uint32_t* bag) {
  const uint32_t lane16 = threadIdx.x & 15;
  const uint64_t j = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) >> 4;
  if (j >= (uint64_t)a.T * (uint64_t)a.B) return;
  const uint32_t t = (uint32_t)(j / (uint64_t)a.B);
  const uint32_t kb = a.tables[t].key_base;
  const int64_t lo = load_idx(a.offsets, a.itype, (int64_t)j);
  const int64_t hi = load_idx(a.offsets, a.itype, (int64_t)j + 1);
  for (int64_t p = lo + lane16; p < hi; p += 16) {
    key[p] = kb + (uint32_t)load_idx(a.indices, a.itype, p);
    bag[p] = (uint32_t)j;
  }
}

// ------------------------------------------------------------- radix sort

__global__ __launch_bounds__(kThreads) void radix_upsweep(const uint32_t* __restrict__ keys,
                                                          uint32_t N, uint32_t shift,
                                                          uint32_t* __restrict__ hist,
                                                          uint32_t ntiles) {
  __shared__ uint32_t h[kThreads / kWave][256];
  for (uint32_t i = threadIdx.x; i < 4 * 256; i += kThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t wave = threadIdx.x / kWave;
  const uint64_t base = (uint64_t)blockIdx.x * kTile;
#pragma unroll
  for (int r = 0; r < kItems / 4; ++r) {
    const uint64_t i = base + ((uint64_t)r * kThreads + threadIdx.x) * 4;
    if (i + 3 < N) {
      const uint4 k = *reinterpret_cast<const uint4*>(keys + i);
      atomicAdd(&h[wave][(k.x >> shift) & 255u], 1u);
      atomicAdd(&h[wave][(k.y >> shift) & 255u], 1u);
      atomicAdd(&h[wave][(k.z >> shift) & 255u], 1u);
      atomicAdd(&h[wave][(k.w >> shift) & 255u], 1u);
    } else {
      for (uint64_t e = i; e < N && e < i + 4; ++e) atomicAdd(&h[wave][(keys[e] >> shift) & 255u], 1u);
    }
  }
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
// ranking by wave-private digit counters keeps the sort stable.
__global__ __launch_bounds__(kThreads) void radix_downsweep(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin,
    uint32_t* __restrict__ kout, uint32_t* __restrict__ vout, uint32_t N, uint32_t shift,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ rowtot, uint32_t ntiles) {
  __shared__ uint32_t s_key[kTile];
  __shared__ uint32_t s_val[kTile];
  __shared__ uint32_t wcnt[kThreads / kWave][256];
  __shared__ uint32_t gbase[256];
  __shared__ uint32_t lstart[256];
  __shared__ uint32_t sh4[4];

  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  const uint32_t tile = blockIdx.x;
  for (uint32_t i = threadIdx.x; i < 4 * 256; i += kThreads) (&wcnt[0][0])[i] = 0u;
  {
    uint32_t total;
    const uint32_t d = threadIdx.x;
    const uint32_t dp = block_excl_scan(rowtot[d], sh4, total);
    gbase[d] = dp + hist[(size_t)d * ntiles + tile];
  }
  __syncthreads();

  const uint64_t wbase = (uint64_t)tile * kTile + (uint64_t)wave * (kTile / 4);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t k[kItems], v[kItems], rk[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const uint64_t i = wbase + (uint64_t)r * kWave + lane;
    const bool valid = i < N;
    k[r] = valid ? kin[i] : 0u;
    v[r] = valid ? (vin ? vin[i] : (uint32_t)i) : 0u;
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
    }
  }
}

// --------------------------------------------------- run-length encoding
// Blocked layout: thread h of a tile owns sorted slots [tile + 16h, tile + 16h + 16).

__device__ __forceinline__ uint32_t head_mask(const uint32_t* __restrict__ key, uint64_t i0,
                                              uint32_t N) {
  uint32_t m = 0;
  if (i0 >= N) return 0u;
  uint32_t prev = i0 == 0 ? 0u : key[i0 - 1];
#pragma unroll
  for (int e = 0; e < kItems; ++e) {
    const uint64_t i = i0 + e;
    if (i < N) {
      const uint32_t k = key[i];
      if (i == 0 || k != prev) m |= 1u << e;
      prev = k;
    }
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
#pragma unroll
  for (int e = 0; e < kItems; ++e) {
    if (m & (1u << e)) {
      run_start[u] = (uint32_t)(i0 + e);
      run_key[u] = key[i0 + e];
      ++u;
    }
  }
}

// ----------------------------------------------------------- classification

struct ClsDev {
  const uint32_t* run_start;
  const uint32_t* run_key;
  uint32_t* counters;
  uint32_t* tile_cls;        // 3 rows x ntiles: short, long, chunk counts
  uint32_t ntiles;
  uint4* short_task;
  uint4* long_task;
  uint32_t* long_cbeg;
  uint32_t* remaining;
  uint4* chunk_task;
  const TableDev* tables;
  const uint32_t* order;     // table ids in ascending key_base order
  const uint32_t* bkb;       // nb+1 bucket key bounds
  uint32_t T, nb;
  uint32_t N, max_long, max_chunks;  // list capacities
};

__device__ __forceinline__ void run_class(uint32_t len, uint32_t& s, uint32_t& l, uint32_t& c) {
  const bool lg = len >= (uint32_t)kLongRun;
  s = lg ? 0u : 1u;
  l = lg ? 1u : 0u;
  c = lg ? (len + kChunk - 1) / kChunk : 0u;
}

__global__ __launch_bounds__(kThreads) void cls_count(ClsDev a) {
  __shared__ uint32_t sh4[4];
  const uint32_t U = a.counters[kCntU];
  const uint64_t u0 = (uint64_t)blockIdx.x * kTile + (uint64_t)threadIdx.x * kItems;
  uint32_t cs = 0, cl = 0, cc = 0;
  for (int e = 0; e < kItems; ++e) {
    const uint64_t u = u0 + e;
    if (u >= U) break;
    uint32_t s, l, c;
    run_class(a.run_start[u + 1] - a.run_start[u], s, l, c);
    cs += s; cl += l; cc += c;
  }
  uint32_t ts, tl, tc;
  block_excl_scan(cs, sh4, ts);
  block_excl_scan(cl, sh4, tl);
  block_excl_scan(cc, sh4, tc);
  if (threadIdx.x == 0) {
    a.tile_cls[blockIdx.x] = ts;
    a.tile_cls[a.ntiles + blockIdx.x] = tl;
    a.tile_cls[2 * a.ntiles + blockIdx.x] = tc;
  }
}

__device__ __forceinline__ uint32_t bucket_of_key(const uint32_t* bkb, uint32_t nb, uint32_t key) {
  uint32_t b = 0;
  for (uint32_t i = 1; i < nb; ++i) b += (bkb[i] <= key) ? 1u : 0u;
  return b;
}

__global__ __launch_bounds__(kThreads) void cls_scan(ClsDev a) {
  __shared__ uint32_t tot[3];
  uint32_t t3[3];
  scan_rows_single_block(a.tile_cls, a.ntiles, 3, t3);
  if (threadIdx.x == 0) {
    tot[0] = t3[0]; tot[1] = t3[1]; tot[2] = t3[2];
    a.counters[kCntShort] = t3[0];
    a.counters[kCntLong] = t3[1];
    a.counters[kCntChunks] = t3[2];
  }
  __syncthreads();
  // begins of the buckets after the last run's bucket (all of them when U == 0)
  const uint32_t U = a.counters[kCntU];
  const int first = U == 0 ? 0 : (int)bucket_of_key(a.bkb, a.nb, a.run_key[U - 1]) + 1;
  for (int b = first + (int)threadIdx.x; b <= (int)a.nb; b += kThreads) {
    for (int k = 0; k < 3; ++k) a.counters[kCntBegins + k * (a.nb + 1) + b] = tot[k];
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
  for (uint32_t i = threadIdx.x; i < a.T; i += kThreads) {
    const uint32_t t = a.order[i];
    s_ord[i] = t;
    s_kb[i] = a.tables[t].key_base;
  }
  for (uint32_t i = threadIdx.x; i <= a.nb; i += kThreads) s_bkb[i] = a.bkb[i];

  const uint64_t u0 = tile0 + (uint64_t)threadIdx.x * kItems;
  uint32_t cs = 0, cl = 0, cc = 0;
  for (int e = 0; e < kItems; ++e) {
    const uint64_t u = u0 + e;
    if (u >= U) break;
    uint32_t s, l, c;
    run_class(a.run_start[u + 1] - a.run_start[u], s, l, c);
    cs += s; cl += l; cc += c;
  }
  uint32_t tot;
  uint32_t ps = a.tile_cls[blockIdx.x] + block_excl_scan(cs, sh4, tot);
  uint32_t pl = a.tile_cls[a.ntiles + blockIdx.x] + block_excl_scan(cl, sh4, tot);
  uint32_t pc = a.tile_cls[2 * a.ntiles + blockIdx.x] + block_excl_scan(cc, sh4, tot);
  // block_excl_scan ends with a barrier, so the LDS tables above are visible

  for (int e = 0; e < kItems; ++e) {
    const uint64_t u = u0 + e;
    if (u >= U) break;
    const uint32_t start = a.run_start[u];
    const uint32_t len = a.run_start[u + 1] - start;
    const uint32_t key = a.run_key[u];
    // table of the key: last table whose key_base <= key
    uint32_t lo = 0, hi = a.T;  // invariant: s_kb[lo] <= key < s_kb[hi] (s_kb[T] = +inf)
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (s_kb[mid] <= key) lo = mid; else hi = mid;
    }
    const uint32_t t = s_ord[lo];
    const uint32_t row = key - s_kb[lo];
    // bucket begins: this run opens buckets (bucket(prev run), bucket(this run)]
    const uint32_t bcur = bucket_of_key(s_bkb, a.nb, key);
    const int bprev = u == 0 ? -1 : (int)bucket_of_key(s_bkb, a.nb, a.run_key[u - 1]);
    for (int b = bprev + 1; b <= (int)bcur; ++b) {
      a.counters[kCntBegins + b] = ps;
      a.counters[kCntBegins + (a.nb + 1) + b] = pl;
      a.counters[kCntBegins + 2 * (a.nb + 1) + b] = pc;
    }
    if (len < (uint32_t)kLongRun) {
      if (ps < a.N) a.short_task[ps] = make_uint4(start, len, row, t);
      ++ps;
    } else {
      const uint32_t nch = (len + kChunk - 1) / kChunk;
      if (pl < a.max_long) {
        a.long_task[pl] = make_uint4(start, len, row, t);
        a.long_cbeg[pl] = pc;
        a.remaining[pl] = nch;
      }
      for (uint32_t k = 0; k < nch && pc + k < a.max_chunks; ++k) {
        const uint32_t cl_len = (len - k * kChunk) < (uint32_t)kChunk ? (len - k * kChunk)
                                                                       : (uint32_t)kChunk;
        a.chunk_task[pc + k] = make_uint4(start + k * kChunk, cl_len, t, pl);
      }
      pc += nch;
      ++pl;
    }
  }
}

}  // namespace

hipError_t launch_preprocess(const PrepArgs& p, int /*grid_persist*/, hipStream_t s) {
  const WsLayout& L = *p.L;
  if (p.N == 0) return hipSuccess;
  uint8_t* ws = p.ws;
  auto u32p = [&](size_t off) { return reinterpret_cast<uint32_t*>(ws + off); };
  PrepDev d{p.tables, p.T, p.nb, p.B, p.itype, p.indices, p.offsets, p.N, L.ntiles};

  const uint64_t nbag = (uint64_t)p.T * (uint64_t)p.B;
  const uint64_t tgrid = (nbag * 16 + kThreads - 1) / kThreads;
  TBE_LAUNCH("transpose", transpose_kernel, dim3((uint32_t)tgrid), dim3(kThreads), s, d,
                     u32p(L.key_a), u32p(L.bag));

  uint32_t* kin = u32p(L.key_a);
  uint32_t* vin = nullptr;  // first pass: values are the positions themselves
  uint32_t* kout = u32p(L.key_b);
  uint32_t* vout = u32p(L.val_b);
  for (int pass = 0; pass < L.npass; ++pass) {
    const uint32_t shift = (uint32_t)(pass * kRadixBits);
    TBE_LAUNCH("radix_upsweep", radix_upsweep, dim3(L.ntiles), dim3(kThreads), s, kin, p.N, shift,
                       u32p(L.hist), L.ntiles);
    TBE_LAUNCH("radix_scan", radix_scan, dim3(256), dim3(kThreads), s, u32p(L.hist), L.ntiles,
                       u32p(L.rowtot));
    TBE_LAUNCH("radix_downsweep", radix_downsweep, dim3(L.ntiles), dim3(kThreads), s, kin, vin, kout,
                       vout, p.N, shift, u32p(L.hist), u32p(L.rowtot), L.ntiles);
    // ping-pong: a -> b -> a ...
    if (kout == u32p(L.key_b)) {
      kin = u32p(L.key_b); vin = u32p(L.val_b);
      kout = u32p(L.key_a); vout = u32p(L.val_a);
    } else {
      kin = u32p(L.key_a); vin = u32p(L.val_a);
      kout = u32p(L.key_b); vout = u32p(L.val_b);
    }
  }
  const uint32_t* skey = kin;
  TBE_LAUNCH("rle_count", rle_count, dim3(L.ntiles), dim3(kThreads), s, skey, p.N,
                     u32p(L.tile_cnt));
  TBE_LAUNCH("rle_scan", rle_scan, dim3(1), dim3(kThreads), s, u32p(L.tile_cnt), L.ntiles, p.N,
                     u32p(L.counters), u32p(L.run_start));
  TBE_LAUNCH("rle_write", rle_write, dim3(L.ntiles), dim3(kThreads), s, skey, p.N,
                     u32p(L.tile_cnt), u32p(L.run_start), u32p(L.run_key));

  ClsDev c{u32p(L.run_start), u32p(L.run_key), u32p(L.counters), u32p(L.tile_cls), L.ntiles,
           reinterpret_cast<uint4*>(ws + L.short_task), reinterpret_cast<uint4*>(ws + L.long_task),
           u32p(L.long_cbeg), u32p(L.remaining), reinterpret_cast<uint4*>(ws + L.chunk_task),
           p.tables, p.order, p.bucket_key_begin, p.T, p.nb, p.N, L.max_long, L.max_chunks};
  TBE_LAUNCH("cls_count", cls_count, dim3(L.ntiles), dim3(kThreads), s, c);
  TBE_LAUNCH("cls_scan", cls_scan, dim3(1), dim3(kThreads), s, c);
  TBE_LAUNCH("cls_write", cls_write, dim3(L.ntiles), dim3(kThreads), s, c);
  return hipGetLastError();
}

}  // namespace tbe
