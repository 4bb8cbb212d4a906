// Backward preprocessing on the device (FBTriton TBE page, "Backward": the
// lookups are transposed from bag order to row order by sorting them on their
// row and run-length encoding the sorted rows; runs shorter than 256 lookups
// and longer runs take different paths; section "Fewer reads and
// synchronizations": how many long runs there are is known only on the
// device, so the task lists are compacted there and later kernels read
// device-resident counts).  HugeCTR's backward walkthrough has the same
// pipeline (sample ids expanded per lookup, radix sort by row with the end
// bit cut to the vocabulary, run flags, scan, run offsets).
//
// Segments.  The lookups of table t are contiguous (table-major bags), so
// sorting by linear key is sorting each table's lookups by row and placing the
// tables in key order.  Each table is a segment sorted on its own: the radix
// passes cover only the bits of the largest table's row range (C5: 23 bits,
// three 8-bit passes, instead of 29 bits of linear key) and tiles never
// straddle two segments.  Tile offsets come from one prefix over all tiles:
// the count of a digit in the segments before a tile's segment is that prefix
// at the segment's first tile, and is subtracted.
//
// Kernels, in launch order (256 threads each, no host readback anywhere):
//   tile_map       per segment (tables in key order) lookup count, output
//                  base, first tile; the segment and the first lookup's bag
//                  of every tile; clears the control block (tickets, error
//                  flag)
//   then per digit of 8 or 10 bits (the fewest passes of at most 10 bits
//   that cover the row range), least significant first:
//   radix_upsweep  per tile, the count of each value of the digit of
//                  (key - key_base) in the pass's input; the first one reads
//                  the rows from the indices, finds each tile's first bag
//                  and clears the look-back status words of rle and classify
//   radix_scan     per digit value, the exclusive prefix over all tiles (in
//                  place) and the total
//   radix_downsweep  a stable scatter of each 4096-key tile to the offsets
//                  of the scan (a decoupled look-back instead of the count
//                  and scan was measured 2-4x slower per pass on MI355X at 34k
//                  tiles: C5, three passes); the first one ("transpose")
//                  forms its tile from the lookups: key = key_base[t] + I[p],
//                  bag = j and, with per-sample weights or a mean table,
//                  scale = S[p]*(1/L)
//   rle            run heads of the sorted keys -> run_start, run_key, U (tile
//                  offsets by look-back)
//   classify       one-lookup / tiny / medium short-run tasks, long-run tasks,
//                  256-lookup chunk tasks, per-bucket begins and the fused
//                  countdowns (five list offsets by look-back)
//
// Look-back protocol: a workgroup takes its tile number from an atomic ticket,
// so every smaller tile belongs to a workgroup that is already running and
// never waits on a larger one; every wait therefore ends.  It publishes its own
// count ("aggregate"), adds the published values of the tiles before it until
// it meets an inclusive prefix, then publishes its own inclusive prefix.  The
// status words are read and written with relaxed device-scope atomics; they
// carry the counts themselves, so no other memory needs ordering.  A wait is
// bounded: past `polls` polls (kSpinLimit unless a test knob lowers it) it
// sets the error flag and goes on, which spoils the result but lets the
// kernel finish; every backward kernel reads the flag first and writes
// nothing when it is set.  With a limit of 0 a tile that has predecessors
// gives up before its first poll.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kItems = kTile / kThreads;  // 16 keys per thread
constexpr int kClsItems = kClsTile / kThreads;  // 4 runs per thread

constexpr uint64_t kStAgg = 1ull << 62;  // the tile's own count is published
constexpr uint64_t kStPre = 2ull << 62;  // the inclusive prefix through the tile is published
constexpr uint64_t kStFlags = 3ull << 62;

struct PrepDev {
  const TableDev* tables;
  uint32_t T, nb;
  int64_t B;
  const void* indices;
  const void* offsets;
  const float* psw;
  uint32_t N;
  const uint32_t* tseg;  // segment (position in key order) of each table
  const uint4* seg;      // per segment {lookups, output base, first tile, key base}
  const uint2* seg2;     // per segment {first position O[t*B], table t}
};

__device__ __forceinline__ void st_publish(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t st_read(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the counts of tiles [0, tile) in column `col` of a status table
// with `stride` words per tile.  The wave is split into groups of GL lanes,
// each looking back for its own column (all 64 lanes call this; `col` is
// uniform in a group): lane i of a group reads predecessor tile - 1 - i, so
// one round trip covers GL tiles.  The ready words nearest the tile are
// consumed up to the first inclusive prefix; an unpublished one stops the
// window there and is polled again.  (One lane reading 16 words per round trip
// made the prefix frontier the limit of the run-length and classification
// passes at C5's ~10k tiles.)
template <int GL>
__device__ uint32_t look_back(uint64_t* st, uint32_t tile, uint32_t stride, uint32_t col,
                              uint32_t* err, uint32_t polls) {
  static_assert(GL == 16 || GL == 32 || GL == 64, "groups of 16, 32 or 64 lanes");
  const uint32_t lane = lane_id();
  const uint32_t i = lane & (GL - 1), base = lane & ~(uint32_t)(GL - 1);
  const uint64_t gmask = GL == 64 ? ~0ull : ((1ull << GL) - 1ull);
  uint32_t excl = 0, spins = 0;
  uint32_t t = tile;  // tiles [0, t) are still to be summed (uniform in the group)
  bool fin = t == 0;
  if (!fin && polls == 0u) {  // no poll allowed: give up at once
    if (i == 0) atomicOr(err, 1u);
    fin = true;
  }
  while (__ballot(!fin)) {
    const bool have = !fin && t > i;
    const uint64_t v = have ? st_read(st + (size_t)(t - 1 - i) * stride + col) : 0ull;
    const uint64_t f = v & kStFlags;
    const uint64_t unpub = (__ballot(have && f == 0) >> base) & gmask;
    const uint64_t pre = (__ballot(have && f == kStPre) >> base) & gmask;
    const uint32_t first_unpub = unpub ? (uint32_t)__builtin_ctzll(unpub) : (uint32_t)GL;
    const uint32_t first_pre = pre ? (uint32_t)__builtin_ctzll(pre) : (uint32_t)GL;
    const uint32_t navail = t < (uint32_t)GL ? t : (uint32_t)GL;  // predecessors in the window
    // lanes consumed: through the first prefix if no gap comes before it,
    // else up to the first gap, else the whole window
    const bool done = first_pre < first_unpub || (first_unpub == (uint32_t)GL && navail == t);
    const uint32_t used = fin ? 0u
                          : first_pre < first_unpub ? first_pre + 1u
                          : (first_unpub < navail ? first_unpub : navail);
    uint32_t c = (i < used) ? (uint32_t)v : 0u;
#pragma unroll
    for (int o = GL / 2; o > 0; o >>= 1) c += __shfl_xor(c, o, kWave);
    if (!fin) {
      excl += c;
      t -= used;
      if (done) {
        fin = true;
      } else if (used == 0u) {  // the nearest predecessor has not published yet
        if (++spins >= polls) {
          if (i == 0) atomicOr(err, 1u);
          fin = true;
        }
      }
    }
    if (__ballot(!fin && used == 0u)) __builtin_amdgcn_s_sleep(1);
  }
  return excl;
}

// Publish a tile's count, look back, publish its inclusive prefix; returns the
// exclusive prefix.  Called by a whole wave; the first lane of each GL-lane
// group publishes its column.
template <int GL>
__device__ __forceinline__ uint32_t publish_and_look_back(uint64_t* st, uint32_t tile,
                                                          uint32_t stride, uint32_t col,
                                                          uint32_t count, uint32_t* err,
                                                          uint32_t polls) {
  uint64_t* mine = st + (size_t)tile * stride + col;
  const bool first = (lane_id() & (GL - 1)) == 0;
  if (tile == 0) {
    if (first) st_publish(mine, kStPre | count);
    return 0;
  }
  if (first) st_publish(mine, kStAgg | count);
  const uint32_t excl = look_back<GL>(st, tile, stride, col, err, polls);
  if (first) st_publish(mine, kStPre | (uint64_t)(uint32_t)(excl + count));
  return excl;
}

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

// NI consecutive values a[i0 .. i0+NI-1] of a workspace array (i0 a multiple
// of NI, NI * 4 bytes dividing kWsAlign) as 16-byte loads, also where the
// group runs past the array's last entry: the array ends on a kWsAlign
// boundary, so a group that starts inside it ends inside it, and entries
// past the end are whatever the padding holds.  (Clamping each entry's
// position instead let the compiler turn every group into 4-byte loads,
// one 64-byte line per lane and instruction.)
template <int NI>
__device__ __forceinline__ void load_ws_group(const uint32_t* __restrict__ a, uint64_t i0,
                                              uint32_t* v) {
  static_assert(NI % 4 == 0 && kWsAlign % (NI * 4) == 0, "groups tile the padded array");
  const uint4* p = reinterpret_cast<const uint4*>(a + i0);
#pragma unroll
  for (int q = 0; q < NI / 4; ++q) {
    const uint4 x = p[q];
    v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
  }
}

// As load_ws_group for a group that starts below n (n entries in use), with
// the entries at or past n replaced by a[n - 1].
template <int NI>
__device__ __forceinline__ void loadn(const uint32_t* __restrict__ a, uint64_t i0, uint64_t n,
                                      uint32_t* v) {
  load_ws_group<NI>(a, i0, v);
  const uint32_t last = a[n - 1];  // (loaded by every lane: no branch holds
                                   // back the loads that follow)
#pragma unroll
  for (int e = 0; e < NI; ++e) v[e] = i0 + e < n ? v[e] : last;
}

// The workgroup's tile number, in the order workgroups start.  One counter
// per class c = workgroup index mod 8, and tile = 8 * ticket + c: workgroups
// go to the eight XCDs round-robin by index, so a class is an XCD, and one
// counter for all workgroups would serialize them (an atomic on one address
// costs about 11 ns per workgroup on MI355X: 0.4 ms for 35k workgroups).  A
// grid of n workgroups has as many members of class c as there are tiles
// below n in that class, so every tile is taken once.  Waits still end: the
// smallest tile not finished is either running (then everything it waits on
// is finished) or not yet taken, and then its XCD runs only workgroups with
// smaller tiles, which finish and make room for it.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* tickets, uint32_t* s_tile) {
  if (threadIdx.x == 0) {
    const uint32_t c = blockIdx.x & 7u;
    *s_tile = atomicAdd(tickets + c * kTicketStride, 1u) * 8u + c;
  }
  __syncthreads();
  return *s_tile;
}

// ------------------------------------------------------------ transposition
// The transposition from bag order to row order is folded into the first
// radix pass.  That pass's input order is the lookups' own order (bags are
// table-major, so a table's lookups are one contiguous range), so its count
// pass reads the indices themselves, and its scatter forms each lookup's key
// = key_base[t] + I[p], bag id and contribution scale S[p] * (1/L if mean)
// (FBTriton page, "Fusion boundaries": the weights scale each contribution
// before the grouping by row) while it loads its tile, where a separate pass
// would write all of them out in lookup order and the scatter read them back.
// Slot i of table t's segment holds position p = O[t*B] + (i - the segment's
// output base).

// Per segment (segment s is table order[s], tables in key order; its lookups
// are [O[t*B], O[(t+1)*B])) from the offsets, into dynamic LDS: lookups,
// output base, first tile and tile count.  Offsets that keep the contract (O[T*B] = N)
// are unchanged by the clamps; others still give segments inside [0, N) and
// at most ntiles_max tiles.  Returns the tile total; ends with a barrier.
template <typename IT>
__device__ uint32_t segment_table(const PrepDev& a, const uint32_t* __restrict__ order,
                                  uint32_t* s_nc, uint32_t* s_on, uint32_t* s_ot, uint32_t* s_nt,
                                  uint32_t* sh4) {
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  uint32_t run_n = 0, run_t = 0;
  for (uint32_t s0 = 0; s0 < a.T; s0 += kThreads) {
    const uint32_t s = s0 + threadIdx.x;
    uint32_t n = 0;
    if (s < a.T) {
      const uint32_t t = order[s];
      n = (uint32_t)(O[(int64_t)(t + 1) * a.B] - O[(int64_t)t * a.B]);
    }
    uint32_t tot_n, tot_t;
    const uint64_t on_raw = (uint64_t)run_n + block_excl_scan(n, sh4, tot_n);
    const uint32_t on = on_raw < a.N ? (uint32_t)on_raw : a.N;
    const uint32_t nc = on_raw < a.N ? (n < a.N - on ? n : a.N - on) : 0u;
    const uint32_t nt = (nc + kTile - 1) / kTile;
    const uint32_t ot = run_t + block_excl_scan(nt, sh4, tot_t);
    if (s < a.T) {
      s_nc[s] = nc;
      s_on[s] = on;
      s_ot[s] = ot;
      s_nt[s] = nt;
    }
    run_n += tot_n;
    run_t += tot_t;
  }
  __syncthreads();
  return run_t;
}

// The segment table, the tile map and the control block, before the first
// count pass.  Every workgroup forms the segment table in LDS (T entries);
// workgroup 0 writes it out (and, per segment, its first position and
// table, so that the first pass reads its tile's lookups after one
// dependent load) with the tile total and clears the control block
// (tickets, error flag); the grid then writes the segment of every tile (the
// last segment whose first tile is at or before it) and, streaming the
// offsets once, the bag of every tile's first lookup: a non-empty bag j of
// table t holds the first lookup of tile k of t's segment when 4096 k lies in
// [O[j], O[j+1]) - O[t*B], so every tile gets the one bag that holds its
// first lookup (for offsets that keep the contract).
template <typename IT>
__global__ __launch_bounds__(kThreads) void tile_map_kernel(PrepDev a,
                                                            const uint32_t* __restrict__ order,
                                                            uint4* __restrict__ seg,
                                                            uint2* __restrict__ seg2,
                                                            uint32_t* __restrict__ tile_seg,
                                                            uint32_t* __restrict__ tile_bag0,
                                                            uint32_t ntiles_max,
                                                            uint32_t* __restrict__ ctl) {
  extern __shared__ uint32_t s_dyn[];  // 4 T words
  __shared__ uint32_t sh4[4];
  uint32_t* s_nc = s_dyn;
  uint32_t* s_on = s_dyn + a.T;
  uint32_t* s_ot = s_dyn + 2 * a.T;
  uint32_t* s_nt = s_dyn + 3 * a.T;
  const uint32_t total = segment_table<IT>(a, order, s_nc, s_on, s_ot, s_nt, sh4);
  const uint32_t ntiles = total < ntiles_max ? total : ntiles_max;
  if (blockIdx.x == 0) {
    for (uint32_t i = threadIdx.x; i < (uint32_t)kCtlWords; i += kThreads)
      if (i != (uint32_t)kCtlTiles) ctl[i] = 0u;
    const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
    for (uint32_t s = threadIdx.x; s < a.T; s += kThreads) {
      const uint32_t t = order[s];
      seg[s] = make_uint4(s_nc[s], s_on[s], s_ot[s], a.tables[t].key_base);
      seg2[s] = make_uint2((uint32_t)O[(int64_t)t * a.B], t);
    }
    if (threadIdx.x == 0) ctl[kCtlTiles] = ntiles;
  }
  const uint32_t gsz = gridDim.x * kThreads, gid = blockIdx.x * kThreads + threadIdx.x;
  for (uint32_t i = gid; i < ntiles; i += gsz) {
    uint32_t lo = 0, hi = a.T;  // s_ot[lo] <= i < s_ot[hi] (s_ot[T] read as past every tile)
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) >> 1;
      if (s_ot[mid] <= i) lo = mid; else hi = mid;
    }
    tile_seg[i] = lo;
  }
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const uint64_t B = (uint64_t)a.B, nbag = (uint64_t)a.T * B;
  for (uint64_t j = gid; j < nbag; j += gsz) {
    const uint32_t t = (uint32_t)(j / B);
    const uint32_t s = a.tseg[t];
    const uint32_t nt = s < a.T ? s_nt[s] : 0u;
    if (nt == 0) continue;
    const int64_t base = (int64_t)O[(uint64_t)t * B];
    const int64_t lo = (int64_t)O[j] - base, hi = (int64_t)O[j + 1] - base;
    if (hi <= lo || hi <= 0) continue;
    const int64_t k0 = lo <= 0 ? 0 : (lo + kTile - 1) / kTile;
    const int64_t k1 = (hi - 1) / kTile < (int64_t)nt - 1 ? (hi - 1) / kTile : (int64_t)nt - 1;
    for (int64_t k = k0; k <= k1; ++k) {
      const uint64_t tile = (uint64_t)s_ot[s] + (uint64_t)k;
      if (tile < ntiles) tile_bag0[tile] = (uint32_t)j;
    }
  }
}

// Position of slot i of a segment (pshift = its table's first position minus
// its output base), clamped into [0, N): inside for offsets that keep the
// contract, and in bounds for any others.
__device__ __forceinline__ uint32_t slot_pos(int64_t pshift, uint32_t i, uint32_t N) {
  const int64_t p = (int64_t)i + pshift;
  return p < 0 ? 0u : (p >= (int64_t)N ? N - 1u : (uint32_t)p);
}

// The row of lookup p: an int64 index is read as its low word (rows < 2^32).
template <typename IT>
__device__ __forceinline__ uint32_t index_lo(const void* I, uint32_t p) {
  return reinterpret_cast<const uint32_t*>(I)[(size_t)p * (sizeof(IT) / 4)];
}

// ------------------------------------------------------------- radix sort

// Tile `tile` of the segmented layout: its segment sid, and its slots [b, e).
__device__ __forceinline__ uint4 tile_span(const uint4* __restrict__ seg,
                                           const uint32_t* __restrict__ tile_seg, uint32_t tile,
                                           uint32_t& sid, uint32_t& b, uint32_t& e) {
  sid = tile_seg[tile];
  const uint4 sg = seg[sid];  // {lookups, output base, first tile, key base}
  b = sg.y + (tile - sg.z) * (uint32_t)kTile;
  const uint32_t se = sg.y + sg.x;
  e = (se - b) < (uint32_t)kTile ? se : b + (uint32_t)kTile;
  return sg;
}

// Tile of this workgroup in the sort passes, XCD-major: workgroup i runs on
// XCD i mod 8, and with a grid of 8 * per workgroups XCD x takes the
// contiguous tiles [x * per, (x + 1) * per).  Neighbouring tiles write
// neighbouring bytes (the digit counts of consecutive tiles share cache
// lines; a digit's keys of consecutive tiles land next to each other), so
// their partial lines merge in one L2 instead of being written back from
// eight.
__device__ __forceinline__ uint32_t xcd_tile() {
  return (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
}

// Adds digit d of this lane's item (when valid) to the workgroup's counts,
// kept in four copies h[c][.] by lane (c = lane mod 4) and shared by the
// waves.  A hot row puts its digit in many lanes of a wave, and the LDS
// serializes the atomics of one instruction that meet at one address; four
// copies make those meetings a quarter as long (MI355X, C5, a count pass
// 229 -> 170 us, against 147 us with the counting's atomics left out).  A
// wave whose valid items all share one digit adds them with one atomic.
template <int R>
__device__ __forceinline__ void count_digit(uint32_t (*h)[R], uint32_t d, bool valid,
                                            uint32_t lane) {
  const uint32_t d0 = __builtin_amdgcn_readfirstlane(d);
  const uint64_t in = __ballot(valid);
  if (__ballot(valid && d != d0) == 0) {
    if (lane == 0 && in != 0) atomicAdd(&h[0][d0], (uint32_t)__popcll(in));
  } else if (valid) {
    atomicAdd(&h[lane & 3u][d], 1u);
  }
}

// As count_digit for items whose equal digits tend to sit in neighbouring
// lanes (a pass after the first: its keys are sorted by the digits below, so
// the many copies of a hot row's key are close together): a stretch of lanes
// with one digit adds its length with one atomic from its last lane.
template <int R>
__device__ __forceinline__ void count_digit_runs(uint32_t (*h)[R], uint32_t d, bool valid,
                                                 uint32_t lane) {
  const uint32_t dp = __shfl_up(d, 1, kWave);
  const uint64_t in = __ballot(valid);
  const bool pv = lane > 0 && ((in >> (lane - 1)) & 1ull);
  const bool cont = valid && pv && dp == d;  // continues the stretch of lane - 1
  const uint64_t cm = __ballot(cont);
  const bool last = valid && (lane == kWave - 1 || ((cm >> (lane + 1)) & 1ull) == 0);
  if (last) {
    // the stretch's first lane: the highest lane at or below this one that
    // does not continue its predecessor
    const uint64_t heads = in & ~cm & (lane == kWave - 1 ? ~0ull : ((2ull << lane) - 1ull));
    const uint32_t first = 63u - (uint32_t)__clzll(heads);
    atomicAdd(&h[lane & 3u][d], lane - first + 1u);
  }
}

// Counts of each digit value of one pass for every tile of the pass's input,
// digit-major: cnt[d * ntiles + tile], digits of DB bits of the row
// (key - key_base), counted by count_digit.  With nst > 0 the kernel also
// clears nst look-back status words of the later kernels.
template <int DB>
__global__ __launch_bounds__(kThreads) void radix_upsweep(const uint32_t* __restrict__ keys,
                                                          const uint4* __restrict__ seg,
                                                          const uint32_t* __restrict__ tile_seg,
                                                          const uint32_t* __restrict__ ctl,
                                                          uint32_t shift,
                                                          uint32_t* __restrict__ cnt,
                                                          uint32_t ntiles,
                                                          uint64_t* __restrict__ st, uint64_t nst) {
  constexpr uint32_t R = 1u << DB;
  __shared__ uint32_t h[4][R];
  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t tile = xcd_tile();
  const bool live = tile < ctl[kCtlTiles];
  for (uint32_t i = threadIdx.x; i < 4u * R; i += kThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
  if (live) {
    uint32_t sid, b, e;
    const uint4 sg = tile_span(seg, tile_seg, tile, sid, b, e);
    const uint32_t wb = b + wave * (kTile / 4);
    uint32_t k[kItems];
    // (slots past e read slot e - 1: no branch around the loads; they are
    // not counted)
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const uint32_t i = wb + (uint32_t)r * kWave + lane;
      k[r] = keys[i < e ? i : e - 1u];
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r)
      count_digit_runs<R>(h, ((k[r] - sg.w) >> shift) & (R - 1u),
                          wb + (uint32_t)r * kWave + lane < e, lane);
  }
  __syncthreads();
  if (live)
    for (uint32_t d = threadIdx.x; d < R; d += kThreads)
      cnt[(size_t)d * ntiles + tile] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < nst; i += stride)
    st[i] = 0ull;
}

// The first pass's counts, from the indices: as radix_upsweep, with the row
// of slot i read at its position in the lookups (the first digit has shift
// 0).
template <typename IT, int DB>
__global__ __launch_bounds__(kThreads) void first_upsweep(PrepDev a,
                                                          const uint32_t* __restrict__ tile_seg,
                                                          const uint32_t* __restrict__ ctl,
                                                          uint32_t* __restrict__ cnt,
                                                          uint32_t ntiles,
                                                          uint64_t* __restrict__ st, uint64_t nst) {
  constexpr uint32_t R = 1u << DB;
  __shared__ uint32_t h[4][R];
  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t tile = xcd_tile();
  const bool live = tile < ctl[kCtlTiles];
  for (uint32_t i = threadIdx.x; i < 4u * R; i += kThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
  if (live) {
    uint32_t sid, b, e;
    const uint4 sg = tile_span(a.seg, tile_seg, tile, sid, b, e);
    const int64_t pshift = (int64_t)a.seg2[sid].x - (int64_t)sg.y;
    const uint32_t wb = b + wave * (kTile / 4);
    uint32_t k[kItems];
    // (slots past e read slot e - 1's lookup: no branch, so all 16 loads are
    // in flight together; they are not counted)
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const uint32_t i = wb + (uint32_t)r * kWave + lane;
      k[r] = index_lo<IT>(a.indices, slot_pos(pshift, i < e ? i : e - 1u, a.N));
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r)
      count_digit<R>(h, k[r] & (R - 1u), wb + (uint32_t)r * kWave + lane < e, lane);
  }
  __syncthreads();
  if (live)
    for (uint32_t d = threadIdx.x; d < R; d += kThreads)
      cnt[(size_t)d * ntiles + tile] = h[0][d] + h[1][d] + h[2][d] + h[3][d];
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x; i < nst; i += stride)
    st[i] = 0ull;
}

// One workgroup per digit value d: the exclusive prefix over all tiles of the
// counts of d, written tile-major (tex[tile * 2^DB + d], so that a tile's
// prefixes of every digit are one contiguous vector for the scatter), and the
// total of d.  At a segment's first tile the prefix is the count of d in all
// earlier segments.  Digits are taken XCD-major (workgroup i runs on XCD
// i mod 8; XCD x takes the x-th eighth of the digits), so the prefixes of
// neighbouring digits, which share cache lines, are written from one L2.
template <int DB>
__global__ __launch_bounds__(kThreads) void radix_scan(const uint32_t* __restrict__ cnt,
                                                       uint32_t ntiles,
                                                       const uint32_t* __restrict__ ctl,
                                                       uint32_t* __restrict__ tex,
                                                       uint32_t* __restrict__ totals) {
  constexpr uint32_t R = 1u << DB;
  __shared__ uint32_t sh4[4];
  const uint32_t d = (blockIdx.x & 7u) * (R / 8u) + (blockIdx.x >> 3);
  const uint32_t nt = ctl[kCtlTiles];
  const uint32_t* row = cnt + (size_t)d * ntiles;
  uint32_t running = 0;
  for (uint32_t c = 0; c < nt; c += kThreads * 4) {
    uint32_t v[4], sum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = c + threadIdx.x * 4 + e;
      v[e] = i < nt ? row[i] : 0u;
      sum += v[e];
    }
    uint32_t total;
    uint32_t x = block_excl_scan(sum, sh4, total) + running;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = c + threadIdx.x * 4 + e;
      if (i < nt) tex[(size_t)i * R + d] = x;
      x += v[e];
    }
    running += total;
  }
  if (threadIdx.x == 0) totals[d] = running;
}

struct SortPass {
  const uint32_t* kin;
  const uint32_t* vin;
  const float* sin;
  uint32_t* kout;
  uint32_t* vout;
  float* sout;
  uint32_t shift;
  const uint4* seg;           // per segment {lookups, output base, first tile, key base}
  const uint32_t* tile_seg;   // segment of each tile
  const uint32_t* tiles;      // number of tiles (ctl[kCtlTiles])
  const uint32_t* totals;     // digit totals of this pass over all segments
  const uint32_t* tile_excl;  // per tile and digit (tile-major), the count in earlier tiles
  uint32_t ntiles;
  // the first pass only: the lookups, and the bag of each tile's first lookup
  const void* indices;
  const void* offsets;
  const float* psw;
  const TableDev* tables;
  const uint2* seg2;          // per segment {first position O[t*B], table t}
  const uint32_t* tile_bag0;
  int64_t B;
  uint32_t N, T;
};

// Stable scatter of one tile to the offsets of the scan: the count of each
// digit in all earlier tiles, minus the prefix at the segment's first tile,
// is the count in the earlier tiles of the same segment.  Wave w holds the contiguous 1024
// slots [b + w*1024, b + (w+1)*1024) of the tile [b, e); in round r lane l
// holds slot b + w*1024 + r*64 + l, so (wave, round, lane) is the position
// order and ranking by wave-private digit counters keeps the sort stable.
// The digit (DB bits) is taken from the row, key - key_base; thread t owns
// the Q = 2^DB / 256 consecutive digit values [tQ, tQ + Q) for the per-digit
// prefixes.  Keys, bag ids and scales pass through one LDS buffer in turn on
// their way to their coalesced global stores.
//
// FIRST: the first pass, which forms its tile from the lookups (the
// transposition above).  Slot i's key and scale come from its position p;
// its bag is the last bag j with O[j] <= p, found by binary search over the
// offsets of the bags from the tile's first lookup's to the next tile's
// (held in the LDS buffer, or read from global memory when there are more
// than 4096 of them, which takes empty bags).
template <int DB, bool SC, bool FIRST, typename IT>
__device__ __forceinline__ void sort_pass_body(const SortPass& p) {
  constexpr uint32_t R = 1u << DB;
  constexpr int Q = (int)(R / kThreads);
  static_assert(Q >= 1 && R % kThreads == 0, "at least one digit value per thread");
  __shared__ uint32_t s_buf[kTile];
  __shared__ uint32_t wcnt[kThreads / kWave][R];
  __shared__ uint32_t gbase[R];
  __shared__ uint32_t lstart[R];
  __shared__ uint32_t sh4[4];

  const uint32_t lane = lane_id(), wave = threadIdx.x / kWave;
  const uint32_t tile = xcd_tile();
  if (tile >= *p.tiles) return;  // the grid is sized for the most tiles segments can need
  // the first pass's tile bags, loaded with the segment (both need only the tile)
  uint32_t tb0 = 0, tb1 = 0;
  if constexpr (FIRST) {
    tb0 = p.tile_bag0[tile];
    tb1 = p.tile_bag0[tile + 1u < p.ntiles ? tile + 1u : tile];
  }
  for (uint32_t i = threadIdx.x; i < 4u * R; i += kThreads) (&wcnt[0][0])[i] = 0u;
  uint32_t sid, b, e;
  const uint4 sg = tile_span(p.seg, p.tile_seg, tile, sid, b, e);
  const uint32_t wbase = b + wave * (kTile / 4);
  // the whole tile is loaded before any ranking
  uint32_t k[kItems], v[kItems], rk[kItems];
  float sc[kItems];
  if constexpr (FIRST) {
    const IT* __restrict__ O = reinterpret_cast<const IT*>(p.offsets);
    const uint2 s2 = p.seg2[sid];
    const uint32_t t = s2.y < p.T ? s2.y : 0u;
    const uint64_t j0 = (uint64_t)t * (uint64_t)p.B;
    const int64_t pshift = (int64_t)s2.x - (int64_t)sg.y;
    // rows and weights in flight while the offsets load
    float sp[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const uint32_t i = wbase + (uint32_t)r * kWave + lane;
      const uint32_t pp = slot_pos(pshift, i < e ? i : e - 1, p.N);
      k[r] = index_lo<IT>(p.indices, pp);
      sp[r] = (SC && p.psw) ? p.psw[pp] : 1.0f;
    }
    // offsets of bags jb .. je + 1 (the clamps hold for what the count pass wrote)
    const uint64_t jlast = j0 + (uint64_t)p.B - 1u;
    const uint32_t z_next = sg.z + (sg.x + kTile - 1) / kTile;
    uint64_t jb = tb0;
    uint64_t je = tile + 1u < z_next ? (uint64_t)tb1 : jlast;
    jb = jb < j0 ? j0 : (jb > jlast ? jlast : jb);
    je = je < jb ? jb : (je > jlast ? jlast : je);
    const uint32_t nw = (uint32_t)(je - jb) + 2u;
    const bool fits = nw <= (uint32_t)kTile;  // uniform
    // top: the largest power of two <= nw - 1; entries [nw, 2 top) are set
    // past every position (2 top <= 4096 when the window fits), so the search
    // below reads any entry it can reach without a bounds check
    const uint32_t top = 1u << (31 - __builtin_clz(nw - 1u));
    if (fits) {
      for (uint32_t i = threadIdx.x; i < nw; i += kThreads) s_buf[i] = (uint32_t)O[jb + i];
      for (uint32_t i = nw + threadIdx.x; i < 2u * top; i += kThreads) s_buf[i] = 0xffffffffu;
    }
    __syncthreads();
    const bool mean = SC && p.tables[t].pooling == POOL_MEAN;
    const uint32_t kb = sg.w;
    // w[r]: the last window entry at or before the slot's position (entry 0
    // is, and entry nw - 1 is past it, for offsets that keep the contract),
    // so bag jb + w holds it.  In the LDS window the slots take the steps
    // top, top / 2, ..., 1 together, so each step issues kItems independent
    // reads.
    uint32_t w[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) w[r] = 0;
    if (fits) {
      uint32_t pp[kItems];
#pragma unroll
      for (int r = 0; r < kItems; ++r) {
        const uint32_t i = wbase + (uint32_t)r * kWave + lane;
        pp[r] = slot_pos(pshift, i < e ? i : e - 1, p.N);
      }
      for (uint32_t step = top; step > 0; step >>= 1) {
        uint32_t o[kItems];
#pragma unroll
        for (int r = 0; r < kItems; ++r) o[r] = s_buf[w[r] + step];
#pragma unroll
        for (int r = 0; r < kItems; ++r) w[r] = o[r] <= pp[r] ? w[r] + step : w[r];
      }
    } else {
#pragma unroll 1
      for (int r = 0; r < kItems; ++r) {
        const uint32_t i = wbase + (uint32_t)r * kWave + lane;
        const uint32_t pp = slot_pos(pshift, i < e ? i : e - 1, p.N);
        uint32_t lo = 0, hi = nw - 1u;  // offset[lo] <= pp < offset[hi]
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if ((uint32_t)O[jb + mid] <= pp) lo = mid; else hi = mid;
        }
        w[r] = lo;
      }
    }
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      k[r] = kb + k[r];
      v[r] = (uint32_t)(jb + w[r]);
      if (SC) {
        const uint32_t L = fits ? s_buf[w[r] + 1u] - s_buf[w[r]]
                                : (uint32_t)O[jb + w[r] + 1u] - (uint32_t)O[jb + w[r]];
        sc[r] = mean ? sp[r] / (float)L : sp[r];
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const uint32_t i = wbase + (uint32_t)r * kWave + lane;
      const uint32_t ii = i < e ? i : e - 1;
      k[r] = p.kin[ii];
      v[r] = p.vin[ii];
      if (SC) sc[r] = p.sin[ii];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t d0 = threadIdx.x * (uint32_t)Q;  // the digits this thread publishes
  __syncthreads();  // wcnt cleared

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const bool valid = wbase + (uint32_t)r * kWave + lane < e;
    const uint32_t d = ((k[r] - sg.w) >> p.shift) & (R - 1u);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < DB; ++bit) {
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
  // per owned digit: the waves' counts become exclusive over the waves, and
  // the digit's count in the tile feeds the tile-local starts
  uint32_t lex[Q], lsum = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    uint32_t c = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) {
      const uint32_t x = wcnt[w][d0 + q];
      wcnt[w][d0 + q] = c;
      c += x;
    }
    lex[q] = lsum;
    lsum += c;
  }
  uint32_t total;
  const uint32_t ls0 = block_excl_scan(lsum, sh4, total);
#pragma unroll
  for (int q = 0; q < Q; ++q) lstart[d0 + q] = ls0 + lex[q];
  __syncthreads();
  // tile-local slots, keys into LDS while the destinations are formed
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const bool valid = wbase + (uint32_t)r * kWave + lane < e;
    const uint32_t d = ((k[r] - sg.w) >> p.shift) & (R - 1u);
    const uint32_t slot = lstart[d] + wcnt[wave][d] + rk[r];
    rk[r] = (valid && slot < (uint32_t)kTile) ? slot : 0xffffffffu;  // always in range when valid
    if (rk[r] != 0xffffffffu) s_buf[rk[r]] = k[r];
  }
  // per owned digit: its count in the segments before this one, in this
  // segment and in the earlier tiles of this segment (taken after the
  // ranking, so that none of it is live across the ranking loop); then the
  // destination base = segment base + the digits below it in the segment +
  // the digit's count in the segment's earlier tiles - its tile-local start
  const uint32_t z_next = sg.z + (sg.x + kTile - 1) / kTile;
  const uint32_t* at_seg = p.tile_excl + (size_t)sg.z * R + d0;
  const uint32_t* at_next = z_next < *p.tiles ? p.tile_excl + (size_t)z_next * R + d0
                                              : p.totals + d0;
  const uint32_t* at_tile = p.tile_excl + (size_t)tile * R + d0;
  uint32_t part[Q], sum = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint32_t before_seg = at_seg[q];
    part[q] = sum + (at_tile[q] - before_seg) - (ls0 + lex[q]);
    sum += at_next[q] - before_seg;
  }
  const uint32_t seg_excl = sg.y + block_excl_scan(sum, sh4, total);  // ends with a barrier
#pragma unroll
  for (int q = 0; q < Q; ++q) gbase[d0 + q] = seg_excl + part[q];
  __syncthreads();

  const uint32_t n = e - b;
  const uint32_t send = sg.y + sg.x;
  uint32_t dst[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const uint32_t sl = threadIdx.x + (uint32_t)r * kThreads;
    dst[r] = 0xffffffffu;
    if (sl < n) {
      const uint32_t key = s_buf[sl];
      const uint32_t g = gbase[((key - sg.w) >> p.shift) & (R - 1u)] + sl;
      if (g >= sg.y && g < send) {  // always true for consistent digit counts
        dst[r] = g;
        p.kout[g] = key;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r)
    if (rk[r] != 0xffffffffu) s_buf[rk[r]] = v[r];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r)
    if (dst[r] != 0xffffffffu) p.vout[dst[r]] = s_buf[threadIdx.x + (uint32_t)r * kThreads];
  if (SC) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r)
      if (rk[r] != 0xffffffffu) s_buf[rk[r]] = __builtin_bit_cast(uint32_t, sc[r]);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r)
      if (dst[r] != 0xffffffffu)
        p.sout[dst[r]] = __builtin_bit_cast(float, s_buf[threadIdx.x + (uint32_t)r * kThreads]);
  }
}

template <int DB, bool SC>
__global__ __launch_bounds__(kThreads) void sort_pass_kernel(SortPass p) {
  sort_pass_body<DB, SC, false, uint32_t>(p);
}

// The first pass, with the transposition folded in.
template <int DB, bool SC, typename IT>
__global__ __launch_bounds__(kThreads) void transpose_scatter_kernel(SortPass p) {
  sort_pass_body<DB, SC, true, IT>(p);
}

// --------------------------------------------------- run-length encoding
// A tile is G consecutive groups of 4096 sorted slots; in group g thread h
// owns slots [tile + g*4096 + 16h, ... + 16), so every load is coalesced,
// and runs are numbered group by group in slot order.  Four groups per tile
// make the look-back chain a quarter as long (deep batches); one gives a
// shallow batch four times the workgroups.

template <int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void rle_kernel(const uint32_t* __restrict__ key, uint32_t N,
                                                       uint32_t ntiles, uint32_t* ticket,
                                                       uint64_t* st, uint32_t* err,
                                                       uint32_t* __restrict__ counters,
                                                       uint32_t* __restrict__ run_start,
                                                       uint32_t* __restrict__ run_key,
                                                       uint32_t polls) {
  __shared__ uint32_t sh4[4];
  __shared__ uint32_t s_tile, s_excl;
  __shared__ uint32_t s_rs[kTile], s_rk[kTile];  // one group's run heads, staged
  const uint32_t tile = take_ticket(ticket, &s_tile);
  uint32_t k[G][kItems], prev0[G];
  uint32_t m[G];  // run heads among this thread's 16 slots of each group
  // every group's keys in flight before any is used (a group that starts
  // at or past N loads nothing; slots past N are not counted)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t i0 = (uint64_t)tile * (G * kTile) + (uint64_t)g * kTile +
                        (uint64_t)threadIdx.x * kItems;
    prev0[g] = (i0 == 0 || i0 > N) ? 0u : key[i0 - 1];
    if (i0 < N) {
      load_ws_group<kItems>(key, i0, k[g]);
    } else {
#pragma unroll
      for (int e = 0; e < kItems; ++e) k[g][e] = 0u;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t i0 = (uint64_t)tile * (G * kTile) + (uint64_t)g * kTile +
                        (uint64_t)threadIdx.x * kItems;
    m[g] = 0;
    uint32_t prev = prev0[g];
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const uint64_t i = i0 + e;
      if (i < N && (i == 0 || k[g][e] != prev)) m[g] |= 1u << e;
      prev = k[g][e];
    }
  }
  uint32_t local[G], gbase[G + 1], total = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint32_t tg;
    gbase[g] = total;
    local[g] = block_excl_scan(__popc(m[g]), sh4, tg);  // within the group
    total += tg;
  }
  gbase[G] = total;
  if (threadIdx.x < (uint32_t)kWave) {  // wave 0
    const uint32_t excl = publish_and_look_back<64>(st, tile, 1, 0, total, err, polls);
    if (threadIdx.x == 0) {
      s_excl = excl;
      if (tile == ntiles - 1) {
        counters[kCntU] = excl + total;
        run_start[excl + total] = N;
      }
    }
  }
  __syncthreads();
  const uint32_t excl = s_excl;
  // a group's run heads go to LDS in run order, then out with coalesced
  // stores (written straight from each thread's slots, most lanes of every
  // store would be masked off: runs are a fraction of the slots)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t i0 = (uint64_t)tile * (G * kTile) + (uint64_t)g * kTile +
                        (uint64_t)threadIdx.x * kItems;
    uint32_t u = local[g];
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      if (m[g] & (1u << e)) {
        s_rs[u] = (uint32_t)(i0 + e);
        s_rk[u] = k[g][e];
        ++u;
      }
    }
    __syncthreads();
    const uint32_t ng = gbase[g + 1] - gbase[g];
    for (uint32_t i = threadIdx.x; i < ng; i += kThreads) {
      run_start[excl + gbase[g] + i] = s_rs[i];
      run_key[excl + gbase[g] + i] = s_rk[i];
    }
    __syncthreads();  // the group's heads are out before the next group's go in
  }
}

// ----------------------------------------------------------- classification
// Runs are listed by length: SL = 1, 2 <= SL < kTinyRun and kTinyRun <= SL <
// 256 are short runs (one program owns the row and updates it with plain
// stores); the split only picks the program shape.  SL >= 256 are long runs,
// cut into chunks of 256.

struct ClsDev {
  const uint32_t* run_start;
  const uint32_t* run_key;
  const uint32_t* sorted_bag;
  uint32_t* counters;
  uint32_t* ticket;
  uint64_t* st;              // ncls_tiles x kClsStride status words
  uint32_t* err;
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
  uint32_t polls;            // look-back poll limit
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

// lengths of runs u0 .. u0+kClsItems-1 (0 past U) from their starts s (run
// u0 + e starts at s[e]; last: the start after them), run_start having U+1
// entries
__device__ __forceinline__ void run_lengths(const uint32_t* s, uint32_t last, uint64_t u0,
                                            uint32_t U, uint32_t* start, uint32_t* len) {
#pragma unroll
  for (int e = 0; e < kClsItems; ++e) {
    const uint32_t nxt = e + 1 < kClsItems ? s[e + 1] : last;
    start[e] = s[e];
    len[e] = (u0 + e < U) ? nxt - s[e] : 0u;
  }
}

__device__ __forceinline__ uint32_t bucket_of_key(const uint32_t* bkb, uint32_t nb, uint32_t key) {
  uint32_t b = 0;
  for (uint32_t i = 1; i < nb; ++i) b += (bkb[i] <= key) ? 1u : 0u;
  return b;
}

// Chunk placement.  A long run's nch chunks take list positions [cb, cb + nch),
// and the backward gives position c to a workgroup on XCD c mod 8 (each XCD has
// its own L2).  A long run's lookups are sorted by position, hence by bag, and
// spread over the bags, so chunk k reads grad_out rows of about the k/nch-th
// slice of the bags.  The positions of residue 0 (mod 8) take the first chunks,
// those of residue 1 the next ones, and so on: the chunks a residue class holds
// are consecutive, so XCD x reads about the x-th eighth of the bags for every
// long run of a table, and a run's partial sums stay contiguous.

constexpr uint32_t kHeavyChunks = 4096;

__global__ __launch_bounds__(kThreads) void classify_kernel(ClsDev a) {
  // dynamic LDS: the T key bases and table ids in key order (2 T words)
  extern __shared__ uint32_t s_dyn[];
  uint32_t* s_kb = s_dyn;
  uint32_t* s_ord = s_dyn + a.T;
  // the tile's single-lookup and tiny-run tasks, staged in list order and
  // written out with coalesced stores after the classification (written
  // straight from each thread's runs, most lanes of every store are masked
  // and the lines fill in pieces)
  __shared__ uint4 s_stage[kClsTile];
  __shared__ uint32_t s_bkb[kMaxBuckets + 1];
  __shared__ uint32_t sh4[4];
  __shared__ uint32_t s_tile;
  __shared__ uint32_t s_tot[kNumLists], s_excl[kNumLists];
  // one step's long runs: first chunk position, long index, table, first slot,
  // length, and the exclusive prefix of their chunk counts
  __shared__ uint32_t s_lr_pc[kThreads], s_lr_pl[kThreads], s_lr_t[kThreads];
  __shared__ uint32_t s_lr_st[kThreads], s_lr_ln[kThreads], s_lr_cb[kThreads + 1];
  const uint32_t U = a.counters[kCntU];
  // workgroups past the last run leave before taking a ticket, so the tickets
  // go to exactly the tiles that hold runs
  if ((uint64_t)blockIdx.x * kClsTile >= U) return;
  const uint32_t tile = take_ticket(a.ticket, &s_tile);
  const uint64_t tile0 = (uint64_t)tile * kClsTile;
  const uint64_t u0 = tile0 + (uint64_t)threadIdx.x * kClsItems;
  uint32_t start[kClsItems] = {}, len[kClsItems] = {}, key[kClsItems] = {}, bag0[kClsItems] = {};
  uint32_t keyprev = 0;
  const bool mine = u0 < U;
  if (mine) {
    // the run starts, keys, the next start and the key before, all in flight
    // together, then the lengths
    uint32_t s[kClsItems];
    loadn<kClsItems>(a.run_start, u0, (uint64_t)U + 1, s);
    loadn<kClsItems>(a.run_key, u0, U, key);
    const uint32_t last = a.run_start[(u0 + kClsItems <= U) ? u0 + kClsItems : U];
    keyprev = u0 == 0 ? 0u : a.run_key[u0 - 1];
    run_lengths(s, last, u0, U, start, len);
#pragma unroll
    for (int e = 0; e < kClsItems; ++e) bag0[e] = a.sorted_bag[start[e] < a.N ? start[e] : a.N - 1];
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
    for (int e = 0; e < kClsItems; ++e) {
      uint32_t c[kNumLists];
      run_class(len[e], c);
      const uint32_t in = (u0 + e < U) ? 1u : 0u;
      for (int q = 0; q < kNumLists; ++q) acc[q] += in * c[q];
    }
  }
  uint32_t pos[kNumLists];
  for (int q = 0; q < kNumLists; ++q) {
    uint32_t tot;
    pos[q] = block_excl_scan(acc[q], sh4, tot);
    if (threadIdx.x == 0) s_tot[q] = tot;
  }
  __syncthreads();
  // wave 0 looks back for lists 0-3 with 16 lanes each, wave 1 for list 4
  // with 64 lanes, at once (whole waves polling every list read more status
  // words per round trip than the coherent level serves quickly)
  {
    const uint32_t w = threadIdx.x / kWave;
    if (w == 0) {
      const uint32_t q = lane_id() / 16u;
      const uint32_t e = publish_and_look_back<16>(a.st, tile, kClsStride, q, s_tot[q], a.err,
                                                    a.polls);
      if ((lane_id() & 15u) == 0) s_excl[q] = e;
    } else if (w == 1) {
      const uint32_t e = publish_and_look_back<64>(a.st, tile, kClsStride, 4, s_tot[4], a.err,
                                                    a.polls);
      if (lane_id() == 0) s_excl[4] = e;
    }
  }
  static_assert(kNumLists == 5 && kThreads / kWave == 4, "list-to-wave map of the look-back");
  __syncthreads();
  const bool last_tile = tile0 + kClsTile >= U;
  if (last_tile) {
    // list totals, and the begins of every bucket after the last run's bucket
    if (threadIdx.x < (uint32_t)kNumLists)
      a.counters[kCntSingle + threadIdx.x] = s_excl[threadIdx.x] + s_tot[threadIdx.x];
    const int first = (int)bucket_of_key(s_bkb, a.nb, a.run_key[U - 1]) + 1;
    for (int b = first + (int)threadIdx.x; b <= (int)a.nb; b += kThreads)
      for (int q = 0; q < kNumLists; ++q)
        a.counters[kCntBegins + q * (a.nb + 1) + b] = s_excl[q] + s_tot[q];
  }
  if (mine)
    for (int q = 0; q < kNumLists; ++q) pos[q] += s_excl[q];
  const uint32_t ex0 = s_excl[0], ex1 = s_excl[1], tot0 = s_tot[0], tot1 = s_tot[1];
  int bprev = u0 == 0 ? -1 : (int)bucket_of_key(s_bkb, a.nb, keyprev);
  // Every thread takes every step (no early exit), so that each step's long
  // runs can be placed by the whole wave or workgroup.
  const bool heavy = s_tot[4] >= kHeavyChunks;  // uniform
#pragma unroll
  for (int e = 0; e < kClsItems; ++e) {
    const bool valid = mine && u0 + e < U;
    uint32_t lp_pc = 0xffffffffu, lp_pl = 0, lp_t = 0;  // this step's long run, if any
    const uint32_t k = key[e], ln = len[e], st = start[e];
    if (valid) {
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
        s_stage[pos[0] - ex0] = make_uint4(st, row, t, bag0[e]);
        ++pos[0];
      } else if (ln < (uint32_t)kTinyRun) {
        s_stage[tot0 + pos[1] - ex1] = make_uint4(st, ln, row, t);
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
        lp_pc = pc;  // its chunks are placed below, by the whole wave
        lp_pl = pl;
        lp_t = t;
        pos[4] += nch;
        ++pos[3];
      }
    }
    // Chunk placement (above): position cp of a run with positions
    // [pc, pc + nch) gets chunk number q, positions taken residue class by
    // residue class (x = 0..7), a class's in ascending order.  One thread per
    // run wrote 512 chunks of each of a table's 64 runs in 240 us; here a tile
    // with at least kHeavyChunks chunks places each step's long runs with the
    // whole workgroup (listed in LDS with the prefix of their chunk counts;
    // thread i takes chunks i, i + 256, ... and finds its run by binary
    // search), any other tile with the whole wave, one run at a time (no
    // barriers).
    const bool has = lp_pc != 0xffffffffu;
    if (!heavy) {
      uint64_t lm = __ballot(has);
      while (lm) {
        const uint32_t l = (uint32_t)__builtin_ctzll(lm);
        lm &= lm - 1;
        const uint32_t pc = (uint32_t)__shfl((int)lp_pc, (int)l, kWave);
        const uint32_t pl = (uint32_t)__shfl((int)lp_pl, (int)l, kWave);
        const uint32_t t = (uint32_t)__shfl((int)lp_t, (int)l, kWave);
        const uint32_t rst = (uint32_t)__shfl((int)st, (int)l, kWave);
        const uint32_t rln = (uint32_t)__shfl((int)ln, (int)l, kWave);
        const uint32_t nch = (rln + kChunk - 1) / kChunk;
        for (uint32_t cp = pc + lane_id(); cp < pc + nch; cp += kWave) {
          const uint32_t x = cp & 7u;
          uint32_t q = (cp - (pc + ((x - pc) & 7u))) / 8u;  // rank inside its class
          for (uint32_t xx = 0; xx < x; ++xx) {             // plus the earlier classes
            const uint32_t f = (xx - pc) & 7u;
            q += f < nch ? (nch - 1u - f) / 8u + 1u : 0u;
          }
          const uint32_t cl_len = (rln - q * kChunk) < (uint32_t)kChunk ? (rln - q * kChunk)
                                                                          : (uint32_t)kChunk;
          if (cp < a.max_chunks) a.chunk_task[cp] = make_uint4(rst + q * kChunk, cl_len, t, pl);
        }
      }
    } else if (__syncthreads_count(has) > 0) {  // uniform
      uint32_t nlr, nchunk;
      const uint32_t r = block_excl_scan(has ? 1u : 0u, sh4, nlr);
      const uint32_t my_nch = has ? (ln + kChunk - 1) / kChunk : 0u;
      const uint32_t cb = block_excl_scan(my_nch, sh4, nchunk);
      if (has) {
        s_lr_pc[r] = lp_pc;
        s_lr_pl[r] = lp_pl;
        s_lr_t[r] = lp_t;
        s_lr_st[r] = st;
        s_lr_ln[r] = ln;
        s_lr_cb[r] = cb;
      }
      if (threadIdx.x == 0) s_lr_cb[nlr] = nchunk;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < nchunk; i += kThreads) {
        uint32_t lo = 0, hi = nlr;  // s_lr_cb[lo] <= i < s_lr_cb[hi]
        while (hi - lo > 1) {
          const uint32_t mid = (lo + hi) >> 1;
          if (s_lr_cb[mid] <= i) lo = mid; else hi = mid;
        }
        const uint32_t pc = s_lr_pc[lo], rln = s_lr_ln[lo];
        const uint32_t nch = (rln + kChunk - 1) / kChunk;
        const uint32_t cp = pc + (i - s_lr_cb[lo]);
        const uint32_t x = cp & 7u;
        uint32_t q = (cp - (pc + ((x - pc) & 7u))) / 8u;  // rank inside its class
        for (uint32_t xx = 0; xx < x; ++xx) {             // plus the earlier classes
          const uint32_t f = (xx - pc) & 7u;
          q += f < nch ? (nch - 1u - f) / 8u + 1u : 0u;
        }
        const uint32_t cl_len = (rln - q * kChunk) < (uint32_t)kChunk ? (rln - q * kChunk)
                                                                        : (uint32_t)kChunk;
        if (cp < a.max_chunks)
          a.chunk_task[cp] = make_uint4(s_lr_st[lo] + q * kChunk, cl_len, s_lr_t[lo], s_lr_pl[lo]);
      }
      __syncthreads();  // the list is rewritten by the next step
    }
  }
  // singles at [0, tot0) and tiny runs at [tot0, tot0 + tot1) of the stage
  // (tot0 + tot1 <= the tile's runs <= kClsTile)
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < tot0; i += kThreads)
    if (ex0 + i < a.N) a.single_task[ex0 + i] = s_stage[i];
  for (uint32_t i = threadIdx.x; i < tot1; i += kThreads)
    if (ex1 + i < a.max_tiny) a.tiny_task[ex1 + i] = s_stage[tot0 + i];
}

// One radix pass of DB-bit digits: counts per tile, prefixes over tiles,
// scatter.
template <int DB>
void launch_sort_pass(const SortPass& sp, uint32_t* cnt, bool sc, uint32_t sgrid,
                      const uint32_t* ctl, uint64_t* st, uint64_t nst, hipStream_t s) {
  uint32_t* tex = const_cast<uint32_t*>(sp.tile_excl);
  uint32_t* totals = const_cast<uint32_t*>(sp.totals);
  TBE_LAUNCH("radix_upsweep", radix_upsweep<DB>, dim3(sgrid), dim3(kThreads), s, sp.kin, sp.seg,
             sp.tile_seg, ctl, sp.shift, cnt, sp.ntiles, st, nst);
  TBE_LAUNCH("radix_scan", radix_scan<DB>, dim3(1u << DB), dim3(kThreads), s, cnt, sp.ntiles, ctl,
             tex, totals);
  if (sc)
    TBE_LAUNCH("radix_downsweep", (sort_pass_kernel<DB, true>), dim3(sgrid), dim3(kThreads), s,
               sp);
  else
    TBE_LAUNCH("radix_downsweep", (sort_pass_kernel<DB, false>), dim3(sgrid), dim3(kThreads), s,
               sp);
}

// The first pass: counts from the lookups, prefixes, the scatter that forms
// its tiles from the lookups (the transposition).
template <int DB, typename IT>
void launch_first_pass(const SortPass& sp, const PrepDev& d, uint32_t* cnt, bool sc,
                       uint32_t sgrid, const uint32_t* ctl, uint64_t* st, uint64_t nst,
                       hipStream_t s) {
  uint32_t* tex = const_cast<uint32_t*>(sp.tile_excl);
  uint32_t* totals = const_cast<uint32_t*>(sp.totals);
  TBE_LAUNCH("radix_upsweep", (first_upsweep<IT, DB>), dim3(sgrid), dim3(kThreads), s, d,
             sp.tile_seg, ctl, cnt, sp.ntiles, st, nst);
  TBE_LAUNCH("radix_scan", radix_scan<DB>, dim3(1u << DB), dim3(kThreads), s, cnt, sp.ntiles, ctl,
             tex, totals);
  if (sc)
    TBE_LAUNCH("transpose", (transpose_scatter_kernel<DB, true, IT>), dim3(sgrid), dim3(kThreads), s,
               sp);
  else
    TBE_LAUNCH("transpose", (transpose_scatter_kernel<DB, false, IT>), dim3(sgrid), dim3(kThreads),
               s, sp);
}

}  // namespace

hipError_t launch_preprocess(const PrepArgs& p, int /*num_cus*/, hipStream_t s) {
  const WsLayout& L = *p.L;
  if (p.N == 0) return hipSuccess;
  uint8_t* ws = p.ws;
  auto u32p = [&](size_t off) { return reinterpret_cast<uint32_t*>(ws + off); };
  auto f32p = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  auto u64p = [&](size_t off) { return reinterpret_cast<uint64_t*>(ws + off); };
  uint32_t* ctl = u32p(L.ctl);
  uint32_t* err = ctl + kCtlErr;
  const bool sc = p.need_scale != 0;
  const uint32_t polls = knob_wait_polls();

  uint4* seg = reinterpret_cast<uint4*>(ws + L.seg);
  uint32_t* tile_seg = u32p(L.tile_seg);
  uint32_t* totals = u32p(L.totals);
  uint2* seg2 = reinterpret_cast<uint2*>(ws + L.seg2);
  PrepDev d{p.tables, p.T, p.nb, p.B, p.indices, p.offsets, p.psw, p.N, p.tseg, seg, seg2};
  uint32_t* bag0 = u32p(L.tile_bag0);
  {
    // at least four bags per thread, at most 1024 workgroups
    const uint64_t nbag = (uint64_t)p.T * (uint64_t)p.B;
    const uint32_t mgrid = (uint32_t)std::min<uint64_t>(1024, std::max<uint64_t>(1, nbag / 1024));
    const size_t mshm = 4 * sizeof(uint32_t) * (size_t)p.T;
    if (p.itype == IT_I32)
      TBE_LAUNCH_SHM("tile_map", tile_map_kernel<int32_t>, dim3(mgrid), dim3(kThreads), mshm, s,
                     d, p.order, seg, seg2, tile_seg, bag0, L.ntiles_max, ctl);
    else
      TBE_LAUNCH_SHM("tile_map", tile_map_kernel<int64_t>, dim3(mgrid), dim3(kThreads), mshm, s,
                     d, p.order, seg, seg2, tile_seg, bag0, L.ntiles_max, ctl);
  }

  // pass 0 forms its tiles from the lookups and writes the b buffers; then
  // ping-pong b -> a -> b ..., so the final buffers are b for an odd pass count
  const uint64_t nst = (L.st_end - L.st_rle) / 8;
  const uint32_t sgrid = 8u * ((L.ntiles_max + 7u) / 8u);  // xcd_tile(): a multiple of 8
  uint32_t* cnt = u32p(L.tile_cnt);
  for (int pass = 0; pass < L.npass; ++pass) {
    const bool ab = (pass % 2) == 0;
    SortPass sp{u32p(ab ? L.key_a : L.key_b), u32p(ab ? L.val_a : L.val_b),
                f32p(ab ? L.sc_a : L.sc_b),   u32p(ab ? L.key_b : L.key_a),
                u32p(ab ? L.val_b : L.val_a), f32p(ab ? L.sc_b : L.sc_a),
                (uint32_t)(pass * L.digit_bits), seg, tile_seg, ctl + kCtlTiles,
                totals, u32p(L.tile_excl), L.ntiles_max,
                p.indices, p.offsets, p.psw, p.tables, seg2, bag0, p.B, p.N, p.T};
    if (pass == 0) {
      if (L.digit_bits == 8) {
        if (p.itype == IT_I32) launch_first_pass<8, int32_t>(sp, d, cnt, sc, sgrid, ctl, u64p(L.st_rle), nst, s);
        else launch_first_pass<8, int64_t>(sp, d, cnt, sc, sgrid, ctl, u64p(L.st_rle), nst, s);
      } else {
        if (p.itype == IT_I32) launch_first_pass<10, int32_t>(sp, d, cnt, sc, sgrid, ctl, u64p(L.st_rle), nst, s);
        else launch_first_pass<10, int64_t>(sp, d, cnt, sc, sgrid, ctl, u64p(L.st_rle), nst, s);
      }
    } else if (L.digit_bits == 8) {
      launch_sort_pass<8>(sp, cnt, sc, sgrid, ctl, u64p(L.st_rle), 0, s);
    } else {
      launch_sort_pass<10>(sp, cnt, sc, sgrid, ctl, u64p(L.st_rle), 0, s);
    }
  }
  const uint32_t* skey = u32p(L.final_in_b ? L.key_b : L.key_a);
  const uint32_t* sbag = u32p(L.final_in_b ? L.val_b : L.val_a);
  if (L.rle_groups == (uint32_t)kRleGroupsDeep)
    TBE_LAUNCH("rle", rle_kernel<kRleGroupsDeep>, dim3(L.nrle_tiles), dim3(kThreads), s, skey, p.N, L.nrle_tiles,
             ctl + kCtlRleTickets, u64p(L.st_rle), err, u32p(L.counters),
             u32p(L.run_start), u32p(L.run_key), polls);
  else
    TBE_LAUNCH("rle", rle_kernel<1>, dim3(L.nrle_tiles), dim3(kThreads), s, skey, p.N, L.nrle_tiles,
             ctl + kCtlRleTickets, u64p(L.st_rle), err, u32p(L.counters),
             u32p(L.run_start), u32p(L.run_key), polls);

  ClsDev c{u32p(L.run_start), u32p(L.run_key), sbag, u32p(L.counters),
           ctl + kCtlClsTickets, u64p(L.st_cls), err,
           reinterpret_cast<uint4*>(ws + L.single_task), reinterpret_cast<uint4*>(ws + L.tiny_task),
           reinterpret_cast<uint4*>(ws + L.med_task),
           reinterpret_cast<uint4*>(ws + L.long_task), u32p(L.long_cbeg), u32p(L.remaining),
           reinterpret_cast<uint4*>(ws + L.chunk_task), p.tables, p.order, p.bucket_key_begin,
           p.T, p.nb, p.N, L.max_tiny, L.max_med, L.max_long, L.max_chunks, polls};
  TBE_LAUNCH_SHM("classify", classify_kernel, dim3(L.ncls_tiles), dim3(kThreads),
                 2 * sizeof(uint32_t) * (size_t)p.T, s, c);
  return hipGetLastError();
}

}  // namespace tbe
