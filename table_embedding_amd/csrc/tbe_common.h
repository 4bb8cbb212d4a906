// Internal declarations shared by the HIP sources of libtbe_hip.so.
// Device descriptors, storage-format helpers, wave64 subgroup reductions and
// the host-side launchers each kernel file provides to the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace tbe {

constexpr int kThreads = 256;       // every kernel runs 256-thread workgroups (4 waves)
constexpr int kWave = 64;
constexpr int kTile = 4096;         // keys per workgroup in the sort / run-length passes
constexpr int kClsTile = 2048;      // runs per workgroup in the classification pass
// 4096-key groups per run-length tile: four from kRleDeepLookups lookups on
// (the look-back chain a quarter as long), else one (more workgroups).
// Measured on MI355X (run-length pass per step, four groups / one): 2.1 M
// lookups 11.6 / 10.7 us, 17 M 32.6 / 45.5 us.
constexpr int kRleGroupsDeep = 4;
// Workspace arrays start and end on multiples of this many bytes (each one's
// size is rounded up), so a 64-byte vector load of an aligned group that
// starts inside an array ends inside it.
constexpr size_t kWsAlign = 256;
constexpr int64_t kRleDeepLookups = 8ll << 20;
// Lookup counts from which the backward gathers keep eight lookups in flight
// and streams its weight rows past the caches (see bwd.hip for the
// measurements behind both).
constexpr int64_t kBwdDeepLookups = 64ll << 20;
constexpr int64_t kBwdStreamRowsLookups = 1ll << 20;
// Polls after which a look-back wait of the preprocessing gives up.
constexpr uint32_t kSpinLimit = 1u << 20;
// Lookup count from which the backward updates the hottest long runs by the
// hot-row contraction (bwd_dense.hip).
constexpr int64_t kDenseMinLookups = 8ll << 20;

// Test knobs (tbe_test_knob): process-wide overrides of the thresholds above
// and of the poll limit, so that small inputs can run the variants that
// deep batches take.  Each accessor returns the override if one is set,
// else the default.
int64_t knob_rle_deep_lookups();
int64_t knob_bwd_deep_lookups();
int64_t knob_bwd_stream_lookups();
uint32_t knob_wait_polls();
int64_t knob_dense_lookups();

constexpr int kLongRun = 256;       // SL >= 256 takes the chunked long-run path
constexpr int kTinyRun = 32;        // short runs below this are owned by a lane subgroup
constexpr int kChunk = 256;         // lookups per long-run chunk
constexpr int kRadixMaxBits = 10;  // widest radix digit (1024 values)
constexpr int kMaxPass = 4;         // 32-bit rows: at most four 8-bit digits
constexpr int kMaxTables = 4096;
// grad_out larger than this (the MALL) takes the bag-ordered chunk walk
constexpr uint64_t kChunkOrderMinGradBytes = 256ull << 20;

enum : int { WD_F32 = 0, WD_F16 = 1, WD_BF16 = 2 };
enum : int { IT_I32 = 0, IT_I64 = 1 };
enum : int { POOL_SUM = 0, POOL_MEAN = 1 };
enum : int { OPT_ROWWISE_ADAGRAD = 0, OPT_ADAGRAD = 1, OPT_SGD = 2 };

// Per-table descriptor, one array of T entries in device memory.
struct TableDev {
  void* w;            // weights, rows x dim, row-major, storage type of the plan
  float* m;           // row-wise Adagrad momentum, rows
  uint32_t dim;       // D_t
  uint32_t pooling;   // POOL_SUM / POOL_MEAN
  uint32_t col;       // first column of the table in out / grad_out rows
  uint32_t key_base;  // first linear row key of the table (tables ordered by bucket, then t)
  uint32_t rows;      // R_t
  uint32_t bucket;    // bucket id (tables bucketed by next_pow2(D))
};

// Lane mapping of one bucket: a row of up to `width` columns is covered by
// `lpr` lanes, each holding `nc` chunks of `vec` consecutive columns.
struct BucketDev {
  const uint32_t* tables;  // table ids of this bucket, ascending
  uint32_t ntables;
  uint32_t lpr;            // lanes per row, power of two <= 64
  uint32_t lpr_log2;
};

constexpr int kMaxBuckets = 9;  // next_pow2 widths 4 .. 1024

// Buckets that share one kernel instantiation are served by one launch:
// workgroups [gbeg[k], gbeg[k+1]) work on bucket id[k] with lane mapping bk[k].
struct BucketSet {
  uint32_t n;
  uint32_t gbeg[kMaxBuckets + 1];
  uint32_t id[kMaxBuckets];
  BucketDev bk[kMaxBuckets];
};

// This workgroup's bucket, its index inside the bucket's range and the range
// size.  The ranges are ascending, so a chain of selects that takes every
// range starting at or before this workgroup ends on its own; no element is
// picked by a computed index (which would send the argument block through
// scratch memory).
__device__ __forceinline__ void set_pick(const BucketSet& S, BucketDev& bk, uint32_t& id,
                                         uint32_t& lb, uint32_t& lg) {
  bk = S.bk[0];
  id = S.id[0];
  uint32_t g0 = S.gbeg[0], g1 = S.gbeg[1];
#pragma unroll
  for (int i = 1; i < kMaxBuckets; ++i) {
    const bool take = i < (int)S.n && blockIdx.x >= S.gbeg[i];
    bk.tables = take ? S.bk[i].tables : bk.tables;
    bk.ntables = take ? S.bk[i].ntables : bk.ntables;
    bk.lpr = take ? S.bk[i].lpr : bk.lpr;
    bk.lpr_log2 = take ? S.bk[i].lpr_log2 : bk.lpr_log2;
    id = take ? S.id[i] : id;
    g0 = take ? S.gbeg[i] : g0;
    g1 = take ? S.gbeg[i + 1] : g1;
  }
  lb = blockIdx.x - g0;
  lg = g1 - g0;
}

// Workspace layout: byte offsets from the workspace base (all 256-B aligned).
struct WsLayout {
  size_t key_a, key_b, val_a, val_b, sc_a, sc_b;  // sort ping-pong: key, bag id, scale
  size_t ctl;                                      // control block, kCtlWords uint32
  size_t seg;       // T uint4 {lookups, output base, first tile, key base}, tables in key order
  size_t seg2;      // T uint2 {first position O[t*B], table t}, the same order
  size_t tile_seg;  // ntiles_max uint32: segment of each sort tile
  size_t tile_bag0;  // ntiles_max uint32: bag of each sort tile's first lookup
  size_t totals;    // 2^digit_bits digit totals of the current pass
  size_t tile_cnt;   // 2^digit_bits x ntiles_max per-tile digit counts of the current pass
                     // (digit-major)
  size_t tile_excl;  // their exclusive prefixes over all tiles (tile-major)
  // look-back status words (uint64), contiguous in [st_rle, st_end): the
  // run-length pass (nrle_tiles) and the classification pass (ncls_tiles x
  // kClsStride)
  size_t st_rle, st_cls, st_end;
  size_t run_start, run_key;
  size_t single_task, tiny_task, med_task, long_task, long_cbeg, remaining, chunk_task;
  size_t partial, counters;
  size_t chunk_perm;  // max_chunks uint32: chunk list position taken at each walk position
  size_t hist_part, hist_cnt;  // histogram backward: partial rows and row counts (or 0 bytes)
  size_t hist_save, hist_hdr;  // row counts per bag saved by the histogram forward, {B, N}
  size_t long_flag, dense_rows, dense_cnt, dense_part;  // hot-row contraction (or 0 bytes)
  bool dense;  // the contraction's regions are present (the plan and N allow it)
  size_t total;
  uint32_t ntiles;          // ceil(N / kTile)
  uint32_t nrle_tiles;      // ceil(N / (rle_groups * kTile)): tiles of the run-length pass
  uint32_t rle_groups;      // 4096-key groups per run-length tile (1 or kRleGroupsDeep)
  uint32_t ntiles_max;      // ceil(N / kTile) + T: bound on the sort tiles of the segments
  uint32_t ncls_tiles;      // ceil(N / kClsTile): runs are at most N
  uint32_t max_tiny;        // capacity of the 2 <= SL < 32 list
  uint32_t max_med;         // capacity of the medium short-run list
  uint32_t max_long;        // capacity of the long-run lists
  uint32_t max_chunks;      // capacity of the chunk list
  uint32_t pstride;         // floats per partial row
  int npass;                // radix passes
  int digit_bits;           // bits per radix digit: 8 or 10
  int final_in_b;           // sorted keys end in key_b/val_b
};

// Counter block: [U, n_tiny, n_medium, n_long, n_chunks, then per list k the
// nb+1 bucket begins at kCntBegins + k*(nb+1)]
// lists: short runs with SL = 1, 2 <= SL < 32, 32 <= SL < 256; long runs; chunks
constexpr int kNumLists = 5;
constexpr int kCntU = 0, kCntSingle = 1, kCntBegins = 1 + kNumLists;

// Control block of the preprocessing: the look-back error flag, the number
// of sort tiles of the segments, and the tile tickets of the run-length and
// classification passes: eight counters each (one per workgroup index mod 8),
// 128 bytes apart.
constexpr int kCtlErr = 8, kCtlTiles = 9;
constexpr int kTicketStride = 32;
constexpr int kCtlRleTickets = 32;
constexpr int kCtlClsTickets = kCtlRleTickets + 8 * kTicketStride;
constexpr int kCtlWords = kCtlClsTickets + 8 * kTicketStride;
constexpr int kClsStride = 8;  // status words per classification tile (five used)

// ------------------------------------------------------------- device helpers

__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}
// round-to-nearest-even float -> binary16 bits
__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// round-to-nearest-even float -> bfloat16 bits (NaN stays a quiet NaN)
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16 or 8 bytes at p, as words; NT: a non-temporal (streaming) access, which
// the caches keep with low priority (for rows read and rewritten once, so that
// they do not push out data that is reused).  A compile-time choice: with a
// run-time one the compiler merges the two loads of one address and drops the
// hint.
// (the pointer is cast to the global address space: a generic pointer would
// give a flat access, which waits on two counters)
typedef __attribute__((address_space(1))) u32x4_t g_u32x4_t;
typedef __attribute__((address_space(1))) u32x2_t g_u32x2_t;
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  const g_u32x4_t* q = (const g_u32x4_t*)p;
  if constexpr (NT) return __builtin_nontemporal_load(q); else return *q;
}
template <bool NT>
__device__ __forceinline__ u32x2_t ld8(const void* p) {
  const g_u32x2_t* q = (const g_u32x2_t*)p;
  if constexpr (NT) return __builtin_nontemporal_load(q); else return *q;
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, u32x4_t x) {
  g_u32x4_t* q = (g_u32x4_t*)p;
  if constexpr (NT) __builtin_nontemporal_store(x, q); else *q = x;
}
template <bool NT>
__device__ __forceinline__ void st8(void* p, u32x2_t x) {
  g_u32x2_t* q = (g_u32x2_t*)p;
  if constexpr (NT) __builtin_nontemporal_store(x, q); else *q = x;
}

// Load VEC consecutive weights starting at element e of a row-major table
// (NT: see ld16).
template <int WD, int VEC, bool NT = false>
__device__ __forceinline__ void load_w(const void* w, int64_t e, float* v) {
  if constexpr (WD == WD_F32) {
    static_assert(VEC == 4, "f32 rows are read 4 at a time");
    const u32x4_t x = ld16<NT>(reinterpret_cast<const float*>(w) + e);
    // components to scalars first (see load_w_buf)
    const uint32_t c[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(float, c[i]);
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + e;
    uint32_t words[VEC / 2];
    if constexpr (VEC == 8) {
      const u32x4_t x = ld16<NT>(p);
      words[0] = x.x; words[1] = x.y; words[2] = x.z; words[3] = x.w;
    } else {
      const u32x2_t x = ld8<NT>(p);
      words[0] = x.x; words[1] = x.y;
    }
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      if constexpr (WD == WD_F16) {
        v[2 * i] = f16_bits_to_float(words[i] & 0xffffu);
        v[2 * i + 1] = f16_bits_to_float(words[i] >> 16);
      } else {
        v[2 * i] = bf16_bits_to_float(words[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_float(words[i] >> 16);
      }
    }
  }
}

// Buffer loads: a 32-bit byte offset per lane against a base held in scalar
// registers (a buffer descriptor) instead of a 64-bit address per lane, which
// saves address registers and 64-bit arithmetic in the gather loops; a read at
// or past `bytes` returns zeros instead of faulting.  The descriptor's fourth
// dword for a raw gfx9 buffer selects the 32-bit data format.
constexpr int kBufDword3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufDword3);
}
__device__ __forceinline__ uint32_t buf_u32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
// load_w through a buffer descriptor: VEC weights at byte offset byte_off.
template <int WD, int VEC>
__device__ __forceinline__ void load_w_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, float* v) {
  if constexpr (WD == WD_F32) {
    static_assert(VEC == 4, "f32 rows are read 4 at a time");
    const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    // components to scalars first: a bit cast of a vector element expression
    // (x.y) reads component 0 with this compiler
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(float, w[i]);
  } else {
    uint32_t words[VEC / 2];
    if constexpr (VEC == 8) {
      const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
      words[0] = x.x; words[1] = x.y; words[2] = x.z; words[3] = x.w;
    } else {
      const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
      words[0] = x.x; words[1] = x.y;
    }
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      if constexpr (WD == WD_F16) {
        v[2 * i] = f16_bits_to_float(words[i] & 0xffffu);
        v[2 * i + 1] = f16_bits_to_float(words[i] >> 16);
      } else {
        v[2 * i] = bf16_bits_to_float(words[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_float(words[i] >> 16);
      }
    }
  }
}

// load_w in two steps: the raw words of VEC weights (VEC for float32 rows,
// VEC / 2 for 16-bit ones), then their conversion to float.  A caller that
// keeps loads in flight behind a scheduling barrier converts after it, so
// that no conversion makes the wave wait for its load before the barrier.
template <int WD, int VEC>
struct RawW {
  uint32_t u[WD == WD_F32 ? VEC : VEC / 2];
};
template <int WD, int VEC, bool NT = false>
__device__ __forceinline__ void load_w_raw(const void* w, int64_t e, RawW<WD, VEC>& r) {
  if constexpr (WD == WD_F32) {
    static_assert(VEC == 4, "f32 rows are read 4 at a time");
    const u32x4_t x = ld16<NT>(reinterpret_cast<const float*>(w) + e);
    r.u[0] = x.x; r.u[1] = x.y; r.u[2] = x.z; r.u[3] = x.w;
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(w) + e;
    if constexpr (VEC == 8) {
      const u32x4_t x = ld16<NT>(p);
      r.u[0] = x.x; r.u[1] = x.y; r.u[2] = x.z; r.u[3] = x.w;
    } else {
      const u32x2_t x = ld8<NT>(p);
      r.u[0] = x.x; r.u[1] = x.y;
    }
  }
}
template <int WD, int VEC>
__device__ __forceinline__ void cvt_w(const RawW<WD, VEC>& r, float* v) {
  if constexpr (WD == WD_F32) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = __builtin_bit_cast(float, r.u[i]);
  } else {
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      if constexpr (WD == WD_F16) {
        v[2 * i] = f16_bits_to_float(r.u[i] & 0xffffu);
        v[2 * i + 1] = f16_bits_to_float(r.u[i] >> 16);
      } else {
        v[2 * i] = bf16_bits_to_float(r.u[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_float(r.u[i] >> 16);
      }
    }
  }
}

// Store VEC floats, rounded to the storage type, at element e (NT: see ld16).
template <int WD, int VEC, bool NT = false>
__device__ __forceinline__ void store_w(void* w, int64_t e, const float* v) {
  if constexpr (WD == WD_F32) {
    const u32x4_t x = {__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                       __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
    st16<NT>(reinterpret_cast<float*>(w) + e, x);
  } else {
    uint32_t words[VEC / 2];
#pragma unroll
    for (int i = 0; i < VEC / 2; ++i) {
      uint32_t lo, hi;
      if constexpr (WD == WD_F16) {
        lo = float_to_f16_bits(v[2 * i]);
        hi = float_to_f16_bits(v[2 * i + 1]);
      } else {
        lo = float_to_bf16_bits(v[2 * i]);
        hi = float_to_bf16_bits(v[2 * i + 1]);
      }
      words[i] = lo | (hi << 16);
    }
    uint16_t* p = reinterpret_cast<uint16_t*>(w) + e;
    if constexpr (VEC == 8)
      st16<NT>(p, (u32x4_t){words[0], words[1], words[2], words[3]});
    else
      st8<NT>(p, (u32x2_t){words[0], words[1]});
  }
}

// Float rows and scalars in device (global) memory: every pointer these take
// points into global memory, and saying so keeps pointers that come out of
// table descriptors (momentum, optimizer state) from becoming flat accesses.
template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float* v) {
#pragma unroll
  for (int i = 0; i < VEC; i += 4) {
    const u32x4_t x = ld16<false>(p + i);
    const uint32_t c[4] = {x.x, x.y, x.z, x.w};  // components to scalars first
#pragma unroll
    for (int e = 0; e < 4; ++e) v[i + e] = __builtin_bit_cast(float, c[e]);
  }
}
template <int VEC>
__device__ __forceinline__ void store_f32(float* p, const float* v) {
#pragma unroll
  for (int i = 0; i < VEC; i += 4)
    st16<false>(p + i, (u32x4_t){__builtin_bit_cast(uint32_t, v[i]),
                                 __builtin_bit_cast(uint32_t, v[i + 1]),
                                 __builtin_bit_cast(uint32_t, v[i + 2]),
                                 __builtin_bit_cast(uint32_t, v[i + 3])});
}
__device__ __forceinline__ float gload(const float* p) {
  return *(const __attribute__((address_space(1))) float*)p;
}
__device__ __forceinline__ void gstore(float* p, float v) {
  *(__attribute__((address_space(1))) float*)p = v;
}

__device__ __forceinline__ int64_t load_idx(const void* a, int itype, int64_t i) {
  return itype == IT_I32 ? (int64_t)reinterpret_cast<const int32_t*>(a)[i]
                         : reinterpret_cast<const int64_t*>(a)[i];
}

// Sum over the `lpr` lanes of a subgroup (lpr a power of two, subgroups aligned).
__device__ __forceinline__ float subgroup_sum(float v, uint32_t lpr) {
  for (uint32_t m = 1; m < lpr; m <<= 1) v += __shfl_xor(v, (int)m, kWave);
  return v;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & (kWave - 1); }

// LDS visibility inside one wave: every lane's stores before any lane's loads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------------ host launchers

// Optional per-kernel timing (tbe_prof_enable): when on, prof_events hands
// out a start/stop event pair and the launch goes through
// hipExtLaunchKernelGGL, which ties the two events to the dispatch's own
// begin and end timestamps (no events enqueued around it).
bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop);

#define TBE_LAUNCH_SHM(name, kernel, grid, block, shm, stream, ...)                        \
  do {                                                                                     \
    hipEvent_t tbe_prof_e0_ = nullptr, tbe_prof_e1_ = nullptr;                             \
    if (::tbe::prof_events((name), &tbe_prof_e0_, &tbe_prof_e1_))                          \
      hipExtLaunchKernelGGL(kernel, (grid), (block), (shm), (stream), tbe_prof_e0_,        \
                            tbe_prof_e1_, 0u, ##__VA_ARGS__);                              \
    else                                                                                   \
      hipLaunchKernelGGL(kernel, (grid), (block), (shm), (stream), ##__VA_ARGS__);         \
  } while (0)
#define TBE_LAUNCH(name, kernel, grid, block, stream, ...) \
  TBE_LAUNCH_SHM(name, kernel, grid, block, 0u, stream, ##__VA_ARGS__)

// Forward: bags per wave.  A wave owns this many consecutive bags of one
// table and splits them among its 64/lpr lane subgroups into contiguous runs
// of whole bags with about equal lookup counts (about `bps` bags per
// subgroup, at most 64 per wave: one offset per lane).  A bucket whose rows
// take all 64 lanes (one subgroup per wave) keeps one bag per wave.
__host__ __device__ inline uint32_t fwd_group_bags(uint32_t lpr, uint32_t bps) {
  const uint32_t nsub = (uint32_t)kWave / lpr;
  if (nsub <= 1u) return 1u;
  const uint32_t g = nsub * bps;
  return g < (uint32_t)kWave ? g : (uint32_t)kWave;
}

struct FwdArgs {
  const TableDev* tables;
  int64_t B;
  int itype;
  const void* indices;
  const void* offsets;
  const float* psw;
  float* out;
  uint32_t dtot;
  uint32_t bps;    // generic forward: bags per lane subgroup in a wave's group (1 .. 4)
  uint32_t split;  // 1: the group's lookups split evenly over its subgroups; 0: one bag each
  uint32_t n;      // lookups N (the equal-piece split needs N * index bytes < 2^32)
  uint32_t T;      // tables
  uint32_t* err;   // nullable: check offsets and indices as they are read (error block of
                   // kValWords words, cleared before the launch)
  uint16_t* hist_save;  // nullable: histogram path, each bag's row counts (B x E) written here
  uint32_t* hist_hdr;   // with hist_save: {B, N} of the batch whose counts are saved
};

struct PrepArgs {
  const TableDev* tables;
  const uint32_t* bucket_key_begin;  // nb+1 linear key bounds of the buckets
  const uint32_t* order;             // table ids in ascending key_base order
  uint32_t T, nb;
  int64_t B;
  int itype;
  const void* indices;
  const void* offsets;
  const float* psw;                  // nullable per-sample weights
  int need_scale;                    // per-sample weights or a mean table: scale per lookup
  uint32_t N;
  uint8_t* ws;
  const WsLayout* L;                 // host pointer (layout), kernels get offsets by value
  const uint32_t* tseg;              // segment (position in key order) of each table
};

struct BwdArgs {
  const TableDev* tables;
  int64_t B;
  int itype;
  const void* offsets;
  const float* psw;
  const float* grad;
  uint32_t dtot;
  float lr, eps;
  int opt;                      // OPT_ROWWISE_ADAGRAD / OPT_ADAGRAD (element-wise) / OPT_SGD
  const uint32_t* sorted_bag;   // bag id of each sorted lookup
  const float* sorted_scale;    // nullable: S[p] * (1/L if mean) of each sorted lookup
  const uint4* single_task;
  const uint4* tiny_task;
  const uint4* med_task;
  const uint4* long_task;
  const uint32_t* long_cbeg;
  uint32_t* remaining;
  const uint4* chunk_task;
  uint32_t* chunk_perm;         // nullable: walk order of the chunk list (identity if null)
  float* partial;
  uint32_t pstride;
  const uint32_t* counters;
  uint32_t nb;
  uint32_t* debug_count;     // nullable, per linear key
  const uint32_t* prep_err;  // the preprocessing's error flag: nonzero, nothing is written
  uint32_t N, T;             // lookups and tables (task sanity bounds)
  uint32_t max_single, max_tiny, max_med, max_long, max_chunks;  // list capacities
  // hot-row contraction (null / 0 when off): see bwd_dense.hip
  const void* indices;       // the batch's indices (the contraction reads them in bag order)
  uint32_t* long_flag;       // per long run: 1 if its row is updated by the contraction
  uint4* dense_rows;         // T x kDenseRows {start, len, row, long index} of each table's hot rows
  uint32_t* dense_cnt;       // T: hot rows per table
  float* dense_part;         // T x kDenseRows x dense_w partial rows of kDensePitch floats
  uint32_t dense_w;          // workgroups per table and column group of the contraction
  uint32_t dense_ncg;        // column groups of the contraction (128 columns each)
  uint32_t dense_min_len;    // smallest run length the contraction takes
};

// Hot-row contraction of the long runs: per table, up to kDenseRows long runs
// of at least dense_min_len lookups (tables with D a multiple of 16 and at
// most kDensePitch columns), their gradients as one counts x grad_out
// contraction over the table's bags on the matrix cores.
constexpr int kDenseRows = 128;
constexpr int kDensePitch = 256;

// Histogram-reuse backward of a plan with one table of at most 64 rows and
// D <= 128, D a multiple of 16.
struct HistArgs {
  TableDev table;
  int64_t B;
  const void* indices;
  const void* offsets;
  const float* psw;       // nullable
  const float* grad;
  uint32_t dtot, col;     // grad_out row stride and the table's first column
  uint32_t N, E, D;
  int mean;
  float lr, eps;
  float* part;            // nwg x E partial rows of pstride floats
  uint32_t* pcnt;         // nwg x E lookup counts
  const uint16_t* saved;  // nullable: row counts per bag saved by the histogram forward
  const uint32_t* saved_hdr;  // {B, N} of the saved counts (used only if they match)
  uint32_t pstride, nwg;
  uint32_t* debug_count;  // nullable, per linear key
};
constexpr uint32_t kHistMaxWorkgroups = 1024;

// Input validation (tbe_validate): error block words and bits.
constexpr int kValWords = 4;
constexpr int kValBits = 0, kValBadIndices = 1, kValFirstBag = 2, kValFirstPos = 3;
constexpr uint32_t kValOffsetStart = 0x1u, kValOffsetEnd = 0x2u, kValOffsetOrder = 0x4u,
                   kValOffsetRange = 0x8u, kValIndexRange = 0x10u;
struct ValArgs {
  const TableDev* tables;
  uint32_t T;
  int64_t B;
  void* indices;
  void* offsets;
  int64_t N;
};
hipError_t launch_validate(const ValArgs& v, int itype, uint32_t* err, bool repair,
                           hipStream_t s);
// The error block to its empty state (no finding; first bag and position
// 0xffffffff), by a one-workgroup kernel.
hipError_t launch_validate_clear(uint32_t* err, hipStream_t s);

// One forward launch for the buckets of S (S.gbeg filled: bags of bucket k
// over workgroups [gbeg[k], gbeg[k+1])).
hipError_t launch_forward_set(const FwdArgs& a, const BucketSet& S, int wd, int vec, int nc,
                              hipStream_t s);
hipError_t launch_forward_hist(const FwdArgs& a, uint32_t E, uint32_t D, int mean, int grid,
                               hipStream_t s);
hipError_t launch_preprocess(const PrepArgs& a, int num_cus, hipStream_t s);
// Most workgroups each backward kernel of one bucket can use (upper bounds
// from host-known sizes); launches clamp them to the co-resident capacity.
struct BwdGrids {
  uint32_t single, tiny, medium, chunk, longrun;
};

// One launch per backward kernel for the buckets of S (S.gbeg is filled here
// from the per-bucket grids g[0 .. S.n-1]).
// Streams of the backward: short runs of one lane subgroup (SL < 32) on
// s[0], medium runs on s[1], chunks and long-run updates on s[2] (all three
// may be the same stream).
hipError_t launch_backward_set(const BwdArgs& a, BucketSet S, const BwdGrids* g, int wd, int vec,
                               int nc, bool fused, int num_cus, const hipStream_t* s);
hipError_t launch_backward_hist(const HistArgs& h, int itype, int wd, hipStream_t s);
// Orders each (table, XCD residue) class of the chunk list by the bag of the
// chunks' first lookups into a.chunk_perm (no-op when a.chunk_perm is null).
hipError_t launch_chunk_order(const BwdArgs& a, hipStream_t s);
// The hot-row contraction (a.long_flag set): selection of each table's hot
// rows (tseg: segment of each table in key order), the contraction's
// partials, and the rows' update (optimizer a.opt, weight storage wd).
hipError_t launch_dense(const BwdArgs& a, const uint32_t* tseg, int wd, int itype,
                        hipStream_t s);
// The update of each hot row from its partials (in bwd.hip, beside the other
// row updates).
hipError_t launch_dense_update(const BwdArgs& a, int wd, hipStream_t s);

}  // namespace tbe
