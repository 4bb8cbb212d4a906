// C-ABI layer of libtbe_hip.so (declared in include/tbe.h): plan metadata,
// workspace layout, host-side argument checks and the launch sequences of
// forward, preprocessing and backward.  Every check happens before anything
// is enqueued; nothing here reads device memory back or synchronizes, except
// plan creation, which uploads a few KB of metadata.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/tbe.h"
#include "tbe_common.h"

using namespace tbe;

// Static workspace of tbe_backward_rowwise_adagrad_noalloc, for callers that
// cannot allocate device memory.  One array per device, held from the
// library's first plan on that device until the process ends; every call on a
// device shares it.  In host code `scratch` only names the array: its device
// address comes from hipGetSymbolAddress, once per device, at plan creation
// (static_ws_of_current_device), and only that address is ever used.
constexpr size_t kStaticWsBytes = 256ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticWsBytes];
static_assert(kStaticWsBytes == TBE_STATIC_WS_BYTES, "static workspace size of the header");

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_static_ws_mu;
void* g_static_ws[kMaxDevices] = {};

// The device address of `scratch` on the current device (resolved on the
// first call for that device).
int static_ws_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TBE_E_HIP;
  std::lock_guard<std::mutex> lk(g_static_ws_mu);
  if (!g_static_ws[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TBE_E_HIP;
    g_static_ws[dev] = p;
  }
  *out = g_static_ws[dev];
  return TBE_OK;
}

struct Bucket {
  uint32_t width;  // next_pow2(D) of its tables
  int vec, nc;
  uint32_t lpr, lpr_log2;
  std::vector<uint32_t> tables;
  uint32_t* d_tables;
};

}  // namespace

struct tbe_plan {
  int32_t T;
  int wdtype;
  std::vector<int64_t> rows;
  std::vector<int32_t> dims, pooling;
  std::vector<uint32_t> key_base, col;
  uint32_t dtot;
  uint64_t sum_rows;
  int row_bits;  // bits of the largest table's row range: the radix passes sort rows
  std::vector<Bucket> buckets;
  uint32_t pstride;
  TableDev* d_tables;
  std::vector<TableDev> h_tables;  // host copy of the table descriptors
  uint32_t* d_order;
  uint32_t* d_tseg;
  uint32_t* d_bkb;
  void* d_mem;
  int num_cus;
  int dense_on;   // hot-row contraction: 1 if some table can take it
  int dense_ncg;  // and its column groups of 128 columns
  int dense_w;    // and workgroups per table and column group (bag ranges)
  // backward fork/join: two default-priority side streams and their events;
  // the lock keeps the record/wait sequence of one call from interleaving
  // with another call's on the same plan
  hipStream_t side[2];
  hipEvent_t ev_fork, ev_join[2];
  mutable std::mutex mu;
};

namespace {

constexpr size_t kAlign = kWsAlign;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

uint32_t next_pow2(uint32_t x) {
  uint32_t p = 1;
  while (p < x) p <<= 1;
  return p;
}

// smallest l with 2^l >= x
int ilog2(uint64_t x) {
  int l = 0;
  while ((1ull << l) < x) ++l;
  return l;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Plans the histogram-reuse backward serves: one table of at most 64 rows,
// D a multiple of 16 up to 128.
bool bwd_hist_capable(const tbe_plan* P) {
  return P->T == 1 && P->rows[0] <= 64 && P->dims[0] % 16 == 0 && P->dims[0] <= 128;
}

// The hot-row contraction: workgroups per table, and the most tables a plan
// may have for it (its partials take T x 1 MiB of workspace).
// Workgroups of the contraction per table (bag ranges): at least 16, and
// together at least kDenseMinWgs, so that a plan of few tables still fills
// the chip.
constexpr int kDenseWgsPerTable = 16;
constexpr int kDenseMinWgs = 512;
constexpr int kDenseMaxTables = 128;

// TBE_BWD_CONCURRENT_AUTO forks the run classes below this many lookups.
// Measured on MI355X (ms per step, one stream / three): 2.1 M lookups 0.333 /
// 0.326, 17 M 2.100 / 1.995, 138 M 16.49 / 19.01 (there the classes compete
// for the last-level cache).
constexpr int64_t kConcurrentMaxLookups = 64ll << 20;

WsLayout layout(const tbe_plan* P, int64_t N) {
  WsLayout L{};
  const uint64_t n = (uint64_t)N;
  L.ntiles = (uint32_t)((n + kTile - 1) / kTile);
  L.rle_groups = N >= knob_rle_deep_lookups() ? (uint32_t)kRleGroupsDeep : 1u;
  L.nrle_tiles = (uint32_t)((n + (uint64_t)L.rle_groups * kTile - 1) / ((uint64_t)L.rle_groups * kTile));
  L.ncls_tiles = (uint32_t)((n + kClsTile - 1) / kClsTile);
  L.max_tiny = (uint32_t)(n / 2 + 1);
  L.max_med = (uint32_t)(n / kTinyRun + 1);
  L.max_long = (uint32_t)(n / kLongRun + 1);
  L.max_chunks = (uint32_t)(n / kChunk + L.max_long + 1);
  L.pstride = P->pstride;
  L.ntiles_max = L.ntiles + (uint32_t)P->T;
  // the fewest passes of at most 10-bit digits, then the narrower digit (8
  // or 10 bits) that covers the row range in that many passes: the count
  // tables and the scatter's LDS grow with 2^digit_bits.  Measured on MI355X
  // (ms per step): 20 row bits in two 10-bit passes instead of three 8-bit
  // ones 0.337 -> 0.332; 21 bits in two 11-bit passes instead of three 8-bit
  // ones 2.104 -> 2.175 (the count and prefix passes cost more than the
  // saved scatter), hence at most 10 bits.
  {
    const int bits = std::max(1, P->row_bits);
    const int np = (bits + kRadixMaxBits - 1) / kRadixMaxBits;
    const int w = (bits + np - 1) / np;
    L.digit_bits = w <= 8 ? 8 : 10;
    L.npass = (bits + L.digit_bits - 1) / L.digit_bits;
  }
  L.final_in_b = L.npass % 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes ? bytes : 1);
    return o;
  };
  L.key_a = take(n * 4);
  L.key_b = take(n * 4);
  L.val_a = take(n * 4);
  L.val_b = take(n * 4);
  L.sc_a = take(n * 4);
  L.sc_b = take(n * 4);
  L.ctl = take((size_t)kCtlWords * 4);
  L.seg = take((size_t)P->T * 16);
  L.seg2 = take((size_t)P->T * 8);
  L.tile_seg = take((size_t)L.ntiles_max * 4);
  L.tile_bag0 = take((size_t)L.ntiles_max * 4);
  L.totals = take(((size_t)1 << L.digit_bits) * 4);
  L.tile_cnt = take(((size_t)1 << L.digit_bits) * L.ntiles_max * 4);
  L.tile_excl = take(((size_t)1 << L.digit_bits) * L.ntiles_max * 4);
  L.st_rle = off;
  L.st_cls = L.st_rle + (size_t)L.nrle_tiles * 8;
  L.st_end = L.st_cls + (size_t)L.ncls_tiles * kClsStride * 8;
  take(L.st_end - L.st_rle);
  L.run_start = take((n + 1) * 4);
  L.run_key = take(n * 4);
  L.single_task = take(n * 16);
  L.tiny_task = take((size_t)L.max_tiny * 16);
  L.med_task = take((size_t)L.max_med * 16);
  L.long_task = take((size_t)L.max_long * 16);
  L.long_cbeg = take((size_t)L.max_long * 4);
  L.remaining = take((size_t)L.max_long * 4);
  L.chunk_task = take((size_t)L.max_chunks * 16);
  L.partial = take((size_t)L.max_chunks * L.pstride * 4);
  L.counters = take((size_t)(kCntBegins + kNumLists * (P->buckets.size() + 1)) * 4);
  L.chunk_perm = take((size_t)L.max_chunks * 4);
  const bool hc = bwd_hist_capable(P);
  L.hist_part = take(hc ? (size_t)kHistMaxWorkgroups * 64 * L.pstride * 4 : 0);
  L.hist_cnt = take(hc ? (size_t)kHistMaxWorkgroups * 64 * 4 : 0);
  // saved counts: B x E uint16 with B <= N / 64 (the histogram forward needs an
  // average bag length of 64) and E <= 64, so at most 2 N + 128 bytes
  L.hist_save = take(hc ? 2 * n + 128 : 0);
  L.hist_hdr = take(hc ? 16 : 0);
  // the hot-row contraction's lists, for batches large enough to take it
  // (the same lookup threshold as the backward's; with a smaller batch the
  // regions are empty and the backward never takes the contraction)
  const bool dc = P->dense_on && N >= knob_dense_lookups();
  L.dense = dc;
  L.long_flag = take(dc ? (size_t)L.max_long * 4 : 0);
  L.dense_rows = take(dc ? (size_t)P->T * kDenseRows * 16 : 0);
  L.dense_cnt = take(dc ? (size_t)P->T * 4 : 0);
  L.dense_part = take(dc ? (size_t)P->T * kDenseRows * P->dense_w * kDensePitch * 4 : 0);
  L.total = off;
  return L;
}

// Shared checks of the per-call lookup arguments.
int check_lookups(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                  const void* offsets, int64_t N) {
  if (!P || B < 0 || N < 0) return TBE_E_ARG;
  if (itype != TBE_I32 && itype != TBE_I64) return TBE_E_ARG;
  const size_t isz = itype == TBE_I32 ? 4 : 8;
  if (!offsets || !aligned(offsets, isz)) return TBE_E_ARG;
  if (N > 0 && (!indices || !aligned(indices, isz))) return TBE_E_ARG;
  if ((uint64_t)P->T * (uint64_t)B >= (1ull << 32) - 1) return TBE_E_RANGE;
  if (N >= (int64_t)(1ll << 31) - 1) return TBE_E_RANGE;
  if (itype == TBE_I32 && P->sum_rows >= (1ull << 31)) return TBE_E_RANGE;
  return TBE_OK;
}

int check_ws(const tbe_plan* P, int64_t N, const void* ws, size_t ws_bytes) {
  if (!ws || !aligned(ws, kAlign)) return TBE_E_WORKSPACE;
  if (ws_bytes < layout(P, N).total) return TBE_E_WORKSPACE;
  return TBE_OK;
}

bool hist_eligible(const tbe_plan* P, int64_t B, int64_t N, const float* psw) {
  return P->T == 1 && P->rows[0] <= 64 && P->dims[0] >= 64 && P->dims[0] <= 128 &&
         P->wdtype == TBE_F16 && psw == nullptr && B > 0 && N >= 64 * B;
}

// Bags per lane subgroup of the generic forward (the wave's group holds
// 64/lpr * bps consecutive bags whose lookups its subgroups split evenly).
// More bags per wave even out more but leave fewer waves; measured on MI355X
// (forward alone): 8 tables x 8192 bags, 48 waves per CU with one bag per
// subgroup: bps 1 / 2 / 4 = 47.3 / 48.8 / 49.5 us; 16 x 16384 bags, ~200
// waves per CU: 538 / 512 / 518 us; 64 x 65536 bags, 4096 waves per CU:
// 3271 / 2905 / 2827 us.
constexpr uint64_t kFwdTwoBagsWavesPerCu = 64;
constexpr uint64_t kFwdFourBagsWavesPerCu = 1024;
uint32_t fwd_bags_per_subgroup(const tbe_plan* P, int64_t B) {
  uint64_t waves = 0;  // with one bag per subgroup
  for (const Bucket& bk : P->buckets) {
    const uint64_t nsub = (uint64_t)kWave / bk.lpr;
    waves += (uint64_t)bk.tables.size() * (((uint64_t)B + nsub - 1) / nsub);
  }
  const uint64_t cus = (uint64_t)P->num_cus;
  return waves >= kFwdFourBagsWavesPerCu * cus ? 4u : waves >= kFwdTwoBagsWavesPerCu * cus ? 2u : 1u;
}

// The equal-piece forward reads rows and indices with 32-bit byte offsets:
// every table and the index array under 4 GiB (else one bag per subgroup).
bool fwd_split_fits(const tbe_plan* P, int64_t N, int32_t itype) {
  const uint64_t es = P->wdtype == TBE_F32 ? 4 : 2;
  const uint64_t lim = 1ull << 32;
  if ((uint64_t)N * (itype == TBE_I64 ? 8u : 4u) >= lim) return false;
  for (int t = 0; t < P->T; ++t)
    if ((uint64_t)P->rows[t] * (uint64_t)P->dims[t] * es >= lim) return false;
  return true;
}

bool any_mean(const tbe_plan* P) {
  for (int32_t p : P->pooling)
    if (p == TBE_MEAN) return true;
  return false;
}

// Buckets that share one kernel instantiation (vec, nc), in bucket order.
std::vector<std::vector<uint32_t>> bucket_groups(const tbe_plan* P) {
  std::vector<std::vector<uint32_t>> groups;
  for (uint32_t b = 0; b < P->buckets.size(); ++b) {
    bool placed = false;
    for (auto& g : groups) {
      const Bucket& h = P->buckets[g[0]];
      if (h.vec == P->buckets[b].vec && h.nc == P->buckets[b].nc) {
        g.push_back(b);
        placed = true;
        break;
      }
    }
    if (!placed) groups.push_back({b});
  }
  return groups;
}

BucketSet bucket_set(const tbe_plan* P, const std::vector<uint32_t>& grp) {
  BucketSet S{};
  S.n = (uint32_t)grp.size();
  for (uint32_t k = 0; k < S.n; ++k) {
    const Bucket& bk = P->buckets[grp[k]];
    S.bk[k] = BucketDev{bk.d_tables, (uint32_t)bk.tables.size(), bk.lpr, bk.lpr_log2};
    S.id[k] = grp[k];
  }
  return S;
}

PrepArgs prep_args(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                   const void* offsets, int64_t N, const float* psw, void* ws,
                   const WsLayout* L) {
  PrepArgs a{};
  a.tables = P->d_tables;
  a.bucket_key_begin = P->d_bkb;
  a.order = P->d_order;
  a.T = (uint32_t)P->T;
  a.nb = (uint32_t)P->buckets.size();
  a.B = B;
  a.itype = itype;
  a.indices = indices;
  a.offsets = offsets;
  a.psw = psw;
  a.need_scale = (psw != nullptr || any_mean(P)) ? 1 : 0;
  a.N = (uint32_t)N;
  a.ws = reinterpret_cast<uint8_t*>(ws);
  a.L = L;
  a.tseg = P->d_tseg;
  return a;
}

// ------------------------------------------------------------ kernel timing

struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};

__global__ void empty_kernel() {}

std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace tbe {

namespace {
// test knob overrides; a negative value means "not set"
std::atomic<int64_t> g_knob_rle_deep{-1}, g_knob_bwd_deep{-1}, g_knob_bwd_stream{-1},
    g_knob_polls{-1}, g_knob_dense{-1};
int64_t knob_or(const std::atomic<int64_t>& k, int64_t dflt) {
  const int64_t v = k.load(std::memory_order_relaxed);
  return v < 0 ? dflt : v;
}
}  // namespace

int64_t knob_rle_deep_lookups() { return knob_or(g_knob_rle_deep, kRleDeepLookups); }
int64_t knob_bwd_deep_lookups() { return knob_or(g_knob_bwd_deep, kBwdDeepLookups); }
int64_t knob_bwd_stream_lookups() { return knob_or(g_knob_bwd_stream, kBwdStreamRowsLookups); }
int64_t knob_dense_lookups() { return knob_or(g_knob_dense, kDenseMinLookups); }
uint32_t knob_wait_polls() {
  const int64_t v = knob_or(g_knob_polls, kSpinLimit);
  return v > (int64_t)0xffffffffll ? 0xffffffffu : (uint32_t)v;
}

bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return false;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r{name, prof_event(), prof_event()};
  if (!r.start || !r.stop) return false;
  g_prof_recs.push_back(r);
  *start = r.start;
  *stop = r.stop;
  return true;
}

}  // namespace tbe

extern "C" {

int tbe_test_knob(int32_t knob, int64_t value) {
  std::atomic<int64_t>* k = nullptr;
  switch (knob) {
    case TBE_KNOB_RLE_DEEP_LOOKUPS: k = &tbe::g_knob_rle_deep; break;
    case TBE_KNOB_BWD_DEEP_LOOKUPS: k = &tbe::g_knob_bwd_deep; break;
    case TBE_KNOB_BWD_STREAM_LOOKUPS: k = &tbe::g_knob_bwd_stream; break;
    case TBE_KNOB_WAIT_POLLS: k = &tbe::g_knob_polls; break;
    case TBE_KNOB_DENSE_LOOKUPS: k = &tbe::g_knob_dense; break;
    default: return TBE_E_ARG;
  }
  k->store(value < 0 ? -1 : value, std::memory_order_relaxed);
  return TBE_OK;
}

int tbe_prof_enable(int enable) {
  g_prof_on.store(enable != 0);
  return TBE_OK;
}

int tbe_prof_read(int32_t max_kernels, char* names, int64_t* launches, double* total_ms,
                  int32_t* count) {
  if (max_kernels < 0 || !count || (max_kernels > 0 && (!names || !launches || !total_ms)))
    return TBE_E_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<const char*> keys;
  std::vector<int64_t> n;
  std::vector<double> ms;
  int rc = TBE_OK;
  for (ProfRec& r : g_prof_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      rc = TBE_E_HIP;
    size_t k = 0;
    while (k < keys.size() && std::strcmp(keys[k], r.name) != 0) ++k;
    if (k == keys.size()) {
      keys.push_back(r.name);
      n.push_back(0);
      ms.push_back(0.0);
    }
    n[k] += 1;
    ms[k] += (double)t;
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
  const int m = std::min<int>((int)keys.size(), max_kernels);
  for (int k = 0; k < m; ++k) {
    std::strncpy(names + (size_t)k * TBE_PROF_NAME_LEN, keys[k], TBE_PROF_NAME_LEN - 1);
    names[(size_t)k * TBE_PROF_NAME_LEN + TBE_PROF_NAME_LEN - 1] = 0;
    launches[k] = n[k];
    total_ms[k] = ms[k];
  }
  *count = (int32_t)keys.size();
  return rc;
}

int tbe_prof_calibrate(int32_t launches, void* stream) {
  if (launches < 0) return TBE_E_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int32_t i = 0; i < launches; ++i)
    TBE_LAUNCH("empty", empty_kernel, dim3(1), dim3(64), s);
  return hipGetLastError() == hipSuccess ? TBE_OK : TBE_E_HIP;
}

const char* tbe_status_string(int s) {
  switch (s) {
    case TBE_OK: return "ok";
    case TBE_E_ARG: return "invalid argument";
    case TBE_E_UNSUPPORTED: return "unsupported shape or option";
    case TBE_E_WORKSPACE: return "workspace too small or misaligned";
    case TBE_E_RANGE: return "size or index range too large for the index type";
    case TBE_E_HIP: return "HIP runtime error";
    case TBE_E_ALLOC: return "allocation failed";
    case TBE_E_TOO_LARGE: return "batch too large for the library's static workspace";
  }
  return "unknown status";
}

int tbe_plan_create(tbe_plan** out, int32_t T, const int64_t* rows, const int32_t* dims,
                    const int32_t* pooling, int32_t wdtype, void* const* weights,
                    float* const* momentum) {
  if (!out) return TBE_E_ARG;
  *out = nullptr;
  if (T < 1 || !rows || !dims || !pooling || !weights || !momentum) return TBE_E_ARG;
  if (wdtype != TBE_F32 && wdtype != TBE_F16 && wdtype != TBE_BF16) return TBE_E_ARG;
  if (T > kMaxTables) return TBE_E_UNSUPPORTED;
  uint64_t sum_rows = 0, dtot = 0;
  for (int t = 0; t < T; ++t) {
    if (pooling[t] != TBE_SUM && pooling[t] != TBE_MEAN) return TBE_E_ARG;
    if (!weights[t] || !aligned(weights[t], 16) || !momentum[t] || !aligned(momentum[t], 4))
      return TBE_E_ARG;
    if (rows[t] < 1) return TBE_E_UNSUPPORTED;
    if (dims[t] < 4 || dims[t] > 1024 || dims[t] % 4) return TBE_E_UNSUPPORTED;
    sum_rows += (uint64_t)rows[t];
    dtot += (uint64_t)dims[t];
    if (sum_rows >= (1ull << 32)) return TBE_E_RANGE;
  }
  tbe_plan* P = new (std::nothrow) tbe_plan();
  if (!P) return TBE_E_ALLOC;
  P->T = T;
  P->wdtype = wdtype;
  P->rows.assign(rows, rows + T);
  P->dims.assign(dims, dims + T);
  P->pooling.assign(pooling, pooling + T);
  P->sum_rows = sum_rows;
  P->dtot = (uint32_t)dtot;
  P->row_bits = 0;
  for (int t = 0; t < T; ++t) P->row_bits = std::max(P->row_bits, ilog2((uint64_t)rows[t]));
  {  // hot-row contraction: tables with D a multiple of 16 up to kDensePitch
    int dmax = 0;
    for (int t = 0; t < T; ++t)
      if (dims[t] % 16 == 0 && dims[t] <= kDensePitch) dmax = std::max(dmax, (int)dims[t]);
    P->dense_on = (T > kDenseMaxTables || dmax == 0) ? 0 : 1;
    P->dense_ncg = dmax > 128 ? 2 : 1;
    P->dense_w = std::max(kDenseWgsPerTable, kDenseMinWgs / std::max(1, (int)T));
  }

  // buckets by next_pow2(D), ascending width; tables keep ascending id inside a bucket
  std::vector<uint32_t> widths;
  for (int t = 0; t < T; ++t) widths.push_back(next_pow2((uint32_t)dims[t]));
  std::vector<uint32_t> uw = widths;
  std::sort(uw.begin(), uw.end());
  uw.erase(std::unique(uw.begin(), uw.end()), uw.end());
  P->pstride = 0;
  for (uint32_t w : uw) {
    Bucket bk{};
    bk.width = w;
    bool all8 = wdtype != TBE_F32 && w >= 8;
    for (int t = 0; t < T; ++t)
      if (widths[t] == w) {
        bk.tables.push_back((uint32_t)t);
        if (dims[t] % 8) all8 = false;
      }
    bk.vec = all8 ? 8 : 4;
    const uint32_t lanes = w / (uint32_t)bk.vec;
    bk.lpr = std::min<uint32_t>(lanes, kWave);
    bk.nc = (int)(lanes / bk.lpr);
    bk.lpr_log2 = (uint32_t)ilog2(bk.lpr);
    P->pstride = std::max(P->pstride, w);
    P->buckets.push_back(bk);
  }
  // linear keys: tables in bucket order, then id
  std::vector<uint32_t> order;
  for (auto& bk : P->buckets) order.insert(order.end(), bk.tables.begin(), bk.tables.end());
  P->key_base.assign(T, 0);
  P->col.assign(T, 0);
  {
    uint64_t kb = 0;
    for (uint32_t t : order) {
      P->key_base[t] = (uint32_t)kb;
      kb += (uint64_t)rows[t];
    }
    uint32_t c = 0;
    for (int t = 0; t < T; ++t) {
      P->col[t] = c;
      c += (uint32_t)dims[t];
    }
  }
  std::vector<TableDev> td(T);
  for (int t = 0; t < T; ++t) {
    td[t].w = weights[t];
    td[t].m = momentum[t];
    td[t].dim = (uint32_t)dims[t];
    td[t].pooling = (uint32_t)pooling[t];
    td[t].col = P->col[t];
    td[t].key_base = P->key_base[t];
    td[t].rows = (uint32_t)rows[t];
  }
  const uint32_t nb = (uint32_t)P->buckets.size();
  std::vector<uint32_t> bkb(nb + 1);
  for (uint32_t b = 0; b < nb; ++b) {
    bkb[b] = P->key_base[P->buckets[b].tables[0]];
    for (uint32_t t : P->buckets[b].tables) td[t].bucket = b;
  }
  bkb[nb] = (uint32_t)std::min<uint64_t>(sum_rows, 0xffffffffull);
  P->h_tables = td;

  // segment of each table: its position in key order
  std::vector<uint32_t> tseg(T);
  for (uint32_t s = 0; s < (uint32_t)T; ++s) tseg[order[s]] = s;

  // one device allocation: tables | order | segments | bucket key bounds | bucket table lists
  const size_t sz_td = align_up(sizeof(TableDev) * T);
  const size_t sz_order = align_up(4 * (size_t)T);
  const size_t sz_tseg = align_up(4 * (size_t)T);
  const size_t sz_bkb = align_up(4 * (size_t)(nb + 1));
  const size_t sz_lists = align_up(4 * (size_t)T);
  void* mem = nullptr;
  if (hipMalloc(&mem, sz_td + sz_order + sz_tseg + sz_bkb + sz_lists) != hipSuccess) {
    delete P;
    return TBE_E_ALLOC;
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(mem);
  P->d_mem = mem;
  P->d_tables = reinterpret_cast<TableDev*>(base);
  P->d_order = reinterpret_cast<uint32_t*>(base + sz_td);
  P->d_tseg = reinterpret_cast<uint32_t*>(base + sz_td + sz_order);
  P->d_bkb = reinterpret_cast<uint32_t*>(base + sz_td + sz_order + sz_tseg);
  uint32_t* lists = reinterpret_cast<uint32_t*>(base + sz_td + sz_order + sz_tseg + sz_bkb);
  bool ok = hipMemcpy(P->d_tables, td.data(), sizeof(TableDev) * T, hipMemcpyHostToDevice) ==
                hipSuccess &&
            hipMemcpy(P->d_order, order.data(), 4 * (size_t)T, hipMemcpyHostToDevice) ==
                hipSuccess &&
            hipMemcpy(P->d_tseg, tseg.data(), 4 * (size_t)T, hipMemcpyHostToDevice) ==
                hipSuccess &&
            hipMemcpy(P->d_bkb, bkb.data(), 4 * (size_t)(nb + 1), hipMemcpyHostToDevice) ==
                hipSuccess &&
            hipMemcpy(lists, order.data(), 4 * (size_t)T, hipMemcpyHostToDevice) == hipSuccess;
  size_t pos = 0;
  for (auto& bk : P->buckets) {
    bk.d_tables = lists + pos;
    pos += bk.tables.size();
  }
  int dev = 0, cus = 0;
  ok = ok && hipGetDevice(&dev) == hipSuccess &&
       hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  P->num_cus = cus > 0 ? cus : 256;
  {  // the static workspace's address on this device, so that the no-alloc
     // backward never loads anything at call time
    void* sw = nullptr;
    ok = ok && static_ws_of_current_device(&sw) == TBE_OK;
  }
  P->side[0] = P->side[1] = nullptr;
  P->ev_fork = P->ev_join[0] = P->ev_join[1] = nullptr;
  for (int i = 0; i < 2 && ok; ++i)
    ok = hipStreamCreateWithFlags(&P->side[i], hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&P->ev_join[i], hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&P->ev_fork, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    (void)tbe_plan_destroy(P);
    return TBE_E_HIP;
  }
  *out = P;
  return TBE_OK;
}

int tbe_plan_destroy(tbe_plan* P) {
  if (!P) return TBE_OK;
  bool ok = hipFree(P->d_mem) == hipSuccess;
  for (int i = 0; i < 2; ++i) {
    if (P->side[i]) ok = hipStreamDestroy(P->side[i]) == hipSuccess && ok;
    if (P->ev_join[i]) ok = hipEventDestroy(P->ev_join[i]) == hipSuccess && ok;
  }
  if (P->ev_fork) ok = hipEventDestroy(P->ev_fork) == hipSuccess && ok;
  delete P;
  return ok ? TBE_OK : TBE_E_HIP;
}

int tbe_plan_key_bases(const tbe_plan* P, int64_t* key_base) {
  if (!P || !key_base) return TBE_E_ARG;
  for (int t = 0; t < P->T; ++t) key_base[t] = (int64_t)P->key_base[t];
  return TBE_OK;
}

int tbe_workspace_size(const tbe_plan* P, int64_t B, int64_t N, size_t* bytes) {
  if (!P || !bytes || B < 0 || N < 0) return TBE_E_ARG;
  if (N >= (int64_t)(1ll << 31) - 1) return TBE_E_RANGE;
  *bytes = layout(P, N).total;
  return TBE_OK;
}

int tbe_workspace_views(const tbe_plan* P, int64_t B, int64_t N, tbe_ws_views* v) {
  if (!P || !v || B < 0 || N < 0) return TBE_E_ARG;
  if (N >= (int64_t)(1ll << 31) - 1) return TBE_E_RANGE;
  const WsLayout L = layout(P, N);
  v->sorted_key = L.final_in_b ? L.key_b : L.key_a;
  v->sorted_bag = L.final_in_b ? L.val_b : L.val_a;
  v->sorted_scale = L.final_in_b ? L.sc_b : L.sc_a;
  v->run_start = L.run_start;
  v->run_key = L.run_key;
  v->single_task = L.single_task;
  v->tiny_task = L.tiny_task;
  v->medium_task = L.med_task;
  v->long_task = L.long_task;
  v->long_cbeg = L.long_cbeg;
  v->chunk_task = L.chunk_task;
  v->chunk_perm = L.chunk_perm;
  v->counters = L.counters;
  v->prep_error = L.ctl + (size_t)kCtlErr * 4;
  v->hist_counts = L.hist_save;
  v->long_flag = L.long_flag;
  v->dense_rows = L.dense_rows;
  v->dense_count = L.dense_cnt;
  v->total = L.total;
  v->num_buckets = (int32_t)P->buckets.size();
  return TBE_OK;
}

namespace {
// Arguments of tbe_forward (TBE_OK or the error code).
int check_forward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                  const void* offsets, int64_t N, const float* psw, float* out, uint32_t flags) {
  int rc = check_lookups(P, B, itype, indices, offsets, N);
  if (rc) return rc;
  if (flags & ~(TBE_FWD_NO_HIST | TBE_FWD_REQUIRE_HIST | TBE_FWD_BALANCE | TBE_FWD_NO_BALANCE))
    return TBE_E_ARG;
  if ((flags & TBE_FWD_NO_HIST) && (flags & TBE_FWD_REQUIRE_HIST)) return TBE_E_ARG;
  if ((flags & TBE_FWD_BALANCE) && (flags & TBE_FWD_NO_BALANCE)) return TBE_E_ARG;
  if (B > 0 && (!out || !aligned(out, 16))) return TBE_E_ARG;
  if (psw && !aligned(psw, 4)) return TBE_E_ARG;
  if ((flags & TBE_FWD_REQUIRE_HIST) && !hist_eligible(P, B, N, psw)) return TBE_E_UNSUPPORTED;
  return TBE_OK;
}

// The forward's launches on s (arguments already checked).
// err: the error block of the checked forward (the generic kernels' CHK
// variant, never the histogram path), or null.
int launch_forward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                   const void* offsets, int64_t N, const float* psw, float* out, uint32_t flags,
                   hipStream_t s, uint32_t* err = nullptr, uint16_t* hist_save = nullptr,
                   uint32_t* hist_hdr = nullptr) {
  const bool hist = !err && hist_eligible(P, B, N, psw);
  if (B == 0) return TBE_OK;
  FwdArgs a{P->d_tables, B, itype, indices, offsets, psw, out, P->dtot, 1u};
  a.T = (uint32_t)P->T;
  a.n = (uint32_t)N;
  a.err = err;
  a.hist_save = hist ? hist_save : nullptr;
  a.hist_hdr = hist_hdr;
  hipError_t e = hipSuccess;
  if (hist && !(flags & TBE_FWD_NO_HIST)) {
    e = launch_forward_hist(a, (uint32_t)P->rows[0], (uint32_t)P->dims[0],
                            P->pooling[0] == TBE_MEAN, P->num_cus * 4, s);
  } else {
    a.split = (flags & TBE_FWD_NO_BALANCE) || !fwd_split_fits(P, N, itype) ? 0u : 1u;
    a.n = (uint32_t)N;
    a.bps = a.split ? fwd_bags_per_subgroup(P, B) : 1u;
    for (const auto& grp : bucket_groups(P)) {
      BucketSet S = bucket_set(P, grp);
      S.gbeg[0] = 0;
      for (uint32_t k = 0; k < S.n; ++k) {
        // one wave per group of fwd_group_bags(lpr, bps) consecutive bags of a table
        const uint64_t G = fwd_group_bags(S.bk[k].lpr, a.bps);
        const uint64_t waves = (uint64_t)S.bk[k].ntables * (((uint64_t)B + G - 1) / G);
        const uint64_t per_block = kThreads / kWave;
        S.gbeg[k + 1] = S.gbeg[k] + (uint32_t)((waves + per_block - 1) / per_block);
      }
      for (uint32_t k = S.n + 1; k <= (uint32_t)kMaxBuckets; ++k) S.gbeg[k] = S.gbeg[S.n];
      const Bucket& b0 = P->buckets[grp[0]];
      e = launch_forward_set(a, S, P->wdtype, b0.vec, b0.nc, s);
      if (e != hipSuccess) break;
    }
  }
  return e == hipSuccess ? TBE_OK : TBE_E_HIP;
}
}  // namespace

int tbe_forward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                const void* offsets, int64_t N, const float* psw, float* out, uint32_t flags,
                void* stream) {
  const int rc = check_forward(P, B, itype, indices, offsets, N, psw, out, flags);
  if (rc) return rc;
  return launch_forward(P, B, itype, indices, offsets, N, psw, out, flags,
                        reinterpret_cast<hipStream_t>(stream));
}

int tbe_forward_checked(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                        const void* offsets, int64_t N, const float* psw, float* out,
                        uint32_t flags, uint32_t* err, void* stream) {
  if (flags & TBE_FWD_REQUIRE_HIST) return TBE_E_UNSUPPORTED;  // the checks are in the generic path
  const int rc = check_forward(P, B, itype, indices, offsets, N, psw, out, flags);
  if (rc) return rc;
  if (!err || !aligned(err, 4)) return TBE_E_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (launch_validate_clear(err, s) != hipSuccess) return TBE_E_HIP;
  return launch_forward(P, B, itype, indices, offsets, N, psw, out, flags, s, err);
}

int tbe_forward_preprocess(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                           const void* offsets, int64_t N, const float* psw, float* out,
                           uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  const bool save = (flags & TBE_FWD_SAVE_HIST) != 0;
  flags &= ~TBE_FWD_SAVE_HIST;
  int rc = check_forward(P, B, itype, indices, offsets, N, psw, out, flags);
  if (rc) return rc;
  rc = check_ws(P, N, ws, ws_bytes);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (save) {
    // the histogram forward keeps its row counts for the histogram backward,
    // which needs nothing else: no run preprocessing
    if ((flags & TBE_FWD_NO_HIST) || !hist_eligible(P, B, N, psw) || !bwd_hist_capable(P))
      return TBE_E_UNSUPPORTED;
    const WsLayout L = layout(P, N);
    uint8_t* w = reinterpret_cast<uint8_t*>(ws);
    return launch_forward(P, B, itype, indices, offsets, N, psw, out, flags, s, nullptr,
                          reinterpret_cast<uint16_t*>(w + L.hist_save),
                          reinterpret_cast<uint32_t*>(w + L.hist_hdr));
  }
  if (N == 0) return launch_forward(P, B, itype, indices, offsets, N, psw, out, flags, s);
  // fork before the forward, so that the side stream waits for the work
  // before it, not for it; the forward is enqueued first (one launch), then
  // the preprocessing's launches on the side stream; `s` joins at the end
  std::lock_guard<std::mutex> lk(P->mu);
  hipStream_t side = P->side[0];
  if (hipEventRecord(P->ev_fork, s) != hipSuccess ||
      hipStreamWaitEvent(side, P->ev_fork, 0) != hipSuccess)
    return TBE_E_HIP;
  rc = launch_forward(P, B, itype, indices, offsets, N, psw, out, flags, s);
  const WsLayout L = layout(P, N);
  PrepArgs a = prep_args(P, B, itype, indices, offsets, N, psw, ws, &L);
  if (launch_preprocess(a, P->num_cus, side) != hipSuccess && rc == TBE_OK) rc = TBE_E_HIP;
  // join even after a failed launch, so `s` never runs ahead of the side stream
  if (hipEventRecord(P->ev_join[0], side) != hipSuccess ||
      hipStreamWaitEvent(s, P->ev_join[0], 0) != hipSuccess)
    rc = TBE_E_HIP;
  return rc;
}

int tbe_validate(const tbe_plan* P, int64_t B, int32_t itype, void* indices, void* offsets,
                 int64_t N, uint32_t* err, uint32_t flags, void* stream) {
  static_assert(kValWords == TBE_VALIDATE_WORDS && kValOffsetStart == TBE_INVALID_OFFSET_START &&
                    kValOffsetEnd == TBE_INVALID_OFFSET_END &&
                    kValOffsetOrder == TBE_INVALID_OFFSET_ORDER &&
                    kValOffsetRange == TBE_INVALID_OFFSET_RANGE &&
                    kValIndexRange == TBE_INVALID_INDEX,
                "validation words and bits of the header");
  int rc = check_lookups(P, B, itype, indices, offsets, N);
  if (rc) return rc;
  if (!err || !aligned(err, 4)) return TBE_E_ARG;
  if (flags & ~TBE_VALIDATE_REPAIR) return TBE_E_ARG;
  ValArgs v{P->d_tables, (uint32_t)P->T, B, indices, offsets, N};
  const hipError_t e = launch_validate(v, itype, err, (flags & TBE_VALIDATE_REPAIR) != 0,
                                       reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? TBE_OK : TBE_E_HIP;
}

int tbe_preprocess(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                   const void* offsets, int64_t N, const float* psw, void* ws, size_t ws_bytes,
                   void* stream) {
  int rc = check_lookups(P, B, itype, indices, offsets, N);
  if (rc) return rc;
  rc = check_ws(P, N, ws, ws_bytes);
  if (rc) return rc;
  if (psw && !aligned(psw, 4)) return TBE_E_ARG;
  if (N == 0) return TBE_OK;
  const WsLayout L = layout(P, N);
  PrepArgs a = prep_args(P, B, itype, indices, offsets, N, psw, ws, &L);
  const hipError_t e =
      launch_preprocess(a, P->num_cus, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? TBE_OK : TBE_E_HIP;
}

}  // extern "C"

namespace {

// Arguments of the backward entry points other than the workspace (TBE_OK or
// the error code).
int check_backward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                   const void* offsets, int64_t N, const float* psw, const float* grad_out,
                   int32_t optimizer, uint32_t flags, const uint32_t* debug_row_updates) {
  static_assert(OPT_ROWWISE_ADAGRAD == TBE_OPT_ROWWISE_ADAGRAD && OPT_ADAGRAD == TBE_OPT_ADAGRAD &&
                    OPT_SGD == TBE_OPT_SGD,
                "optimizer codes of the header");
  if (optimizer != TBE_OPT_ROWWISE_ADAGRAD && optimizer != TBE_OPT_ADAGRAD &&
      optimizer != TBE_OPT_SGD)
    return TBE_E_ARG;
  const int rc = check_lookups(P, B, itype, indices, offsets, N);
  if (rc) return rc;
  if (flags & ~(TBE_BWD_PREPROCESSED | TBE_BWD_FUSED_LONG | TBE_BWD_CONCURRENT |
                TBE_BWD_ORDER_CHUNKS | TBE_BWD_NO_ORDER_CHUNKS | TBE_BWD_HIST |
                TBE_BWD_CONCURRENT_AUTO))
    return TBE_E_ARG;
  if ((flags & TBE_BWD_HIST) && (!bwd_hist_capable(P) || optimizer != TBE_OPT_ROWWISE_ADAGRAD))
    return TBE_E_UNSUPPORTED;
  if ((flags & TBE_BWD_ORDER_CHUNKS) && (flags & TBE_BWD_NO_ORDER_CHUNKS)) return TBE_E_ARG;
  if (B > 0 && (!grad_out || !aligned(grad_out, 16))) return TBE_E_ARG;
  if (psw && !aligned(psw, 4)) return TBE_E_ARG;
  if (debug_row_updates && !aligned(debug_row_updates, 4)) return TBE_E_ARG;
  return TBE_OK;
}

// The backward's launches on `stream` into the workspace ws (arguments and
// workspace already checked).
int run_backward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                 const void* offsets, int64_t N, const float* psw, const float* grad_out,
                 int32_t optimizer, float lr, float eps, void* ws, uint32_t flags,
                 uint32_t* debug_row_updates, void* stream) {
  if (N == 0) return TBE_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsLayout L = layout(P, N);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  if (flags & TBE_BWD_HIST) {  // no preprocessing: one contraction and a row update
    HistArgs h{};
    h.table = P->h_tables[0];
    h.B = B;
    h.indices = indices;
    h.offsets = offsets;
    h.psw = psw;
    h.grad = grad_out;
    h.dtot = P->dtot;
    h.col = P->col[0];
    h.N = (uint32_t)N;
    h.E = (uint32_t)P->rows[0];
    h.D = (uint32_t)P->dims[0];
    h.mean = P->pooling[0] == TBE_MEAN;
    h.lr = lr;
    h.eps = eps;
    h.part = reinterpret_cast<float*>(w + L.hist_part);
    h.pcnt = reinterpret_cast<uint32_t*>(w + L.hist_cnt);
    h.pstride = L.pstride;
    h.nwg = (uint32_t)std::min<int64_t>(kHistMaxWorkgroups, (B + 127) / 128);
    if (flags & TBE_BWD_PREPROCESSED) {  // the forward's saved counts, when they are this batch's
      h.saved = reinterpret_cast<const uint16_t*>(w + L.hist_save);
      h.saved_hdr = reinterpret_cast<const uint32_t*>(w + L.hist_hdr);
    }
    h.debug_count = debug_row_updates;
    return launch_backward_hist(h, itype, P->wdtype, s) == hipSuccess ? TBE_OK : TBE_E_HIP;
  }
  if (!(flags & TBE_BWD_PREPROCESSED)) {
    PrepArgs pa = prep_args(P, B, itype, indices, offsets, N, psw, ws, &L);
    if (launch_preprocess(pa, P->num_cus, s) != hipSuccess) return TBE_E_HIP;
  }
  BwdArgs a{};
  a.tables = P->d_tables;
  a.B = B;
  a.itype = itype;
  a.offsets = offsets;
  a.psw = psw;
  a.grad = grad_out;
  a.dtot = P->dtot;
  a.lr = lr;
  a.eps = eps;
  a.opt = optimizer;
  a.sorted_bag = reinterpret_cast<const uint32_t*>(w + (L.final_in_b ? L.val_b : L.val_a));
  a.sorted_scale = (psw || any_mean(P))
                       ? reinterpret_cast<const float*>(w + (L.final_in_b ? L.sc_b : L.sc_a))
                       : nullptr;
  a.single_task = reinterpret_cast<const uint4*>(w + L.single_task);
  a.tiny_task = reinterpret_cast<const uint4*>(w + L.tiny_task);
  a.med_task = reinterpret_cast<const uint4*>(w + L.med_task);
  a.long_task = reinterpret_cast<const uint4*>(w + L.long_task);
  a.long_cbeg = reinterpret_cast<const uint32_t*>(w + L.long_cbeg);
  a.remaining = reinterpret_cast<uint32_t*>(w + L.remaining);
  a.chunk_task = reinterpret_cast<const uint4*>(w + L.chunk_task);
  a.partial = reinterpret_cast<float*>(w + L.partial);
  // chunk order by bag: pays when grad_out is larger than the MALL (C5: the
  // chunk kernel 4.08 -> 3.61 ms), not when it fits (C3: no change)
  const bool order = (flags & TBE_BWD_ORDER_CHUNKS) ||
                     (!(flags & TBE_BWD_NO_ORDER_CHUNKS) &&
                      (uint64_t)B * P->dtot * 4 > kChunkOrderMinGradBytes);
  a.chunk_perm = order ? reinterpret_cast<uint32_t*>(w + L.chunk_perm) : nullptr;
  a.pstride = L.pstride;
  a.counters = reinterpret_cast<const uint32_t*>(w + L.counters);
  a.nb = (uint32_t)P->buckets.size();
  a.debug_count = debug_row_updates;
  a.prep_err = reinterpret_cast<const uint32_t*>(w + L.ctl) + kCtlErr;
  a.N = (uint32_t)N;
  a.T = (uint32_t)P->T;
  a.max_single = (uint32_t)N;
  a.max_tiny = L.max_tiny;
  a.max_med = L.max_med;
  a.max_long = L.max_long;
  a.max_chunks = L.max_chunks;
  const bool fused = flags & TBE_BWD_FUSED_LONG;
  const bool fork = (flags & TBE_BWD_CONCURRENT) != 0 ||
                    ((flags & TBE_BWD_CONCURRENT_AUTO) != 0 && N < kConcurrentMaxLookups);
  std::unique_lock<std::mutex> lk(P->mu, std::defer_lock);
  hipStream_t ss[3] = {s, s, s};
  if (fork) {
    lk.lock();
    ss[1] = P->side[0];
    ss[2] = P->side[1];
    if (hipEventRecord(P->ev_fork, s) != hipSuccess ||
        hipStreamWaitEvent(ss[1], P->ev_fork, 0) != hipSuccess ||
        hipStreamWaitEvent(ss[2], P->ev_fork, 0) != hipSuccess)
      return TBE_E_HIP;
  }
  // the hottest long runs by the contraction (their chunks and long-run
  // updates are skipped), on the long runs' stream before their kernels;
  // batches without per-sample weights only (integer counts)
  const bool dense = L.dense && psw == nullptr;
  if (dense) {
    a.indices = indices;
    a.long_flag = reinterpret_cast<uint32_t*>(w + L.long_flag);
    a.dense_rows = reinterpret_cast<uint4*>(w + L.dense_rows);
    a.dense_cnt = reinterpret_cast<uint32_t*>(w + L.dense_cnt);
    a.dense_part = reinterpret_cast<float*>(w + L.dense_part);
    a.dense_w = (uint32_t)P->dense_w;
    a.dense_ncg = (uint32_t)P->dense_ncg;
    a.dense_min_len = (uint32_t)std::max<int64_t>(kLongRun, std::min<int64_t>(B / 256, 1ll << 30));
  }
  int rc_launch = TBE_OK;
  if (dense && launch_dense(a, P->d_tseg, P->wdtype, itype, ss[2]) != hipSuccess)
    rc_launch = TBE_E_HIP;
  if (launch_chunk_order(a, ss[2]) != hipSuccess) rc_launch = TBE_E_HIP;
  for (const auto& grp : bucket_groups(P)) {
    if (rc_launch != TBE_OK) break;
    BucketSet S = bucket_set(P, grp);
    BwdGrids g[kMaxBuckets];
    for (uint32_t k = 0; k < S.n; ++k) {
      const uint64_t sgs = kThreads / S.bk[k].lpr;  // subgroups per workgroup
      g[k].single = (uint32_t)std::min<uint64_t>((uint64_t)N / (2 * sgs) + 1, 1u << 30);
      g[k].tiny = (uint32_t)std::min<uint64_t>(L.max_tiny / sgs + 1, 1u << 30);
      g[k].medium = L.max_med;
      g[k].chunk = L.max_chunks;
      g[k].longrun = L.max_long;
    }
    const Bucket& b0 = P->buckets[grp[0]];
    if (launch_backward_set(a, S, g, P->wdtype, b0.vec, b0.nc, fused, P->num_cus, ss) !=
        hipSuccess) {
      rc_launch = TBE_E_HIP;
      break;
    }
  }
  if (fork) {  // join even after a failed launch, so `s` never runs ahead of the side streams
    for (int i = 0; i < 2; ++i)
      if (hipEventRecord(P->ev_join[i], ss[1 + i]) != hipSuccess ||
          hipStreamWaitEvent(s, P->ev_join[i], 0) != hipSuccess)
        rc_launch = TBE_E_HIP;
  }
  return rc_launch;
}

}  // namespace

extern "C" {

int tbe_backward(const tbe_plan* P, int64_t B, int32_t itype, const void* indices,
                 const void* offsets, int64_t N, const float* psw, const float* grad_out,
                 int32_t optimizer, float lr, float eps, void* ws, size_t ws_bytes,
                 uint32_t flags, uint32_t* debug_row_updates, void* stream) {
  int rc = check_backward(P, B, itype, indices, offsets, N, psw, grad_out, optimizer, flags,
                          debug_row_updates);
  if (rc) return rc;
  rc = check_ws(P, N, ws, ws_bytes);
  if (rc) return rc;
  return run_backward(P, B, itype, indices, offsets, N, psw, grad_out, optimizer, lr, eps, ws,
                      flags, debug_row_updates, stream);
}

int tbe_backward_rowwise_adagrad_noalloc(const tbe_plan* P, int64_t B, int32_t itype,
                                         const void* indices, const void* offsets, int64_t N,
                                         const float* psw, const float* grad_out, float lr,
                                         float eps, uint32_t flags,
                                         uint32_t* debug_row_updates, void* stream) {
  int rc = check_backward(P, B, itype, indices, offsets, N, psw, grad_out,
                          TBE_OPT_ROWWISE_ADAGRAD, flags, debug_row_updates);
  if (rc) return rc;
  // no preprocessing result can be handed in: the static workspace is only
  // written by this call
  if (flags & TBE_BWD_PREPROCESSED) return TBE_E_ARG;
  if (layout(P, N).total > kStaticWsBytes) return TBE_E_TOO_LARGE;
  void* ws = nullptr;
  rc = static_ws_of_current_device(&ws);
  if (rc) return rc;
  return run_backward(P, B, itype, indices, offsets, N, psw, grad_out, TBE_OPT_ROWWISE_ADAGRAD,
                      lr, eps, ws, flags, debug_row_updates, stream);
}

int tbe_backward_rowwise_adagrad(const tbe_plan* P, int64_t B, int32_t itype,
                                 const void* indices, const void* offsets, int64_t N,
                                 const float* psw, const float* grad_out, float lr, float eps,
                                 void* ws, size_t ws_bytes, uint32_t flags,
                                 uint32_t* debug_row_updates, void* stream) {
  return tbe_backward(P, B, itype, indices, offsets, N, psw, grad_out, TBE_OPT_ROWWISE_ADAGRAD, lr,
                      eps, ws, ws_bytes, flags, debug_row_updates, stream);
}

}  // extern "C"
