// Hot-row contraction of the long runs (FBTriton TBE page, "Forward": small
// tables turn their irregular reads into tensor-core work by counting how
// often each row occurs in a bag and multiplying the counts by the table;
// section "Fusion boundaries": the backward can reuse such a histogram).
//
// The same algebra serves the hottest rows of a large table in the backward.
// A run of SL lookups gathers SL grad_out rows; for the rows of a table whose
// runs are long enough, the row gradients are one contraction over the bags,
//   grad[h][d] = sum_b C[b][h] * G[b][c_t + d],
// with C[b][h] the number of bag b's lookups of hot row h, and G scaled by
// 1/L_b for a mean table.  Computed that way, each of the table's grad_out
// rows is read once instead of once per lookup of every hot row (on a
// 64-table batch of 138 M lookups the long runs' gathers read 25 GB from
// beyond the L2 per step).
//
// dense_select_kernel (one workgroup per table): the table's long runs, in
// the long list's key order, are the candidates; the threshold is the
// smallest length of at least dense_min_len that at most kDenseRows runs
// reach (a binary search over lengths); those runs become the table's hot
// rows (flagged in long_flag, so that the chunk and long-run update kernels
// skip them).  Tables whose D is not a multiple of 16 or exceeds kDensePitch
// take none.
//
// dense_partial_kernel (dense_w workgroups per table and column group of
// 128 columns, each a contiguous range of the table's bags; eight waves, so
// that the count pass is shared by more waves and two workgroups per CU
// keep sixteen waves there): per block of 64 bags, the block's lookups are
// read coalesced, four consecutive ones per thread; a lookup of a hot row
// (found in a small open-addressing table in LDS) adds one with an integer
// LDS atomic to its bag's count, the bag found by binary search over the
// block's bag boundaries for a thread's first lookup and by stepping on for
// the next three.  Integer counts are exact in any order, so the result does
// not depend on the atomics' timing.  The block's grad_out operands are
// loaded into registers first, so they arrive while the counts are built.
// Then C^T [hot rows x K bags] x G [K bags x D] on the matrix cores, exact
// in its products: when no bag of the block has more than 255 lookups,
// every count is an integer of at most 8 bits, exact in bfloat16 (packed
// so once per block for all waves), and each fp32 gradient is the exact
// sum of three bfloat16 parts (its significand cut into three 8-bit
// pieces), so three v_mfma_f32_16x16x32_bf16 per tile give the fp32
// products without rounding; otherwise each count is cut into four 8-bit
// parts and the block takes four such passes.  Either way the products are
// exact and only the fp32 accumulation rounds.
// Wave w owns the 16-column tile w of the group for all row tiles, so every
// grad_out element of the block is loaded once, and the accumulators stay
// in registers across the workgroup's blocks.  Each workgroup writes its
// partial rows; the update kernel (bwd.hip) adds the dense_w partials of a
// row in a fixed order and applies the optimizer.  Every floating-point sum
// has a data-determined order, so repeated calls give the same bits, and the
// fused and two-launch long-run paths, which both leave the hot rows to this
// contraction, stay bit-identical.
//
// Only batches without per-sample weights take this path: with them the
// coefficients are float sums, which atomics would add in a varying order,
// and the long runs keep the chunked gather.
#include "count_mma.h"

namespace tbe {
namespace {

__device__ __forceinline__ bool dense_prep_failed(const BwdArgs& a) { return *a.prep_err != 0u; }

// First position in [lo, hi) of the long list whose table sits at or after
// segment `seg` in key order (the long list is in key order).
__device__ __forceinline__ uint32_t long_lower(const BwdArgs& a, const uint32_t* tseg,
                                               uint32_t lo, uint32_t hi, uint32_t seg) {
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    const uint32_t t = a.long_task[mid].w;
    if ((t < a.T ? tseg[t] : 0xffffffffu) < seg) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* sh4) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  __syncthreads();
  if (lane_id() == 0) sh4[threadIdx.x / kWave] = v;
  __syncthreads();
  return sh4[0] + sh4[1] + sh4[2] + sh4[3];
}

__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* sh4) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o, kWave));
  __syncthreads();
  if (lane_id() == 0) sh4[threadIdx.x / kWave] = v;
  __syncthreads();
  return max(max(sh4[0], sh4[1]), max(sh4[2], sh4[3]));
}

__global__ __launch_bounds__(kThreads) void dense_select_kernel(BwdArgs a, const uint32_t* tseg) {
  if (dense_prep_failed(a)) return;
  __shared__ uint32_t sh4[4];
  __shared__ uint32_t s_base;
  const uint32_t t = blockIdx.x;
  const TableDev td = a.tables[t];
  const uint32_t n_long = min(a.counters[kCntSingle + 3], a.max_long);
  const uint32_t l0 = long_lower(a, tseg, 0, n_long, tseg[t]);
  const uint32_t l1 = long_lower(a, tseg, l0, n_long, tseg[t] + 1);
  const bool eligible = td.dim % 16u == 0 && td.dim <= (uint32_t)kDensePitch;
  // the smallest length >= dense_min_len that at most kDenseRows runs reach
  uint32_t thr = a.dense_min_len > 0 ? a.dense_min_len : 1u;
  if (eligible) {
    uint32_t c = 0, mx = 0;
    for (uint32_t l = l0 + threadIdx.x; l < l1; l += kThreads) {
      const uint32_t len = a.long_task[l].y;
      c += len >= thr;
      mx = max(mx, len);
    }
    if (block_sum(c, sh4) > (uint32_t)kDenseRows) {
      // count(len >= t) is non-increasing in t and 0 past the longest run:
      // binary search over (thr, longest + 1]
      uint32_t lo = thr + 1u, hi = block_max(mx, sh4) + 1u;
      while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2u;
        uint32_t cm = 0;
        for (uint32_t l = l0 + threadIdx.x; l < l1; l += kThreads) cm += a.long_task[l].y >= mid;
        if (block_sum(cm, sh4) <= (uint32_t)kDenseRows) hi = mid; else lo = mid + 1u;
      }
      thr = lo;
    }
  }
  if (threadIdx.x == 0) s_base = 0;
  __syncthreads();
  for (uint32_t c0 = l0; c0 < l1; c0 += kThreads) {
    const uint32_t l = c0 + threadIdx.x;
    const uint4 task = l < l1 ? a.long_task[l] : make_uint4(0, 0, 0, 0);
    const bool hot = eligible && l < l1 && task.y >= thr;
    // rank among this batch's hot runs, in list order
    const uint64_t bal = __ballot(hot);
    const uint32_t in_wave = (uint32_t)__popcll(bal & ((lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()))));
    if (lane_id() == 0) sh4[threadIdx.x / kWave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t before = s_base;
    for (uint32_t w = 0; w < threadIdx.x / kWave; ++w) before += sh4[w];
    const uint32_t total = sh4[0] + sh4[1] + sh4[2] + sh4[3];
    if (l < l1) {
      const uint32_t rank = before + in_wave;
      const bool take = hot && rank < (uint32_t)kDenseRows;  // (never false: thr caps the count)
      if (take) a.dense_rows[(size_t)t * kDenseRows + rank] = make_uint4(task.x, task.y, task.z, l);
      a.long_flag[l] = take ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dense_cnt[t] = min(s_base, (uint32_t)kDenseRows);
}

// Open-addressing table of the hot rows in LDS: row -> rank, linear probing,
// at most kDenseRows of kHashSlots slots in use.  The longest probe distance
// of an insert bounds every search, so a lookup reads a fixed number of
// slots (the same for all lanes) instead of probing until an empty slot.
constexpr uint32_t kHashSlots = 1024;
constexpr uint32_t kHashEmpty = 0xffffffffu;  // no row has this key (rows < 2^32 - 1)
__device__ __forceinline__ uint32_t hash_slot(uint32_t row) {
  return (row * 2654435761u) >> 22;  // top 10 bits
}

constexpr int kPer = 4;  // consecutive lookups per thread in the counting pass
static_assert(kPer == 4, "load_lookups4 loads four lookups");

// Lookups p .. p + 3 (p a multiple of 4) as row ids, positions clamped to
// the last one before `end`; one 16-byte (int32) or two (int64) vector loads
// when the indices are 16-byte aligned and all four exist.
template <typename IT>
__device__ __forceinline__ void load_lookups4(const IT* __restrict__ I, uint32_t p, uint32_t end,
                                              bool vec, uint32_t (&rr)[4]) {
  if (vec && p + 3u < end) {
    if constexpr (sizeof(IT) == 4) {
      const int4 v = *reinterpret_cast<const int4*>(I + p);
      rr[0] = (uint32_t)v.x; rr[1] = (uint32_t)v.y; rr[2] = (uint32_t)v.z; rr[3] = (uint32_t)v.w;
    } else {
      const longlong2 v0 = *reinterpret_cast<const longlong2*>(I + p);
      const longlong2 v1 = *reinterpret_cast<const longlong2*>(I + p + 2u);
      rr[0] = (uint32_t)v0.x; rr[1] = (uint32_t)v0.y; rr[2] = (uint32_t)v1.x; rr[3] = (uint32_t)v1.y;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) rr[u] = (uint32_t)I[min(p + (uint32_t)u, end - 1u)];
  }
}
constexpr uint32_t kMaxExactCount = 255;  // counts of at most 8 bits are exact in bfloat16
constexpr int kRowTiles = kDenseRows / 16;

// Bags per block: K of the block's contraction (a lane holds K/4 grad_out
// operands of the block in registers); a workgroup's columns are one group
// of kGroupCols: eight waves of one 16-column tile each.
struct DenseShape {
  static constexpr int kDT = 1;              // 16-column tiles per wave
  static constexpr int kNW = 8;              // waves of the workgroup
  static constexpr int kNT = 64 * kNW;       // threads of the workgroup
  static constexpr int kWin = kPer * kNT;    // lookups per counting window
  static constexpr int kBags = 64;
  static constexpr int kPitch = kBags + 4;  // count row pitch (words; = 4 mod 64)
  static constexpr int kPitchB = kBags / 2 + 4;  // bfloat16 count row pitch (words)
  static constexpr int kSteps = kBags / 32; // K steps of 32 bags
  static constexpr uint32_t kGroupCols = 16u * kDT * kNW;
};

// Two workgroups per CU (LDS allows two): four waves per SIMD, so at most
// 128 registers per lane.
template <typename IT>
__global__ __launch_bounds__(DenseShape::kNT) __attribute__((amdgpu_waves_per_eu(4)))
void dense_partial_kernel(BwdArgs a) {
  using S = DenseShape;
  constexpr int DT = S::kDT;
  if (dense_prep_failed(a)) return;
  // counts of the block, [hot row][bag] (integer atomic adds: exact in any
  // order); the 16 rows of a tile fall in distinct banks
  __shared__ __attribute__((aligned(16))) uint32_t cnt[kDenseRows][S::kPitch];
  // the counts (or one 8-bit part of them, in a block with wider counts) as
  // packed bfloat16, converted once per block for all waves' operand reads
  __shared__ __attribute__((aligned(16))) uint32_t cbf[kDenseRows][S::kPitchB];
  __shared__ __attribute__((aligned(16))) float s_inv[S::kBags];  // 1 / bag length (mean)
  __shared__ uint32_t s_key[kHashSlots];
  __shared__ uint8_t s_hrank[kHashSlots];
  __shared__ uint32_t s_dmax;  // longest probe distance of an insert
  __shared__ uint32_t s_off[S::kBags + 1];  // positions (< 2^31)
  // workgroup = (table, bag range, column group)
  const uint32_t cg = blockIdx.x % a.dense_ncg, tw = blockIdx.x / a.dense_ncg;
  const uint32_t t = tw / a.dense_w, w = tw % a.dense_w;
  const uint32_t H = min(a.dense_cnt[t], (uint32_t)kDenseRows);
  const TableDev td = a.tables[t];
  if (H == 0 || cg * S::kGroupCols >= td.dim) return;
  const uint32_t D = td.dim;
  const bool mean = td.pooling == POOL_MEAN;
  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const int64_t N = (int64_t)a.N;
  const bool vec4 = (reinterpret_cast<uintptr_t>(I) & 15u) == 0;  // uniform
  for (uint32_t x = threadIdx.x; x < kHashSlots; x += S::kNT) s_key[x] = kHashEmpty;
  if (threadIdx.x == 0) s_dmax = 0;
  __syncthreads();
  if (threadIdx.x < H) {  // the table's hot rows are distinct: one insert each
    const uint32_t row = a.dense_rows[(size_t)t * kDenseRows + threadIdx.x].z;
    uint32_t q = hash_slot(row), d = 0;
    while (atomicCAS(&s_key[q], kHashEmpty, row) != kHashEmpty) {
      q = (q + 1u) & (kHashSlots - 1u);
      ++d;
    }
    s_hrank[q] = (uint8_t)threadIdx.x;
    atomicMax(&s_dmax, d);
  }
  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t i = lane & 15u, kq = lane >> 4;  // A row / B column; K lane group
  const uint32_t nrt = (H + 15u) / 16u;           // row tiles in use
  cm_f4 acc[kRowTiles][DT];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) acc[rt][nt] = (cm_f4){0.f, 0.f, 0.f, 0.f};
  // this workgroup's bags [b_lo, b_hi) of the table
  const int64_t B = a.B;
  const int64_t b_lo = B * (int64_t)w / (int64_t)a.dense_w;
  const int64_t b_hi = B * (int64_t)(w + 1) / (int64_t)a.dense_w;
  const int64_t jt = (int64_t)t * B;  // the table's first bag
  const float* gtab = a.grad + td.col;
  const uint32_t c0 = cg * S::kGroupCols + wave * (uint32_t)DT * 16u + i;  // this lane's first column
  // first lookup of the current block (the previous block's end)
  uint32_t P0 = 0;
  if (b_lo < b_hi) {
    const int64_t o = (int64_t)O[jt + b_lo];
    P0 = (uint32_t)(o < 0 ? 0 : (o > N ? N : o));
  }
  for (int64_t j0 = b_lo; j0 < b_hi; j0 += S::kBags) {
    const uint32_t nb = (uint32_t)min((int64_t)S::kBags, b_hi - j0);
    // Loads in the order they are needed (vector loads complete in order),
    // none waited for before grad_out's are issued: the bag boundaries (bag
    // min(x, nb) for thread x, so every index is in range), the block's first
    // window of lookups from P0 (positions clamped to the last lookup; those
    // past the block's end are dropped once its end is known), then grad_out.
    const int64_t o_lo = (int64_t)O[jt + j0 + min(threadIdx.x, nb)];
    const int64_t o_hi = (int64_t)O[jt + j0 + min(threadIdx.x + 1u, nb)];
    // windows of kWin lookups start at P0 rounded down to a multiple of 4
    const uint32_t qa = P0 & ~3u;
    uint32_t r[kPer];
    if (N > 0) load_lookups4(I, qa + (uint32_t)kPer * threadIdx.x, (uint32_t)N, vec4, r);
    // the block's grad_out operands of this lane: gv[ks][e][nt] is bag
    // 32 ks + 8 kq + e at column c0 + 16 nt (the B operand layout of the
    // 16x16x32 product), all in flight while the counts are built.  A full
    // block of columns that all exist reads at a uniform row base plus a
    // 32-bit lane offset; otherwise the bag and column are clamped into range
    // and the value is zeroed after the counting pass.
    float gv[S::kSteps][8][DT];
    const bool full = nb == (uint32_t)S::kBags && c0 - i + (uint32_t)DT * 16u <= D;  // wave-uniform
    if (full) {
      const float* __restrict__ gblk = gtab + j0 * (int64_t)a.dtot;
      const uint32_t loff = 8u * kq * a.dtot + c0;
#pragma unroll
      for (int ks = 0; ks < S::kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* __restrict__ gk = gblk + (int64_t)(32 * ks + e) * a.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) gv[ks][e][nt] = gk[loff + (uint32_t)nt * 16u];
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < S::kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t jb = 32u * (uint32_t)ks + 8u * kq + (uint32_t)e;
          const float* __restrict__ grow = gtab + (j0 + min(jb, nb - 1u)) * (int64_t)a.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt)  // (zeroed outside the block below, once loaded)
            gv[ks][e][nt] = grow[min(c0 + (uint32_t)nt * 16u, D - 1u)];
        }
    }
    {  // clear the rows in use
      const uint32_t n4 = nrt * 16u * (uint32_t)S::kPitch / 4u;
      for (uint32_t x = threadIdx.x; x < n4; x += S::kNT)
        reinterpret_cast<uint4*>(&cnt[0][0])[x] = make_uint4(0u, 0u, 0u, 0u);
    }
    // bag boundaries, clamped to the lookups (entries past nb repeat the end
    // of bag nb - 1), and the mean's divisor from the raw offsets
    if (threadIdx.x <= (uint32_t)S::kBags)
      s_off[threadIdx.x] = (uint32_t)(o_lo < 0 ? 0 : (o_lo > N ? N : o_lo));
    if (threadIdx.x < (uint32_t)S::kBags) {
      const int64_t L = o_hi - o_lo;
      s_inv[threadIdx.x] = !mean ? 1.f : (threadIdx.x < nb && L > 0 ? 1.f / (float)L : 0.f);
    }
    __syncthreads();  // also the hash table on the first block
    const uint32_t dmax = s_dmax;
    const uint32_t P1 = min(max(s_off[nb], (uint32_t)P0), (uint32_t)N);  // the block's lookups are [P0, P1)
    // counting pass (the next window's lookups in flight while this one is
    // counted): a lookup of a hot row adds one to its bag's count (integer
    // adds: the same counts in any order).  A thread takes kPer consecutive
    // lookups of the window; the first one's bag is found by binary search
    // over the bag boundaries and each next one's by stepping on from it.
    // The kPer lookups go through the hash probe together, so a probe step
    // costs one LDS round trip for all of them.
    for (uint32_t q0 = qa; q0 < P1; q0 += (uint32_t)S::kWin) {
      const uint32_t pb = q0 + (uint32_t)kPer * threadIdx.x;  // this thread's first lookup
      // lookups outside the block's [P0, P1) are dropped here, where their
      // values are first needed (not where they are loaded)
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (pb + (uint32_t)u < P0 || pb + (uint32_t)u >= P1) r[u] = kHashEmpty;
      const uint32_t qn = q0 + (uint32_t)S::kWin;
      uint32_t rn[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) rn[u] = kHashEmpty;
      if (qn < P1) load_lookups4(I, qn + (uint32_t)kPer * threadIdx.x, P1, vec4, rn);
      // the hot-row slot of each lookup (kHashSlots: not hot, or dropped:
      // kHashEmpty would match an empty slot, so it is excluded)
      uint32_t slot[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) slot[u] = kHashSlots;
      for (uint32_t d = 0; d <= dmax; ++d) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const uint32_t q = (hash_slot(r[u]) + d) & (kHashSlots - 1u);
          slot[u] = (s_key[q] == r[u] && r[u] != kHashEmpty) ? q : slot[u];
        }
      }
      // the last bag whose start is at or before p (p clamped into the
      // block, so the walk ends: s_off[m] for m >= nb is the block's end,
      // past every p counted here, and m < kBags always)
      uint32_t bag[kPer];
      {
        const uint32_t p = min(pb, P1 - 1u);
        uint32_t m0 = 0u;
#pragma unroll
        for (uint32_t step = (uint32_t)S::kBags / 2u; step > 0u; step >>= 1) {
          const uint32_t m = m0 + step;
          m0 = s_off[m] <= p ? m : m0;
        }
        bag[0] = m0;
      }
#pragma unroll
      for (int u = 1; u < kPer; ++u) {
        const uint32_t p = min(pb + (uint32_t)u, P1 - 1u);
        uint32_t m = bag[u - 1];
        while (m < (uint32_t)S::kBags - 1u && s_off[m + 1u] <= p) ++m;
        bag[u] = m;
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (slot[u] < kHashSlots) atomicAdd(&cnt[s_hrank[slot[u]]][bag[u]], 1u);
#pragma unroll
      for (int u = 0; u < kPer; ++u) r[u] = rn[u];
    }
    // a bag of more than kMaxExactCount lookups may hold a count that one
    // bfloat16 cannot carry
    const bool wide = __syncthreads_or(threadIdx.x < nb &&
                                       s_off[threadIdx.x + 1] - s_off[threadIdx.x] > kMaxExactCount);
    if (!full) {  // bags past nb and columns past D contribute nothing
#pragma unroll
      for (int ks = 0; ks < S::kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) {
            const uint32_t jb = 32u * (uint32_t)ks + 8u * kq + (uint32_t)e;
            const uint32_t keep = (jb < nb && c0 + (uint32_t)nt * 16u < D) ? 0xffffffffu : 0u;
            gv[ks][e][nt] = __uint_as_float(__float_as_uint(gv[ks][e][nt]) & keep);
          }
    }
    // mean: G scaled by 1/L of its bag (one rounding, as each lookup's scale)
    if (mean) {
#pragma unroll
      for (int ks = 0; ks < S::kSteps; ++ks) {
        const cm_f4 i0 = *reinterpret_cast<const cm_f4*>(&s_inv[32 * ks + 8 * kq]);
        const cm_f4 i1 = *reinterpret_cast<const cm_f4*>(&s_inv[32 * ks + 8 * kq + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) gv[ks][e][nt] *= e < 4 ? i0[e & 3] : i1[e & 3];
      }
    }
    // C^T [rows, K bags] x G [K bags, this wave's columns], exact products:
    // the counts packed as bfloat16 once for all the waves, whole when they
    // fit 8 bits, else in four 8-bit parts, one product pass each
    const uint32_t nparts = wide ? 4u : 1u;
    for (uint32_t ap = 0; ap < nparts; ++ap) {
      if (ap > 0) __syncthreads();  // the previous part's operand reads are done
      cm_counts_to_bf16<S::kBags, S::kPitch, S::kPitchB>(
          cnt, cbf, nrt * 16u, wide ? 0xffu << (8u * ap) : 0xffffffffu, threadIdx.x, S::kNT);
      __syncthreads();
      cm_bf16_x_grad<S::kSteps, DT, kRowTiles, S::kPitchB>(acc, cbf, gv, nrt, i, kq);
    }
    P0 = s_off[nb];  // the next block's first lookup
    __syncthreads();  // the counts are cleared (and s_off rewritten) for the next block
  }
  // partial rows of this workgroup: hot row 16 rt + 4 kq + r, column c0 + 16 nt
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    if ((uint32_t)rt >= nrt) break;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const uint32_t col = c0 + (uint32_t)nt * 16u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = (uint32_t)rt * 16u + 4u * kq + (uint32_t)r;
        if (row < H && col < D)
          a.dense_part[(((size_t)t * kDenseRows + row) * a.dense_w + w) * kDensePitch + col] =
              acc[rt][nt][r];
      }
    }
  }
}

template <typename IT>
hipError_t launch_partial(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(a.T * a.dense_w * a.dense_ncg), block(DenseShape::kNT);
  TBE_LAUNCH("dense_partial", dense_partial_kernel<IT>, grid, block, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_update(const BwdArgs& a, int wd, hipStream_t s);

hipError_t launch_dense(const BwdArgs& a, const uint32_t* tseg, int wd, int itype,
                        hipStream_t s) {
  if (!a.long_flag || a.T == 0) return hipSuccess;
  TBE_LAUNCH("dense_select", dense_select_kernel, dim3(a.T), dim3(kThreads), s, a, tseg);
  const hipError_t e = itype == IT_I32 ? launch_partial<int32_t>(a, s)
                                       : launch_partial<int64_t>(a, s);
  if (e != hipSuccess) return e;
  return launch_dense_update(a, wd, s);
}

}  // namespace tbe
