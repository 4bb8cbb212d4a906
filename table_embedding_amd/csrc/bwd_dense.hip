// Hot-row contraction of the long runs (FBTriton TBE page, "Forward": small
// tables turn their irregular reads into tensor-core work by counting how
// often each row occurs in a bag and multiplying the counts by the table;
// section "Fusion boundaries": the backward can reuse such a histogram).
//
// The same algebra serves the hottest rows of a large table in the backward.
// A run of SL lookups gathers SL grad_out rows; for the few rows of a table
// whose runs are long enough to touch a large share of the table's bags, the
// row gradients are one contraction over the bags,
//   grad[h][d] = sum_b C[b][h] * G[b][c_t + d],
// with C[b][h] the sum of the contribution scales S[p] * (1/L_b if mean) of
// bag b's lookups of hot row h.  Computed that way, each of the table's
// grad_out rows is read once instead of once per lookup of every hot row (on
// a 64-table batch of 138 M lookups the long runs' gathers read 25 GB from
// beyond the L2 per step; their hottest rows hold about four fifths of those
// lookups).
//
// dense_select_kernel (one workgroup per table): the table's long runs, in
// the long list's key order, are the candidates; the threshold starts at
// dense_min_len and doubles until at most kDenseRows runs reach it; those
// runs become the table's hot rows (flagged in long_flag, so that the chunk
// and long-run update kernels skip them).  Tables whose D is not a multiple
// of 16 or exceeds kDensePitch take none.
//
// dense_partial_kernel (dense_w workgroups per table, each a contiguous
// range of the table's bags): per block of K bags (128; 64 when a wave owns
// four column tiles), the block's lookups are read coalesced, a lookup of a
// hot row (found in a small open-addressing table in LDS) finds its bag by
// binary search over the block's bag boundaries, and one integer LDS atomic
// adds it to C's count.  Integer counts are exact in any order, so the
// result does not depend on the atomics' timing; with mean pooling the count
// is multiplied by 1/L_b when it enters the product.  The block's grad_out
// operands are loaded into registers first, so they arrive while the counts
// are built.  Then C^T [hot rows x K bags] x G [K bags x D] on
// v_mfma_f32_16x16x4f32 (fp32: the counts enter exactly and the gradients
// unrounded): wave w owns the 16-column tiles [w*DT, (w+1)*DT) for all row
// tiles, so every grad_out element of the block is loaded once, and the
// accumulators stay in registers across the workgroup's blocks.  Each
// workgroup writes its partial rows; the update kernel (bwd.hip) adds the
// dense_w partials of a row in workgroup order and applies the optimizer.
// Every floating-point sum has a data-determined order, so repeated calls
// give the same bits, and the fused and two-launch long-run paths, which both
// leave the hot rows to this contraction, stay bit-identical.
//
// Only batches without per-sample weights take this path: with them the
// coefficients are float sums, which atomics would add in a varying order,
// and the long runs keep the chunked gather.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kDBags = 128;  // bags per block (K of the block's contraction)

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
  // the smallest doubling of dense_min_len that at most kDenseRows runs reach
  uint32_t thr = a.dense_min_len > 0 ? a.dense_min_len : 1u;
  if (eligible) {
    for (int k = 0; k < 32; ++k) {
      uint32_t c = 0;
      for (uint32_t l = l0 + threadIdx.x; l < l1; l += kThreads) c += a.long_task[l].y >= thr;
      if (block_sum(c, sh4) <= (uint32_t)kDenseRows) break;
      thr = thr >= 0x80000000u ? 0xffffffffu : thr * 2u;
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

typedef float float4v __attribute__((ext_vector_type(4)));

// Open-addressing table of the hot rows in LDS: row -> rank, linear probing,
// at most 64 of kHashSlots slots in use.  The longest probe distance of an
// insert bounds every search, so a lookup reads a fixed number of slots
// (the same for all lanes) instead of probing until an empty slot.
constexpr uint32_t kHashSlots = 1024;
constexpr uint32_t kHashEmpty = 0xffffffffu;  // no row has this key (rows < 2^32 - 1)
__device__ __forceinline__ uint32_t hash_slot(uint32_t row) {
  return (row * 2654435761u) >> 22;  // top 10 bits
}

constexpr int kPer = 8;  // lookups per thread in flight in the counting pass

// Bags per block: K of the block's contraction (a lane holds K/4 * DT
// grad_out operands of the block in registers).
template <int DT>
struct DenseShape {
  static constexpr int kBags = DT >= 4 ? 64 : 128;
  static constexpr int kPitch = kBags + 4;  // count row pitch (words)
  static constexpr int kSteps = kBags / 4;  // K steps of 4 bags
};

template <typename IT, int DT>
__global__ __launch_bounds__(kThreads) void dense_partial_kernel(BwdArgs a) {
  using S = DenseShape<DT>;
  if (dense_prep_failed(a)) return;
  // counts of the block, [hot row][bag]; bag k is consumed in K step k % kSteps
  // by lane group k / kSteps, so that a lane's A operands of four consecutive
  // K steps are one 16-byte read, and the 16 rows of a tile fall in distinct
  // banks (pitch = 4 mod 64 words)
  __shared__ __attribute__((aligned(16))) uint32_t cnt[kDenseRows][S::kPitch];
  __shared__ __attribute__((aligned(16))) float s_inv[S::kBags];  // mean: 1 / bag length
  __shared__ uint32_t s_key[kHashSlots];
  __shared__ uint8_t s_hrank[kHashSlots];
  __shared__ uint32_t s_dmax;  // longest probe distance of an insert
  __shared__ uint32_t s_off[S::kBags + 1];  // positions (< 2^31)
  const uint32_t t = blockIdx.x / a.dense_w, w = blockIdx.x % a.dense_w;
  const uint32_t H = min(a.dense_cnt[t], (uint32_t)kDenseRows);
  if (H == 0) return;
  const TableDev td = a.tables[t];
  const uint32_t D = td.dim;
  const bool mean = td.pooling == POOL_MEAN;
  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const int64_t N = (int64_t)a.N;
  for (uint32_t x = threadIdx.x; x < kHashSlots; x += kThreads) s_key[x] = kHashEmpty;
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
  float4v acc[4][DT];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) acc[rt][nt] = (float4v){0.f, 0.f, 0.f, 0.f};
  // this workgroup's bags [b_lo, b_hi) of the table
  const int64_t B = a.B;
  const int64_t b_lo = B * (int64_t)w / (int64_t)a.dense_w;
  const int64_t b_hi = B * (int64_t)(w + 1) / (int64_t)a.dense_w;
  const int64_t jt = (int64_t)t * B;  // the table's first bag
  const float* gtab = a.grad + td.col;
  for (int64_t j0 = b_lo; j0 < b_hi; j0 += S::kBags) {
    const uint32_t nb = (uint32_t)min((int64_t)S::kBags, b_hi - j0);
    // the block's grad_out operands of this lane (bag kq * kSteps + ks, this
    // wave's columns), all in flight while the counts are built: a full block
    // of columns that all exist reads at a uniform row base plus a 32-bit lane
    // offset; otherwise the bag and column are clamped into range and the
    // value is zeroed
    float gv[S::kSteps][DT];
    {
      const uint32_t c0 = wave * (uint32_t)DT * 16u + i;  // this lane's first column
      if (nb == (uint32_t)S::kBags && (wave + 1u) * (uint32_t)DT * 16u <= D) {
        const float* __restrict__ gblk = gtab + j0 * (int64_t)a.dtot;
        const uint32_t loff = kq * (uint32_t)S::kSteps * a.dtot + c0;
#pragma unroll
        for (int ks = 0; ks < S::kSteps; ++ks) {
          const float* __restrict__ gk = gblk + (int64_t)ks * a.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) gv[ks][nt] = gk[loff + (uint32_t)nt * 16u];
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < S::kSteps; ++ks) {
          const uint32_t jb = kq * (uint32_t)S::kSteps + (uint32_t)ks;
          const float* __restrict__ grow = gtab + (j0 + min(jb, nb - 1u)) * (int64_t)a.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) {
            const uint32_t col = c0 + (uint32_t)nt * 16u;
            const uint32_t keep = (jb < nb && col < D) ? 0xffffffffu : 0u;
            gv[ks][nt] = __uint_as_float(__float_as_uint(grow[min(col, D - 1u)]) & keep);
          }
        }
      }
    }
    {  // clear the rows in use
      const uint32_t n4 = nrt * 16u * (uint32_t)S::kPitch / 4u;
      for (uint32_t x = threadIdx.x; x < n4; x += kThreads)
        reinterpret_cast<uint4*>(&cnt[0][0])[x] = make_uint4(0u, 0u, 0u, 0u);
    }
    // bag boundaries, clamped to the lookups (entries past nb repeat the end
    // of bag nb - 1); the mean's divisor from the raw offsets
    if (threadIdx.x <= (uint32_t)S::kBags) {
      const uint32_t x = min(threadIdx.x, nb);
      const int64_t o = (int64_t)O[jt + j0 + x];
      s_off[threadIdx.x] = (uint32_t)(o < 0 ? 0 : (o > N ? N : o));
    }
    if (threadIdx.x < (uint32_t)S::kBags) {
      float inv = 0.f;
      if (threadIdx.x < nb) {
        const int64_t L = (int64_t)O[jt + j0 + threadIdx.x + 1] - (int64_t)O[jt + j0 + threadIdx.x];
        inv = !mean ? 1.f : (L > 0 ? 1.f / (float)L : 0.f);
      }
      s_inv[threadIdx.x] = inv;
    }
    __syncthreads();  // also the hash table on the first block
    const uint32_t dmax = s_dmax;
    // counting pass: coalesced reads of the block's lookups (the next window's
    // in flight while this one is counted); a lookup of a hot row finds its
    // bag by binary search over the bag boundaries and adds one to its count
    // (integer adds: the same counts in any order).  The kPer lookups of a
    // thread go through the hash probe and each search level together, so
    // a level costs one LDS round trip for all of them.
    // (reads past the block's end are clamped to its last lookup and their
    // key replaced by kHashEmpty)
    const uint32_t P0 = s_off[0], P1 = max(s_off[nb], P0);
    uint32_t r[kPer];
    if (P0 < P1) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const uint32_t p = P0 + threadIdx.x + (uint32_t)u * kThreads;
        const uint32_t v = (uint32_t)I[min(p, P1 - 1u)];
        r[u] = p < P1 ? v : kHashEmpty;
      }
    }
    for (uint32_t q0 = P0; q0 < P1; q0 += (uint32_t)(kPer * kThreads)) {
      const uint32_t qn = q0 + (uint32_t)(kPer * kThreads);
      uint32_t rn[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) rn[u] = kHashEmpty;
      if (qn < P1) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const uint32_t p = qn + threadIdx.x + (uint32_t)u * kThreads;
          const uint32_t v = (uint32_t)I[min(p, P1 - 1u)];
          rn[u] = p < P1 ? v : kHashEmpty;
        }
      }
      // the hot-row slot of each lookup (kHashSlots: not hot, or past the
      // block: kHashEmpty would match an empty slot, so it is excluded)
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
      uint32_t bag[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) bag[u] = 0u;
      // the last bag whose start is at or before p: m < kBags always, and
      // s_off[m] for m >= nb is the block's end, past every p counted here
#pragma unroll
      for (uint32_t step = (uint32_t)S::kBags / 2u; step > 0u; step >>= 1) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          const uint32_t p = q0 + threadIdx.x + (uint32_t)u * kThreads;
          const uint32_t m = bag[u] + step;
          bag[u] = s_off[m] <= p ? m : bag[u];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (slot[u] < kHashSlots) atomicAdd(&cnt[s_hrank[slot[u]]][bag[u]], 1u);
#pragma unroll
      for (int u = 0; u < kPer; ++u) r[u] = rn[u];
    }
    __syncthreads();
    // C^T [rows, K bags] x G [K bags, this wave's columns] on the matrix cores
    // (A = count, times 1 / bag length for the mean)
#pragma unroll
    for (int g = 0; g < S::kSteps / 4; ++g) {
      const uint32_t c0 = kq * (uint32_t)S::kSteps + 4u * (uint32_t)g;
      const float4v inv = *reinterpret_cast<const float4v*>(&s_inv[c0]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if ((uint32_t)rt >= nrt) break;  // uniform
        const uint4 c4 = *reinterpret_cast<const uint4*>(&cnt[(uint32_t)rt * 16u + i][c0]);
        float av[4] = {(float)c4.x, (float)c4.y, (float)c4.z, (float)c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (mean) av[e] *= inv[e];
#pragma unroll
          for (int nt = 0; nt < DT; ++nt)
            acc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], gv[4 * g + e][nt],
                                                              acc[rt][nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the counts are cleared for the next block
  }
  // partial rows of this workgroup: hot row 16 rt + 4 kq + r, column 16 (wave DT + nt) + i
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if ((uint32_t)rt >= nrt) break;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const uint32_t col = (wave * (uint32_t)DT + (uint32_t)nt) * 16u + i;
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
hipError_t launch_partial(const BwdArgs& a, int dt, hipStream_t s) {
  const dim3 grid(a.T * a.dense_w), block(kThreads);
  if (dt <= 1)
    TBE_LAUNCH("dense_partial", (dense_partial_kernel<IT, 1>), grid, block, s, a);
  else if (dt == 2)
    TBE_LAUNCH("dense_partial", (dense_partial_kernel<IT, 2>), grid, block, s, a);
  else
    TBE_LAUNCH("dense_partial", (dense_partial_kernel<IT, 4>), grid, block, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_update(const BwdArgs& a, int wd, hipStream_t s);

hipError_t launch_dense(const BwdArgs& a, const uint32_t* tseg, int wd, int itype, int dt,
                        hipStream_t s) {
  if (!a.long_flag || a.T == 0) return hipSuccess;
  TBE_LAUNCH("dense_select", dense_select_kernel, dim3(a.T), dim3(kThreads), s, a, tseg);
  const hipError_t e = itype == IT_I32 ? launch_partial<int32_t>(a, dt, s)
                                       : launch_partial<int64_t>(a, dt, s);
  if (e != hipSuccess) return e;
  return launch_dense_update(a, wd, s);
}

}  // namespace tbe
