// Histogram-reuse backward for one small table (FBTriton TBE page, "Forward":
// the small-table path multiplies per-bag row counts by the table on the
// matrix cores; section "Fusion boundaries": the backward can reuse that
// histogram).  With E rows the weight gradient is one contraction,
//   grad[e][d] = sum_j C[j][e] * G[j][d],
// where C[j][e] sums the contribution scales S[p] * (1/L_j if mean) of bag
// j's lookups of row e, and K = B bags.  It replaces the sort, the run
// classes and the per-lookup gathers of grad_out rows (C4: 8.4M lookups of
// 64 rows, 4.3 GB of row gathers) by one pass over grad_out.
//
// gfx950 design.  Without per-sample weights (bwd_hist_count_kernel) every
// coefficient is a row count: each workgroup takes a contiguous range of
// bags in blocks of 64, builds the block's counts in LDS (from the saved
// histogram or from its lookups, integer adds), and multiplies C^T by the
// block's grad_out rows on v_mfma_f32_16x16x32_bf16 with every product exact
// (count_mma.h), accumulating in registers across blocks.  With per-sample
// weights (bwd_hist_weighted_kernel) the coefficients are float sums: two
// threads per bag of a 128-bag block sum the first and the second half of
// its lookups' coefficients, in lookup order, into two LDS copies added in a
// fixed order (deterministic, no float atomics), and wave w multiplies rows
// [16w, 16w + 16) of C^T by the block's grad_out rows with
// v_mfma_f32_16x16x4f32.  Both write a partial [E x D] and row counts per
// workgroup.  bwd_hist_update: a workgroup per row sums the partials in a
// fixed order (four interleaved accumulators per stripe, stripes combined in
// order) and applies row-wise Adagrad to rows with at least one lookup.
// Determinism: every floating-point sum is in a data-determined order, so
// repeated calls give the same bits.
//
// Reuse of the forward's histogram (tbe_forward_preprocess with
// TBE_FWD_SAVE_HIST, then this backward with TBE_BWD_PREPROCESSED): the
// counts of a block's bags come from the saved uint16 row counts (C4:
// 8.4 MB) instead of the indices (67 MB of int64).  Both sources give the
// same integer counts, so the same bits; a block with a bag of 65536 lookups
// or more, or counts saved for another batch (the header's {B, N} differ),
// takes the indices.
#include "count_mma.h"

namespace tbe {
namespace {

constexpr int kHBags = 128;  // bags (K) per block
constexpr int kHRows = 64;   // most rows
constexpr int kHCols = 128;  // widest row

typedef float float4v __attribute__((ext_vector_type(4)));

template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_hist_weighted_kernel(HistArgs h) {
  __shared__ float coef[2][kHBags][kHRows + 1];  // [half][bag][row], padded
  __shared__ uint32_t cnt[kHRows];
  __shared__ float s_len[kHBags];                // bag lengths of the block
  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t i = lane & 15u, kq = lane >> 4;  // A row / B column; K lane group
  const IT* __restrict__ I = reinterpret_cast<const IT*>(h.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(h.offsets);
  const uint32_t E = h.E, D = h.D;
  const bool mean = h.mean != 0;
  float4v acc[kHCols / 16];
#pragma unroll
  for (int nt = 0; nt < kHCols / 16; ++nt) acc[nt] = (float4v){0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x < (uint32_t)kHRows) cnt[threadIdx.x] = 0u;
  // without per-sample weights a coefficient is a row count, scaled by 1/L
  // once (mean) when it enters the contraction
  const bool counts = h.psw == nullptr;
  const bool use_saved = counts && h.saved != nullptr && h.saved_hdr[0] == (uint32_t)h.B &&
                         h.saved_hdr[1] == h.N;  // uniform
  const int64_t nblk = (h.B + kHBags - 1) / kHBags;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t j0 = blk * kHBags;
    const uint32_t nb = (uint32_t)min((int64_t)kHBags, h.B - j0);
    for (uint32_t x = threadIdx.x; x < (uint32_t)(2 * kHBags * (kHRows + 1)); x += kThreads)
      (&coef[0][0][0])[x] = 0.f;
    bool wide = false;  // a bag whose counts a uint16 may not hold
    if (threadIdx.x < nb) {
      const int64_t L = (int64_t)O[j0 + threadIdx.x + 1] - (int64_t)O[j0 + threadIdx.x];
      s_len[threadIdx.x] = (float)L;
      wide = L >= 65536;
    }
    // (the barrier runs for every block: no short-circuit past it)
    const int any_wide = __syncthreads_or(wide ? 1 : 0);  // also the barrier
    const bool from_saved = use_saved && !any_wide;
    if (from_saved) {  // the block's saved counts, bag-major and coalesced
      for (uint32_t x = threadIdx.x; x < nb * E; x += kThreads) {
        const uint32_t b = x / E, e = x % E;
        const uint32_t c = h.saved[(j0 + b) * (int64_t)E + e];
        coef[0][b][e] = (float)c;
        if (c) atomicAdd(&cnt[e], c);
      }
    } else {
      const uint32_t bag = threadIdx.x % kHBags, half = threadIdx.x / kHBags;
      if (bag < nb) {  // half `half` of this bag's coefficients, in lookup order
        const int64_t lo = (int64_t)O[j0 + bag], hi = (int64_t)O[j0 + bag + 1];
        const float fl = (float)(hi - lo);
        const int64_t mid = lo + (hi - lo) / 2;
        const int64_t ps = half ? mid : lo, pe0 = half ? hi : mid;
        const int64_t pe = pe0 < (int64_t)h.N ? pe0 : (int64_t)h.N;
        // 16 indices (and weights) in flight, then their updates in order
        for (int64_t p0 = ps < 0 ? 0 : ps; p0 < pe; p0 += 16) {
          int64_t r[16];
          float sp[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const bool in = p0 + u < pe;
            r[u] = in ? (int64_t)I[p0 + u] : -1;
            sp[u] = (in && h.psw) ? h.psw[p0 + u] : 1.0f;
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            if (r[u] < 0 || r[u] >= (int64_t)E) continue;
            // with per-sample weights, the contribution scale of the lookup as the
            // transposition computes it; else a count (exact in float32)
            coef[half][bag][r[u]] += counts ? 1.0f : (mean ? sp[u] / fl : sp[u]);
            atomicAdd(&cnt[r[u]], 1u);
          }
        }
      }
    }
    __syncthreads();
    // C^T[rows 16w.., bags] x G[bags, cols] on the matrix cores
    if (16u * wave < E) {
#pragma unroll 4
      for (uint32_t ks = 0; ks < (uint32_t)kHBags / 4u; ++ks) {
        const uint32_t jb = ks * 4u + kq;  // this lane's bag in the K step
        float av = coef[0][jb][16u * wave + i] + coef[1][jb][16u * wave + i];
        // (an empty bag has no count to scale)
        if (counts && mean && jb < nb && s_len[jb] > 0.f) av = av / s_len[jb];
        const bool bag_ok = jb < nb;
        const float* grow = h.grad + (j0 + (bag_ok ? jb : 0u)) * (int64_t)h.dtot + h.col;
#pragma unroll
        for (int nt = 0; nt < kHCols / 16; ++nt) {
          const uint32_t c = (uint32_t)nt * 16u + i;
          if ((uint32_t)nt * 16u >= D) break;  // uniform
          const float bv = (bag_ok && c < D) ? grow[c] : 0.f;
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[nt], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // coef is cleared for the next block
  }
  // partial of this workgroup: rows 16w + 4 kq + r, column 16 nt + i
  float* part = h.part + (size_t)blockIdx.x * E * h.pstride;
  if (16u * wave < E) {
#pragma unroll
    for (int nt = 0; nt < kHCols / 16; ++nt) {
      const uint32_t c = (uint32_t)nt * 16u + i;
      if ((uint32_t)nt * 16u >= D) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t row = 16u * wave + 4u * kq + (uint32_t)r;
        if (row < E && c < D) part[(size_t)row * h.pstride + c] = acc[nt][r];
      }
    }
  }
  if (threadIdx.x < E) h.pcnt[(size_t)blockIdx.x * E + threadIdx.x] = cnt[threadIdx.x];
}

// Without per-sample weights every coefficient is a row count: workgroup w
// takes bags [B w / nwg, B (w + 1) / nwg) in blocks of 64.  A block's counts
// come from the forward's saved histogram (coalesced uint16 reads, written
// transposed into LDS) when those are this batch's and no bag of the block
// reaches 65536 lookups, else from its lookups (coalesced index reads, the
// bag of a lookup by binary search over the block's boundaries, one integer
// LDS atomic each).  The block's grad_out operands are loaded first, so they
// arrive while the counts are built; the product is count_mma.h's, exact in
// every product (G scaled by 1/L per bag for a mean table).  Row totals come
// from the count rows, so a row with a lookup is known without atomics.
template <typename IT, int DT>
__global__ __launch_bounds__(kThreads) void bwd_hist_count_kernel(HistArgs h) {
  constexpr int kBags = 64, kPitch = kBags + 4, kSteps = kBags / 32, kRT = kHRows / 16;
  constexpr int kPer = 4;                            // lookups in flight per thread
  constexpr int kSavedPer = kBags * kHRows / kThreads;  // saved counts per thread
  __shared__ __attribute__((aligned(16))) uint32_t cnt[kHRows][kPitch];  // [row][bag]
  __shared__ __attribute__((aligned(16))) float s_inv[kBags];
  __shared__ uint32_t s_off[kBags + 1];
  const uint32_t wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t i = lane & 15u, kq = lane >> 4;  // A row / B column; K lane group
  const IT* __restrict__ I = reinterpret_cast<const IT*>(h.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(h.offsets);
  const uint32_t E = h.E, D = h.D, N = h.N;
  const bool mean = h.mean != 0;
  const uint32_t nrt = (E + 15u) / 16u;
  const uint32_t c0 = wave * (uint32_t)DT * 16u + i;  // this lane's first column
  const bool use_saved = h.saved != nullptr && h.saved_hdr[0] == (uint32_t)h.B &&
                         h.saved_hdr[1] == N;  // uniform
  cm_f4 acc[kRT][DT];
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) acc[rt][nt] = (cm_f4){0.f, 0.f, 0.f, 0.f};
  uint32_t rowtot = 0;  // thread e < E: lookups of row e in this workgroup's bags
  const int64_t b_lo = h.B * (int64_t)blockIdx.x / (int64_t)h.nwg;
  const int64_t b_hi = h.B * (int64_t)(blockIdx.x + 1) / (int64_t)h.nwg;
  uint32_t P0 = 0;  // first lookup of the current block (the previous block's end)
  if (b_lo < b_hi) {
    const int64_t o = (int64_t)O[b_lo];
    P0 = (uint32_t)(o < 0 ? 0 : (o > (int64_t)N ? (int64_t)N : o));
  }
  for (int64_t j0 = b_lo; j0 < b_hi; j0 += kBags) {
    const uint32_t nb = (uint32_t)min((int64_t)kBags, b_hi - j0);
    // loads in the order they are needed, none waited for before grad_out's
    // are issued: bag boundaries, the counts' source, grad_out
    const int64_t o_lo = (int64_t)O[j0 + min(threadIdx.x, nb)];
    const int64_t o_hi = (int64_t)O[j0 + min(threadIdx.x + 1u, nb)];
    uint32_t sv[kSavedPer];  // saved counts: element x = b E + e of the block
    IT r[kPer];              // or the first window of lookups from P0 (full width)
    if (use_saved) {
#pragma unroll
      for (int k = 0; k < kSavedPer; ++k)
        sv[k] = h.saved[j0 * (int64_t)E + min(threadIdx.x + (uint32_t)k * kThreads, nb * E - 1u)];
    } else if (N > 0) {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        r[u] = I[min(P0 + threadIdx.x + (uint32_t)u * kThreads, N - 1u)];
    }
    float gv[kSteps][8][DT];
    const bool full = nb == (uint32_t)kBags && c0 - i + (uint32_t)DT * 16u <= D;  // wave-uniform
    if (full) {
      const float* __restrict__ gblk = h.grad + h.col + j0 * (int64_t)h.dtot;
      const uint32_t loff = 8u * kq * h.dtot + c0;
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float* __restrict__ gk = gblk + (int64_t)(32 * ks + e) * h.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) gv[ks][e][nt] = gk[loff + (uint32_t)nt * 16u];
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t jb = 32u * (uint32_t)ks + 8u * kq + (uint32_t)e;
          const float* __restrict__ grow = h.grad + h.col + (j0 + min(jb, nb - 1u)) * (int64_t)h.dtot;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt)  // (zeroed outside the block below, once loaded)
            gv[ks][e][nt] = grow[min(c0 + (uint32_t)nt * 16u, D - 1u)];
        }
    }
    {  // clear the rows in use
      const uint32_t n4 = nrt * 16u * (uint32_t)kPitch / 4u;
      for (uint32_t x = threadIdx.x; x < n4; x += kThreads)
        reinterpret_cast<uint4*>(&cnt[0][0])[x] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (threadIdx.x <= (uint32_t)kBags)
      s_off[threadIdx.x] = (uint32_t)(o_lo < 0 ? 0 : (o_lo > (int64_t)N ? (int64_t)N : o_lo));
    if (threadIdx.x < (uint32_t)kBags) {
      const int64_t L = o_hi - o_lo;
      s_inv[threadIdx.x] = !mean ? 1.f : (threadIdx.x < nb && L > 0 ? 1.f / (float)L : 0.f);
    }
    // saved counts cap at 65535: a block with a bag that reaches 65536
    // lookups counts its lookups instead (also the barrier, which runs for
    // every block: no short-circuit past it)
    const int any_long = __syncthreads_or(threadIdx.x < nb && o_hi - o_lo >= 65536);
    const bool from_saved = use_saved && !any_long;
    const uint32_t P1 = min(max(s_off[nb], P0), N);  // the block's lookups are [P0, P1)
    if (from_saved) {
#pragma unroll
      for (int k = 0; k < kSavedPer; ++k) {
        const uint32_t x = threadIdx.x + (uint32_t)k * kThreads;
        if (x < nb * E) cnt[x % E][x / E] = sv[k];
      }
    } else {
      if (use_saved && N > 0) {  // (the first window was not loaded)
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          r[u] = I[min(P0 + threadIdx.x + (uint32_t)u * kThreads, N - 1u)];
      }
      for (uint32_t q0 = P0; q0 < P1; q0 += (uint32_t)(kPer * kThreads)) {
        // lookups past the block's end are dropped where first needed
        // (an index outside [0, E), by its full value, counts nowhere)
        uint32_t row[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          row[u] = (q0 + threadIdx.x + (uint32_t)u * kThreads < P1 &&
                    (uint64_t)(int64_t)r[u] < (uint64_t)E)
                       ? (uint32_t)r[u]
                       : 0xffffffffu;
        const uint32_t qn = q0 + (uint32_t)(kPer * kThreads);
        if (qn < P1) {
#pragma unroll
          for (int u = 0; u < kPer; ++u)
            r[u] = I[min(qn + threadIdx.x + (uint32_t)u * kThreads, P1 - 1u)];
        }
        // the last bag whose start is at or before p (s_off[m] for m >= nb is
        // the block's end, past every p counted here)
        uint32_t bag[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) bag[u] = 0u;
#pragma unroll
        for (uint32_t step = (uint32_t)kBags / 2u; step > 0u; step >>= 1) {
#pragma unroll
          for (int u = 0; u < kPer; ++u) {
            const uint32_t m = bag[u] + step;
            bag[u] = s_off[m] <= q0 + threadIdx.x + (uint32_t)u * kThreads ? m : bag[u];
          }
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if (row[u] < E) atomicAdd(&cnt[row[u]][bag[u]], 1u);
      }
    }
    // a bag of more than 255 lookups may hold a count wider than 8 bits
    const bool wide = __syncthreads_or(threadIdx.x < nb &&
                                       s_off[threadIdx.x + 1] - s_off[threadIdx.x] > 255u);
    if (threadIdx.x < E) {  // row totals of the block
#pragma unroll
      for (int b4 = 0; b4 < kBags / 4; ++b4) {
        const uint4 c4 = *reinterpret_cast<const uint4*>(&cnt[threadIdx.x][4 * b4]);
        rowtot += c4.x + c4.y + c4.z + c4.w;
      }
    }
    if (!full) {  // bags past nb and columns past D contribute nothing
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) {
            const uint32_t jb = 32u * (uint32_t)ks + 8u * kq + (uint32_t)e;
            const uint32_t keep = (jb < nb && c0 + (uint32_t)nt * 16u < D) ? 0xffffffffu : 0u;
            gv[ks][e][nt] = __uint_as_float(__float_as_uint(gv[ks][e][nt]) & keep);
          }
    }
    if (mean) {  // G scaled by 1/L of its bag
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) {
        const cm_f4 i0 = *reinterpret_cast<const cm_f4*>(&s_inv[32 * ks + 8 * kq]);
        const cm_f4 i1 = *reinterpret_cast<const cm_f4*>(&s_inv[32 * ks + 8 * kq + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) gv[ks][e][nt] *= e < 4 ? i0[e & 3] : i1[e & 3];
      }
    }
    cm_counts_x_grad<kSteps, DT, kRT, kPitch>(acc, cnt, gv, nrt, wide, i, kq);
    P0 = s_off[nb];  // the next block's first lookup
    __syncthreads();  // the counts are cleared (and s_off rewritten) for the next block
  }
  // partial of this workgroup: rows 16 rt + 4 kq + r, column c0 + 16 nt
  float* part = h.part + (size_t)blockIdx.x * E * h.pstride;
#pragma unroll
  for (int rt = 0; rt < kRT; ++rt) {
    if ((uint32_t)rt >= nrt) break;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      const uint32_t col = c0 + (uint32_t)nt * 16u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t row = (uint32_t)rt * 16u + 4u * kq + (uint32_t)q;
        if (row < E && col < D) part[(size_t)row * h.pstride + col] = acc[rt][nt][q];
      }
    }
  }
  if (threadIdx.x < E) h.pcnt[(size_t)blockIdx.x * E + threadIdx.x] = rowtot;
}

// One workgroup per row e: the row's gradient from the nwg partials, then
// row-wise Adagrad if the row has a lookup.  Thread t sums column t mod D2
// (D2 = D rounded up to a power of two) of partials w = t / D2 + S * k (S =
// 256 / D2 stripes), eight accumulators interleaved (32 loads in flight,
// then eight, then one) and combined in a fixed tree; stripes are combined
// in ascending order.
template <int WD>
__global__ __launch_bounds__(kThreads) void bwd_hist_update_kernel(HistArgs h) {
  __shared__ float red[kThreads];
  __shared__ float wsq[kThreads / kWave];
  const uint32_t e = blockIdx.x;
  const uint32_t D = h.D, E = h.E;
  uint32_t D2 = 16;
  while (D2 < D) D2 <<= 1;
  const uint32_t S = kThreads / D2;
  const uint32_t c = threadIdx.x % D2, stripe = threadIdx.x / D2;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < D) {
    const float* base = h.part + (size_t)e * h.pstride + c;
    const size_t wstep = (size_t)E * h.pstride;
    uint32_t w = stripe;
    for (; w + 31u * S < h.nwg; w += 32u * S) {  // 32 loads in flight, added in a fixed order
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = base[(size_t)(w + (uint32_t)u * S) * wstep];
#pragma unroll
      for (int u = 0; u < 32; ++u) acc[u & 7] += v[u];
    }
    for (; w + 7u * S < h.nwg; w += 8u * S) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = base[(size_t)(w + (uint32_t)u * S) * wstep];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[u];
    }
    for (; w < h.nwg; w += S) acc[0] += base[(size_t)w * wstep];
  }
  red[threadIdx.x] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  // touched: some workgroup counted a lookup of the row
  bool any = false;
  for (uint32_t w = threadIdx.x; w < h.nwg; w += kThreads) any |= h.pcnt[(size_t)w * E + e] != 0u;
  const int touched = __syncthreads_or(any ? 1 : 0);
  float g = 0.f, sq = 0.f;
  if (threadIdx.x < D) {
    for (uint32_t s = 0; s < S; ++s) g += red[s * D2 + threadIdx.x];
    sq = g * g;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) sq += __shfl_xor(sq, o, kWave);
  if (lane_id() == 0) wsq[threadIdx.x / kWave] = sq;
  __syncthreads();
  if (!touched) return;  // untouched rows are not written
  const TableDev td = h.table;
  const float m = gload(td.m + e) + (((wsq[0] + wsq[1]) + wsq[2]) + wsq[3]) / (float)D;
  const float den = sqrtf(m) + h.eps;
  if (threadIdx.x < D) {
    const int64_t idx = (int64_t)e * D + threadIdx.x;
    float w;
    if constexpr (WD == WD_F32) {
      w = reinterpret_cast<const float*>(td.w)[idx];
      reinterpret_cast<float*>(td.w)[idx] = w - (h.lr * g) / den;
    } else {
      const uint16_t bits = reinterpret_cast<const uint16_t*>(td.w)[idx];
      w = WD == WD_F16 ? f16_bits_to_float(bits) : bf16_bits_to_float(bits);
      const float o = w - (h.lr * g) / den;
      reinterpret_cast<uint16_t*>(td.w)[idx] =
          WD == WD_F16 ? float_to_f16_bits(o) : float_to_bf16_bits(o);
    }
  }
  __syncthreads();  // every thread has read td.m[e] before it changes
  if (threadIdx.x == 0) {
    gstore(td.m + e, m);
    if (h.debug_count) atomicAdd(&h.debug_count[td.key_base + e], 1u);
  }
}

}  // namespace

hipError_t launch_backward_hist(const HistArgs& h, int itype, int wd, hipStream_t s) {
  if (h.B <= 0 || h.E == 0) return hipSuccess;
  const dim3 grid(h.nwg), block(kThreads);
  if (h.psw) {
    if (itype == IT_I32)
      TBE_LAUNCH("bwd_hist_partial", bwd_hist_weighted_kernel<int32_t>, grid, block, s, h);
    else
      TBE_LAUNCH("bwd_hist_partial", bwd_hist_weighted_kernel<int64_t>, grid, block, s, h);
  } else if (h.D <= 64) {
    if (itype == IT_I32)
      TBE_LAUNCH("bwd_hist_partial", (bwd_hist_count_kernel<int32_t, 1>), grid, block, s, h);
    else
      TBE_LAUNCH("bwd_hist_partial", (bwd_hist_count_kernel<int64_t, 1>), grid, block, s, h);
  } else {
    if (itype == IT_I32)
      TBE_LAUNCH("bwd_hist_partial", (bwd_hist_count_kernel<int32_t, 2>), grid, block, s, h);
    else
      TBE_LAUNCH("bwd_hist_partial", (bwd_hist_count_kernel<int64_t, 2>), grid, block, s, h);
  }
  if (wd == WD_F32)
    TBE_LAUNCH("bwd_hist_update", bwd_hist_update_kernel<WD_F32>, dim3(h.E), dim3(kThreads), s,
               h);
  else if (wd == WD_F16)
    TBE_LAUNCH("bwd_hist_update", bwd_hist_update_kernel<WD_F16>, dim3(h.E), dim3(kThreads), s,
               h);
  else
    TBE_LAUNCH("bwd_hist_update", bwd_hist_update_kernel<WD_BF16>, dim3(h.E), dim3(kThreads), s,
               h);
  return hipGetLastError();
}

}  // namespace tbe
