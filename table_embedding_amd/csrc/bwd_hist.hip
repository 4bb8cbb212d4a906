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
// gfx950 design.  bwd_hist_partial: each workgroup loops over blocks of
// kHBags bags; two threads per bag sum the first and the second half of its
// lookups' coefficients, in lookup order, into two LDS copies added in a
// fixed order (deterministic, no float atomics), and count lookups per row;
// wave w multiplies rows [16w, 16w + 16) of C^T by the block's grad_out rows
// with v_mfma_f32_16x16x4f32 (fp32 inputs: no fp16 split of grad_out; counts
// and scales are exact in fp32), accumulating in registers across blocks, and
// writes its partial [E x D] and row counts.  bwd_hist_update: a workgroup
// per row sums the partials in a fixed order (four interleaved accumulators
// per stripe, stripes combined in order) and applies row-wise Adagrad to rows
// with at least one lookup.  Determinism: every sum is in a data-determined
// order, so repeated calls give the same bits.
//
// Reuse of the forward's histogram (tbe_forward_preprocess with
// TBE_FWD_SAVE_HIST, then this backward with TBE_BWD_PREPROCESSED): the
// coefficients of a block's bags come from the saved uint16 row counts
// (C4: 8.4 MB) instead of the indices (67 MB of int64).  Without per-sample
// weights both paths form a bag's coefficient the same way, count times
// (1/L if mean) as one float32 count divided by L, so they give the same
// bits; a block with a bag of 65536 lookups or more, or counts saved for
// another batch (the header's {B, N} differ), takes the indices.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kHBags = 128;  // bags (K) per block
constexpr int kHRows = 64;   // most rows
constexpr int kHCols = 128;  // widest row

typedef float float4v __attribute__((ext_vector_type(4)));

template <typename IT>
__global__ __launch_bounds__(kThreads) void bwd_hist_partial_kernel(HistArgs h) {
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
    const bool from_saved = use_saved && !__syncthreads_or(wide ? 1 : 0);  // also the barrier
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

// One workgroup per row e: the row's gradient from the nwg partials, then
// row-wise Adagrad if the row has a lookup.  Thread t sums column t mod D2
// (D2 = D rounded up to a power of two) of partials w = t / D2 + S * k (S =
// 256 / D2 stripes), eight accumulators interleaved (eight loads in flight)
// and combined in a fixed tree; stripes are combined in ascending order.
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
  if (itype == IT_I32)
    TBE_LAUNCH("bwd_hist_partial", bwd_hist_partial_kernel<int32_t>, dim3(h.nwg),
               dim3(kThreads), s, h);
  else
    TBE_LAUNCH("bwd_hist_partial", bwd_hist_partial_kernel<int64_t>, dim3(h.nwg),
               dim3(kThreads), s, h);
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
