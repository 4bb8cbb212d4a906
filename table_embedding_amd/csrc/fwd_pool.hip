// Generic forward gather-pool (FBTriton TBE page, "Forward": each bag gathers
// its indexed rows and pools them; 16-bit weights accumulate in float32 and
// float32 weights in float64; tables are bucketed by next_pow2(D) so narrow
// tables do not idle lanes sized for the widest one, section "Fewer reads and
// synchronizations").
//
// Lane mapping: a subgroup of `lpr` lanes covers one row; lane k holds
// columns k*VEC + c*lpr*VEC (c < NC), read with 16-byte (VEC element) loads,
// so a row of the bucket width is one coalesced sweep of the subgroup.
//
// Balance (fwd_bal_kernel, the default): a wave owns G = fwd_group_bags(lpr,
// bps) consecutive bags of one table (their lookups are contiguous) and
// splits the group's lookups into 64/lpr equal pieces in lookup order, one
// per subgroup, cutting through bags.  With one bag per subgroup a wave lasts
// as long as its longest bag while the other subgroups idle (C2's lengths,
// uniform in [1, 64], leave about half the lanes idle); with equal pieces
// every subgroup issues the same number of loads.  A subgroup streams its
// piece in order.  A bag that starts and ends in the piece is written by it
// directly; a bag cut by piece boundaries is summed per piece (the piece
// where it starts and every piece it fills keep their part in LDS, the piece
// where it ends adds those parts in piece order to its own and writes the
// row), so every bag has one writer, plain stores, and a sum order fixed by
// the offsets alone: repeated calls give the same bits.  bps (1, 2 or 4 bags
// per subgroup and wave) trades evenness for the number of waves; the host
// picks it from the batch size.  fwd_pool_kernel (TBE_FWD_NO_BALANCE) gives
// each subgroup one whole bag and sums it in lookup order.
//
// Memory-level parallelism: lookups are taken eight at a time.  The eight
// indices are loaded, then the eight rows, then the eight rows are
// accumulated in lookup order; scheduling barriers keep the compiler from
// sinking each row load next to its use, which would leave one row in flight.
// A partial last batch repeats the last index and drops the repeats with a
// select (the repeated row is a cache hit).  The indices of the next batch
// load while the rows of the current one are in flight.
//
// Fused input checks (CHK, tbe_forward_checked; FBTriton page, "Forward":
// bounds checks fused into the forward, off by default).  Offsets are clamped
// into [0, N] as they are read and, inside a wave's bag group, made
// non-decreasing by a running maximum; an index outside [0, R_t) (an int64
// one by its full value) is replaced by row 0 and its contribution dropped,
// so the bag keeps its length for mean pooling.  Every access then stays
// inside the inputs and outputs.  Findings go to the error block with the
// conventions of tbe_validate (bits, bad-index count, first bag, first bad
// position); valid inputs give the unchecked kernel's bits.
#include "tbe_common.h"

namespace tbe {
namespace {

constexpr int kInFlight = 8;

template <int WD>
struct Acc {
  using T = float;
};
template <>
struct Acc<WD_F32> {
  using T = double;
};

// acc + s*v with one rounding, written out so that every forward kernel
// rounds the same way whatever the compiler would contract (a padded slot
// has s = 0 and leaves acc unchanged).
__device__ __forceinline__ float fma_acc(float s, float v, float acc) {
  return __builtin_fmaf(s, v, acc);
}
__device__ __forceinline__ double fma_acc(double s, float v, double acc) {
  return __builtin_fma(s, (double)v, acc);
}

// Offset findings of bag j (lo = O[j], hi = O[j+1], as stored) with
// tbe_validate's conventions: the start offset belongs to bag 0, the end
// offset to the last bag.
__device__ __forceinline__ uint32_t offset_bits(int64_t lo, int64_t hi, uint64_t j,
                                                uint64_t nbag, int64_t n) {
  uint32_t bits = 0;
  if (j == 0 && lo != 0) bits |= kValOffsetStart;
  if (j + 1 == nbag && hi != n) bits |= kValOffsetEnd;
  if (lo > hi) bits |= kValOffsetOrder;
  if (lo < 0 || lo > n || hi < 0 || hi > n) bits |= kValOffsetRange;
  return bits;
}
__device__ __forceinline__ void report_offsets(uint32_t* err, uint32_t bits, uint64_t j) {
  atomicOr(&err[kValBits], bits);
  atomicMin(&err[kValFirstBag], (uint32_t)j);
}
__device__ __forceinline__ void report_index(uint32_t* err, uint32_t pos, uint64_t j) {
  atomicOr(&err[kValBits], kValIndexRange);
  atomicAdd(&err[kValBadIndices], 1u);
  atomicMin(&err[kValFirstPos], pos);
  atomicMin(&err[kValFirstBag], (uint32_t)j);
}
__device__ __forceinline__ int64_t clamp_n(int64_t o, int64_t n) {
  return o < 0 ? 0 : (o > n ? n : o);
}

template <int WD, int VEC, int NC, typename IT, bool PSW, bool CHK>
__global__ __launch_bounds__(kThreads) void fwd_bal_kernel(FwdArgs a, BucketSet S) {
  using AT = typename Acc<WD>::T;
  constexpr uint32_t kWaves = kThreads / kWave;
  // fragments exist only with two or more subgroups per wave, hence NC == 1
  constexpr uint32_t kFrag = NC == 1 ? (uint32_t)kWave * VEC : 1u;
  __shared__ uint32_t s_off[kWaves][kWave + 1];
  __shared__ AT s_tail[kWaves][kFrag];  // [subgroup * width + column]
  __shared__ AT s_head[kWaves][kFrag];
  BucketDev bk;
  uint32_t bucket_id, lb, lg;
  set_pick(S, bk, bucket_id, lb, lg);
  // the wave index is uniform: say so, so that the table descriptor and the
  // buffer descriptors built from it live in scalar registers
  const uint32_t lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t lpr = bk.lpr, lg2 = bk.lpr_log2;
  const uint32_t nsub = (uint32_t)kWave >> lg2;
  const uint32_t sgi = lane >> lg2, lane_in = lane & (lpr - 1);
  const uint32_t G = fwd_group_bags(lpr, a.bps);
  const uint64_t B = (uint64_t)a.B;
  const uint64_t gpt = (B + G - 1) / G;  // bag groups per table
  const uint64_t wv = (uint64_t)lb * kWaves + wave;
  if (wv >= gpt * (uint64_t)bk.ntables) return;  // the whole wave; only wave-level syncs follow
  const uint32_t slot = (uint32_t)(wv / gpt);
  const uint64_t g0 = (wv - (uint64_t)slot * gpt) * G;
  const uint32_t nbw = (uint32_t)((B - g0) < (uint64_t)G ? (B - g0) : (uint64_t)G);
  const uint32_t t = bk.tables[slot];
  const TableDev td = a.tables[t];
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const uint64_t j0 = (uint64_t)t * B + g0;
  const uint32_t D = td.dim;

  // offsets of the group's bags: off[q] = O[j0 + q], q = 0 .. nbw (positions < 2^31)
  uint32_t* off = s_off[wave];
  if constexpr (CHK) {
    // each offset read once, checked, clamped into [0, N] and made
    // non-decreasing by a running maximum over the group
    const int64_t n64 = (int64_t)a.n;
    const int64_t o = lane <= nbw ? (int64_t)O[j0 + lane] : 0;
    const int64_t o64 = (int64_t)O[j0 + nbw];  // the group's end offset (lane nbw's, or the 65th)
    int64_t nx = __shfl_down(o, 1, kWave);     // O[j0 + lane + 1]
    if (lane + 1 == nbw) nx = o64;
    const uint64_t nbag = (uint64_t)a.T * B;
    const uint32_t bits = lane < nbw ? offset_bits(o, nx, j0 + lane, nbag, n64) : 0u;
    const uint64_t bad = __ballot(bits != 0u);
    if (bad) {
      const uint32_t first = (uint32_t)__builtin_ctzll(bad);
      uint32_t all = bits;
#pragma unroll
      for (int m = 1; m < kWave; m <<= 1) all |= __shfl_xor(all, m, kWave);
      if (lane == first) report_offsets(a.err, all, j0 + lane);
    }
    uint32_t c = (uint32_t)clamp_n(o, n64);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {  // inclusive running maximum in lane order
      const uint32_t y = __shfl_up(c, d, kWave);
      if (lane >= (uint32_t)d) c = y > c ? y : c;
    }
    if (lane <= nbw) off[lane] = c;
    if (nbw == (uint32_t)kWave && lane == kWave - 1) {
      const uint32_t e = (uint32_t)clamp_n(o64, n64);
      off[kWave] = e > c ? e : c;
    }
  } else {
    if (lane <= nbw) off[lane] = (uint32_t)O[j0 + lane];
    if (nbw == (uint32_t)kWave && lane == 0) off[kWave] = (uint32_t)O[j0 + kWave];
  }
  wave_lds_sync();

  // This subgroup's piece [plo, phi) of the group's lookups: equal shares in
  // lookup order, cutting through bags.  Its bag ends are the bags whose last
  // lookup lies in the piece (and subgroup 0 also the empty bags at the start;
  // the last non-empty piece the empty bags at the end).
  const uint32_t P0 = off[0], Pe = off[nbw];
  const uint32_t tot = Pe - P0;
  uint32_t share = (tot + nsub - 1) / nsub;
  share = share > 0 ? share : 1u;
  const uint32_t plo = sgi * share < tot ? P0 + sgi * share : Pe;
  const uint32_t phi = (sgi + 1) * share < tot ? P0 + (sgi + 1) * share : Pe;
  uint32_t cur = 0;  // bag being summed
  if (sgi > 0) {
    if (plo < phi) {  // the bag holding position plo: the last q with off[q] <= plo
      uint32_t lo = 0, hi = nbw;
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (off[mid] <= plo) lo = mid; else hi = mid;
      }
      cur = lo;
    } else {
      cur = nbw;  // an empty piece past the end: nothing to do
    }
  }
  uint32_t nxt = cur < nbw ? off[cur + 1] : Pe;  // its end

  AT acc[NC][VEC];
  bool act[NC];
  uint32_t colc[NC], cold[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[c][v] = AT(0);
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
    act[c] = colc[c] < D;
    cold[c] = act[c] ? colc[c] : 0u;  // idle lanes read column 0 and discard it
  }
  const bool mean = td.pooling == POOL_MEAN;
  const uint32_t fbase = sgi * lpr * VEC;  // this subgroup's fragment slot
  // 32-bit byte offsets (the host sends tables and index arrays under 4 GiB
  // here); an int64 index is read as its low word (rows < 2^32)
  constexpr uint32_t kEs = WD == WD_F32 ? 4u : 2u;
  const __amdgpu_buffer_rsrc_t wres = buf_rsrc(td.w, td.rows * D * kEs);
  const __amdgpu_buffer_rsrc_t ires = buf_rsrc(a.indices, a.n * (uint32_t)sizeof(IT));
  const __amdgpu_buffer_rsrc_t pres = buf_rsrc(a.psw, PSW ? a.n * 4u : 0u);
  const uint32_t rowb = D * kEs;
  uint32_t colb[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) colb[c] = cold[c] * kEs;
  // write bag q's pooled row from its sums v (mean: divided by its length)
  auto write_row = [&](uint32_t q, const AT (*v)[VEC]) {
    const uint32_t L = off[q + 1] - off[q];
    float* orow = a.out + (int64_t)(g0 + q) * (int64_t)a.dtot + td.col;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!act[c]) continue;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        o[e] = (float)((mean && L > 0) ? v[c][e] / AT(L) : v[c][e]);
      store_f32<VEC>(orow + colc[c], o);
    }
  };
  // bag q ends in this piece: written out if it started in the piece, else
  // its last part is kept for the combination below
  uint32_t head_bag = nbw;
  auto end_bag = [&](uint32_t q) {
    bool whole = true;
    if constexpr (NC == 1) {
      if (off[q] < plo) {
        head_bag = q;
        whole = false;
#pragma unroll
        for (int e = 0; e < VEC; ++e) s_head[wave][fbase + colc[0] + e] = acc[0][e];
      }
    }
    if (whole) write_row(q, acc);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[c][e] = AT(0);
  };

  const uint32_t pb = plo, pe = phi;
  // CHK with int64 indices: the high word too (an index is valid only if it is 0)
  constexpr bool kHi = CHK && sizeof(IT) == 8;
  uint32_t nrow[kInFlight], nhi[kInFlight];
  float ns[kInFlight];
  if (pb < pe) {
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const uint32_t q = pb + k < pe ? pb + k : pe - 1;
      nrow[k] = buf_u32(ires, q * (uint32_t)sizeof(IT));
      nhi[k] = kHi ? buf_u32(ires, q * (uint32_t)sizeof(IT) + 4u) : 0u;
      ns[k] = PSW ? __builtin_bit_cast(float, buf_u32(pres, q * 4u)) : 1.0f;
    }
  }
  for (uint32_t p = pb; p < pe; p += kInFlight) {
    uint32_t row[kInFlight];
    float s[kInFlight];
    bool ok[kInFlight], use[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      row[k] = nrow[k];
      s[k] = ns[k];
      ok[k] = p + k < pe;
      use[k] = ok[k];
    }
    if constexpr (CHK) {
      bool any = false;
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) {
        const bool bad = ok[k] && (nhi[k] != 0u || row[k] >= td.rows);
        use[k] = ok[k] && !bad;
        row[k] = bad ? 0u : row[k];
        any |= bad;
      }
      if (__ballot(any && lane_in == 0)) {  // rare: report each bad lookup once
        if (lane_in == 0) {
#pragma unroll
          for (int k = 0; k < kInFlight; ++k) {
            if (!ok[k] || use[k]) continue;
            const uint32_t pos = p + (uint32_t)k;
            uint32_t lo = 0, hi = nbw;  // its bag: the last q with off[q] <= pos
            while (hi - lo > 1) {
              const uint32_t mid = (lo + hi) >> 1;
              if (off[mid] <= pos) lo = mid; else hi = mid;
            }
            report_index(a.err, pos, j0 + lo);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // NC > 1 only for rows that take all 64 lanes, which get one bag per wave,
    // so a bag can only end inside the c = 0 sweep when NC == 1
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float v[kInFlight][VEC];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) load_w_buf<WD, VEC>(wres, row[k] * rowb + colb[c], v[k]);
      if (c == 0) {
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
          const uint32_t q = p + kInFlight + k < pe ? p + kInFlight + k : pe - 1;
          nrow[k] = buf_u32(ires, q * (uint32_t)sizeof(IT));
          nhi[k] = kHi ? buf_u32(ires, q * (uint32_t)sizeof(IT) + 4u) : 0u;
          ns[k] = PSW ? __builtin_bit_cast(float, buf_u32(pres, q * 4u)) : 1.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) {
        if (NC == 1 && ok[k]) {
          while (p + k >= nxt) {  // lookup p+k opens a later bag: finish the current one(s)
            end_bag(cur);
            ++cur;
            nxt = off[cur + 1];
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[c][e] = fma_acc(use[k] ? AT(s[k]) : AT(0), v[k][e], acc[c][e]);
      }
    }
  }
  // the bags ending at the end of the piece, empty ones included
  for (; cur < nbw && off[cur + 1] <= phi; ++cur) end_bag(cur);
  if constexpr (NC == 1) {
    if (cur < nbw) {  // the current bag goes on: this piece's part of it
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_tail[wave][fbase + colc[0] + e] = acc[0][e];
    }
    if (nsub == 1) return;
    wave_lds_sync();
    if (head_bag < nbw) {
      // a bag that began in piece i0 < sgi: the parts of pieces i0 .. sgi-1
      // (each ends inside the bag) and this piece's part, in piece order
      uint32_t i0 = (off[head_bag] - P0) / share;
      i0 = i0 < sgi ? i0 : sgi;
      AT sum[NC][VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) sum[0][e] = AT(0);
      for (uint32_t k = i0; k < sgi; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) sum[0][e] += s_tail[wave][k * lpr * VEC + colc[0] + e];
#pragma unroll
      for (int e = 0; e < VEC; ++e) sum[0][e] += s_head[wave][fbase + colc[0] + e];
      write_row(head_bag, sum);
    }
  }
}

// One bag per lane subgroup (bps == 1): subgroup sg of the launch pools bag sg
// of the bucket; the offsets and indices load straight from global memory.
template <int WD, int VEC, int NC, typename IT, bool PSW, bool CHK>
__global__ __launch_bounds__(kThreads) void fwd_pool_kernel(FwdArgs a, BucketSet S) {
  using AT = typename Acc<WD>::T;
  BucketDev bk;
  uint32_t bucket_id, lb, lg;
  set_pick(S, bk, bucket_id, lb, lg);
  const uint32_t lpr = bk.lpr;
  const uint32_t lane_in = threadIdx.x & (lpr - 1);
  const uint64_t sg = ((uint64_t)lb * kThreads + threadIdx.x) >> bk.lpr_log2;
  const uint64_t nbags = (uint64_t)bk.ntables * (uint64_t)a.B;
  if (sg >= nbags) return;
  const uint32_t slot = (uint32_t)(sg / (uint64_t)a.B);
  const int64_t b = (int64_t)(sg - (uint64_t)slot * (uint64_t)a.B);
  const uint32_t t = bk.tables[slot];
  const TableDev td = a.tables[t];
  const IT* __restrict__ I = reinterpret_cast<const IT*>(a.indices);
  const IT* __restrict__ O = reinterpret_cast<const IT*>(a.offsets);
  const int64_t j = (int64_t)t * a.B + b;
  int64_t lo = O[j];
  int64_t hi = O[j + 1];
  if constexpr (CHK) {  // checked, then clamped into [0, N] with hi >= lo
    const int64_t n64 = (int64_t)a.n;
    const uint32_t bits = offset_bits(lo, hi, (uint64_t)j, (uint64_t)a.T * (uint64_t)a.B, n64);
    if (bits && lane_in == 0) report_offsets(a.err, bits, (uint64_t)j);
    lo = clamp_n(lo, n64);
    hi = clamp_n(hi, n64);
    hi = hi < lo ? lo : hi;
  }
  const uint32_t D = td.dim;

  AT acc[NC][VEC];
  bool act[NC];
  uint32_t colc[NC], cold[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[c][v] = AT(0);
    colc[c] = (lane_in + (uint32_t)c * lpr) * VEC;
    act[c] = colc[c] < D;
    cold[c] = act[c] ? colc[c] : 0u;  // idle lanes read column 0 and discard it
  }

  // software pipeline: the indices of batch i+1 are loaded while the rows of
  // batch i are in flight, so a batch costs one memory round trip
  int64_t nrow[kInFlight];
  float ns[kInFlight];
  if (lo < hi) {
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const int64_t q = lo + k < hi ? lo + k : hi - 1;
      nrow[k] = (int64_t)I[q];
      ns[k] = PSW ? a.psw[q] : 1.0f;
    }
  }
  for (int64_t p = lo; p < hi; p += kInFlight) {
    int64_t row[kInFlight];
    float s[kInFlight];
    bool ok[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      row[k] = nrow[k];
      s[k] = ns[k];
      ok[k] = p + k < hi;
      if constexpr (CHK) {  // a bad index reads row 0 and contributes nothing
        const bool bad = ok[k] && (uint64_t)row[k] >= (uint64_t)td.rows;
        if (bad && lane_in == 0) report_index(a.err, (uint32_t)(p + k), (uint64_t)j);
        ok[k] = ok[k] && !bad;
        row[k] = bad ? 0 : row[k];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float v[kInFlight][VEC];
#pragma unroll
      for (int k = 0; k < kInFlight; ++k) load_w<WD, VEC>(td.w, row[k] * D + cold[c], v[k]);
      if (c == 0) {
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
          const int64_t q = p + kInFlight + k < hi ? p + kInFlight + k : hi - 1;
          nrow[k] = (int64_t)I[q];
          ns[k] = PSW ? a.psw[q] : 1.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kInFlight; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[c][e] = fma_acc(ok[k] ? AT(s[k]) : AT(0), v[k][e], acc[c][e]);
    }
  }

  const bool mean = td.pooling == POOL_MEAN && hi > lo;
  const AT L = AT(hi - lo);
  float* orow = a.out + b * (int64_t)a.dtot + td.col;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (!act[c]) continue;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = (float)(mean ? acc[c][e] / L : acc[c][e]);
    store_f32<VEC>(orow + colc[c], o);
  }
}

template <int WD, int VEC, int NC, typename IT, bool PSW, bool CHK>
hipError_t launch_c(const FwdArgs& a, const BucketSet& S, hipStream_t s) {
  const uint32_t grid = S.gbeg[S.n];
  if (grid == 0) return hipSuccess;
  if (a.split)
    TBE_LAUNCH("fwd_pool", (fwd_bal_kernel<WD, VEC, NC, IT, PSW, CHK>), dim3(grid),
               dim3(kThreads), s, a, S);
  else
    TBE_LAUNCH("fwd_pool", (fwd_pool_kernel<WD, VEC, NC, IT, PSW, CHK>), dim3(grid),
               dim3(kThreads), s, a, S);
  return hipGetLastError();
}

template <int WD, int VEC, int NC, typename IT, bool PSW>
hipError_t launch_t(const FwdArgs& a, const BucketSet& S, hipStream_t s) {
  return a.err ? launch_c<WD, VEC, NC, IT, PSW, true>(a, S, s)
               : launch_c<WD, VEC, NC, IT, PSW, false>(a, S, s);
}

template <int WD, int VEC, int NC>
hipError_t launch(const FwdArgs& a, const BucketSet& S, hipStream_t s) {
  if (a.itype == IT_I32)
    return a.psw ? launch_t<WD, VEC, NC, int32_t, true>(a, S, s)
                 : launch_t<WD, VEC, NC, int32_t, false>(a, S, s);
  return a.psw ? launch_t<WD, VEC, NC, int64_t, true>(a, S, s)
               : launch_t<WD, VEC, NC, int64_t, false>(a, S, s);
}

}  // namespace

hipError_t launch_forward_set(const FwdArgs& a, const BucketSet& bk, int wd, int vec, int nc,
                              hipStream_t s) {
#define TBE_FWD_CASE(W, V, N) \
  if (wd == W && vec == V && nc == N) return launch<W, V, N>(a, bk, s);
  TBE_FWD_CASE(WD_F32, 4, 1)
  TBE_FWD_CASE(WD_F32, 4, 2)
  TBE_FWD_CASE(WD_F32, 4, 4)
  TBE_FWD_CASE(WD_F16, 4, 1)
  TBE_FWD_CASE(WD_F16, 4, 2)
  TBE_FWD_CASE(WD_F16, 4, 4)
  TBE_FWD_CASE(WD_F16, 8, 1)
  TBE_FWD_CASE(WD_F16, 8, 2)
  TBE_FWD_CASE(WD_BF16, 4, 1)
  TBE_FWD_CASE(WD_BF16, 4, 2)
  TBE_FWD_CASE(WD_BF16, 4, 4)
  TBE_FWD_CASE(WD_BF16, 8, 1)
  TBE_FWD_CASE(WD_BF16, 8, 2)
#undef TBE_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tbe
