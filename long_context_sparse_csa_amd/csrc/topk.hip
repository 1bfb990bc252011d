// Top-k selection with ties to the lower entry index.
//
// Pages: a top-k selector keeps only the best-scoring compressed entries for
// core attention, k = 1024 in V4-Pro ("DeepSeek-V4: Making a Million Tokens
// Affordable", section "Two ways to shrink attention, interleaved"; "DeepSeek-V4,
// explained", step 4).  Below the budget nothing is dropped ("DeepSeek-V4,
// explained", introduction).
//
// Design: exact selection in LDS, no sorting.  Scores map to order-preserving
// 32-bit keys.  A workgroup loads up to 16384 keys of one query into LDS and
// runs a bucket select: each pass bins the live key range [lo, hi] linearly
// into at most 2048 LDS-atomic buckets (starting from the part's actual min
// and max, so a clustered score distribution still spreads over the buckets
// instead of piling onto a few exponent bins), keeps the bucket holding the
// k-th key and stops when it is one key wide or needed whole -- at most three
// passes for 32-bit keys.  A stream compaction in position order then writes every key above
// tau and the lowest-positioned ties, so the output comes out in ascending
// index order without a sort.  Longer rows are cut into parts: the union of
// the parts' exact top-k always contains the row's top-k, so a second pass
// over the candidates (at most 16384 for a million-token context) finishes
// the job.  Candidates keep position order, which keeps the tie rule exact.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 2048;
constexpr int kTopkRounds = kTopkPart / kTopkThreads;
static_assert(kTopkRounds * kTopkWaves <= kTopkThreads, "one scan entry per thread");

TopkPlan topk_plan(int64_t vmax, int k) {
  TopkPlan p;
  p.parts0 = vmax > 0 ? (vmax + kTopkPart - 1) / kTopkPart : 1;
  p.stages = 1;
  int64_t parts = p.parts0;
  p.cand_elems = 0;
  while (parts > 1) {
    const int64_t n = parts * (int64_t)k;
    if (n > p.cand_elems) p.cand_elems = n;
    parts = (n + kTopkPart - 1) / kTopkPart;
    p.stages++;
  }
  return p;
}

// Exclusive scan of one value per thread across the block; returns the
// prefix and writes the block total to *total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int s = s_wave[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__device__ __forceinline__ unsigned wave_min_u(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o));
  return v;
}

template <bool FIRST>
__global__ __launch_bounds__(kTopkThreads) void topk_stage_kernel(
    const float* __restrict__ scores, int64_t score_stride, const unsigned* __restrict__ in_key,
    const int* __restrict__ in_idx, int64_t in_stride, int Tq, int64_t n_entries,
    int64_t q_pos0, int m, int k, int last, unsigned* __restrict__ out_key,
    int* __restrict__ out_idx, int64_t out_stride, int32_t* __restrict__ topk,
    float* __restrict__ topk_score) {
  extern __shared__ unsigned smem[];
  unsigned* s_key = smem;                                   // [kTopkPart]
  unsigned* s_hist = smem + kTopkPart;                      // [kHistBins]
  int* s_idx = reinterpret_cast<int*>(s_hist + kHistBins);  // [kTopkPart] (!FIRST)
  __shared__ int s_wave[kTopkWaves];
  __shared__ unsigned s_mm[2][kTopkWaves];
  __shared__ int s_blk[2][kTopkRounds * kTopkWaves];  // per (round, wave) block
  __shared__ unsigned s_sel[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t qr = blockIdx.y;
  const int part = blockIdx.x;
  int64_t n_in;
  if (FIRST) {
    const int64_t t = q_pos0 + (qr % Tq);
    n_in = (t + 1) / m;
    if (n_in > n_entries) n_in = n_entries;
  } else {
    n_in = in_stride;
  }
  const int64_t beg = (int64_t)part * kTopkPart;
  int len = 0;
  if (n_in > beg) len = (int)((n_in - beg) < kTopkPart ? (n_in - beg) : kTopkPart);

  // load keys (and candidate indices) into LDS; count present keys and take
  // their min and max.  All of a thread's 16-byte loads are issued before any
  // is consumed (indices past the part re-read its last vector).
  int nvalid = 0;
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
  auto note = [&](unsigned key) {
    nvalid += key != 0u;
    if (key != 0u) {
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  };
  constexpr int U = kTopkPart / 4 / kTopkThreads;
  const int64_t src0 = FIRST ? qr * score_stride + beg : qr * in_stride + beg;
  const bool vec = FIRST ? (score_stride & 3) == 0 : (in_stride & 3) == 0;
  const int len4 = vec ? (len >> 2) : 0;
  if (len4 > 0) {
    u32x4 kv[U];
    u32x4 iv[FIRST ? 1 : U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = min(tid + u * kTopkThreads, len4 - 1);
      if (FIRST) {
        kv[u] = *reinterpret_cast<const u32x4*>(scores + src0 + 4 * i4);
      } else {
        kv[u] = *reinterpret_cast<const u32x4*>(in_key + src0 + 4 * i4);
        iv[FIRST ? 0 : u] = *reinterpret_cast<const u32x4*>(in_idx + src0 + 4 * i4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i4 = tid + u * kTopkThreads;
      if (i4 < len4) {
        u32x4 k4 = kv[u];
        if (FIRST) {
          k4.x = score_key(__uint_as_float(k4.x));
          k4.y = score_key(__uint_as_float(k4.y));
          k4.z = score_key(__uint_as_float(k4.z));
          k4.w = score_key(__uint_as_float(k4.w));
        } else {
          *reinterpret_cast<u32x4*>(&s_idx[4 * i4]) = iv[FIRST ? 0 : u];
        }
        *reinterpret_cast<u32x4*>(&s_key[4 * i4]) = k4;
        note(k4.x);
        note(k4.y);
        note(k4.z);
        note(k4.w);
      }
    }
  }
#pragma unroll 8
  for (int i = 4 * len4 + tid; i < len; i += kTopkThreads) {
    unsigned key;
    if (FIRST) {
      key = score_key(scores[src0 + i]);
    } else {
      key = in_key[src0 + i];
      s_idx[i] = in_idx[src0 + i];
    }
    s_key[i] = key;
    note(key);
  }
  kmin = wave_min_u(kmin);
  kmax = wave_max_u(kmax);
  if (lane == 0) {
    s_mm[0][wave] = kmin;
    s_mm[1][wave] = kmax;
  }
  int total_valid;
  (void)block_excl_scan(nvalid, s_wave, &total_valid);  // also syncs after the LDS writes
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    kmin = min(kmin, s_mm[0][w]);
    kmax = max(kmax, s_mm[1][w]);
  }

  // Bucket select: the kept keys form the contiguous key range [lo, hi]; each
  // pass bins that range linearly into at most 2048 buckets (so the bins
  // follow the data, not the exponent bits), keeps the bucket holding the
  // k-th key and accounts for everything above it.  It ends when the bucket
  // is one key wide (ties by position) or needed whole.
  const bool all = total_valid <= k;
  unsigned lo = kmin, hi = kmax;
  int need = all ? total_valid : k;
  if (!all) {
    while (true) {
      const unsigned span = hi - lo;   // width - 1
      int shift = 0;
      while ((span >> shift) >= (unsigned)kHistBins) ++shift;
      const int nb = (int)(span >> shift) + 1;   // <= kHistBins
      for (int i = tid; i < nb; i += kTopkThreads) s_hist[i] = 0u;
      __syncthreads();
#pragma unroll 4
      for (int i = tid; i < len; i += kTopkThreads) {
        const unsigned key = s_key[i];
        if (key != 0u && key >= lo && key <= hi) atomicAdd(&s_hist[(key - lo) >> shift], 1u);
      }
      __syncthreads();
      // thread t owns buckets nb-1-2t and nb-2-2t (high buckets first)
      int loc = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int d = nb - 1 - (2 * tid + u);
        loc += d >= 0 ? (int)s_hist[d] : 0;
      }
      int tot;
      int above = block_excl_scan(loc, s_wave, &tot);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int d = nb - 1 - (2 * tid + u);
        const int cnt = d >= 0 ? (int)s_hist[d] : 0;
        if (d >= 0 && above < need && above + cnt >= need) {
          s_sel[0] = (unsigned)d;
          s_sel[1] = (unsigned)above;
          s_sel[2] = (unsigned)cnt;
        }
        above += cnt;
      }
      __syncthreads();
      const unsigned d = s_sel[0];
      const int cnt_gt = (int)s_sel[1], cnt_eq = (int)s_sel[2];
      __syncthreads();
      need -= cnt_gt;
      const unsigned nlo = lo + (d << shift);
      const uint64_t nhi = (uint64_t)nlo + (1ull << shift) - 1u;
      hi = nhi < (uint64_t)hi ? (unsigned)nhi : hi;
      lo = nlo;
      if (cnt_eq == need || lo == hi) break;
    }
  }

  // Stream compaction in position order.  Round r covers positions
  // [r*threads, (r+1)*threads); (round, wave) blocks are in position order.
  // Pass A counts each block's keys above the bucket and in it with ballots,
  // one scan over the (at most 256) blocks turns that into the first output
  // slot and the first tie rank of every block, and pass B writes.
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  const int n_sel_total = all ? total_valid : k;
  const int nrounds = (len + kTopkThreads - 1) / kTopkThreads;
  auto classify = [&](int i, unsigned& key, bool& gt, bool& eq) {
    key = i < len ? s_key[i] : 0u;
    if (all) {
      gt = key != 0u;
      eq = false;
    } else {
      gt = key != 0u && key > hi;
      eq = key != 0u && key >= lo && key <= hi;
    }
  };
#pragma unroll 4
  for (int rnd = 0; rnd < nrounds; ++rnd) {
    unsigned key;
    bool gt, eq;
    classify(rnd * kTopkThreads + tid, key, gt, eq);
    const unsigned long long bg = __ballot(gt), be = __ballot(eq);
    if (lane == 0) {
      s_blk[0][rnd * kTopkWaves + wave] = __popcll(bg);
      s_blk[1][rnd * kTopkWaves + wave] = __popcll(be);
    }
  }
  __syncthreads();
  {
    const int e = tid;   // block (round e / waves, wave e % waves), position order
    const bool own = e < nrounds * kTopkWaves;
    const int cg = own ? s_blk[0][e] : 0, ce = own ? s_blk[1][e] : 0;
    int tot;
    const int eq_before = block_excl_scan(ce, s_wave, &tot);
    int take = need - eq_before;
    take = take < 0 ? 0 : (take > ce ? ce : take);
    const int sel_before = block_excl_scan(cg + take, s_wave, &tot);
    if (own) {
      s_blk[0][e] = sel_before;
      s_blk[1][e] = eq_before;
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int rnd = 0; rnd < nrounds; ++rnd) {
    const int i = rnd * kTopkThreads + tid;
    unsigned key;
    bool gt, eq;
    classify(i, key, gt, eq);
    const unsigned long long bg = __ballot(gt), be = __ballot(eq);
    const int e = rnd * kTopkWaves + wave;
    const int sel_before = s_blk[0][e], eq_before = s_blk[1][e];
    const int eq_lt = __popcll(be & lt_mask);
    const bool sel = gt || (eq && eq_before + eq_lt < need);
    if (sel) {
      int take_lt = need - eq_before;
      take_lt = take_lt < 0 ? 0 : (take_lt > eq_lt ? eq_lt : take_lt);
      const int pos = sel_before + __popcll(bg & lt_mask) + take_lt;
      const int idx = FIRST ? (int)(beg + i) : s_idx[i];
      if (last) {
        topk[qr * k + pos] = idx;
        if (topk_score) topk_score[qr * k + pos] = key_score(key);
      } else {
        out_key[qr * out_stride + (int64_t)part * k + pos] = key;
        out_idx[qr * out_stride + (int64_t)part * k + pos] = idx;
      }
    }
  }
  // padding
  for (int p = n_sel_total + tid; p < k; p += kTopkThreads) {
    if (last) {
      topk[qr * k + p] = -1;
      if (topk_score) topk_score[qr * k + p] = -INFINITY;
    } else {
      out_key[qr * out_stride + (int64_t)part * k + p] = 0u;
      out_idx[qr * out_stride + (int64_t)part * k + p] = -1;
    }
  }
}

static bool g_topk_attr_set = false;

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& plan, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  const size_t lds_first = (kTopkPart + kHistBins) * sizeof(unsigned);
  const size_t lds_next = lds_first + kTopkPart * sizeof(int);
  if (!g_topk_attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)topk_stage_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_first);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)topk_stage_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_next);
    if (e != hipSuccess) return e;
    g_topk_attr_set = true;
  }
  int64_t parts = plan.parts0;
  int cur = 0;
  {
    const int last = plan.stages == 1;
    dim3 grid((unsigned)parts, (unsigned)rows);
    topk_stage_kernel<true><<<grid, kTopkThreads, lds_first, st>>>(
        a.scores, a.score_stride, nullptr, nullptr, 0, a.Tq, a.n_entries, a.q_pos0, a.m, a.k,
        last, a.cand_key[0], a.cand_idx[0], parts * a.k, a.topk, a.topk_score);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int s = 1; s < plan.stages; ++s) {
    const int64_t n = parts * (int64_t)a.k;
    const int64_t nparts = (n + kTopkPart - 1) / kTopkPart;
    const int last = s == plan.stages - 1;
    dim3 grid((unsigned)nparts, (unsigned)rows);
    topk_stage_kernel<false><<<grid, kTopkThreads, lds_next, st>>>(
        nullptr, 0, a.cand_key[cur], a.cand_idx[cur], n, a.Tq, a.n_entries, a.q_pos0, a.m,
        a.k, last, a.cand_key[cur ^ 1], a.cand_idx[cur ^ 1], nparts * a.k, a.topk,
        a.topk_score);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    parts = nparts;
    cur ^= 1;
  }
  return hipSuccess;
}

}  // namespace v4
