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
// runs an MSB-first radix select (11/11/10-bit digits, histograms with LDS
// atomics, one block scan per pass) that fixes the exact k-th key tau and how
// many of its ties are needed; it stops early once a digit bucket is needed
// whole.  A stream compaction in position order then writes every key above
// tau and the lowest-positioned ties, so the output comes out in ascending
// index order without a sort.  Longer rows are cut into parts: the union of
// the parts' exact top-k always contains the row's top-k, so a second pass
// over the candidates (at most 16384 for a million-token context) finishes
// the job.  Candidates keep position order, which keeps the tie rule exact.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kHistBins = 2048;

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

// Exclusive scan of one value per thread across the block (512 threads);
// returns the prefix and writes the block total to *total.
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
  __shared__ int s_cnt[2][kTopkWaves][2];
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

  // load keys (and candidate indices) into LDS, count present keys.  All of
  // a thread's 16-byte loads are issued before any is consumed, so the part
  // arrives in about one memory latency instead of one per element.
  int nvalid = 0;
  constexpr int U = kTopkPart / 4 / kTopkThreads;
  const int64_t src0 = FIRST ? qr * score_stride + beg : qr * in_stride + beg;
  const bool vec = FIRST ? (score_stride & 3) == 0 : (in_stride & 3) == 0;
  const int len4 = vec ? (len >> 2) : 0;
  if (len4 > 0) {
    // unconditional loads (indices past the part re-read its last vector),
    // so every load of the thread is in flight at once
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
        nvalid += (k4.x != 0u) + (k4.y != 0u) + (k4.z != 0u) + (k4.w != 0u);
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
    nvalid += key != 0u;
  }
  int total_valid;
  (void)block_excl_scan(nvalid, s_wave, &total_valid);  // also syncs after the LDS writes

  // radix select: find prefix (pbits bits) of the k-th key and the ties needed
  const bool all = total_valid <= k;
  unsigned prefix = 0;
  int pbits = 0;
  int need = all ? total_valid : k;
  if (!all) {
    for (int pass = 0; pass < 3; ++pass) {
      const int bits = pass < 2 ? 11 : 10;
      const int nb = 1 << bits;
      const int shift = 32 - pbits - bits;
      for (int i = tid; i < nb; i += kTopkThreads) s_hist[i] = 0u;
      __syncthreads();
      for (int i = tid; i < len; i += kTopkThreads) {
        const unsigned key = s_key[i];
        const bool in_group = key != 0u && (pbits == 0 || (key >> (32 - pbits)) == prefix);
        if (in_group) atomicAdd(&s_hist[(key >> shift) & (unsigned)(nb - 1)], 1u);
      }
      __syncthreads();
      // thread t owns digits nb-1-per*t down to nb-per*(t+1) (high digits first)
      const int per = nb / kTopkThreads;
      int loc = 0;
      for (int u = 0; u < per; ++u) loc += (int)s_hist[nb - 1 - (per * tid + u)];
      int tot;
      int above = block_excl_scan(loc, s_wave, &tot);
      for (int u = 0; u < per; ++u) {
        const int d = nb - 1 - (per * tid + u);
        const int cnt = (int)s_hist[d];
        if (above < need && above + cnt >= need) {
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
      prefix = (prefix << bits) | d;
      pbits += bits;
      if (cnt_eq == need) break;  // the whole bucket is selected
    }
  }

  // stream compaction in position order
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  int base_sel = 0, base_eq = 0;
  const int n_sel_total = all ? total_valid : k;
  for (int r0 = 0, rnd = 0; r0 < len; r0 += kTopkThreads, ++rnd) {
    const int i = r0 + tid;
    const unsigned key = i < len ? s_key[i] : 0u;
    bool gt, eq;
    if (all) {
      gt = key != 0u;
      eq = false;
    } else {
      const unsigned top = key >> (32 - pbits);
      gt = key != 0u && top > prefix;
      eq = key != 0u && top == prefix;
    }
    const unsigned long long bg = __ballot(gt), be = __ballot(eq);
    const int par = rnd & 1;
    if (lane == 0) {
      s_cnt[par][wave][0] = __popcll(bg);
      s_cnt[par][wave][1] = __popcll(be);
    }
    __syncthreads();
    int sel_before = 0, eq_before = base_eq, rnd_sel = 0, rnd_eq = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const int cg = s_cnt[par][w][0], ce = s_cnt[par][w][1];
      int take = need - (base_eq + rnd_eq);
      take = take < 0 ? 0 : (take > ce ? ce : take);
      if (w < wave) {
        sel_before += cg + take;
        eq_before += ce;
      }
      rnd_sel += cg + take;
      rnd_eq += ce;
    }
    const int my_eq_rank = eq_before + __popcll(be & lt_mask);
    const bool sel = gt || (eq && my_eq_rank < need);
    if (sel) {
      int take_lt = need - eq_before;
      const int eq_lt = __popcll(be & lt_mask);
      take_lt = take_lt < 0 ? 0 : (take_lt > eq_lt ? eq_lt : take_lt);
      const int pos = base_sel + sel_before + __popcll(bg & lt_mask) + take_lt;
      const int idx = FIRST ? (int)(beg + i) : s_idx[i];
      if (last) {
        topk[qr * k + pos] = idx;
        if (topk_score) topk_score[qr * k + pos] = key_score(key);
      } else {
        out_key[qr * out_stride + (int64_t)part * k + pos] = key;
        out_idx[qr * out_stride + (int64_t)part * k + pos] = idx;
      }
    }
    base_sel += rnd_sel;
    base_eq += rnd_eq;
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
