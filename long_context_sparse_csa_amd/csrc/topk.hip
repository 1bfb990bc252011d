// Top-k selection with ties to the lower entry index.
//
// Pages: a top-k selector keeps only the best-scoring compressed entries for
// core attention, k = 1024 in V4-Pro ("DeepSeek-V4: Making a Million Tokens
// Affordable", section "Two ways to shrink attention, interleaved"; "DeepSeek-V4,
// explained", step 4).  Below the budget nothing is dropped ("DeepSeek-V4,
// explained", introduction).
//
// Design: exact selection, no sorting.  Scores map to order-preserving
// 32-bit keys (NaN -> 0, never selected).  A row of up to 16384 keys is
// selected by one workgroup in LDS.  A longer row is first cut into parts of
// 1024 scores, one wave each, over the whole chip: each part takes as its
// threshold x_p the 16th largest of its 64 lane maxima (a bitwise search over
// one ballot per bit; x_p is at most the part's 16th largest key) and stores
// its keys >= x_p in position order, at most 32, recording the largest key it
// had to leave out.  The per-row workgroup then
//   1. selects the top-k of the stored keys (in position order); their k-th
//      largest lo, the k-th largest of a subset of the row, is <= the row's
//      k-th largest;
//   2. checks every part: one with x_p <= lo that left out no key >= lo
//      stored every key >= lo.  If every part passes (the usual case: a part
//      rarely holds dozens of the row's top 1024) the selection is the
//      answer;
//   3. otherwise selects again over the stored keys of the complete parts and
//      every key >= lo of the others (re-read), which contains the row's
//      top-k.
// More than 16384 candidates are taken in chunks: the top-k of what has been
// seen so far is kept and merged with the next chunk, which keeps position
// order and so the tie rule.  The exact selection is a bucket select: each
// pass bins the live key range [lo, hi] linearly into at most 2048 LDS-atomic
// buckets (from the actual min and max, so clustered scores still spread),
// keeps the bucket holding the k-th key and stops when it is one key wide or
// needed whole -- at most three passes for 32-bit keys; a position-ordered
// stream compaction then writes every key above the bucket and the
// lowest-positioned keys inside it, so the output comes out in ascending
// index order.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kHistBins = 2048;
constexpr int kSelRounds = kTopkSel / kSelThreads;
static_assert(kSelRounds * kSelWaves <= kSelThreads, "one scan entry per thread");
constexpr int kBucketsPerThread = kHistBins / kSelThreads;
static_assert(kTopkPartLen == 16 * 64, "a part is at most 16 keys per lane of one wave");

// Rows up to kTopkSel keys are selected by one workgroup straight from the
// scores; for a small k a row of more than 2048 keys is spread over part
// waves first (each part's leaders hold every one of its keys in the row's
// top 16, so the per-row step sees ~32 keys a part instead of 1024).
TopkPlan topk_plan(int64_t vmin, int64_t vmax, int k) {
  TopkPlan p;
  p.direct_max = k <= 32 ? 2048 : kTopkSel;
  p.parts = vmax > p.direct_max;
  // a row's part count is largest at its own length or just below a length
  // where the part length halves
  int64_t np = 0;
  auto consider = [&](int64_t V) {
    if (V <= 0) return;
    const int P = topk_part_len(V, k);
    np = std::max(np, (V + P - 1) / P);
  };
  consider(vmax);
  for (int P = kTopkPartLen; P > kTopkPartMin; P >>= 1) {   // P halves below V = k P / 4
    const int64_t v = (int64_t)k * P / 4 - 1;
    if (v >= vmin && v <= vmax) consider(v);
  }
  p.nparts = p.parts ? (int)np : 0;
  return p;
}

__device__ __forceinline__ int64_t visible_of(const TopkArgs& a, int64_t qr) {
  const int Tq = a.Tq;   // rows below 2^31 take 32-bit divisions
  const int64_t b = qr < (1ll << 31) ? (int64_t)((uint32_t)qr / (uint32_t)Tq) : qr / Tq;
  const int64_t t = (a.ragged ? a.pos.p[b] : a.q_pos0) + (qr - b * Tq);
  const int64_t v = (uint64_t)(t + 1) < (1ull << 31) ? (int64_t)((uint32_t)(t + 1) / (uint32_t)a.m)
                                                     : (t + 1) / a.m;
  return v < a.n_entries ? v : a.n_entries;
}

// Every argument read in one round at the top of a kernel, before any
// branch: each dependent round trip to the argument segment costs a memory
// latency, and the compiler would otherwise issue the reads where they are
// first used, one round after another (the empty asm statements pin them).
__device__ __forceinline__ void read_args(const TopkArgs& a) {
  asm volatile("" ::"s"(a.scores), "s"(a.score_stride), "s"(a.q_pos0), "s"(a.n_entries),
               "s"(a.direct_max), "s"(a.part_tau), "s"(a.part_cnt), "s"(a.part_over));
  asm volatile("" ::"s"(a.cand_key), "s"(a.cand_idx), "s"(a.topk), "s"(a.topk_score),
               "s"(a.run_key), "s"(a.Tq), "s"(a.m), "s"(a.k), "s"(a.nparts), "s"((int)a.ragged));
}

// Parts of a row of V entries with parts of P (a power of two) entries.
__device__ __forceinline__ int64_t parts_of(int64_t V, int P) {
  return (V + P - 1) >> __builtin_ctz((unsigned)P);
}

// Exclusive scan of one value per thread across the block; returns the
// prefix and writes the block total to *total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan_i(v, 0, [](int a, int b) { return a + b; });
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = s_wave[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}


// The keys of lane `lane` in the part starting at `base` of row qr:
// positions base + 64r + lane for r < P / 64 (absent past the part
// and past the row's visible entries).  part_loads issues the loads and
// returns how many of the part's keys exist; part_keys turns the loaded
// scores into keys once they are needed.  The loads go through one buffer
// resource over the part's scores: they share the lane's offset (each with
// its own immediate offset), and a read past the part returns 0 without a
// memory access, so no per-load address arithmetic or clamping is needed.
__device__ __forceinline__ int part_loads(const TopkArgs& a, int64_t qr, int64_t V, int64_t base,
                                          int P, int lane, float (&f)[16]) {
  // every caller's part is the same across the wave: say so, so that the
  // buffer resource is a scalar one
  base = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)base) |
         ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32);
  int64_t end = base + P;
  if (end > V) end = V;
  const int n = end > base ? (int)(end - base) : 0;   // the part's keys (none past the row)
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(a.scores + qr * a.score_stride + base, (uint32_t)n * 4u);
  const uint32_t lo = (uint32_t)lane * 4u;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    f[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, lo + 256u * r, 0, 0));
  return n;
}

__device__ __forceinline__ void part_keys(const float (&f)[16], int n, int lane,
                                          unsigned (&key)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) key[r] = lane < n - 64 * r ? score_key(f[r]) : 0u;
}

__device__ __forceinline__ void load_part(const TopkArgs& a, int64_t qr, int64_t V, int64_t base,
                                          int P, int lane, unsigned (&key)[16]) {
  float f[16];
  const int n = part_loads(a, qr, V, base, P, lane, f);
  part_keys(f, n, lane, key);
}

// ---- part leaders: x_p = the 16th largest lane maximum (0 if fewer than 16
// lanes hold a valid key), then the part's keys >= max(x_p, 1) in position
// order, the first kTopkPartCap stored, the largest of the rest recorded.
__global__ __launch_bounds__(256) void topk_part_kernel(TopkArgs a) {
  read_args(a);
  // the wave index as a scalar: the part's buffer resources are then
  // uniform (no per-lane waterfall around each buffer access)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t qr = blockIdx.y;
  const int64_t V = visible_of(a, qr);
  if (V <= a.direct_max) return;   // such a row is selected directly
  const int P = topk_part_len(V, a.k);
  const int np = (int)parts_of(V, P);
  // A wave takes parts p, p + stride, ... of its row (one part a wave when
  // the grid spans the row's parts; several when rows are many), the next
  // part's loads in flight while it works on the current one.  A part past
  // the row loads nothing (its buffer range is empty).
  const int stride = (int)gridDim.x * 4;
  int p = blockIdx.x * 4 + wave;
  if (p >= np) return;   // past this row's parts
  float f[16];
  int n = part_loads(a, qr, V, (int64_t)p * P, P, lane, f);
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (; p < np; p += stride) {
    unsigned key[16];
    part_keys(f, n, lane, key);
    n = part_loads(a, qr, V, (int64_t)(p + stride) * P, P, lane, f);   // the next part
    const int64_t base = (int64_t)p * P;
    unsigned x = 0u, over = 0u;
    int cnt = 0;
    unsigned lmax = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) lmax = max(lmax, key[r]);
    // largest x with at least 16 lane maxima >= x, one bit at a time
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = x | (1u << bit);
      if (__popcll(__ballot(lmax >= cand)) >= 16) x = cand;
    }
    const unsigned thr = x > 0u ? x : 1u;
    // the part's candidate slots through buffer resources (32-bit offsets,
    // no 64-bit address arithmetic per store)
    const int64_t cbase = ((int64_t)qr * a.nparts + p) * kTopkPartCap;
    const __amdgpu_buffer_rsrc_t rk = buf_rsrc(a.cand_key + cbase, kTopkPartCap * 4u);
    const __amdgpu_buffer_rsrc_t ri = buf_rsrc(a.cand_idx + cbase, kTopkPartCap * 4u);
    const int ib = (int)base + lane;   // parts start below 2^31
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool pass = key[r] >= thr;
      const unsigned long long bl = __ballot(pass);
      const int pos = cnt + __popcll(bl & lt);
      if (pass && pos < kTopkPartCap) {
        __builtin_amdgcn_raw_buffer_store_b32(key[r], rk, (uint32_t)pos * 4u, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32((unsigned)(ib + 64 * r), ri, (uint32_t)pos * 4u, 0, 0);
      } else if (pass) {
        over = max(over, key[r]);
      }
      cnt += __popcll(bl);
    }
    over = wave_max_u(over);
    if (lane == 0) {
      a.part_tau[qr * a.nparts + p] = x;
      a.part_cnt[qr * a.nparts + p] = cnt;
      a.part_over[qr * a.nparts + p] = over;
    }
  }
}

// ---- select: exact top-k of one row in LDS (every row length; the rows
// that the fast path in topk_select_kernel settles never get here).  Kept
// here as a function of its own.
__device__ __forceinline__ void topk_select_general(const TopkArgs& a, unsigned* smem) {
  unsigned* s_key = smem;                                   // [kTopkSel]
  unsigned* s_hist = smem + kTopkSel;                       // [kHistBins]
  int* s_idx = reinterpret_cast<int*>(s_hist + kHistBins);  // [kTopkSel]
  int* s_off = s_idx + kTopkSel;                            // [nparts + 1] (parts path)
  unsigned* s_raw = reinterpret_cast<unsigned*>(s_off + kTopkMaxParts + 1);  // [nparts / 32]
  __shared__ int s_wave[kSelWaves];
  __shared__ unsigned s_mm[2][kSelWaves];
  __shared__ int s_blk[2][kSelRounds * kSelWaves];  // per (round, wave) block
  __shared__ unsigned s_sel[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t qr = blockIdx.x;
  const int64_t V = visible_of(a, qr);
  const int k = a.k;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  int32_t* topk = a.topk + qr * k;
  float* tks = a.topk_score ? a.topk_score + qr * k : nullptr;

  // Select the top-k of s_key[0, len) (0 = absent) and hand each selected
  // (position, key, index) to out(), positions in ascending index order.
  // Returns how many were selected (min(k, present keys)); *lower gets the
  // k-th largest present key (1 when at most k keys are present).
  // out_key (nullable: then the scores go to topk_score, if given) and
  // out_idx receive the selection; one instantiation for every use.
  auto select = [&](int len, unsigned* lower, unsigned* out_key, int32_t* out_idx) -> int {
    // this thread's keys, positions tid + r * threads, held in registers
    const int nrounds = (len + kSelThreads - 1) / kSelThreads;
    unsigned kr[kSelRounds];
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      const int i = r * kSelThreads + tid;
      kr[r] = (r < nrounds && i < len) ? s_key[i] : 0u;
    }
    int nvalid = 0;
    unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      const unsigned key = kr[r];
      nvalid += key != 0u;
      kmin = key != 0u ? min(kmin, key) : kmin;
      kmax = max(kmax, key);
    }
    kmin = wave_min_u(kmin);
    kmax = wave_max_u(kmax);
    if (lane == 0) {
      s_mm[0][wave] = kmin;
      s_mm[1][wave] = kmax;
    }
    int total_valid;
    (void)block_excl_scan(nvalid, s_wave, &total_valid);
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      kmin = min(kmin, s_mm[0][w]);
      kmax = max(kmax, s_mm[1][w]);
    }
    // bucket select: the kept keys form the contiguous key range [lo, hi]
    const bool all = total_valid <= k;
    unsigned lo = kmin, hi = kmax;
    int need = all ? total_valid : k;
    if (!all) {
      while (true) {
        const unsigned span = hi - lo;   // width - 1
        int shift = 0;
        while ((span >> shift) >= (unsigned)kHistBins) ++shift;
        const int nb = (int)(span >> shift) + 1;   // <= kHistBins
        for (int i = tid; i < nb; i += kSelThreads) s_hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kSelRounds; ++r) {
          const unsigned key = kr[r];
          if (key != 0u && key >= lo && key <= hi) atomicAdd(&s_hist[(key - lo) >> shift], 1u);
        }
        __syncthreads();
        // thread t owns buckets nb-1-B*t .. nb-B*t-B (high buckets first)
        int loc = 0;
#pragma unroll
        for (int u = 0; u < kBucketsPerThread; ++u) {
          const int d = nb - 1 - (kBucketsPerThread * tid + u);
          loc += d >= 0 ? (int)s_hist[d] : 0;
        }
        int tot;
        int above = block_excl_scan(loc, s_wave, &tot);
#pragma unroll
        for (int u = 0; u < kBucketsPerThread; ++u) {
          const int d = nb - 1 - (kBucketsPerThread * tid + u);
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
    // Stream compaction in position order: round r covers positions
    // [r*threads, (r+1)*threads); (round, wave) blocks are in position
    // order.  Pass A counts each block's keys above the bucket and in it,
    // one scan turns that into first output slots and tie ranks, pass B
    // hands out the selected keys.
    auto is_gt = [&](unsigned key) { return all ? key != 0u : (key != 0u && key > hi); };
    auto is_eq = [&](unsigned key) { return !all && key != 0u && key >= lo && key <= hi; };
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      if (r < nrounds) {
        const unsigned long long bg = __ballot(is_gt(kr[r])), be = __ballot(is_eq(kr[r]));
        if (lane == 0) {
          s_blk[0][r * kSelWaves + wave] = __popcll(bg);
          s_blk[1][r * kSelWaves + wave] = __popcll(be);
        }
      }
    }
    __syncthreads();
    {
      const int e = tid;   // block (round e / waves, wave e % waves), position order
      const bool own = e < nrounds * kSelWaves;
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
    unsigned smin = 0xFFFFFFFFu;   // smallest selected key
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      if (r < nrounds) {
        const unsigned key = kr[r];
        const bool gt = is_gt(key), eq = is_eq(key);
        const unsigned long long bg = __ballot(gt), be = __ballot(eq);
        const int e = r * kSelWaves + wave;
        const int sel_before = s_blk[0][e], eq_before = s_blk[1][e];
        const int eq_lt = __popcll(be & lt_mask);
        if (gt || (eq && eq_before + eq_lt < need)) {
          int take_lt = need - eq_before;
          take_lt = take_lt < 0 ? 0 : (take_lt > eq_lt ? eq_lt : take_lt);
          const int pos = sel_before + __popcll(bg & lt_mask) + take_lt;
          out_idx[pos] = s_idx[r * kSelThreads + tid];
          if (out_key) out_key[pos] = key;
          else if (tks) tks[pos] = key_score(key);
          smin = min(smin, key);
        }
      }
    }
    smin = wave_min_u(smin);
    if (lane == 0) s_mm[0][wave] = smin;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) smin = min(smin, s_mm[0][w]);
    *lower = all ? 1u : smin;   // the k-th largest present key
    __syncthreads();
    return all ? total_valid : k;
  };

  auto final_out = [&](int pos, unsigned key, int idx) {
    topk[pos] = idx;
    if (tks) tks[pos] = key_score(key);
  };
  auto pad = [&](int n_sel) {
    for (int q = n_sel + tid; q < k; q += kSelThreads) {
      topk[q] = -1;
      if (tks) tks[q] = -INFINITY;
    }
  };
  unsigned lower;

  if (V <= a.direct_max) {
    // the whole row in LDS
    const int len = (int)(V > 0 ? V : 0);
    const float* src = a.scores + qr * a.score_stride;
    // every load in flight before the first use (a loop of load -> store
    // would wait out the memory latency once per round)
    float sv[kSelRounds];
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      const int i = r * kSelThreads + tid;
      sv[r] = i < len ? src[i] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kSelRounds; ++r) {
      const int i = r * kSelThreads + tid;
      if (i < len) {
        s_key[i] = score_key(sv[r]);
        s_idx[i] = i;
      }
    }
    __syncthreads();
    pad(select(len, &lower, nullptr, topk));
    return;
  }

  const int ns = a.nparts;                       // part slots per row (strides)
  const int P = topk_part_len(V, a.k);
  const int np = (int)((V + P - 1) / P);          // this row's parts
  const int ppt = (np + kSelThreads - 1) / kSelThreads;   // parts per thread (<= 8)
  const unsigned* ptau = a.part_tau + qr * ns;
  const int* pcnt = a.part_cnt + qr * ns;
  const unsigned* pover = a.part_over + qr * ns;
  // this thread's parts' records, loaded up front (their latency overlaps
  // the first selection instead of sitting before the offsets and the check)
  constexpr int kMaxPpt = (kTopkMaxParts + kSelThreads - 1) / kSelThreads;
  int my_cnt[kMaxPpt];
  unsigned my_tau[kMaxPpt], my_over[kMaxPpt];
#pragma unroll
  for (int u = 0; u < kMaxPpt; ++u) {
    const int q = tid * ppt + u;
    const bool own = u < ppt && q < np;
    my_cnt[u] = own ? pcnt[q] : 0;
    my_tau[u] = own ? ptau[q] : 0u;
    my_over[u] = own ? pover[q] : 0u;
  }
  const unsigned* ck = a.cand_key + qr * (int64_t)ns * kTopkPartCap;
  const int* ci = a.cand_idx + qr * (int64_t)ns * kTopkPartCap;
  unsigned* rk = a.run_key + qr * k;

  // Offsets of the parts' candidates given each part's count (cnt_of).
  // cnt_of(u, q): the count of this thread's u-th part q
  auto offsets = [&](auto cnt_of) -> int {
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kMaxPpt; ++u) {
      const int q = tid * ppt + u;
      mine += (u < ppt && q < np) ? cnt_of(u, q) : 0;
    }
    int C;
    int off = block_excl_scan(mine, s_wave, &C);
#pragma unroll
    for (int u = 0; u < kMaxPpt; ++u) {
      const int q = tid * ppt + u;
      if (u < ppt && q < np) {
        s_off[q] = off;
        off += cnt_of(u, q);
      }
    }
    if (tid == 0) s_off[np] = C;
    __syncthreads();
    return C;
  };
  auto is_raw = [&](int q) { return (s_raw[q >> 5] >> (q & 31)) & 1u; };

  // Select over the candidates s_off describes: a part's candidates are its
  // stored leaders, or (raw parts) its keys >= thr re-read in position order.
  // Taken in chunks of what fits beside the running selection.
  auto run_select = [&](unsigned thr, bool any_raw, unsigned* low) -> int {
    const int C = s_off[np];
    int run = 0;   // keys of the partial selection, kept in rk / topk between chunks
    for (int c0 = 0;;) {
      const int take = min(C - c0, kTopkSel - run);
      for (int i = tid; i < run; i += kSelThreads) {
        s_key[i] = rk[i];
        s_idx[i] = topk[i];
      }
      // stored leaders: thread t copies parts t, t + threads, ..., clipped to
      // candidates [c0, c0 + take); all 32 slots of a part are loaded at once
      static_assert(kTopkPartCap == 32, "eight 16-byte loads per part");
      // two threads a part, 16 slots each
      for (int h2 = tid; h2 < 2 * np; h2 += kSelThreads) {
        const int q = h2 >> 1, half = h2 & 1;
        const int o0 = s_off[q], cq = s_off[q + 1] - o0;
        if (is_raw(q) || o0 + cq <= c0 || o0 >= c0 + take || 16 * half >= cq) continue;
        u32x4 kk[4], ii[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kk[u] = *reinterpret_cast<const u32x4*>(ck + q * kTopkPartCap + 16 * half + 4 * u);
          ii[u] = *reinterpret_cast<const u32x4*>(ci + q * kTopkPartCap + 16 * half + 4 * u);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int e = o0 + 16 * half + j;
          if (16 * half + j < cq && e >= c0 && e < c0 + take) {
            s_key[run + e - c0] = kk[j >> 2][j & 3];
            s_idx[run + e - c0] = (int)ii[j >> 2][j & 3];
          }
        }
      }
      for (int q = wave; any_raw && q < np; q += kSelWaves) {
        const int o0 = s_off[q], o1 = s_off[q + 1];
        if (!is_raw(q) || o1 <= c0 || o0 >= c0 + take) continue;
        unsigned key[16];
        const int64_t base = (int64_t)q * P;
        load_part(a, qr, V, base, P, lane, key);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool pass = key[r] >= thr;
          const unsigned long long bl = __ballot(pass);
          const int e = o0 + cnt + __popcll(bl & lt_mask);
          if (pass && e >= c0 && e < c0 + take) {
            s_key[run + e - c0] = key[r];
            s_idx[run + e - c0] = (int)(base + 64 * r + lane);
          }
          cnt += __popcll(bl);
        }
      }
      __syncthreads();
      const int len = run + take;
      c0 += take;
      if (c0 >= C) return select(len, low, nullptr, topk);
      unsigned dummy;
      run = select(len, &dummy, rk, topk);
      __threadfence_block();
      __syncthreads();
    }
  };

  // 1. the stored leaders of every part
  for (int w = tid; w < (np + 31) / 32; w += kSelThreads) s_raw[w] = 0u;
  __syncthreads();
  (void)offsets([&](int u, int) { return min(my_cnt[u], kTopkPartCap); });
  int n_sel = run_select(0u, false, &lower);
  // 2. parts that may hold keys >= lower they did not store (pover is 0 when
  // nothing was left out, and lower >= 1)
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kMaxPpt; ++u) {
    const int q = tid * ppt + u;
    if (u < ppt && q < np && (my_tau[u] > lower || my_over[u] >= lower)) {
      atomicOr(&s_raw[q >> 5], 1u << (q & 31));
      ++bad;
    }
  }
  int nbad;
  (void)block_excl_scan(bad, s_wave, &nbad);
  if (nbad == 0) {
    pad(n_sel);
    return;
  }
  // 3. again over the complete parts' leaders and every key >= lower of the
  // others (the parts' counts first, in s_idx, one wave per re-read part)
  const unsigned thr = lower;
  for (int q = tid; q < np; q += kSelThreads) s_idx[q] = min(pcnt[q], kTopkPartCap);
  __syncthreads();
  for (int q = wave; q < np; q += kSelWaves) {
    if (!is_raw(q)) continue;
    unsigned key[16];
    load_part(a, qr, V, (int64_t)q * P, P, lane, key);
    int c = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) c += __popcll(__ballot(key[r] >= thr));
    if (lane == 0) s_idx[q] = c;
  }
  __syncthreads();
  (void)offsets([&](int, int q) { return s_idx[q]; });
  pad(run_select(thr, true, &lower));
}

// ---- the per-row kernel.  Fast path (rows of at most kSelThreads parts):
// the parts' stored leaders sit in registers, part q's slots with threads
// q*TPP .. q*TPP+TPP-1 (KPT = 32/TPP slots each, in position order), so
// thread order is the row's position order.  A bucket select over the
// registers finds the k-th largest leader lo; one scan over the threads then
// places each thread's selected leaders.  If every part stored all its keys
// >= lo (the check of step 2 of the general path) this is the answer;
// otherwise, and for every other row, the general path runs.  Rows of at
// most kSelThreads/2 parts take two threads a part (half the serial work
// per thread).
template <int KPT>
__device__ __forceinline__ bool topk_select_fast(const TopkArgs& a, unsigned* smem, int64_t qr,
                                                 int np) {
  constexpr int TPP = kTopkPartCap / KPT;   // threads per part
  unsigned* s_key = smem;                                   // [kTopkSel + 64]
  unsigned* s_hist = smem + kTopkSel;                       // [kHistBins]
  int* s_idx = reinterpret_cast<int*>(s_hist + kHistBins);  // [kTopkSel + 64]
  __shared__ int s_wave[kSelWaves];
  __shared__ unsigned s_mm[2][kSelWaves];
  __shared__ unsigned s_sel[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ns = a.nparts;   // part slots per row
  const int k = a.k;
  int32_t* topk = a.topk + qr * k;
  float* tks = a.topk_score ? a.topk_score + qr * k : nullptr;
  const unsigned* ck = a.cand_key + qr * (int64_t)ns * kTopkPartCap;
  const int* ci = a.cand_idx + qr * (int64_t)ns * kTopkPartCap;
  const int q = tid / TPP, s0 = (tid % TPP) * KPT;   // part, first slot
  const bool own = q < np;
  const bool lead = own && s0 == 0;                     // the part's record holder
  // Every record and leader load is issued before any is used (a load in a
  // branch is waited for at once): a thread past the row's parts reads part
  // np - 1's (np >= 1 here) and drops it.
  const int qc = own ? q : np - 1;
  const int cnt_raw = a.part_cnt[qr * ns + qc];
  const unsigned tau_raw = a.part_tau[qr * ns + qc];
  const unsigned over_raw = a.part_over[qr * ns + qc];
  u32x4 kk[KPT / 4], ii[KPT / 4];
#pragma unroll
  for (int u = 0; u < KPT / 4; ++u) {
    kk[u] = *reinterpret_cast<const u32x4*>(ck + qc * kTopkPartCap + s0 + 4 * u);
    ii[u] = *reinterpret_cast<const u32x4*>(ci + qc * kTopkPartCap + s0 + 4 * u);
  }
  const int cpart = own ? min(cnt_raw, kTopkPartCap) : 0;
  const int cq = max(0, min(cpart - s0, KPT));          // this thread's stored leaders
  const unsigned tau = lead ? tau_raw : 0u;
  const unsigned over = lead ? over_raw : 0u;
  unsigned key[KPT];
  int idx[KPT];
#pragma unroll
  for (int u = 0; u < KPT / 4; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[4 * u + e] = 4 * u + e < cq ? kk[u][e] : 0u;
      idx[4 * u + e] = (int)ii[u][e];
    }
  // range of the present leaders and their number
  unsigned kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    kmin = key[j] != 0u ? min(kmin, key[j]) : kmin;
    kmax = max(kmax, key[j]);
  }
  kmin = wave_min_u(kmin);
  kmax = wave_max_u(kmax);
  if (lane == 0) {
    s_mm[0][wave] = kmin;
    s_mm[1][wave] = kmax;
  }
  int total;
  (void)block_excl_scan(cq, s_wave, &total);
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kmin = min(kmin, s_mm[0][w]);
    kmax = max(kmax, s_mm[1][w]);
  }
  // bucket select: the kept keys form the contiguous key range [lo, hi]
  const bool all = total <= k;
  unsigned lo = kmin, hi = kmax;
  int need = all ? total : k;
  if (!all) {
    while (true) {
      const unsigned span = hi - lo;
      int shift = 0;
      while ((span >> shift) >= (unsigned)kHistBins) ++shift;
      const int nb = (int)(span >> shift) + 1;
      for (int i = tid; i < nb; i += kSelThreads) s_hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (key[j] != 0u && key[j] >= lo && key[j] <= hi) atomicAdd(&s_hist[(key[j] - lo) >> shift], 1u);
      __syncthreads();
      int loc = 0;
#pragma unroll
      for (int u = 0; u < kBucketsPerThread; ++u) {
        const int d = nb - 1 - (kBucketsPerThread * tid + u);
        loc += d >= 0 ? (int)s_hist[d] : 0;
      }
      int tot;
      int above = block_excl_scan(loc, s_wave, &tot);
#pragma unroll
      for (int u = 0; u < kBucketsPerThread; ++u) {
        const int d = nb - 1 - (kBucketsPerThread * tid + u);
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
  // per thread: keys above the bucket (key > hi_e) and in it
  // (lo_e <= key <= hi); in-bucket keys go to the lowest positions first.
  // With every leader kept, hi_e = 0 (present keys are >= 1) and no key is
  // in the bucket.  Branch-free: a key that is not taken is written to a
  // per-lane slot past the selection area.
  const unsigned hi_e = all ? 0u : hi, lo_e = all ? 0xFFFFFFFFu : lo;
  int ngt = 0, neq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    ngt += key[j] > hi_e ? 1 : 0;
    neq += (key[j] >= lo_e && key[j] <= hi) ? 1 : 0;
  }
  int tot;
  const int eq_before = block_excl_scan(neq, s_wave, &tot);
  int take = need - eq_before;
  take = take < 0 ? 0 : (take > neq ? neq : take);
  int pos = block_excl_scan(ngt + take, s_wave, &tot);
  // the selection goes to LDS first (a part's slots are contiguous there),
  // then out in coalesced rows
  const int dummy = kTopkSel + lane;   // s_key / s_idx slots past the selection
  unsigned smin = 0xFFFFFFFFu;
  int taken = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool eq = key[j] >= lo_e && key[j] <= hi;
    const bool sel = key[j] > hi_e || (eq && taken < take);
    const int slot = sel ? pos : dummy;
    s_key[slot] = key[j];
    s_idx[slot] = idx[j];
    pos += sel ? 1 : 0;
    taken += eq ? 1 : 0;
    smin = sel ? min(smin, key[j]) : smin;
  }
  smin = wave_min_u(smin);
  if (lane == 0) s_mm[0][wave] = smin;
  __syncthreads();
  const int n_out = all ? total : k;
  for (int i = tid; i < n_out; i += kSelThreads) {
    topk[i] = s_idx[i];
    if (tks) tks[i] = key_score(s_key[i]);
  }
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) smin = min(smin, s_mm[0][w]);
  const unsigned low = all ? 1u : smin;   // the k-th largest leader
  // step 2's check
  const int bad = (lead && (tau > low || over >= low)) ? 1 : 0;
  int nbad;
  (void)block_excl_scan(bad, s_wave, &nbad);
  if (nbad == 0) {
    for (int i = n_out + tid; i < k; i += kSelThreads) {
      topk[i] = -1;
      if (tks) tks[i] = -INFINITY;
    }
    return true;
  }
  __syncthreads();
  return false;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkArgs a) {
  extern __shared__ unsigned smem[];
  read_args(a);
  const int64_t qr = blockIdx.x;
  const int64_t V = visible_of(a, qr);
  const int np = V > a.direct_max ? (int)parts_of(V, topk_part_len(V, a.k)) : 0;
  if (V > a.direct_max && np <= kSelThreads / 2) {
    if (topk_select_fast<kTopkPartCap / 2>(a, smem, qr, np)) return;
  } else if (V > a.direct_max && np <= kSelThreads) {
    if (topk_select_fast<kTopkPartCap>(a, smem, qr, np)) return;
  }
  topk_select_general(a, smem);
}


// devices (bit d: device d < 64) on which the select kernel's dynamic LDS
// limit has been raised; the attribute is set once per device, the first
// time a launch there needs it (setting it twice is harmless)
static std::atomic<uint64_t> g_topk_attr_devices{0};

hipError_t launch_topk(const TopkArgs& a, const TopkPlan& plan, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  if (rows == 0) return hipSuccess;
  const size_t lds =
      (size_t)(2 * kTopkSel + kHistBins + kTopkMaxParts + 1 + kTopkMaxParts / 32) * sizeof(unsigned);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (!bit || !(g_topk_attr_devices.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)topk_select_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    g_topk_attr_devices.fetch_or(bit, std::memory_order_release);
  }
  if (plan.parts) {
    // one part a wave over the chip when the rows are few (decode); with
    // more than ~64K parts in all, four parts a wave, each wave's next part
    // loading while it works on the current one
    const int ppw = (int64_t)plan.nparts * rows > 65536 ? 4 : 1;
    const dim3 grid((unsigned)((plan.nparts + 4 * ppw - 1) / (4 * ppw)), (unsigned)rows);
    topk_part_kernel<<<grid, 256, 0, st>>>(a);
  }
  topk_select_kernel<<<(unsigned)rows, kSelThreads, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace v4
