// Shared-KV multi-query core attention over packed compressed entries plus
// the uncompressed window, with per-head sink and inverse output rotation.
//
// Pages: attention over the selected positions only ("DeepSeek-V4,
// explained", step 5); CSA attends to the top-k entries, HCA to every entry,
// both with a 128-token window branch, learnable sinks and a shared-KV
// multi-query layout ("DeepSeek-V4 Explained: Compressed Sparse Attention and
// 1M Context at 10% KV", section "The attention stack, and why it is two
// mechanisms"); RMSNorm on queries, RoPE on the last 64 dims, an entry is key
// and value, RoPE at -i on the output ("DeepSeek-V4: Making a Million Tokens
// Affordable", section "Two ways to shrink attention, interleaved").  The
// window, the entries and the sink share one softmax.
//
// Design.  One workgroup of eight waves owns one query token and one range of
// its rows (entries, then window rows), so every packed row is fetched from
// HBM once for all 64 heads.  Rows are gathered (CSA: through the top-k list)
// 32 at a time with 16-byte coalesced loads, double-buffered through
// registers, and widened once at staging (E4M3 -> bf16 is exact) into a bf16
// LDS tile, so no wave converts anything in its inner loop.  Waves w
// and w+4 share heads 16(w%4)..+15 and split the 512 dims in halves: each
// contracts S over its half (holding only that half of q~), the pair adds the
// two partial S through LDS, both run the same softmax, and each accumulates
// the output for the same half of the dims.  Every wave therefore reads the
// same 288 bytes of each row for both products, and the per-wave registers
// (half of q~, half of the output) leave room for two workgroups per CU.
//   S^T = K q~^T : K rows are the A operand (one 16-byte LDS read per lane),
//                  q~ is the B operand held in registers for the whole kernel;
//                  the result puts one head per lane column and keys down the
//                  lane groups, so the softmax statistics need two cross-lane
//                  steps;
//   O^T += V^T P^T : V^T comes straight from the row-major tile with the
//                  gfx950 transposing LDS read ds_read_b64_tr_b16; the
//                  probabilities stay in the registers the S^T accumulators
//                  left them in, because the MFMA's key order is permuted to
//                  match (k slot j of lane group g = key 4g+j or 16+4g+j-4).
// O^T keeps one head per lane, so the online-softmax rescale needs no
// shuffles, and the running maximum moves only when it grows by more than
// 2^8 (probabilities stay below 256, exact enough in bf16 and fp32), which
// skips almost every rescale.  Long rows are split over several workgroups
// whose (O, max, sum) partials a merge kernel combines with the sink.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kAttTile = 32;      // rows per LDS tile
constexpr int kAttThreads = 512;  // eight waves: four head groups x two halves
constexpr int kMaxTopk = 4096;    // largest k the CSA kernel stages in LDS
constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max moves
constexpr float kNoMax = -1.0e30f; // running-max floor (no key seen yet)

template <int D>
struct AttGeom {
  static constexpr int R = 64;
  static constexpr int ROW = D + R;            // packed bytes per row in HBM
  static constexpr int BSTR = 2 * D + 32;      // bf16 LDS row stride (8-bank shift per row)
  static constexpr int KSTEPS = D / 32;        // 32-dim k-steps of S^T
  static constexpr int KSH = KSTEPS / 2;       // k-steps per half
  static constexpr int DB = D / 16;            // 16-dim blocks of O^T
  static constexpr int DBH = DB / 2;           // blocks per half
  static constexpr int CPR = ROW / 16;         // 16-byte chunks per packed row
  static constexpr int FP8_CPR = (D - R) / 16; // of which E4M3
  static constexpr int CHUNKS = kAttTile * CPR;
  static constexpr int CH = (CHUNKS + kAttThreads - 1) / kAttThreads;
};

struct RowSpace {
  int64_t n_ent;    // entry rows (CSA: k slots; HCA: visible entries)
  int64_t win_lo;   // first window position
  int64_t n_rows;   // entries + window rows
};

__device__ __forceinline__ RowSpace row_space(const AttendArgs& a, bool csa, int64_t t) {
  RowSpace rs;
  if (csa) {
    rs.n_ent = a.k;
  } else {
    int64_t v = (t + 1) / a.m;
    rs.n_ent = v < a.n_entries ? v : a.n_entries;
  }
  int64_t lo = t - a.W + 1;
  rs.win_lo = lo > 0 ? lo : 0;
  const int64_t n_win = a.W > 0 ? (t - rs.win_lo + 1) : 0;
  rs.n_rows = rs.n_ent + n_win;
  return rs;
}

template <int D, bool CSA>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendArgs a) {
  using G = AttGeom<D>;
  constexpr int R = G::R;
  const int qr = blockIdx.y;
  const int split = blockIdx.x;
  const int b = qr / a.Tq, r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave & 3, hf = wave >> 2;   // head group, dim half
  const int g = lane >> 4, c = lane & 15;
  const int head = hg * 16 + c;
  const bool active = hg * 16 < a.H;

  // bf16 tiles: E4M3 dims are widened once here, at staging, not per wave
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kAttTile * G::BSTR];
  __shared__ __attribute__((aligned(16))) f32x4 s_x[8][64][2];  // partial S^T for the pair
  __shared__ unsigned s_valid[2];
  __shared__ float s_cs[R / 2][2];
  __shared__ int s_sel[CSA ? kMaxTopk : 1];  // this split's slice of the top-k list

  const RowSpace rs = row_space(a, CSA, t);
  int64_t chunk = (rs.n_rows + a.splits - 1) / a.splits;
  chunk = (chunk + kAttTile - 1) / kAttTile * kAttTile;
  const int64_t row_beg = (int64_t)split * chunk;
  int64_t row_end = row_beg + chunk;
  if (row_end > rs.n_rows) row_end = rs.n_rows;
  const int ntiles = row_end > row_beg ? (int)((row_end - row_beg + kAttTile - 1) / kAttTile) : 0;
  // split-local row numbers fit in 32 bits; offsets within one sequence's
  // cache fit in 32 bits (checked on the host)
  const int nloc = (int)(row_end - row_beg);
  const int ent_loc = (int)max((int64_t)0, min(rs.n_ent, row_end) - row_beg);  // entry rows here
  const uint8_t* ent_b = a.entries + (int64_t)b * a.Ncap * G::ROW;
  const uint8_t* win_b = a.win + ((int64_t)b * (a.Tq + a.W - 1) +
                                  (rs.win_lo - (a.q_pos0 - (a.W - 1)))) * G::ROW;
  const int64_t win_first = rs.n_ent - row_beg;   // split-local row of the first window row

  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, tid, R, a.rope_base, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  if constexpr (CSA) {
    const int32_t* sel = a.topk + (int64_t)qr * a.k + row_beg;
    for (int x = tid; x < ent_loc; x += kAttThreads) s_sel[x] = sel[x];
    __syncthreads();
  }

  // local row x -> byte offset from its base (32-bit: one sequence's cache is
  // below 4 GiB), or -1 if absent
  const int row_beg32 = (int)row_beg;
  const int win_first32 = (int)win_first;
  auto row_src = [&](int x, const uint8_t*& base) -> int {
    if (x >= nloc) return -1;
    if (x < ent_loc) {
      int j = x + row_beg32;
      if constexpr (CSA) {
        j = s_sel[x];
        if (j < 0 || (int64_t)j >= a.Ncap) return -1;
      }
      base = ent_b;
      return j * G::ROW;
    }
    base = win_b;
    return (x - win_first32) * G::ROW;
  };

  // ---- staging: this thread's chunks u -> (row, 16-byte column), fixed per tile
  int crow[G::CH], ccol[G::CH];
#pragma unroll
  for (int u = 0; u < G::CH; ++u) {
    const int cidx = min(tid + u * kAttThreads, G::CHUNKS - 1);
    crow[u] = cidx / G::CPR;
    ccol[u] = cidx % G::CPR;
  }
  const uint8_t* dummy = a.Ncap > 0 ? a.entries : a.win;
  u32x4 pref[G::CH];
  bool pval[G::CH];
  auto fetch_rows = [&](int tile) {
#pragma unroll
    for (int u = 0; u < G::CH; ++u) {
      const uint8_t* base = ent_b;
      const int off = row_src(tile * kAttTile + crow[u], base);
      pval[u] = (u + 1) * kAttThreads <= G::CHUNKS || tid + u * kAttThreads < G::CHUNKS;
      pval[u] = pval[u] && off >= 0;
      // absent rows read a valid address and are zeroed at the store, so the
      // loads are unconditional and all in flight together
      const uint8_t* src = pval[u] ? base + (unsigned)off + ccol[u] * 16 : dummy;
      pref[u] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_rows = [&](int tile, int buf) {
    uint8_t* T = s_tile[buf];
#pragma unroll
    for (int u = 0; u < G::CH; ++u) {
      if ((u + 1) * kAttThreads <= G::CHUNKS || tid + u * kAttThreads < G::CHUNKS) {
        const int row = crow[u], col = ccol[u];
        const u32x4 v = pval[u] ? pref[u] : u32x4{0u, 0u, 0u, 0u};
        if (col < G::FP8_CPR) {   // 16 E4M3 values -> 16 bf16 (exact)
          const u32x2 lo = fp8x4_to_bf16x4(v.x), hi = fp8x4_to_bf16x4(v.y);
          const u32x2 lo2 = fp8x4_to_bf16x4(v.z), hi2 = fp8x4_to_bf16x4(v.w);
          u32x4* dst = reinterpret_cast<u32x4*>(T + row * G::BSTR + col * 32);
          dst[0] = u32x4{lo.x, lo.y, hi.x, hi.y};
          dst[1] = u32x4{lo2.x, lo2.y, hi2.x, hi2.y};
        } else {                  // 8 bf16 values
          *reinterpret_cast<u32x4*>(T + row * G::BSTR + 2 * (D - R) + (col - G::FP8_CPR) * 16) = v;
        }
      }
    }
    if (tid < 64) {
      const uint8_t* base = ent_b;
      const bool ok = tid < kAttTile && row_src(tile * kAttTile + tid, base) >= 0;
      const unsigned long long m = __ballot(ok);
      if (tid == 0) s_valid[buf] = (unsigned)m;
    }
  };

  if (ntiles > 0) {
    fetch_rows(0);
    store_rows(0, 0);
  }
  __syncthreads();

  // ---- q~ = RoPE_t(RMSNorm(q)) as the B operand: head c, dims ks*32 + g*8 + e
  // for this wave's half of the k-steps (hf*KSH ..)
  constexpr int KSH = G::KSH;
  bf16x8 qb[KSH];
  {
    float ss = 0.f;
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + min(head, a.H - 1)) * D + g * 8;
    u32x4 qv[G::KSTEPS];
    f32x4 gv[KSH][2];   // gamma_q for this wave's dims, loaded with q
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) qv[ks] = *reinterpret_cast<const u32x4*>(qp + ks * 32);
#pragma unroll
    for (int u = 0; u < KSH; ++u) {
      const float* gp = a.gamma_q + (hf * KSH + u) * 32 + g * 8;
      gv[u][0] = *reinterpret_cast<const f32x4*>(gp);
      gv[u][1] = *reinterpret_cast<const f32x4*>(gp + 4);
    }
    if (head >= a.H) {
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) qv[ks] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      const unsigned w[4] = {qv[ks].x, qv[ks].y, qv[ks].z, qv[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_bits_to_f32(w[e] & 0xFFFFu), hi = bf16_bits_to_f32(w[e] >> 16);
        ss += lo * lo + hi * hi;
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rsn = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int u = 0; u < KSH; ++u) {
      const int ks = hf * KSH + u;
      const int d0 = ks * 32 + g * 8;
      u32x4 q4 = qv[0];
#pragma unroll
      for (int kk = 0; kk < G::KSTEPS; ++kk)
        if (kk == ks) q4 = qv[kk];
      const unsigned w[4] = {q4.x, q4.y, q4.z, q4.w};
      const float gm[8] = {gv[u][0].x, gv[u][0].y, gv[u][0].z, gv[u][0].w,
                           gv[u][1].x, gv[u][1].y, gv[u][1].z, gv[u][1].w};
      float qf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[2 * e] = gm[2 * e] * (bf16_bits_to_f32(w[e] & 0xFFFFu) * rsn);
        qf[2 * e + 1] = gm[2 * e + 1] * (bf16_bits_to_f32(w[e] >> 16) * rsn);
      }
      if (d0 >= D - R) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int i = (d0 + e - (D - R)) >> 1;
          const float cs = s_cs[i][0], sn = s_cs[i][1];
          const float x0 = qf[e], x1 = qf[e + 1];
          qf[e] = x0 * cs - x1 * sn;
          qf[e + 1] = x0 * sn + x1 * cs;
        }
      }
      u32x4 pk = {pack_bf16x2(qf[0], qf[1]), pack_bf16x2(qf[2], qf[3]),
                  pack_bf16x2(qf[4], qf[5]), pack_bf16x2(qf[6], qf[7])};
      qb[u] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  const float sl2 = a.scale * kLog2e;
  // running max starts at a finite floor, so masked keys (-inf) give p = 0
  // without special cases; an untouched max marks "no row seen"
  float m_run = kNoMax, l_run = 0.f;  // per head (lane column), log2 units
  f32x4 o[G::DBH];
#pragma unroll
  for (int db = 0; db < G::DBH; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets of the transposing V^T reads (k slot j of lane group
  // g is key 4g+j for j < 4, key 16+4g+j-4 otherwise)
  const int jv16 = (lane & 15) >> 2;
  const int off16a = (4 * g + jv16) * G::BSTR + 8 * (lane & 3);
  const int off16b = (16 + 4 * g + jv16) * G::BSTR + 8 * (lane & 3);
  const int db0 = hf * G::DBH;       // this wave's first output dim block

  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    const bool more = tile + 1 < ntiles;
    if (more) fetch_rows(tile + 1);
    const uint8_t* T = s_tile[cur];
    // partial S^T over this wave's half of the dims, both 16-key blocks
    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (active) {
#pragma unroll
      for (int u = 0; u < KSH; ++u) {
        const int ks = hf * KSH + u;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(T + (kb * 16 + c) * G::BSTR +
                                                          2 * (ks * 32 + g * 8));
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), qb[u],
                                                          s[kb], 0, 0, 0);
        }
      }
    }
    s_x[wave][lane][0] = s[0];
    s_x[wave][lane][1] = s[1];
    __syncthreads();
    if (active) {
      // full S: own half + partner's half (a + b == b + a, so both waves agree)
      f32x4 sk[2];
      sk[0] = s[0] + s_x[wave ^ 4][lane][0];
      sk[1] = s[1] + s_x[wave ^ 4][lane][1];
      // online softmax for head c over this lane's 8 keys: kb*16 + 4g + i
      const unsigned vmask = __builtin_amdgcn_readfirstlane(s_valid[cur]);
      float x[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kb][i] = sk[kb][i] * sl2;
      if (vmask != 0xFFFFFFFFu) {   // partial tile: mask the absent rows
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((vmask >> (kb * 16 + 4 * g + i)) & 1u)) x[kb][i] = -INFINITY;
      }
      float mt = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      // move the running max only when it grows past the headroom
      if (__any(mt > m_run + kLazyMax)) {
        const float m_new = fmaxf(m_run, mt);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= corr;
#pragma unroll
        for (int db = 0; db < G::DBH; ++db) o[db] *= corr;
        m_run = m_new;
      }
      float p[2][4];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(x[kb][i] - m_run);
          ls += p[kb][i];
        }
      l_run += ls;
      const u32x4 pk = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                        pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
      // O^T += V^T P^T for this wave's half of the dims
#pragma unroll
      for (int u = 0; u < G::DBH; ++u) {
        const int dofs = 2 * (db0 + u) * 16;
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((V4_LDS i16x4*)(T + off16a + dofs)));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((V4_LDS i16x4*)(T + off16b + dofs)));
        o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), pb, o[u], 0, 0, 0);
      }
    }
    if (more) store_rows(tile + 1, cur ^ 1);
    __syncthreads();
  }

  if (!active || head >= a.H) return;
  // full denominator of this lane's head: sum the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (a.splits > 1) {
    // unnormalised partial (O, max, sum); the merge kernel adds the sink
    float* po = a.part_o + (((int64_t)qr * a.splits + split) * a.H + head) * D;
#pragma unroll
    for (int u = 0; u < G::DBH; ++u)
      *reinterpret_cast<f32x4*>(po + (db0 + u) * 16 + g * 4) = o[u];
    if (g == 0 && hf == 0) {
      float* pm = a.part_ml + (((int64_t)qr * a.splits + split) * a.H + head) * 2;
      pm[0] = l_run > 0.f ? m_run : -INFINITY;
      pm[1] = l_run;
    }
    return;
  }
  const bool seen = l_run > 0.f;
  const float mr = seen ? m_run : -INFINITY;
  const float z2 = a.sink[head] * kLog2e;
  const float M = fmaxf(mr, z2);
  float scale_o = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    const float wr = seen ? exp2f(mr - M) : 0.f;
    const float den = l_run * wr + exp2f(z2 - M);
    scale_o = wr / den;
    lse = (M + log2f(den)) * 0.69314718055994531f;
  }
  uint16_t* op = a.out + ((int64_t)qr * a.H + head) * D;
#pragma unroll
  for (int u = 0; u < G::DBH; ++u) {
    const int d0 = (db0 + u) * 16 + g * 4;
    float v[4] = {o[u][0] * scale_o, o[u][1] * scale_o, o[u][2] * scale_o, o[u][3] * scale_o};
    if (d0 >= D - R) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const int i = (d0 + e - (D - R)) >> 1;
        const float cs = s_cs[i][0], sn = s_cs[i][1];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs + x1 * sn;       // rotation by -t
        v[e + 1] = -x0 * sn + x1 * cs;
      }
    }
    const u32x2 pkd = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(op + d0) = pkd;
  }
  if (a.lse && g == 0 && hf == 0) a.lse[(int64_t)qr * a.H + head] = lse;
}

// Combine split partials with the sink, rotate by -t, store bf16 and lse.
// Grid: (ceil(H/8), B*Tq); 256 threads; each workgroup owns 8 heads.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a) {
  constexpr int R = 64;
  const int qr = blockIdx.y;
  const int h0 = blockIdx.x * 8;
  const int64_t t = a.q_pos0 + (qr % a.Tq);
  const int S = a.splits;
  __shared__ float s_w[8][64];   // per head, per split weight (splits <= 64)
  __shared__ float s_cs[R / 2][2];
  const int tid = threadIdx.x;
  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, tid, R, a.rope_base, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  if (tid < 8) {
    const int h = h0 + tid;
    if (h < a.H) {
      const float* pm = a.part_ml + ((int64_t)qr * S * a.H + h) * 2;
      const float z2 = a.sink[h] * kLog2e;
      float M = z2;
      for (int s = 0; s < S; ++s) M = fmaxf(M, pm[(int64_t)s * a.H * 2]);
      float den = M == -INFINITY ? 0.f : exp2f(z2 - M);
      for (int s = 0; s < S; ++s) {
        const float ms = pm[(int64_t)s * a.H * 2], ls = pm[(int64_t)s * a.H * 2 + 1];
        const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
        s_w[tid][s] = w;
        den += ls * w;
      }
      const float inv = den > 0.f ? 1.0f / den : 0.f;
      for (int s = 0; s < S; ++s) s_w[tid][s] *= inv;
      if (a.lse) a.lse[(int64_t)qr * a.H + h] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f
                                                           : -INFINITY;
    }
  }
  __syncthreads();
  // each thread: a pair of dims of one head per step
  for (int e = tid; e < 8 * (D / 2); e += 256) {
    const int hh = e / (D / 2), d = 2 * (e % (D / 2));
    const int h = h0 + hh;
    if (h >= a.H) continue;
    float x0 = 0.f, x1 = 0.f;
    const float* po = a.part_o + ((int64_t)qr * S * a.H + h) * D + d;
    for (int s0 = 0; s0 < S; s0 += 8) {   // eight split partials in flight
      f32x2 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const f32x2*>(po + (int64_t)min(s0 + u, S - 1) * a.H * D);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = s0 + u < S ? s_w[hh][s0 + u] : 0.f;
        x0 = fmaf(w, v[u].x, x0);
        x1 = fmaf(w, v[u].y, x1);
      }
    }
    if (d >= D - R) {
      const int i = (d - (D - R)) >> 1;
      const float cs = s_cs[i][0], sn = s_cs[i][1];
      const float y0 = x0 * cs + x1 * sn, y1 = -x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
    }
    *reinterpret_cast<unsigned*>(a.out + ((int64_t)qr * a.H + h) * D + d) = pack_bf16x2(x0, x1);
  }
}

int attend_splits(int B, int Tq, int64_t rows_max) {
  const int64_t q = (int64_t)B * Tq;
  if (q <= 0 || rows_max <= 0) return 1;
  int64_t s = (512 + q - 1) / q;                     // about two workgroups per CU
  const int64_t by_rows = (rows_max + 127) / 128;    // at least 128 rows per split
  if (s > by_rows) s = by_rows;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  const int64_t q = (int64_t)a.B * a.Tq;
  if (q == 0) return hipSuccess;
  const bool csa = a.topk != nullptr;
  dim3 grid(a.splits, (unsigned)q);
#define V4_ATT(D)                                                             \
  do {                                                                        \
    if (csa) attend_kernel<D, true><<<grid, kAttThreads, 0, st>>>(a);         \
    else attend_kernel<D, false><<<grid, kAttThreads, 0, st>>>(a);            \
    if (a.splits > 1)                                                         \
      attend_merge_kernel<D><<<dim3((a.H + 7) / 8, (unsigned)q), 256, 0, st>>>(a); \
  } while (0)
  switch (a.D) {
    case 128: V4_ATT(128); break;
    case 256: V4_ATT(256); break;
    default: V4_ATT(512); break;
  }
#undef V4_ATT
  return hipGetLastError();
}

}  // namespace v4
