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
// Design.  One workgroup of four waves owns one query token and one range of
// its rows (entries, then window rows); wave w owns heads 16w..16w+15, so
// every packed row is fetched from HBM once for all 64 heads.  Rows are
// gathered (CSA: through the top-k list) 32 at a time into an LDS tile as raw
// 576-byte packed rows (E4M3 | bf16), double-buffered through registers with
// 16-byte coalesced loads.
//   S^T = K q~^T : K rows are the A operand (one 8-byte E4M3 read or one
//                  16-byte bf16 read per lane, widened exactly to bf16), q~ is
//                  the B operand held in registers for the whole kernel;
//                  the result puts one head per lane column and keys down the
//                  lane groups, so the softmax statistics need only two
//                  cross-lane steps;
//   O^T += V^T P^T : V^T comes straight from the row-major tile with the
//                  gfx950 transposing LDS reads (ds_read_b64_tr_b8 for the
//                  E4M3 dims, ds_read_b64_tr_b16 for the bf16 dims); the
//                  probabilities stay in the registers the S^T accumulators
//                  left them in, because the MFMA's key order is permuted to
//                  match (k slot j of lane group g = key 4g+j or 16+4g+j-4).
// O^T keeps one head per lane, so the online-softmax rescale needs no
// shuffles and the inverse rotation pairs sit in one lane.  Long rows are
// split over several workgroups whose (O, max, sum) partials a merge kernel
// combines with the sink.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kAttTile = 32;      // rows per LDS tile
constexpr int kAttThreads = 256;  // four waves
constexpr int kMaxTopk = 4096;    // largest k the CSA kernel stages in LDS

template <int D>
struct AttGeom {
  static constexpr int R = 64;
  static constexpr int ROW = D + R;            // packed bytes per row
  static constexpr int LSTR = ROW + 16;        // LDS row stride (spreads banks)
  static constexpr int KSTEPS = D / 32;        // 32-dim k-steps of S^T
  static constexpr int FP8_KSTEPS = (D - R) / 32;
  static constexpr int DB = D / 16;            // 16-dim blocks of O^T
  static constexpr int FP8_DB = (D - R) / 16;
  static constexpr int CPR = ROW / 16;         // 16-byte chunks per row
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
  const int g = lane >> 4, c = lane & 15;
  const int head = wave * 16 + c;
  const bool active = wave * 16 < a.H;

  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][kAttTile * G::LSTR];
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

  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, tid, R, a.rope_base, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  if constexpr (CSA) {
    const int32_t* sel = a.topk + (int64_t)qr * a.k;
    const int64_t ent_end = row_end < rs.n_ent ? row_end : rs.n_ent;
    for (int64_t x = row_beg + tid; x < ent_end; x += kAttThreads) s_sel[x - row_beg] = sel[x];
    __syncthreads();
  }

  // row x of this split -> its packed row in HBM, or nullptr if absent
  auto row_ptr = [&](int64_t x) -> const uint8_t* {
    if (x >= row_end) return nullptr;
    if (x < rs.n_ent) {
      int64_t j = x;
      if constexpr (CSA) {
        j = s_sel[x - row_beg];
        if (j < 0 || j >= a.Ncap) return nullptr;
      }
      return a.entries + ((int64_t)b * a.Ncap + j) * G::ROW;
    }
    const int64_t p = rs.win_lo + (x - rs.n_ent);
    const int64_t wrow = p - (a.q_pos0 - (a.W - 1));
    return a.win + ((int64_t)b * (a.Tq + a.W - 1) + wrow) * G::ROW;
  };

  // ---- tile staging: chunk u of this thread -> (row, 16-byte column)
  u32x4 pref[G::CH];
  auto fetch_rows = [&](int tile) {
#pragma unroll
    for (int u = 0; u < G::CH; ++u) {
      const int cidx = tid + u * kAttThreads;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (cidx < G::CHUNKS) {
        const uint8_t* p = row_ptr(row_beg + (int64_t)tile * kAttTile + cidx / G::CPR);
        if (p) v = *reinterpret_cast<const u32x4*>(p + (cidx % G::CPR) * 16);
      }
      pref[u] = v;
    }
  };
  auto store_rows = [&](int tile, int buf) {
#pragma unroll
    for (int u = 0; u < G::CH; ++u) {
      const int cidx = tid + u * kAttThreads;
      if (cidx < G::CHUNKS)
        *reinterpret_cast<u32x4*>(&s_tile[buf][(cidx / G::CPR) * G::LSTR + (cidx % G::CPR) * 16]) =
            pref[u];
    }
    if (tid < 64) {
      const bool ok = tid < kAttTile && row_ptr(row_beg + (int64_t)tile * kAttTile + tid) != nullptr;
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
  bf16x8 qb[G::KSTEPS];
  {
    float qf[G::KSTEPS][8];
    float ss = 0.f;
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + head) * D + g * 8;
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < a.H) v = *reinterpret_cast<const u32x4*>(qp + ks * 32);
      unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks][2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
        qf[ks][2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
        ss += qf[ks][2 * e] * qf[ks][2 * e] + qf[ks][2 * e + 1] * qf[ks][2 * e + 1];
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rsn = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      const int d0 = ks * 32 + g * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = a.gamma_q[d0 + e] * (qf[ks][e] * rsn);
      if (d0 >= D - R) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int i = (d0 + e - (D - R)) >> 1;
          const float cs = s_cs[i][0], sn = s_cs[i][1];
          const float x0 = qf[ks][e], x1 = qf[ks][e + 1];
          qf[ks][e] = x0 * cs - x1 * sn;
          qf[ks][e + 1] = x0 * sn + x1 * cs;
        }
      }
      u32x4 pk = {pack_bf16x2(qf[ks][0], qf[ks][1]), pack_bf16x2(qf[ks][2], qf[ks][3]),
                  pack_bf16x2(qf[ks][4], qf[ks][5]), pack_bf16x2(qf[ks][6], qf[ks][7])};
      qb[ks] = __builtin_bit_cast(bf16x8, pk);
    }
  }

  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;  // per head (lane column), log2 units
  f32x4 o[G::DB];
#pragma unroll
  for (int db = 0; db < G::DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets of the transposing V^T reads
  const int jv8 = (lane & 15) >> 1;  // tr8: k slot served by this lane
  const int key8 = jv8 < 4 ? 4 * g + jv8 : 12 + 4 * g + jv8;
  const int off8 = key8 * G::LSTR + 8 * (lane & 1);
  const int jv16 = (lane & 15) >> 2;  // tr16: k slot served by this lane
  const int off16a = (4 * g + jv16) * G::LSTR + (D - R) + 8 * (lane & 3);
  const int off16b = (16 + 4 * g + jv16) * G::LSTR + (D - R) + 8 * (lane & 3);

  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    const bool more = tile + 1 < ntiles;
    if (more) fetch_rows(tile + 1);
    if (active) {
      const uint8_t* T = s_tile[cur];
      // S^T = K q~^T over two 16-key blocks
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < G::KSTEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint8_t* rowp = T + (kb * 16 + c) * G::LSTR;
          bf16x8 ka;
          if (ks < G::FP8_KSTEPS) {
            u32x2 w = *reinterpret_cast<const u32x2*>(rowp + ks * 32 + g * 8);
            ka = fp8x8_to_bf16x8(w);
          } else {
            u32x4 w = *reinterpret_cast<const u32x4*>(rowp + (D - R) + 2 * (ks * 32 + g * 8 - (D - R)));
            ka = __builtin_bit_cast(bf16x8, w);
          }
          s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ks], s[kb], 0, 0, 0);
        }
      }
      // online softmax for head c over this lane's 8 keys: kb*16 + 4g + i
      const unsigned vmask = s_valid[cur];
      float x[2][4];
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (vmask >> (kb * 16 + 4 * g + i)) & 1u;
          x[kb][i] = ok ? s[kb][i] * sl2 : -INFINITY;
          mt = fmaxf(mt, x[kb][i]);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run, mt);
      float corr = 1.f;
      float p[2][4];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) p[kb][i] = 0.f;
      } else {
        corr = exp2f(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = exp2f(x[kb][i] - m_new);
            ls += p[kb][i];
          }
        l_run = l_run * corr + ls;
        m_run = m_new;
      }
#pragma unroll
      for (int db = 0; db < G::DB; ++db) o[db] *= corr;
      u32x4 pk = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                  pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < G::FP8_DB; ++db) {
        const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (V4_LDS i32x2*)(T + off8 + db * 16));
        const bf16x8 va = fp8x8_to_bf16x8(u32x2{(unsigned)w.x, (unsigned)w.y});
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
      }
#pragma unroll
      for (int db = G::FP8_DB; db < G::DB; ++db) {
        const int dofs = 2 * (db * 16 - (D - R));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((V4_LDS i16x4*)(T + off16a + dofs));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((V4_LDS i16x4*)(T + off16b + dofs));
        u32x4 vv = {(unsigned)(uint16_t)lo.x | ((unsigned)(uint16_t)lo.y << 16),
                    (unsigned)(uint16_t)lo.z | ((unsigned)(uint16_t)lo.w << 16),
                    (unsigned)(uint16_t)hi.x | ((unsigned)(uint16_t)hi.y << 16),
                    (unsigned)(uint16_t)hi.z | ((unsigned)(uint16_t)hi.w << 16)};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vv), pb, o[db],
                                                        0, 0, 0);
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
    for (int db = 0; db < G::DB; ++db)
      *reinterpret_cast<f32x4*>(po + db * 16 + g * 4) = o[db];
    if (g == 0) {
      float* pm = a.part_ml + (((int64_t)qr * a.splits + split) * a.H + head) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
    return;
  }
  const float z2 = a.sink[head] * kLog2e;
  const float M = fmaxf(m_run, z2);
  float scale_o = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    const float wr = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
    const float den = l_run * wr + exp2f(z2 - M);
    scale_o = wr / den;
    lse = (M + log2f(den)) * 0.69314718055994531f;
  }
  uint16_t* op = a.out + ((int64_t)qr * a.H + head) * D;
#pragma unroll
  for (int db = 0; db < G::DB; ++db) {
    const int d0 = db * 16 + g * 4;
    float v[4] = {o[db][0] * scale_o, o[db][1] * scale_o, o[db][2] * scale_o, o[db][3] * scale_o};
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
    u32x2 pkd = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2*>(op + d0) = pkd;
  }
  if (a.lse && g == 0) a.lse[(int64_t)qr * a.H + head] = lse;
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
    for (int s = 0; s < S; ++s) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(po + (int64_t)s * a.H * D);
      x0 = fmaf(s_w[hh][s], v.x, x0);
      x1 = fmaf(s_w[hh][s], v.y, x1);
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
