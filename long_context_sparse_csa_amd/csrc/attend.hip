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
// 64 at a time straight into LDS with global_load_lds (no staging registers,
// no conversion on the way; four waves move 16 rows each) and kept in their
// packed form: 576 bytes a row, E4M3 then bf16, 16-byte chunks XOR-swizzled
// by row so that both LDS read patterns below are free of bank conflicts.
// Two tile buffers alternate: the next tile lands while the current one is
// used.
//   Waves w and w+4 share heads 16(w%4)..+15 and split the dims in halves:
// each contracts S over its half (holding only that half of q~), the pair
// adds the two partial S through LDS, both run the same softmax, and each
// accumulates the output for its half of the dims:
//   S^T = K q~^T : K rows are the A operand, read 16 bytes a lane (two k-steps
//                  of E4M3, widened exactly to bf16 in registers); q~ is the B
//                  operand, held in registers with its dims permuted to match
//                  the order in which the lanes read the row;
//   O^T += V^T P^T : V^T comes from the packed rows with the gfx950
//                  transposing LDS reads (ds_read_b64_tr_b8 for E4M3 dims,
//                  ds_read_b64_tr_b16 for the bf16 ones), so nothing is stored
//                  twice; the probabilities stay in the registers the S^T
//                  accumulators left them in, because the key order of the
//                  transposing reads is permuted to match (k slot j of lane
//                  group g = key 4g+j or 16+4g+j-4 of each 32-key half).
// O^T keeps one head per lane, so the online-softmax rescale needs no
// shuffles, and the running maximum moves only when it grows by more than
// 2^8 (probabilities stay below 256, exact enough in bf16 and fp32), which
// skips almost every rescale.  Long rows are split over several workgroups
// whose (O, max, sum) partials a merge kernel combines with the sink.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kAttTile = 64;      // rows per LDS tile
constexpr int kAttThreads = 512;  // eight waves: four head groups x two dim halves
constexpr int kMaxTopk = 4096;    // largest k the CSA kernel stages in LDS
constexpr float kLazyMax = 8.0f;  // log2 headroom before the running max moves
constexpr float kNoMax = -1.0e30f; // running-max floor (no key seen yet)

// Source of absent rows (masked out of the softmax; zeros keep 0 * V finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[1024];

template <int D>
struct AttGeom {
  static constexpr int R = 64;
  static constexpr int ROW = D + R;            // packed bytes per row (HBM and LDS)
  static constexpr int CPR = ROW / 16;         // 16-byte chunks per row
  static constexpr int FP8_CPR = (D - R) / 16; // of which E4M3
  static constexpr int KSTEPS = D / 32;        // 32-dim k-steps of S^T
  static constexpr int NF8 = (D - 128) / 128;  // 128-dim E4M3 k-steps on the f8f6f4 MFMA
  static constexpr int NF0 = (NF8 + 1) / 2;    // of which in dim half 0
  static constexpr int TAIL = D - 128;         // first dim of the bf16-MFMA tail
  static_assert(D % 128 == 0, "head dim is a multiple of 128");
  static constexpr int DB = D / 16;            // 16-dim blocks of O^T
  static constexpr int FB = (D - R) / 16;      // of which over E4M3 dims
  static constexpr int TILE_BYTES = kAttTile * ROW;
  static constexpr int DBH = DB / 2;           // output blocks per dim half
  static constexpr int WPW = CPR / 4;          // 1 KiB copies per staging wave per tile (16 rows)
  static constexpr int HALF = 32 * ROW;        // byte offset of the second 32-key half
  static_assert(FP8_CPR % 4 == 0 && CPR % 4 == 0, "the chunk swizzle stays inside a region");
  static_assert(ROW <= 1024, "absent rows read the zero row");
};

// Physical chunk = logical chunk ^ swz(row): rows 4i..4i+3 rotate the four
// chunks of every aligned group differently, which spreads 16 rows of one
// logical chunk over all 16 chunk slots of a 256-byte bank line.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// 64 lanes x 16 bytes from per-lane global addresses into 1 KiB of LDS at
// `dst` (+16 bytes per lane).  Written as asm so that the compiler does not
// track it (it would otherwise wait for the copy before every LDS read): the
// tile loop waits for these copies itself (vmcnt) before the barrier that
// publishes a tile.  The instruction has no register result; its address
// registers are read at issue.
__device__ __forceinline__ void copy_to_lds16(const void* src, V4_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

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

  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][G::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) f32x4 s_x[8][4][64];  // partial S^T for the pair
  __shared__ unsigned s_v[2][4];   // per buffer: row-present bits, 16 rows per staging wave
  __shared__ float s_cs[R / 2][2];
  __shared__ __attribute__((aligned(16))) float s_gamma[D];
  __shared__ int s_sel[CSA ? kMaxTopk : 1];  // this split's slice of the top-k list

  const RowSpace rs = row_space(a, CSA, t);
  int64_t chunk = (rs.n_rows + a.splits - 1) / a.splits;
  chunk = (chunk + kAttTile - 1) / kAttTile * kAttTile;
  const int64_t row_beg = (int64_t)split * chunk;
  int64_t row_end = row_beg + chunk;
  if (row_end > rs.n_rows) row_end = rs.n_rows;
  const int ntiles = row_end > row_beg ? (int)((row_end - row_beg + kAttTile - 1) / kAttTile) : 0;
  // split-local row numbers fit in 32 bits
  const int nloc = (int)(row_end - row_beg);
  const int ent_loc = (int)max((int64_t)0, min(rs.n_ent, row_end) - row_beg);  // entry rows here
  const uint8_t* ent_b = a.entries + (int64_t)b * a.Ncap * G::ROW;
  const uint8_t* win_b = a.win + ((int64_t)b * (a.Tq + a.W - 1) +
                                  (rs.win_lo - (a.q_pos0 - (a.W - 1)))) * G::ROW;
  const int win_first = (int)(rs.n_ent - row_beg);   // split-local row of the first window row

  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, tid, R, a.rope_base, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  for (int d = 4 * tid; d < D; d += 4 * kAttThreads)
    *reinterpret_cast<f32x4*>(&s_gamma[d]) = *reinterpret_cast<const f32x4*>(a.gamma_q + d);
  if constexpr (CSA) {
    const int32_t* sel = a.topk + (int64_t)qr * a.k + row_beg;
    for (int x = tid; x < ent_loc; x += kAttThreads) s_sel[x] = sel[x];
  }
  __syncthreads();

  // split-local row x -> its packed row in HBM, or nullptr if absent
  auto row_ptr = [&](int x) -> const uint8_t* {
    const bool ent = x < ent_loc;
    int64_t j = (int64_t)x + row_beg;
    bool ok = x < nloc;
    if constexpr (CSA) {
      j = s_sel[ent ? x : 0];
      ok = ok && (!ent || (j >= 0 && j < a.Ncap));
    }
    const uint8_t* p = ent ? ent_b + j * G::ROW : win_b + (int64_t)(x - win_first) * G::ROW;
    return ok ? p : nullptr;
  };

  // ---- staging (waves 0-3): wave w copies tile rows 16w..16w+15 as WPW
  // windows of 64 16-byte slots; slot s holds physical chunk s % CPR of row
  // s / CPR, loaded from logical chunk (s % CPR) ^ swz(row).  Lane l resolves
  // row 16w + l%16.
  const uint8_t* zero_row = g_zero_row;
  auto issue_tile = [&](int tile, int buf) {
    const uint8_t* rp = row_ptr(tile * kAttTile + 16 * wave + (lane & 15));
    const bool ok = rp != nullptr;
    const unsigned long long bal = __ballot(ok);
    if (lane == 0) s_v[buf][wave] = (unsigned)(bal & 0xFFFFull);
    const long long rpl = (long long)(uintptr_t)(ok ? rp : zero_row);
    uint8_t* Tw = s_tile[buf] + 16 * wave * G::ROW;
#pragma unroll
    for (int i = 0; i < G::WPW; ++i) {
      const int sl = 64 * i + lane;
      const int rl = sl / G::CPR, pc = sl - rl * G::CPR;
      const uint8_t* src = (const uint8_t*)(uintptr_t)__shfl(rpl, rl) + 16 * (pc ^ swz(rl));
      copy_to_lds16(src, (V4_LDS void*)(Tw + 1024 * i));
    }
  };

  if (ntiles > 0 && wave < 4) issue_tile(0, 0);

  // ---- q~ = RoPE_t(RMSNorm(q)) scaled by 2^qe (per head, exact), as the B
  // operand of S^T.  The E4M3 dims run on the f8f6f4 MFMA with q~ split into
  // two E4M3 terms (hi + lo: about 2^-8 relative, the scale keeps the lo term
  // out of the subnormals); the last 64 E4M3 dims and the bf16 dims run on
  // the bf16 MFMA.  Lane group g owns 8-dim slots: per f8 k-step s the dims
  // 128s + 32g .. +31 (slots 4s .. 4s+3), then four tail slots t with dims
  // TAIL + 32t + 8g .. +7 (E4M3 for t < 2, bf16 for t = 2, 3).  Dim half 0
  // contracts f8 k-steps [0, NF0) and the bf16 tail, half 1 the f8 k-steps
  // [NF0, NF8) and the E4M3 tail.
  constexpr int NF8 = G::NF8, NF0 = G::NF0, TAIL = G::TAIL;
  constexpr int NQ = NF0 > 0 ? NF0 : 1;
  i32x8 qh[NQ], ql[NQ];
  bf16x8 qt[2];
  float qscale_inv;   // 2^-qe
  {
    auto slot_dim = [&](int sl) {
      return sl < 4 * NF8 ? 128 * (sl >> 2) + 32 * g + 8 * (sl & 3) : TAIL + 32 * (sl - 4 * NF8) + 8 * g;
    };
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + min(head, a.H - 1)) * D;
    u32x4 qv[G::KSTEPS];
#pragma unroll
    for (int sl = 0; sl < G::KSTEPS; ++sl)
      qv[sl] = *reinterpret_cast<const u32x4*>(qp + slot_dim(sl));
    if (head >= a.H) {
#pragma unroll
      for (int sl = 0; sl < G::KSTEPS; ++sl) qv[sl] = u32x4{0u, 0u, 0u, 0u};
    }
    float ss = 0.f;
#pragma unroll
    for (int sl = 0; sl < G::KSTEPS; ++sl) {
      const unsigned w[4] = {qv[sl].x, qv[sl].y, qv[sl].z, qv[sl].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_bits_to_f32(w[e] & 0xFFFFu), hi = bf16_bits_to_f32(w[e] >> 16);
        ss += lo * lo + hi * hi;
      }
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float rsn = 1.0f / sqrtf(ss / (float)D + a.eps);
    // q~ of one slot (8 dims), rotated where the dims are rotary
    auto qtilde = [&](int sl, float (&qf)[8]) {
      const int d0 = slot_dim(sl);
      const unsigned w[4] = {qv[sl].x, qv[sl].y, qv[sl].z, qv[sl].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[2 * e] = s_gamma[d0 + 2 * e] * (bf16_bits_to_f32(w[e] & 0xFFFFu) * rsn);
        qf[2 * e + 1] = s_gamma[d0 + 2 * e + 1] * (bf16_bits_to_f32(w[e] >> 16) * rsn);
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
    };
    // per-head scale: the largest |q~| lands in [128, 256)
    float mx = 0.f;
#pragma unroll
    for (int sl = 0; sl < G::KSTEPS; ++sl) {
      float qf[8];
      qtilde(sl, qf);
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qf[e]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const int qe = mx > 0.f ? 8 - __builtin_amdgcn_frexp_expf(mx) : 0;
    qscale_inv = ldexpf(1.0f, -qe);
    // The operands of this wave's half; the half is a compile-time constant
    // inside so that every slot index is one (no run-time register indexing).
    auto build = [&](auto half) {
      constexpr int HF = decltype(half)::value;
      // f8 k-steps: hi and lo E4M3 terms, 4 bytes per dword in dim order
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int s8 = HF == 0 ? u : NF0 + u;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float qf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (s8 < NF8) qtilde(4 * s8 + v, qf);
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = ldexpf(qf[4 * h2 + e], qe);
            int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
            hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hw, true);
            const float r[4] = {x[0] - __builtin_amdgcn_cvt_f32_fp8(hw, 0),
                                x[1] - __builtin_amdgcn_cvt_f32_fp8(hw, 1),
                                x[2] - __builtin_amdgcn_cvt_f32_fp8(hw, 2),
                                x[3] - __builtin_amdgcn_cvt_f32_fp8(hw, 3)};
            int lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
            lw = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lw, true);
            qh[u][2 * v + h2] = hw;
            ql[u][2 * v + h2] = lw;
          }
        }
      }
      // tail k-steps: half 0 the bf16 dims (t = 2, 3), half 1 the E4M3 tail (t = 0, 1)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        float qf[8];
        qtilde(4 * NF8 + (HF == 0 ? 2 : 0) + t2, qf);
        u32x4 pk = {pack_bf16x2(ldexpf(qf[0], qe), ldexpf(qf[1], qe)),
                    pack_bf16x2(ldexpf(qf[2], qe), ldexpf(qf[3], qe)),
                    pack_bf16x2(ldexpf(qf[4], qe), ldexpf(qf[5], qe)),
                    pack_bf16x2(ldexpf(qf[6], qe), ldexpf(qf[7], qe))};
        qt[t2] = __builtin_bit_cast(bf16x8, pk);
      }
    };
    if (hf == 0) build(std::integral_constant<int, 0>{});
    else build(std::integral_constant<int, 1>{});
  }

  const float sl2 = a.scale * kLog2e * qscale_inv;   // undoes the q~ scale
  // running max starts at a finite floor, so masked keys (-inf) give p = 0
  // without special cases; an untouched max marks "no row seen"
  float m_run = kNoMax, l_run = 0.f;  // per head (lane column), log2 units
  f32x4 o[G::DBH];
#pragma unroll
  for (int db = 0; db < G::DBH; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane LDS offsets within a tile (second 32-key half: + HALF)
  //  K rows of the bf16 tail (A of S^T): row kb*16 + c, chunk FP8_CPR + 4t + g
  int koff[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = kb * 16 + c;
    koff[kb] = row * G::ROW + 16 * (g ^ swz(row));
  }
  //  K rows for the f8f6f4 k-steps: chunks 8s + 2g + i (i = 0, 1) -> + 128s
  int koff8[2][2];
  //  K rows for the E4M3 tail: dims TAIL + 32t + 8g, 8 bytes
  int ktoff[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = kb * 16 + c, sw = swz(row);
#pragma unroll
    for (int i = 0; i < 2; ++i) koff8[kb][i] = row * G::ROW + 16 * ((2 * g + i) ^ sw);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      ktoff[kb][t2] = row * G::ROW + 16 * (TAIL / 16 + ((2 * t2 + (g >> 1)) ^ sw)) + 8 * (g & 1);
  }
  //  V^T via tr_b8: source lane (g, j = (lane&15)>>1, h = lane&1) addresses
  //  key slot j of group g, dims 16db + 8h; chunk 4a + b -> + 64a
  int v8off[4];
  {
    const int j = (lane & 15) >> 1, h = lane & 1;
    const int row = j < 4 ? 4 * g + j : 16 + 4 * g + j - 4;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) v8off[bb] = row * G::ROW + 16 * (bb ^ swz(row)) + 8 * h;
  }
  //  V^T via tr_b16 (bf16 dims): source lane (g, j = (lane&15)>>2, q = lane&3)
  //  addresses keys 4g+j (lo) and 16+4g+j (hi), dims (D-R) + 16e + 4q
  int v16off[2][2];
  {
    const int j = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const int row = hl * 16 + 4 * g + j;
#pragma unroll
      for (int e1 = 0; e1 < 2; ++e1)
        v16off[hl][e1] = row * G::ROW + 16 * (G::FP8_CPR + ((2 * e1 + (q >> 1)) ^ swz(row))) +
                         8 * (q & 1);
    }
  }

  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // Tile t lives in buffer t & 1.  A tile issues the copies of tile t+1 (into
  // the buffer every wave finished reading before the last barrier), uses
  // tile t, waits for its own copies and meets the other waves at the
  // barrier, so tile t+1 is complete in LDS and every read of tile t is done.
  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    if (tile + 1 < ntiles && wave < 4) issue_tile(tile + 1, cur ^ 1);
    const uint8_t* T = s_tile[cur];
    // partial S^T over this wave's half of the k-steps, 64 keys
    f32x4 s[2][2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[hh][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (active) {
      // f8f6f4 k-steps of this half: K straight from the tile, q~ as hi + lo
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int s8 = hf == 0 ? u : NF0 + u;
        if (s8 < NF8 && (hf == 1 || u < NF0)) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const u32x4 w0 = *reinterpret_cast<const u32x4*>(T + koff8[kb][0] + hh * G::HALF + 128 * s8);
              const u32x4 w1 = *reinterpret_cast<const u32x4*>(T + koff8[kb][1] + hh * G::HALF + 128 * s8);
              const i32x8 ka = __builtin_bit_cast(
                  i32x8, u32x8{w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w});
              s[hh][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qh[u], s[hh][kb], 0, 0, 0,
                                                                           127, 0, 127);
              s[hh][kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, ql[u], s[hh][kb], 0, 0, 0,
                                                                           127, 0, 127);
            }
        }
      }
      if (hf == 0) {   // bf16 (rotary) dims
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const u32x4 w = *reinterpret_cast<const u32x4*>(T + koff[kb] + hh * G::HALF +
                                                              16 * G::FP8_CPR + 64 * t2);
              s[hh][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w), qt[t2],
                                                                  s[hh][kb], 0, 0, 0);
            }
      } else {         // E4M3 tail, widened to bf16
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              const u32x2 w = *reinterpret_cast<const u32x2*>(T + ktoff[kb][t2] + hh * G::HALF);
              const u32x2 lo = fp8x4_to_bf16x4(w.x), hi = fp8x4_to_bf16x4(w.y);
              s[hh][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), qt[t2], s[hh][kb], 0, 0, 0);
            }
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s_x[wave][2 * hh + kb][lane] = s[hh][kb];
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (active) {
      // full S: own half + partner's half (a + b == b + a, so both waves agree)
      unsigned vmask[2];
      vmask[0] = __builtin_amdgcn_readfirstlane(s_v[cur][0] | (s_v[cur][1] << 16));
      vmask[1] = __builtin_amdgcn_readfirstlane(s_v[cur][2] | (s_v[cur][3] << 16));
      float x[2][2][4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const f32x4 sk = s[hh][kb] + s_x[wave ^ 4][2 * hh + kb][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[hh][kb][i] = sk[i] * sl2;
        }
      // online softmax for head c over this lane's 16 keys: 32hh + 16kb + 4g + i
      if ((vmask[0] & vmask[1]) != 0xFFFFFFFFu) {   // partial tile: mask the absent rows
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (!((vmask[hh] >> (kb * 16 + 4 * g + i)) & 1u)) x[hh][kb][i] = -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          mt = fmaxf(mt, fmaxf(fmaxf(x[hh][kb][0], x[hh][kb][1]), fmaxf(x[hh][kb][2], x[hh][kb][3])));
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
      bf16x8 pb[2];
      float ls = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float p[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = __builtin_amdgcn_exp2f(x[hh][kb][i] - m_run);
            ls += p[kb][i];
          }
        const u32x4 pk = {pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                          pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])};
        pb[hh] = __builtin_bit_cast(bf16x8, pk);
      }
      l_run += ls;
      // O^T += V^T P^T for this wave's half of the dim blocks
#pragma unroll
      for (int u = 0; u < G::DBH; ++u) {
        const int db = hf * G::DBH + u;
        if (db < G::FB) {   // E4M3 dims
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (V4_LDS i32x2*)(T + v8off[db & 3] + hh * G::HALF + 64 * (db >> 2)));
            const u32x2 lo = fp8x4_to_bf16x4((unsigned)v.x), hi = fp8x4_to_bf16x4((unsigned)v.y);
            o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), pb[hh], o[u], 0, 0, 0);
          }
        } else {            // bf16 dims
          const int e = db - G::FB;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const u32x2 lo = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (V4_LDS i16x4*)(T + v16off[0][e & 1] + hh * G::HALF + 64 * (e >> 1))));
            const u32x2 hi = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (V4_LDS i16x4*)(T + v16off[1][e & 1] + hh * G::HALF + 64 * (e >> 1))));
            o[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y}), pb[hh], o[u], 0, 0, 0);
          }
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }

  if (!active || head >= a.H) return;
  // full denominator of this lane's head: sum the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const int db0 = hf * G::DBH;       // this wave's first output dim block
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
// Grid: (ceil(H / HPW), B*Tq) with HPW = 1024 / D heads per workgroup of 256
// threads.  Wave w first turns the (max, sum) pairs of heads h0 + w, h0 + w + 4,
// .. into one weight per split (splits <= 64: one lane each); then every thread merges
// four dims of one head, all of its split loads in flight together.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a) {
  constexpr int R = 64;
  constexpr int QPH = D / 4;          // threads per head (four dims each)
  constexpr int HPW = 256 / QPH;      // heads per workgroup
  const int qr = blockIdx.y;
  const int h0 = blockIdx.x * HPW;
  const int64_t t = a.q_pos0 + (qr % a.Tq);
  const int S = a.splits;
  __shared__ float s_w[HPW][64];
  __shared__ float s_cs[R / 2][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, tid, R, a.rope_base, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  for (int hw = wave; hw < HPW; hw += 4) {
    const int h = h0 + hw;
    if (h >= a.H) break;
    const float* pm = a.part_ml + ((int64_t)qr * S * a.H + h) * 2;
    const bool own = lane < S;
    const f32x2 ml = own ? *reinterpret_cast<const f32x2*>(pm + (int64_t)lane * a.H * 2)
                         : f32x2{-INFINITY, 0.f};
    const float z2 = a.sink[h] * kLog2e;
    const float M = fmaxf(wave_max(ml.x), z2);
    const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    float den = wave_sum(ml.y * w);
    if (M != -INFINITY) den += exp2f(z2 - M);
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    s_w[hw][lane] = w * inv;
    if (a.lse && lane == 0)
      a.lse[(int64_t)qr * a.H + h] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
  __syncthreads();
  const int hh = tid / QPH, d = 4 * (tid % QPH);
  const int h = h0 + hh;
  if (hh >= HPW || h >= a.H) return;
  const float* po = a.part_o + ((int64_t)qr * S * a.H + h) * D + d;
  const int64_t sstride = (int64_t)a.H * D;
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {   // eight split partials in flight
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)min(s0 + u, S - 1) * sstride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = s0 + u < S ? s_w[hh][s0 + u] : 0.f;
      x += w * v[u];
    }
  }
  float y[4] = {x[0], x[1], x[2], x[3]};
  if (d >= D - R) {
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const int i = (d + e - (D - R)) >> 1;
      const float cs = s_cs[i][0], sn = s_cs[i][1];
      const float x0 = y[e], x1 = y[e + 1];
      y[e] = x0 * cs + x1 * sn;       // rotation by -t
      y[e + 1] = -x0 * sn + x1 * cs;
    }
  }
  const u32x2 pk = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  *reinterpret_cast<u32x2*>(a.out + ((int64_t)qr * a.H + h) * D + d) = pk;
}

int attend_splits(int B, int Tq, int64_t rows_max) {
  const int64_t q = (int64_t)B * Tq;
  if (q <= 0 || rows_max <= 0) return 1;
  int64_t s = (256 + q - 1) / q;                               // about one workgroup per CU
  const int64_t by_rows = (rows_max + kAttTile - 1) / kAttTile;  // at least one tile per split
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
      attend_merge_kernel<D><<<dim3((a.H + 1024 / (D) - 1) / (1024 / (D)), (unsigned)q), 256, 0, st>>>(a); \
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
