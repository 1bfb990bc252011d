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
// its rows (entries, then window rows), so every packed row is fetched from
// HBM once for all heads.  Rows are gathered (CSA: through the top-k list)
// 128 at a time straight into LDS with global_load_lds (no staging
// registers, no conversion; each wave moves 32 rows) and kept in their packed
// form: 576 bytes a row, E4M3 then bf16, 16-byte chunks XOR-swizzled by row
// so that every LDS read pattern below is free of bank conflicts.  Two tile
// buffers alternate: the next tile lands while the current one is used.
//   Wave w owns heads 16w..16w+15 over all dims and all rows, with its own
// online softmax, so the waves share nothing but the tiles.  Both products
// run on the 16x16 MFMAs with one head per lane column:
//   S^T = K q~^T : K rows are the A operand straight from the tile; the E4M3
//                  dims take the f8f6f4 MFMA (16x16x128) with q~ as two E4M3
//                  terms (hi + lo), the bf16 dims the bf16 MFMA (16x16x32);
//   O^T += V^T P^T : V^T comes from the packed rows with the gfx950
//                  transposing LDS reads (ds_read_b64_tr_b8 for E4M3 dims,
//                  ds_read_b64_tr_b16 for bf16), so the E4M3 dims go into the
//                  f8f6f4 MFMA as stored; P stays in the registers the S^T
//                  accumulators left it in, because the row order of the
//                  transposing reads is permuted to match.
// P enters the f8f6f4 product as two E4M3 terms as well.  Each 64-row scale
// block of one head is exponentiated against its own power of two (its
// largest p lands in (128, 256]), and the MFMA's per-block E8M0 scale on that
// operand brings it back to the head's running maximum, so rows far below the
// maximum keep their relative precision instead of flushing to zero.  O^T
// keeps one head per lane column, so the online-softmax rescale needs no
// shuffles, and the running maximum moves only when it grows by more than
// 2^64 (fp32 and the E8M0 scales hold that range), in practice once, outside
// the hot loop.  Long rows are split over several workgroups whose
// (O, max, sum) partials a merge kernel combines with the sink.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

constexpr int kAttRows = 128;      // rows per LDS tile
constexpr int kAttThreads = 256;   // four waves of 16 heads
constexpr int kSelCap = 2048;      // CSA: top-k slots of one split staged in LDS
constexpr float kLazyMax = 64.0f;  // log2 headroom before the running max moves
constexpr float kNoMax = -1.0e30f; // running-max floor (no key seen yet)

// Source of absent rows (masked out of the softmax; zeros keep 0 * V finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[1024];

template <int D>
struct AttGeom {
  static constexpr int R = 64;
  static constexpr int ROW = D + R;            // packed bytes per row (HBM and LDS)
  static constexpr int CPR = ROW / 16;         // 16-byte chunks per row
  static constexpr int FP8_CPR = (D - R) / 16; // of which E4M3
  static constexpr int NJ = (D - R + 127) / 128; // 128-dim E4M3 k-steps of S^T (the last half full)
  static constexpr int NB8 = (D - R) / 16;     // 16-dim E4M3 blocks of O^T
  static constexpr int NB = D / 16;            // all 16-dim blocks (the last four bf16)
  static constexpr int TILE_BYTES = kAttRows * ROW;
  static constexpr int WPW = ROW / 32;         // 1 KiB copies per wave per tile (32 rows)
  static_assert(D >= 128 && (D - R) % 128 == 64, "E4M3 dims end half way through a k-step");
  static_assert(FP8_CPR % 4 == 0 && CPR % 4 == 0, "the chunk swizzle stays inside a region");
  static_assert(ROW <= 1024 && ROW % 32 == 0, "absent rows read the zero row");
};

// Physical chunk = logical chunk ^ swz(row) within aligned groups of four
// chunks.  swz takes row bit 2 and bits 3 ^ 4: 16 consecutive rows spread one
// logical chunk over all 16 chunk slots of a 256-byte bank line, and so do
// the row sets of the transposing reads below.
__device__ __forceinline__ int swz(int row) { return ((row >> 2) & 1) | ((((row >> 3) ^ (row >> 4)) & 1) << 1); }

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

// The same copy from a uniform 64-bit base plus a per-lane 32-bit offset
// (the scalar-base addressing form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void copy_to_lds16_sbase(const void* base, unsigned off, V4_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

struct RowSpace {
  int64_t n_ent;    // entry rows (CSA: k slots; HCA: visible entries)
  int64_t win_lo;   // first window position
  int64_t n_rows;   // entries + window rows
};

__device__ __forceinline__ RowSpace row_space(bool csa, int64_t t, int k, int m, int64_t n_entries,
                                               int W) {
  RowSpace rs;
  if (csa) {
    rs.n_ent = k;
  } else {   // positions below 2^31 take the 32-bit division
    const int64_t v = (uint64_t)(t + 1) < (1ull << 31) ? (int64_t)((uint32_t)(t + 1) / (uint32_t)m)
                                                       : (t + 1) / m;
    rs.n_ent = v < n_entries ? v : n_entries;
  }
  int64_t lo = t - W + 1;
  rs.win_lo = lo > 0 ? lo : 0;
  const int64_t n_win = W > 0 ? (t - rs.win_lo + 1) : 0;
  rs.n_rows = rs.n_ent + n_win;
  return rs;
}

// Rows of one key range per split: a whole number of tiles.
__host__ __device__ inline int64_t split_chunk(int64_t n_rows, int splits) {
  const int64_t c = (n_rows + splits - 1) / splits;
  return (c + kAttRows - 1) / kAttRows * kAttRows;
}
// The same for n_rows below 2^31, with a 32-bit division.
__device__ __forceinline__ int64_t split_chunk32(int n_rows, int splits) {
  const unsigned c = ((unsigned)n_rows + (unsigned)splits - 1u) / (unsigned)splits;
  return (int64_t)((c + kAttRows - 1) / kAttRows * kAttRows);
}

// out = g1 * y + g0 * o0 + g2 * o2 for four dims (the gated sum of the
// NSA-style variant, applied where the last branch is finalised), else y.
template <bool MIX>
__device__ __forceinline__ u32x2 final_bf16x4(const AttendArgs& a, int64_t off, int64_t qh,
                                              const float (&y)[4]) {
  if (!MIX || !a.mix_gates) return u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
  const float g0 = a.mix_gates[3 * qh], g1 = a.mix_gates[3 * qh + 1], g2 = a.mix_gates[3 * qh + 2];
  const u32x2 u0 = *reinterpret_cast<const u32x2*>(a.mix_o0 + off);
  const u32x2 u2 = *reinterpret_cast<const u32x2*>(a.mix_o2 + off);
  const float x0[4] = {bf16_bits_to_f32(u0.x & 0xFFFFu), bf16_bits_to_f32(u0.x >> 16),
                       bf16_bits_to_f32(u0.y & 0xFFFFu), bf16_bits_to_f32(u0.y >> 16)};
  const float x2[4] = {bf16_bits_to_f32(u2.x & 0xFFFFu), bf16_bits_to_f32(u2.x >> 16),
                       bf16_bits_to_f32(u2.y & 0xFFFFu), bf16_bits_to_f32(u2.y >> 16)};
  float z[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = fmaf(g2, x2[e], fmaf(g0, x0[e], g1 * y[e]));
  return u32x2{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
}

template <int D, bool CSA>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendBatch ab) {
  using G = AttGeom<D>;
  constexpr int R = G::R, NJ = G::NJ, NB8 = G::NB8, NB = G::NB, ROW = G::ROW;
  constexpr int BFC = G::FP8_CPR;   // first bf16 chunk
  const AttendArgs& a = ab.p[blockIdx.z];   // the problem of this grid layer
  // wave as a scalar: the LDS destinations of the tile copies (m0) are then
  // formed with scalar arithmetic instead of a vector add and a readfirstlane
  // per copy
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Every argument the prologue needs is read in one round, before any
  // branch: each dependent round trip to the argument segment costs a memory
  // latency, and the compiler would otherwise sink the reads into the
  // branches that use them, one after another (the empty asm statements pin
  // them here).
  const bool flat = a.flat, ragged = a.ragged;
  const int B = a.B, Tq = a.Tq, H = a.H, W = a.W, splits = a.splits, kk = a.k, m = a.m;
  const int sel_m = a.sel_m, slot_first = a.slot0[0];
  const int64_t q_pos0 = a.q_pos0, Ncap = a.Ncap, n_entries = a.n_entries;
  const uint16_t* const qg = a.q;
  const uint8_t* const entries = a.entries;
  const uint8_t* const wing = a.win;
  const float* const gamma_q = a.gamma_q;
  const int32_t* const topk = a.topk;
  asm volatile("" ::"s"(qg), "s"(entries), "s"(wing), "s"(gamma_q), "s"(topk), "s"(q_pos0),
               "s"(Ncap), "s"(n_entries));
  asm volatile("" ::"s"((int)flat), "s"((int)ragged), "s"(B), "s"(Tq), "s"(H), "s"(W), "s"(splits),
               "s"(kk), "s"(m), "s"(sel_m), "s"(slot_first));
  const double rturn = a.rope.t[lane & 31];
  // The per-sequence tables are read only where they are used, through the
  // argument segment's address with a run-time offset (the compiler hoists
  // reads of `a` out of branches, and a value in flight that is never used
  // holds its register until the compiler waits for it to reuse that;
  // taking the address of a member of `a` would copy the whole argument
  // block to scratch memory).
  static_assert(kMaxRagged == 64, "one lane per sequence of a flat grid");
  const char* const my_args =
      (const char*)__builtin_amdgcn_kernarg_segment_ptr() +
      offsetof(AttendBatch, p) + (size_t)blockIdx.z * sizeof(AttendArgs);
  int qr, split, nsplit;
  int64_t slot;   // this split's partial slot
  if (flat) {   // ragged decode: workgroup x is slot x of sequence b
    // lane l: the slot after sequence l's last
    const int slot_nx =
        *reinterpret_cast<const int*>(my_args + offsetof(AttendArgs, slot0) + sizeof(int) * (lane + 1));
    const int x = blockIdx.x;
    if (x >= __builtin_amdgcn_readlane(slot_nx, B - 1)) return;
    // slot0 ascends: b = the number of sequences (but the last) whose slots end at or before x
    const int bb = (int)__popcll(__ballot(lane + 1 < B && x >= slot_nx));
    const int s0 = bb > 0 ? __builtin_amdgcn_readlane(slot_nx, bb - 1) : slot_first;
    qr = bb;
    split = x - s0;
    nsplit = __builtin_amdgcn_readlane(slot_nx, bb) - s0;
    slot = x;
  } else {
    qr = blockIdx.y;
    split = blockIdx.x;
    if (split >= splits) return;   // a layer with fewer splits than the grid
    nsplit = splits;
    slot = (int64_t)qr * splits + split;
  }
  const int b = qr / Tq, r = qr % Tq;
  int64_t qpos = q_pos0;   // this sequence's first query
  if (ragged)
    qpos = *reinterpret_cast<const int64_t*>(my_args + offsetof(AttendArgs, pos) +
                                             sizeof(int64_t) * (b & (kMaxRagged - 1)));
  const int64_t t = qpos + r;
  const int c = lane & 15, g = lane >> 4;   // lane column (head / row / dim), k group
  const int head = wave * 16 + c;

  __shared__ __attribute__((aligned(16))) uint8_t s_tile[2][G::TILE_BYTES];
  __shared__ unsigned s_v[2][4];   // per buffer: row-present bits, 32 rows per staging wave
  __shared__ float s_cs[R / 2][2];
  __shared__ int s_sel[CSA ? kSelCap : 1];  // this split's slice of the top-k list
  __shared__ __attribute__((aligned(16))) uint8_t s_zero[32];   // K bytes past the E4M3 dims
  __shared__ __attribute__((aligned(16))) float s_gamma[D];      // gamma_q, read per q~ slot

  const RowSpace rs = row_space(CSA, t, kk, m, n_entries, W);
  const int64_t chunk = rs.n_rows < (1ll << 31) ? split_chunk32((int)rs.n_rows, nsplit)
                                                 : split_chunk(rs.n_rows, nsplit);
  const int64_t row_beg = (int64_t)split * chunk;
  int64_t row_end = row_beg + chunk;
  if (row_end > rs.n_rows) row_end = rs.n_rows;
  const int ntiles = row_end > row_beg ? (int)((row_end - row_beg + kAttRows - 1) / kAttRows) : 0;
  // split-local row numbers fit in 32 bits
  const int nloc = (int)(row_end - row_beg);
  const int ent_loc = (int)max((int64_t)0, min(rs.n_ent, row_end) - row_beg);  // entry rows here
  const uint8_t* ent_b = entries + (int64_t)b * Ncap * ROW;
  const uint8_t* win_b = wing + ((int64_t)b * (Tq + W - 1) + (rs.win_lo - (qpos - (W - 1)))) * ROW;
  const int win_first = (int)(rs.n_ent - row_beg);   // split-local row of the first window row

  // The loads the first barrier waits for go out first (a wave's vector loads
  // complete in order): this split's slice of the top-k list and the top-k
  // slots of the first tile's rows (CSA), and gamma_q.  Then q, before the
  // first tile's copies, so that its loads are not queued behind them; they
  // stay in flight across the barrier.  No load sits in a branch (the
  // compiler waits for a load inside a branch at once): the top-k slots are
  // read through a buffer resource over the query's list, an index past it
  // reading 0, and the other addresses are in bounds for every lane.
  constexpr int SELR = CSA ? kSelCap / kAttThreads : 1;
  int selv[SELR];   // the slot's value as read; turned into a row when stored to LDS
  int sel0 = 0;     // top-k slot of this lane's row of tile 0 (32 wave + lane % 32)
  if constexpr (CSA) {
    const int nsl = sel_m > 1 ? kk / sel_m : kk;   // list entries per query
    const __amdgpu_buffer_rsrc_t rsel = buf_rsrc(topk + (int64_t)qr * nsl, (uint32_t)nsl * 4u);
    const uint32_t past = (uint32_t)nsl * 4u;
#pragma unroll
    for (int i = 0; i < SELR; ++i) {
      const int x = tid + i * kAttThreads;
      const int p = (int)row_beg + x;
      const uint32_t off = x < ent_loc ? (uint32_t)(sel_m > 1 ? p / sel_m : p) * 4u : past;
      selv[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(rsel, off, 0, 0);
    }
    const int x0 = 32 * wave + (lane & 31);
    sel0 = (int)__builtin_amdgcn_raw_buffer_load_b32(
        rsel, x0 < ent_loc && sel_m <= 1 ? (uint32_t)((int)row_beg + x0) * 4u : past, 0, 0);
  }
  const f32x4 gv = reinterpret_cast<const f32x4*>(gamma_q)[tid & (D / 4 - 1)];
  constexpr int NSL = 4 * NJ + 2;
  auto slot_dim = [&](int sl) {
    return sl < 4 * NJ ? 128 * (sl >> 2) + 32 * g + 8 * (sl & 3) : (D - R) + 32 * (sl - 4 * NJ) + 8 * g;
  };
  // slots of the last E4M3 k-step beyond the E4M3 dims stay zero
  auto slot_ok = [&](int sl) { return sl >= 4 * NJ || slot_dim(sl) < D - R; };
  // (slots past the E4M3 dims read rotary dims, in the row; they count as zero)
  const uint16_t* qp = qg + ((int64_t)qr * H + min(head, H - 1)) * D;
  u32x4 qv[NSL];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) qv[sl] = *reinterpret_cast<const u32x4*>(qp + slot_dim(sl));

  // ---- staging: wave w copies tile rows 32w..32w+31 as WPW windows of 64
  // 16-byte slots; slot s holds physical chunk s % CPR of row s / CPR, loaded
  // from logical chunk (s % CPR) ^ swz(row).  Lane l resolves row 32w + l%32.
  const uint8_t* zero_row = g_zero_row;
  // Per-lane source offsets of the copies within a run of contiguous rows:
  // slot 64 i + lane -> row 32w + s / CPR, logical chunk of physical s % CPR.
  unsigned coff[G::WPW];
#pragma unroll
  for (int i = 0; i < G::WPW; ++i) {
    const int sl = 64 * i + lane;
    const int rl = sl / G::CPR, pc = sl - rl * G::CPR;
    coff[i] = (unsigned)((32 * wave + rl) * ROW + 16 * ((pc & ~3) | ((pc & 3) ^ swz(rl))));
  }
  // A whole tile of contiguous present rows (HCA entries, or window rows) is
  // copied from one uniform base, without per-row lookups; its copies are
  // spread over the S^T steps of the previous tile (contig_base), the rest go
  // out at once (issue_tile).
  auto contig_base = [&](int tile) -> const uint8_t* {
    const int x0 = tile * kAttRows;
    const bool full = x0 + kAttRows <= nloc;
    const bool all_ent = x0 + kAttRows <= ent_loc, all_win = x0 >= ent_loc;
    if (!full || !((!CSA && all_ent) || all_win)) return nullptr;
    return all_win ? win_b + (int64_t)(x0 - win_first) * ROW : ent_b + (int64_t)(row_beg + x0) * ROW;
  };
  auto issue_copy = [&](const uint8_t* base, int buf, int i) {
    copy_to_lds16_sbase(base, coff[i], (V4_LDS void*)(s_tile[buf] + 32 * wave * ROW + 1024 * i));
  };
  // Copies of one tile whose rows are gathered: lane l of wave w holds the
  // packed row pointer of tile row 32w + l % 32 (nullptr: absent).
  auto issue_rows = [&](const uint8_t* rp, int buf) {
    const bool ok = rp != nullptr;
    const unsigned long long bal = __ballot(ok);
    if (lane == 0) s_v[buf][wave] = (unsigned)(bal & 0xFFFFFFFFull);
    const long long rpl = (long long)(uintptr_t)(ok ? rp : zero_row);
    uint8_t* Tw = s_tile[buf] + 32 * wave * ROW;
    // the slot arithmetic below is redone per tile (an opaque lane index keeps
    // the compiler from hoisting ~2 registers per copy out of the tile loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < G::WPW; ++i) {
      const int sl = 64 * i + ln;
      const int rl = sl / G::CPR, pc = sl - rl * G::CPR;
      const uint8_t* src = (const uint8_t*)(uintptr_t)__shfl(rpl, rl) +
                           16 * ((pc & ~3) | ((pc & 3) ^ swz(rl)));
      copy_to_lds16(src, (V4_LDS void*)(Tw + 1024 * i));
    }
  };
  // A contiguous tile 0 goes out now, behind only the loads above, so its
  // HBM latency overlaps the rest of the prologue.
  const uint8_t* base0 = ntiles > 0 ? contig_base(0) : nullptr;
  if (base0) {
    if (lane == 0) s_v[0][wave] = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < G::WPW; ++i) issue_copy(base0, 0, i);
  }
  // CSA: a gathered tile 0 too, its row indices read straight from the top-k
  // list (the LDS copy of the split's slice serves the later tiles).
  bool early0 = false;
  if constexpr (CSA) {
    if (!base0 && ntiles > 0 && sel_m <= 1) {
      const int x = 32 * wave + (lane & 31);
      const uint8_t* rp = nullptr;
      if (x < nloc) {
        if (x < ent_loc) {
          const int64_t j = sel0;
          if (j >= 0 && j < Ncap) rp = ent_b + j * ROW;
        } else {
          rp = win_b + (int64_t)(x - win_first) * ROW;
        }
      }
      issue_rows(rp, 0);
      early0 = true;
    }
  }

  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, rturn, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  if constexpr (CSA) {
#pragma unroll
    for (int i = 0; i < SELR; ++i) {
      const int x = tid + i * kAttThreads;
      const int p = (int)row_beg + x;
      // sel_m > 1: the slot holds a block of sel_m rows (-1: empty)
      const int row = sel_m > 1 ? (selv[i] >= 0 ? selv[i] * sel_m + p % sel_m : -1) : selv[i];
      if (x < ent_loc) s_sel[x] = row;
    }
  }
  if (tid < 8) reinterpret_cast<unsigned*>(s_zero)[tid] = 0u;
  if (tid < D / 4) reinterpret_cast<f32x4*>(s_gamma)[tid] = gv;
  // LDS writes only: the q loads stay in flight across this barrier
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // split-local row x -> its packed row in HBM, or nullptr if absent
  auto row_ptr = [&](int x) -> const uint8_t* {
    const bool ent = x < ent_loc;
    int64_t j = (int64_t)x + row_beg;
    bool ok = x < nloc;
    if constexpr (CSA) {
      j = s_sel[ent ? x : 0];
      ok = ok && (!ent || (j >= 0 && j < a.Ncap));
    }
    const uint8_t* p = ent ? ent_b + j * ROW : win_b + (int64_t)(x - win_first) * ROW;
    return ok ? p : nullptr;
  };

  auto issue_tile = [&](int tile, int buf) {
    if (const uint8_t* base = contig_base(tile)) {
      if (lane == 0) s_v[buf][wave] = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < G::WPW; ++i) issue_copy(base, buf, i);
      return;
    }
    issue_rows(row_ptr(tile * kAttRows + 32 * wave + (lane & 31)), buf);
  };
  if (ntiles > 0 && !base0 && !early0) issue_tile(0, 0);

  // ---- q~ = RoPE_t(RMSNorm(q)) in fp32, scaled by 2^qe (per head, exact;
  // qe puts the head's largest |q~| in [128, 256)), as the B operand of S^T.
  // Lane (c, g) holds head c's dims 128 j + 32 g + [0, 32) of every E4M3
  // k-step j (zero past the E4M3 dims) and dims (D - R) + 32 s + 8 g + [0, 8)
  // of the two bf16 k-steps s.  On the E4M3 dims the fp32 value goes into the
  // f8f6f4 MFMA as the sum of two E4M3 terms: hi = its E4M3 rounding, lo = the
  // E4M3 rounding of the exact remainder x - hi.  The pair carries at least
  // the eight significant bits of a bf16 rounding and, because the remainder
  // is usually well inside hi's half-ulp, about 2.6x less rounding error on
  // average.  The rotary dims enter the bf16 MFMA rounded to bf16.
  // Slots of 8 dims: 4j + v for the E4M3 dims, 4 NJ + s for the bf16 ones
  // (loaded at the top of the kernel).
  i32x8 qh[NJ], ql[NJ];
  bf16x8 qt[2];
  float qscale_inv;   // 2^-qe
  {
    if (head >= H) {
#pragma unroll
      for (int sl = 0; sl < NSL; ++sl) qv[sl] = u32x4{0u, 0u, 0u, 0u};
    }
    // one pass over q: the sum of squares, and a bound on the largest |q~|
    // before the RMS scale (|gamma q| on the E4M3 dims; on the rotary dims
    // the length of each rotated pair, which bounds both of its components)
    float ss = 0.f, mb = 0.f, mr2 = 0.f;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int d0 = slot_ok(sl) ? slot_dim(sl) : 0;
      const f32x4 ga = *reinterpret_cast<const f32x4*>(s_gamma + d0);
      const f32x4 gb = *reinterpret_cast<const f32x4*>(s_gamma + d0 + 4);
      const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool ok = slot_ok(sl);
        const float lo = ok ? bf16_bits_to_f32(qv[sl][e] & 0xFFFFu) : 0.f;
        const float hi = ok ? bf16_bits_to_f32(qv[sl][e] >> 16) : 0.f;
        ss += lo * lo + hi * hi;
        const float glo = gm[2 * e] * lo, ghi = gm[2 * e + 1] * hi;
        if (sl >= 4 * NJ) mr2 = fmaxf(mr2, glo * glo + ghi * ghi);
        else mb = fmaxf(mb, fmaxf(fabsf(glo), fabsf(ghi)));
      }
    }
    ss = lane_pair<16>(ss, [](float a, float b) { return a + b; });
    ss = lane_pair<32>(ss, [](float a, float b) { return a + b; });
    mb = fmaxf(mb, sqrtf(mr2));
    mb = lane_pair<16>(mb, [](float a, float b) { return fmaxf(a, b); });
    mb = lane_pair<32>(mb, [](float a, float b) { return fmaxf(a, b); });
    const float rsn = 1.0f / sqrtf(ss / (float)D + a.eps);
    // 2^qe puts the bound (so every |q~|) at most 256, the largest near it
    const float mx = mb * rsn;
    const int qe = mx > 0.f ? 8 - __builtin_amdgcn_frexp_expf(mx) : 0;
    qscale_inv = ldexpf(1.0f, -qe);
    const float rs2 = ldexpf(rsn, qe);
    // second pass: q~ 2^qe = gamma q rsn 2^qe; the E4M3 slots split into
    // hi + lo, the rotary slots rotated and rounded to bf16
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int d0 = slot_ok(sl) ? slot_dim(sl) : 0;
      const f32x4 ga = *reinterpret_cast<const f32x4*>(s_gamma + d0);
      const f32x4 gb = *reinterpret_cast<const f32x4*>(s_gamma + d0 + 4);
      const float gm[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = (gm[2 * e] * bf16_bits_to_f32(qv[sl][e] & 0xFFFFu)) * rs2;
        x[2 * e + 1] = (gm[2 * e + 1] * bf16_bits_to_f32(qv[sl][e] >> 16)) * rs2;
      }
      if (sl < 4 * NJ) {
        const int j = sl >> 2, v = sl & 3;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float x0 = x[4 * h2], x1 = x[4 * h2 + 1], x2 = x[4 * h2 + 2], x3 = x[4 * h2 + 3];
          int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
          hw = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hw, true);
          const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
          const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
          int lw = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b01.x, x1 - b01.y, 0, false);
          lw = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b23.x, x3 - b23.y, lw, true);
          qh[j][2 * v + h2] = slot_ok(sl) ? hw : 0;
          ql[j][2 * v + h2] = slot_ok(sl) ? lw : 0;
        }
      } else {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const int i = (d0 + e - (D - R)) >> 1;
          const float cs = s_cs[i][0], sn = s_cs[i][1];
          const float x0 = x[e], x1 = x[e + 1];
          pk[e >> 1] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
        }
        qt[sl - 4 * NJ] = __builtin_bit_cast(bf16x8, pk);
      }
    }
  }

  const float sl2 = a.scale * kLog2e * qscale_inv;   // undoes the q~ scale
  // running max (log2 units, an integer once set) starts at a finite floor,
  // so masked keys (-inf) give p = 0 without special cases
  float m_run = kNoMax, l_run = 0.f;   // per head (lane column); l_run: this lane's rows
  f32x4 o[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets.  Accumulator i of S^T row block rb (16 rows) in
  // lane group g is row 16 rb + 4 g + i; swz(16 rb + x) = swz(x) ^ 2 (rb & 1).
  //  K, E4M3 k-step j (A of S^T): row 16 rb + c, chunks 8j + 2g + x:
  //   koff[rb & 1][x] + 16 rb ROW + 128 j
  int koff[2][2];
  //  K, bf16 k-step s: chunk BFC + 4s + g: ktoff[rb & 1] + 16 rb ROW + 64 s
  int ktoff[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int sw = swz(c) ^ (2 * p);
#pragma unroll
    for (int x = 0; x < 2; ++x) koff[p][x] = c * ROW + 64 * (g >> 1) + 16 * ((2 * (g & 1) + x) ^ sw);
    ktoff[p] = c * ROW + 16 * (BFC + (g ^ sw));
  }
  //  V^T via tr_b8: source lane (G = lane/16, j = (lane%16)/2, h = lane%2) of
  //  read nn addresses the row of operand byte 8 nn + j of lane group G,
  //  32 nn + 16 (j/4) + 4G + j%4 (swizzle independent of nn), dims 16 db + 8h:
  //  v8off[db & 3] + 32 nn ROW + 64 (db >> 2)
  int v8off[4];
  {
    const int j = (lane & 15) >> 1, h = lane & 1;
    const int row = 16 * (j >> 2) + 4 * g + (j & 3);
#pragma unroll
    for (int d3 = 0; d3 < 4; ++d3) v8off[d3] = row * ROW + 16 * (d3 ^ swz(row)) + 8 * h;
  }
  //  V^T via tr_b16 (bf16 dims, 16-dim block e): source lane (G, j = (lane%16)/4,
  //  q = lane%4) of k-step s, half hl addresses the row of operand element
  //  4 hl + j of lane group G, 16 (2s + (hl ^ G%2)) + 4G + j, dims
  //  (D - R) + 16 e + 4q: v16off[hl][e & 1] + 32 s ROW + 64 (e >> 1)
  int v16off[2][2];
  {
    const int j = (lane & 15) >> 2, q = lane & 3;
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) {
      const int row = 16 * (hl ^ (g & 1)) + 4 * g + j;
#pragma unroll
      for (int e1 = 0; e1 < 2; ++e1)
        v16off[hl][e1] = row * ROW + 16 * (BFC + ((2 * e1 + (q >> 1)) ^ swz(row))) + 8 * (q & 1);
    }
  }

  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  //  qk: S^T for 128 rows x 16 heads, absent rows at -inf, and the logit
  //      maximum per head of each 64-row scale block, for this lane's pair of
  //      lane groups (mp) and the other pair (mo).  Row blocks go in pairs
  //      (two accumulator chains); the operands of each step are read one
  //      step ahead, and the scheduling fences keep the compiler from
  //      hoisting every read of the tile.
  auto qk = [&](const uint8_t* T, int cur, f32x4 (&sacc)[8], float (&mp)[2], float (&mo)[2], auto&& side) {
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NS = NJ + 2;   // steps per row-block pair: E4M3 k-steps, then bf16
    static_assert(G::WPW <= 4 * NS, "every copy of the next tile gets a step");
    auto load = [&](int st, i32x8 (&k8)[2], u32x4 (&kt)[2]) {
      const int rp = st / NS, ks = st % NS;
#pragma unroll
      for (int x2 = 0; x2 < 2; ++x2) {
        const int rb = 2 * rp + x2;
        if (ks < NJ) {
          const uint8_t* kp = T + 16 * rb * ROW + 128 * ks;
          const uint8_t* p0 = kp + koff[rb & 1][0];
          const uint8_t* p1 = kp + koff[rb & 1][1];
          if (ks == NJ - 1 && g >= 2) {   // past the E4M3 dims: zeros (q~ is zero there too)
            p0 = s_zero;
            p1 = s_zero + 16;
          }
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(p0);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(p1);
          k8[x2] = __builtin_bit_cast(i32x8, u32x8{w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w});
        } else {
          kt[x2] = *reinterpret_cast<const u32x4*>(T + 16 * rb * ROW + ktoff[rb & 1] + 64 * (ks - NJ));
        }
      }
    };
    i32x8 k8[2][2];
    u32x4 kt[2][2];
    load(0, k8[0], kt[0]);
#pragma unroll
    for (int st = 0; st < 4 * NS; ++st) {
      if (st + 1 < 4 * NS) load(st + 1, k8[(st + 1) & 1], kt[(st + 1) & 1]);
      const int rp = st / NS, ks = st % NS;
      if (ks < NJ) {
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2)
          sacc[2 * rp + x2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              k8[st & 1][x2], qh[ks], sacc[2 * rp + x2], 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2)
          sacc[2 * rp + x2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              k8[st & 1][x2], ql[ks], sacc[2 * rp + x2], 0, 0, 0, 127, 0, 127);
      } else {
#pragma unroll
        for (int x2 = 0; x2 < 2; ++x2)
          sacc[2 * rp + x2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kt[st & 1][x2]), qt[ks - NJ], sacc[2 * rp + x2], 0, 0, 0);
      }
      side(st);   // e.g. one copy of the next tile, behind this step's MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
    // row 16 rb + 4g + i is bit 16 (rb & 1) + 4g + i of staging word rb / 2
    unsigned vm[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) vm[w] = __builtin_amdgcn_readfirstlane(s_v[cur][w]);
    if ((vm[0] & vm[1] & vm[2] & vm[3]) != 0xFFFFFFFFu) {   // partial tile: mask the absent rows
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const unsigned vl = vm[rb >> 1] >> (16 * (rb & 1) + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((vl >> i) & 1u)) sacc[rb][i] = -INFINITY;
      }
    }
    // sl2 > 0, so the raw maximum scales to the logit maximum
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float m = sacc[4 * h][0];
#pragma unroll
      for (int rb = 4 * h; rb < 4 * h + 4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[rb][i]);
      m *= sl2;
      mp[h] = lane_pair<16>(m, [](float a, float b) { return fmaxf(a, b); });
      mo[h] = lane_xor32(mp[h]);
    }
  };
  //  pv: online softmax of the tile against the running max m_run, then
  //      O^T += V^T P^T.  Operand byte 4 rb + i of lane group g is row
  //      16 rb + 4g + i; bytes 0-15 of lane groups {0,1} / {2,3} form one E8M0
  //      scale block, bytes 16-31 another.  Block (pair, half) is
  //      exponentiated as p' = 2^(x - c) with c an integer that puts its
  //      largest p' in (128, 256]; its weight 2^(c - m_run) is the operand's
  //      E8M0 scale on the E4M3 dims and is applied in fp32 on the bf16 dims.
  auto pv = [&](const uint8_t* T, f32x4 (&sacc)[8], const float (&mp)[2], const float (&mo)[2]) {
    float cown[2];
    int eown[2], eoth[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cown[h] = fmaxf(ceilf(mp[h]) - 8.0f, m_run - 120.0f);
      const float coth = fmaxf(ceilf(mo[h]) - 8.0f, m_run - 120.0f);
      eown[h] = (int)fminf(fmaxf(cown[h] - m_run, -127.0f), 127.0f);
      eoth[h] = (int)fminf(fmaxf(coth - m_run, -127.0f), 127.0f);
    }
    float ls[2] = {0.f, 0.f};
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sacc[rb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[rb][i], sl2, -cown[rb >> 2]));
        ls[rb >> 2] += sacc[rb][i];
      }
    l_run += ldexpf(ls[0], eown[0]) + ldexpf(ls[1], eown[1]);
    // hi + lo E4M3 terms, dword rb = the four rows of row block rb
    i32x8 ph, pl;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
      const float p0 = sacc[rb][0], p1 = sacc[rb][1], p2 = sacc[rb][2], p3 = sacc[rb][3];
      int hw = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      hw = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, hw, true);
      const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
      const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
      int lw = __builtin_amdgcn_cvt_pk_fp8_f32(p0 - b01.x, p1 - b01.y, 0, false);
      lw = __builtin_amdgcn_cvt_pk_fp8_f32(p2 - b23.x, p3 - b23.y, lw, true);
      ph[rb] = hw;
      pl[rb] = lw;
    }
    // lane group g supplies the scale of block (pair g % 2, half g / 2): its
    // own pair (g / 2) for g = 0, 3, the other pair for g = 1, 2
    const int hsel = g >> 1;
    const int eo = hsel ? eown[1] : eown[0], et = hsel ? eoth[1] : eoth[0];
    const int sc = 127 + ((g == 0 || g == 3) ? eo : et);
    __builtin_amdgcn_sched_barrier(0);
    auto load_v8 = [&](int db, i32x8& v) {
      i32x2 w[4];
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
        w[nn] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (V4_LDS i32x2*)(T + v8off[db & 3] + 32 * nn * ROW + 64 * (db >> 2)));
      v = i32x8{w[0].x, w[0].y, w[1].x, w[1].y, w[2].x, w[2].y, w[3].x, w[3].y};
    };
    auto load_v16 = [&](int s2, bf16x8 (&v)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u32x2 lo = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (V4_LDS i16x4*)(T + v16off[0][e & 1] + 32 * s2 * ROW + 64 * (e >> 1))));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (V4_LDS i16x4*)(T + v16off[1][e & 1] + 32 * s2 * ROW + 64 * (e >> 1))));
        v[e] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      }
    };
    // bf16 dims first (p relative to the running max), so p' dies before the
    // E4M3 dims.  k-step s covers row blocks 2s and 2s + 1: element 4 hl + j
    // of lane group g is row 16 (2s + (hl ^ g%2)) + 4g + j.
    bf16x8 vt[2][4];
    load_v16(0, vt[0]);
    const bool godd = (g & 1) != 0;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      if (s2 + 1 < 4) load_v16(s2 + 1, vt[(s2 + 1) & 1]);
      const int es = s2 < 2 ? eown[0] : eown[1];
      const f32x4 a0 = godd ? sacc[2 * s2 + 1] : sacc[2 * s2];
      const f32x4 a1 = godd ? sacc[2 * s2] : sacc[2 * s2 + 1];
      const u32x4 pk = {pack_bf16x2(ldexpf(a0[0], es), ldexpf(a0[1], es)),
                        pack_bf16x2(ldexpf(a0[2], es), ldexpf(a0[3], es)),
                        pack_bf16x2(ldexpf(a1[0], es), ldexpf(a1[1], es)),
                        pack_bf16x2(ldexpf(a1[2], es), ldexpf(a1[3], es))};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[NB8 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[s2 & 1][e], pb, o[NB8 + e], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // E4M3 dims, two blocks a step (two accumulator chains), operands one step ahead
    i32x8 vf[2][2];
    load_v8(0, vf[0][0]);
    load_v8(1, vf[0][1]);
#pragma unroll
    for (int st = 0; st < NB8 / 2; ++st) {
      if (st + 1 < NB8 / 2) {
        load_v8(2 * st + 2, vf[(st + 1) & 1][0]);
        load_v8(2 * st + 3, vf[(st + 1) & 1][1]);
      }
#pragma unroll
      for (int x2 = 0; x2 < 2; ++x2)
        o[2 * st + x2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf[st & 1][x2], ph, o[2 * st + x2],
                                                                          0, 0, 0, 127, 0, sc);
#pragma unroll
      for (int x2 = 0; x2 < 2; ++x2)
        o[2 * st + x2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf[st & 1][x2], pl, o[2 * st + x2],
                                                                          0, 0, 0, 127, 0, sc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile t lives in buffer t & 1.  A tile issues the copies of tile t+1 (into
  // the buffer every wave finished reading before the last barrier), uses
  // tile t, waits for its own copies and meets the other waves at the
  // barrier, so tile t+1 is complete in LDS and every read of tile t is done.
  // A tile whose logits pass the running max by more than the headroom
  // leaves the inner loop, which then never touches the accumulators outside
  // the MFMAs; the rescale and that tile finish outside it (always once, at
  // the first tile with a present row).
  int tile = 0;
  while (tile < ntiles) {
    f32x4 sacc[8];
    float mp[2], mo[2];
    const uint8_t* T = nullptr;
    bool grow = false;
    for (; tile < ntiles; ++tile) {
      const int cur = tile & 1;
      const uint8_t* nbase = tile + 1 < ntiles ? contig_base(tile + 1) : nullptr;
      if (nbase) {
        if (lane == 0) s_v[cur ^ 1][wave] = 0xFFFFFFFFu;
      } else if (tile + 1 < ntiles) {
        issue_tile(tile + 1, cur ^ 1);
      }
      T = s_tile[cur];
      // two instances of the step sequence, so that no branch splits it (a
      // branch around each copy let the compiler move the MFMAs of several
      // steps past the loads and copies of the next ones)
      if (nbase)
        qk(T, cur, sacc, mp, mo, [&](int st) {
          if (st < G::WPW) issue_copy(nbase, cur ^ 1, st);
        });
      else
        qk(T, cur, sacc, mp, mo, [](int) {});
      if (!CSA && a.logits2 && head < a.H) {   // the tile's logits (log2 units; absent rows -inf)
        float* lp = a.logits2 + ((int64_t)qr * a.logits_stride + row_beg +
                                 (int64_t)tile * kAttRows + 4 * g) * 64 + head;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) lp[(16 * rb + i) * 64] = sacc[rb][i] * sl2;
      }
      if (__any(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mo[0], mo[1])) > m_run + kLazyMax)) {
        grow = true;
        break;
      }
      pv(T, sacc, mp, mo);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (!grow) break;
    const float mt = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mo[0], mo[1]));
    const float m_new = mt > m_run + kLazyMax ? ceilf(mt) : m_run;
    if (m_run != kNoMax) {   // before the first present row O and l are still zero
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < NB; ++db) o[db] *= corr;
    }
    m_run = m_new;
    pv(T, sacc, mp, mo);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    ++tile;
  }

  if (head >= a.H) return;
  // full denominator of this lane's head: all four lane groups
  l_run = lane_pair<16>(l_run, [](float a, float b) { return a + b; });
  l_run = lane_pair<32>(l_run, [](float a, float b) { return a + b; });
  // accumulator i of block db holds dim 16 db + 4g + i
  if (nsplit > 1) {
    // unnormalised partial O in block floating point: 16-bit signed
    // normalised integers and one power-of-two scale per (split, head), 2^e
    // the head's largest |O| rounded up, so every element lands within
    // 2^-15 of that largest value (bf16's bytes, fp32-like precision where
    // it matters: the dominant elements of the dominant split); (max, sum,
    // e) in fp32.  The merge kernel adds the sink.
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[db][i]));
    amax = lane_pair<16>(amax, [](float a, float b) { return fmaxf(a, b); });
    amax = lane_pair<32>(amax, [](float a, float b) { return fmaxf(a, b); });
    const int ex = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;   // amax < 2^ex
    const float to_unit = ldexpf(1.0f, -ex);   // |O| 2^-ex < 1: snorm16 = round(32767 |O| 2^-ex)
    uint16_t* po = a.part_o + (slot * a.H + head) * D;
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const s16x2 lo = __builtin_amdgcn_cvt_pknorm_i16(o[db][0] * to_unit, o[db][1] * to_unit);
      const s16x2 hi = __builtin_amdgcn_cvt_pknorm_i16(o[db][2] * to_unit, o[db][3] * to_unit);
      *reinterpret_cast<u32x2*>(po + 16 * db + 4 * g) =
          u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
    }
    if (g == 0) {
      float* pm = a.part_ml + (slot * a.H + head) * 4;
      *reinterpret_cast<f32x4*>(pm) =
          f32x4{l_run > 0.f ? m_run : -INFINITY, l_run, (float)ex, 0.f};
    }
    return;
  }
  const bool seen = l_run > 0.f;
  const float mr = seen ? m_run : -INFINITY;
  const float z2 = a.sink ? a.sink[head] * kLog2e : -INFINITY;   // no sink: -inf
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
  for (int db = 0; db < NB; ++db) {
    const int d0 = 16 * db + 4 * g;
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
    const int64_t qh = (int64_t)qr * a.H + head;
    *reinterpret_cast<u32x2*>(op + d0) = final_bf16x4<CSA>(a, qh * D + d0, qh, v);   // mix: CSA only
  }
  if (a.lse && g == 0) a.lse[(int64_t)qr * a.H + head] = lse;
}

// Combine split partials with the sink, rotate by -t, store bf16 and lse.
// Grid: (ceil(H / HPW), B*Tq) with HPW = 1024 / D heads per workgroup of 256
// threads.  Wave w first turns the (max, sum) pairs of heads h0 + w, h0 + w + 4,
// .. into one weight per split (splits <= 64: one lane each); then every thread merges
// four dims of one head, all of its split loads in flight together.
template <int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendBatch ab) {
  const AttendArgs& a = ab.p[blockIdx.z];
  const int qr = blockIdx.y;
  // every argument read in one round before any branch, as in attend_kernel
  const bool flat = a.flat, ragged = a.ragged;
  const int B = a.B, Tq = a.Tq, H = a.H, splits = a.splits;
  const int64_t q_pos0 = a.q_pos0;
  const uint16_t* const part_o = a.part_o;
  const float* const part_ml = a.part_ml;
  const float* const sink = a.sink;
  float* const lse = a.lse;
  uint16_t* const out = a.out;
  const float* const mix_gates = a.mix_gates;
  asm volatile("" ::"s"(part_o), "s"(part_ml), "s"(sink), "s"(lse), "s"(out), "s"(mix_gates),
               "s"(q_pos0));
  asm volatile("" ::"s"((int)flat), "s"((int)ragged), "s"(B), "s"(Tq), "s"(H), "s"(splits));
  const double rturn = a.rope.t[threadIdx.x & 31];
  if (qr >= B * Tq) return;
  // the per-sequence tables through the argument segment's address (see attend_kernel)
  const char* const my_args = (const char*)__builtin_amdgcn_kernarg_segment_ptr() +
                              offsetof(AttendBatch, p) + (size_t)blockIdx.z * sizeof(AttendArgs);
  int S = splits;
  int64_t slot0 = (int64_t)qr * S;   // this query's first partial slot
  if (flat) {
    const int* sl = reinterpret_cast<const int*>(my_args + offsetof(AttendArgs, slot0)) + qr;
    slot0 = sl[0];
    S = sl[1] - sl[0];
  }
  if (S <= 1) return;   // the attention kernel stored this query's output itself
  int64_t qpos = q_pos0;
  if (ragged)
    qpos = *reinterpret_cast<const int64_t*>(my_args + offsetof(AttendArgs, pos) +
                                             sizeof(int64_t) * ((qr / Tq) & (kMaxRagged - 1)));
  constexpr int R = 64;
  constexpr int QPH = D / 4;          // threads per head (four dims each)
  constexpr int HPW = 256 / QPH;      // heads per workgroup
  const int h0 = blockIdx.x * HPW;
  const int64_t t = qpos + (qr % Tq);
  __shared__ float s_w[HPW][64];
  __shared__ float s_cs[R / 2][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The partials do not depend on the weights: the first kSp of them are
  // requested before the (max, sum, scale) records, so the two round trips
  // overlap (slots past S read as zero and touch no memory).
  constexpr int kSp = 16;
  const int hh = tid / QPH, d = 4 * (tid % QPH);
  const int h = h0 + hh;
  const bool mine = hh < HPW && h < H;
  const int64_t sstride = (int64_t)H * D;   // elements between a query's split slots
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(part_o + slot0 * sstride, (uint32_t)(S * sstride * 2));
  const uint32_t voff = mine ? (uint32_t)((h * D + d) * 2) : 0x7FFFFF00u;
  u32x2 v0[kSp];
#pragma unroll
  for (int u = 0; u < kSp; ++u) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, voff + (uint32_t)(u * sstride * 2), 0, 0);
    v0[u] = u32x2{w[0], w[1]};
  }
  if (tid < R / 2) {
    float cs, sn;
    rope_cos_sin(t, rturn, &cs, &sn);
    s_cs[tid][0] = cs;
    s_cs[tid][1] = sn;
  }
  for (int hw = wave; hw < HPW; hw += 4) {
    const int hx = h0 + hw;
    if (hx >= H) break;
    // both records of the head through buffer resources (no load in a
    // branch: the compiler would wait for each at once): split `lane`'s
    // (max, sum, e), reading 0 past the S splits, and the sink
    const bool own = lane < S;
    const __amdgpu_buffer_rsrc_t rml =
        buf_rsrc(part_ml + (slot0 * H + hx) * 4, (uint32_t)(S * H * 16));
    const __amdgpu_buffer_rsrc_t rsk = buf_rsrc(sink, (uint32_t)(H * 4));
    const auto mlv = __builtin_amdgcn_raw_buffer_load_b128(
        rml, own ? (uint32_t)(lane * H * 16) : 0x7FFFFF00u, 0, 0);
    const unsigned skv = __builtin_amdgcn_raw_buffer_load_b32(
        rsk, sink ? (uint32_t)(hx * 4) : 0x7FFFFF00u, 0, 0);
    const f32x4 ml = own ? f32x4{__uint_as_float(mlv[0]), __uint_as_float(mlv[1]),
                                 __uint_as_float(mlv[2]), __uint_as_float(mlv[3])}
                         : f32x4{-INFINITY, 0.f, 0.f, 0.f};
    const float z2 = sink ? __uint_as_float(skv) * kLog2e : -INFINITY;
    const float M = fmaxf(wave_max(ml.x), z2);
    const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    float den = wave_sum(ml.y * w);
    if (M != -INFINITY) den += exp2f(z2 - M);
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    // also undoes the partial's scale: O = q 2^e / 32767
    s_w[hw][lane] = ldexpf(w * inv, (int)ml.z) * (1.0f / 32767.0f);
    if (lse && lane == 0)
      lse[(int64_t)qr * H + hx] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
  __syncthreads();
  if (!mine) return;
  auto add = [](f32x4& x, float w, u32x2 v) {
    x += w * f32x4{(float)(int)(short)(v.x & 0xFFFFu), (float)((int)v.x >> 16),
                   (float)(int)(short)(v.y & 0xFFFFu), (float)((int)v.y >> 16)};
  };
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kSp; ++u) add(x, u < S ? s_w[hh][u] : 0.f, v0[u]);
  const uint16_t* po = part_o + (slot0 * H + h) * D + d;
  for (int s0 = kSp; s0 < S; s0 += 8) {   // more splits: eight partials in flight
    u32x2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const u32x2*>(po + (int64_t)min(s0 + u, S - 1) * sstride);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(x, s0 + u < S ? s_w[hh][s0 + u] : 0.f, v[u]);
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
  const int64_t qh = (int64_t)qr * H + h;
  *reinterpret_cast<u32x2*>(out + qh * D + d) = final_bf16x4<true>(a, qh * D + d, qh, y);
}

int attend_splits(int B, int Tq, int64_t rows_max, bool csa, int wg_budget) {
  const int64_t q = (int64_t)B * Tq;
  if (q <= 0 || rows_max <= 0) return 1;
  // about one workgroup per CU (one fits a CU); within a smaller budget, at
  // most the budget
  int64_t s = wg_budget >= 256 ? (256 + q - 1) / q : wg_budget / q;
  const int64_t by_rows = (rows_max + kAttRows - 1) / kAttRows;  // at least one tile per split
  if (s > by_rows) s = by_rows;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  // CSA stages a split's top-k slots in LDS: at most kSelCap rows a split
  if (csa)
    while (s < 64 && split_chunk(rows_max, (int)s) > kSelCap) ++s;
  return (int)s;
}

hipError_t launch_attend_batch(const AttendBatch& ab, int n, hipStream_t st) {
  const AttendArgs& a = ab.p[0];
  const int64_t q = (int64_t)a.B * a.Tq;
  if (q == 0) return hipSuccess;
  const bool csa = a.topk != nullptr;
  int gx = 1;
  bool merge = false;
  for (int z = 0; z < n; ++z) {
    const AttendArgs& x = ab.p[z];
    // one kernel instance serves the batch: same kind, shapes, query block
    // and grid form
    if ((x.topk != nullptr) != csa || x.D != a.D || x.H != a.H || x.B != a.B || x.Tq != a.Tq ||
        x.flat != a.flat)
      return hipErrorInvalidValue;
    // every split's slice of the top-k list must fit the kernel's LDS copy
    if (csa && !x.flat && split_chunk(x.rows_max, x.splits) > kSelCap) return hipErrorInvalidValue;
    if (csa && x.sel_m > 1 && x.k % x.sel_m != 0) return hipErrorInvalidValue;
    const int xs = x.flat ? x.slot0[x.B] : x.splits;
    gx = xs > gx ? xs : gx;
    merge = merge || (x.flat ? x.slot0[x.B] > x.B : x.splits > 1);
  }
  dim3 grid(gx, a.flat ? 1u : (unsigned)q, n);
#define V4_ATT(D)                                                             \
  do {                                                                        \
    if (csa) attend_kernel<D, true><<<grid, kAttThreads, 0, st>>>(ab);        \
    else attend_kernel<D, false><<<grid, kAttThreads, 0, st>>>(ab);           \
    if (merge)                                                                \
      attend_merge_kernel<D><<<dim3((a.H + 1024 / (D) - 1) / (1024 / (D)), (unsigned)q, n), 256, 0, st>>>(ab); \
  } while (0)
  switch (a.D) {
    case 128: V4_ATT(128); break;
    case 256: V4_ATT(256); break;
    default: V4_ATT(512); break;
  }
#undef V4_ATT
  return hipGetLastError();
}

void plan_flat_splits(AttendArgs& a, const int64_t* rows, bool csa) {
  const int B = a.B;
  a.flat = false;
  if (B < 1 || B > kMaxRagged || a.Tq != 1) return;
  const int64_t cap = (int64_t)B * a.splits;          // the partial slots the workspace holds
  const int64_t want = cap < 256 ? cap : (B > 256 ? B : 256);   // about one workgroup per CU
  int64_t tiles[kMaxRagged], total = 0;
  for (int b = 0; b < B; ++b) {
    tiles[b] = (rows[b] + kAttRows - 1) / kAttRows;
    total += tiles[b] > 0 ? tiles[b] : 1;
  }
  auto splits_of = [&](int b, int64_t per) {
    int64_t s = (tiles[b] + per - 1) / per;
    if (csa)   // a split's slice of the top-k list fits the kernel's LDS copy
      while (split_chunk(rows[b], (int)s) > kSelCap) ++s;
    s = s < 1 ? 1 : (s > 64 ? 64 : s);
    return s;
  };
  for (int64_t per = (total + want - 1) / want; per <= (1 << 20); ++per) {
    int64_t sum = 0;
    for (int b = 0; b < B; ++b) sum += splits_of(b, per);
    if (sum <= cap) {
      int acc = 0;
      for (int b = 0; b < B; ++b) {
        a.slot0[b] = acc;
        acc += (int)splits_of(b, per);
      }
      a.slot0[B] = acc;
      a.flat = true;
      return;
    }
  }
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  AttendBatch ab{};
  ab.p[0] = a;
  return launch_attend_batch(ab, 1, st);
}

}  // namespace v4
