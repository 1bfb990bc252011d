// Lightning-indexer scores: score_{t,j} = sum_h w_{t,h} * ReLU(q_{t,h} . k_j).
//
// Pages: a lightning indexer scores each query against the compressed entries
// ("DeepSeek-V4: Making a Million Tokens Affordable", section "Two ways to
// shrink attention, interleaved"); it is a few small heads, cheap next to the
// main attention ("DeepSeek-V4, explained", step 3 of how one query's layer
// works).  One indexer key per entry is shared by all indexer heads.
//
// Design (decode, few queries): the dense contraction [HI heads x dI] x
// [dI x keys] runs on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, the
// faster bf16 shape) with the query's heads as M and 32 keys as N.  q (all
// heads of the query) and the head weights sit in LDS, shared by the four
// waves, which keeps the registers small.  The row's keys are cut into
// 32-key chunks dealt round-robin over the row's waves (the waves of a row
// read one compact front of the key array, which measured faster than a
// contiguous range per wave); a chunk is read with streaming (non-temporal)
// loads, every instruction covering 1 KiB of contiguous keys, staged in the
// wave's own padded LDS rows and read back in the MFMA's operand layout,
// while the next chunk's loads are in flight.
// The ReLU, the head weights and the head sum are applied to the fp32
// accumulators in registers (32 heads per lane, then one cross-lane add), so
// only 4 bytes per entry leave the kernel.  At 1M tokens this kernel streams
// 64 MiB of keys per query and is HBM-bound (64 FLOP per byte).
//
// Design (prefill, a block of queries of one sequence): every key is shared
// by all queries, so the contraction is MFMA-bound and the keys are read once
// per 8 queries (from the Infinity Cache, where a million-token key set fits).
// A workgroup of 8 waves holds one query per wave (q for 64 heads x 128 dims
// in registers as the A operands of v_mfma_f32_32x32x16_bf16, the faster bf16
// shape on this chip) and walks its key range in
// 128-key tiles copied straight to LDS with global_load_lds (four 1 KiB
// copies per wave per tile, two tiles in turn, chunks XOR-swizzled by row so
// the operand reads are free of bank conflicts).  The vector ALU work per
// MFMA (ReLU and weighted head sum) is about half the MFMA time, so it is
// kept lean: the ReLU is one integer max, and the scores of a tile are stored
// at the start of the next step, off the path of the copy wait.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

// max(x, 0) as one integer max on the bits: a negative float (sign bit set)
// is a negative int and becomes +0, a non-negative one is unchanged (fmaxf
// would first quiet a possible signalling NaN, a second instruction).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

template <int DI, int MB>
__global__ __launch_bounds__(256) void index_score_kernel(IndexScoreArgs a) {
  constexpr int M2 = (MB + 1) / 2;   // 32-head blocks (the MFMA's M)
  constexpr int QSTR = 2 * DI + 16;  // LDS bytes per q row (16-byte skew per head)
  constexpr int KSTR = 2 * DI + 16;  // LDS bytes per staged key row (16-byte skew)
  constexpr int RB = 2 * DI;         // key row bytes
  constexpr int P = RB / 16;         // 16-byte pieces per key row
  constexpr int KPI = 64 / P;        // keys per load instruction
  constexpr int NL = 32 / KPI;       // load instructions per 32-key chunk
  // every argument read in one round before any branch (each dependent round
  // trip to the argument segment costs a memory latency; the empty asm
  // statements keep the compiler from issuing the reads where first used)
  asm volatile("" ::"s"(a.q_idx), "s"(a.w_idx), "s"(a.k_idx), "s"(a.Ncap), "s"(a.n_entries),
               "s"(a.q_pos0), "s"(a.scores), "s"(a.score_stride));
  asm volatile("" ::"s"(a.B), "s"(a.Tq), "s"(a.HI), "s"(a.m), "s"((int)a.ragged));
  int b = blockIdx.z, blk = blockIdx.x, nblk = gridDim.x;
  const int r = blockIdx.y;
  if (a.ragged && a.Tq == 1) {   // flat grid: find this workgroup's sequence
    b = 0;
    while (b + 1 < a.B && (int)blockIdx.x >= a.wg_start[b + 1]) ++b;
    blk = blockIdx.x - a.wg_start[b];
    nblk = a.wg_start[b + 1] - a.wg_start[b];
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = (a.ragged ? a.pos.p[b] : a.q_pos0) + r;
  // positions below 2^31 take the 32-bit division
  int64_t V = (uint64_t)(t + 1) < (1ull << 31) ? (int64_t)((uint32_t)(t + 1) / (uint32_t)a.m)
                                               : (t + 1) / a.m;
  if (V > a.n_entries) V = a.n_entries;
  // 32-key chunks are dealt round-robin over the row's waves, so at any time
  // the waves of a row read one compact front of the key array
  const int64_t nch = (V + 31) / 32;
  const int64_t NW = (int64_t)nblk * 4;
  const int64_t gw = (int64_t)blk * 4 + wave;
  if ((int64_t)blk * 4 >= nch) return;   // the whole block is past the visible keys

  __shared__ __attribute__((aligned(16))) uint8_t s_q[M2 * 32 * QSTR];
  __shared__ __attribute__((aligned(16))) uint8_t s_k[4][32 * KSTR];
  __shared__ __attribute__((aligned(16))) float s_w[M2 * 32];

  // A chunk is read with fully contiguous loads (1 KiB per instruction: lane
  // l takes 16-byte piece l % P of key l / P of each group of KPI keys).
  // Keys past the row re-read the last visible key (score not stored).
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx + (int64_t)b * a.Ncap * DI);
  u32x4 kv[NL];
  auto load = [&](int64_t j0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t j = min(j0 + i * KPI + lane / P, V - 1);
      kv[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + j * RB + 16 * (lane % P)));
    }
  };
  if (gw < nch) load(gw * 32);   // in flight while q and w are staged

  // q of this query (all heads) and the head weights in LDS, shared by the waves
  const int64_t qrow = (int64_t)b * a.Tq + r;
  const uint16_t* qp = a.q_idx + qrow * a.HI * DI;
  for (int x = tid; x < M2 * 32 * DI / 8; x += 256) {
    const int h = x / (DI / 8), d8 = x % (DI / 8);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < a.HI) v = *reinterpret_cast<const u32x4*>(qp + (int64_t)h * DI + d8 * 8);
    *reinterpret_cast<u32x4*>(s_q + h * QSTR + d8 * 16) = v;
  }
  if (tid < M2 * 32) s_w[tid] = tid < a.HI ? a.w_idx[qrow * a.HI + tid] : 0.f;
  __syncthreads();
  if (gw >= nch) return;

  float* sp = a.scores + qrow * a.score_stride;
  uint8_t* kst = s_k[wave];
  for (int64_t ch = gw; ch < nch; ch += NW) {
    // stage the chunk in this wave's LDS rows, start the next one, then read
    // it back in the MFMA's operand layout (lane l: dims 16ks + 8(l/32) of key l % 32)
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *reinterpret_cast<u32x4*>(kst + (i * KPI + lane / P) * KSTR + 16 * (lane % P)) = kv[i];
    if (ch + NW < nch) load((ch + NW) * 32);
    // q is re-read from LDS for every chunk: an opaque offset keeps the
    // compiler from holding it in registers across chunks
    int qo = (lane & 31) * QSTR + 16 * (lane >> 5);
    asm volatile("" : "+v"(qo));
    const uint8_t* qa = s_q + qo;
    f32x16 acc[M2];
#pragma unroll
    for (int hb = 0; hb < M2; ++hb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) {
      const bf16x8 kb = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(kst + (lane & 31) * KSTR + 32 * ks + 16 * (lane >> 5)));
#pragma unroll
      for (int hb = 0; hb < M2; ++hb) {
        const bf16x8 q8 = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(qa + hb * 32 * QSTR + 32 * ks));
        acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q8, kb, acc[hb], 0, 0, 0);
      }
    }
    // lane holds key lane % 32, heads hb*32 + (i/4)*8 + (lane/32)*4 + i%4
    float sc = 0.f;
#pragma unroll
    for (int hb = 0; hb < M2; ++hb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_w[hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu(acc[hb][4 * i4 + i]), sc);
      }
    sc += __shfl_xor(sc, 32);
    const int64_t j = ch * 32 + (lane & 31);
    if (lane < 32 && j < V) sp[j] = sc;
  }
}

constexpr int kBlkWaves = 8;    // waves per workgroup
constexpr int kBlkQPW = 1;      // queries per wave
constexpr int kBlkQ = kBlkWaves * kBlkQPW;   // queries per workgroup
constexpr int kBlkKeys = 128;   // keys per LDS tile

// 64 lanes x 16 bytes from per-lane global addresses into 1 KiB of LDS at
// `dst` (+16 bytes per lane).  Written as asm so that the compiler does not
// wait for the copy before every LDS read; the tile loop waits for it itself
// (vmcnt) before the barrier that publishes a tile.  No register result; the
// address registers are read at issue.
__device__ __forceinline__ void idx_copy_to_lds16(const void* src, V4_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

__global__ __launch_bounds__(kBlkWaves * 64) void index_score_block_kernel(IndexScoreArgs a,
                                                                           int64_t key_chunk) {
  constexpr int KEYS = kBlkKeys;
  constexpr int NBUF = 2;                  // tiles in LDS
  constexpr int DI = 128;
  constexpr int RB = 2 * DI;               // key row bytes
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
  constexpr int TILE = KEYS * RB;      // bytes per tile
  constexpr int KS = DI / 16;              // 32x32x16 k-steps
  constexpr int CPW = TILE / 1024 / kBlkWaves;   // 1 KiB copies per wave per tile
  static_assert(CPW * 1024 * kBlkWaves == TILE, "whole copies per wave");
  static_assert(CPR == 16, "the row swizzle spans 16 chunks");
  const int b = blockIdx.z, qg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = qg * kBlkQ + wave * kBlkQPW;      // this wave's first query
  const int64_t qpos = a.ragged ? a.pos.p[b] : a.q_pos0;
  auto visible = [&](int rr) {
    const int64_t t = qpos + rr;
    const int64_t v = (t + 1) / a.m;
    return v < a.n_entries ? v : a.n_entries;
  };
  const int64_t Vlast = visible(min(qg * kBlkQ + kBlkQ - 1, a.Tq - 1));  // largest in group
  const int64_t kc0 = (int64_t)blockIdx.x * key_chunk;
  const int64_t kc1 = min(kc0 + key_chunk, Vlast);
  if (kc0 >= kc1) return;
  const int ntiles = (int)((kc1 - kc0 + KEYS - 1) / KEYS);

  __shared__ __attribute__((aligned(16))) uint8_t s_k[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float s_w[kBlkQ][64];

  const bool wok = r0 < a.Tq;   // the wave has at least one query
  int64_t qrow[kBlkQPW], jmax[kBlkQPW];
#pragma unroll
  for (int u = 0; u < kBlkQPW; ++u) {
    const int r = r0 + u;
    qrow[u] = (int64_t)b * a.Tq + min(r, a.Tq - 1);
    jmax[u] = r < a.Tq ? min(kc1, visible(r)) : 0;   // the query stores keys below it
    s_w[wave * kBlkQPW + u][lane] = (r < a.Tq && lane < a.HI) ? a.w_idx[qrow[u] * a.HI + lane] : 0.f;
  }

  // A operands: head hb*32 + (lane & 31), dims 16s + 8(lane >> 5) .. +8
  bf16x8 qa[kBlkQPW][2][KS];
#pragma unroll
  for (int u = 0; u < kBlkQPW; ++u) {
    const uint16_t* qp = a.q_idx + qrow[u] * a.HI * DI;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = hb * 32 + (lane & 31);
      const bool hv = r0 + u < a.Tq && h < a.HI;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qp + (int64_t)min(h, a.HI - 1) * DI + 16 * s +
                                                  8 * (lane >> 5));
        if (!hv) v = u32x4{0u, 0u, 0u, 0u};
        qa[u][hb][s] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // tile copy: copy i of wave w moves slots 64(CPW w + i) + lane, i.e. row
  // (64(CPW w + i) + lane) / 16, physical chunk lane % 16 <- logical chunk
  // (lane % 16) ^ (row & 15)
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx + (int64_t)b * a.Ncap * DI);
  auto issue = [&](int tile, uint8_t* T) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int win = CPW * wave + i;
      const int row = 4 * win + (lane >> 4);   // 64 slots of 16 bytes = 4 rows per copy
      int64_t j = kc0 + (int64_t)tile * KEYS + row;
      j = j < kc1 ? j : kc1 - 1;   // past the range: re-read a valid key (score not stored)
      const int lc = (lane & 15) ^ (row & 15);
      idx_copy_to_lds16(kbase + j * RB + 16 * lc, (V4_LDS void*)(T + 1024 * win));
    }
  };

  constexpr int NKB = KEYS / 32;
  auto compute = [&](int tile, const uint8_t* T, float* scv) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 acc[kBlkQPW][2];
#pragma unroll
      for (int u = 0; u < kBlkQPW; ++u)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[u][hb][i] = 0.f;
      const int row = kb * 32 + (lane & 31);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int lc = 2 * s + (lane >> 5);
        const bf16x8 kv = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(T + row * RB + 16 * (lc ^ (row & 15))));
#pragma unroll
        for (int u = 0; u < kBlkQPW; ++u)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
            acc[u][hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[u][hb][s], kv, acc[u][hb], 0, 0, 0);
      }
      // lane holds key (lane & 31), heads hb*32 + (i/4)*8 + (lane>>5)*4 + i%4
      const int64_t j = kc0 + (int64_t)tile * KEYS + kb * 32 + (lane & 31);
#pragma unroll
      for (int u = 0; u < kBlkQPW; ++u) {
        float sc = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(
                &s_w[wave * kBlkQPW + u][hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu(acc[u][hb][4 * i4 + i]), sc);
          }
        sc += __shfl_xor(sc, 32);
        scv[kb] = sc;
      }
    }
  };
  auto flush = [&](int tile, const float* scv) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int64_t j = kc0 + (int64_t)tile * KEYS + kb * 32 + (lane & 31);
      if (lane < 32 && j < jmax[0]) a.scores[qrow[0] * a.score_stride + j] = scv[kb];
    }
  };

  // Tile t lives in buffer t % NBUF.  A step first stores the previous
  // tile's scores (held in registers, so that the store latency overlaps a
  // whole step and the copies issued after them are the newest memory
  // operations), issues tile t + NBUF - 1, uses tile t, then waits for its own
  // copies of tile t+1 (later tiles may stay in flight) and meets the other
  // waves at the barrier.
  for (int p = 0; p < NBUF - 1 && p < ntiles; ++p) issue(p, s_k[p]);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float scv[NKB];
  for (int tile = 0; tile < ntiles; ++tile) {
    if (tile > 0 && wok) flush(tile - 1, scv);
    const bool pre = tile + NBUF - 1 < ntiles;
    if (pre) issue(tile + NBUF - 1, s_k[(tile + NBUF - 1) % NBUF]);
    if (wok) compute(tile, s_k[tile % NBUF], scv);
    if (pre)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(CPW * (NBUF - 2)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (ntiles > 0 && wok) flush(ntiles - 1, scv);
}

#ifndef V4_ROW_WAVES
#define V4_ROW_WAVES (256 * 12)   // 256 CUs x 12 waves (three workgroups)
#endif
int64_t index_row_waves(int B, int Tq, int64_t vmax) {
  const int64_t rows = (int64_t)B * Tq;
  const int64_t nch = (vmax + 31) / 32;
  int64_t per_row = (V4_ROW_WAVES + rows - 1) / rows;
  const int64_t cpw = (nch + per_row - 1) / per_row; // chunks per wave, then as few waves as that needs
  per_row = (nch + cpw - 1) / cpw;
  return (per_row + 3) / 4 * 4;
}

hipError_t launch_index_score(const IndexScoreArgs& a, hipStream_t st) {
  if (a.vmax <= 0 || a.B == 0 || a.Tq == 0) return hipSuccess;
  if (a.Tq >= kBlkQ && a.dI == 128 && a.HI <= 64) {
    const int64_t groups = (int64_t)a.B * ((a.Tq + kBlkQ - 1) / kBlkQ);
    int64_t splits = (512 + groups - 1) / groups;          // about two workgroups per CU
    int64_t chunk = (a.vmax + splits - 1) / splits;
    chunk = (chunk + kBlkKeys - 1) / kBlkKeys * kBlkKeys;
    if (chunk < kBlkKeys) chunk = kBlkKeys;
    splits = (a.vmax + chunk - 1) / chunk;
    dim3 grid((unsigned)splits, (unsigned)((a.Tq + kBlkQ - 1) / kBlkQ), (unsigned)a.B);
    index_score_block_kernel<<<grid, kBlkWaves * 64, 0, st>>>(a, chunk);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(a.row_waves / 4), a.Tq, a.B);
  if (a.ragged && a.Tq == 1) grid = dim3((unsigned)a.wg_start[a.B], 1, 1);
  const int mb = (a.HI + 15) / 16;
#define V4_IDX(DI, MB) index_score_kernel<DI, MB><<<grid, 256, 0, st>>>(a)
#define V4_IDX_MB(DI)          \
  switch (mb) {                \
    case 1: V4_IDX(DI, 1); break; \
    case 2: V4_IDX(DI, 2); break; \
    case 3: V4_IDX(DI, 3); break; \
    default: V4_IDX(DI, 4); break; \
  }
  switch (a.dI) {
    case 32: V4_IDX_MB(32); break;
    case 64: V4_IDX_MB(64); break;
    default: V4_IDX_MB(128); break;
  }
#undef V4_IDX_MB
#undef V4_IDX
  return hipGetLastError();
}

}  // namespace v4
