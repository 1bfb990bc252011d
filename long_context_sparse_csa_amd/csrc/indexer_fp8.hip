// FP8 lightning-indexer scores:
//   score_{t,j} = sum_h w_{t,h} * ReLU((sq_{t,h} q8_{t,h}) . (sk_j k8_j))
// with q8, k8 OCP E4M3 codes and positive fp32 scales sq (one per query
// head) and sk (one per key).
//
// Pages: the indexer is a few small heads run in FP8 ("DeepSeek-V4,
// explained", step 3 of how one query's layer works), and V4 runs the
// indexer's attention at reduced precision ("DeepSeek-V4: Making a Million
// Tokens Affordable", section "Two ways to shrink attention, interleaved").
// The form of the score is the one of the bf16 indexer; the scales are the
// plain reading of an FP8 tensor with one scale per row.
//
// Arithmetic: since sk_j > 0, ReLU(sk_j x) = sk_j ReLU(x), so
//   score_{t,j} = sk_j * sum_h (w_{t,h} sq_{t,h}) ReLU(q8_{t,h} . k8_j):
// the E4M3 dot products run on the f8f6f4 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales; every E4M3
// product is exact in fp32, the sum accumulates in fp32), w sq is one fp32
// product per head, and sk_j multiplies the head sum.
//
// Design (decode, few queries): as the bf16 decode kernel, at half the bytes
// per key.  q (all heads, E4M3) sits in registers as the MFMA's A operands
// (32 heads x 64 dims per operand), the folded weights w sq in LDS.  A row's
// keys are cut into 64-key chunks (8 KiB, the bytes per wave in flight of the
// bf16 kernel; 32-key chunks measured 1% slower, 128-key ones 15%) dealt
// round-robin over the row's waves; a chunk is read with non-temporal loads,
// 1 KiB of contiguous keys per instruction, with its key scales, staged in
// the wave's padded LDS rows and read back as the B operand of two 32-key
// blocks while the next chunk is in flight.
//
// Design (prefill, a block of queries of one sequence): eight waves, one
// query each (q in registers), share 128-key tiles (16 KiB) copied straight
// to LDS with global_load_lds, two tiles in turn, 16-byte chunks XOR-swizzled
// by row so the operand reads are free of bank conflicts.  MFMA-bound: four
// 32x32x64 MFMAs per 32 keys and query.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

namespace {

// max(x, 0) as one integer max on the bits (a negative float is a negative int)
__device__ __forceinline__ float relu8(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ f32x16 mfma_e4m3(const i32x8& a, const i32x8& b, const f32x16& c) {
  // formats 0/0: E4M3 x E4M3; E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& lo, const u32x4& hi) {
  return __builtin_bit_cast(i32x8, u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
}

// A operands of one query: head hb*32 + lane%32, bytes 64 ks + 32 (lane/32) .. +32
template <int DI>
__device__ __forceinline__ void load_q8(const IndexScoreFp8Args& a, int64_t qrow, bool ok, int lane,
                                        i32x8 (&qa)[2][DI / 64]) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = hb * 32 + (lane & 31);
    const bool hv = ok && h < a.HI;
    const uint8_t* qp = a.q8 + (qrow * a.HI + min(h, a.HI - 1)) * DI + 32 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < DI / 64; ++ks) {
      u32x4 lo = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
      u32x4 hi = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
      if (!hv) lo = hi = u32x4{0u, 0u, 0u, 0u};
      qa[hb][ks] = cat8(lo, hi);
    }
  }
}

}  // namespace

template <int DI, int CK>
__global__ __launch_bounds__(256) void index_score_fp8_kernel(IndexScoreFp8Args a) {
  constexpr int KS = DI / 64;        // 32x32x64 k-steps
  constexpr int RB = DI;             // key row bytes
  constexpr int P = RB / 16;         // 16-byte pieces per key
  constexpr int KPI = 64 / P;        // keys per load instruction
  constexpr int NL = CK / KPI;       // load instructions per CK-key chunk
  constexpr int NB = CK / 32;        // 32-key MFMA blocks per chunk
  constexpr int KSTR = RB + 16;      // padded LDS row: the operand reads hit distinct banks
  const int b = blockIdx.z, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = a.q_pos0 + r;
  int64_t V = (t + 1) / a.m;
  if (V > a.n_entries) V = a.n_entries;
  const int64_t nch = (V + CK - 1) / CK;
  const int64_t NW = (int64_t)gridDim.x * 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if ((int64_t)blockIdx.x * 4 >= nch) return;   // the whole block is past the visible keys

  __shared__ __attribute__((aligned(16))) uint8_t s_k[4][CK * KSTR];
  __shared__ __attribute__((aligned(16))) float s_w[64];

  const uint8_t* kbase = a.k8 + (int64_t)b * a.Ncap * DI;
  const float* sbase = a.k_scale + (int64_t)b * a.Ncap;
  u32x4 kv[NL];
  float ks_n[NB];   // scales of keys 32 nb + lane % 32 of the chunk in flight
  auto load = [&](int64_t j0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t j = min(j0 + i * KPI + lane / P, V - 1);
      kv[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + j * RB + 16 * (lane % P)));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ks_n[nb] = sbase[min(j0 + 32 * nb + (lane & 31), V - 1)];
  };
  if (gw < nch) load(gw * CK);   // in flight while q and the weights load

  const int64_t qrow = (int64_t)b * a.Tq + r;
  i32x8 qa[2][KS];
  load_q8<DI>(a, qrow, true, lane, qa);
  if (tid < 64) s_w[tid] = tid < a.HI ? a.w_idx[qrow * a.HI + tid] * a.q_scale[qrow * a.HI + tid] : 0.f;
  __syncthreads();
  if (gw >= nch) return;

  float* sp = a.scores + qrow * a.score_stride;
  uint8_t* kst = s_k[wave];
  for (int64_t ch = gw; ch < nch; ch += NW) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *reinterpret_cast<u32x4*>(kst + (i * KPI + lane / P) * KSTR + 16 * (lane % P)) = kv[i];
    float ksc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ksc[nb] = ks_n[nb];
    if (ch + NW < nch) load((ch + NW) * CK);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x16 acc[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint8_t* kp = kst + (32 * nb + (lane & 31)) * KSTR + 64 * ks + 32 * (lane >> 5);
        const i32x8 kb = cat8(*reinterpret_cast<const u32x4*>(kp), *reinterpret_cast<const u32x4*>(kp + 16));
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[hb] = mfma_e4m3(qa[hb][ks], kb, acc[hb]);
      }
      // lane holds key 32 nb + lane % 32, heads hb*32 + (i/4)*8 + (lane/32)*4 + i%4
      float sc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_w[hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu8(acc[hb][4 * i4 + i]), sc);
        }
      sc += __shfl_xor(sc, 32);
      const int64_t j = ch * CK + 32 * nb + (lane & 31);
      if (lane < 32 && j < V) sp[j] = ksc[nb] * sc;
    }
  }
}

#ifndef V4_F8_CHUNK
#define V4_F8_CHUNK 64
#endif
constexpr int kF8Chunk = V4_F8_CHUNK;   // keys per decode chunk (a multiple of 32)
constexpr int kF8Waves = 8;      // waves (queries) per workgroup
constexpr int kF8Keys = 128;     // keys per LDS tile

__device__ __forceinline__ void f8_copy_to_lds16(const void* src, V4_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

__global__ __launch_bounds__(kF8Waves * 64) void index_score_fp8_block_kernel(IndexScoreFp8Args a,
                                                                              int64_t key_chunk) {
  constexpr int DI = 128;
  constexpr int KS = DI / 64;
  constexpr int RB = DI;                       // key row bytes = 8 chunks of 16
  constexpr int TILE = kF8Keys * RB;           // 16 KiB
  constexpr int NKB = kF8Keys / 32;            // 32-key blocks per tile
  constexpr int CPW = TILE / 1024 / kF8Waves;  // 1 KiB copies per wave per tile
  constexpr int NBUF = 2;
  static_assert(CPW * 1024 * kF8Waves == TILE, "whole copies per wave");
  const int b = blockIdx.z, qg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = qg * kF8Waves + wave;          // this wave's query
  auto visible = [&](int rr) {
    const int64_t t = a.q_pos0 + rr;
    const int64_t v = (t + 1) / a.m;
    return v < a.n_entries ? v : a.n_entries;
  };
  const int64_t Vlast = visible(min(qg * kF8Waves + kF8Waves - 1, a.Tq - 1));
  const int64_t kc0 = (int64_t)blockIdx.x * key_chunk;
  const int64_t kc1 = min(kc0 + key_chunk, Vlast);
  if (kc0 >= kc1) return;
  const int ntiles = (int)((kc1 - kc0 + kF8Keys - 1) / kF8Keys);

  __shared__ __attribute__((aligned(16))) uint8_t s_k[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float s_w[kF8Waves][64];

  const bool wok = r < a.Tq;
  const int64_t qrow = (int64_t)b * a.Tq + min(r, a.Tq - 1);
  const int64_t jmax = wok ? min(kc1, visible(r)) : 0;   // the query stores keys below it
  s_w[wave][lane] = (wok && lane < a.HI) ? a.w_idx[qrow * a.HI + lane] * a.q_scale[qrow * a.HI + lane] : 0.f;
  i32x8 qa[2][KS];
  load_q8<DI>(a, qrow, wok, lane, qa);

  // 16-byte chunk c of tile row x sits at physical chunk c ^ ((x >> 1) & 7)
  const uint8_t* kbase = a.k8 + (int64_t)b * a.Ncap * DI;
  const float* sbase = a.k_scale + (int64_t)b * a.Ncap;
  float ksv[NKB], ksn[NKB];   // scales of keys kb*32 + lane%32 of the current / next tile
  auto issue = [&](int tile, uint8_t* T) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int win = CPW * wave + i;
      const int row = 8 * win + (lane >> 3);   // 64 slots of 16 bytes = 8 rows per copy
      int64_t j = kc0 + (int64_t)tile * kF8Keys + row;
      j = j < kc1 ? j : kc1 - 1;               // past the range: re-read a valid key
      const int lc = (lane & 7) ^ ((row >> 1) & 7);
      f8_copy_to_lds16(kbase + j * RB + 16 * lc, (V4_LDS void*)(T + 1024 * win));
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      int64_t j = kc0 + (int64_t)tile * kF8Keys + kb * 32 + (lane & 31);
      ksn[kb] = sbase[j < kc1 ? j : kc1 - 1];
    }
  };

  auto compute = [&](const uint8_t* T, float* scv) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 acc[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[hb][i] = 0.f;
      const int row = kb * 32 + (lane & 31);
      const int sw = (row >> 1) & 7;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = 4 * ks + 2 * (lane >> 5);
        const i32x8 kv = cat8(*reinterpret_cast<const u32x4*>(T + row * RB + 16 * (c0 ^ sw)),
                              *reinterpret_cast<const u32x4*>(T + row * RB + 16 * ((c0 + 1) ^ sw)));
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[hb] = mfma_e4m3(qa[hb][ks], kv, acc[hb]);
      }
      float sc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_w[wave][hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu8(acc[hb][4 * i4 + i]), sc);
        }
      sc += __shfl_xor(sc, 32);
      scv[kb] = ksv[kb] * sc;
    }
  };
  auto flush = [&](int tile, const float* scv) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int64_t j = kc0 + (int64_t)tile * kF8Keys + kb * 32 + (lane & 31);
      if (lane < 32 && j < jmax) a.scores[qrow * a.score_stride + j] = scv[kb];
    }
  };

  // Tile t lives in buffer t % 2.  A step stores the previous tile's scores
  // (so that the copies issued after them are the newest memory operations),
  // issues tile t+1, uses tile t, waits for its copies and meets the other
  // waves at the barrier.
  issue(0, s_k[0]);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float scv[NKB];
  for (int tile = 0; tile < ntiles; ++tile) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) ksv[kb] = ksn[kb];
    if (tile > 0 && wok) flush(tile - 1, scv);
    if (tile + 1 < ntiles) issue(tile + 1, s_k[(tile + 1) % NBUF]);
    if (wok) compute(s_k[tile % NBUF], scv);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (ntiles > 0 && wok) flush(ntiles - 1, scv);
}

int64_t index_fp8_row_waves(int B, int Tq, int64_t vmax) {
  const int64_t rows = (int64_t)B * Tq;
  const int64_t nch = (vmax + kF8Chunk - 1) / kF8Chunk;
  int64_t per_row = (256 * 12 + rows - 1) / rows;   // 256 CUs x 12 waves (three workgroups)
  const int64_t cpw = (nch + per_row - 1) / per_row;
  per_row = (nch + cpw - 1) / cpw;
  return (per_row + 3) / 4 * 4;
}

hipError_t launch_index_score_fp8(const IndexScoreFp8Args& a, hipStream_t st) {
  if (a.vmax <= 0 || a.B == 0 || a.Tq == 0) return hipSuccess;
  if (a.Tq >= kF8Waves && a.dI == 128) {
    const int64_t groups = (int64_t)a.B * ((a.Tq + kF8Waves - 1) / kF8Waves);
    int64_t splits = (512 + groups - 1) / groups;   // about two workgroups per CU
    int64_t chunk = (a.vmax + splits - 1) / splits;
    chunk = (chunk + kF8Keys - 1) / kF8Keys * kF8Keys;
    if (chunk < kF8Keys) chunk = kF8Keys;
    splits = (a.vmax + chunk - 1) / chunk;
    dim3 grid((unsigned)splits, (unsigned)((a.Tq + kF8Waves - 1) / kF8Waves), (unsigned)a.B);
    index_score_fp8_block_kernel<<<grid, kF8Waves * 64, 0, st>>>(a, chunk);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(a.row_waves / 4), a.Tq, a.B);
  if (a.dI == 64)
    index_score_fp8_kernel<64, kF8Chunk><<<grid, 256, 0, st>>>(a);
  else
    index_score_fp8_kernel<128, kF8Chunk><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace v4
