// MXFP4 lightning-indexer scores:
//   score_{t,j} = sum_h w_{t,h} * ReLU(q_{t,h} . k_j)
// with q and k in the OCP MX FP4 format: E2M1 elements, one E8M0 scale per
// block of 32 consecutive dims, two elements per byte (the lower-indexed one
// in the low nibble).
//
// Pages: V4 runs the indexer's attention in FP4 ("DeepSeek-V4: Making a
// Million Tokens Affordable", section "Two ways to shrink attention,
// interleaved"); the form of the score is the one of the bf16 indexer.
//
// Arithmetic: the MX blocks are exactly what the f8f6f4 matrix cores take:
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in format 4 (E2M1)
// reads 32 elements (16 bytes) and one E8M0 scale per lane, lane l holding
// row l % 32 and the k range 32 (l / 32) .. +32 of the 64 -- one MX block
// per lane (probed on this chip).  So a key row goes into the MFMA as stored,
// with its block scales, and so does q.  The sum accumulates in fp32 (the
// matrix core's own summation), then ReLU, head weights and head sum in fp32.
//
// Design: the FP8 kernels at 68 B per key (d_I = 128: 64 bytes of codes and
// 4 scale bytes, one dword).  Decode: 128-key chunks (8 KiB, the bytes per
// wave in flight of the other decode kernels) dealt round-robin over the
// row's waves, 1 KiB of contiguous keys per load instruction, staged in
// padded LDS rows and read back as B operands; the chunk's scale dwords come
// with it.  Prefill: eight waves, one query each, 128-key tiles of 8 KiB by
// global_load_lds, two tiles in turn, 16-byte chunks XOR-swizzled by
// (row / 4) mod 4.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

namespace {

__device__ __forceinline__ float relu4(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// E2M1 x E2M1 (format 4) with per-lane E8M0 block scales
__device__ __forceinline__ f32x16 mfma_mxfp4(const i32x8& a, int sa, const i32x8& b, int sb,
                                             const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8 widen16(const u32x4& v) {
  return __builtin_bit_cast(i32x8, u32x8{v.x, v.y, v.z, v.w, 0u, 0u, 0u, 0u});
}

// Scale bytes of one key (d_I/32 of them) as one word
template <int DI>
__device__ __forceinline__ unsigned load_key_scales(const uint8_t* p) {
  if constexpr (DI == 128) return *reinterpret_cast<const unsigned*>(p);
  else return *reinterpret_cast<const unsigned short*>(p);
}

// A operands of one query: head hb*32 + lane%32, elements 64 ks + 32 (lane/32)
// .. +32 (16 bytes) and that block's scale byte
template <int DI>
__device__ __forceinline__ void load_q4(const IndexScoreMxfp4Args& a, int64_t qrow, bool ok,
                                        int lane, i32x8 (&qa)[2][DI / 64], int (&qs)[2][DI / 64]) {
  constexpr int RB = DI / 2, NBLK = DI / 32;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = hb * 32 + (lane & 31);
    const bool hv = ok && h < a.HI;
    const int64_t hr = qrow * a.HI + min(h, a.HI - 1);
#pragma unroll
    for (int ks = 0; ks < DI / 64; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(a.q4 + hr * RB + 32 * ks + 16 * (lane >> 5));
      if (!hv) v = u32x4{0u, 0u, 0u, 0u};
      qa[hb][ks] = widen16(v);
      qs[hb][ks] = a.q_sc[hr * NBLK + 2 * ks + (lane >> 5)];
    }
  }
}

}  // namespace

template <int DI>
__global__ __launch_bounds__(256) void index_score_mxfp4_kernel(IndexScoreMxfp4Args a) {
  constexpr int KS = DI / 64;        // 32x32x64 k-steps
  constexpr int RB = DI / 2;         // key row bytes
  constexpr int NBLK = DI / 32;      // scale bytes per key
  constexpr int P = RB / 16;         // 16-byte pieces per key
  constexpr int KPI = 64 / P;        // keys per load instruction
  constexpr int CK = 128;            // keys per chunk
  constexpr int NL = CK / KPI;       // load instructions per chunk
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

  const uint8_t* kbase = a.k4 + (int64_t)b * a.Ncap * RB;
  const uint8_t* sbase = a.k_sc + (int64_t)b * a.Ncap * NBLK;
  u32x4 kv[NL];
  unsigned ks_n[NB];   // scale bytes of keys 32 nb + lane % 32 of the chunk in flight
  auto load = [&](int64_t j0) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t j = min(j0 + i * KPI + lane / P, V - 1);
      kv[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + j * RB + 16 * (lane % P)));
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      ks_n[nb] = load_key_scales<DI>(sbase + min(j0 + 32 * nb + (lane & 31), V - 1) * NBLK);
  };
  if (gw < nch) load(gw * CK);   // in flight while q and the weights load

  const int64_t qrow = (int64_t)b * a.Tq + r;
  i32x8 qa[2][KS];
  int qs[2][KS];
  load_q4<DI>(a, qrow, true, lane, qa, qs);
  if (tid < 64) s_w[tid] = tid < a.HI ? a.w_idx[qrow * a.HI + tid] : 0.f;
  __syncthreads();
  if (gw >= nch) return;

  float* sp = a.scores + qrow * a.score_stride;
  uint8_t* kst = s_k[wave];
  for (int64_t ch = gw; ch < nch; ch += NW) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *reinterpret_cast<u32x4*>(kst + (i * KPI + lane / P) * KSTR + 16 * (lane % P)) = kv[i];
    unsigned ksc[NB];
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
        const i32x8 kb = widen16(*reinterpret_cast<const u32x4*>(
            kst + (32 * nb + (lane & 31)) * KSTR + 32 * ks + 16 * (lane >> 5)));
        const int sb = (ksc[nb] >> (8 * (2 * ks + (lane >> 5)))) & 0xFF;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[hb] = mfma_mxfp4(qa[hb][ks], qs[hb][ks], kb, sb, acc[hb]);
      }
      // lane holds key 32 nb + lane % 32, heads hb*32 + (i/4)*8 + (lane/32)*4 + i%4
      float sc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_w[hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu4(acc[hb][4 * i4 + i]), sc);
        }
      sc += __shfl_xor(sc, 32);
      const int64_t j = ch * CK + 32 * nb + (lane & 31);
      if (lane < 32 && j < V) sp[j] = sc;
    }
  }
}

constexpr int kF4Waves = 8;      // waves (queries) per workgroup
constexpr int kF4Keys = 128;     // keys per LDS tile

__device__ __forceinline__ void f4_copy_to_lds16(const void* src, V4_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

__global__ __launch_bounds__(kF4Waves * 64) void index_score_mxfp4_block_kernel(
    IndexScoreMxfp4Args a, int64_t key_chunk) {
  constexpr int DI = 128;
  constexpr int KS = DI / 64;
  constexpr int RB = DI / 2;                   // key row bytes = 4 chunks of 16
  constexpr int NBLK = DI / 32;
  constexpr int TILE = kF4Keys * RB;           // 8 KiB
  constexpr int NKB = kF4Keys / 32;            // 32-key blocks per tile
  constexpr int CPW = TILE / 1024 / kF4Waves;  // 1 KiB copies per wave per tile
  constexpr int NBUF = 2;
  static_assert(CPW * 1024 * kF4Waves == TILE, "whole copies per wave");
  const int b = blockIdx.z, qg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = qg * kF4Waves + wave;          // this wave's query
  auto visible = [&](int rr) {
    const int64_t t = a.q_pos0 + rr;
    const int64_t v = (t + 1) / a.m;
    return v < a.n_entries ? v : a.n_entries;
  };
  const int64_t Vlast = visible(min(qg * kF4Waves + kF4Waves - 1, a.Tq - 1));
  const int64_t kc0 = (int64_t)blockIdx.x * key_chunk;
  const int64_t kc1 = min(kc0 + key_chunk, Vlast);
  if (kc0 >= kc1) return;
  const int ntiles = (int)((kc1 - kc0 + kF4Keys - 1) / kF4Keys);

  __shared__ __attribute__((aligned(16))) uint8_t s_k[NBUF][TILE];
  __shared__ __attribute__((aligned(16))) float s_w[kF4Waves][64];

  const bool wok = r < a.Tq;
  const int64_t qrow = (int64_t)b * a.Tq + min(r, a.Tq - 1);
  const int64_t jmax = wok ? min(kc1, visible(r)) : 0;   // the query stores keys below it
  s_w[wave][lane] = (wok && lane < a.HI) ? a.w_idx[qrow * a.HI + lane] : 0.f;
  i32x8 qa[2][KS];
  int qs[2][KS];
  load_q4<DI>(a, qrow, wok, lane, qa, qs);

  // 16-byte chunk c of tile row x sits at physical chunk c ^ ((x >> 2) & 3)
  const uint8_t* kbase = a.k4 + (int64_t)b * a.Ncap * RB;
  const uint8_t* sbase = a.k_sc + (int64_t)b * a.Ncap * NBLK;
  unsigned ksv[NKB], ksn[NKB];   // scale words of keys kb*32 + lane%32, current / next tile
  auto issue = [&](int tile, uint8_t* T) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int win = CPW * wave + i;
      const int row = 16 * win + (lane >> 2);   // 64 slots of 16 bytes = 16 rows per copy
      int64_t j = kc0 + (int64_t)tile * kF4Keys + row;
      j = j < kc1 ? j : kc1 - 1;                // past the range: re-read a valid key
      const int lc = (lane & 3) ^ ((row >> 2) & 3);
      f4_copy_to_lds16(kbase + j * RB + 16 * lc, (V4_LDS void*)(T + 1024 * win));
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int64_t j = kc0 + (int64_t)tile * kF4Keys + kb * 32 + (lane & 31);
      ksn[kb] = load_key_scales<DI>(sbase + (j < kc1 ? j : kc1 - 1) * NBLK);
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
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = (2 * ks + (lane >> 5)) ^ ((row >> 2) & 3);
        const i32x8 kv = widen16(*reinterpret_cast<const u32x4*>(T + row * RB + 16 * c));
        const int sb = (ksv[kb] >> (8 * (2 * ks + (lane >> 5)))) & 0xFF;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) acc[hb] = mfma_mxfp4(qa[hb][ks], qs[hb][ks], kv, sb, acc[hb]);
      }
      float sc = 0.f;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 w4 = *reinterpret_cast<const f32x4*>(&s_w[wave][hb * 32 + i4 * 8 + (lane >> 5) * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc = fmaf(w4[i], relu4(acc[hb][4 * i4 + i]), sc);
        }
      sc += __shfl_xor(sc, 32);
      scv[kb] = sc;
    }
  };
  auto flush = [&](int tile, const float* scv) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int64_t j = kc0 + (int64_t)tile * kF4Keys + kb * 32 + (lane & 31);
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

int64_t index_mxfp4_row_waves(int B, int Tq, int64_t vmax) {
  const int64_t rows = (int64_t)B * Tq;
  const int64_t nch = (vmax + 127) / 128;
  int64_t per_row = (256 * 12 + rows - 1) / rows;   // 256 CUs x 12 waves (three workgroups)
  const int64_t cpw = (nch + per_row - 1) / per_row;
  per_row = (nch + cpw - 1) / cpw;
  return (per_row + 3) / 4 * 4;
}

hipError_t launch_index_score_mxfp4(const IndexScoreMxfp4Args& a, hipStream_t st) {
  if (a.vmax <= 0 || a.B == 0 || a.Tq == 0) return hipSuccess;
  if (a.Tq >= kF4Waves && a.dI == 128) {
    const int64_t groups = (int64_t)a.B * ((a.Tq + kF4Waves - 1) / kF4Waves);
    int64_t splits = (512 + groups - 1) / groups;   // about two workgroups per CU
    int64_t chunk = (a.vmax + splits - 1) / splits;
    chunk = (chunk + kF4Keys - 1) / kF4Keys * kF4Keys;
    if (chunk < kF4Keys) chunk = kF4Keys;
    splits = (a.vmax + chunk - 1) / chunk;
    dim3 grid((unsigned)splits, (unsigned)((a.Tq + kF4Waves - 1) / kF4Waves), (unsigned)a.B);
    index_score_mxfp4_block_kernel<<<grid, kF4Waves * 64, 0, st>>>(a, chunk);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(a.row_waves / 4), a.Tq, a.B);
  if (a.dI == 64)
    index_score_mxfp4_kernel<64><<<grid, 256, 0, st>>>(a);
  else
    index_score_mxfp4_kernel<128><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace v4
