// Lightning-indexer scores: score_{t,j} = sum_h w_{t,h} * ReLU(q_{t,h} . k_j).
//
// Pages: a lightning indexer scores each query against the compressed entries
// ("DeepSeek-V4: Making a Million Tokens Affordable", section "Two ways to
// shrink attention, interleaved"); it is a few small heads, cheap next to the
// main attention ("DeepSeek-V4, explained", step 3 of how one query's layer
// works).  One indexer key per entry is shared by all indexer heads.
//
// Design (decode): the dense contraction [HI heads x dI] x [dI x keys] runs on
// the bf16 matrix cores (v_mfma_f32_16x16x32_bf16) with the query's heads as
// the M dimension, loaded once per wave and held in registers, and the keys as
// N.  q (all heads of the query) sits in LDS and is read per MFMA, which
// keeps the registers small; each wave streams one contiguous range of keys
// in 32-key chunks with streaming (non-temporal) loads, every load
// instruction covering 1 KiB of contiguous keys (the pattern that measured
// fastest on this HBM), stages them in its own padded LDS rows and reads them
// back in the MFMA's operand layout; the other waves on the SIMD hide the
// latency.
// The ReLU, the head weights and the head sum are applied to the fp32
// accumulators in registers (16 heads per lane, then two cross-lane adds), so
// only 4 bytes per entry leave the kernel.  At 1M tokens this kernel streams
// 64 MiB of keys per query and is HBM-bound (64 FLOP per byte).
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

template <int DI, int MB>
__global__ __launch_bounds__(256) void index_score_kernel(IndexScoreArgs a) {
  constexpr int KS = DI / 32;        // MFMA k-steps per key block
  constexpr int QSTR = 2 * DI + 16;  // LDS bytes per q row (16-byte skew per head)
  const int b = blockIdx.z, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = a.q_pos0 + r;
  int64_t V = (t + 1) / a.m;
  if (V > a.n_entries) V = a.n_entries;
  const int64_t gw0 = (int64_t)blockIdx.x * 4;          // first wave range of the block
  if (gw0 * a.keys_per_wave >= V) return;              // whole block past the visible keys
  const int64_t gw = gw0 + wave;                        // this wave's key range
  const int64_t jbeg = gw * a.keys_per_wave;
  const int64_t jend = min(jbeg + a.keys_per_wave, V);

  // q of this query (all heads) in LDS: the A operand of every wave
  __shared__ __attribute__((aligned(16))) uint8_t s_q[MB * 16 * QSTR];
  constexpr int KSTR = 2 * DI + 16;  // LDS bytes per staged key row (16-byte skew)
  __shared__ __attribute__((aligned(16))) uint8_t s_k[4][32 * KSTR];
  const int64_t qrow = (int64_t)b * a.Tq + r;
  const uint16_t* qp = a.q_idx + qrow * a.HI * DI;
  for (int x = tid; x < MB * 16 * DI / 8; x += 256) {
    const int h = x / (DI / 8), d8 = x % (DI / 8);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < a.HI) v = *reinterpret_cast<const u32x4*>(qp + (int64_t)h * DI + d8 * 8);
    *reinterpret_cast<u32x4*>(s_q + h * QSTR + d8 * 16) = v;
  }
  // head weights for the accumulator rows this lane holds: mb*16 + g*4 + i
  float wv[MB][4];
  const float* wp = a.w_idx + qrow * a.HI;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = mb * 16 + g * 4 + i;
      const float x = wp[min(h, a.HI - 1)];
      wv[mb][i] = h < a.HI ? x : 0.f;
    }
  __syncthreads();
  if (jbeg >= V) return;

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(a.k_idx + (int64_t)b * a.Ncap * DI);
  float* sp = a.scores + qrow * a.score_stride;
  const int qa0 = c * QSTR + 16 * g;   // + mb*16*QSTR + 64*ks

  // 32-key chunks.  The chunk is read with fully contiguous loads (1 KiB
  // per instruction: lane l takes 16-byte piece l % P of key l / P of each
  // group of 64 / P keys), staged in this wave's LDS rows and read back in
  // the MFMA's operand layout (lane (g, c): dims ks*32 + g*8 of key c).
  // Keys past the range re-read the last visible key (score not stored).
  constexpr int NB = 2;                 // 16-key blocks per chunk
  constexpr int RB = 2 * DI;            // key row bytes
  constexpr int P = RB / 16;            // 16-byte pieces per key row
  constexpr int KPI = 64 / P;           // keys per load instruction
  constexpr int NL = 16 * NB / KPI;     // load instructions per chunk
  uint8_t* kst = s_k[wave];
  for (int64_t j0 = jbeg; j0 < jend; j0 += 16 * NB) {
    u32x4 kv[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int64_t j = min(j0 + i * KPI + lane / P, V - 1);
      kv[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + j * RB + 16 * (lane % P)));
    }
#pragma unroll
    for (int i = 0; i < NL; ++i)
      *reinterpret_cast<u32x4*>(kst + (i * KPI + lane / P) * KSTR + 16 * (lane % P)) = kv[i];
    // q is re-read from LDS for every block: an opaque offset keeps the
    // compiler from keeping it in registers across blocks
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int qo = qa0;
      asm volatile("" : "+v"(qo));
      const uint8_t* qa = s_q + qo;
      f32x4 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kb = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(kst + (nb * 16 + c) * KSTR + 64 * ks + 16 * g));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const bf16x8 q8 = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(qa + mb * 16 * QSTR + 64 * ks));
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q8, kb, acc[mb], 0, 0, 0);
        }
      }
      // lane holds key column c, heads mb*16 + g*4 + i
      float sc = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc = fmaf(wv[mb][i], fmaxf(acc[mb][i], 0.f), sc);
      sc += __shfl_xor(sc, 16);
      sc += __shfl_xor(sc, 32);
      const int64_t j = j0 + nb * 16 + c;
      if (g == 0 && j < jend) sp[j] = sc;
    }
  }
}

int64_t index_keys_per_wave(int B, int Tq, int64_t vmax) {
  const int64_t total = (int64_t)B * Tq * vmax;
  const int64_t waves = 256 * 12;                // 256 CUs x 12 waves (three workgroups)
  int64_t kpw = (total + waves - 1) / waves;
  kpw = (kpw + 31) / 32 * 32;
  if (kpw < 32) kpw = 32;
  if (kpw > 8192) kpw = 8192;
  return kpw;
}

hipError_t launch_index_score(const IndexScoreArgs& a, hipStream_t st) {
  if (a.vmax <= 0 || a.B == 0 || a.Tq == 0) return hipSuccess;
  dim3 grid((unsigned)((a.vmax + 4 * a.keys_per_wave - 1) / (4 * a.keys_per_wave)), a.Tq, a.B);
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
