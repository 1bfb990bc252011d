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
// N.  Each wave streams one contiguous range of keys in 64-key chunks, two
// chunks deep, straight from HBM into MFMA operand registers: the MFMA
// contracts over dI, so dI may be permuted freely as long as q and k agree;
// each lane therefore owns one contiguous dI/4-element slice of a key row
// (64 contiguous bytes at dI = 128) instead of four scattered 16-byte pieces.
// The ReLU, the head weights and the head sum are applied to the fp32
// accumulators in registers (16 heads per lane, then two cross-lane adds), so
// only 4 bytes per entry leave the kernel.  At 1M tokens this kernel streams
// 64 MiB of keys per query and is HBM-bound (64 FLOP per byte).
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

template <int DI, int MB>
__global__ __launch_bounds__(256) void index_score_kernel(IndexScoreArgs a) {
  constexpr int KS = DI / 32;   // MFMA k-steps per key block
  constexpr int LPK = DI / 4;   // elements of a key row one lane owns
  const int b = blockIdx.z, r = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = a.q_pos0 + r;
  int64_t V = (t + 1) / a.m;
  if (V > a.n_entries) V = a.n_entries;
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;   // this wave's key range
  const int64_t jbeg = gw * a.keys_per_wave;
  if (jbeg >= V) return;
  const int64_t jend = min(jbeg + a.keys_per_wave, V);

  const int64_t qrow = (int64_t)b * a.Tq + r;
  // A operand: head mb*16 + c, dims g*LPK + ks*8 .. +8 (the shared permutation)
  bf16x8 qa[MB][KS];
  const uint16_t* qp = a.q_idx + qrow * a.HI * DI;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int h = min(mb * 16 + c, a.HI - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qp + (int64_t)h * DI + g * LPK + ks * 8);
      if (mb * 16 + c >= a.HI) v = u32x4{0u, 0u, 0u, 0u};
      qa[mb][ks] = __builtin_bit_cast(bf16x8, v);
    }
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

  const uint16_t* kp = a.k_idx + (int64_t)b * a.Ncap * DI + g * LPK;
  float* sp = a.scores + qrow * a.score_stride;

  // 64-key chunks (four 16-key blocks), two chunks in registers: the next
  // chunk's loads are in flight while the current one is contracted.  Keys
  // past the range re-read the last visible key (its score is not stored).
  auto load = [&](u32x4 (&kv)[4][KS], int64_t j0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t j = min(j0 + nb * 16 + c, V - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kv[nb][ks] = *reinterpret_cast<const u32x4*>(kp + j * DI + ks * 8);
    }
  };
  auto score = [&](const u32x4 (&kv)[4][KS], int64_t j0) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 acc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kb = __builtin_bit_cast(bf16x8, kv[nb][ks]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mb][ks], kb, acc[mb], 0, 0, 0);
      }
      // lane holds key column c, heads mb*16 + g*4 + i
      float s = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wv[mb][i], fmaxf(acc[mb][i], 0.f), s);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int64_t j = j0 + nb * 16 + c;
      if (g == 0 && j < jend) sp[j] = s;
    }
  };

  u32x4 ka[4][KS], kb[4][KS];
  load(ka, jbeg);
  for (int64_t j0 = jbeg; j0 < jend; j0 += 128) {
    load(kb, j0 + 64);
    score(ka, j0);
    if (j0 + 64 >= jend) break;
    load(ka, j0 + 128);
    score(kb, j0 + 64);
  }
}

int64_t index_keys_per_wave(int B, int Tq, int64_t vmax) {
  const int64_t total = (int64_t)B * Tq * vmax;
  const int64_t waves = 256 * 8;                 // 256 CUs x 8 waves
  int64_t kpw = (total + waves - 1) / waves;
  kpw = (kpw + 63) / 64 * 64;
  if (kpw < 64) kpw = 64;
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
