// The small kernels of the NSA-style variant: block scores from the
// compressed branch's logits, block -> token expansion, and the gated sum of
// the three branch outputs.  The branches themselves run on the attention
// kernel (attend.hip).
//
// Pages: in NSA the block scores come from attention over compressed block
// representations, the k best blocks are attended at full fidelity beside a
// sliding window of recent tokens, and learned gates mix the compressed,
// selected and window outputs ("DeepSeek-V4, explained", the numbered steps of
// how a compress-then-select layer handles one query: scoring, top-k, combining
// branches).
//
// Readings: selection block j is the m tokens [j m, (j+1) m) that compressed
// entry j summarises; its score is the compressed branch's attention
// probability of entry j summed over the heads (one shared KV); no sink in any
// branch.

#include "kernels.hpp"

namespace v4 {

namespace {

constexpr float kLog2eN = 1.4426950408889634f;

// score[q, j] = sum_h 2^(l2[q, h, j] - lse[q, h] log2 e) for j < V_t.  One
// thread per entry; the head loop reads one coalesced row of logits per head.
__global__ __launch_bounds__(256) void nsa_block_score_kernel(NsaBlockScoreArgs a) {
  __shared__ float s_lse2[64];
  const int q = blockIdx.y;
  const int64_t t = a.q_pos0 + q % a.Tq;
  int64_t v = (t + 1) / a.m;
  if (v > a.n_entries) v = a.n_entries;
  if (threadIdx.x < a.H) s_lse2[threadIdx.x] = a.lse[(int64_t)q * a.H + threadIdx.x] * kLog2eN;
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= v) return;
  const float* lp = a.logits2 + (int64_t)q * a.H * a.logits_stride + j;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  int h = 0;
  for (; h + 4 <= a.H; h += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      s[u] += exp2f(lp[(int64_t)(h + u) * a.logits_stride] - s_lse2[h + u]);
  }
  for (; h < a.H; ++h) s[0] += exp2f(lp[(int64_t)h * a.logits_stride] - s_lse2[h]);
  a.score[(int64_t)q * a.score_stride + j] = (s[0] + s[1]) + (s[2] + s[3]);
}

// tok[q, i m + u] = blk[q, i] m + u, or -1 where the block slot is empty.
__global__ __launch_bounds__(256) void nsa_expand_kernel(NsaExpandArgs a) {
  const int q = blockIdx.y;
  const int n = a.n_sel * a.m;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const int i = x / a.m, u = x - i * a.m;
  const int32_t blk = a.blocks[(int64_t)q * a.n_sel + i];
  a.tok[(int64_t)q * n + x] = blk >= 0 ? blk * a.m + u : -1;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack2(float x, float y) {
  // round to nearest even (finite inputs)
  auto rn = [](float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  };
  return rn(x) | (rn(y) << 16);
}

// out = g0 o_cmp + g1 o_slc + g2 o_win in fp32, stored as bf16.  One thread
// per 8 dims of one (query, head).
__global__ __launch_bounds__(256) void nsa_combine_kernel(NsaCombineArgs a) {
  const int64_t n8 = (int64_t)a.rows * a.D / 8;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n8) return;
  const int64_t qh = x / (a.D / 8);
  const float g0 = a.gates[3 * qh], g1 = a.gates[3 * qh + 1], g2 = a.gates[3 * qh + 2];
  const uint4 u0 = reinterpret_cast<const uint4*>(a.o_cmp)[x];
  const uint4 u1 = reinterpret_cast<const uint4*>(a.o_slc)[x];
  const uint4 u2 = reinterpret_cast<const uint4*>(a.o_win)[x];
  const uint32_t w0[4] = {u0.x, u0.y, u0.z, u0.w};
  const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w};
  const uint32_t w2[4] = {u2.x, u2.y, u2.z, u2.w};
  uint32_t r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float lo = fmaf(g2, bf16_lo(w2[e]), fmaf(g1, bf16_lo(w1[e]), g0 * bf16_lo(w0[e])));
    const float hi = fmaf(g2, bf16_hi(w2[e]), fmaf(g1, bf16_hi(w1[e]), g0 * bf16_hi(w0[e])));
    r[e] = pack2(lo, hi);
  }
  reinterpret_cast<uint4*>(a.out)[x] = uint4{r[0], r[1], r[2], r[3]};
}

}  // namespace

hipError_t launch_nsa_block_score(const NsaBlockScoreArgs& a, hipStream_t st) {
  const int64_t q = (int64_t)a.B * a.Tq;
  if (q == 0 || a.vmax == 0) return hipSuccess;
  nsa_block_score_kernel<<<dim3((unsigned)((a.vmax + 255) / 256), (unsigned)q), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_nsa_expand(const NsaExpandArgs& a, hipStream_t st) {
  const int n = a.n_sel * a.m;
  if (a.rows == 0 || n == 0) return hipSuccess;
  nsa_expand_kernel<<<dim3((unsigned)((n + 255) / 256), (unsigned)a.rows), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_nsa_combine(const NsaCombineArgs& a, hipStream_t st) {
  const int64_t n8 = (int64_t)a.rows * a.D / 8;
  if (n8 == 0) return hipSuccess;
  nsa_combine_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace v4
