// Block scores of the NSA-style variant from the compressed branch's logits.
// The branches themselves run on the attention kernel (attend.hip), which
// also expands the selected blocks into their tokens and forms the gated sum
// of the three branch outputs.
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

#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

namespace {

constexpr float kLog2eN = 1.4426950408889634f;

// score[q, j] = sum_h 2^(l2[q, j, h] - lse[q, h] log2 e) for j < V_t.  The
// heads of one row are 256 contiguous bytes: 16 lanes read them as float4s
// and add across lanes; a wave covers 16 rows, all its loads in flight
// together.
__global__ __launch_bounds__(256) void nsa_block_score_kernel(NsaBlockScoreArgs a) {
  const int q = blockIdx.y;
  const int64_t t = a.q_pos0 + q % a.Tq;
  int64_t v = (t + 1) / a.m;
  if (v > a.n_entries) v = a.n_entries;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane & 15, rsub = lane >> 4;   // heads 4 hq .. 4 hq + 3; row in a group of 4
  const int64_t j0 = (int64_t)blockIdx.x * 64 + wave * 16;
  if (j0 >= v) return;
  float l2s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * hq + e;
    l2s[e] = h < a.H ? a.lse[(int64_t)q * a.H + h] * kLog2eN : 0.f;
  }
  const float* lp = a.logits2 + (int64_t)q * a.logits_stride * 64 + 4 * hq;
  f32x4 x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = j0 + 4 * u + rsub;
    x[u] = j < v ? *reinterpret_cast<const f32x4*>(lp + j * 64) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * hq + e < a.H) s += exp2f(x[u][e] - l2s[e]);   // slots >= H hold no logit
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    const int64_t j = j0 + 4 * u + rsub;
    if (hq == 0 && j < v) a.score[(int64_t)q * a.score_stride + j] = s;
  }
}

}  // namespace

hipError_t launch_nsa_block_score(const NsaBlockScoreArgs& a, hipStream_t st) {
  const int64_t q = (int64_t)a.B * a.Tq;
  if (q == 0 || a.vmax == 0) return hipSuccess;
  nsa_block_score_kernel<<<dim3((unsigned)((a.vmax + 63) / 64), (unsigned)q), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace v4
