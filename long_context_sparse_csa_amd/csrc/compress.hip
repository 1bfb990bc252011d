// Sequence compression: overlapping 2m-window softmax pooling of raw latents
// into compressed entries, and per-token packing of window rows.
//
// Pages: "DeepSeek-V4: Making a Million Tokens Affordable", section "Two ways
// to shrink attention, interleaved" (per-token compression weights and
// positional biases over 2m source tokens, one entry per m tokens; RMSNorm on
// entries; RoPE on the last 64 dims), and "DeepSeek-V4 Explained: Compressed
// Sparse Attention and 1M Context at 10% KV", section "The attention stack,
// and why it is two mechanisms" (BF16 rotary dims, FP8 for the rest).
//
// Design: HBM-bound and tiny next to the attention reads (one entry per m
// decoded tokens), so latency matters more than bandwidth.  One 1024-thread
// workgroup per entry: the 2m weights are formed once per window in LDS, each
// of the 16 waves pools every 16th window row with every lane owning D/64
// contiguous channels (coalesced 16-byte loads at D = 512, eight rows in
// flight per wave, so a 256-row window is two rounds of loads), the partial
// sums meet in LDS and wave 0 normalises, rotates and packs the 576-byte row.
// Each entry depends only on its own window, so streaming (one entry per
// call) and batch calls produce identical bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

template <int VPL>
__device__ __forceinline__ void load_bf16_row(const uint16_t* p, float (&x)[VPL]) {
  if constexpr (VPL == 8) {
    u32x4 w = *reinterpret_cast<const u32x4*>(p);
    unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(ws[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(ws[i] >> 16);
    }
  } else if constexpr (VPL == 4) {
    u32x2 w = *reinterpret_cast<const u32x2*>(p);
    x[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
    x[1] = bf16_bits_to_f32(w.x >> 16);
    x[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
    x[3] = bf16_bits_to_f32(w.y >> 16);
  } else {
    unsigned w = *reinterpret_cast<const unsigned*>(p);
    x[0] = bf16_bits_to_f32(w & 0xFFFFu);
    x[1] = bf16_bits_to_f32(w >> 16);
  }
}

// y holds this lane's VPL channels (lane*VPL ..) of an RMSNorm'd row.  Rotate
// the channels that fall in the last R dims by position `pos` and store the
// packed row: E4M3 for channels < D-R, bf16 for the rest.
template <int VPL>
__device__ __forceinline__ void rotate_and_pack(uint8_t* row, float (&y)[VPL], int lane, int R,
                                                int64_t pos, const RopeTurns& rope) {
  constexpr int D = VPL * 64;
  const int d0 = lane * VPL;
  if (d0 >= D - R) {
#pragma unroll
    for (int v = 0; v < VPL; v += 2) {
      float c, s;
      rope_cos_sin(pos, rope.t[(d0 + v - (D - R)) >> 1], &c, &s);
      float a = y[v], b = y[v + 1];
      y[v] = a * c - b * s;
      y[v + 1] = a * s + b * c;
    }
    uint8_t* dst = row + (D - R) + 2 * (d0 - (D - R));
    if constexpr (VPL == 8) {
      u32x4 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                 pack_bf16x2(y[6], y[7])};
      *reinterpret_cast<u32x4*>(dst) = w;
    } else if constexpr (VPL == 4) {
      u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      *reinterpret_cast<u32x2*>(dst) = w;
    } else {
      *reinterpret_cast<unsigned*>(dst) = pack_bf16x2(y[0], y[1]);
    }
  } else {
    uint8_t* dst = row + d0;
    if constexpr (VPL == 8) {
      u32x2 w = {pack_fp8x2(y[0], y[1]) | (pack_fp8x2(y[2], y[3]) << 16),
                 pack_fp8x2(y[4], y[5]) | (pack_fp8x2(y[6], y[7]) << 16)};
      *reinterpret_cast<u32x2*>(dst) = w;
    } else if constexpr (VPL == 4) {
      *reinterpret_cast<unsigned*>(dst) = pack_fp8x2(y[0], y[1]) | (pack_fp8x2(y[2], y[3]) << 16);
    } else {
      *reinterpret_cast<unsigned short*>(dst) = (unsigned short)pack_fp8x2(y[0], y[1]);
    }
  }
}

// RMSNorm of a row held as VPL channels per lane across one wave.
template <int VPL>
__device__ __forceinline__ void rmsnorm_wave(float (&y)[VPL], const float* __restrict__ gamma,
                                             int lane, float eps) {
  constexpr int D = VPL * 64;
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) ss += y[v] * y[v];
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int v = 0; v < VPL; ++v) y[v] = gamma[lane * VPL + v] * (y[v] * rs);
}

constexpr int kPoolThreads = 1024;   // sixteen waves pool one entry's window
constexpr int kPoolWaves = kPoolThreads / 64;

// Entry j of sequence b, written to `row`: the whole 1024-thread workgroup.
template <int VPL>
__device__ __forceinline__ void pool_entry(
    const uint16_t* __restrict__ raw, const float* __restrict__ score,
    const float* __restrict__ bias, const float* __restrict__ gamma, int L, int R,
    int64_t raw_pos0, int m, int64_t j, int b, float eps, const RopeTurns& rope,
    uint8_t* __restrict__ row,
    const uint16_t* __restrict__ raw_idx, int dI, uint16_t* __restrict__ kidx_row) {
  constexpr int D = VPL * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float s_alpha[512];
  __shared__ float s_part[kPoolWaves][D];
  __shared__ float s_red[2][kPoolWaves];

  const int64_t wlo = (j - 1) * (int64_t)m;  // window start; may be negative
  const int64_t plo = wlo > 0 ? wlo : 0;       // first existing position
  const int nw = (int)((j + 1) * (int64_t)m - plo);
  const int64_t r0 = plo - raw_pos0;           // raw row of plo
  const float* srow = score + (int64_t)b * L + r0;

  // rows in batches of U per wave, all loads of a batch in flight together
  // (loads are unconditional -- rows past the window re-read the last row
  // with weight 0 -- so the compiler keeps the whole batch in flight); the
  // first batch is issued before the weights are formed
  constexpr int U = 64 / VPL;
  const uint16_t* base = raw + ((int64_t)b * L + r0) * D + lane * VPL;
  float x[U][VPL];
  auto load_batch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + kPoolWaves * u, nw - 1);
      load_bf16_row<VPL>(base + (int64_t)t * D, x[u]);
    }
  };
  load_batch(wave);

  // weights alpha_t = softmax over the window of (s_t + b_{t - wlo})
  float mx = -INFINITY;
  for (int t = tid; t < nw; t += kPoolThreads) {
    const float lg = srow[t] + bias[plo - wlo + t];
    s_alpha[t] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = wave_max(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kPoolWaves; ++w) mx = fmaxf(mx, s_red[0][w]);
  float sum = 0.f;
  for (int t = tid; t < nw; t += kPoolThreads) {
    const float e = expf(s_alpha[t] - mx);
    s_alpha[t] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) s_red[1][wave] = sum;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kPoolWaves; ++w) tot += s_red[1][w];
  const float inv = 1.0f / tot;

  // pooled = sum_t alpha_t c_t : wave w takes rows w, w+16, ...
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.f;
  for (int t0 = wave;;) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + kPoolWaves * u;
      const float a = t < nw ? s_alpha[t] : 0.f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) acc[v] = fmaf(a, x[u][v], acc[v]);
    }
    t0 += kPoolWaves * U;
    if (t0 >= nw) break;
    load_batch(t0);
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) s_part[wave][lane * VPL + v] = acc[v];
  __syncthreads();
  if (kidx_row) {
    // the entry's indexer key: the token indexer keys pooled with the same
    // weights (no norm, no rotation), bf16; wave w takes rows w, w+16, ..
    __shared__ float s_kp[kPoolWaves][128];
    const uint16_t* kb = raw_idx + ((int64_t)b * L + r0) * dI;
    for (int d = lane; d < 128; d += 64) {
      float z = 0.f;
      if (d < dI)
        for (int t = wave; t < nw; t += kPoolWaves)
          z = fmaf(s_alpha[t], __uint_as_float((uint32_t)kb[(int64_t)t * dI + d] << 16), z);
      s_kp[wave][d] = z;
    }
    __syncthreads();
    if (tid < dI) {
      float z = 0.f;
#pragma unroll
      for (int w = 0; w < kPoolWaves; ++w) z += s_kp[w][tid];
      kidx_row[tid] = (uint16_t)(pack_bf16x2(z * inv, 0.f) & 0xFFFFu);
    }
  }
  if (wave != 0) return;

  float y[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int d = lane * VPL + v;
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < kPoolWaves; ++w) z += s_part[w][d];
    y[v] = z * inv;
  }
  rmsnorm_wave<VPL>(y, gamma, lane, eps);
  rotate_and_pack<VPL>(row, y, lane, R, j * (int64_t)m, rope);
}

template <int VPL>
__global__ __launch_bounds__(kPoolThreads) void compress_pool_kernel(
    const uint16_t* __restrict__ raw, const float* __restrict__ score,
    const float* __restrict__ bias, const float* __restrict__ gamma, int L, int R,
    int64_t raw_pos0, int m, int64_t entry0, float eps, const RopeTurns rope,
    uint8_t* __restrict__ out, int64_t out_rows, const uint16_t* __restrict__ raw_idx, int dI,
    uint16_t* __restrict__ kidx_out) {
  constexpr int D = VPL * 64;
  const int b = blockIdx.y;
  pool_entry<VPL>(raw, score, bias, gamma, L, R, raw_pos0, m, entry0 + blockIdx.x, b, eps, rope,
                  out + ((int64_t)b * out_rows + blockIdx.x) * (D + R), raw_idx, dI,
                  kidx_out ? kidx_out + ((int64_t)b * out_rows + blockIdx.x) * dI : nullptr);
}

// One wave per raw row: RMSNorm, RoPE at the row's own position, pack.
template <int VPL>
__global__ __launch_bounds__(256) void compress_pack_kernel(
    const uint16_t* __restrict__ raw, const float* __restrict__ gamma, int L, int R,
    int64_t raw_pos0, int n_out, float eps, const RopeTurns rope, uint8_t* __restrict__ out,
    int64_t out_rows) {
  constexpr int D = VPL * 64;
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_out) return;
  float y[VPL];
  load_bf16_row<VPL>(raw + ((int64_t)b * L + r) * D + lane * VPL, y);
  rmsnorm_wave<VPL>(y, gamma, lane, eps);
  uint8_t* row = out + ((int64_t)b * out_rows + r) * (D + R);
  rotate_and_pack<VPL>(row, y, lane, R, raw_pos0 + r, rope);
}

// One decode step of the compressor: block 0 of each sequence pools the entry
// the new token completes (if any), the last block packs the token's window
// row; both run side by side in one launch.
// One decode step of one or more layers' compressors (grid layer z runs
// layer z): block 0 of each sequence pools the entry its token completes
// (if any), the last block packs the token's window row.
template <int VPL>
__global__ __launch_bounds__(kPoolThreads) void compress_step_kernel(CompressStepBatch bt) {
  constexpr int D = VPL * 64;
  const CompressStepArgs& a = bt.s[blockIdx.z];
  const int b = blockIdx.y;
  if (b >= a.B) return;   // a layer with fewer sequences than the grid
  int64_t t = a.t, raw_pos0 = a.raw_pos0;
  if (a.ragged) {   // this sequence's token; its raw rows end at it
    t = a.pos.p[b];
    raw_pos0 = t - a.L + 1;
  }
  if (blockIdx.x == 0 && gridDim.x == 2 && (t + 1) % a.m != 0) return;   // no entry completes
  if (blockIdx.x == gridDim.x - 1) {
    if (threadIdx.x >= 64) return;
    const int lane = threadIdx.x;
    float y[VPL];
    load_bf16_row<VPL>(a.raw + ((int64_t)b * a.L + (t - raw_pos0)) * D + lane * VPL, y);
    rmsnorm_wave<VPL>(y, a.gamma, lane, a.eps);
    rotate_and_pack<VPL>(a.win + ((int64_t)b * a.win_rows + a.win_row) * (D + a.R), y, lane, a.R, t,
                         a.rope);
    return;
  }
  const int64_t j = (t + 1) / a.m - 1;
  pool_entry<VPL>(a.raw, a.tok_score, a.pos_bias, a.gamma, a.L, a.R, raw_pos0, a.m, j, b, a.eps,
                  a.rope, a.ent + ((int64_t)b * a.ent_rows + j) * (D + a.R), a.raw_idx, a.dI,
                  a.kidx ? a.kidx + ((int64_t)b * a.ent_rows + j) * a.dI : nullptr);
}

hipError_t launch_compress_steps(const CompressStepArgs* a, int n, hipStream_t st) {
  if (n < 1 || n > kMaxSteps) return hipErrorInvalidValue;
  CompressStepBatch bt{};
  bool pool = false;
  int maxB = 0;
  for (int z = 0; z < n; ++z) {
    if (a[z].D != a[0].D) return hipErrorInvalidValue;   // one kernel instance
    bt.s[z] = a[z];
    maxB = a[z].B > maxB ? a[z].B : maxB;
    if (a[z].ragged) {
      for (int b = 0; b < a[z].B; ++b) pool = pool || (a[z].pos.p[b] + 1) % a[z].m == 0;
    } else {
      pool = pool || (a[z].B > 0 && (a[z].t + 1) % a[z].m == 0);
    }
  }
  if (maxB == 0) return hipSuccess;
  dim3 grid(pool ? 2 : 1, maxB, n);
#define V4_STEP(VPL) compress_step_kernel<VPL><<<grid, kPoolThreads, 0, st>>>(bt)
  switch (a[0].D) {
    case 128: V4_STEP(2); break;
    case 256: V4_STEP(4); break;
    default: V4_STEP(8); break;
  }
#undef V4_STEP
  return hipGetLastError();
}

hipError_t launch_compress_step(const CompressStepArgs& a, hipStream_t st) {
  return launch_compress_steps(&a, 1, st);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
  if (a.n_out == 0 || a.B == 0) return hipSuccess;
  if (a.mode == 0) {
    dim3 grid(a.n_out, a.B);
#define V4_POOL(VPL)                                                                       \
  compress_pool_kernel<VPL><<<grid, kPoolThreads, 0, st>>>(a.raw, a.tok_score, a.pos_bias, a.gamma,  \
                                                  a.L, a.R, a.raw_pos0, a.m, a.entry0,     \
                                                  a.eps, a.rope, a.out, a.out_rows, a.raw_idx, \
                                                  a.dI, a.kidx)
    switch (a.D) {
      case 128: V4_POOL(2); break;
      case 256: V4_POOL(4); break;
      default: V4_POOL(8); break;
    }
#undef V4_POOL
  } else {
    dim3 grid((a.n_out + 3) / 4, a.B);
#define V4_PACK(VPL)                                                                     \
  compress_pack_kernel<VPL><<<grid, 256, 0, st>>>(a.raw, a.gamma, a.L, a.R, a.raw_pos0,   \
                                                  a.n_out, a.eps, a.rope, a.out,     \
                                                  a.out_rows)
    switch (a.D) {
      case 128: V4_PACK(2); break;
      case 256: V4_PACK(4); break;
      default: V4_PACK(8); break;
    }
#undef V4_PACK
  }
  return hipGetLastError();
}

}  // namespace v4
