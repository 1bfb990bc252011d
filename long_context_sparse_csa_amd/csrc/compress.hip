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
// A window row is one wave's work, with the row, gamma and the rotary turn
// all requested before any is used.  Each entry depends only on its own
// window, so streaming (one entry per call) and batch calls produce
// identical bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

__device__ __forceinline__ float buf_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// A lane's VPL bf16 channels of a row as they are loaded (one 4, 8 or 16
// byte load), converted to fp32 when used.
template <int VPL> struct RawRow;
template <> struct RawRow<8> {
  using T = u32x4;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  }
  __device__ static void to_f32(const T& w, float (&x)[8]) {
    const unsigned ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_bits_to_f32(ws[i] & 0xFFFFu);
      x[2 * i + 1] = bf16_bits_to_f32(ws[i] >> 16);
    }
  }
};
template <> struct RawRow<4> {
  using T = u32x2;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return u32x2{v[0], v[1]};
  }
  __device__ static void to_f32(const T& w, float (&x)[4]) {
    x[0] = bf16_bits_to_f32(w.x & 0xFFFFu);
    x[1] = bf16_bits_to_f32(w.x >> 16);
    x[2] = bf16_bits_to_f32(w.y & 0xFFFFu);
    x[3] = bf16_bits_to_f32(w.y >> 16);
  }
};
template <> struct RawRow<2> {
  using T = unsigned;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ static void to_f32(const T& w, float (&x)[2]) {
    x[0] = bf16_bits_to_f32(w & 0xFFFFu);
    x[1] = bf16_bits_to_f32(w >> 16);
  }
};

// (cos, sin) of the rotary pairs among this lane's VPL channels (lane*VPL ..)
// at position `pos` (lanes without rotary channels get (1, 0)).
template <int VPL>
__device__ __forceinline__ void lane_rope(int lane, int R, int64_t pos, const RopeTurns& rope,
                                          float (&cs)[VPL / 2], float (&sn)[VPL / 2]) {
  constexpr int D = VPL * 64;
  const int d0 = lane * VPL;
#pragma unroll
  for (int v = 0; v < VPL; v += 2) {
    cs[v / 2] = 1.f;
    sn[v / 2] = 0.f;
    if (d0 >= D - R) rope_cos_sin(pos, rope.t[(d0 + v - (D - R)) >> 1], &cs[v / 2], &sn[v / 2]);
  }
}

// y holds this lane's VPL channels (lane*VPL ..) of an RMSNorm'd row.  Rotate
// the channels that fall in the last R dims by the given (cos, sin) of their
// pairs and store the packed row: E4M3 for channels < D-R, bf16 for the rest.
template <int VPL>
__device__ __forceinline__ void rotate_and_pack_cs(uint8_t* row, float (&y)[VPL], int lane, int R,
                                                   const float (&cs)[VPL / 2],
                                                   const float (&sn)[VPL / 2]) {
  constexpr int D = VPL * 64;
  const int d0 = lane * VPL;
  if (d0 >= D - R) {
#pragma unroll
    for (int v = 0; v < VPL; v += 2) {
      const float c = cs[v / 2], s = sn[v / 2];
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

// One wave packs one window row: the raw bf16 row at src, RMSNorm'd with
// gamma, its last R channels rotated at position pos, stored at dst.  The
// row, gamma and the rotary turns are all requested before any is used.
template <int VPL>
__device__ __forceinline__ void pack_row_wave(const uint16_t* src, const float* gamma,
                                              uint8_t* dst, int64_t pos, const RopeTurns& rope,
                                              int R, float eps, int lane) {
  constexpr int D = VPL * 64;
  using Raw = typename RawRow<VPL>::T;
  const double tv = rope.t[lane & 31];   // pair lane mod 32's turns per position
  const Raw w = RawRow<VPL>::load(buf_rsrc(src, D * 2), lane * VPL * 2);
  const __amdgpu_buffer_rsrc_t rs_g = buf_rsrc(gamma, D * 4);
  float g[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) g[v] = buf_f32(rs_g, (lane * VPL + v) * 4);
  float y[VPL];
  RawRow<VPL>::to_f32(w, y);
  float ss = 0.f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) ss += y[v] * y[v];
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
  for (int v = 0; v < VPL; ++v) y[v] = g[v] * (y[v] * rs);
  // lane i < R/2 rotates pair i; the lanes holding the pair's channels fetch it
  float c0, s0;
  rope_cos_sin(pos, tv, &c0, &s0);
  float cs[VPL / 2], sn[VPL / 2];
#pragma unroll
  for (int v = 0; v < VPL; v += 2) {
    const int pr = (lane * VPL + v - (D - R)) >> 1;
    const float c = __shfl(c0, pr & 63), sv = __shfl(s0, pr & 63);
    cs[v / 2] = pr >= 0 ? c : 1.f;
    sn[v / 2] = pr >= 0 ? sv : 0.f;
  }
  rotate_and_pack_cs<VPL>(dst, y, lane, R, cs, sn);
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

  // Every load the entry needs goes out first, before any barrier: the rows
  // this wave pools (rows wave, wave + 16, .., as packed bf16, U at a time)
  // and the first of its token indexer keys; wave 0, which packs the row,
  // also works out the rotation of the entry's position.  The row loads are
  // unconditional (past the window they re-read the last row, weighted 0), so
  // the whole batch stays in flight.
  constexpr int U = VPL >= 8 ? 8 : 16;   // 32 registers of rows in flight
  using Raw = typename RawRow<VPL>::T;
  const uint16_t* base = raw + ((int64_t)b * L + r0) * D + lane * VPL;
  Raw x[U];
  auto load_batch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + kPoolWaves * u, nw - 1);
      x[u] = *reinterpret_cast<const Raw*>(base + (int64_t)t * D);
    }
  };
  load_batch(wave);
  const uint16_t* kb = kidx_row ? raw_idx + ((int64_t)b * L + r0) * dI : nullptr;
  uint16_t k0[2] = {0, 0};   // the key dims lane, lane + 64 of row `wave`
  if (kb && wave < nw) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (lane + 64 * h < dI) k0[h] = kb[(int64_t)wave * dI + lane + 64 * h];
  }
  __shared__ float s_rot[2][D / 2];   // (cos, sin) per channel pair, kept in LDS
  if (wave == 0) {
    float cs[VPL / 2], sn[VPL / 2];
    lane_rope<VPL>(lane, R, j * (int64_t)m, rope, cs, sn);
#pragma unroll
    for (int v = 0; v < VPL / 2; ++v) {
      s_rot[0][lane * (VPL / 2) + v] = cs[v];
      s_rot[1][lane * (VPL / 2) + v] = sn[v];
    }
  }

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
      float xf[VPL];
      RawRow<VPL>::to_f32(x[u], xf);
#pragma unroll
      for (int v = 0; v < VPL; ++v) acc[v] = fmaf(a, xf[v], acc[v]);
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
    for (int h = 0; h < 2; ++h) {
      const int d = lane + 64 * h;
      float z = 0.f;
      if (d < dI) {
        if (wave < nw) z = s_alpha[wave] * __uint_as_float((uint32_t)k0[h] << 16);
        for (int t = wave + kPoolWaves; t < nw; t += kPoolWaves)
          z = fmaf(s_alpha[t], __uint_as_float((uint32_t)kb[(int64_t)t * dI + d] << 16), z);
      }
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
  float cs[VPL / 2], sn[VPL / 2];
#pragma unroll
  for (int v = 0; v < VPL / 2; ++v) {
    cs[v] = s_rot[0][lane * (VPL / 2) + v];
    sn[v] = s_rot[1][lane * (VPL / 2) + v];
  }
  rotate_and_pack_cs<VPL>(row, y, lane, R, cs, sn);
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
  pack_row_wave<VPL>(raw + ((int64_t)b * L + r) * D, gamma,
                     out + ((int64_t)b * out_rows + r) * (D + R), raw_pos0 + r, rope, R, eps, lane);
}

// One decode step of one or more layers' compressors.  Workgroup (b, k, 0)
// pools the entry that sequence b's token completes in the k-th layer in
// launch order (if it completes one), workgroup (b, k, 1) packs the token's
// window row (wave 0; the grid is one deep when no token completes an entry).
// The host puts the layers with the longest windows first and the pooling
// workgroups go out before the window rows: they take the longest.
template <int VPL>
__global__ __launch_bounds__(kPoolThreads) void compress_step_kernel(CompressStepBatch bt) {
  constexpr int D = VPL * 64;
  const CompressStepArgs& a = bt.s[blockIdx.y];
  const int b = blockIdx.x;
  const bool win_block = blockIdx.z == gridDim.z - 1;
  // every argument read up front, before any branch, so the reads go out
  // together (each round trip to the argument segment costs a memory
  // latency; the empty asm keeps the compiler from sinking them into the
  // branches that use them)
  const int B = a.B, L = a.L, m = a.m, R = a.R, dI = a.dI;
  const bool ragged = a.ragged;
  const int64_t pb = a.pos.p[b & (kMaxRagged - 1)];
  const uint16_t* raw = a.raw;
  const float* tok_score = a.tok_score;
  const float* pos_bias = a.pos_bias;
  const uint16_t* raw_idx = a.raw_idx;
  uint16_t* kidx = a.kidx;
  uint8_t* win = a.win;
  uint8_t* ent = a.ent;
  const int64_t win_rows = a.win_rows, win_row = a.win_row, ent_rows = a.ent_rows;
  const float* gamma = a.gamma;
  const float eps = a.eps;
  int64_t t = a.t, raw_pos0 = a.raw_pos0;
  asm volatile("" ::"s"(raw), "s"(tok_score), "s"(pos_bias), "s"(raw_idx), "s"(kidx), "s"(win),
               "s"(ent), "s"(gamma), "s"(pb), "s"(t), "s"(raw_pos0), "s"(win_rows), "s"(win_row),
               "s"(ent_rows));
  asm volatile("" ::"s"(B), "s"(L), "s"(m), "s"(R), "s"(dI), "s"(eps), "s"((int)ragged));
  if (b >= B) return;   // a layer with fewer sequences than the grid
  if (ragged) {   // this sequence's token; its raw rows end at it (b < kMaxRagged)
    t = pb;
    raw_pos0 = t - L + 1;
  }
  if (win_block) {
    if (threadIdx.x >= 64) return;
    pack_row_wave<VPL>(raw + ((int64_t)b * L + (t - raw_pos0)) * D, gamma,
                       win + ((int64_t)b * win_rows + win_row) * (D + R), t, a.rope, R, eps,
                       threadIdx.x);
    return;
  }
  // t + 1 = (j + 1) m + r (positions below 2^31 take the 32-bit division)
  int64_t j1;
  int r;
  if ((uint64_t)(t + 1) < (1ull << 31)) {
    j1 = (uint32_t)(t + 1) / (uint32_t)m;
    r = (int)((uint32_t)(t + 1) - (uint32_t)j1 * (uint32_t)m);
  } else {
    j1 = (t + 1) / m;
    r = (int)((t + 1) - j1 * m);
  }
  if (r != 0) return;   // no entry completes
  const int64_t j = j1 - 1;
  pool_entry<VPL>(raw, tok_score, pos_bias, gamma, L, R, raw_pos0, m, j, b, eps, a.rope,
                  ent + ((int64_t)b * ent_rows + j) * (D + R), raw_idx, dI,
                  kidx ? kidx + ((int64_t)b * ent_rows + j) * dI : nullptr);
}

hipError_t launch_compress_steps(const CompressStepArgs* a, int n, hipStream_t st) {
  if (n < 1 || n > kMaxSteps) return hipErrorInvalidValue;
  int order[kMaxSteps];
  int maxB = 0;
  bool pool = false;
  for (int z = 0; z < n; ++z) {
    if (a[z].D != a[0].D) return hipErrorInvalidValue;   // one kernel instance
    order[z] = z;
    maxB = a[z].B > maxB ? a[z].B : maxB;
    if (a[z].ragged) {
      for (int b = 0; b < a[z].B; ++b) pool = pool || (a[z].pos.p[b] + 1) % a[z].m == 0;
    } else {
      pool = pool || (a[z].B > 0 && (a[z].t + 1) % a[z].m == 0);
    }
  }
  if (maxB == 0) return hipSuccess;
  // longest pooling windows first: they take the longest
  for (int i = 1; i < n; ++i)
    for (int k = i; k > 0 && a[order[k]].m > a[order[k - 1]].m; --k) {
      const int tmp = order[k];
      order[k] = order[k - 1];
      order[k - 1] = tmp;
    }
  CompressStepBatch bt{};
  for (int k = 0; k < n; ++k) bt.s[k] = a[order[k]];
  const dim3 grid((unsigned)maxB, (unsigned)n, pool ? 2u : 1u);
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
