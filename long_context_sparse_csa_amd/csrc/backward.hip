// Backward of the core attention (CSA and HCA): gradients with respect to
// the raw queries, every attended row (entries and window rows), the sinks
// and gamma_q.
//
// Pages: the attention step is trained end to end except the hard top-k
// choice ("DeepSeek-V4, explained", step 7).  The forward is the one of
// attend.hip: q~ = RoPE_t(RMSNorm(q)), one softmax over the rows and the
// sink, out = RoPE_{-t}(sum p x).
//
// Design: per chunk of queries, every attended row is gathered once as bf16
// (the E4M3 and bf16 stored values are exact in bf16) into X [q, n, D]; the
// query side [q~; do] (do = RoPE_t(dout)) is Y [q, 128, D] (64 head slots
// each).  Then, per query, three batched bf16 matrix-core products
//     [S; dP]   = Y X^T                     (logits / scale, and do . x)
//     dq~       = (scale dL) X
//     dX        = [scale dL; P]^T Y        (key and value paths at once)
// with P = exp(scale S - lse) and dL = P (dP - D), D_h = dout_h . out_h, in
// between (an elementwise kernel).  dX rows are added into the caller's
// row gradients with atomics (a row may be attended by many queries); dq~
// goes back through RoPE_t and the RMSNorm.

#include "common.hpp"
#include "kernels.hpp"

namespace v4 {

namespace {

constexpr float kL2e = 1.4426950408889634f;
constexpr int kLdsK = 40;   // padded k stride of the staged tiles (bf16)

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {   // round to nearest even (finite)
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// C[z] = alpha A[z] B[z] on 64 x 64 tiles, K in steps of 32 (all multiples:
// the caller pads).  A is M x K (AT: stored K x M), B is K x N (BT: stored
// N x K); bf16 in, fp32 accumulate.  Four waves, 32 x 32 each.
template <bool AT, bool BT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[64][kLdsK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[64][kLdsK];
  const int z = blockIdx.z;
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const uint16_t* A = g.a + (int64_t)z * g.a_batch;
  const uint16_t* B = g.b + (int64_t)z * g.b_batch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, c = lane & 15, gq = lane >> 4;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // a tile [64 rows][32 k] from a row-major (rows x k) matrix, or from a
  // (k x rows) one, transposed on the way into LDS; the next k-tile's global
  // loads are in flight while the current one's MFMAs run
  auto fetch = [&](const uint16_t* p, int64_t ld, int r0, int k0, bool tr) -> uint4 {
    if (!tr) {
      const int r = tid >> 2, ch = tid & 3;
      return *reinterpret_cast<const uint4*>(p + (int64_t)(r0 + r) * ld + k0 + 8 * ch);
    }
    const int kk = tid >> 3, ch = tid & 7;
    return *reinterpret_cast<const uint4*>(p + (int64_t)(k0 + kk) * ld + r0 + 8 * ch);
  };
  auto put = [&](uint16_t (*s)[kLdsK], uint4 v, bool tr) {
    if (!tr) {
      const int r = tid >> 2, ch = tid & 3;
      *reinterpret_cast<uint4*>(&s[r][8 * ch]) = v;
    } else {
      const int kk = tid >> 3, ch = tid & 7;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[8 * ch + 2 * e][kk] = (uint16_t)(w[e] & 0xFFFFu);
        s[8 * ch + 2 * e + 1][kk] = (uint16_t)(w[e] >> 16);
      }
    }
  };
  uint4 ra = fetch(A, g.lda, m0, 0, AT), rb = fetch(B, g.ldb, n0, 0, !BT);
  for (int k0 = 0; k0 < g.K; k0 += 32) {
    put(sA, ra, AT);
    put(sB, rb, !BT);
    __syncthreads();
    if (k0 + 32 < g.K) {
      ra = fetch(A, g.lda, m0, k0 + 32, AT);
      rb = fetch(B, g.ldb, n0, k0 + 32, !BT);
    }
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(&sA[wm * 32 + 16 * i + c][8 * gq]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const bf16x8*>(&sB[wn * 32 + 16 * j + c][8 * gq]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    __syncthreads();
  }
  // lane (c, gq) holds rows 4 gq + v, column c of each 16 x 16 block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 32 + 16 * i + 4 * gq + v;
        const int n = n0 + wn * 32 + 16 * j + c;
        const float x = g.alpha * acc[i][j][v];
        if (n >= g.n_valid) continue;
        if (!g.rowmap) {
          g.c[(int64_t)z * g.c_batch + (int64_t)m * g.ldc + n] = x;
        } else {
          const int64_t r = g.rowmap[(int64_t)z * g.rowmap_batch + m];
          if (r >= 0) atomicAdd(g.c + r * g.ldc + n, x);
          else if (r <= -2) atomicAdd(g.c2 + (-2 - r) * g.ldc + n, x);
        }
      }
}

// X[qc, x, :] = the query's row x as bf16 (zeros if absent), rowmap = where
// its gradient goes: entry b Ncap + j (>= 0), window row -2 - (b (Tq+W-1) + r),
// or -1.  One wave per row slot.
__global__ __launch_bounds__(256) void bwd_gather_kernel(BwdArgs a, int q0) {
  const int qc = blockIdx.y, qr = q0 + qc;
  const int b = qr / a.Tq, r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int x = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (x >= a.np) return;
  int64_t n_ent;
  if (a.topk) {
    n_ent = a.k;
  } else {
    const int64_t v = (t + 1) / a.m;
    n_ent = v < a.n_entries ? v : a.n_entries;
  }
  const int64_t lo = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
  const int64_t n_win = a.W > 0 ? t - lo + 1 : 0;
  const int ROW = a.D + a.R;
  const uint8_t* src = nullptr;
  int64_t map = -1;
  if (x < n_ent) {
    const int64_t j = a.topk ? (int64_t)a.topk[(int64_t)qr * a.k + x] : (int64_t)x;
    if (j >= 0 && j < a.Ncap) {
      src = a.entries + ((int64_t)b * a.Ncap + j) * ROW;
      map = (int64_t)b * a.Ncap + j;
    }
  } else if (x < n_ent + n_win) {
    const int64_t wrow = lo + (x - n_ent) - (a.q_pos0 - (a.W - 1));
    const int64_t grow = (int64_t)b * (a.Tq + a.W - 1) + wrow;
    src = a.win + grow * ROW;
    map = -2 - grow;
  }
  uint16_t* dst = a.X + ((int64_t)qc * a.np + x) * a.D;
  const int E = a.D - a.R;
  const int d = 8 * lane;   // this lane's 8 dims (E and D are multiples of 8)
  if (d < a.D) {
    uint4 o = {0u, 0u, 0u, 0u};
    if (src) {
      if (d < E) {   // 8 E4M3 bytes -> 8 bf16 (exact)
        const uint2 b8 = *reinterpret_cast<const uint2*>(src + d);
        const uint32_t w2[2] = {b8.x, b8.y};
        uint32_t r[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w2[h], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w2[h], true);
          r[2 * h] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xFFFF0000u);
          r[2 * h + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xFFFF0000u);
        }
        o = uint4{r[0], r[1], r[2], r[3]};
      } else {       // bf16 dims as stored
        o = *reinterpret_cast<const uint4*>(src + E + 2 * (d - E));
      }
    }
    *reinterpret_cast<uint4*>(dst + d) = o;
  }
  if (lane == 0) a.rowmap[(int64_t)qc * a.np + x] = map;
}

// Y[qc] = [q~ (64 head slots); do = RoPE_t(dout) (64 slots)] as bf16, Dh =
// dout . out, dsink += -p_sink Dh.  One wave per head; lane holds the dim
// pairs (2 lane + 128 e, +1).
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a, int q0) {
  const int qc = blockIdx.y, qr = q0 + qc;
  const int r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint16_t* yq = a.Y + ((int64_t)qc * 128 + h) * a.D;
  uint16_t* yd = a.Y + ((int64_t)qc * 128 + 64 + h) * a.D;
  if (h >= a.H) {
    for (int d = lane; d < a.D; d += 64) yq[d] = yd[d] = 0;
    return;
  }
  const uint16_t* qp = a.q + ((int64_t)qr * a.H + h) * a.D;
  const uint16_t* gp = a.dout + ((int64_t)qr * a.H + h) * a.D;
  const uint16_t* op = a.out + ((int64_t)qr * a.H + h) * a.D;
  const int NP = a.D / 128;   // pairs per lane
  float ss = 0.f, dd = 0.f;
  for (int e = 0; e < NP; ++e) {
    const int d = 2 * lane + 128 * e;
    const float q0v = bf16f(qp[d]), q1v = bf16f(qp[d + 1]);
    ss += q0v * q0v + q1v * q1v;
    dd += bf16f(gp[d]) * bf16f(op[d]) + bf16f(gp[d + 1]) * bf16f(op[d + 1]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    ss += __shfl_xor(ss, o);
    dd += __shfl_xor(dd, o);
  }
  const float rsn = 1.0f / sqrtf(ss / (float)a.D + a.eps);
  for (int e = 0; e < NP; ++e) {
    const int d = 2 * lane + 128 * e;
    float x0 = a.gamma_q[d] * (bf16f(qp[d]) * rsn), x1 = a.gamma_q[d + 1] * (bf16f(qp[d + 1]) * rsn);
    float g0 = bf16f(gp[d]), g1 = bf16f(gp[d + 1]);
    if (d >= a.D - a.R) {
      float cs, sn;
      rope_cos_sin(t, a.rope.t[(d - (a.D - a.R)) >> 1], &cs, &sn);
      const float y0 = x0 * cs - x1 * sn, y1 = x0 * sn + x1 * cs;
      x0 = y0;
      x1 = y1;
      const float u0 = g0 * cs - g1 * sn, u1 = g0 * sn + g1 * cs;   // do = RoPE_t(dout)
      g0 = u0;
      g1 = u1;
    }
    yq[d] = f2bf(x0);
    yq[d + 1] = f2bf(x1);
    yd[d] = f2bf(g0);
    yd[d + 1] = f2bf(g1);
  }
  if (lane == 0) {
    a.Dh[(int64_t)qc * 64 + h] = dd;
    if (a.sink && a.d_sink) {
      const float lse = a.lse[(int64_t)qr * a.H + h];
      const float pz = lse == -INFINITY ? 0.f : expf(a.sink[h] - lse);
      atomicAdd(a.d_sink + h, -pz * dd);
    }
  }
}

// T[qc] = [scale dL; P] (bf16, 64 head slots each) from [S; dP]: P =
// exp(scale S - lse), dL = P (dP - Dh); absent rows and head slots >= H: 0.
// One thread per row slot, all heads; p_sel (entry slots) is the head sum.
__global__ __launch_bounds__(256) void bwd_softmax_kernel(BwdArgs a, int q0) {
  __shared__ float s_l2[64], s_dh[64];
  const int qc = blockIdx.y, qr = q0 + qc;
  if (threadIdx.x < 64) {
    const int h = threadIdx.x;
    const float lse = h < a.H ? a.lse[(int64_t)qr * a.H + h] : -INFINITY;
    s_l2[h] = lse * kL2e;
    s_dh[h] = a.Dh[(int64_t)qc * 64 + h];
  }
  __syncthreads();
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= a.np) return;
  const float* sp = a.SP + (int64_t)qc * 128 * a.np + x;
  uint16_t* tp = a.T + (int64_t)qc * 128 * a.np + x;
  const bool present = a.rowmap[(int64_t)qc * a.np + x] != -1;
  const float sl2 = a.scale * kL2e;
  float psum = 0.f;
  for (int h = 0; h < 64; ++h) {
    float p = 0.f, dl = 0.f;
    if (present && s_l2[h] != -INFINITY) {
      p = exp2f(sp[(int64_t)h * a.np] * sl2 - s_l2[h]);
      dl = p * (sp[(int64_t)(64 + h) * a.np] - s_dh[h]);
    }
    psum += p;
    tp[(int64_t)h * a.np] = f2bf(a.scale * dl);
    tp[(int64_t)(64 + h) * a.np] = f2bf(p);
  }
  if (a.p_sel && x < a.k_sel) a.p_sel[(int64_t)qr * a.k_sel + x] = psum;
}

// dq = RMSNorm backward of RoPE_t^T(dq~); d_gamma_q += sum over heads.  A
// workgroup takes four heads of one query (one a wave); lane holds dim pairs.
__global__ __launch_bounds__(256) void bwd_q_kernel(BwdArgs a, int q0) {
  __shared__ float s_dg[4][512];
  const int qc = blockIdx.y, qr = q0 + qc;
  const int r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NP = a.D / 128;
  float dg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dg[i] = 0.f;
  if (blockIdx.x * 4 >= a.H) return;
  for (int h = blockIdx.x * 4 + wave; h < a.H && h < blockIdx.x * 4 + 4; h += 4) {
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + h) * a.D;
    const float* gq = a.DQT + ((int64_t)qc * 64 + h) * a.D;
    float ss = 0.f;
    for (int e = 0; e < NP; ++e) {
      const int d = 2 * lane + 128 * e;
      ss += bf16f(qp[d]) * bf16f(qp[d]) + bf16f(qp[d + 1]) * bf16f(qp[d + 1]);
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float rsn = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    float gx[8], xq[8];
    float dot = 0.f;
    for (int e = 0; e < NP; ++e) {
      const int d = 2 * lane + 128 * e;
      float u0 = gq[d], u1 = gq[d + 1];
      if (d >= a.D - a.R) {   // RoPE_t transposed = rotation by -t
        float cs, sn;
        rope_cos_sin(t, a.rope.t[(d - (a.D - a.R)) >> 1], &cs, &sn);
        const float v0 = u0 * cs + u1 * sn, v1 = -u0 * sn + u1 * cs;
        u0 = v0;
        u1 = v1;
      }
      xq[2 * e] = bf16f(qp[d]);
      xq[2 * e + 1] = bf16f(qp[d + 1]);
      dg[2 * e] += u0 * xq[2 * e] * rsn;
      dg[2 * e + 1] += u1 * xq[2 * e + 1] * rsn;
      gx[2 * e] = u0 * a.gamma_q[d];
      gx[2 * e + 1] = u1 * a.gamma_q[d + 1];
      dot += gx[2 * e] * xq[2 * e] + gx[2 * e + 1] * xq[2 * e + 1];
    }
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    const float c3 = dot * rsn * rsn * rsn / (float)a.D;
    float* dqp = a.dq + ((int64_t)qr * a.H + h) * a.D;
    for (int e = 0; e < NP; ++e) {
      const int d = 2 * lane + 128 * e;
      dqp[d] = gx[2 * e] * rsn - xq[2 * e] * c3;
      dqp[d + 1] = gx[2 * e + 1] * rsn - xq[2 * e + 1] * c3;
    }
  }
  if (!a.d_gamma_q) return;
  for (int e = 0; e < NP; ++e) {
    const int d = 2 * lane + 128 * e;
    s_dg[wave][d] = dg[2 * e];
    s_dg[wave][d + 1] = dg[2 * e + 1];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < a.D; d += 256)
    atomicAdd(a.d_gamma_q + d, s_dg[0][d] + s_dg[1][d] + s_dg[2][d] + s_dg[3][d]);
}

// ---- compressor backward: one workgroup per (sequence, entry).  Recomputes
// the window weights alpha and the pooled vector, then
//   dy = RoPE_{jm}^T(de), RMSNorm backward -> dpooled and d gamma,
//   d c_t += alpha_t dpooled,  dalpha_t = c_t . dpooled,
//   dlogit_t = alpha_t (dalpha_t - sum alpha dalpha) -> d s_t and d b.
// Thread i owns the dim pair (2i, 2i+1); a token is in two windows, so the
// latent and score gradients are added with atomics.
__global__ __launch_bounds__(256) void compress_bwd_kernel(CompressBwdArgs a) {
  __shared__ float s_alpha[512];
  __shared__ float s_dp[512];
  __shared__ float s_red[8];
  __shared__ float s_da[512];
  const int b = blockIdx.y;
  const int64_t j = a.entry0 + blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.D, m = a.m;
  const int64_t wlo = (j - 1) * (int64_t)m;
  const int64_t plo = wlo > 0 ? wlo : 0;
  const int nw = (int)((j + 1) * (int64_t)m - plo);
  const int64_t r0 = plo - a.raw_pos0;
  auto block_sum = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    return s_red[0] + s_red[1] + s_red[2] + s_red[3];
  };
  auto block_max = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    __syncthreads();
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  };
  // window weights
  float mx = -INFINITY;
  for (int t = tid; t < nw; t += 256) {
    const float lg = a.tok_score[(int64_t)b * a.L + r0 + t] + a.pos_bias[plo - wlo + t];
    s_alpha[t] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = block_max(mx);
  float sum = 0.f;
  for (int t = tid; t < nw; t += 256) {
    const float e = expf(s_alpha[t] - mx);
    s_alpha[t] = e;
    sum += e;
  }
  sum = block_sum(sum);
  const float inv = 1.0f / sum;
  for (int t = tid; t < nw; t += 256) s_alpha[t] *= inv;
  __syncthreads();
  // pooled vector (this thread's pair)
  const bool own = 2 * tid < D;
  const int d = 2 * tid;
  const uint16_t* rb = a.raw + ((int64_t)b * a.L + r0) * D;
  float p0 = 0.f, p1 = 0.f;
  if (own)
    for (int t = 0; t < nw; ++t) {
      const uint32_t w2 = *reinterpret_cast<const uint32_t*>(rb + (int64_t)t * D + d);
      p0 += s_alpha[t] * bf16f((uint16_t)(w2 & 0xFFFFu));
      p1 += s_alpha[t] * bf16f((uint16_t)(w2 >> 16));
    }
  const float ms = block_sum(own ? p0 * p0 + p1 * p1 : 0.f) / (float)D;
  const float rsn = 1.0f / sqrtf(ms + a.eps);
  // dy = RoPE at j m, transposed
  float g0 = 0.f, g1 = 0.f;
  if (own) {
    g0 = a.de[((int64_t)b * a.n_out + blockIdx.x) * D + d];
    g1 = a.de[((int64_t)b * a.n_out + blockIdx.x) * D + d + 1];
    if (d >= D - a.R) {
      float cs, sn;
      rope_cos_sin(j * m, a.rope.t[(d - (D - a.R)) >> 1], &cs, &sn);
      const float u0 = g0 * cs + g1 * sn, u1 = -g0 * sn + g1 * cs;
      g0 = u0;
      g1 = u1;
    }
  }
  const float ga = own ? g0 * a.gamma[d] : 0.f, gb = own ? g1 * a.gamma[d + 1] : 0.f;
  const float dot = block_sum(ga * p0 + gb * p1);
  const float c3 = dot * rsn * rsn * rsn / (float)D;
  if (own) {
    s_dp[d] = ga * rsn - p0 * c3;
    s_dp[d + 1] = gb * rsn - p1 * c3;
    if (a.d_gamma) {
      atomicAdd(a.d_gamma + d, g0 * p0 * rsn);
      atomicAdd(a.d_gamma + d + 1, g1 * p1 * rsn);
    }
  }
  __syncthreads();
  // per token: latent gradient and dalpha (one wave per token)
  for (int t = wave; t < nw; t += 4) {
    const uint16_t* ct = rb + (int64_t)t * D;
    float* dct = a.d_raw + ((int64_t)b * a.L + r0 + t) * D;
    const float al = s_alpha[t];
    float da = 0.f;
    for (int e = lane; e < D; e += 64) {
      da += bf16f(ct[e]) * s_dp[e];
      atomicAdd(dct + e, al * s_dp[e]);
    }
    for (int o = 32; o > 0; o >>= 1) da += __shfl_xor(da, o);
    if (lane == 0) s_da[t] = da;
  }
  __syncthreads();
  float sad = 0.f;
  for (int t = tid; t < nw; t += 256) sad += s_alpha[t] * s_da[t];
  sad = block_sum(sad);
  for (int t = tid; t < nw; t += 256) {
    const float dl = s_alpha[t] * (s_da[t] - sad);
    atomicAdd(a.d_score + (int64_t)b * a.L + r0 + t, dl);
    if (a.d_bias) atomicAdd(a.d_bias + (plo - wlo + t), dl);
  }
}

// ---- indexer KL backward, per query: from A = q^I K^T (64 head slots x
// set), s_j = sum_h w_h relu(A_hj), Q = softmax(s) over the valid slots, P
// the normalised target; loss = sum P (log P - log Q); ds = Q - P;
// G_hj = ds_j w_h [A_hj > 0] (bf16) and dw_h = sum_j ds_j relu(A_hj).
// Three kernels: scores (a thread per slot), the per-query softmax and loss
// (a workgroup per query), G and dw (a thread per slot).
__global__ __launch_bounds__(256) void kl_score_kernel(KlArgs a, int q0) {
  __shared__ float s_w[64];
  const int qc = blockIdx.y, qr = q0 + qc;
  if (threadIdx.x < 64) s_w[threadIdx.x] = threadIdx.x < a.HI ? a.w_idx[(int64_t)qr * a.HI + threadIdx.x] : 0.f;
  __syncthreads();
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= a.nsp) return;
  const float* A = a.Am + (int64_t)qc * 64 * a.nsp + x;
  float sc = 0.f;
  for (int h = 0; h < a.HI; ++h) sc += s_w[h] * fmaxf(A[(int64_t)h * a.nsp], 0.f);
  const bool valid = x < a.ns && a.rowmap[(int64_t)qc * a.nsp + x] >= 0;
  a.Sb[(int64_t)qc * a.nsp + x] = valid ? sc : -INFINITY;
}

__global__ __launch_bounds__(256) void kl_reduce_kernel(KlArgs a, int q0) {
  __shared__ float s_red[8];
  const int qc = blockIdx.x, qr = q0 + qc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* S = a.Sb + (int64_t)qc * a.nsp;
  const float* tg = a.target + (int64_t)qr * a.ns;
  auto block_sum = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    return s_red[0] + s_red[1] + s_red[2] + s_red[3];
  };
  auto block_max = [&](float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    __syncthreads();
    if (lane == 0) s_red[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  };
  float mx = -INFINITY, ptot = 0.f;
  for (int x = tid; x < a.ns; x += 256) {
    mx = fmaxf(mx, S[x]);
    ptot += S[x] == -INFINITY ? 0.f : tg[x];
  }
  mx = block_max(mx);
  ptot = block_sum(ptot);
  float se = 0.f;
  for (int x = tid; x < a.ns; x += 256) se += S[x] == -INFINITY ? 0.f : expf(S[x] - mx);
  se = block_sum(se);
  const float lz = mx + logf(se);
  const float pin = ptot > 0.f ? 1.0f / ptot : 0.f;
  float loss = 0.f;
  for (int x = tid; x < a.nsp; x += 256) {
    float ds = 0.f;
    if (x < a.ns && S[x] != -INFINITY) {
      const float P = tg[x] * pin;
      const float lq = S[x] - lz;
      if (P > 0.f) loss += P * (logf(P) - lq);
      ds = (ptot > 0.f ? expf(lq) : 0.f) - P;
    }
    S[x] = ds;
  }
  loss = block_sum(loss);
  if (tid == 0 && a.loss) a.loss[qr] = loss;
  if (tid < a.HI) a.dw[(int64_t)qr * a.HI + tid] = 0.f;
}

__global__ __launch_bounds__(256) void kl_grad_kernel(KlArgs a, int q0) {
  __shared__ float s_w[64];
  const int qc = blockIdx.y, qr = q0 + qc;
  if (threadIdx.x < 64) s_w[threadIdx.x] = threadIdx.x < a.HI ? a.w_idx[(int64_t)qr * a.HI + threadIdx.x] : 0.f;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x * 256 + threadIdx.x;   // nsp is a multiple of 64: whole waves
  if (x >= a.nsp) return;
  const float ds = a.Sb[(int64_t)qc * a.nsp + x];
  const float* A = a.Am + (int64_t)qc * 64 * a.nsp + x;
  uint16_t* G = a.Gm + (int64_t)qc * 64 * a.nsp + x;
  for (int h = 0; h < 64; ++h) {
    const float av = h < a.HI ? A[(int64_t)h * a.nsp] : 0.f;
    G[(int64_t)h * a.nsp] = f2bf(av > 0.f ? ds * s_w[h] : 0.f);
    if (h < a.HI) {
      float dw = ds * fmaxf(av, 0.f);
      for (int o = 32; o > 0; o >>= 1) dw += __shfl_xor(dw, o);
      if (lane == 0) atomicAdd(a.dw + (int64_t)qr * a.HI + h, dw);
    }
  }
}

// Gathers a query's set of indexer keys as bf16 (dims padded to dIp with
// zeros) and the query's heads (64 slots); rowmap = b Ncap + j or -1.
__global__ __launch_bounds__(256) void kl_gather_kernel(KlArgs a, int q0) {
  const int qc = blockIdx.y, qr = q0 + qc;
  const int b = qr / a.Tq;
  const int x = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (x < a.nsp) {
    const int32_t j = x < a.ns ? a.sel[(int64_t)qr * a.ns + x] : -1;
    const bool ok = j >= 0 && j < a.Ncap;
    uint16_t* dst = a.K + ((int64_t)qc * a.nsp + x) * a.dIp;
    const uint16_t* src = a.k_idx + ((int64_t)b * a.Ncap + (ok ? j : 0)) * a.dI;
    for (int e = 8 * lane; e < a.dIp; e += 512)   // 16-byte pieces
      *reinterpret_cast<uint4*>(dst + e) =
          ok && e < a.dI ? *reinterpret_cast<const uint4*>(src + e) : uint4{0u, 0u, 0u, 0u};
    if (lane == 0) a.rowmap[(int64_t)qc * a.nsp + x] = ok ? (int64_t)b * a.Ncap + j : -1;
  }
  if (blockIdx.x < 16) {   // 64 head slots of q^I, four a workgroup
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    uint16_t* dst = a.Qi + ((int64_t)qc * 64 + h) * a.dIp;
    const uint16_t* src = a.q_idx + ((int64_t)qr * a.HI + (h < a.HI ? h : 0)) * a.dI;
    for (int e = 8 * lane; e < a.dIp; e += 512)
      *reinterpret_cast<uint4*>(dst + e) =
          h < a.HI && e < a.dI ? *reinterpret_cast<const uint4*>(src + e) : uint4{0u, 0u, 0u, 0u};
  }
}

// dq^I rows of the query (the first HI slots, dI dims) from the padded product
__global__ __launch_bounds__(256) void kl_dq_kernel(KlArgs a, int q0) {
  const int qc = blockIdx.x, qr = q0 + qc;
  for (int i = threadIdx.x; i < a.HI * a.dI; i += 256) {
    const int h = i / a.dI, e = i - h * a.dI;
    a.dq[(int64_t)qr * a.HI * a.dI + i] = a.DQ[((int64_t)qc * 64 + h) * a.dIp + e];
  }
}

template <bool AT, bool BT>
hipError_t gemm(const GemmArgs& g, int M, int N, int Z, hipStream_t st) {
  gemm_bf16_kernel<AT, BT><<<dim3(N / 64, M / 64, Z), 256, 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_rows_padded(int64_t rows_max) { return (rows_max + 63) / 64 * 64; }

size_t bwd_query_bytes(int D, int64_t np) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  return al((size_t)np * D * 2)          // X
         + al((size_t)np * 8)            // rowmap
         + al((size_t)128 * D * 2)       // Y
         + al((size_t)64 * 4)            // Dh
         + al((size_t)128 * np * 4)      // [S; dP]
         + al((size_t)128 * np * 2)      // T
         + al((size_t)64 * D * 4);       // dq~
}

hipError_t launch_attend_backward(BwdArgs a, int qchunk, void* ws, hipStream_t st) {
  const int nq = a.B * a.Tq;
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const int64_t np = a.np;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.X = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * np * a.D * 2);
  a.rowmap = reinterpret_cast<int64_t*>(w);    w += al((size_t)qchunk * np * 8);
  a.Y = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * 128 * a.D * 2);
  a.Dh = reinterpret_cast<float*>(w);          w += al((size_t)qchunk * 64 * 4);
  a.SP = reinterpret_cast<float*>(w);          w += al((size_t)qchunk * 128 * np * 4);
  a.T = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * 128 * np * 2);
  a.DQT = reinterpret_cast<float*>(w);
  for (int q0 = 0; q0 < nq; q0 += qchunk) {
    const int qc = nq - q0 < qchunk ? nq - q0 : qchunk;
    bwd_gather_kernel<<<dim3((unsigned)((np + 3) / 4), qc), 256, 0, st>>>(a, q0);
    bwd_prep_kernel<<<dim3(16, qc), 256, 0, st>>>(a, q0);
    // [S; dP] = Y X^T: M = 128, N = np, K = D
    GemmArgs g1{};
    g1.a = a.Y; g1.lda = a.D; g1.a_batch = 128 * (int64_t)a.D;
    g1.b = a.X; g1.ldb = a.D; g1.b_batch = np * a.D;
    g1.c = a.SP; g1.ldc = np; g1.c_batch = 128 * np; g1.K = a.D; g1.alpha = 1.f; g1.n_valid = (int)np;
    hipError_t e = gemm<false, true>(g1, 128, (int)np, qc, st);
    if (e != hipSuccess) return e;
    bwd_softmax_kernel<<<dim3((unsigned)((np + 255) / 256), qc), 256, 0, st>>>(a, q0);
    // dq~ = (scale dL) X: M = 64, N = D, K = np
    GemmArgs g2{};
    g2.a = a.T; g2.lda = np; g2.a_batch = 128 * np;
    g2.b = a.X; g2.ldb = a.D; g2.b_batch = np * a.D;
    g2.c = a.DQT; g2.ldc = a.D; g2.c_batch = 64 * (int64_t)a.D; g2.K = (int)np; g2.alpha = 1.f;
    g2.n_valid = a.D;
    e = gemm<false, false>(g2, 64, a.D, qc, st);
    if (e != hipSuccess) return e;
    // dX = T^T Y, added into the row gradients: M = np, N = D, K = 128
    GemmArgs g3{};
    g3.a = a.T; g3.lda = np; g3.a_batch = 128 * np;
    g3.b = a.Y; g3.ldb = a.D; g3.b_batch = 128 * (int64_t)a.D;
    g3.c = a.d_entries; g3.c2 = a.d_win; g3.ldc = a.D; g3.K = 128; g3.alpha = 1.f; g3.n_valid = a.D;
    g3.rowmap = a.rowmap; g3.rowmap_batch = np;
    e = gemm<true, false>(g3, (int)np, a.D, qc, st);
    if (e != hipSuccess) return e;
    bwd_q_kernel<<<dim3((unsigned)((a.H + 3) / 4), qc), 256, 0, st>>>(a, q0);
  }
  return hipGetLastError();
}

hipError_t launch_compress_backward(const CompressBwdArgs& a, hipStream_t st) {
  if (a.B == 0 || a.n_out == 0) return hipSuccess;
  compress_bwd_kernel<<<dim3((unsigned)a.n_out, (unsigned)a.B), 256, 0, st>>>(a);
  return hipGetLastError();
}

size_t kl_query_bytes(int64_t nsp, int dIp) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  return al((size_t)nsp * dIp * 2) + al((size_t)nsp * 8) + al((size_t)64 * dIp * 2) +
         al((size_t)64 * nsp * 4) + al((size_t)64 * nsp * 2) + al((size_t)64 * dIp * 4) +
         al((size_t)nsp * 4);
}

hipError_t launch_index_kl_backward(KlArgs a, int qchunk, void* ws, hipStream_t st) {
  const int nq = a.B * a.Tq;
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int64_t nsp = a.nsp;
  a.K = reinterpret_cast<uint16_t*>(w);      w += al((size_t)qchunk * nsp * a.dIp * 2);
  a.rowmap = reinterpret_cast<int64_t*>(w);  w += al((size_t)qchunk * nsp * 8);
  a.Qi = reinterpret_cast<uint16_t*>(w);     w += al((size_t)qchunk * 64 * a.dIp * 2);
  a.Am = reinterpret_cast<float*>(w);        w += al((size_t)qchunk * 64 * nsp * 4);
  a.Gm = reinterpret_cast<uint16_t*>(w);     w += al((size_t)qchunk * 64 * nsp * 2);
  a.DQ = reinterpret_cast<float*>(w);        w += al((size_t)qchunk * 64 * a.dIp * 4);
  a.Sb = reinterpret_cast<float*>(w);
  for (int q0 = 0; q0 < nq; q0 += qchunk) {
    const int qc = nq - q0 < qchunk ? nq - q0 : qchunk;
    const unsigned gx = (unsigned)((nsp + 3) / 4 > 16 ? (nsp + 3) / 4 : 16);
    kl_gather_kernel<<<dim3(gx, qc), 256, 0, st>>>(a, q0);
    // A = Qi K^T: M = 64, N = nsp, K = dIp
    GemmArgs g1{};
    g1.a = a.Qi; g1.lda = a.dIp; g1.a_batch = 64 * (int64_t)a.dIp;
    g1.b = a.K; g1.ldb = a.dIp; g1.b_batch = nsp * a.dIp;
    g1.c = a.Am; g1.ldc = nsp; g1.c_batch = 64 * nsp; g1.K = a.dIp; g1.alpha = 1.f;
    g1.n_valid = (int)nsp;
    hipError_t e = gemm<false, true>(g1, 64, (int)nsp, qc, st);
    if (e != hipSuccess) return e;
    kl_score_kernel<<<dim3((unsigned)((nsp + 255) / 256), qc), 256, 0, st>>>(a, q0);
    kl_reduce_kernel<<<qc, 256, 0, st>>>(a, q0);
    kl_grad_kernel<<<dim3((unsigned)((nsp + 255) / 256), qc), 256, 0, st>>>(a, q0);
    // dq = G K: M = 64, N = dIp, K = nsp
    GemmArgs g2{};
    g2.a = a.Gm; g2.lda = nsp; g2.a_batch = 64 * nsp;
    g2.b = a.K; g2.ldb = a.dIp; g2.b_batch = nsp * a.dIp;
    g2.c = a.DQ; g2.ldc = a.dIp; g2.c_batch = 64 * (int64_t)a.dIp; g2.K = (int)nsp; g2.alpha = 1.f;
    g2.n_valid = a.dIp;
    e = gemm<false, false>(g2, 64, a.dIp, qc, st);
    if (e != hipSuccess) return e;
    kl_dq_kernel<<<qc, 256, 0, st>>>(a, q0);
    // dK = G^T Qi, added into dk rows: M = nsp, N = dIp (first dI kept), K = 64
    GemmArgs g3{};
    g3.a = a.Gm; g3.lda = nsp; g3.a_batch = 64 * nsp;
    g3.b = a.Qi; g3.ldb = a.dIp; g3.b_batch = 64 * (int64_t)a.dIp;
    g3.c = a.dk; g3.ldc = a.dI; g3.K = 64; g3.alpha = 1.f; g3.n_valid = a.dI;
    g3.rowmap = a.rowmap; g3.rowmap_batch = nsp;
    e = gemm<true, false>(g3, (int)nsp, a.dIp, qc, st);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace v4
