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
// between (an elementwise kernel).  A row may be attended by many queries:
// with room in the workspace, every slot's dX row is stored densely, the
// slots are sorted by destination row (a counting sort) and each row's
// gradient is added once; otherwise the dX rows are added with atomics.
// dq~ goes back through RoPE_t and the RMSNorm.

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

typedef unsigned u32x3 __attribute__((ext_vector_type(3)));

// Dense per-slot gradients are kept as 24-bit floats (fp32 with the low 8
// mantissa bits rounded off, to nearest even): four values in three words.
// The relative rounding, 2^-16, is far below the bf16 roundings the products
// already carry (2^-9), and the dense round trip moves 3/4 of the bytes.
__device__ __forceinline__ uint32_t f24_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7Fu + ((u >> 8) & 1u)) >> 8;
}
__device__ __forceinline__ u32x3 f24_pack4(float a, float b, float c, float d) {
  const uint32_t u0 = f24_bits(a), u1 = f24_bits(b), u2 = f24_bits(c), u3 = f24_bits(d);
  return u32x3{u0 | (u1 << 24), (u1 >> 8) | (u2 << 16), (u2 >> 16) | (u3 << 8)};
}
__device__ __forceinline__ void f24_unpack4(uint32_t w0, uint32_t w1, uint32_t w2, float* o) {
  o[0] = __uint_as_float(w0 << 8);
  o[1] = __uint_as_float(((w0 >> 24) | (w1 << 8)) << 8);
  o[2] = __uint_as_float(((w1 >> 16) | (w2 << 16)) << 8);
  o[3] = __uint_as_float((w2 >> 8) << 8);
}

// The tile (x, y) and batch z of this workgroup in a batched launch.
// Workgroups go to the eight XCDs in turn (linear id mod 8), each XCD with
// its own L2; when the batch count is a multiple of 8 the linear id is
// remapped so that XCD c runs every tile of batches c, c + 8, ..., one batch
// after another, and each batch's operands are read into one L2 only.
struct BatchTile { int x, y, z; };
__device__ __forceinline__ BatchTile xcd_batch_tile() {
  const int gx = gridDim.x, gy = gridDim.y;
  if (gridDim.z & 7) return BatchTile{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
  const int P = gx * gy;
  const int L = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int j = L >> 3, p = j % P;
  return BatchTile{p % gx, p / gx, (j / P) * 8 + (L & 7)};
}

// C[z] = alpha A[z] B[z] on 64 x 64 tiles, K in steps of 32 (all multiples:
// the caller pads).  A is M x K (AT: stored K x M), B is K x N (BT: stored
// N x K); bf16 in, fp32 accumulate.  Four waves, 32 x 32 each.
template <bool AT, bool BT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[64][kLdsK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[64][kLdsK];
  const BatchTile bt = xcd_batch_tile();
  const int z = bt.z;
  const int n0 = bt.x * 64, m0 = bt.y * 64;
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
  // lane (c, gq) holds rows 4 gq + v, column c of each 16 x 16 block.  The
  // tile goes through LDS so that one wave's store (or atomic) instruction
  // covers 64 consecutive floats of one row (two whole cache lines) rather
  // than 16 floats of four rows.
  __shared__ float sC[64][65];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) sC[wm * 32 + 16 * i + 4 * gq + v][wn * 32 + 16 * j + c] = acc[i][j][v];
  __syncthreads();
  if (!g.rowmap && g.f24) {   // rows of ldc 24-bit values; 16 lanes a row, 4 values a lane
    const int cg = lane & 15;
    if (n0 + 4 * cg >= g.n_valid) return;   // n_valid is a multiple of 4
    uint32_t* cz = reinterpret_cast<uint32_t*>(g.c) + ((int64_t)z * g.c_batch + n0) / 4 * 3 + 3 * cg;
#pragma unroll 4
    for (int mm = 4 * wave + (lane >> 4); mm < 64; mm += 16)
      __builtin_nontemporal_store(f24_pack4(g.alpha * sC[mm][4 * cg], g.alpha * sC[mm][4 * cg + 1],
                                            g.alpha * sC[mm][4 * cg + 2], g.alpha * sC[mm][4 * cg + 3]),
                                  reinterpret_cast<u32x3*>(cz + (int64_t)(m0 + mm) * (g.ldc / 4 * 3)));
    return;
  }
  const int n = n0 + lane;
  if (n >= g.n_valid) return;
  if (!g.rowmap) {
    float* cz = g.c + (int64_t)z * g.c_batch + n;
#pragma unroll 4
    for (int mm = wave; mm < 64; mm += 4) cz[(int64_t)(m0 + mm) * g.ldc] = g.alpha * sC[mm][lane];
    return;
  }
  // scattered adds
#pragma unroll 4
  for (int mm = wave; mm < 64; mm += 4) {
    const int64_t r = g.rowmap[(int64_t)z * g.rowmap_batch + m0 + mm];
    const float x = g.alpha * sC[mm][lane];
    if (r >= 0) atomicAdd(g.c + r * g.ldc + n, x);
    else if (r <= -2) atomicAdd(g.c2 + (-2 - r) * g.ldc + n, x);
  }
}

// Tiles of C[z] = A[z] B[z], TM x 128, k in steps of 32 (M, N and K
// multiples of TM, 128 and 32).  Four waves as 2 x 2, each (TM / 2) x 64 on
// the 32x32x16 bf16 MFMAs; the next k-step's tiles come from global memory
// while the current one's MFMAs run and go to the other of two LDS buffers
// (one barrier a step).  A is M x K (AT: stored K x M), B is K x N (BT:
// stored N x K); a source stored k-major is transposed on its way into LDS.
// (dq~ = T X, whose X operand is k-major, stays on gemm_bf16_kernel:
// transposing X element by element into these larger tiles cost more than
// the faster MFMAs saved.  dX = T^T Y runs here on operands that the
// softmax-gradient and prep kernels also write transposed.)
template <int TM>
constexpr int gemm32_smem_bytes() {
  return 2 * (TM + 128) * 40 * 2 > TM * 129 * 4 ? 2 * (TM + 128) * 40 * 2 : TM * 129 * 4;
}

// The main loop of gemm32: this workgroup's TM x 128 tile of A[z] B[z] in acc
// (lane: column lane % 32 of each 32 x 32 block, rows (e/4) 8 + (lane/32) 4 + e % 4).
// PF k-tiles are in flight from global memory (K a multiple of PF x 32).
template <int TM, bool AT, bool BT, int PF>
__device__ __forceinline__ void gemm32_main(const GemmArgs& g, uint8_t* smem, f32x16 (&acc)[TM / 64][2],
                                            int n0, int m0, int z) {
  constexpr int TN = 128, BK = 32, KP = 40;   // KP: padded k stride (elements) of the LDS tiles
  constexpr int WM = TM / 2, MB = WM / 32;    // rows per wave, 32-row blocks per wave
  constexpr int LA = TM * BK / 8 / 256;       // 16-byte loads per thread per step (A)
  constexpr int LB = TN * BK / 8 / 256;       // (B)
  auto sA = reinterpret_cast<uint16_t (*)[TM][KP]>(smem);
  auto sB = reinterpret_cast<uint16_t (*)[TN][KP]>(smem + 2 * TM * KP * 2);
  const uint16_t* A = g.a + (int64_t)z * g.a_batch;
  const uint16_t* B = g.b + (int64_t)z * g.b_batch;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // load i of this thread: rows x k source: row x / 4, k chunk x % 4; k x rows
  // source: k x / (ROWS / 8), row chunk x % (ROWS / 8)  (x = tid + 256 i)
  auto fetch = [&](const uint16_t* p, int64_t ld, int r0, int k0, bool tr, int rows, int i) -> uint4 {
    const int x = tid + 256 * i;
    if (!tr) return *reinterpret_cast<const uint4*>(p + (int64_t)(r0 + (x >> 2)) * ld + k0 + 8 * (x & 3));
    const int cpr = rows / 8;
    return *reinterpret_cast<const uint4*>(p + (int64_t)(k0 + x / cpr) * ld + r0 + 8 * (x % cpr));
  };
  auto put = [&](uint16_t (*s)[KP], uint4 v, bool tr, int rows, int i) {
    const int x = tid + 256 * i;
    if (!tr) {
      *reinterpret_cast<uint4*>(&s[x >> 2][8 * (x & 3)]) = v;
      return;
    }
    const int cpr = rows / 8, kk = x / cpr, ch = x % cpr;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[8 * ch + 2 * e][kk] = (uint16_t)(w[e] & 0xFFFFu);
      s[8 * ch + 2 * e + 1][kk] = (uint16_t)(w[e] >> 16);
    }
  };
  uint4 ra[PF][LA], rb[PF][LB];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    if (p * BK < g.K) {
#pragma unroll
      for (int i = 0; i < LA; ++i) ra[p][i] = fetch(A, g.lda, m0, p * BK, AT, TM, i);
#pragma unroll
      for (int i = 0; i < LB; ++i) rb[p][i] = fetch(B, g.ldb, n0, p * BK, !BT, TN, i);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;
  int buf = 0;
  for (int k00 = 0; k00 < g.K; k00 += PF * BK) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int k0 = k00 + p * BK;
#pragma unroll
      for (int i = 0; i < LA; ++i) put(sA[buf], ra[p][i], AT, TM, i);
#pragma unroll
      for (int i = 0; i < LB; ++i) put(sB[buf], rb[p][i], !BT, TN, i);
      __syncthreads();   // buffer buf complete; every wave is done with buf ^ 1's last reads
      if (k0 + PF * BK < g.K) {
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[p][i] = fetch(A, g.lda, m0, k0 + PF * BK, AT, TM, i);
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[p][i] = fetch(B, g.ldb, n0, k0 + PF * BK, !BT, TN, i);
      }
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8 av[MB], bv[2];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          av[mb] = *reinterpret_cast<const bf16x8*>(&sA[buf][wm * WM + 32 * mb + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bv[nb] = *reinterpret_cast<const bf16x8*>(&sB[buf][wn * 64 + 32 * nb + (lane & 31)][16 * ks + 8 * (lane >> 5)]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mb], bv[nb], acc[mb][nb], 0, 0, 0);
      }
      buf ^= 1;
    }
  }
}

// [S; dP] = Y X^T for one query (z) and 128 row slots, with the softmax
// gradient as its epilogue: T = [scale dL; P] (bf16) with P = exp(scale S -
// lse), dL = P (dP - D_h), 0 for absent rows and head slots >= H, and p_sel
// (the head sum of P) for entry slots.  The fp32 [S; dP] never leaves LDS.
__global__ __launch_bounds__(256) void bwd_sdp_kernel(GemmArgs g, BwdArgs a, int q0) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[gemm32_smem_bytes<128>()];
  __shared__ float s_l2[64], s_dh[64], s_ps[128];
  const BatchTile bt = xcd_batch_tile();
  const int z = bt.z, qr = q0 + z;
  const int n0 = bt.x * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) {
    const float lse = tid < a.H ? a.lse[(int64_t)qr * a.H + tid] : -INFINITY;
    s_l2[tid] = lse * kL2e;
    s_dh[tid] = a.Dh[(int64_t)z * 64 + tid];
  }
  f32x16 acc[2][2];
  gemm32_main<128, false, true, 2>(g, smem, acc, n0, 0, z);
  const int wm = wave >> 1, wn = wave & 1;
  __syncthreads();   // the operand tiles are done with: the space holds [S; dP]
  auto sC = reinterpret_cast<float (*)[129]>(smem);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sC[wm * 64 + 32 * mb + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)][wn * 64 + 32 * nb + (lane & 31)] =
            acc[mb][nb][e];
  __syncthreads();
  // thread: row slot c = tid % 128 of the tile, heads 32 (tid / 128) .. + 31
  const int c = tid & 127, hh = tid >> 7;
  const int64_t x = n0 + c;
  const bool present = a.rowmap[(int64_t)z * a.np + x] != -1;
  const float sl2 = a.scale * kL2e;
  uint16_t* tp = a.T + (int64_t)z * 64 * a.np + x;        // scale dL, head rows (dq~)
  float psum = 0.f;
  uint32_t tdl[16], tpp[16];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int h = 32 * hh + i;
    float p = 0.f, dl = 0.f;
    if (present && s_l2[h] != -INFINITY) {
      p = exp2f(sC[h][c] * sl2 - s_l2[h]);
      dl = p * (sC[64 + h][c] - s_dh[h]);
    }
    psum += p;
    const uint32_t bdl = f2bf(a.scale * dl), bp = f2bf(p);
    tp[(int64_t)h * a.np] = (uint16_t)bdl;
    // [scale dL; P] of slot x, head-contiguous, for dX
    tdl[i >> 1] = (i & 1) ? tdl[i >> 1] | (bdl << 16) : bdl;
    tpp[i >> 1] = (i & 1) ? tpp[i >> 1] | (bp << 16) : bp;
  }
  // the tile's TT rows (128 slots x 256 bytes, one contiguous block) go out
  // through LDS as whole 1 KB wave stores
  __syncthreads();   // every thread is done reading [S; dP]
  auto sT = reinterpret_cast<uint4 (*)[17]>(smem);   // [slot][16 units + 1 pad] of 8 bf16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sT[c][4 * hh + v] = uint4{tdl[4 * v], tdl[4 * v + 1], tdl[4 * v + 2], tdl[4 * v + 3]};
    sT[c][8 + 4 * hh + v] = uint4{tpp[4 * v], tpp[4 * v + 1], tpp[4 * v + 2], tpp[4 * v + 3]};
  }
  __syncthreads();
  uint4* tt = reinterpret_cast<uint4*>(a.TT + ((int64_t)z * a.np + n0) * 128);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int u = tid + 256 * i;   // 16-byte unit u % 16 of slot u / 16
    tt[u] = sT[u >> 4][u & 15];
  }
  if (hh == 1) s_ps[c] = psum;
  __syncthreads();
  if (hh == 0 && a.p_sel && x < a.k_sel) a.p_sel[(int64_t)qr * a.k_sel + x] = psum + s_ps[c];
}

// dX = [scale dL; P]^T [q~; do] for one query (z), a tile of 128 row slots x
// 128 dims, K = 128 head slots: both operands read k-contiguous (TT and YT).
// The tile is stored densely past the caches (it is read back once, by the
// grouped sum) or, with rowmap, added into the row gradients with atomics.
__global__ __launch_bounds__(256) void bwd_dx_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[gemm32_smem_bytes<128>()];
  const BatchTile bt = xcd_batch_tile();
  const int z = bt.z, n0 = bt.x * 128, m0 = bt.y * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  f32x16 acc[2][2];
  gemm32_main<128, false, true, 1>(g, smem, acc, n0, m0, z);
  const int wm = wave >> 1, wn = wave & 1;
  __syncthreads();   // the operand tiles are done with: the space holds the C tile
  auto sC = reinterpret_cast<float (*)[129]>(smem);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sC[wm * 64 + 32 * mb + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3)][wn * 64 + 32 * nb + (lane & 31)] =
            acc[mb][nb][e];
  __syncthreads();
  if (!g.rowmap) {   // rows of ldc 24-bit values (3 ldc / 4 words); two rows a wave store
    uint32_t* cz = reinterpret_cast<uint32_t*>(g.c) + ((int64_t)z * g.c_batch + n0) / 4 * 3;
    const int half = lane >> 5, l = lane & 31;
#pragma unroll 4
    for (int mm = 2 * wave + half; mm < 128; mm += 8) {
      u32x3* dst = reinterpret_cast<u32x3*>(cz + (int64_t)(m0 + mm) * (g.ldc / 4 * 3) + 3 * l);
      __builtin_nontemporal_store(
          f24_pack4(sC[mm][4 * l], sC[mm][4 * l + 1], sC[mm][4 * l + 2], sC[mm][4 * l + 3]), dst);
    }
    return;
  }
#pragma unroll 4
  for (int mm = wave; mm < 128; mm += 4) {
    const int64_t r = g.rowmap[(int64_t)z * g.rowmap_batch + m0 + mm];
    float* row = r >= 0 ? g.c + r * g.ldc : (r <= -2 ? g.c2 + (-2 - r) * g.ldc : nullptr);
    if (row) {
      atomicAdd(row + n0 + lane, sC[mm][lane]);
      atomicAdd(row + n0 + 64 + lane, sC[mm][64 + lane]);
    }
  }
}

// X[qc, x, :] = the query's row x as bf16 (zeros if absent), rowmap = where
// its gradient goes: entry b Ncap + j (>= 0), window row -2 - (b (Tq+W-1) + r),
// or -1.  One wave per kGatherRows row slots (their loads in flight together).
#ifndef V4_GATHER_ROWS
#define V4_GATHER_ROWS 2
#endif
constexpr int kGatherRows = V4_GATHER_ROWS;
__global__ __launch_bounds__(256) void bwd_gather_kernel(BwdArgs a, int q0) {
  // the arguments are read in one round before any branch (the empty asm
  // statements keep the compiler from sinking each read into the branch
  // that uses it, one dependent round trip after another)
  const int Tq = a.Tq, k = a.k, m = a.m, W = a.W, D = a.D, R = a.R, group_q0 = a.group_q0;
  const int64_t np = a.np, q_pos0 = a.q_pos0, Ncap = a.Ncap, n_entries = a.n_entries, nent = a.nent;
  const int32_t* const topk = a.topk;
  const uint8_t* const entries = a.entries;
  const uint8_t* const win = a.win;
  uint16_t* const X = a.X;
  int64_t* const rowmap = a.rowmap;
  int32_t* const dest = a.dest;
  uint32_t* const cnt = a.cnt;
  const bool grouped = a.dXd != nullptr;
  asm volatile("" ::"s"(topk), "s"(entries), "s"(win), "s"(X), "s"(rowmap), "s"(dest), "s"(cnt),
               "s"(np), "s"(q_pos0), "s"(Ncap), "s"(n_entries), "s"(nent));
  asm volatile("" ::"s"(Tq), "s"(k), "s"(m), "s"(W), "s"(D), "s"(R), "s"(group_q0),
               "s"((int)grouped));
  const int qc = blockIdx.y, qr = q0 + qc;
  const int b = qr / Tq, r = qr % Tq;
  const int64_t t = q_pos0 + r;
  constexpr int RPW = kGatherRows;
  const int x0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW, lane = threadIdx.x & 63;
  if (x0 >= np) return;   // np is a multiple of 128: all RPW slots exist
  int64_t n_ent;
  if (topk) {
    n_ent = k;
  } else {
    const int64_t v = (t + 1) / m;
    n_ent = v < n_entries ? v : n_entries;
  }
  const int64_t lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int64_t n_win = W > 0 ? t - lo + 1 : 0;
  const int ROW = D + R;
  const uint8_t* src[RPW];
  int64_t map[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    const int x = x0 + u;
    src[u] = nullptr;
    map[u] = -1;
    if (x < n_ent) {
      const int64_t j = topk ? (int64_t)topk[(int64_t)qr * k + x] : (int64_t)x;
      if (j >= 0 && j < Ncap) {
        src[u] = entries + ((int64_t)b * Ncap + j) * ROW;
        map[u] = (int64_t)b * Ncap + j;
      }
    } else if (x < n_ent + n_win) {
      const int64_t wrow = lo + (x - n_ent) - (q_pos0 - (W - 1));
      const int64_t grow = (int64_t)b * (Tq + W - 1) + wrow;
      src[u] = win + grow * ROW;
      map[u] = -2 - grow;
    }
  }
  if (lane < RPW) {   // lane u: slot x0 + u's bookkeeping
    int64_t mp = map[0];
#pragma unroll
    for (int u = 1; u < RPW; ++u) mp = lane == u ? map[u] : mp;
    rowmap[(int64_t)qc * np + x0 + lane] = mp;
    if (grouped) {   // grouped row gradients: the destination and its count
      const int64_t d = mp >= 0 ? mp : (mp <= -2 ? nent + (-2 - mp) : -1);
      dest[(int64_t)(qr - group_q0) * np + x0 + lane] = (int32_t)d;
      if (d >= 0) atomicAdd(cnt + d, 1u);
    }
  }
  const int E = D - R;
  const int d = 8 * lane;   // this lane's 8 dims (E and D are multiples of 8)
  if (d >= D) return;
  // every slot's load is issued before the first conversion and store
  uint4 o[RPW];
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    o[u] = uint4{0u, 0u, 0u, 0u};
    if (src[u]) {
      if (d < E) {
        const uint2 b8 = *reinterpret_cast<const uint2*>(src[u] + d);
        o[u] = uint4{b8.x, b8.y, 0u, 0u};
      } else {
        o[u] = *reinterpret_cast<const uint4*>(src[u] + E + 2 * (d - E));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < RPW; ++u) {
    uint4 w = o[u];
    if (src[u] && d < E) {   // 8 E4M3 bytes -> 8 bf16 (exact)
      const uint32_t w2[2] = {o[u].x, o[u].y};
      uint32_t rr[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x2 lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w2[h], false);
        const f32x2 hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w2[h], true);
        rr[2 * h] = (__float_as_uint(lo2[0]) >> 16) | (__float_as_uint(lo2[1]) & 0xFFFF0000u);
        rr[2 * h + 1] = (__float_as_uint(hi2[0]) >> 16) | (__float_as_uint(hi2[1]) & 0xFFFF0000u);
      }
      w = uint4{rr[0], rr[1], rr[2], rr[3]};
    }
    *reinterpret_cast<uint4*>(X + ((int64_t)qc * np + x0 + u) * D + d) = w;
  }
}

// The eight bf16 of a 16-byte word as floats.
__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float (&x)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(ws[i] << 16);
    x[2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint4 f32_to_bf16x8(const float (&x)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f2bf(x[2 * i]) | ((uint32_t)f2bf(x[2 * i + 1]) << 16);
  return uint4{w[0], w[1], w[2], w[3]};
}

// (cos, sin) of the rotary pairs among dims d .. d + 7 at position t ((1, 0)
// below the rotary dims); the turn table is read with clamped indices, so
// every lane loads and no branch waits on a load.
__device__ __forceinline__ void lane_rot8(const BwdArgs& a, int d, int64_t t, float (&cs)[4],
                                          float (&sn)[4]) {
  double tv[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int i = (d + 2 * p - (a.D - a.R)) >> 1;
    tv[p] = a.rope.t[i < 0 ? 0 : (i > 31 ? 31 : i)];
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    cs[p] = 1.f;
    sn[p] = 0.f;
    if (d + 2 * p >= a.D - a.R) rope_cos_sin(t, tv[p], &cs[p], &sn[p]);
  }
}

// Y[qc] = [q~ (64 head slots); do = RoPE_t(dout) (64 slots)] as bf16, and
// the same transposed (YT[qc], dims x head slots, through LDS), Dh = dout .
// out, the query's d_sink share -p_sink Dh.  One wave per head, 16 heads a
// workgroup; lane l holds dims 8 l .. 8 l + 7 (16-byte loads and stores).
__global__ __launch_bounds__(1024) void bwd_prep_kernel(BwdArgs a, int q0) {
  __shared__ __attribute__((aligned(16))) uint16_t s_y[2][16][512];
  const int qc = blockIdx.y, qr = q0 + qc;
  const int r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int h = blockIdx.x * 16 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int d = 8 * lane;
  const bool act = d < a.D;
  uint16_t* yq = a.Y + ((int64_t)qc * 128 + h) * a.D + d;
  uint16_t* yd = a.Y + ((int64_t)qc * 128 + 64 + h) * a.D + d;
  const bool live = h < a.H;   // head slots >= H are zeros
  const int64_t off = ((int64_t)qr * a.H + (live ? h : 0)) * a.D + d;
  uint4 qw{0u, 0u, 0u, 0u}, gw{0u, 0u, 0u, 0u}, ow{0u, 0u, 0u, 0u};
  float gm[8];
  if (act && live) {
    qw = *reinterpret_cast<const uint4*>(a.q + off);
    gw = *reinterpret_cast<const uint4*>(a.dout + off);
    ow = *reinterpret_cast<const uint4*>(a.out + off);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = act ? a.gamma_q[d + e] : 0.f;
  float cs[4], sn[4];
  lane_rot8(a, d, t, cs, sn);
  float x[8], g[8], o[8];
  bf16x8_to_f32(qw, x);
  bf16x8_to_f32(gw, g);
  bf16x8_to_f32(ow, o);
  float ss = 0.f, dd = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ss += x[e] * x[e];
    dd += g[e] * o[e];
  }
  ss = wave_sum(ss);
  dd = wave_sum(dd);
  const float rsn = 1.0f / sqrtf(ss / (float)a.D + a.eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = gm[e] * (x[e] * rsn);
  if (d >= a.D - a.R) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = x[2 * p], x1 = x[2 * p + 1], g0 = g[2 * p], g1 = g[2 * p + 1];
      x[2 * p] = x0 * cs[p] - x1 * sn[p];
      x[2 * p + 1] = x0 * sn[p] + x1 * cs[p];
      g[2 * p] = g0 * cs[p] - g1 * sn[p];       // do = RoPE_t(dout)
      g[2 * p + 1] = g0 * sn[p] + g1 * cs[p];
    }
  }
  const int w = threadIdx.x >> 6;
  if (act) {
    const uint4 vq = live ? f32_to_bf16x8(x) : uint4{0u, 0u, 0u, 0u};
    const uint4 vd = live ? f32_to_bf16x8(g) : uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(yq) = vq;
    *reinterpret_cast<uint4*>(yd) = vd;
    *reinterpret_cast<uint4*>(&s_y[0][w][d]) = vq;
    *reinterpret_cast<uint4*>(&s_y[1][w][d]) = vd;
  }
  __syncthreads();
  // YT[qc][e][64 p + 16 blockIdx.x ..]: this workgroup's 16 head slots of
  // dim e (32 bytes), a (dim, half) pair per thread
  uint16_t* yt = a.YT + (int64_t)qc * a.D * 128 + 16 * blockIdx.x;
  for (int i = threadIdx.x; i < 2 * a.D; i += 1024) {
    const int e = i >> 1, p = i & 1;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = (uint32_t)s_y[p][2 * j][e] | ((uint32_t)s_y[p][2 * j + 1][e] << 16);
    uint4* dst = reinterpret_cast<uint4*>(yt + (int64_t)e * 128 + 64 * p);
    dst[0] = uint4{v[0], v[1], v[2], v[3]};
    dst[1] = uint4{v[4], v[5], v[6], v[7]};
  }
  if (lane == 0 && live) {
    a.Dh[(int64_t)qc * 64 + h] = dd;
    float ds = 0.f;
    if (a.sink) {
      const float lse = a.lse[(int64_t)qr * a.H + h];
      const float pz = lse == -INFINITY ? 0.f : expf(a.sink[h] - lse);
      ds = -pz * dd;
    }
    // row qc sums the shares of the queries qc, qc + chunk, .. (the chunks
    // run in order on one stream); bwd_reduce_kernel adds the rows at the end
    float* dsp = a.DS + (int64_t)qc * 64 + h;
    *dsp = (q0 == 0 ? 0.f : *dsp) + ds;
  }
}

// dq = RMSNorm backward of RoPE_t^T(dq~); the query's d_gamma_q share
// (summed over its heads) is added to row qc of G.  One workgroup of 16 waves per
// query; wave w takes heads w, w + 16, ..; lane l holds dims 8 l .. 8 l + 7.
// (Adding every workgroup's share into d_gamma_q directly put ~1,000 atomic
// adds per chunk on each of its addresses.)
__global__ __launch_bounds__(1024) void bwd_q_kernel(BwdArgs a, int q0) {
  __shared__ float s_dg[16][512];
  const int qc = blockIdx.x, qr = q0 + qc;
  const int r = qr % a.Tq;
  const int64_t t = a.q_pos0 + r;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d = 8 * lane;
  const bool act = d < a.D;
  float dg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) dg[e] = 0.f;
  float gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gm[e] = act ? a.gamma_q[d + e] : 0.f;
  float cs[4], sn[4];
  lane_rot8(a, d, t, cs, sn);
  for (int h = wave; h < a.H; h += 16) {
    uint4 qw{0u, 0u, 0u, 0u};
    f32x4 u0{0.f, 0.f, 0.f, 0.f}, u1{0.f, 0.f, 0.f, 0.f};
    if (act) {
      qw = *reinterpret_cast<const uint4*>(a.q + ((int64_t)qr * a.H + h) * a.D + d);
      const float* gq = a.DQT + ((int64_t)qc * 64 + h) * a.D + d;
      u0 = *reinterpret_cast<const f32x4*>(gq);
      u1 = *reinterpret_cast<const f32x4*>(gq + 4);
    }
    float xq[8], u[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
    bf16x8_to_f32(qw, xq);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xq[e] * xq[e];
    ss = wave_sum(ss);
    const float rsn = 1.0f / sqrtf(ss / (float)a.D + a.eps);
    if (d >= a.D - a.R) {   // RoPE_t transposed = rotation by -t
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float v0 = u[2 * p], v1 = u[2 * p + 1];
        u[2 * p] = v0 * cs[p] + v1 * sn[p];
        u[2 * p + 1] = -v0 * sn[p] + v1 * cs[p];
      }
    }
    float gx[8], dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      dg[e] += u[e] * xq[e] * rsn;
      gx[e] = u[e] * gm[e];
      dot += gx[e] * xq[e];
    }
    dot = wave_sum(dot);
    const float c3 = dot * rsn * rsn * rsn / (float)a.D;
    if (act) {
      float* dqp = a.dq + ((int64_t)qr * a.H + h) * a.D + d;
      *reinterpret_cast<f32x4*>(dqp) = f32x4{gx[0] * rsn - xq[0] * c3, gx[1] * rsn - xq[1] * c3,
                                             gx[2] * rsn - xq[2] * c3, gx[3] * rsn - xq[3] * c3};
      *reinterpret_cast<f32x4*>(dqp + 4) = f32x4{gx[4] * rsn - xq[4] * c3, gx[5] * rsn - xq[5] * c3,
                                                 gx[6] * rsn - xq[6] * c3, gx[7] * rsn - xq[7] * c3};
    }
  }
  if (act) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_dg[wave][d + e] = dg[e];
  }
  __syncthreads();
  for (int x = threadIdx.x; x < a.D; x += 1024) {
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) z += s_dg[w][x];
    float* gp = a.G + (int64_t)qc * a.D + x;   // accumulated over the chunks, as DS
    *gp = (q0 == 0 ? 0.f : *gp) + z;
  }
}

// After the last chunk: d_gamma_q += the G rows summed, d_sink += the DS rows
// summed (one atomic add per address).  Thread x of the grid takes column x.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a, int qc_n) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (a.d_gamma_q && x < a.D) {
    float z = 0.f;
#pragma unroll 8
    for (int q = 0; q < qc_n; ++q) z += a.G[(int64_t)q * a.D + x];
    atomicAdd(a.d_gamma_q + x, z);
  }
  if (a.sink && a.d_sink && blockIdx.x == 0 && x < a.H) {
    float z = 0.f;
#pragma unroll 8
    for (int q = 0; q < qc_n; ++q) z += a.DS[(int64_t)q * 64 + x];
    atomicAdd(a.d_sink + x, z);
  }
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
  // key rows: dIp / 8 threads a row, 16 bytes each (16 or 32 rows a workgroup)
  const int cpr = a.dIp >> 3;
  const int x = blockIdx.x * (256 / cpr) + threadIdx.x / cpr, e = 8 * (threadIdx.x % cpr);
  if (x < a.nsp) {
    const int32_t j = x < a.ns ? a.sel[(int64_t)qr * a.ns + x] : -1;
    const bool ok = j >= 0 && j < a.Ncap;
    uint16_t* dst = a.K + ((int64_t)qc * a.nsp + x) * a.dIp;
    const uint16_t* src = a.k_idx + ((int64_t)b * a.Ncap + (ok ? j : 0)) * a.dI;
    *reinterpret_cast<uint4*>(dst + e) =
        ok && e < a.dI ? *reinterpret_cast<const uint4*>(src + e) : uint4{0u, 0u, 0u, 0u};
    if (e == 0) {
      const int64_t d = ok ? (int64_t)b * a.Ncap + j : -1;
      a.rowmap[(int64_t)qc * a.nsp + x] = d;
      if (a.dKd) {   // grouped key gradients: the destination and its count
        a.dest[(int64_t)(qr - a.group_q0) * a.nsp + x] = (int32_t)d;
        if (d >= 0) atomicAdd(a.cnt + d, 1u);
      }
    }
  }
  if (blockIdx.x < 16) {   // 64 head slots of q^I, four a workgroup
    const int lane = threadIdx.x & 63;
    const int h = blockIdx.x * 4 + (threadIdx.x >> 6);
    uint16_t* dst = a.Qi + ((int64_t)qc * 64 + h) * a.dIp;
    const uint16_t* src = a.q_idx + ((int64_t)qr * a.HI + (h < a.HI ? h : 0)) * a.dI;
    for (int e2 = 8 * lane; e2 < a.dIp; e2 += 512)
      *reinterpret_cast<uint4*>(dst + e2) =
          h < a.HI && e2 < a.dI ? *reinterpret_cast<const uint4*>(src + e2) : uint4{0u, 0u, 0u, 0u};
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


// ---- grouped row gradients: a counting sort of the group's (query, row
// slot) gradients by destination row, then one sum per destination.

__global__ __launch_bounds__(256) void bwd_fill_u32_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0u;
}

// off[0..n] = exclusive prefix sum of cnt[0..n), in tiles of 4096
// destinations (a workgroup of 256 threads, 16 consecutive counts a thread):
// the tiles' sums, their exclusive scan (one workgroup), then each tile's
// offsets; the last pass clears cnt (it becomes the destinations' cursors).
constexpr int kGroupTile = 4096;

__device__ inline void load16_u32(const uint32_t* p, int64_t i0, int64_t n, uint32_t (&c)[16]) {
  if (i0 + 16 <= n) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 u = *reinterpret_cast<const uint4*>(p + i0 + 4 * v);
      c[4 * v] = u.x; c[4 * v + 1] = u.y; c[4 * v + 2] = u.z; c[4 * v + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) c[v] = i0 + v < n ? p[i0 + v] : 0u;
  }
}

// Exclusive scan over a 256-thread workgroup; *total receives the sum.
__device__ inline uint32_t block_excl_scan_256(uint32_t x, uint32_t* s_w, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = (uint32_t)wave_incl_scan_i((int)x, 0, [](int u, int v) { return u + v; });
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  uint32_t base = 0u;
  for (int w = 0; w < wave; ++w) base += s_w[w];
  *total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
  return base + inc - x;
}

__global__ __launch_bounds__(256) void bwd_group_tile_sum_kernel(const uint32_t* cnt, uint32_t* tsum,
                                                                 int64_t n) {
  __shared__ uint32_t s_w[4];
  uint32_t c[16];
  load16_u32(cnt, (int64_t)blockIdx.x * kGroupTile + 16 * threadIdx.x, n, c);
  uint32_t x = 0u;
#pragma unroll
  for (int v = 0; v < 16; ++v) x += c[v];
  uint32_t total;
  block_excl_scan_256(x, s_w, &total);
  if (threadIdx.x == 0) tsum[blockIdx.x] = total;
}

// tsum[0..nt) -> its exclusive scan, in place; off[n] = the grand total.
__global__ __launch_bounds__(256) void bwd_group_tile_scan_kernel(uint32_t* tsum, int64_t nt,
                                                                  uint32_t* off, int64_t n) {
  __shared__ uint32_t s_w[4];
  uint32_t carry = 0u;
  for (int64_t i0 = 0; i0 < nt; i0 += 256) {
    const int64_t i = i0 + threadIdx.x;
    const uint32_t x = i < nt ? tsum[i] : 0u;
    uint32_t total;
    const uint32_t e = block_excl_scan_256(x, s_w, &total);
    if (i < nt) tsum[i] = carry + e;
    carry += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) off[n] = carry;
}

__global__ __launch_bounds__(256) void bwd_group_tile_offsets_kernel(uint32_t* cnt, uint32_t* off,
                                                                     const uint32_t* tsum, int64_t n) {
  __shared__ uint32_t s_w[4];
  uint32_t c[16];
  const int64_t i0 = (int64_t)blockIdx.x * kGroupTile + 16 * threadIdx.x;
  load16_u32(cnt, i0, n, c);
  uint32_t x = 0u;
#pragma unroll
  for (int v = 0; v < 16; ++v) x += c[v];
  uint32_t total;
  uint32_t run = tsum[blockIdx.x] + block_excl_scan_256(x, s_w, &total);
  if (i0 + 16 <= n) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint4 o;
      o.x = run; run += c[4 * v];
      o.y = run; run += c[4 * v + 1];
      o.z = run; run += c[4 * v + 2];
      o.w = run; run += c[4 * v + 3];
      *reinterpret_cast<uint4*>(off + i0 + 4 * v) = o;
      *reinterpret_cast<uint4*>(cnt + i0 + 4 * v) = uint4{0u, 0u, 0u, 0u};
    }
  } else {
    for (int v = 0; v < 16 && i0 + v < n; ++v) {
      off[i0 + v] = run;
      run += c[v];
      cnt[i0 + v] = 0u;
    }
  }
}

// list[off[d] ..] = the slots whose destination is d (in no fixed order).
__global__ __launch_bounds__(256) void bwd_group_scatter_kernel(const int32_t* dest, uint32_t* cnt,
                                                                const uint32_t* off, int32_t* list,
                                                                int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int32_t d = dest[i];
    if (d >= 0) list[off[d] + atomicAdd(cnt + d, 1u)] = (int32_t)i;
  }
}

// The sum of each destination row's slots (dense rows of D floats, D / 8
// lanes a row, 64 / (D / 8) rows a wave), added to row d of out1 (d < n1)
// or row d - n1 of out2.  Four slots' rows are in flight at a time; a group
// past the list re-reads the last slot and drops it.
template <int LPR, bool F24>
__global__ __launch_bounds__(256) void group_reduce_kernel(const float* dense, const int32_t* list,
                                                           const uint32_t* off, int64_t ndest, int D,
                                                           float* out1, int64_t n1, float* out2) {
  const int lane = threadIdx.x & 63;
  const int64_t d = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / LPR) + lane / LPR;
  if (d >= ndest) return;
  const int dd = 8 * (lane % LPR);
  const uint32_t o0 = off[d], o1 = off[d + 1];
  if (o0 == o1) return;
  f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;
  for (uint32_t o = o0; o < o1; o += 4) {
    f32x4 v0[4], v1[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t id = list[min(o + (uint32_t)u, o1 - 1u)];
      if constexpr (F24) {   // 8 values in six words (three 8-byte loads)
        const uint2* r = reinterpret_cast<const uint2*>(reinterpret_cast<const uint32_t*>(dense) +
                                                        id * (D / 4 * 3) + dd / 4 * 3);
        const uint2 a = r[0], b = r[1], c = r[2];
        float f[8];
        f24_unpack4(a.x, a.y, b.x, f);
        f24_unpack4(b.y, c.x, c.y, f + 4);
        v0[u] = f32x4{f[0], f[1], f[2], f[3]};
        v1[u] = f32x4{f[4], f[5], f[6], f[7]};
      } else {
        const float* r = dense + id * D + dd;
        v0[u] = *reinterpret_cast<const f32x4*>(r);
        v1[u] = *reinterpret_cast<const f32x4*>(r + 4);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (o + (uint32_t)u < o1) {
        s0 += v0[u];
        s1 += v1[u];
      }
  }
  float* t = d < n1 ? out1 + d * D + dd : out2 + (d - n1) * D + dd;
  f32x4* t4 = reinterpret_cast<f32x4*>(t);
  t4[0] = t4[0] + s0;
  t4[1] = t4[1] + s1;
}

// Buffers of a grouped sum: per-destination counts (zeroed before the
// group; the gather counts into them), offsets, tile sums and slot lists.
struct GroupBufs {
  int32_t* dest;
  int32_t* list;
  uint32_t* cnt;
  uint32_t* off;
  uint32_t* tsum;
  int64_t ndest;
};

uint8_t* group_layout(GroupBufs& gb, uint8_t* w, int64_t slots, int64_t ndest) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  gb.ndest = ndest;
  gb.dest = reinterpret_cast<int32_t*>(w);  w += al((size_t)slots * 4);
  gb.list = reinterpret_cast<int32_t*>(w);  w += al((size_t)slots * 4);
  gb.cnt = reinterpret_cast<uint32_t*>(w);  w += al((size_t)(ndest + 1) * 4);
  gb.off = reinterpret_cast<uint32_t*>(w);  w += al((size_t)(ndest + 1) * 4);
  gb.tsum = reinterpret_cast<uint32_t*>(w); w += al((size_t)((ndest + kGroupTile - 1) / kGroupTile) * 4);
  return w;
}

size_t group_bytes(int64_t slots, int64_t ndest) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  return 2 * al((size_t)slots * 4) + 2 * al((size_t)(ndest + 1) * 4) +
         al((size_t)((ndest + kGroupTile - 1) / kGroupTile) * 4);
}

hipError_t group_begin(const GroupBufs& gb, hipStream_t st) {
  bwd_fill_u32_kernel<<<256, 256, 0, st>>>(gb.cnt, gb.ndest + 1);
  return hipGetLastError();
}

// After a group of nslots slots: counts to offsets, the slots listed by
// destination, and each destination's sum added into its row.
hipError_t group_sum(const GroupBufs& gb, int64_t nslots, const float* dense, int D, bool f24,
                     float* out1, int64_t n1, float* out2, hipStream_t st) {
  const int64_t ntile = (gb.ndest + kGroupTile - 1) / kGroupTile;
  if (ntile == 0) return hipSuccess;
  bwd_group_tile_sum_kernel<<<(unsigned)ntile, 256, 0, st>>>(gb.cnt, gb.tsum, gb.ndest);
  bwd_group_tile_scan_kernel<<<1, 256, 0, st>>>(gb.tsum, ntile, gb.off, gb.ndest);
  bwd_group_tile_offsets_kernel<<<(unsigned)ntile, 256, 0, st>>>(gb.cnt, gb.off, gb.tsum, gb.ndest);
  const int64_t sb = (nslots + 255) / 256;
  bwd_group_scatter_kernel<<<(unsigned)(sb < 4096 ? sb : 4096), 256, 0, st>>>(gb.dest, gb.cnt, gb.off,
                                                                               gb.list, nslots);
  const int lpr = D / 8;
  const int64_t per_wg = 4 * (64 / lpr);
  const unsigned grid = (unsigned)((gb.ndest + per_wg - 1) / per_wg);
#define V4_GROUP_REDUCE(L)                                                                       \
  (f24 ? group_reduce_kernel<L, true><<<grid, 256, 0, st>>>(dense, gb.list, gb.off, gb.ndest, D, \
                                                             out1, n1, out2)                      \
       : group_reduce_kernel<L, false><<<grid, 256, 0, st>>>(dense, gb.list, gb.off, gb.ndest, D, \
                                                              out1, n1, out2))
  switch (lpr) {
    case 4: V4_GROUP_REDUCE(4); break;
    case 8: V4_GROUP_REDUCE(8); break;
    case 16: V4_GROUP_REDUCE(16); break;
    case 32: V4_GROUP_REDUCE(32); break;
    case 64: V4_GROUP_REDUCE(64); break;
    default: return hipErrorInvalidValue;
  }
#undef V4_GROUP_REDUCE
  return hipGetLastError();
}

}  // namespace

int64_t bwd_rows_padded(int64_t rows_max) { return (rows_max + 127) / 128 * 128; }

size_t bwd_query_bytes(int D, int64_t np) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  return al((size_t)np * D * 2)          // X
         + al((size_t)np * 8)            // rowmap
         + al((size_t)128 * D * 2)       // Y
         + al((size_t)D * 128 * 2)       // YT
         + al((size_t)64 * 4)            // Dh
         + al((size_t)64 * np * 2)       // T
         + al((size_t)np * 128 * 2)      // TT
         + al((size_t)64 * D * 4)        // dq~
         + al((size_t)D * 4)             // G
         + al((size_t)64 * 4);           // DS
}

size_t bwd_group_bytes(int D, int64_t np, int64_t gq, int64_t ndest) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  if (gq <= 0) return 0;
  return al((size_t)gq * np * D * 3) + group_bytes(gq * np, ndest);   // dense dX (24-bit), then the sort
}

hipError_t launch_attend_backward(BwdArgs a, int qchunk, int64_t gq, void* ws, hipStream_t st) {
  const int nq = a.B * a.Tq;
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  const int64_t np = a.np;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.X = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * np * a.D * 2);
  a.rowmap = reinterpret_cast<int64_t*>(w);    w += al((size_t)qchunk * np * 8);
  a.Y = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * 128 * a.D * 2);
  a.YT = reinterpret_cast<uint16_t*>(w);       w += al((size_t)qchunk * a.D * 128 * 2);
  a.Dh = reinterpret_cast<float*>(w);          w += al((size_t)qchunk * 64 * 4);
  a.T = reinterpret_cast<uint16_t*>(w);        w += al((size_t)qchunk * 64 * np * 2);
  a.TT = reinterpret_cast<uint16_t*>(w);       w += al((size_t)qchunk * np * 128 * 2);
  a.DQT = reinterpret_cast<float*>(w);       w += al((size_t)qchunk * 64 * a.D * 4);
  a.G = reinterpret_cast<float*>(w);         w += al((size_t)qchunk * a.D * 4);
  a.DS = reinterpret_cast<float*>(w);        w += al((size_t)qchunk * 64 * 4);
  a.dXd = nullptr;
  GroupBufs gb{};
  if (gq > 0) {
    a.dXd = reinterpret_cast<float*>(w);     w += al((size_t)gq * np * a.D * 3);   // 24-bit values
    group_layout(gb, w, gq * np, a.ndest);
    a.dest = gb.dest;
    a.cnt = gb.cnt;
  }
  const int64_t gstep = gq > 0 ? gq : nq;
  for (int64_t g0 = 0; g0 < nq; g0 += gstep) {
    const int64_t g1 = g0 + gstep < nq ? g0 + gstep : nq;
    if (gq > 0) {
      a.group_q0 = (int)g0;
      const hipError_t e = group_begin(gb, st);
      if (e != hipSuccess) return e;
    }
    for (int q0 = (int)g0; q0 < g1; q0 += qchunk) {
      const int qc = g1 - q0 < qchunk ? (int)(g1 - q0) : qchunk;
      bwd_gather_kernel<<<dim3((unsigned)((np + 4 * kGatherRows - 1) / (4 * kGatherRows)), qc), 256, 0,
                          st>>>(a, q0);
      bwd_prep_kernel<<<dim3(4, qc), 1024, 0, st>>>(a, q0);
      // [S; dP] = Y X^T (M = 128, N = np, K = D) and, from it, T = [scale dL; P]
      GemmArgs g1{};
      g1.a = a.Y; g1.lda = a.D; g1.a_batch = 128 * (int64_t)a.D;
      g1.b = a.X; g1.ldb = a.D; g1.b_batch = np * a.D;
      g1.K = a.D; g1.alpha = 1.f; g1.n_valid = (int)np;
      bwd_sdp_kernel<<<dim3((unsigned)(np / 128), 1, qc), 256, 0, st>>>(g1, a, q0);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      // dq~ = (scale dL) X: M = 64, N = D, K = np
      GemmArgs g2{};
      g2.a = a.T; g2.lda = np; g2.a_batch = 64 * np;
      g2.b = a.X; g2.ldb = a.D; g2.b_batch = np * a.D;
      g2.c = a.DQT; g2.ldc = a.D; g2.c_batch = 64 * (int64_t)a.D; g2.K = (int)np; g2.alpha = 1.f;
      g2.n_valid = a.D;
      e = gemm<false, false>(g2, 64, a.D, qc, st);
      if (e != hipSuccess) return e;
      // dX = T^T Y: M = np, N = D, K = 128; added into the row gradients
      // (atomics), or stored densely for the group's sum by destination
      GemmArgs g3{};
      g3.a = a.TT; g3.lda = 128; g3.a_batch = np * 128;
      g3.b = a.YT; g3.ldb = 128; g3.b_batch = (int64_t)a.D * 128;
      g3.ldc = a.D; g3.K = 128; g3.alpha = 1.f; g3.n_valid = a.D;
      if (a.dXd) {
        // 24-bit values: the chunk's first slot is 3 np D (q0 - g0) bytes in
        g3.c = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.dXd) +
                                        (size_t)(q0 - g0) * np * a.D * 3);
        g3.c_batch = np * a.D;
      } else {
        g3.c = a.d_entries; g3.c2 = a.d_win; g3.rowmap = a.rowmap; g3.rowmap_batch = np;
      }
      bwd_dx_kernel<<<dim3((unsigned)(a.D / 128), (unsigned)(np / 128), qc), 256, 0, st>>>(g3);
      bwd_q_kernel<<<qc, 1024, 0, st>>>(a, q0);
    }
    if (gq > 0) {
      const hipError_t e =
          group_sum(gb, (g1 - g0) * np, a.dXd, a.D, true, a.d_entries, a.nent, a.d_win, st);
      if (e != hipSuccess) return e;
    }
  }
  if (a.d_gamma_q || (a.sink && a.d_sink))
    bwd_reduce_kernel<<<(unsigned)((a.D + 255) / 256), 256, 0, st>>>(a, nq < qchunk ? nq : qchunk);
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

size_t kl_group_bytes(int dI, int64_t nsp, int64_t gq, int64_t ndest) {
  auto al = [](size_t n) { return (n + 255) / 256 * 256; };
  if (gq <= 0) return 0;
  return al((size_t)gq * nsp * dI * 3) + group_bytes(gq * nsp, ndest);   // dense dK (24-bit), then the sort
}

hipError_t launch_index_kl_backward(KlArgs a, int qchunk, int64_t gq, int64_t ndest, void* ws,
                                    hipStream_t st) {
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
  a.Sb = reinterpret_cast<float*>(w);      w += al((size_t)qchunk * nsp * 4);
  a.dKd = nullptr;
  GroupBufs gb{};
  if (gq > 0) {
    a.dKd = reinterpret_cast<float*>(w);     w += al((size_t)gq * nsp * a.dI * 3);   // 24-bit values
    group_layout(gb, w, gq * nsp, ndest);
    a.dest = gb.dest;
    a.cnt = gb.cnt;
  }
  const int64_t gstep = gq > 0 ? gq : nq;
  for (int64_t g0 = 0; g0 < nq; g0 += gstep) {
    const int64_t g1 = g0 + gstep < nq ? g0 + gstep : nq;
    if (gq > 0) {
      a.group_q0 = (int)g0;
      const hipError_t e = group_begin(gb, st);
      if (e != hipSuccess) return e;
    }
    for (int q0 = (int)g0; q0 < g1; q0 += qchunk) {
      const int qc = g1 - q0 < qchunk ? (int)(g1 - q0) : qchunk;
      const int64_t rpw = 2048 / a.dIp;   // key rows a gather workgroup
      const unsigned gx = (unsigned)((nsp + rpw - 1) / rpw > 16 ? (nsp + rpw - 1) / rpw : 16);
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
      // dK = G^T Qi: M = nsp, N = dIp (first dI kept), K = 64; stored densely
      // for the group's sum by destination, or added into dk rows (atomics)
      GemmArgs g3{};
      g3.a = a.Gm; g3.lda = nsp; g3.a_batch = 64 * nsp;
      g3.b = a.Qi; g3.ldb = a.dIp; g3.b_batch = 64 * (int64_t)a.dIp;
      g3.ldc = a.dI; g3.K = 64; g3.alpha = 1.f; g3.n_valid = a.dI;
      if (a.dKd) {   // 24-bit values: the chunk's first slot is 3 nsp dI (q0 - g0) bytes in
        g3.c = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a.dKd) +
                                        (size_t)(q0 - g0) * nsp * a.dI * 3);
        g3.c_batch = nsp * a.dI; g3.f24 = 1;
      } else {
        g3.c = a.dk; g3.rowmap = a.rowmap; g3.rowmap_batch = nsp;
      }
      e = gemm<true, false>(g3, (int)nsp, a.dIp, qc, st);
      if (e != hipSuccess) return e;
    }
    if (gq > 0) {
      const hipError_t e = group_sum(gb, (g1 - g0) * nsp, a.dKd, a.dI, true, a.dk, ndest, nullptr, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

}  // namespace v4
