// C ABI of libv4attn.so (declared in include/v4attn.h): argument validation,
// workspace layout and kernel launches.  Every check runs before any HIP call,
// so invalid calls return an error without touching the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/v4attn.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err.clear();
    return V4ATTN_OK;
  }
  return fail(V4ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxK = 4096;
constexpr int kMaxW = 4096;

int check_dr(int D, int R) {
  if (R != 64) return fail(V4ATTN_EUNSUPPORTED, "R = %d: only R = 64 rotary dims are built", R);
  if (D != 128 && D != 256 && D != 512)
    return fail(V4ATTN_EUNSUPPORTED, "D = %d: only D in {128, 256, 512} is built", D);
  return V4ATTN_OK;
}

int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Largest visible-entry count over queries q_pos0 .. q_pos0+Tq-1.
int64_t vmax_of(int Tq, int64_t n_entries, int64_t q_pos0, int m) {
  if (Tq <= 0) return 0;
  return min64(n_entries, (q_pos0 + Tq) / m);
}

// Per-sequence positions (host array, nullable): every p >= 0 and their
// largest equal to q_pos0, which sizes workspaces and is validated as
// before.  Passed to the kernels by value.
int load_seq_pos(const int64_t* seq_pos, int B, int64_t q_pos0, v4::SeqPos* sp, bool* ragged) {
  *ragged = seq_pos != nullptr;
  if (!seq_pos) return V4ATTN_OK;
  if (B > v4::kMaxRagged)
    return fail(V4ATTN_EUNSUPPORTED, "B = %d: per-sequence positions are built for B <= %d", B,
                v4::kMaxRagged);
  int64_t mx = -1;
  for (int b = 0; b < B; ++b) {
    if (seq_pos[b] < 0) return fail(V4ATTN_EINVAL, "negative position of sequence %d", b);
    sp->p[b] = seq_pos[b];
    mx = seq_pos[b] > mx ? seq_pos[b] : mx;
  }
  if (B > 0 && mx != q_pos0)
    return fail(V4ATTN_EINVAL, "q_pos0 %lld must be the largest sequence position (%lld)",
                (long long)q_pos0, (long long)mx);
  return V4ATTN_OK;
}

struct TopkWs {
  v4::TopkPlan plan;
  size_t part_bytes, cand_bytes, run_bytes, total;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

TopkWs topk_ws(int B, int Tq, int64_t n_entries, int64_t q_pos0, int m, int k) {
  TopkWs w;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  w.plan = v4::topk_plan(0, vmax, k);   // any row length up to vmax
  const int64_t rows = (int64_t)B * Tq;
  const int64_t np = w.plan.nparts;
  w.part_bytes = align256((size_t)(rows * np) * sizeof(int));
  w.cand_bytes = align256((size_t)(rows * np * v4::kTopkPartCap) * sizeof(int));
  w.run_bytes = align256((size_t)(rows * k) * sizeof(unsigned));
  // part thresholds, counts and overflow maxima, leader keys and indices,
  // partial-selection keys
  w.total = w.plan.parts ? 3 * w.part_bytes + 2 * w.cand_bytes + w.run_bytes : 0;
  return w;
}

struct IndexWs {
  int64_t score_stride;
  size_t scores_bytes, total;
  TopkWs tk;
};

IndexWs index_ws(int B, int Tq, int64_t n_entries, int64_t q_pos0, int m, int k) {
  IndexWs w;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  w.score_stride = (vmax + 63) / 64 * 64;
  const int64_t rows = (int64_t)B * Tq;
  w.scores_bytes = (size_t)(rows * w.score_stride) * sizeof(float);
  w.scores_bytes = (w.scores_bytes + 255) / 256 * 256;
  w.tk = topk_ws(B, Tq, n_entries, q_pos0, m, k);
  w.total = w.scores_bytes + w.tk.total;
  return w;
}

// Attention workspace (splits > 1): the split partials, O (signed
// normalised 16-bit integers with a power-of-two scale per split and head),
// then (max, sum, scale exponent, unused) in fp32.
size_t attend_o_bytes(int64_t q, int s, int H, int D) {
  return ((size_t)(q * s * H * D) * sizeof(uint16_t) + 255) / 256 * 256;
}

size_t attend_ws(int B, int Tq, int H, int D, int64_t rows_max, bool csa, int* splits) {
  const int s = v4::attend_splits(B, Tq, rows_max, csa);
  if (splits) *splits = s;
  if (s <= 1) return 0;
  const int64_t q = (int64_t)B * Tq;
  return attend_o_bytes(q, s, H, D) + (size_t)(q * s * H * 4) * sizeof(float);
}

// Points the kernel arguments at their parts of the workspace.
void attend_ws_layout(v4::AttendArgs& a, void* ws) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.part_o = reinterpret_cast<uint16_t*>(w);
  const size_t o_bytes = attend_o_bytes((int64_t)a.B * a.Tq, a.splits, a.H, a.D);
  a.part_ml = a.splits > 1 ? reinterpret_cast<float*>(w + o_bytes) : nullptr;
}

// Ragged decode batches (Tq = 1): each sequence gets its own split count
// (about the same tiles per workgroup everywhere) instead of the longest
// sequence's.  csa: rows = k + window rows; else visible entries + window.
void plan_ragged_attend(v4::AttendArgs& a, bool csa) {
  if (!a.ragged || a.Tq != 1 || a.B < 1) return;
  int64_t rows[v4::kMaxRagged];
  for (int b = 0; b < a.B; ++b) {
    const int64_t t = a.pos.p[b];
    const int64_t lo = t - a.W + 1 > 0 ? t - a.W + 1 : 0;
    const int64_t n_win = a.W > 0 ? t - lo + 1 : 0;
    const int64_t v = (t + 1) / a.m < a.n_entries ? (t + 1) / a.m : a.n_entries;
    rows[b] = (csa ? (int64_t)a.k : v) + n_win;
  }
  v4::plan_flat_splits(a, rows, csa);
}

// need_sink: the call takes a per-head sink (every attention call but the
// NSA-style variant, whose branches have none).
int check_attend_common(const uint16_t* q, const uint8_t* entries, const uint8_t* win,
                        const float* gamma_q, const float* sink, int B, int Tq, int H, int D,
                        int R, int64_t Ncap, int W, int64_t q_pos0, float scale, float eps,
                        float rope_base, const uint16_t* out, bool need_sink = true) {
  if (!q || !gamma_q || (need_sink && !sink) || !out)
    return fail(V4ATTN_EINVAL, "null q, gamma_q, sink or out");
  if (B < 0 || Tq < 0) return fail(V4ATTN_EINVAL, "negative B or Tq");
  if (int st = check_dr(D, R)) return st;
  if (H < 1 || H > 64) return fail(V4ATTN_EUNSUPPORTED, "H = %d: 1 <= H <= 64 is built", H);
  if (Ncap < 0) return fail(V4ATTN_EINVAL, "negative Ncap");
  if (Ncap * (int64_t)(D + R) >= ((int64_t)1 << 32))
    return fail(V4ATTN_EUNSUPPORTED, "one sequence's entry cache must be below 4 GiB");
  if (W < 0 || W > kMaxW) return fail(V4ATTN_EUNSUPPORTED, "W = %d: 0 <= W <= %d", W, kMaxW);
  if (q_pos0 < 0) return fail(V4ATTN_EINVAL, "negative q_pos0");
  if (W > 0 && !win) return fail(V4ATTN_EINVAL, "null window buffer with W > 0");
  if (Ncap > 0 && !entries) return fail(V4ATTN_EINVAL, "null entries with Ncap > 0");
  if (!std::isfinite(scale) || !(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f))
    return fail(V4ATTN_EINVAL, "bad scale, eps or rope_base");
  if (!aligned16(q) || !aligned16(entries) || !aligned16(win) || !aligned16(out) ||
      !aligned16(gamma_q))
    return fail(V4ATTN_EINVAL, "q, entries, win, gamma_q and out must be 16-byte aligned");
  return V4ATTN_OK;
}

}  // namespace

extern "C" {

int v4attn_version(void) { return (0 << 16) | 1; }

const char* v4attn_status_string(int status) {
  switch (status) {
    case V4ATTN_OK: return "ok";
    case V4ATTN_EINVAL: return "invalid argument";
    case V4ATTN_EUNSUPPORTED: return "unsupported size";
    case V4ATTN_EWORKSPACE: return "workspace missing or too small";
    case V4ATTN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* v4attn_last_error(void) { return g_err.c_str(); }

int v4attn_compress(const uint16_t* raw, const float* tok_score, const float* pos_bias,
                    const float* gamma, int B, int L, int D, int R, int64_t raw_pos0, int mode,
                    int m, int64_t entry0, int n_out, float eps, float rope_base, uint8_t* out,
                    int64_t out_rows, const uint16_t* raw_idx, int dI, uint16_t* k_idx_out,
                    void* stream) {
  if (!raw || !gamma || !out) return fail(V4ATTN_EINVAL, "null raw, gamma or out");
  if (B < 0 || L < 0 || n_out < 0 || out_rows < 0)
    return fail(V4ATTN_EINVAL, "negative B, L, n_out or out_rows");
  if (int st = check_dr(D, R)) return st;
  if (mode != V4ATTN_POOL && mode != V4ATTN_PACK) return fail(V4ATTN_EINVAL, "bad mode %d", mode);
  if (n_out > out_rows) return fail(V4ATTN_EINVAL, "n_out %d > out_rows %lld", n_out, (long long)out_rows);
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f))
    return fail(V4ATTN_EINVAL, "bad eps or rope_base");
  if (!aligned16(raw) || !aligned16(out)) return fail(V4ATTN_EINVAL, "raw and out must be 16-byte aligned");
  if (mode == V4ATTN_POOL) {
    if (!tok_score || !pos_bias) return fail(V4ATTN_EINVAL, "POOL needs tok_score and pos_bias");
    if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
    if (entry0 < 0) return fail(V4ATTN_EINVAL, "negative entry0");
    if (n_out > 0) {
      const int64_t lo = (entry0 - 1) * (int64_t)m;
      const int64_t first = lo > 0 ? lo : 0;
      const int64_t last = (entry0 + n_out) * (int64_t)m;  // exclusive end of the last window
      if (first < raw_pos0 || last > raw_pos0 + L)
        return fail(V4ATTN_EINVAL,
                    "entries %lld..%lld need positions [%lld, %lld) but rows hold [%lld, %lld)",
                    (long long)entry0, (long long)(entry0 + n_out - 1), (long long)first,
                    (long long)last, (long long)raw_pos0, (long long)(raw_pos0 + L));
    }
  } else {
    if (n_out > L) return fail(V4ATTN_EINVAL, "PACK n_out %d > L %d", n_out, L);
  }
  if (raw_idx && (!k_idx_out || (dI != 32 && dI != 64 && dI != 128)))
    return fail(V4ATTN_EINVAL, "indexer keys need k_idx_out and dI in {32, 64, 128}");
  v4::CompressArgs a{raw, tok_score, pos_bias, gamma, B, L, D, R, raw_pos0, mode, m, entry0,
                     n_out, eps, rope_base, out, out_rows, v4::rope_turns(rope_base, R),
                     mode == V4ATTN_POOL ? raw_idx : nullptr, dI,
                     mode == V4ATTN_POOL && raw_idx ? k_idx_out : nullptr};
  return hip_status(v4::launch_compress(a, (hipStream_t)stream), "compress launch");
}

}  // extern "C"

namespace {

// Validates one layer's decode-step arguments and fills the kernel's.
int step_args(const uint16_t* raw, const float* tok_score, const float* pos_bias,
              const float* gamma, int B, int L, int D, int R, int64_t raw_pos0, int m, int64_t t,
              const int64_t* seq_pos, float eps, float rope_base, uint8_t* entries,
              int64_t ent_rows, uint8_t* win, int64_t win_rows, int64_t win_row,
              const uint16_t* raw_idx, int dI, uint16_t* k_idx, v4::CompressStepArgs* out) {
  if (!raw || !gamma || !win) return fail(V4ATTN_EINVAL, "null raw, gamma or win");
  if (B < 0 || L < 0 || ent_rows < 0 || win_rows < 0)
    return fail(V4ATTN_EINVAL, "negative B, L, ent_rows or win_rows");
  if (int st = check_dr(D, R)) return st;
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f))
    return fail(V4ATTN_EINVAL, "bad eps or rope_base");
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, t, &sp, &ragged)) return st;
  if (win_row < 0 || win_row >= win_rows)
    return fail(V4ATTN_EINVAL, "win_row %lld outside [0, %lld)", (long long)win_row,
                (long long)win_rows);
  if (!aligned16(raw) || !aligned16(win)) return fail(V4ATTN_EINVAL, "raw and win must be 16-byte aligned");
  // every sequence's token (with per-sequence positions its raw rows are the
  // L positions ending at it)
  for (int b = 0; b < (ragged ? B : 1); ++b) {
    const int64_t tb = ragged ? sp.p[b] : t;
    const int64_t p0 = ragged ? tb - L + 1 : raw_pos0;
    if (tb < 0 || tb < p0 || tb >= p0 + L)
      return fail(V4ATTN_EINVAL, "position %lld is not in the raw rows [%lld, %lld)", (long long)tb,
                  (long long)p0, (long long)(p0 + L));
    if ((tb + 1) % m != 0) continue;
    const int64_t j = (tb + 1) / m - 1;
    const int64_t lo = (j - 1) * (int64_t)m;
    const int64_t first = lo > 0 ? lo : 0;
    if (!tok_score || !pos_bias || !entries)
      return fail(V4ATTN_EINVAL, "a completed entry needs tok_score, pos_bias and entries");
    if (!aligned16(entries)) return fail(V4ATTN_EINVAL, "entries must be 16-byte aligned");
    if (j >= ent_rows)
      return fail(V4ATTN_EINVAL, "entry %lld outside %lld entry rows", (long long)j, (long long)ent_rows);
    if (first < p0)
      return fail(V4ATTN_EINVAL, "entry %lld needs positions from %lld but rows start at %lld",
                  (long long)j, (long long)first, (long long)p0);
  }
  v4::CompressStepArgs a{raw, tok_score, pos_bias, gamma, B, L, D, R, raw_pos0, m, t, eps,
                         v4::rope_turns(rope_base, R), entries, ent_rows, win, win_rows, win_row};
  a.ragged = ragged;
  if (ragged) a.pos = sp;
  if (raw_idx && (!k_idx || (dI != 32 && dI != 64 && dI != 128)))
    return fail(V4ATTN_EINVAL, "indexer keys need k_idx and dI in {32, 64, 128}");
  a.raw_idx = raw_idx;
  a.dI = dI;
  a.kidx = raw_idx ? k_idx : nullptr;
  *out = a;
  return V4ATTN_OK;
}

}  // namespace

extern "C" {

int v4attn_compress_step(const uint16_t* raw, const float* tok_score, const float* pos_bias,
                         const float* gamma, int B, int L, int D, int R, int64_t raw_pos0, int m,
                         int64_t t, const int64_t* seq_pos, float eps, float rope_base,
                         uint8_t* entries, int64_t ent_rows, uint8_t* win, int64_t win_rows,
                         int64_t win_row, const uint16_t* raw_idx, int dI, uint16_t* k_idx,
                         void* stream) {
  v4::CompressStepArgs a;
  if (int st = step_args(raw, tok_score, pos_bias, gamma, B, L, D, R, raw_pos0, m, t, seq_pos, eps,
                         rope_base, entries, ent_rows, win, win_rows, win_row, raw_idx, dI, k_idx,
                         &a))
    return st;
  return hip_status(v4::launch_compress_step(a, (hipStream_t)stream), "compress step launch");
}

int v4attn_compress_steps(const v4attn_compress_step_desc* steps, int n, void* stream) {
  if (!steps) return fail(V4ATTN_EINVAL, "null steps");
  if (n < 1 || n > v4::kMaxSteps)
    return fail(V4ATTN_EUNSUPPORTED, "n = %d: 1 <= n <= %d layers are built", n, v4::kMaxSteps);
  v4::CompressStepArgs a[v4::kMaxSteps];
  for (int z = 0; z < n; ++z) {
    const v4attn_compress_step_desc& d = steps[z];
    if (int st = step_args(d.raw, d.tok_score, d.pos_bias, d.gamma, d.B, d.L, d.D, d.R,
                           d.raw_pos0, d.m, d.t, d.seq_pos, d.eps, d.rope_base, d.entries,
                           d.ent_rows, d.win, d.win_rows, d.win_row, d.raw_idx, d.dI, d.k_idx,
                           &a[z]))
      return st;
    if (d.D != steps[0].D) return fail(V4ATTN_EUNSUPPORTED, "every layer of one call needs the same D");
  }
  return hip_status(v4::launch_compress_steps(a, n, (hipStream_t)stream), "compress steps launch");
}

size_t v4attn_index_topk_workspace(int B, int Tq, int64_t n_entries, int64_t q_pos0, int m,
                                   int k) {
  if (B < 0 || Tq < 0 || n_entries < 0 || q_pos0 < 0 || m < 1 || k < 1) return 0;
  return index_ws(B, Tq, n_entries, q_pos0, m, k).total;
}

size_t v4attn_topk_select_workspace(int B, int Tq, int64_t n_entries, int64_t q_pos0, int m,
                                    int k) {
  if (B < 0 || Tq < 0 || n_entries < 0 || q_pos0 < 0 || m < 1 || k < 1) return 0;
  return topk_ws(B, Tq, n_entries, q_pos0, m, k).total;
}

namespace {

// The selector keeps one offset per 1024-entry part of a row in LDS.
int check_topk_len(int Tq, int64_t n_entries, int64_t q_pos0, int m) {
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  const int64_t lim = (int64_t)v4::kTopkMaxParts * v4::kTopkPartLen;
  if (vmax > lim)
    return fail(V4ATTN_EUNSUPPORTED, "%lld visible entries: at most %lld per query are built",
                (long long)vmax, (long long)lim);
  return V4ATTN_OK;
}

int check_index_common(int B, int Tq, int64_t n_entries, int64_t q_pos0, int m) {
  if (B < 0 || Tq < 0) return fail(V4ATTN_EINVAL, "negative B or Tq");
  if (n_entries < 0) return fail(V4ATTN_EINVAL, "negative n_entries");
  if (n_entries >= (int64_t)1 << 31) return fail(V4ATTN_EUNSUPPORTED, "n_entries >= 2^31");
  if (q_pos0 < 0) return fail(V4ATTN_EINVAL, "negative q_pos0");
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  return V4ATTN_OK;
}

int check_score_args(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx, int B,
                     int Tq, int HI, int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                     int m) {
  if (!q_idx || !w_idx) return fail(V4ATTN_EINVAL, "null q_idx or w_idx");
  if (int st = check_index_common(B, Tq, n_entries, q_pos0, m)) return st;
  if (HI < 1 || HI > 64) return fail(V4ATTN_EUNSUPPORTED, "HI = %d: 1 <= HI <= 64 is built", HI);
  if (dI != 32 && dI != 64 && dI != 128)
    return fail(V4ATTN_EUNSUPPORTED, "dI = %d: dI in {32, 64, 128} is built", dI);
  if (Ncap < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (n_entries > 0 && !k_idx) return fail(V4ATTN_EINVAL, "null k_idx");
  if (!aligned16(q_idx) || !aligned16(k_idx))
    return fail(V4ATTN_EINVAL, "q_idx and k_idx must be 16-byte aligned");
  return V4ATTN_OK;
}

hipError_t run_score(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx, int B,
                     int Tq, int HI, int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                     int m, float* scores, int64_t stride, const v4::SeqPos* sp, hipStream_t st) {
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  v4::IndexScoreArgs ia{q_idx, w_idx, k_idx, B, Tq, HI, dI, Ncap, n_entries, q_pos0, m,
                        vmax, scores, stride, v4::index_row_waves(B, Tq, vmax)};
  ia.ragged = sp != nullptr;
  if (sp) {
    ia.pos = *sp;
    if (Tq == 1) {
      // workgroups in proportion to each sequence's visible entries (the
      // launch's total as for B rows of the longest), whole multiples of 4 waves
      int64_t tot = 0, vis[v4::kMaxRagged];
      for (int b = 0; b < B; ++b) {
        const int64_t v = min64(n_entries, (sp->p[b] + 1) / m);
        vis[b] = v;
        tot += v;
      }
      const int64_t budget = (int64_t)B * (ia.row_waves / 4);
      int acc = 0;
      for (int b = 0; b < B; ++b) {
        ia.wg_start[b] = acc;
        int64_t n = tot > 0 ? (budget * vis[b] + tot - 1) / tot : 1;
        const int64_t need = (vis[b] + 127) / 128;   // at least one chunk per wave
        if (n > need) n = need;
        if (n < 1) n = 1;
        acc += (int)n;
      }
      ia.wg_start[B] = acc;
    }
  }
  return v4::launch_index_score(ia, st);
}

hipError_t run_topk(const float* scores, int64_t stride, int B, int Tq, int64_t n_entries,
                    int64_t q_pos0, int m, int k, int32_t* topk, float* topk_score, void* ws,
                    const TopkWs& w, hipStream_t st, const v4::SeqPos* sp = nullptr) {
  uint8_t* cb = static_cast<uint8_t*>(ws);
  v4::TopkArgs ta;
  ta.ragged = sp != nullptr;
  if (sp) ta.pos = *sp;
  ta.scores = scores;
  ta.score_stride = stride;
  ta.B = B;
  ta.Tq = Tq;
  ta.n_entries = n_entries;
  ta.q_pos0 = q_pos0;
  ta.m = m;
  ta.k = k;
  // the launch's own rows: visible counts from the first query of the
  // earliest sequence to vmax (part slots at most the workspace's)
  int64_t vmin = min64(n_entries, (q_pos0 + 1) / m);
  if (sp)
    for (int b = 0; b < B; ++b) vmin = std::min(vmin, min64(n_entries, (sp->p[b] + 1) / m));
  const v4::TopkPlan plan = v4::topk_plan(vmin, vmax_of(Tq, n_entries, q_pos0, m), k);
  ta.direct_max = plan.direct_max;
  ta.nparts = plan.nparts;
  ta.part_tau = ta.part_over = nullptr;
  ta.part_cnt = nullptr;
  ta.cand_key = ta.run_key = nullptr;
  ta.cand_idx = nullptr;
  if (w.plan.parts) {
    ta.part_tau = reinterpret_cast<unsigned*>(cb);
    ta.part_cnt = reinterpret_cast<int*>(cb + w.part_bytes);
    ta.part_over = reinterpret_cast<unsigned*>(cb + 2 * w.part_bytes);
    uint8_t* c2 = cb + 3 * w.part_bytes;
    ta.cand_key = reinterpret_cast<unsigned*>(c2);
    ta.cand_idx = reinterpret_cast<int*>(c2 + w.cand_bytes);
    ta.run_key = reinterpret_cast<unsigned*>(c2 + 2 * w.cand_bytes);
  }
  ta.topk = topk;
  ta.topk_score = topk_score;
  return v4::launch_topk(ta, plan, st);
}

int check_score_fp8_args(const uint8_t* q8, const float* q_scale, const float* w_idx,
                         const uint8_t* k8, const float* k_scale, int B, int Tq, int HI, int dI,
                         int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m) {
  if (!q8 || !q_scale || !w_idx) return fail(V4ATTN_EINVAL, "null q8, q_scale or w_idx");
  if (int st = check_index_common(B, Tq, n_entries, q_pos0, m)) return st;
  if (HI < 1 || HI > 64) return fail(V4ATTN_EUNSUPPORTED, "HI = %d: 1 <= HI <= 64 is built", HI);
  if (dI != 64 && dI != 128)
    return fail(V4ATTN_EUNSUPPORTED, "dI = %d: the FP8 indexer builds dI in {64, 128}", dI);
  if (Ncap < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (n_entries > 0 && (!k8 || !k_scale)) return fail(V4ATTN_EINVAL, "null k8 or k_scale");
  if (!aligned16(q8) || !aligned16(k8)) return fail(V4ATTN_EINVAL, "q8 and k8 must be 16-byte aligned");
  return V4ATTN_OK;
}

hipError_t run_score_fp8(const uint8_t* q8, const float* q_scale, const float* w_idx,
                         const uint8_t* k8, const float* k_scale, int B, int Tq, int HI, int dI,
                         int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m, float* scores,
                         int64_t stride, hipStream_t st) {
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  v4::IndexScoreFp8Args ia{q8, q_scale, w_idx, k8, k_scale, B, Tq, HI, dI, Ncap, n_entries,
                           q_pos0, m, vmax, scores, stride, v4::index_fp8_row_waves(B, Tq, vmax)};
  return v4::launch_index_score_fp8(ia, st);
}

int check_score_mxfp4_args(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                           const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI, int dI,
                           int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m) {
  if (!q4 || !q_sc || !w_idx) return fail(V4ATTN_EINVAL, "null q4, q_sc or w_idx");
  if (int st = check_index_common(B, Tq, n_entries, q_pos0, m)) return st;
  if (HI < 1 || HI > 64) return fail(V4ATTN_EUNSUPPORTED, "HI = %d: 1 <= HI <= 64 is built", HI);
  if (dI != 64 && dI != 128)
    return fail(V4ATTN_EUNSUPPORTED, "dI = %d: the MXFP4 indexer builds dI in {64, 128}", dI);
  if (Ncap < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (n_entries > 0 && (!k4 || !k_sc)) return fail(V4ATTN_EINVAL, "null k4 or k_sc");
  if (!aligned16(q4) || !aligned16(k4)) return fail(V4ATTN_EINVAL, "q4 and k4 must be 16-byte aligned");
  if (((uintptr_t)k_sc) % (dI / 32) != 0)
    return fail(V4ATTN_EINVAL, "k_sc must be %d-byte aligned", dI / 32);
  return V4ATTN_OK;
}

hipError_t run_score_mxfp4(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                           const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI, int dI,
                           int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m, float* scores,
                           int64_t stride, hipStream_t st) {
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  v4::IndexScoreMxfp4Args ia{q4, q_sc, w_idx, k4, k_sc, B, Tq, HI, dI, Ncap, n_entries,
                             q_pos0, m, vmax, scores, stride, v4::index_mxfp4_row_waves(B, Tq, vmax)};
  return v4::launch_index_score_mxfp4(ia, st);
}

}  // namespace

int v4attn_index_score(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx, int B,
                       int Tq, int HI, int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                       const int64_t* seq_pos, int m, float* scores, int64_t score_stride,
                       void* stream) {
  if (int st = check_score_args(q_idx, w_idx, k_idx, B, Tq, HI, dI, Ncap, n_entries, q_pos0, m))
    return st;
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, q_pos0, &sp, &ragged)) return st;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  if (vmax > 0 && (!scores || score_stride < vmax))
    return fail(V4ATTN_EINVAL, "scores missing or score_stride %lld < %lld",
                (long long)score_stride, (long long)vmax);
  return hip_status(run_score(q_idx, w_idx, k_idx, B, Tq, HI, dI, Ncap, n_entries, q_pos0, m,
                              scores, score_stride, ragged ? &sp : nullptr, (hipStream_t)stream),
                    "index score launch");
}

int v4attn_topk_select(const float* scores, int64_t score_stride, int B, int Tq,
                       int64_t n_entries, int64_t q_pos0, const int64_t* seq_pos, int m, int k,
                       int32_t* topk, float* topk_score, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (int st = check_index_common(B, Tq, n_entries, q_pos0, m)) return st;
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, q_pos0, &sp, &ragged)) return st;
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  if (int st = check_topk_len(Tq, n_entries, q_pos0, m)) return st;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  if (vmax > 0 && (!scores || score_stride < vmax))
    return fail(V4ATTN_EINVAL, "scores missing or score_stride %lld < %lld",
                (long long)score_stride, (long long)vmax);
  const TopkWs w = topk_ws(B, Tq, n_entries, q_pos0, m, k);
  if (w.total > 0 && (!ws || ws_bytes < w.total))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  if ((int64_t)B * Tq == 0) return hip_status(hipSuccess, "");
  return hip_status(run_topk(scores, score_stride, B, Tq, n_entries, q_pos0, m, k, topk,
                             topk_score, ws, w, (hipStream_t)stream, ragged ? &sp : nullptr),
                    "top-k launch");
}

int v4attn_index_topk(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx, int B,
                      int Tq, int HI, int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                      const int64_t* seq_pos, int m, int k, int32_t* topk, float* topk_score,
                      void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_score_args(q_idx, w_idx, k_idx, B, Tq, HI, dI, Ncap, n_entries, q_pos0, m))
    return st;
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, q_pos0, &sp, &ragged)) return st;
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  if (int st = check_topk_len(Tq, n_entries, q_pos0, m)) return st;
  const IndexWs w = index_ws(B, Tq, n_entries, q_pos0, m, k);
  if (w.total > 0 && (!ws || ws_bytes < w.total))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  if ((int64_t)B * Tq == 0) return hip_status(hipSuccess, "");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(base);
  hipError_t e = run_score(q_idx, w_idx, k_idx, B, Tq, HI, dI, Ncap, n_entries, q_pos0, m,
                           scores, w.score_stride, ragged ? &sp : nullptr, st);
  if (e != hipSuccess) return hip_status(e, "index score launch");
  return hip_status(run_topk(scores, w.score_stride, B, Tq, n_entries, q_pos0, m, k, topk,
                             topk_score, base + w.scores_bytes, w.tk, st, ragged ? &sp : nullptr),
                    "top-k launch");
}

int v4attn_index_score_fp8(const uint8_t* q8, const float* q_scale, const float* w_idx,
                           const uint8_t* k8, const float* k_scale, int B, int Tq, int HI, int dI,
                           int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m, float* scores,
                           int64_t score_stride, void* stream) {
  if (int st = check_score_fp8_args(q8, q_scale, w_idx, k8, k_scale, B, Tq, HI, dI, Ncap,
                                    n_entries, q_pos0, m))
    return st;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  if (vmax > 0 && (!scores || score_stride < vmax))
    return fail(V4ATTN_EINVAL, "scores missing or score_stride %lld < %lld",
                (long long)score_stride, (long long)vmax);
  return hip_status(run_score_fp8(q8, q_scale, w_idx, k8, k_scale, B, Tq, HI, dI, Ncap,
                                  n_entries, q_pos0, m, scores, score_stride, (hipStream_t)stream),
                    "FP8 index score launch");
}

int v4attn_index_topk_fp8(const uint8_t* q8, const float* q_scale, const float* w_idx,
                          const uint8_t* k8, const float* k_scale, int B, int Tq, int HI, int dI,
                          int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m, int k,
                          int32_t* topk, float* topk_score, void* ws, size_t ws_bytes,
                          void* stream) {
  if (int st = check_score_fp8_args(q8, q_scale, w_idx, k8, k_scale, B, Tq, HI, dI, Ncap,
                                    n_entries, q_pos0, m))
    return st;
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  if (int st = check_topk_len(Tq, n_entries, q_pos0, m)) return st;
  const IndexWs w = index_ws(B, Tq, n_entries, q_pos0, m, k);
  if (w.total > 0 && (!ws || ws_bytes < w.total))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  if ((int64_t)B * Tq == 0) return hip_status(hipSuccess, "");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(base);
  hipError_t e = run_score_fp8(q8, q_scale, w_idx, k8, k_scale, B, Tq, HI, dI, Ncap, n_entries,
                               q_pos0, m, scores, w.score_stride, st);
  if (e != hipSuccess) return hip_status(e, "FP8 index score launch");
  return hip_status(run_topk(scores, w.score_stride, B, Tq, n_entries, q_pos0, m, k, topk,
                             topk_score, base + w.scores_bytes, w.tk, st),
                    "top-k launch");
}

int v4attn_index_score_mxfp4(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                             const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI,
                             int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m,
                             float* scores, int64_t score_stride, void* stream) {
  if (int st = check_score_mxfp4_args(q4, q_sc, w_idx, k4, k_sc, B, Tq, HI, dI, Ncap, n_entries,
                                      q_pos0, m))
    return st;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  if (vmax > 0 && (!scores || score_stride < vmax))
    return fail(V4ATTN_EINVAL, "scores missing or score_stride %lld < %lld",
                (long long)score_stride, (long long)vmax);
  return hip_status(run_score_mxfp4(q4, q_sc, w_idx, k4, k_sc, B, Tq, HI, dI, Ncap, n_entries,
                                    q_pos0, m, scores, score_stride, (hipStream_t)stream),
                    "MXFP4 index score launch");
}

int v4attn_index_topk_mxfp4(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                            const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI, int dI,
                            int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m, int k,
                            int32_t* topk, float* topk_score, void* ws, size_t ws_bytes,
                            void* stream) {
  if (int st = check_score_mxfp4_args(q4, q_sc, w_idx, k4, k_sc, B, Tq, HI, dI, Ncap, n_entries,
                                      q_pos0, m))
    return st;
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  if (int st = check_topk_len(Tq, n_entries, q_pos0, m)) return st;
  const IndexWs w = index_ws(B, Tq, n_entries, q_pos0, m, k);
  if (w.total > 0 && (!ws || ws_bytes < w.total))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  if ((int64_t)B * Tq == 0) return hip_status(hipSuccess, "");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* scores = reinterpret_cast<float*>(base);
  hipError_t e = run_score_mxfp4(q4, q_sc, w_idx, k4, k_sc, B, Tq, HI, dI, Ncap, n_entries,
                                 q_pos0, m, scores, w.score_stride, st);
  if (e != hipSuccess) return hip_status(e, "MXFP4 index score launch");
  return hip_status(run_topk(scores, w.score_stride, B, Tq, n_entries, q_pos0, m, k, topk,
                             topk_score, base + w.scores_bytes, w.tk, st),
                    "top-k launch");
}

size_t v4attn_csa_attend_workspace(int B, int Tq, int H, int D, int k, int W) {
  if (B < 0 || Tq < 0 || H < 1 || D < 1 || k < 1 || W < 0) return 0;
  return attend_ws(B, Tq, H, D, (int64_t)k + W, true, nullptr);
}

int v4attn_csa_attend(const uint16_t* q, const uint8_t* entries, const int32_t* topk,
                      const uint8_t* win, const float* gamma_q, const float* sink, int B, int Tq,
                      int H, int D, int R, int64_t Ncap, int k, int W, int64_t q_pos0,
                      const int64_t* seq_pos, float scale, float eps, float rope_base,
                      uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_attend_common(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, W,
                                   q_pos0, scale, eps, rope_base, out))
    return st;
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, q_pos0, &sp, &ragged)) return st;
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  int splits = 1;
  const size_t need = attend_ws(B, Tq, H, D, (int64_t)k + W, true, &splits);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  v4::AttendArgs a{};
  a.q = q; a.entries = entries; a.topk = topk; a.win = win; a.gamma_q = gamma_q; a.sink = sink;
  a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = R; a.Ncap = Ncap; a.k = k; a.n_entries = 0;
  a.m = 1; a.W = W; a.q_pos0 = q_pos0; a.scale = scale; a.eps = eps; a.rope_base = rope_base;
  a.rope = v4::rope_turns(rope_base, R);
  a.out = out; a.lse = lse; a.splits = splits;
  attend_ws_layout(a, ws);
  a.rows_max = (int64_t)k + W;
  a.ragged = ragged;
  if (ragged) a.pos = sp;
  plan_ragged_attend(a, true);
  return hip_status(v4::launch_attend(a, (hipStream_t)stream), "CSA attend launch");
}

}  // extern "C"

// The fixed device scratch of v4attn_hca_attend_noalloc: the split partials
// go here instead of into a caller's workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, so the device address of each GPU's copy is
// looked up once (with that GPU current) and only that address is used.
static __device__ __align__(256) uint8_t scratch[V4ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

// Validates an HCA attention call and fills its kernel arguments (all but
// the workspace views); *need = the split partials' bytes.
int hca_attend_args(const uint16_t* q, const uint8_t* entries, const uint8_t* win,
                    const float* gamma_q, const float* sink, int B, int Tq, int H, int D, int R,
                    int64_t Ncap, int64_t n_entries, int m, int W, int64_t q_pos0,
                    const int64_t* seq_pos, float scale, float eps, float rope_base,
                    uint16_t* out, float* lse, v4::AttendArgs* ap, size_t* need) {
  if (int st = check_attend_common(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, W,
                                   q_pos0, scale, eps, rope_base, out))
    return st;
  v4::SeqPos sp;
  bool ragged;
  if (int st = load_seq_pos(seq_pos, B, q_pos0, &sp, &ragged)) return st;
  if (n_entries < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  const int64_t rows_max = vmax_of(Tq, n_entries, q_pos0, m) + W;
  int splits = 1;
  *need = attend_ws(B, Tq, H, D, rows_max, false, &splits);
  v4::AttendArgs& a = *ap;
  a.q = q; a.entries = entries; a.topk = nullptr; a.win = win; a.gamma_q = gamma_q; a.sink = sink;
  a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = R; a.Ncap = Ncap; a.k = 0; a.n_entries = n_entries;
  a.m = m; a.W = W; a.q_pos0 = q_pos0; a.scale = scale; a.eps = eps; a.rope_base = rope_base;
  a.rope = v4::rope_turns(rope_base, R);
  a.out = out; a.lse = lse; a.splits = splits;
  a.rows_max = rows_max;
  a.ragged = ragged;
  if (ragged) a.pos = sp;
  plan_ragged_attend(a, false);
  return V4ATTN_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the scratch on the stream's device.
int scratch_of_stream_device(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(V4ATTN_EUNSUPPORTED, "device %d: devices 0..%d are supported", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) return hip_status(e2, "hipSetDevice");
    }
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(V4ATTN_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return V4ATTN_OK;
}

}  // namespace

extern "C" {

size_t v4attn_hca_attend_workspace(int B, int Tq, int H, int D, int64_t n_entries, int m,
                                   int64_t q_pos0, int W) {
  if (B < 0 || Tq < 0 || H < 1 || D < 1 || n_entries < 0 || m < 1 || q_pos0 < 0 || W < 0) return 0;
  return attend_ws(B, Tq, H, D, vmax_of(Tq, n_entries, q_pos0, m) + W, false, nullptr);
}

int v4attn_hca_attend(const uint16_t* q, const uint8_t* entries, const uint8_t* win,
                      const float* gamma_q, const float* sink, int B, int Tq, int H, int D, int R,
                      int64_t Ncap, int64_t n_entries, int m, int W, int64_t q_pos0,
                      const int64_t* seq_pos, float scale, float eps, float rope_base,
                      uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  v4::AttendArgs a{};
  size_t need = 0;
  if (int st = hca_attend_args(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, n_entries, m,
                               W, q_pos0, seq_pos, scale, eps, rope_base, out, lse, &a, &need))
    return st;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  attend_ws_layout(a, ws);
  return hip_status(v4::launch_attend(a, (hipStream_t)stream), "HCA attend launch");
}

int v4attn_hca_attend_noalloc(const uint16_t* q, const uint8_t* entries, const uint8_t* win,
                              const float* gamma_q, const float* sink, int B, int Tq, int H, int D,
                              int R, int64_t Ncap, int64_t n_entries, int m, int W, int64_t q_pos0,
                              const int64_t* seq_pos, float scale, float eps, float rope_base,
                              uint16_t* out, float* lse, void* stream) {
  v4::AttendArgs a{};
  size_t need = 0;
  if (int st = hca_attend_args(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, n_entries, m,
                               W, q_pos0, seq_pos, scale, eps, rope_base, out, lse, &a, &need))
    return st;
  if (need > V4ATTN_NOALLOC_SCRATCH_BYTES)
    return fail(V4ATTN_EWORKSPACE,
                "the split partials need %zu bytes; the fixed scratch holds %zu (use "
                "v4attn_hca_attend with a workspace)",
                need, (size_t)V4ATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0)
    if (int st = scratch_of_stream_device((hipStream_t)stream, &ws)) return st;
  attend_ws_layout(a, ws);
  return hip_status(v4::launch_attend(a, (hipStream_t)stream), "HCA attend launch");
}

namespace {

// NSA-style variant workspace: the compressed branch's logits and lse, its
// output and the window branch's, block scores, the top-k scratch, the
// selected blocks, then the attention partials: the compressed and window
// branches run in one launch (separate regions); the selected branch reuses
// the compressed branch's region after it.
struct NsaWs {
  int64_t vmax, lstride, sstride;
  size_t logits, lse, o_cmp, o_win, score, topk, blocks, att_cmp, att_win, total;
  TopkWs tk;
};

// Where the window branch runs.  One attention workgroup fills a CU, so it
// goes beside the selected branch (few workgroups) when that branch merges
// split partials in a later pass, which then reads the finished window
// output for the gated sum; otherwise beside the compressed branch.
bool nsa_win_with_selected(int B, int Tq, int n_sel, int m) {
  return v4::attend_splits(B, Tq, (int64_t)n_sel * m, true) > 1;
}

NsaWs nsa_ws(int B, int Tq, int H, int D, int64_t n_entries, int m, int64_t q_pos0, int W,
             int n_sel) {
  NsaWs w;
  const int64_t q = (int64_t)B * Tq;
  w.vmax = vmax_of(Tq, n_entries, q_pos0, m);
  w.lstride = (w.vmax + 127) / 128 * 128;   // the kernel writes whole 128-row tiles
  w.sstride = (w.vmax + 63) / 64 * 64;
  const size_t o_bytes = align256((size_t)(q * H * D) * sizeof(uint16_t));
  size_t o = 0;
  w.logits = o; o += align256((size_t)(q * w.lstride * 64) * sizeof(float));
  w.lse = o;    o += align256((size_t)(q * H) * sizeof(float));
  w.o_cmp = o;  o += o_bytes;
  w.o_win = o;  o += o_bytes;
  w.score = o;  o += align256((size_t)(q * w.sstride) * sizeof(float));
  w.tk = topk_ws(B, Tq, n_entries, q_pos0, m, n_sel);
  w.topk = o;   o += align256(w.tk.total);
  w.blocks = o; o += align256((size_t)(q * n_sel) * sizeof(int32_t));
  const size_t a_cmp = align256(attend_ws(B, Tq, H, D, w.vmax, false, nullptr));
  const size_t a_win = align256(attend_ws(B, Tq, H, D, W, false, nullptr));
  const size_t a_sel = align256(attend_ws(B, Tq, H, D, (int64_t)n_sel * m, true, nullptr));
  w.att_cmp = o;
  w.att_win = o + std::max(a_cmp, a_sel);
  w.total = w.att_win + a_win;
  return w;
}

}  // namespace

size_t v4attn_nsa_attend_workspace(int B, int Tq, int H, int D, int64_t n_entries, int m,
                                   int64_t q_pos0, int W, int n_sel) {
  if (B < 0 || Tq < 0 || H < 1 || D < 1 || n_entries < 0 || m < 1 || q_pos0 < 0 || W < 0 ||
      n_sel < 1)
    return 0;
  return nsa_ws(B, Tq, H, D, n_entries, m, q_pos0, W, n_sel).total;
}

int v4attn_nsa_attend(const uint16_t* q, const uint8_t* entries, const uint8_t* tokens,
                      const uint8_t* win, const float* gamma_q, const float* gates, int B,
                      int Tq, int H, int D, int R, int64_t Ncap, int64_t n_entries, int m,
                      int64_t Ntok, int W, int n_sel, int64_t q_pos0, float scale, float eps,
                      float rope_base, uint16_t* out, int32_t* blocks, float* block_score,
                      void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_attend_common(q, entries, win, gamma_q, nullptr, B, Tq, H, D, R, Ncap, W,
                                   q_pos0, scale, eps, rope_base, out, false))
    return st;
  if (!gates) return fail(V4ATTN_EINVAL, "null gates");
  if (n_entries < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (n_entries >= (int64_t)1 << 31) return fail(V4ATTN_EUNSUPPORTED, "n_entries >= 2^31");
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  if (n_sel < 1 || (int64_t)n_sel * m > kMaxK)
    return fail(V4ATTN_EUNSUPPORTED, "n_sel = %d, m = %d: 1 <= n_sel and n_sel m <= %d are built",
                n_sel, m, kMaxK);
  if (int st = check_topk_len(Tq, n_entries, q_pos0, m)) return st;
  const int64_t vmax = vmax_of(Tq, n_entries, q_pos0, m);
  if (Ntok < vmax * m)
    return fail(V4ATTN_EINVAL, "Ntok %lld < %lld: the tokens of every visible block are needed",
                (long long)Ntok, (long long)(vmax * m));
  if (Ntok * (int64_t)(D + R) >= ((int64_t)1 << 32))
    return fail(V4ATTN_EUNSUPPORTED, "one sequence's token cache must be below 4 GiB");
  if (Ntok > 0 && !tokens) return fail(V4ATTN_EINVAL, "null tokens with Ntok > 0");
  if (!aligned16(tokens)) return fail(V4ATTN_EINVAL, "tokens must be 16-byte aligned");
  const NsaWs w = nsa_ws(B, Tq, H, D, n_entries, m, q_pos0, W, n_sel);
  if (w.total > 0 && (!ws || ws_bytes < w.total))
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  const int64_t nq = (int64_t)B * Tq;
  if (nq == 0) return hip_status(hipSuccess, "");
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* logits = reinterpret_cast<float*>(base + w.logits);
  float* lse = reinterpret_cast<float*>(base + w.lse);
  uint16_t* o_cmp = reinterpret_cast<uint16_t*>(base + w.o_cmp);
  uint16_t* o_win = reinterpret_cast<uint16_t*>(base + w.o_win);
  float* score = reinterpret_cast<float*>(base + w.score);
  int32_t* blk = blocks ? blocks : reinterpret_cast<int32_t*>(base + w.blocks);

  v4::AttendArgs a{};
  a.q = q; a.win = win; a.gamma_q = gamma_q; a.sink = nullptr;
  a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = R;
  a.q_pos0 = q_pos0; a.scale = scale; a.eps = eps; a.rope_base = rope_base;
  a.rope = v4::rope_turns(rope_base, R);

  const bool win_late = nsa_win_with_selected(B, Tq, n_sel, m);
  // window branch: the window rows only (as an HCA problem with no entries,
  // or a CSA problem with no top-k slots)
  v4::AttendArgs wn = a;
  wn.entries = entries; wn.Ncap = Ncap; wn.n_entries = 0; wn.m = 1; wn.W = W;
  wn.out = o_win; wn.rows_max = W;
  if (win_late) { wn.topk = blk; wn.k = 0; }
  wn.splits = v4::attend_splits(B, Tq, wn.rows_max, win_late);
  attend_ws_layout(wn, base + w.att_win);

  // 1. compressed branch: every visible entry, logits and lse kept
  v4::AttendBatch ab{};
  v4::AttendArgs& c = ab.p[0];
  c = a;
  c.entries = entries; c.Ncap = Ncap; c.n_entries = n_entries; c.m = m; c.W = 0;
  c.out = o_cmp; c.lse = lse; c.rows_max = vmax;
  c.logits2 = logits; c.logits_stride = w.lstride;
  c.splits = v4::attend_splits(B, Tq, c.rows_max, false);
  attend_ws_layout(c, base + w.att_cmp);
  if (!win_late) ab.p[1] = wn;
  hipError_t e = v4::launch_attend_batch(ab, win_late ? 1 : 2, st);
  if (e != hipSuccess) return hip_status(e, "NSA compressed branch launch");
  // 2. block scores and the top n_sel blocks
  v4::NsaBlockScoreArgs bs{logits, lse, B, Tq, H, w.lstride, n_entries, q_pos0, m, vmax,
                           score, w.sstride};
  e = v4::launch_nsa_block_score(bs, st);
  if (e != hipSuccess) return hip_status(e, "NSA block score launch");
  e = run_topk(score, w.sstride, B, Tq, n_entries, q_pos0, m, n_sel, blk, block_score,
               base + w.topk, w.tk, st);
  if (e != hipSuccess) return hip_status(e, "NSA block top-k launch");
  // 3. selected branch over the tokens of the selected blocks; its final
  //    store forms the gated sum with the other two branches
  v4::AttendBatch sb{};
  v4::AttendArgs& sl = sb.p[0];
  sl = a;
  sl.entries = tokens; sl.topk = blk; sl.sel_m = m; sl.Ncap = Ntok; sl.k = n_sel * m; sl.W = 0;
  sl.out = out; sl.rows_max = (int64_t)n_sel * m;
  sl.mix_gates = gates; sl.mix_o0 = o_cmp; sl.mix_o2 = o_win;
  sl.splits = v4::attend_splits(B, Tq, sl.rows_max, true);
  attend_ws_layout(sl, base + w.att_cmp);
  if (win_late) sb.p[1] = wn;
  return hip_status(v4::launch_attend_batch(sb, win_late ? 2 : 1, st),
                    "NSA selected branch launch");
}

namespace {

// Attention backward: queries are processed in chunks of at most 128 whose
// per-query buffers (gathered rows, [S; dP], [scale dL; P], ...) fit about
// 1 GiB (128 rather than 64 queries a chunk: 11.8 -> 11.2 ms at 4096 x 1152
// rows; 256 gained nothing more).
int bwd_chunk(int64_t nq, int D, int64_t np) {
  const size_t per = v4::bwd_query_bytes(D, np);
  int64_t c = (int64_t)(((size_t)1 << 30) / per);
  if (c < 1) c = 1;
  if (c > 128) c = 128;
  return (int)(c < nq ? c : (nq > 0 ? nq : 1));
}

size_t bwd_ws(int B, int Tq, int D, int64_t rows_max) {
  const int64_t nq = (int64_t)B * Tq;
  const int64_t np = v4::bwd_rows_padded(rows_max > 0 ? rows_max : 1);
  return (size_t)bwd_chunk(nq, D, np) * v4::bwd_query_bytes(D, np);
}

// Grouped row gradients: destinations (entry rows, then window rows), and
// the queries per group: a whole multiple of the query chunk (or all
// queries) whose dense gradients fit both 12 GiB and what the workspace holds
// beyond the per-chunk buffers; 0 (atomic row gradients) when not even one
// chunk fits or the ids overflow 32 bits.
int64_t bwd_ndest(int B, int Tq, int W, int64_t Ncap) {
  return (int64_t)B * Ncap + (W > 0 ? (int64_t)B * (Tq + W - 1) : 0);
}
int64_t bwd_group_queries(int B, int Tq, int D, int64_t rows_max, int64_t ndest,
                          size_t ws_bytes) {
  const int64_t nq = (int64_t)B * Tq;
  const int64_t np = v4::bwd_rows_padded(rows_max > 0 ? rows_max : 1);
  if (nq == 0 || ndest + 1 >= ((int64_t)1 << 31) || nq * np >= ((int64_t)1 << 31)) return 0;
  const int64_t qc = bwd_chunk(nq, D, np);
  const size_t base = bwd_ws(B, Tq, D, rows_max);
  const auto fits = [&](int64_t g) {
    const size_t need = base + v4::bwd_group_bytes(D, np, g, ndest);
    return need <= ws_bytes && (size_t)g * np * D * 3 <= ((size_t)12 << 30);   // 24-bit values
  };
  if (fits(nq)) return nq;
  int64_t lo = 0, hi = (nq - 1) / qc;  // chunks per group: fits(lo * qc) holds or lo = 0
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (fits(mid * qc)) lo = mid; else hi = mid - 1;
  }
  return lo * qc;
}
size_t bwd_ws_grouped(int B, int Tq, int D, int64_t rows_max, int W, int64_t Ncap) {
  const int64_t np = v4::bwd_rows_padded(rows_max > 0 ? rows_max : 1);
  const int64_t nd = bwd_ndest(B, Tq, W, Ncap);
  const int64_t gq = bwd_group_queries(B, Tq, D, rows_max, nd, ~(size_t)0);
  return bwd_ws(B, Tq, D, rows_max) + v4::bwd_group_bytes(D, np, gq, nd);
}

int run_backward(const uint16_t* q, const uint8_t* entries, const int32_t* topk,
                 const uint8_t* win, const float* gamma_q, const float* sink, int B, int Tq, int H,
                 int D, int R, int64_t Ncap, int k, int64_t n_entries, int m, int W,
                 int64_t q_pos0, float scale, float eps, float rope_base, const uint16_t* out,
                 const float* lse, const uint16_t* dout, float* dq, float* d_entries,
                 float* d_win, float* d_sink, float* d_gamma_q, float* p_sel, int64_t rows_max,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!out || !lse || !dout || !dq) return fail(V4ATTN_EINVAL, "null out, lse, dout or dq");
  if (Ncap > 0 && !d_entries) return fail(V4ATTN_EINVAL, "null d_entries with Ncap > 0");
  if (W > 0 && !d_win) return fail(V4ATTN_EINVAL, "null d_win with W > 0");
  if (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(dq))
    return fail(V4ATTN_EINVAL, "q, out, dout and dq must be 16-byte aligned");
  const size_t need = bwd_ws(B, Tq, D, rows_max);
  if (!ws || ws_bytes < need)
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  // the grouped row gradients (16-byte row adds) when the workspace holds
  // them and the row gradients are 16-byte aligned, else atomics
  const int64_t ndest = bwd_ndest(B, Tq, W, Ncap);
  const bool rows_aligned = (!d_entries || aligned16(d_entries)) && (!d_win || aligned16(d_win));
  const int64_t gq = rows_aligned ? bwd_group_queries(B, Tq, D, rows_max, ndest, ws_bytes) : 0;
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  const int64_t nq = (int64_t)B * Tq;
  if (nq == 0) return hip_status(hipSuccess, "");
  v4::BwdArgs a{};
  a.q = q; a.entries = entries; a.topk = topk; a.win = win; a.gamma_q = gamma_q; a.sink = sink;
  a.out = out; a.lse = lse; a.dout = dout;
  a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = R; a.Ncap = Ncap; a.k = k; a.n_entries = n_entries;
  a.m = m; a.W = W; a.q_pos0 = q_pos0; a.scale = scale; a.eps = eps;
  a.rope = v4::rope_turns(rope_base, R);
  a.np = v4::bwd_rows_padded(rows_max > 0 ? rows_max : 1);
  a.dq = dq; a.d_entries = d_entries; a.d_win = d_win; a.d_sink = d_sink; a.d_gamma_q = d_gamma_q;
  a.p_sel = p_sel; a.k_sel = topk ? k : 0;
  a.nent = (int64_t)B * Ncap; a.ndest = ndest;
  return hip_status(v4::launch_attend_backward(a, bwd_chunk(nq, D, a.np), gq, ws, (hipStream_t)stream),
                    "attention backward launch");
}

}  // namespace

size_t v4attn_csa_attend_backward_workspace(int B, int Tq, int H, int D, int k, int W,
                                            int64_t Ncap) {
  if (B < 0 || Tq < 0 || H < 1 || D < 1 || k < 1 || W < 0 || Ncap < 0) return 0;
  return bwd_ws_grouped(B, Tq, D, (int64_t)k + W, W, Ncap);
}

int v4attn_csa_attend_backward(const uint16_t* q, const uint8_t* entries, const int32_t* topk,
                               const uint8_t* win, const float* gamma_q, const float* sink, int B,
                               int Tq, int H, int D, int R, int64_t Ncap, int k, int W,
                               int64_t q_pos0, float scale, float eps, float rope_base,
                               const uint16_t* out, const float* lse, const uint16_t* dout,
                               float* dq, float* d_entries, float* d_win, float* d_sink,
                               float* d_gamma_q, float* p_sel, void* ws, size_t ws_bytes,
                               void* stream) {
  if (int st = check_attend_common(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, W,
                                   q_pos0, scale, eps, rope_base, out))
    return st;
  if (!topk) return fail(V4ATTN_EINVAL, "null topk");
  if (k < 1 || k > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "k = %d: 1 <= k <= %d is built", k, kMaxK);
  return run_backward(q, entries, topk, win, gamma_q, sink, B, Tq, H, D, R, Ncap, k, 0, 1, W,
                      q_pos0, scale, eps, rope_base, out, lse, dout, dq, d_entries, d_win,
                      d_sink, d_gamma_q, p_sel, (int64_t)k + W, ws, ws_bytes, stream);
}

size_t v4attn_hca_attend_backward_workspace(int B, int Tq, int H, int D, int64_t n_entries, int m,
                                            int64_t q_pos0, int W, int64_t Ncap) {
  if (B < 0 || Tq < 0 || H < 1 || D < 1 || n_entries < 0 || m < 1 || q_pos0 < 0 || W < 0 ||
      Ncap < 0)
    return 0;
  return bwd_ws_grouped(B, Tq, D, vmax_of(Tq, n_entries, q_pos0, m) + W, W, Ncap);
}

int v4attn_hca_attend_backward(const uint16_t* q, const uint8_t* entries, const uint8_t* win,
                               const float* gamma_q, const float* sink, int B, int Tq, int H,
                               int D, int R, int64_t Ncap, int64_t n_entries, int m, int W,
                               int64_t q_pos0, float scale, float eps, float rope_base,
                               const uint16_t* out, const float* lse, const uint16_t* dout,
                               float* dq, float* d_entries, float* d_win, float* d_sink,
                               float* d_gamma_q, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_attend_common(q, entries, win, gamma_q, sink, B, Tq, H, D, R, Ncap, W,
                                   q_pos0, scale, eps, rope_base, out))
    return st;
  if (n_entries < 0 || n_entries > Ncap) return fail(V4ATTN_EINVAL, "need 0 <= n_entries <= Ncap");
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  return run_backward(q, entries, nullptr, win, gamma_q, sink, B, Tq, H, D, R, Ncap, 0, n_entries,
                      m, W, q_pos0, scale, eps, rope_base, out, lse, dout, dq, d_entries, d_win,
                      d_sink, d_gamma_q, nullptr, vmax_of(Tq, n_entries, q_pos0, m) + W, ws,
                      ws_bytes, stream);
}

int v4attn_compress_backward(const uint16_t* raw, const float* tok_score, const float* pos_bias,
                             const float* gamma, int B, int L, int D, int R, int64_t raw_pos0,
                             int m, int64_t entry0, int n_out, float eps, float rope_base,
                             const float* d_entries, float* d_raw, float* d_score, float* d_bias,
                             float* d_gamma, void* stream) {
  if (!raw || !tok_score || !pos_bias || !gamma || !d_entries || !d_raw || !d_score)
    return fail(V4ATTN_EINVAL, "null raw, tok_score, pos_bias, gamma, d_entries, d_raw or d_score");
  if (B < 0 || L < 0 || n_out < 0) return fail(V4ATTN_EINVAL, "negative B, L or n_out");
  if (int st = check_dr(D, R)) return st;
  if (m < 1 || m > 256) return fail(V4ATTN_EUNSUPPORTED, "m = %d: 1 <= m <= 256 is built", m);
  if (entry0 < 0) return fail(V4ATTN_EINVAL, "negative entry0");
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f))
    return fail(V4ATTN_EINVAL, "bad eps or rope_base");
  if (n_out > 0) {
    const int64_t lo = (entry0 - 1) * (int64_t)m;
    const int64_t first = lo > 0 ? lo : 0;
    const int64_t last = (entry0 + n_out) * (int64_t)m;
    if (first < raw_pos0 || last > raw_pos0 + L)
      return fail(V4ATTN_EINVAL, "entries %lld..%lld need positions [%lld, %lld) but rows hold [%lld, %lld)",
                  (long long)entry0, (long long)(entry0 + n_out - 1), (long long)first,
                  (long long)last, (long long)raw_pos0, (long long)(raw_pos0 + L));
  }
  if (!aligned16(raw)) return fail(V4ATTN_EINVAL, "raw must be 16-byte aligned");
  v4::CompressBwdArgs a{raw, tok_score, pos_bias, gamma, B, L, D, R, raw_pos0, m, entry0, n_out,
                        eps, v4::rope_turns(rope_base, R), d_entries, d_raw, d_score, d_bias,
                        d_gamma};
  return hip_status(v4::launch_compress_backward(a, (hipStream_t)stream), "compress backward launch");
}

}  // extern "C"

namespace {

int kl_chunk(int64_t nq, int64_t nsp, int dIp) {
  int64_t c = (int64_t)(((size_t)1 << 30) / v4::kl_query_bytes(nsp, dIp));
  if (c < 1) c = 1;
  if (c > 256) c = 256;
  return (int)(c < nq ? c : (nq > 0 ? nq : 1));
}

size_t kl_ws(int B, int Tq, int dI, int ns) {
  const int64_t nsp = (ns + 63) / 64 * 64;
  const int dIp = (dI + 63) / 64 * 64;
  return (size_t)kl_chunk((int64_t)B * Tq, nsp, dIp) * v4::kl_query_bytes(nsp, dIp);
}

// Grouped key gradients (as the attention backward's row gradients): the
// queries per group, a whole multiple of the chunk (or all queries) whose
// dense dK fits both 12 GiB and what the workspace holds beyond the
// per-chunk buffers; 0 (atomic adds) when not even one chunk fits or the
// ids overflow 32 bits.
int64_t kl_group_queries(int B, int Tq, int dI, int ns, int64_t ndest, size_t ws_bytes) {
  const int64_t nq = (int64_t)B * Tq;
  const int64_t nsp = (ns + 63) / 64 * 64;
  const int dIp = (dI + 63) / 64 * 64;
  if (nq == 0 || ndest + 1 >= ((int64_t)1 << 31) || nq * nsp >= ((int64_t)1 << 31)) return 0;
  const int64_t qc = kl_chunk(nq, nsp, dIp);
  const size_t base = kl_ws(B, Tq, dI, ns);
  const auto fits = [&](int64_t g) {
    return base + v4::kl_group_bytes(dI, nsp, g, ndest) <= ws_bytes &&
           (size_t)g * nsp * dI * 3 <= ((size_t)12 << 30);   // 24-bit values
  };
  if (fits(nq)) return nq;
  int64_t lo = 0, hi = (nq - 1) / qc;   // chunks per group: fits(lo * qc) holds or lo = 0
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (fits(mid * qc)) lo = mid; else hi = mid - 1;
  }
  return lo * qc;
}

size_t kl_ws_grouped(int B, int Tq, int dI, int ns, int64_t Ncap) {
  const int64_t nsp = (ns + 63) / 64 * 64;
  const int64_t nd = (int64_t)B * Ncap;
  const int64_t gq = kl_group_queries(B, Tq, dI, ns, nd, ~(size_t)0);
  return kl_ws(B, Tq, dI, ns) + v4::kl_group_bytes(dI, nsp, gq, nd);
}

}  // namespace

extern "C" {

size_t v4attn_index_kl_backward_workspace(int B, int Tq, int dI, int ns, int64_t Ncap) {
  if (B < 0 || Tq < 0 || dI < 1 || ns < 1 || Ncap < 0) return 0;
  return kl_ws_grouped(B, Tq, dI, ns, Ncap);
}

int v4attn_index_kl_backward(const uint16_t* q_idx, const float* w_idx, const uint16_t* k_idx,
                             const int32_t* sel, const float* target, int B, int Tq, int HI,
                             int dI, int64_t Ncap, int ns, float* loss, float* dq_idx,
                             float* dw_idx, float* dk_idx, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!q_idx || !w_idx || !sel || !target || !dq_idx || !dw_idx || !dk_idx)
    return fail(V4ATTN_EINVAL, "null q_idx, w_idx, sel, target, dq_idx, dw_idx or dk_idx");
  if (Ncap > 0 && !k_idx) return fail(V4ATTN_EINVAL, "null k_idx");
  if (B < 0 || Tq < 0 || Ncap < 0) return fail(V4ATTN_EINVAL, "negative B, Tq or Ncap");
  if (HI < 1 || HI > 64) return fail(V4ATTN_EUNSUPPORTED, "HI = %d: 1 <= HI <= 64 is built", HI);
  if (dI != 32 && dI != 64 && dI != 128)
    return fail(V4ATTN_EUNSUPPORTED, "dI = %d: dI in {32, 64, 128} is built", dI);
  if (ns < 1 || ns > kMaxK) return fail(V4ATTN_EUNSUPPORTED, "ns = %d: 1 <= ns <= %d is built", ns, kMaxK);
  if (!aligned16(q_idx) || !aligned16(k_idx)) return fail(V4ATTN_EINVAL, "q_idx and k_idx must be 16-byte aligned");
  const size_t need = kl_ws(B, Tq, dI, ns);
  if (!ws || ws_bytes < need)
    return fail(V4ATTN_EWORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (!aligned16(ws)) return fail(V4ATTN_EINVAL, "workspace must be 16-byte aligned");
  const int64_t nq = (int64_t)B * Tq;
  if (nq == 0) return hip_status(hipSuccess, "");
  v4::KlArgs a{};
  a.q_idx = q_idx; a.w_idx = w_idx; a.k_idx = k_idx; a.sel = sel; a.target = target;
  a.B = B; a.Tq = Tq; a.HI = HI; a.dI = dI; a.dIp = (dI + 63) / 64 * 64; a.Ncap = Ncap;
  a.ns = ns; a.nsp = (ns + 63) / 64 * 64;
  a.loss = loss; a.dq = dq_idx; a.dw = dw_idx; a.dk = dk_idx;
  // the grouped key gradients (16-byte row adds) when the workspace holds
  // them and dk is 16-byte aligned, else atomics
  const int64_t ndest = (int64_t)B * Ncap;
  const int64_t gq = aligned16(dk_idx) ? kl_group_queries(B, Tq, dI, ns, ndest, ws_bytes) : 0;
  return hip_status(v4::launch_index_kl_backward(a, kl_chunk(nq, a.nsp, a.dIp), gq, ndest, ws,
                                                 (hipStream_t)stream),
                    "indexer KL backward launch");
}

}  // extern "C"
