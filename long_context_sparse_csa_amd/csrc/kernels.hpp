// Internal launch interface between the C-ABI layer (api.cpp) and the
// kernels.  Arguments are validated by the caller before a launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace v4 {

// Per-sequence positions of a ragged batch (decode path), passed by value
// with the kernel arguments: sequence b's first query is at p[b].
constexpr int kMaxRagged = 64;
struct SeqPos {
  int64_t p[kMaxRagged];
};

struct CompressArgs {
  const uint16_t* raw;
  const float* tok_score;
  const float* pos_bias;
  const float* gamma;
  int B, L, D, R;
  int64_t raw_pos0;
  int mode, m;
  int64_t entry0;
  int n_out;
  float eps, rope_base;
  uint8_t* out;
  int64_t out_rows;
  RopeTurns rope;        // from rope_base (host)
  const uint16_t* raw_idx;  // POOL, nullable: [B, L, dI] token indexer keys
  int dI;
  uint16_t* kidx;           // [B, out_rows, dI] pooled indexer keys (rows as out)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);

// One decode step of the compressor: the window row of the token at t and,
// when (t+1) % m == 0, the entry (t+1)/m - 1 it completes, in one launch.
struct CompressStepArgs {
  const uint16_t* raw;     // [B, L, D], positions raw_pos0 ..
  const float* tok_score;  // [B, L]
  const float* pos_bias;   // [2m]
  const float* gamma;      // [D]
  int B, L, D, R;
  int64_t raw_pos0;
  int m;
  int64_t t;
  float eps;
  RopeTurns rope;
  uint8_t* ent;            // [B, ent_rows, D+R], entry j at row j
  int64_t ent_rows;
  uint8_t* win;            // [B, win_rows, D+R]
  int64_t win_rows, win_row;
  bool ragged;             // token of sequence b at pos.p[b]; raw rows hold its
  SeqPos pos;              // positions p[b]-L+1 .. p[b] (t, raw_pos0 unused)
  const uint16_t* raw_idx; // nullable: [B, L, dI] token indexer keys
  int dI;
  uint16_t* kidx;          // [B, ent_rows, dI]: the entry's pooled indexer key at row j
};
hipError_t launch_compress_step(const CompressStepArgs& a, hipStream_t st);
// Several layers' decode steps (same D) in one launch.
constexpr int kMaxSteps = 2;   // the arguments of every layer travel in the kernel arguments
struct CompressStepBatch {
  CompressStepArgs s[kMaxSteps];   // in launch order
};
hipError_t launch_compress_steps(const CompressStepArgs* a, int n, hipStream_t st);

// Lightning-indexer scoring into a dense fp32 score buffer.
struct IndexScoreArgs {
  const uint16_t* q_idx;  // [B, Tq, HI, dI]
  const float* w_idx;     // [B, Tq, HI]
  const uint16_t* k_idx;  // [B, Ncap, dI]
  int B, Tq, HI, dI;
  int64_t Ncap, n_entries, q_pos0;
  int m;
  int64_t vmax;           // max visible entries over the query block
  float* scores;          // [B*Tq, score_stride]
  int64_t score_stride;
  int64_t row_waves;      // waves sharing one query row (multiple of 4)
  bool ragged;            // query block of sequence b starts at pos.p[b]
  SeqPos pos;
  // ragged decode (Tq = 1): a flat grid, sequence b owning workgroups
  // wg_start[b] .. wg_start[b+1]-1 (in proportion to its visible entries)
  int wg_start[kMaxRagged + 1];
};
// Waves per query row that spread a launch over three workgroups per CU.
int64_t index_row_waves(int B, int Tq, int64_t vmax);
hipError_t launch_index_score(const IndexScoreArgs& a, hipStream_t st);

// FP8 lightning-indexer scoring: q and k as OCP E4M3 codes with positive
// fp32 scales (one per query head, one per key); same score buffer.
struct IndexScoreFp8Args {
  const uint8_t* q8;       // [B, Tq, HI, dI] E4M3
  const float* q_scale;    // [B, Tq, HI]
  const float* w_idx;      // [B, Tq, HI]
  const uint8_t* k8;       // [B, Ncap, dI] E4M3
  const float* k_scale;    // [B, Ncap]
  int B, Tq, HI, dI;
  int64_t Ncap, n_entries, q_pos0;
  int m;
  int64_t vmax;            // max visible entries over the query block
  float* scores;           // [B*Tq, score_stride]
  int64_t score_stride;
  int64_t row_waves;       // waves sharing one query row (multiple of 4)
};
int64_t index_fp8_row_waves(int B, int Tq, int64_t vmax);
hipError_t launch_index_score_fp8(const IndexScoreFp8Args& a, hipStream_t st);

// MXFP4 lightning-indexer scoring: q and k as OCP MX FP4 rows (packed E2M1
// codes, one E8M0 scale byte per 32 dims); same score buffer.
struct IndexScoreMxfp4Args {
  const uint8_t* q4;       // [B, Tq, HI, dI/2]
  const uint8_t* q_sc;     // [B, Tq, HI, dI/32]
  const float* w_idx;      // [B, Tq, HI]
  const uint8_t* k4;       // [B, Ncap, dI/2]
  const uint8_t* k_sc;     // [B, Ncap, dI/32]
  int B, Tq, HI, dI;
  int64_t Ncap, n_entries, q_pos0;
  int m;
  int64_t vmax;
  float* scores;
  int64_t score_stride;
  int64_t row_waves;
};
int64_t index_mxfp4_row_waves(int B, int Tq, int64_t vmax);
hipError_t launch_index_score_mxfp4(const IndexScoreMxfp4Args& a, hipStream_t st);

// Top-k selection: per-part leaders -> exact per-row select.
constexpr int kTopkSel = 16384;     // keys the per-row selection holds in LDS
constexpr int kTopkPartLen = 1024;  // scores per part (the longest; 128 to 512 for short rows)
constexpr int kTopkPartMin = 128;   // the shortest part
constexpr int kTopkPartCap = 32;    // leaders a part stores
constexpr int kTopkMaxParts = 4096; // parts per row (entries <= 4M)

// Scores per part of a row of V entries: short enough that a part holds
// on average at most 4 of the row's top k (a part stores its keys from the
// 16th largest of its 64 lane maxima up, so it rarely misses one of the
// row's top k: a miss sends the row to the re-read path); 128 to 1024.
__host__ __device__ inline int topk_part_len(int64_t V, int k) {
  int P = kTopkPartLen;
  while (P > kTopkPartMin && (int64_t)k * P > 4 * V) P >>= 1;
  return P;
}

struct TopkPlan {
  int64_t direct_max;  // rows of at most this many entries are selected directly
  bool parts;          // longer rows exist: run the part kernel
  int nparts;          // part slots per row (the most any row of the launch has)
};
// The plan for rows of vmin .. vmax visible entries (part slots for the most
// parts any length in that range takes).
TopkPlan topk_plan(int64_t vmin, int64_t vmax, int k);

struct TopkArgs {
  const float* scores;     // [B*Tq, score_stride]
  int64_t score_stride;
  int B, Tq;
  int64_t n_entries, q_pos0;
  int m, k;
  int64_t direct_max;      // TopkPlan::direct_max
  int nparts;              // part slots per row (a row uses topk_part_len of its own V)
  unsigned* part_tau;      // [rows, nparts] the part's leader threshold (0: none)
  int* part_cnt;           // [rows, nparts] keys >= it in the part
  unsigned* part_over;     // [rows, nparts] largest of them not stored (0: none)
  unsigned* cand_key;      // [rows, nparts, kTopkPartCap] the stored ones, position order
  int* cand_idx;
  unsigned* run_key;       // [rows, k] keys of a partial selection
  int32_t* topk;           // [B*Tq, k]
  float* topk_score;       // nullable
  bool ragged;             // query block of sequence b starts at pos.p[b]
  SeqPos pos;
};
hipError_t launch_topk(const TopkArgs& a, const TopkPlan& plan, hipStream_t st);

// Core attention (CSA when topk != nullptr, else HCA).
struct AttendArgs {
  const uint16_t* q;        // [B, Tq, H, D]
  const uint8_t* entries;   // [B, Ncap, D+R]
  const int32_t* topk;      // [B, Tq, k] or nullptr
  const uint8_t* win;       // [B, Tq+W-1, D+R]
  const float* gamma_q;
  const float* sink;        // [H], or nullptr for no sink
  int B, Tq, H, D, R;
  int64_t Ncap;
  int k;                    // CSA: top-k slots
  int64_t n_entries;        // HCA: entries that exist
  int m;                    // HCA: compression ratio
  int W;
  int64_t q_pos0;
  float scale, eps, rope_base;
  RopeTurns rope;           // from rope_base (host)
  uint16_t* out;            // [B, Tq, H, D]
  float* lse;               // [B, Tq, H] or nullptr
  int splits;               // key-range splits per query (1 = no merge pass)
  uint16_t* part_o;         // [B*Tq, splits, H, D] snorm16 q: unnormalised O = q 2^e / 32767
  float* part_ml;           // [B*Tq, splits, H, 4]  (max, sum, e, unused)
  int64_t rows_max;         // max rows (entries + window) over the block
  float* logits2;           // HCA only: nullptr, or [B*Tq, logits_stride, 64]: every row's logit
                            // per head (heads innermost, slots >= H unused) times
                            // log2(e), absent rows -inf; logits_stride >= rows
                            // rounded up to 128
  int64_t logits_stride;
  int sel_m;                // CSA: 0 or 1 = topk holds row indices; > 1 = topk
                            // [B*Tq, k / sel_m] holds blocks of sel_m rows
                            // (row b sel_m + u), -1 = empty
  const float* mix_gates;   // CSA only: nullptr, or [B*Tq, H, 3]: the stored output is
                            // g1 * this + g0 * mix_o0 + g2 * mix_o2
  const uint16_t* mix_o0;   // bf16 [B*Tq, H, D]
  const uint16_t* mix_o2;
  bool ragged;              // query block of sequence b starts at pos.p[b]
  SeqPos pos;               // (its window buffer rows are relative to it)
  // ragged decode (Tq = 1) with its own split count per sequence: sequence b
  // owns split slots slot0[b] .. slot0[b+1]-1 (a flat grid of slot0[B]
  // workgroups; partials at those slots); false: `splits` for every query
  bool flat;
  int slot0[kMaxRagged + 1];
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
// Per-sequence split counts for a ragged decode batch (rows[b] rows for
// sequence b): about the same number of tiles per workgroup everywhere,
// within the B * a.splits partial slots of the uniform plan.  Sets a.flat
// and a.slot0.
void plan_flat_splits(AttendArgs& a, const int64_t* rows, bool csa);

// Up to two problems of the same kind, head count, head dim and query block
// in one launch (grid layer z runs p[z]); each keeps its own splits and
// workspace.
struct AttendBatch {
  AttendArgs p[2];
};
hipError_t launch_attend_batch(const AttendBatch& ab, int n, hipStream_t st);

// Number of key-range splits the attention uses for a problem (shared by
// the workspace query and the launch so both agree).
int attend_splits(int B, int Tq, int64_t rows_max, bool csa, int wg_budget = 256);

// NSA-style variant: block scores from the compressed branch's logits.
struct NsaBlockScoreArgs {
  const float* logits2;     // [B*Tq, logits_stride, 64], log2 units
  const float* lse;         // [B*Tq, H], natural log
  int B, Tq, H;
  int64_t logits_stride;
  int64_t n_entries, q_pos0;
  int m;
  int64_t vmax;             // max visible entries over the block
  float* score;             // [B*Tq, score_stride]
  int64_t score_stride;
};
hipError_t launch_nsa_block_score(const NsaBlockScoreArgs& a, hipStream_t st);

// Batched bf16 matrix-core product C[z] = alpha A[z] B[z] (fp32 out; M, N
// multiples of 64, K of 32).  With rowmap, row m of C[z] is instead added
// (atomically) into c row rowmap[z, m] (>= 0), c2 row -2 - rowmap (<= -2),
// or dropped (-1).
struct GemmArgs {
  const uint16_t* a;
  int64_t lda, a_batch;
  const uint16_t* b;
  int64_t ldb, b_batch;
  float* c;
  float* c2;
  int64_t ldc, c_batch;
  const int64_t* rowmap;
  int64_t rowmap_batch;
  int K;
  float alpha;
  int n_valid;               // columns >= n_valid are not stored
  int f24;                   // dense C stored as 24-bit values (4 in 3 words)
};

// Attention backward (both kinds: CSA when topk != nullptr).
struct BwdArgs {
  const uint16_t* q;         // [B, Tq, H, D]
  const uint8_t* entries;    // [B, Ncap, D+R]
  const int32_t* topk;       // [B, Tq, k] or nullptr (dense visible entries)
  const uint8_t* win;        // [B, Tq+W-1, D+R]
  const float* gamma_q;      // [D]
  const float* sink;         // [H] or nullptr
  const uint16_t* out;       // forward output [B, Tq, H, D]
  const float* lse;          // forward lse [B, Tq, H]
  const uint16_t* dout;      // [B, Tq, H, D]
  int B, Tq, H, D, R;
  int64_t Ncap;
  int k;
  int64_t n_entries;
  int m, W;
  int64_t q_pos0;
  float scale, eps;
  RopeTurns rope;
  int64_t np;                // row slots per query, padded to 64
  float* dq;                 // [B, Tq, H, D] (written)
  float* d_entries;          // [B, Ncap, D] (added)
  float* d_win;              // [B, Tq+W-1, D] (added)
  float* d_sink;             // [H] (added), nullable
  float* d_gamma_q;          // [D] (added), nullable
  float* p_sel;              // [B, Tq, k_sel] sum over heads of p of the entry
                             // slots (written), nullable
  int k_sel;
  // workspace views (set by the launcher)
  uint16_t* X;
  int64_t* rowmap;
  uint16_t* Y;                // [chunk, 128, D] [q~; do] (head slot rows)
  uint16_t* YT;               // [chunk, D, 128] the same, transposed
  float* Dh;
  uint16_t* T;                // [chunk, 64, np] scale dL (head slot rows)
  uint16_t* TT;               // [chunk, np, 128] [scale dL; P] per row slot
  float* DQT;
  float* G;                  // [chunk, D] a query's d_gamma_q share (its heads summed)
  float* DS;                 // [chunk, 64] a query's d_sink share per head
  // grouped row gradients (dXd != nullptr): the dX product stores every
  // (query, row slot)'s gradient densely; after each group of queries the
  // slots are grouped by destination row (a counting sort) and each row's
  // slots summed once into d_entries / d_win
  float* dXd;                // [group, np, D]
  int32_t* dest;             // [group, np] destination row: b Ncap + j, or
                             // B Ncap + window row, or -1
  uint32_t* cnt;             // [ndest + 1] slots per destination
  int64_t nent;              // B Ncap: destinations below are entries
  int64_t ndest;             // B Ncap + B (Tq + W - 1)
  int group_q0;              // first query of the current group
};
int64_t bwd_rows_padded(int64_t rows_max);
size_t bwd_query_bytes(int D, int64_t np);
// Workspace bytes of the grouped row gradients for groups of `gq` queries
// (0: none) and ndest destination rows.
size_t bwd_group_bytes(int D, int64_t np, int64_t gq, int64_t ndest);
// gq = 0: row gradients by atomic adds; gq > 0: grouped, gq queries (a
// multiple of qchunk) per group, ndest destinations.
hipError_t launch_attend_backward(BwdArgs a, int qchunk, int64_t gq, void* ws, hipStream_t st);

// Compressor (POOL) backward for entries entry0 .. entry0+n_out-1.
struct CompressBwdArgs {
  const uint16_t* raw;       // [B, L, D], positions raw_pos0 ..
  const float* tok_score;    // [B, L]
  const float* pos_bias;     // [2m]
  const float* gamma;        // [D]
  int B, L, D, R;
  int64_t raw_pos0;
  int m;
  int64_t entry0;
  int n_out;
  float eps;
  RopeTurns rope;
  const float* de;           // [B, n_out, D] gradient of the entries' values
  float* d_raw;              // [B, L, D] (added)
  float* d_score;            // [B, L] (added)
  float* d_bias;             // [2m] (added), nullable
  float* d_gamma;            // [D] (added), nullable
};
hipError_t launch_compress_backward(const CompressBwdArgs& a, hipStream_t st);

// Indexer KL loss backward over one entry set per query.
struct KlArgs {
  const uint16_t* q_idx;     // [B, Tq, HI, dI]
  const float* w_idx;        // [B, Tq, HI]
  const uint16_t* k_idx;     // [B, Ncap, dI]
  const int32_t* sel;        // [B, Tq, ns] entry indices, -1 = empty
  const float* target;       // [B, Tq, ns] target weights (normalised here)
  int B, Tq, HI, dI, dIp;
  int64_t Ncap;
  int ns;
  int64_t nsp;               // ns padded to 64
  float* loss;               // [B, Tq] (written), nullable
  float* dq;                 // [B, Tq, HI, dI] (written)
  float* dw;                 // [B, Tq, HI] (written)
  float* dk;                 // [B, Ncap, dI] (added)
  uint16_t* K;
  int64_t* rowmap;
  uint16_t* Qi;
  float* Am;
  uint16_t* Gm;
  float* DQ;
  float* Sb;                 // [chunk, nsp] scores, then d loss / d score
  // grouped key gradients (dKd != nullptr), as the attention backward's
  // row gradients: dense dK per (query, slot), summed per destination row
  float* dKd;                // [group, nsp, dI]
  int32_t* dest;             // [group, nsp] b Ncap + j, or -1
  uint32_t* cnt;             // [B Ncap + 1] slots per destination
  int group_q0;
};
size_t kl_query_bytes(int64_t nsp, int dIp);
// Workspace bytes of the grouped key gradients for groups of gq queries.
size_t kl_group_bytes(int dI, int64_t nsp, int64_t gq, int64_t ndest);
// gq = 0: key gradients by atomic adds; gq > 0: grouped (a multiple of
// qchunk, or all queries), ndest = B Ncap destinations.
hipError_t launch_index_kl_backward(KlArgs a, int qchunk, int64_t gq, int64_t ndest, void* ws,
                                    hipStream_t st);

}  // namespace v4
