/*
 * v4attn.h -- C ABI of libv4attn.so: DeepSeek-V4 hybrid compressed attention
 * (CSA + HCA) on AMD Instinct MI355X (gfx950).
 *
 * The method (from the pages "DeepSeek-V4: Making a Million Tokens
 * Affordable", section "Two ways to shrink attention, interleaved", and
 * "DeepSeek-V4 Explained: Compressed Sparse Attention and 1M Context at 10%
 * KV", section "The attention stack, and why it is two mechanisms"):
 *   - the KV stream of every m consecutive tokens is pooled into one entry
 *     with learned per-token weights and positional biases over an
 *     overlapping 2m-token window (CSA m = 4, HCA m' = 128);
 *   - CSA scores each query against all entries with a lightning indexer,
 *     keeps the top-k, and runs shared-KV multi-query attention over them
 *     plus a 128-token uncompressed window;
 *   - HCA attends densely to every entry plus the same window;
 *   - queries and entries get RMSNorm, RoPE acts on the last 64 dims, the
 *     output is rotated back by RoPE at -t, and a per-head sink logit lets
 *     the attention weights sum to less than one;
 *   - entries are stored with BF16 rotary dims and FP8 for the rest.
 *
 * Conventions shared by every call
 *   - Tensors are caller-owned, contiguous DEVICE buffers (16-byte aligned),
 *     row-major in the shapes given.  bf16 values are passed as uint16_t bit
 *     patterns.  The library never allocates, frees or synchronises, and
 *     keeps no state between calls; calls are thread-safe.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     and the call returns before the GPU finishes.  Device-side faults
 *     surface at the caller's next synchronisation.
 *   - Return value: V4ATTN_OK, or a negative status; on error nothing is
 *     launched and v4attn_last_error() describes the problem.
 *   - Positions are absolute token positions (int64).  A batch shares them:
 *     every sequence of the batch has the same length.
 *   - Packed row: (D - R) bytes of OCP FP8 E4M3FN (dims 0..D-R-1), then R
 *     little-endian bf16 (dims D-R..D-1): D + R bytes (576 at D = 512).
 *   - RoPE: adjacent pairs (D-R+2i, D-R+2i+1) rotate by p * base^(-2i/R).
 *   - Supported sizes: D in {128, 256, 512}, R = 64, 1 <= H <= 64,
 *     1 <= HI <= 64, dI in {32, 64, 128}, 1 <= m <= 256, 1 <= k <= 4096,
 *     0 <= W <= 4096.  Others return V4ATTN_EUNSUPPORTED.
 */
#ifndef V4ATTN_H
#define V4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define V4ATTN_OK            0
#define V4ATTN_EINVAL       (-1) /* bad pointer, shape or position          */
#define V4ATTN_EUNSUPPORTED (-2) /* valid but not built (e.g. R != 64)      */
#define V4ATTN_EWORKSPACE   (-3) /* workspace missing or too small          */
#define V4ATTN_EHIP         (-4) /* HIP runtime error (no device, launch)   */

/* Bytes of the fixed device scratch v4attn_hca_attend_noalloc uses on each
 * GPU (24 MiB: the split partials of 32 decode queries x 64 heads x 512 dims
 * over 8 splits take 17.0 MB). */
#define V4ATTN_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)

/* v4attn_compress modes. */
#define V4ATTN_POOL 0 /* pool 2m-token windows into compressed entries     */
#define V4ATTN_PACK 1 /* one window row per raw token (no pooling)          */

/* Library version, (major << 16) | minor. */
int v4attn_version(void);

/* Static description of a status code. */
const char* v4attn_status_string(int status);

/* Message for the last failed call on this thread ("" if none). */
const char* v4attn_last_error(void);

/*
 * v4attn_compress -- sequence compression and window-row packing.
 *
 * Defines: per-token compression weights with positional biases over an
 * overlapping 2m-token window, one entry per m tokens ("Two ways to shrink
 * attention, interleaved"); the extra RMSNorm on entries and RoPE on their
 * last R dims (same section); BF16-rotary / FP8-rest storage ("The attention
 * stack, and why it is two mechanisms").
 *
 *   raw       bf16 [B, L, D]  raw latent c_t; row r is position raw_pos0 + r
 *   tok_score f32  [B, L]     per-token score s_t          (POOL only)
 *   pos_bias  f32  [2m]       positional bias b_0..b_2m-1  (POOL only)
 *   gamma     f32  [D]        RMSNorm gain
 *   mode      V4ATTN_POOL or V4ATTN_PACK
 *   m         compression ratio (POOL only; ignored by PACK)
 *   entry0, n_out
 *             POOL: entries j = entry0 .. entry0+n_out-1 are written.  Entry
 *             j pools positions [(j-1)m, (j+1)m) that exist (>= 0) with
 *             weights softmax(s_t + b_{t-(j-1)m}); every such position must
 *             lie in [raw_pos0, raw_pos0 + L), else V4ATTN_EINVAL.  Then
 *             RMSNorm(gamma, eps), RoPE at position j*m, pack.
 *             PACK: n_out rows are written, raw rows 0..n_out-1
 *             (n_out <= L), each RMSNorm'd, rotated at its own position and
 *             packed; entry0 is ignored.
 *   out       u8 [B, out_rows, D+R]: output i of sequence b goes to row
 *             b*out_rows + i (i = j - entry0 for POOL).  n_out <= out_rows.
 * FP8 values are rounded to nearest-even after clamping to +-448.
 *   raw_idx    bf16 [B, L, dI], nullable (POOL only): the tokens' indexer
 *              keys, pooled by the same compressor: entry j's indexer key is
 *              sum_t alpha_{j,t} kI_t with the entry's own weights, no norm,
 *              no rotation, bf16 (RNE) -> k_idx_out [B, out_rows, dI], rows
 *              as out (dI in {32, 64, 128})
 */
int v4attn_compress(const uint16_t* raw, const float* tok_score,
                    const float* pos_bias, const float* gamma,
                    int B, int L, int D, int R, int64_t raw_pos0,
                    int mode, int m, int64_t entry0, int n_out,
                    float eps, float rope_base,
                    uint8_t* out, int64_t out_rows,
                    const uint16_t* raw_idx, int dI, uint16_t* k_idx_out,
                    void* stream);

/*
 * v4attn_compress_step -- one decode step of the compressor, in one launch:
 * the window row of the new token at position t (as V4ATTN_PACK) and, when
 * t completes a group ((t+1) % m == 0), the compressed entry j = (t+1)/m - 1
 * it completes (as V4ATTN_POOL).  Same definitions and bytes as the two
 * v4attn_compress calls (the pooling over [(j-1)m, (j+1)m), RMSNorm, RoPE,
 * packing: "Two ways to shrink attention, interleaved").
 *
 *   raw        bf16 [B, L, D]  positions raw_pos0 .. raw_pos0+L-1; must hold
 *                              t and, for a completed entry, its window
 *   tok_score  f32 [B, L], pos_bias f32 [2m]  (needed only for an entry)
 *   gamma      f32 [D]
 *   entries    u8 [B, ent_rows, D+R] out: entry j at row j (nullable when
 *              no entry completes)
 *   win        u8 [B, win_rows, D+R] out: the new token's row at win_row
 *   seq_pos    host i64 [B], nullable: per-sequence token positions (a ragged
 *              batch, B <= 64); then t must be their largest, sequence b's
 *              raw rows are the L positions ending at seq_pos[b] (raw_pos0
 *              is ignored) and each sequence pools its own completed entry
 *   raw_idx    bf16 [B, L, dI], nullable: token indexer keys; a completed
 *              entry's pooled key (as v4attn_compress) -> k_idx [B, ent_rows,
 *              dI] row j
 * Errors: EINVAL for null/misaligned buffers, t outside the raw rows, a
 * window that starts before raw_pos0, j >= ent_rows or win_row out of range.
 */
int v4attn_compress_step(const uint16_t* raw, const float* tok_score, const float* pos_bias,
                         const float* gamma, int B, int L, int D, int R, int64_t raw_pos0,
                         int m, int64_t t, const int64_t* seq_pos, float eps,
                         float rope_base, uint8_t* entries,
                         int64_t ent_rows, uint8_t* win, int64_t win_rows, int64_t win_row,
                         const uint16_t* raw_idx, int dI, uint16_t* k_idx,
                         void* stream);

/*
 * v4attn_compress_steps -- v4attn_compress_step for n layers (1 <= n <= 2,
 * the same D) in one launch: each descriptor holds one layer's arguments,
 * with the meaning, checks and errors of v4attn_compress_step (the first
 * failing layer's status is returned and nothing is launched).  For a
 * decode step over an interleaved stack, whose layers' compress steps are
 * independent of each other.
 */
typedef struct {
  const uint16_t* raw;
  const float* tok_score;
  const float* pos_bias;
  const float* gamma;
  int B, L, D, R;
  int64_t raw_pos0;
  int m;
  int64_t t;
  const int64_t* seq_pos;
  float eps, rope_base;
  uint8_t* entries;
  int64_t ent_rows;
  uint8_t* win;
  int64_t win_rows, win_row;
  const uint16_t* raw_idx;
  int dI;
  uint16_t* k_idx;
} v4attn_compress_step_desc;
int v4attn_compress_steps(const v4attn_compress_step_desc* steps, int n,
                          void* stream);

/*
 * Ragged batches (v4attn_index_topk, v4attn_index_score,
 * v4attn_topk_select, v4attn_csa_attend, v4attn_hca_attend): seq_pos is a
 * nullable HOST array i64 [B] (B <= 64) of per-sequence positions; sequence
 * b's query r is then at seq_pos[b] + r (its window buffer rows relative to
 * seq_pos[b]), and q_pos0 must equal the largest of them (it sizes the
 * workspaces and is validated as before).  NULL: every sequence at q_pos0.
 */

/*
 * v4attn_index_topk -- lightning-indexer scores and top-k selection.
 *
 * Defines: a lightweight indexer scores each query against every compressed
 * entry and a top-k selector keeps the best k (k = 1024 in V4-Pro) ("Two
 * ways to shrink attention, interleaved"; "DeepSeek-V4, explained", steps 3
 * and 4 of how one query's layer works).  The score form is the ReLU-weighted
 * head sum score_{t,j} = sum_h w_{t,h} ReLU(q_{t,h} . k_j) with ONE indexer
 * key per entry shared by all heads, accumulated in fp32 from bf16 inputs.
 *
 *   q_idx  bf16 [B, Tq, HI, dI]   indexer queries; query r is at q_pos0 + r
 *   w_idx  f32  [B, Tq, HI]       per-query head weights
 *   k_idx  bf16 [B, Ncap, dI]     indexer keys, entry j at row j
 *   n_entries  entries that exist (<= Ncap)
 *   m          compression ratio: query at t sees j < V_t =
 *              min(n_entries, floor((t+1)/m))
 *   topk   i32  [B, Tq, k] out    the min(k, V_t) best entries under
 *              (score descending, index ascending) -- ties go to the lower
 *              entry index -- written in ascending index order, then -1.
 *   topk_score f32 [B, Tq, k] out, nullable: their scores (-inf for -1).
 *   ws / ws_bytes  device workspace of at least
 *              v4attn_index_topk_workspace(...) bytes; contents on entry
 *              are ignored.
 * NaN scores are never selected.
 */
size_t v4attn_index_topk_workspace(int B, int Tq, int64_t n_entries,
                                   int64_t q_pos0, int m, int k);
int v4attn_index_topk(const uint16_t* q_idx, const float* w_idx,
                      const uint16_t* k_idx, int B, int Tq, int HI, int dI,
                      int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                      const int64_t* seq_pos, int m,
                      int k, int32_t* topk, float* topk_score,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * v4attn_index_score / v4attn_topk_select -- the two halves of
 * v4attn_index_topk, for callers that want the raw indexer scores (same
 * definitions as above).
 *
 * v4attn_index_score writes scores f32 [B*Tq, score_stride]: row b*Tq + r
 * holds score_{t,j} for j < V_t (t = q_pos0 + r); the rest of the row is not
 * written.  score_stride >= min(n_entries, floor((q_pos0+Tq)/m)).
 *
 * v4attn_topk_select reads such a score buffer and writes topk (and
 * topk_score, nullable) exactly as v4attn_index_topk does; its workspace is
 * at least v4attn_topk_select_workspace(...) bytes (0 is possible: then ws
 * may be NULL).
 */
int v4attn_index_score(const uint16_t* q_idx, const float* w_idx,
                       const uint16_t* k_idx, int B, int Tq, int HI, int dI,
                       int64_t Ncap, int64_t n_entries, int64_t q_pos0,
                       const int64_t* seq_pos, int m,
                       float* scores, int64_t score_stride, void* stream);
size_t v4attn_topk_select_workspace(int B, int Tq, int64_t n_entries,
                                    int64_t q_pos0, int m, int k);
int v4attn_topk_select(const float* scores, int64_t score_stride, int B,
                       int Tq, int64_t n_entries, int64_t q_pos0,
                       const int64_t* seq_pos, int m, int k,
                       int32_t* topk, float* topk_score, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * v4attn_index_score_fp8 / v4attn_index_topk_fp8 -- the lightning indexer
 * with FP8 inputs.
 *
 * Defines: the indexer is a few small heads run in FP8 ("DeepSeek-V4,
 * explained", step 3 of how one query's layer works; "DeepSeek-V4: Making a
 * Million Tokens Affordable", section "Two ways to shrink attention,
 * interleaved", on the indexer's reduced precision).  Queries and keys are OCP
 * E4M3FN codes, each row with a positive fp32 scale:
 *   score_{t,j} = sum_h w_{t,h} ReLU((sq_{t,h} q8_{t,h}) . (sk_j k8_j)),
 * formed on the FP8 matrix cores as sk_j * sum_h (w_{t,h} sq_{t,h})
 * ReLU(q8_{t,h} . k8_j) (exact E4M3 products, fp32 accumulation; w sq is one
 * fp32 product).  Visibility, top-k rule and outputs are those of
 * v4attn_index_topk / v4attn_index_score.
 *
 *   q8       u8  [B, Tq, HI, dI]  E4M3 indexer queries (16-byte aligned)
 *   q_scale  f32 [B, Tq, HI]      per query head, > 0
 *   w_idx    f32 [B, Tq, HI]      per-query head weights
 *   k8       u8  [B, Ncap, dI]    E4M3 indexer keys (16-byte aligned)
 *   k_scale  f32 [B, Ncap]        per key, > 0 (a scale <= 0 or not finite
 *                                 gives scores the formula above does not)
 *   dI in {64, 128}; HI <= 64.  The workspace of v4attn_index_topk_fp8 is
 *   v4attn_index_topk_workspace(...) bytes; contents on entry are ignored.
 * q8 and k8 must hold finite codes (0x7F and 0xFF are NaN in E4M3FN).
 */
int v4attn_index_score_fp8(const uint8_t* q8, const float* q_scale, const float* w_idx,
                           const uint8_t* k8, const float* k_scale, int B, int Tq, int HI,
                           int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m,
                           float* scores, int64_t score_stride, void* stream);
int v4attn_index_topk_fp8(const uint8_t* q8, const float* q_scale, const float* w_idx,
                          const uint8_t* k8, const float* k_scale, int B, int Tq, int HI,
                          int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m,
                          int k, int32_t* topk, float* topk_score, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * v4attn_index_score_mxfp4 / v4attn_index_topk_mxfp4 -- the lightning
 * indexer with MXFP4 inputs.
 *
 * Defines: V4 runs the indexer's attention in FP4 ("DeepSeek-V4: Making a
 * Million Tokens Affordable", section "Two ways to shrink attention,
 * interleaved").  Queries and keys are in the OCP MX FP4 format: E2M1
 * elements, two per byte (the lower-indexed one in the low nibble), one
 * E8M0 scale byte (2^(x-127)) per 32 consecutive dims.  The score is the one
 * of v4attn_index_topk on the dequantised rows, sum_h w_h ReLU(q_h . k_j),
 * formed on the FP4 matrix cores (the MX blocks go in as stored; fp32
 * accumulation).  Visibility, top-k rule and outputs as v4attn_index_topk.
 *
 *   q4    u8  [B, Tq, HI, dI/2]   packed E2M1 queries (16-byte aligned)
 *   q_sc  u8  [B, Tq, HI, dI/32]  E8M0 scales of the queries
 *   w_idx f32 [B, Tq, HI]         per-query head weights
 *   k4    u8  [B, Ncap, dI/2]     packed E2M1 keys (16-byte aligned)
 *   k_sc  u8  [B, Ncap, dI/32]    E8M0 scales of the keys (dI/32-byte aligned)
 *   dI in {64, 128}; HI <= 64.  Scale byte 255 (NaN) gives unspecified
 *   scores.  The workspace of v4attn_index_topk_mxfp4 is
 *   v4attn_index_topk_workspace(...) bytes; contents on entry are ignored.
 */
int v4attn_index_score_mxfp4(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                             const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI,
                             int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m,
                             float* scores, int64_t score_stride, void* stream);
int v4attn_index_topk_mxfp4(const uint8_t* q4, const uint8_t* q_sc, const float* w_idx,
                            const uint8_t* k4, const uint8_t* k_sc, int B, int Tq, int HI,
                            int dI, int64_t Ncap, int64_t n_entries, int64_t q_pos0, int m,
                            int k, int32_t* topk, float* topk_score, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * v4attn_csa_attend -- CSA core attention: shared-KV multi-query attention
 * over the selected entries plus the uncompressed window, with sink.
 *
 * Defines: attention runs over the selected positions only ("DeepSeek-V4,
 * explained", step 5); a sliding-window branch of uncompressed recent tokens
 * and a per-head attention sink ("The attention stack, and why it is two
 * mechanisms"); RMSNorm on queries, RoPE on the last 64 dims, an entry is
 * key and value, RoPE at -t on the output ("Two ways to shrink attention,
 * interleaved").  Window and selected rows share ONE softmax with the sink:
 *   q~  = RoPE_t(RMSNorm_gamma_q(q)),  l_x = scale * q~ . x,
 *   p_x = exp(l_x) / (exp(sink_h) + sum_y exp(l_y)),
 *   out = RoPE_{-t}(sum_x p_x x),      lse = log(exp(sink_h) + sum exp(l)).
 *
 *   q       bf16 [B, Tq, H, D]      query r at position t = q_pos0 + r
 *   entries u8   [B, Ncap, D+R]     packed compressed entries
 *   topk    i32  [B, Tq, k]         entry indices; values outside
 *                                   [0, Ncap) (e.g. -1) are skipped
 *   win     u8   [B, Tq+W-1, D+R]   packed window rows; row r is position
 *                                   q_pos0-(W-1)+r.  The query at t uses
 *                                   positions max(0, t-W+1)..t.
 *   gamma_q f32 [D] (16-byte aligned);  sink f32 [H]
 *   out     bf16 [B, Tq, H, D] out;  lse f32 [B, Tq, H] out, nullable
 *   ws / ws_bytes  >= v4attn_csa_attend_workspace(...) bytes (split
 *              partials of long rows; 0 is possible); contents on entry are
 *              ignored
 * Accumulation is fp32; a long row's split partials are kept as 16-bit
 * integers with one power-of-two scale per split and head (every element
 * within 2^-15 of the head's largest).  On the E4M3 dims q~ (fp32)
 * enters the FP8 matrix cores as the sum of two E4M3 terms (its rounding and
 * the rounding of the remainder: at least bf16's eight significant bits), and
 * so do the probabilities (each 64-row block of a head scaled by its own
 * power of two, which the cores undo); on the bf16 dims both are rounded to
 * bf16.  Rows are never widened: the E4M3 bytes go into the matrix cores as
 * stored.
 */
size_t v4attn_csa_attend_workspace(int B, int Tq, int H, int D, int k, int W);
int v4attn_csa_attend(const uint16_t* q, const uint8_t* entries,
                      const int32_t* topk, const uint8_t* win,
                      const float* gamma_q, const float* sink,
                      int B, int Tq, int H, int D, int R, int64_t Ncap,
                      int k, int W, int64_t q_pos0,
                      const int64_t* seq_pos, float scale, float eps,
                      float rope_base, uint16_t* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * v4attn_hca_attend -- HCA core attention: dense attention over every
 * visible compressed entry plus the same window and sink.
 *
 * Defines: heavy compression (m' = 128) with fully dense attention over the
 * result plus the same sliding-window branch ("Two ways to shrink
 * attention, interleaved"; "DeepSeek-V4" visual-learn notes, "A coarse
 * overview alongside local detail").  As v4attn_csa_attend, except that the
 * query at t attends to every entry j < min(n_entries, floor((t+1)/m)).
 *
 *   entries u8 [B, Ncap, D+R]; n_entries <= Ncap
 */
size_t v4attn_hca_attend_workspace(int B, int Tq, int H, int D,
                                   int64_t n_entries, int m, int64_t q_pos0,
                                   int W);
int v4attn_hca_attend(const uint16_t* q, const uint8_t* entries,
                      const uint8_t* win, const float* gamma_q,
                      const float* sink, int B, int Tq, int H, int D, int R,
                      int64_t Ncap, int64_t n_entries, int m, int W,
                      int64_t q_pos0, const int64_t* seq_pos, float scale, float eps, float rope_base,
                      uint16_t* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * v4attn_hca_attend_noalloc -- v4attn_hca_attend without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Arguments, results and errors as v4attn_hca_attend (the outputs are
 * identical to its); the split partials go to a fixed scratch array the
 * library holds on each GPU (V4ATTN_NOALLOC_SCRATCH_BYTES, kept until the
 * process ends) instead of a caller's workspace.  The call allocates and
 * frees nothing.  A call whose partials need more than the scratch holds
 * returns V4ATTN_EWORKSPACE and launches nothing.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents (nothing
 * in it needs to start at zero): calls that overlap on one GPU (e.g. on two
 * streams) race and must be serialised by the caller.  The first call on a
 * device looks up that device's copy of the scratch (hipGetSymbolAddress).
 */
int v4attn_hca_attend_noalloc(const uint16_t* q, const uint8_t* entries,
                              const uint8_t* win, const float* gamma_q,
                              const float* sink, int B, int Tq, int H, int D,
                              int R, int64_t Ncap, int64_t n_entries, int m,
                              int W, int64_t q_pos0, const int64_t* seq_pos,
                              float scale, float eps, float rope_base,
                              uint16_t* out, float* lse, void* stream);

/*
 * v4attn_nsa_attend -- the NSA-style compress-select-window variant: a
 * compressed branch over the visible compressed entries, a selected branch
 * over the full-fidelity tokens of the n_sel best blocks, a window branch,
 * mixed per query and head by three gates.
 *
 * Defines: NSA scores blocks with attention over compressed block
 * representations, keeps the k best blocks at full fidelity plus a sliding
 * window of recent tokens, and mixes the compressed, selected and window
 * outputs with learned gates ("DeepSeek-V4, explained", the numbered steps of
 * how a compress-then-select layer handles one query: scoring, top-k,
 * combining branches).  The page gives no formulas; this library reads them
 * as follows, with q~, logits, the -t output rotation and the packed row
 * format exactly as v4attn_csa_attend, and NO sink in any branch:
 *   V_t    = min(n_entries, floor((t+1)/m)) visible entries;
 *   o_cmp  = attention over entries 0..V_t-1, probabilities p_{h,j};
 *   block j = tokens [j m, (j+1) m) (the tokens entry j summarises);
 *   s_j    = sum_h p_{h,j};  the n_sel best blocks by s (ties to the lower
 *            block; fewer than n_sel visible -> all of them, -1 padded);
 *   o_slc  = attention over the tokens of the selected blocks;
 *   o_win  = attention over the window positions max(0, t-W+1)..t;
 *   out    = g0 o_cmp + g1 o_slc + g2 o_win  (a branch with no rows is 0).
 *
 *   q       bf16 [B, Tq, H, D]        query r at position t = q_pos0 + r
 *   entries u8   [B, Ncap, D+R]       packed compressed entries
 *   tokens  u8   [B, Ntok, D+R]       packed full-fidelity rows, row i =
 *                                     position i; Ntok >= V_t m for every
 *                                     query of the block
 *   win     u8   [B, Tq+W-1, D+R]     packed window rows (as csa_attend)
 *   gamma_q f32 [D] (16-byte aligned)
 *   gates   f32  [B, Tq, H, 3]        (compressed, selected, window)
 *   out     bf16 [B, Tq, H, D] out
 *   blocks  i32  [B, Tq, n_sel] out, nullable: the selected blocks,
 *           ascending, -1 padded
 *   block_score f32 [B, Tq, n_sel] out, nullable: their scores s_j
 *   ws / ws_bytes  >= v4attn_nsa_attend_workspace(...) bytes, 16-byte
 *           aligned; holds the compressed branch's logits (B Tq H V_max
 *           floats) and every intermediate; contents on entry are ignored
 * 1 <= n_sel, n_sel m <= 4096, 1 <= m <= 256.  Accumulation is fp32; the
 * branch outputs are rounded to bf16 before the gated sum (in fp32).
 * Errors: V4ATTN_EINVAL / EUNSUPPORTED / EWORKSPACE as the other calls; on an
 * error nothing is launched.
 */
size_t v4attn_nsa_attend_workspace(int B, int Tq, int H, int D,
                                   int64_t n_entries, int m, int64_t q_pos0,
                                   int W, int n_sel);
int v4attn_nsa_attend(const uint16_t* q, const uint8_t* entries,
                      const uint8_t* tokens, const uint8_t* win,
                      const float* gamma_q, const float* gates,
                      int B, int Tq, int H, int D, int R, int64_t Ncap,
                      int64_t n_entries, int m, int64_t Ntok, int W,
                      int n_sel, int64_t q_pos0, float scale, float eps,
                      float rope_base, uint16_t* out, int32_t* blocks,
                      float* block_score, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * v4attn_csa_attend_backward / v4attn_hca_attend_backward -- gradients of
 * v4attn_csa_attend / v4attn_hca_attend.
 *
 * Defines: the attention step is trained end to end except the top-k choice,
 * a hard selection with no gradient ("DeepSeek-V4, explained", step 7); the
 * selected set and the window are therefore constants here.  The chain rule
 * of the forward's definition (q~ = RoPE_t(RMSNorm_gamma_q(q)), l = scale
 * q~ . x, one softmax with the sink, out = RoPE_{-t}(sum p x)):
 *   do = RoPE_t(dout),  D_h = dout_h . out_h,  dl_x = p_x (do . x - D_h),
 *   d x     += scale sum_h dl_hx q~_h + sum_h p_hx do_h   (key and value)
 *   d sink_h += -exp(sink_h - lse_h) D_h
 *   dq       = RMSNorm backward of RoPE_t^T(scale sum_x dl_x x);
 *   d gamma_q += its gamma part.
 * A row's gradient is taken with respect to its stored (dequantised) value.
 *
 *   q, entries, topk, win, gamma_q, sink, sizes: as the forward call
 *   out  bf16 [B, Tq, H, D], lse f32 [B, Tq, H]: the forward's outputs
 *   dout bf16 [B, Tq, H, D]: gradient of out (16-byte aligned)
 *   dq   f32  [B, Tq, H, D] out (written, 16-byte aligned)
 *   d_entries f32 [B, Ncap, D], d_win f32 [B, Tq+W-1, D]: ADDED to (the
 *            caller zeroes them); required when Ncap > 0 / W > 0
 *   d_sink f32 [H], d_gamma_q f32 [D]: added to; nullable
 *   p_sel f32 [B, Tq, k] (CSA only, nullable): written with sum_h p_hx of
 *            every top-k slot (0 for -1 slots): the indexer loss's target
 *   ws / ws_bytes: device workspace, 16-byte aligned.  With the bytes the
 *            matching *_backward_workspace(...) query returns, the row
 *            gradients are grouped: every (query, row slot) gradient is
 *            stored densely as a 24-bit float (fp32 rounded to 16 mantissa
 *            bits, nearest even; at most 12 GiB per group of queries), the
 *            slots are sorted by destination row and each row is added to
 *            once in fp32.
 *            A smaller workspace (fewer queries per group) or, down to the
 *            per-chunk buffers alone (the minimum V4ATTN_EWORKSPACE
 *            reports), d_entries / d_win not 16-byte aligned or ids past
 *            32 bits add the row gradients with fp32 atomics instead; the
 *            results agree to rounding.  The queries' Ncap is the entry
 *            capacity of d_entries (the destinations the sort counts).
 * Arithmetic: every attended row is gathered as bf16 (exact); q~, do and the
 * probabilities and dl enter bf16 matrix-core products with fp32
 * accumulation.  A row shared by several queries gets their gradients in an
 * order that varies from run to run (the sort by destination, or the
 * atomics), so the last bits of those rows vary too.
 */
size_t v4attn_csa_attend_backward_workspace(int B, int Tq, int H, int D,
                                            int k, int W, int64_t Ncap);
int v4attn_csa_attend_backward(const uint16_t* q, const uint8_t* entries,
                               const int32_t* topk, const uint8_t* win,
                               const float* gamma_q, const float* sink,
                               int B, int Tq, int H, int D, int R,
                               int64_t Ncap, int k, int W, int64_t q_pos0,
                               float scale, float eps, float rope_base,
                               const uint16_t* out, const float* lse,
                               const uint16_t* dout, float* dq,
                               float* d_entries, float* d_win, float* d_sink,
                               float* d_gamma_q, float* p_sel, void* ws,
                               size_t ws_bytes, void* stream);
size_t v4attn_hca_attend_backward_workspace(int B, int Tq, int H, int D,
                                            int64_t n_entries, int m,
                                            int64_t q_pos0, int W,
                                            int64_t Ncap);
int v4attn_hca_attend_backward(const uint16_t* q, const uint8_t* entries,
                               const uint8_t* win, const float* gamma_q,
                               const float* sink, int B, int Tq, int H, int D,
                               int R, int64_t Ncap, int64_t n_entries, int m,
                               int W, int64_t q_pos0, float scale, float eps,
                               float rope_base, const uint16_t* out,
                               const float* lse, const uint16_t* dout,
                               float* dq, float* d_entries, float* d_win,
                               float* d_sink, float* d_gamma_q, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * v4attn_compress_backward -- gradient of v4attn_compress (POOL) for entries
 * entry0 .. entry0+n_out-1 with respect to the raw latents, token scores,
 * positional biases and gamma.
 *
 * Defines: as v4attn_compress (weights softmax(s_t + b_{t-(j-1)m}) over
 * [(j-1)m, (j+1)m), pool, RMSNorm, RoPE at j m); trained end to end
 * ("DeepSeek-V4, explained", step 7).  d_entries is the gradient with
 * respect to the entries' stored values: the E4M3 / bf16 rounding is passed
 * straight through.
 *   raw, tok_score, pos_bias, gamma, sizes, raw_pos0, m, entry0, n_out: as
 *        the forward (the windows must lie in the rows)
 *   d_entries f32 [B, n_out, D]
 *   d_raw f32 [B, L, D], d_score f32 [B, L]: added to
 *   d_bias f32 [2m], d_gamma f32 [D]: added to, nullable
 * fp32 arithmetic; a token is in two windows, so its gradients are added
 * with atomics (the last bits vary from run to run).
 */
int v4attn_compress_backward(const uint16_t* raw, const float* tok_score,
                             const float* pos_bias, const float* gamma, int B,
                             int L, int D, int R, int64_t raw_pos0, int m,
                             int64_t entry0, int n_out, float eps,
                             float rope_base, const float* d_entries,
                             float* d_raw, float* d_score, float* d_bias,
                             float* d_gamma, void* stream);

/*
 * v4attn_index_kl_backward -- the indexer's KL alignment loss over one entry
 * set per query and its gradients with respect to q^I, w and k^I.
 *
 * Defines: DSA trains its lightning indexer with a KL-divergence loss that
 * pulls the indexer's scores toward the main attention's distribution, with
 * the indexer's input detached, first over every entry, then over the
 * selected ones ("DeepSeek-V4, explained", step 7).  Reading: over the set
 * S of a query (sel, -1 slots excluded), P_j = target_j / sum_S target
 * (target: the attention probabilities of the entries summed over heads,
 * e.g. p_sel of v4attn_csa_attend_backward), Q = softmax_S(score) with the
 * score of v4attn_index_score, loss = sum_j P_j (log P_j - log Q_j);
 * d score_j = Q_j - P_j; P is a constant.
 *   q_idx bf16 [B, Tq, HI, dI], w_idx f32 [B, Tq, HI], k_idx bf16 [B, Ncap, dI]
 *   (q_idx and k_idx 16-byte aligned)
 *   sel i32 [B, Tq, ns], target f32 [B, Tq, ns]
 *   loss f32 [B, Tq] (written, nullable); dq_idx f32 [B, Tq, HI, dI] and
 *   dw_idx f32 [B, Tq, HI] (written); dk_idx f32 [B, Ncap, dI] (added to)
 *   ws / ws_bytes: device workspace, 16-byte aligned.  With the bytes of
 *            v4attn_index_kl_backward_workspace(B, Tq, dI, ns, Ncap) and a
 *            16-byte aligned dk_idx, the key gradients are grouped: every
 *            (query, slot) dk row is stored densely as 24-bit floats (fp32
 *            rounded to 16 mantissa bits, nearest even; at most 12 GiB per
 *            group of queries), the slots are sorted by entry and each
 *            entry's row is added to once in fp32.  A smaller workspace, down to the
 *            per-chunk buffers (the minimum V4ATTN_EWORKSPACE reports), adds
 *            the dk rows with fp32 atomics instead.
 * 1 <= ns <= 4096, dI in {32, 64, 128}, HI <= 64.  q^I.k^I in fp32 from the
 * bf16 inputs (exact products); ds w [q.k > 0] enters the dq and dk
 * products as bf16; an entry chosen by several queries gets their dk rows
 * in an order that varies from run to run (the last bits vary).
 */
size_t v4attn_index_kl_backward_workspace(int B, int Tq, int dI, int ns, int64_t Ncap);
int v4attn_index_kl_backward(const uint16_t* q_idx, const float* w_idx,
                             const uint16_t* k_idx, const int32_t* sel,
                             const float* target, int B, int Tq, int HI,
                             int dI, int64_t Ncap, int ns, float* loss,
                             float* dq_idx, float* dw_idx, float* dk_idx,
                             void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* V4ATTN_H */
