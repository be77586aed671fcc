// Internal launch interface between the host side (api.cpp) and the kernels.  Not part of the ABI.
#pragma once
#include "common.h"
#include "../../include/dflash.h"

namespace df {

// ---------------------------------------------------------------- GEMM: Y = X W^T with fused epilogues
constexpr int kGemmMaxSeg = 16;
constexpr int kGemmMaxRows = 64;  // X operand rows per launch (low planes included); the host chunks longer inputs

enum EpiKind { EPI_STORE_F32 = 0, EPI_PARTIAL = 2, EPI_SWIGLU = 3, EPI_RESID_NORM = 4 };
enum SegRole { ROLE_PLAIN = 0, ROLE_Q = 1, ROLE_K = 2, ROLE_V = 3 };

struct GemmSeg {
  const void *w;  // [n, K] row-major weight rows of this segment
  int32_t n;      // rows
};

struct GemmArgs {
  const void *x;  // X in the activation type (fp16 for bf16 models, see ActOf)
  int32_t ldx;
  int32_t M, N, K;      // N: output columns (SWIGLU: ffn width; otherwise total segment rows)
  int32_t nseg;         // segments concatenated along N (SWIGLU: 0 = gate, 1 = up)
  GemmSeg seg[kGemmMaxSeg];
  int32_t epi;
  float *out_f32;       // EPI_STORE_F32; EPI_PARTIAL: K range s writes out_f32 + s * part_stride
  void *out_act;        // EPI_SWIGLU (an X operand, activation type)
  int32_t ld_out;
  int32_t ksplit;       // K ranges, one per grid row (> 1 only with EPI_PARTIAL)
  int64_t part_stride;  // EPI_PARTIAL: elements between the K ranges' output slices
  int32_t row_off;      // global row of local row 0
  // Optional selection of the X rows (x_take > 0): global row r reads X row (r / x_take) * x_stride +
  // x_off + r % x_take of the unmoved x -- e.g. the last x_take of every x_stride rows.
  // Without it local row r reads X row r of x (row chunks move x).
  int32_t x_take, x_stride, x_off;
  // Optional RMSNorm of the X rows, applied to Y (EPI_STORE_F32, EPI_PARTIAL, EPI_SWIGLU): X holds
  // act(x * gain) and Y[m] is scaled by rstd[m] = 1 / sqrt(sum_p ss_in[(row_off + m) * ss_ld + p] /
  // norm_dim + eps), the ss_n partial sums of squares added in order (ss_ld a multiple of 4).
  const float *ss_in;
  int32_t ss_n, ss_ld, norm_dim;
  float eps;
  // EPI_RESID_NORM (32-column tiles): v = (resid ? resid[m][n] : 0) + Y[m][n]; resid[m][n] = v;
  // feat[m][n] = act(v) (optional); rows selected by (sel_take, sel_stride, sel_offset), compacted to
  // o = (r / sel_stride) * sel_take + r % sel_stride - sel_offset, also get xg[o][n] = act(v * gain[n])
  // and ss_out[o * ss_out_ld + tile] = the sum of v^2 over the tile's 32 columns (the next projection's
  // ss_in, ss_n = N / 32).
  // feat and xg are X operands of later projections (activation type).
  float *resid;
  int32_t ld_resid;
  void *feat;
  int32_t ld_feat;
  const float *gain;
  void *xg;
  int32_t ld_xg;
  float *ss_out;
  int32_t ss_out_ld;
  int32_t sel_take, sel_stride, sel_offset;
  // Optional stream-K scratch (null: one work-group per tile).  With it, at most 16 X operand rows (M,
  // or 2M with a low plane), ksplit 1 and K a whole number of 256-byte super-steps, the launcher may
  // spread the projection's (tile, super-step)
  // items evenly over one work-group per CU: sk_part holds 2 * kSkTileElems fp32 partial-tile entries
  // per work-group (at most sk_max_wg work-groups), sk_cnt one arrival counter per tile (at most
  // sk_max_tiles), zero before the launch and zero again after it.
  float *sk_part;
  int32_t *sk_cnt;
  int32_t sk_max_wg, sk_max_tiles;
  int32_t sk_force;  // take the stream-K kernel whatever the epilogue (launch_gemm fails if it cannot)
};
constexpr int kSkTileElems = 16 * 32;  // entries of one partial tile (16 rows x 32 columns)
constexpr int kSkMaxWg = 1024;         // stream-K work-groups at most (one per CU)
// Stream-K scratch of a projection with N output columns, as one block: the partial tiles of up to
// kSkMaxWg work-groups (fp32), then one arrival counter per 16-column tile (int32, zero between launches).
constexpr size_t kSkPartBytes = (size_t)kSkMaxWg * 2 * kSkTileElems * sizeof(float);
inline size_t sk_scratch_bytes(int N) { return kSkPartBytes + (size_t)(N / 16) * sizeof(int32_t); }
// Zero n int32 values (a fill kernel, so that the call may be captured into a graph).
hipError_t launch_zero_i32(int32_t *p, int32_t n, hipStream_t s);

// dtype: 0 bf16, 1 fp32.  e0 / e1 (may be null): events recorded at the kernel's start and end.
hipError_t launch_gemm(const GemmArgs &a, int dtype, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// K ranges for an EPI_PARTIAL projection of M rows: enough work-groups to cover the CUs several times
// over, each range a whole number of 256-byte super-steps, and split * M * N <= cap_elems.
int gemm_ksplit(int M, int N, int K, int dtype, size_t cap_elems);

// Tiled MFMA projection over many rows (gemm_tc.hip): X in fp16 (no deferred
// norm), the bf16 weights are converted to fp16 as they are staged.  EPI_STORE_F32, EPI_PARTIAL (with
// up to kTcMaxRanges K ranges, range z at out_f32 + z * part_stride) and EPI_SWIGLU (fp16 activation).
// bm: tile rows (64 / 128 / 256); um: units of 32 weight rows per chunk at most; nch: chunks of the
// units (grid x); ranges, steps: K ranges (grid z) and 64-wide K steps per range; nwv: waves per work-group.
struct TcPlan {
  int bm, um, nch, ranges, steps;
  int nwv;  // waves per work-group (4 or 8)
};
constexpr int kTcMaxRanges = 8;
// false if the projection does not suit the kernel; range_cap: elements available for ranges * M * N
bool gemm_tc_plan(const GemmArgs &a, int64_t range_cap, TcPlan *p);
hipError_t launch_gemm_tc(const GemmArgs &a, const TcPlan &p, hipStream_t s, hipEvent_t e0 = nullptr,
                          hipEvent_t e1 = nullptr);

// Per-head q/k RMSNorm + RoPE, then q to a dense buffer and k/v to the paged cache.
struct PostSeg {
  int32_t heads;
  int32_t role;       // ROLE_Q / ROLE_K / ROLE_V
  const float *gain;  // head-dim RMSNorm gain (Q, K)
  void *dst;          // Q: dense [rows][ld_dst]; K/V: KV pool base of the layer
  int32_t ld_dst;
};
struct QkvPostArgs {
  const float *src;  // [n_part][rows][ld_src] fp32 partial projections, summed in order
  int32_t ld_src;
  int32_t n_part;
  int64_t part_stride;
  int32_t n_rows;
  int32_t nseg;
  PostSeg seg[kGemmMaxSeg];
  int32_t total_heads;
  Rows rows;
  const int32_t *block_table;
  int32_t bt_stride;
  KVLayout kv;
  const float2 *rope;  // [position][head_dim / 2] (cos, sin) of the rotary angles
  int32_t rope_rows;   // positions in the table
  float eps;
  int32_t *err;
};
hipError_t launch_qkv_post(const QkvPostArgs &a, int dtype, hipStream_t s);

// ---------------------------------------------------------------- small kernels
struct PrepArgs {
  int32_t batch;
  int32_t slots[64];
  int32_t q_len;
  int32_t new_sequence;
  SlotState *state;
  Rows rows;
  const int32_t *tokens;  // verify: caller tokens [batch*q_len]
  int32_t mode;           // 0 verify, 1 draft-inject rows, 2 draft block rows
  int32_t row_skip;       // mode 1: the call's rows of a sequence are the verified rows row_skip .. + q_len - 1
  int32_t mask_id;
  int32_t vocab;
  int32_t *block_out;     // mode 2: block[b * q_len] = anchor
  int32_t *err;
};
hipError_t launch_prep(const PrepArgs &a, hipStream_t s);

// x[r] = embed[tok[r]] (fp32 residual stream)
hipError_t launch_embed(const void *embed, int dtype, const Rows &rows, int32_t n_rows, int32_t hidden, int32_t vocab,
                        float *x, int32_t *err, hipStream_t s);

// Residual update + RMSNorm over n_rows rows r:
//   v = (x ? x[r] : 0) + sum_s part[s][r]   (s in order; part may be null)
//   x[r] = v (if x), feat[r] = act(v) (if feat),
//   and, when offset <= r % stride < offset + take, out[(r / stride) * take + r % stride - offset] =
//   act(v / sqrt(mean(v^2) + eps) * gain).
struct NormArgs {
  float *x;
  int32_t ld_x;
  const float *part;
  int32_t n_part, ld_part;
  int64_t part_stride;
  void *feat;            // X operand (activation type)
  int32_t ld_feat;
  const float *gain;
  float eps;
  int32_t hidden;
  void *out;             // X operand (activation type)
  int32_t ld_out;
  int32_t n_rows, take, stride, offset;
  // Deferred normalisation: when set, selected rows get out = act(v * gain) (no 1/rms factor) and
  // ss_out[o * ss_ld] = sum of v^2 (a single partial for a projection's ss_in, ss_n = 1).
  float *ss_out;
  int32_t ss_ld;
};
hipError_t launch_norm(const NormArgs &a, int dtype, hipStream_t s);

// table[p][i] = (cos, sin) of p * theta^(-2 i / head_dim), angles in fp64, for p < n_pos, i < head_dim / 2
hipError_t launch_rope_table(float2 *table, float theta, int32_t head_dim, int32_t n_pos, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void *q;
  int32_t ldq;
  const void *kv;  // layer pool base
  KVLayout kvl;
  const int32_t *block_table;
  int32_t bt_stride;
  Rows rows;
  int32_t n_seq, q_len;  // rows are [n_seq][q_len]
  int32_t q_heads;
  int32_t mode;          // 0 causal (keys <= query position); 1 draft (block keys + window context)
  int32_t window;        // draft: context key k allowed when qpos - k < window (0: unbounded)
  int32_t q_tile;        // query positions per work-group
  int32_t n_splits;      // key-range splits
  int32_t split_tokens;  // keys per split (multiple of page_tokens)
  float *part_o;         // [rows*q_heads][n_splits][head_dim]
  float *part_ml;        // [rows*q_heads][n_splits][2]
  void *out;             // [rows][q_heads*head_dim]: the o projection's X operand (activation type)
  int32_t ldo;
  int32_t *err;
  // Fused post-processing (calls with one query tile per sequence; q is then unused): q, k, v of the
  // block arrive as raw fp32 projections, row r at raw + r * ld_raw with q heads at column 0, k heads
  // at q_heads * d and v heads at (q_heads + kv_heads) * d.  Each work-group RMS-normalises (q_gain /
  // k_gain) and rotates its query vectors, writes the block's k / v that fall in its key range to the
  // pool, and the last split of a (sequence, KV head, query tile) to finish merges all splits
  // (counters: one per (sequence, KV head, query tile), zero between calls).
  const float *raw;
  int32_t ld_raw;
  const float *q_gain, *k_gain;
  float eps;
  const float2 *rope;
  int32_t rope_rows;
  int32_t *counters;
  // Host-known facts that shorten the kernel's dependent-load chain: abs_range = 1 when no sequence's
  // key range starts after key 0 (causal calls, or drafter calls whose allocated context fits the
  // window), so the block-table entries of a split are read up front; the slot of every sequence.
  // (Fields the kernel's prologue reads sit in the first 256 bytes; seq_slot follows.)
  int32_t abs_range;
  int32_t seq_slot[64];
};
hipError_t launch_attention(const AttnArgs &a, int dtype, hipStream_t s);
// Flash-style prefill attention (causal, fp16 models, head_dim 128, 16-token pages): whether a call
// with keys up to max_key_pos qualifies, and its launch (a.q, rows, block table, out as for
// launch_attention; no splits).
bool attn_prefill_fits(const AttnArgs &a, int dtype, int max_key_pos);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t s);

// ---------------------------------------------------------------- sampler
struct FilterArgs {
  const float *logits;  // [rows][vocab]
  int32_t rows, vocab;
  int32_t rows_per_seq;
  float temperature[64];  // per sequence; 0 = greedy
  int32_t top_k[64];
  float top_p[64];
  int32_t *cand_id;     // [rows][kMaxTopK]
  float *cand_p;        // [rows][kMaxTopK]
  int32_t *cand_n;      // [rows]
  // two-stage plan (filter_plan) and its scratch: [rows][n_chunks][kmax] candidate keys and ids
  int32_t chunk, n_chunks, kmax;
  uint32_t *stage_key;
  int32_t *stage_idx;
  // argmax mode (drafts): row r's argmax goes to argmax_out[(r / take) * stride + offset + r % take]
  int32_t *argmax_out;
  int32_t am_take, am_stride, am_offset;
  // score mode (the selector's candidates): the top_k ids and their scores z / T (z for T = 1) go to
  // cand_id / cand_s, no distribution
  float *cand_s;
};
constexpr int kMaxTopK = 256;
constexpr int kFilterScratch = 8192;  // stage-1 candidates per row (chunks * kmax)
void filter_plan(FilterArgs &a, int kmax);
hipError_t launch_filter(const FilterArgs &a, hipStream_t s);

// ---------------------------------------------------------------- DFlash2 drafter variants (dflash2.hip)
constexpr int kConvMaxTaps = 4;
constexpr int kSelMaxK = 32;
constexpr int kSelMaxSteps = DFLASH_MAX_BLOCK - 1;
// Dynamic convolution of the block rows x (the layer's attention input, rows b * block + i) into out.
struct ConvArgs {
  const void *x;     // [rows][ldx] activation type: act(x * gain) awaiting 1/rms (ss set) or normalised
  int32_t ldx;
  const float *ss;   // deferred-norm partial sums of squares of the rows (or null), ss_n per row
  int32_t ss_n, ss_ld;
  float eps;
  const float *u;    // [rows][ld_u] tap logits (group-major: u[g * taps + t]), already scaled by 1/rms
  int32_t ld_u;
  void *out;         // [rows][ld_out] activation type
  int32_t ld_out;
  int32_t rows, hidden, block, taps, group;
};
hipError_t launch_dyn_conv(const ConvArgs &a, int dtype, hipStream_t s);
// Selector over `batch` requests of nd draft rows with K candidates each.
struct SelArgs {
  int32_t batch, nd, K, rank, hidden, vocab;
  const int32_t *block;  // anchors at block[b * block_stride]
  int32_t block_stride;
  const int32_t *cand_id;  // [batch * nd][cand_ld] (logit desc, id asc)
  const float *cand_s;     // their logits
  int32_t cand_ld;
  const void *embed;       // [vocab][hidden] model type
  void *x;                 // gather output: [batch][1 + nd K][hidden] activation type
  const float *proj;       // [batch][1 + nd K][ld_proj] fp32: U E (rank r), then V E (rank r)
  int32_t ld_proj;
  float inv_sqrt_r;
  float *trans;            // [batch][nd][K][K] fp32 transitions (row 0 of the first: from the anchor)
  int32_t *out;            // drafts at out[b * block_stride + i], i = 1 .. nd
};
hipError_t launch_sel_gather(const SelArgs &a, int dtype, hipStream_t s);
hipError_t launch_sel_viterbi(const SelArgs &a, hipStream_t s);

struct DecideArgs {
  int32_t batch;
  int32_t slots[64];
  uint64_t seed[64];
  int32_t n_draft;
  const int32_t *block;   // [batch][n_draft + 1]: anchor, then drafts
  const int32_t *cand_id;
  const float *cand_p;
  const int32_t *cand_n;
  SlotState *state;
  int32_t *out;
  int32_t *n_out;
  int32_t *err;
  // Stochastic drafts (null: deterministic drafts): the drafter's candidate distribution of draft i of
  // request b at row b * n_draft + i - 1, [rows][kMaxTopK] ids (-1 past the kept ones) and fp32 p.
  const int32_t *q_id;
  const float *q_p;
};
hipError_t launch_decide(const DecideArgs &a, hipStream_t s);

// Stochastic drafts: draft i of request b (position seq_len + i) is drawn by inverse CDF from its
// candidate row b * nd + i - 1 with the uniform of Philox stream 1; the rows are then padded with
// -1 / 0 past their cand_n kept entries.
struct DraftSampleArgs {
  int32_t batch, nd, block;  // requests, drafts per request, block length (nd + 1)
  int32_t slots[64];
  uint64_t seed[64];
  const SlotState *state;
  int32_t *q_id;       // [batch * nd][kMaxTopK]
  float *q_p;          // [batch * nd][kMaxTopK]
  const int32_t *q_n;  // [batch * nd]
  int32_t *out;        // [batch][block]: draft i goes to out[b * block + i]
};
hipError_t launch_draft_sample(const DraftSampleArgs &a, hipStream_t s);

// ---------------------------------------------------------------- operator-level entry points (api.cpp)
// The projection on the stream-K kernel, scratch block at d_scratch (sk_scratch_bytes(N) bytes, 256-byte
// aligned): checks the arguments, zeroes the tile counters, launches.
dflash_status op_linear_sk(hipStream_t s, int32_t dtype, int32_t M, int32_t N, int32_t K, const void *d_x,
                           const void *d_w, float *d_y, void *d_scratch);
// Records msg as the calling thread's last error and returns st.
dflash_status set_error(dflash_status st, const char *msg);

// copy candidate lists out for tests
hipError_t launch_copy_cands(const int32_t *cid, const float *cp, const int32_t *cn, int32_t rows, int32_t *oid,
                             float *op, hipStream_t s);

}  // namespace df
