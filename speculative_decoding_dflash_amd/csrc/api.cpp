// Host side of libdflash: argument checking, workspace layout, KV page tables, and the launch
// sequences of the three step calls.  See include/dflash.h for the contract.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace df;

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIP_OK(expr)                                                                                 \
  do {                                                                                               \
    hipError_t e_ = (expr);                                                                          \
    if (e_ != hipSuccess) return fail(DFLASH_E_DEVICE, "%s: %s", #expr, hipGetErrorString(e_));      \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int esize(const dflash_model_cfg *c) { return c->dtype == DFLASH_BF16 ? 2 : 4; }
// Planes of a projection input (X operand): bf16 models hold a high and a low bf16 plane (store_x).

constexpr int kAttnSplitMax = 64;
constexpr int kAttnWgTarget = 512;  // work-groups a batched decode attention call aims at
constexpr int kAttnFusedMaxSeqs = 4;  // decode calls of more sequences post-process q / k / v separately
constexpr int kAttnWholeBlockPages = 256;  // key pages from which a batched call's work-groups hold whole blocks
constexpr int kMaxKSplit = 8;
// Calls of a bf16 model with at least this many rows run in x16 mode (dflash_ctx::x16).
constexpr int kTcMinRows = DFLASH_F16_MIN_ROWS;
constexpr size_t kTcRangeRows = 256;  // rows for which the workspace holds K-range partials
constexpr int kMaxQTiles = 64;  // query tiles per sequence in a decode-sized attention call

// Workspace carve-up; offsets in bytes.
struct Layout {
  size_t state, err, cnt, skc, bt, dbt, rows[3][4], x, xn, ss, rope, qbuf, attn, ffn, part, skp, tcr, att_o, att_ml, dlogits,
      cid, cp, cn, skey, sidx, cu, xc, sel_id, sel_s, sel_x, sel_y, sel_t, total;
  size_t part_elems, att_rows, tcr_elems;
  int ss_ld, sk_tiles;
};

// Pages per slot of the drafter's page ring ([P3] "结构一览": the drafter attends over a sliding window
// of W context keys).  A drafter call for a block at n reads keys [n - W + 1, n + B) and, after an accept
// of nd < B drafts, injects rows from n - nd - W at the lowest, so it touches fewer than W + 2 B
// consecutive positions, and keys older than the window are never read again: position p of a slot can
// live at ring position p mod R pt (page index i in ring page i mod R).  0 (no ring: the drafter shares
// the target's page ids) without a window, or when the ring would not make the drafter pool smaller.
int drafter_ring_pages(const dflash_drafter_cfg *d, const dflash_capacity *cap) {
  static const bool off = getenv("DFLASH_DRAFTER_RING") && atoi(getenv("DFLASH_DRAFTER_RING")) == 0;  // A/B runs
  if (off || d->window <= 0 || cap->page_tokens < 1) return 0;
  const int r = (d->window + 2 * d->block_size + cap->page_tokens - 1) / cap->page_tokens + 1;
  return r < cap->max_pages_per_seq && (int64_t)cap->max_slots * r < cap->num_pages ? r : 0;
}

Layout make_layout(const dflash_model_cfg *c, const dflash_drafter_cfg *d, const dflash_capacity *cap) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t R = cap->max_rows, H = c->hidden, QD = (size_t)c->q_heads * c->head_dim,
               KD = (size_t)c->kv_heads * c->head_dim, F = c->ffn, V = c->vocab, es = esize(c);
  const size_t B = d->block_size;
  L.state = take(sizeof(SlotState) * cap->max_slots);
  L.err = take(sizeof(int32_t) * ERR_COUNT);
  // attention merge counters, one per (slot, KV head, query tile of a block), zeroed
  L.cnt = take(sizeof(int32_t) * cap->max_slots * c->kv_heads * kMaxQTiles);
  // stream-K projection tile counters (16-column tiles of the widest projection output), zeroed
  L.sk_tiles = (int)(std::max({(size_t)c->ffn, (size_t)c->vocab, QD + 2 * KD, (size_t)d->layers * 2 * KD, H}) / 16);
  L.skc = take(sizeof(int32_t) * L.sk_tiles);
  L.bt = take(sizeof(int32_t) * cap->max_slots * cap->max_pages_per_seq);
  L.dbt = take(sizeof(int32_t) * cap->max_slots * cap->max_pages_per_seq);  // the drafter's page ring
  for (int s = 0; s < 3; ++s)
    for (int k = 0; k < 4; ++k) L.rows[s][k] = take(sizeof(int32_t) * R);
  L.x = take(sizeof(float) * R * H);
  // rotary (cos, sin) for every position a sequence can reach
  L.rope = take(sizeof(float) * 2 * (size_t)cap->max_pages_per_seq * cap->page_tokens * (c->head_dim / 2));
  // per-32-column sums of squares of the rows awaiting RMSNorm: [R][ss_ld]
  L.ss_ld = (int)((H / 32 + 3) / 4 * 4);
  L.ss = take(sizeof(float) * L.ss_ld * R);
  // projection inputs, q: the activation type (fp16 for bf16 models, fp32 otherwise)
  L.xn = take(es * R * H);
  L.qbuf = take(es * R * QD);
  L.attn = take(es * R * QD);
  L.ffn = take(es * R * F);
  // fp32 K-range partials of one projection: up to kMaxKSplit ranges of a single row chunk, or one
  // range over all rows
  const size_t part_cols = std::max({QD + 2 * KD, (size_t)d->layers * 2 * KD, H});
  L.part_elems = std::max(R, (size_t)kMaxKSplit * kGemmMaxRows) * part_cols;
  L.part = take(sizeof(float) * L.part_elems);
  L.skp = take(sizeof(float) * kSkMaxWg * 2 * kSkTileElems);  // stream-K partial tiles
  // K-range partials of a tiled fp16 projection over a decode batch (kTcMinRows .. kTcRangeRows rows):
  // room for kTcMaxRanges ranges of the widest partial output (the planner uses fewer ranges, or one
  // range in L.part, where they do not fit)
  const size_t rdec = std::min<size_t>((size_t)cap->max_slots * B, kTcRangeRows);
  L.tcr_elems = rdec >= (size_t)kTcMinRows ? kTcMaxRanges * rdec * part_cols : 0;
  L.tcr = take(sizeof(float) * std::max<size_t>(L.tcr_elems, 1));
  L.att_rows = (size_t)cap->max_slots * B;
  L.att_o = take(sizeof(float) * L.att_rows * c->q_heads * kAttnSplitMax * c->head_dim);
  L.att_ml = take(sizeof(float) * L.att_rows * c->q_heads * kAttnSplitMax * 2);
  L.dlogits = take(sizeof(float) * cap->max_slots * (B > 1 ? B - 1 : 1) * V);
  const size_t srows = (size_t)cap->max_slots * std::max<size_t>(B, 1);
  L.cid = take(sizeof(int32_t) * srows * kMaxTopK);
  L.cp = take(sizeof(float) * srows * kMaxTopK);
  L.cn = take(sizeof(int32_t) * srows);
  L.skey = take(sizeof(uint32_t) * srows * kFilterScratch);
  L.sidx = take(sizeof(int32_t) * srows * kFilterScratch);
  // DFlash2 variants: the dynamic convolution's tap logits and output rows; the selector's candidates,
  // gathered embedding rows, their rank-r projections and the transitions
  if (d->conv_kernel > 0) {
    L.cu = take(sizeof(float) * R * (d->conv_kernel * H / d->conv_group));
    L.xc = take(es * R * H);
  }
  if (d->selector_top_k > 0) {
    const size_t nd = B > 1 ? B - 1 : 1, K = d->selector_top_k, per = 1 + nd * K;
    L.sel_id = take(sizeof(int32_t) * cap->max_slots * nd * kMaxTopK);
    L.sel_s = take(sizeof(float) * cap->max_slots * nd * kMaxTopK);
    L.sel_x = take(es * cap->max_slots * per * H);
    L.sel_y = take(sizeof(float) * cap->max_slots * per * 2 * d->selector_rank);
    L.sel_t = take(sizeof(float) * cap->max_slots * nd * K * K);
  }
  L.total = off;
  return L;
}

const char *check_cfg(const dflash_model_cfg *c, const dflash_drafter_cfg *d, const dflash_capacity *cap) {
  if (!c || !d || !cap) return "null configuration";
  if (c->dtype != DFLASH_BF16 && c->dtype != DFLASH_F32) return "dtype must be DFLASH_BF16 or DFLASH_F32";
  if (c->layers < 1 || c->hidden < 32 || c->q_heads < 1 || c->kv_heads < 1 || c->ffn < 16 || c->vocab < 2)
    return "model dimensions must be positive";
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return "head_dim must be 32, 64 or 128";
  if (c->q_heads % c->kv_heads) return "q_heads must be a multiple of kv_heads";
  if (c->q_heads / c->kv_heads > 64) return "at most 64 query heads per KV head";
  const int qd = c->q_heads * c->head_dim, kd = c->kv_heads * c->head_dim;
  if (c->hidden % 128 || qd % 128 || kd % 128 || c->vocab % 128)
    return "hidden, q_heads*head_dim, kv_heads*head_dim and vocab must be multiples of 128";
  if (c->ffn % 64) return "ffn must be a multiple of 64";
  if (!(c->rope_theta > 0.f) || !(c->rms_eps > 0.f)) return "rope_theta and rms_eps must be positive";
  if (d->layers < 1 || d->n_taps < 1 || d->n_taps > DFLASH_MAX_TAPS) return "drafter layers / taps out of range";
  for (int i = 0; i < d->n_taps; ++i)
    if (d->taps[i] < 0 || d->taps[i] >= c->layers) return "tap layer out of range";
  if (d->block_size < 1 || d->block_size > DFLASH_MAX_BLOCK) return "block_size out of range";
  if (d->mask_id < 0 || d->mask_id >= c->vocab) return "mask_id out of range";
  if (d->window < 0) return "window must be >= 0";
  if (d->conv_kernel < 0 || d->conv_kernel > kConvMaxTaps) return "conv_kernel must be in [0, 4]";
  if (d->conv_kernel > 0) {
    if (d->conv_group < 1 || c->hidden % d->conv_group) return "conv_group must divide hidden";
    const int n = d->conv_kernel * c->hidden / d->conv_group;
    if (n % (c->dtype == DFLASH_BF16 ? 32 : 16)) return "conv_kernel * hidden / conv_group must be a multiple of 32 (bf16) or 16";
  }
  if (d->selector_top_k < 0 || d->selector_top_k > kSelMaxK || d->selector_top_k > c->vocab)
    return "selector_top_k must be in [0, 32] and at most vocab";
  if (d->selector_top_k > 0 && (d->selector_rank < 1 || d->selector_rank % 32 || d->selector_rank > 512 || d->block_size < 2))
    return "selector_rank must be a multiple of 32 in [32, 512] (and block_size >= 2)";
  if (cap->max_slots < 1 || cap->max_slots > DFLASH_MAX_BATCH) return "max_slots out of range";
  if (cap->max_rows < cap->max_slots * d->block_size) return "max_rows must be at least max_slots * block_size";
  if (cap->page_tokens != 16) return "page_tokens must be 16";
  if (cap->num_pages < 1 || cap->max_pages_per_seq < 1) return "page counts must be positive";
  return nullptr;
}

}  // namespace

struct dflash_ctx {
  dflash_model_cfg cfg;
  dflash_drafter_cfg dcfg;
  dflash_capacity cap;
  std::vector<dflash_layer_weights> tl, dl;
  const void *embed, *final_norm, *lm_head, *fc, *hidden_norm, *d_final_norm, *sel_u, *sel_v;
  char *tkv, *dkv, *ws;
  Layout L;
  KVLayout kvl;
  size_t layer_elems;  // elements of one layer's pool
  size_t d_layer_elems;  // elements of one drafter layer's pool (the page ring when dring > 0)
  int dring = 0;         // drafter pages per slot when the drafter's window recycles them, else 0
  // host page tables
  std::vector<std::vector<int32_t>> pages;
  std::vector<int32_t> free_pages;
  std::vector<int> prefilled;
  // the last verify call, for draft / accept consistency
  int last_qlen = 0, last_nlogit = 0, last_batch = 0;
  // drafts of the accept that followed the last verify (-1: no accept since that verify)
  int last_nd = -1;
  std::vector<int32_t> last_slots;
  bool verified = false;
  // Set while a call of a bf16 model over kTcMinRows rows or more runs (x16 mode): its projections take
  // the tiled fp16 kernel of gemm_tc.hip, every RMSNorm is applied at once (no deferred 1/rms), and the
  // residual projections write K-range partial sums that norm_kernel adds to the residual and
  // normalises.  Smaller calls keep the row-chunked kernels.
  bool x16 = false;
  int sel_batch = 0;  // requests of the last selector pass (dflash_selector_state)
  // measurement: the projection launches issued while profiling is on, kept for replay
  bool profiling = false;
  struct Rec {
    GemmArgs a;
    int rows;
    bool x16;
    TcPlan plan;
  };
  std::vector<Rec> recorded;

  template <typename P> P *wsp(size_t off) const { return reinterpret_cast<P *>(ws + off); }
  SlotState *state() const { return wsp<SlotState>(L.state); }
  int32_t *err() const { return wsp<int32_t>(L.err); }
  int32_t *bt() const { return wsp<int32_t>(L.bt); }
  // the drafter's block table: its page ring (slot s, page index i -> page s * dring + i % dring) when
  // the window recycles pages, else the target's table (page ids shared by both pools)
  int32_t *dbt() const { return dring ? wsp<int32_t>(L.dbt) : bt(); }
  Rows rows(int s) const {
    Rows r;
    r.pos = wsp<int32_t>(L.rows[s][0]);
    r.slot = wsp<int32_t>(L.rows[s][1]);
    r.valid = wsp<int32_t>(L.rows[s][2]);
    r.tok = wsp<int32_t>(L.rows[s][3]);
    return r;
  }
  int dt() const { return cfg.dtype == DFLASH_BF16 ? 0 : 1; }
  int rope_rows() const { return cap.max_pages_per_seq * cap.page_tokens; }
  int es() const { return esize(&cfg); }
  void *tlayer(int l) const { return tkv + (size_t)l * layer_elems * es(); }
  void *dlayer(int l) const { return dkv + (size_t)l * d_layer_elems * es(); }
  int max_ctx(const int32_t *slots, int batch) const {
    int m = 0;
    for (int b = 0; b < batch; ++b) m = std::max<int>(m, (int)pages[slots[b]].size() * cap.page_tokens);
    return m;
  }
};

namespace {

GemmArgs gemm_base(const void *x, int ldx, int M, int N, int K, int epi) {
  GemmArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.ldx = ldx;
  a.M = M;
  a.N = N;
  a.K = K;
  a.epi = epi;
  a.ksplit = 1;
  return a;
}

// Run a GEMM over R rows in chunks of kGemmMaxRows on the row-chunked kernels.  `a.x` points at row 0;
// input rows advance by ldx.  e0 / e1 (may be null) time the first chunk's start and the last chunk's end.
dflash_status run_gemm(int es, int dt, GemmArgs a, int R, hipStream_t s, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr) {
  const int cr = kGemmMaxRows;
  const char *x0 = (const char *)a.x;
  for (int r0 = 0; r0 < R; r0 += cr) {
    GemmArgs b = a;
    b.M = std::min(cr, R - r0);
    if (!a.x_take) b.x = x0 + (size_t)r0 * a.ldx * es;  // a row selection addresses X by global row
    b.row_off = r0;
    HIP_OK(launch_gemm(b, dt, s, r0 == 0 ? e0 : nullptr, r0 + cr >= R ? e1 : nullptr));
  }
  return DFLASH_OK;
}

// x16 mode: all R rows in one launch of the tiled fp16 kernel (range_cap: elements of a.out_f32 that
// K ranges may fill; 0 keeps one range).
dflash_status plan_tc(GemmArgs &a, int R, int64_t range_cap, TcPlan *p) {
  a.M = R;
  a.row_off = 0;
  if (!gemm_tc_plan(a, range_cap, p))
    return fail(DFLASH_E_INVAL, "projection %d x %d x %d (epilogue %d) does not suit the fp16 tiled kernel", R, a.N, a.K,
                a.epi);
  return DFLASH_OK;
}

dflash_status launch_tc(dflash_ctx *c, GemmArgs a, int R, const TcPlan &p, hipStream_t s) {
  if (a.epi == EPI_PARTIAL) a.part_stride = (int64_t)R * a.N;
  if (c->profiling) c->recorded.push_back({a, R, true, p});
  HIP_OK(launch_gemm_tc(a, p, s));
  return DFLASH_OK;
}

dflash_status run_gemm_tc(dflash_ctx *c, GemmArgs a, int R, hipStream_t s) {
  TcPlan p;
  dflash_status st = plan_tc(a, R, 0, &p);
  return st != DFLASH_OK ? st : launch_tc(c, a, R, p, s);
}

dflash_status run_gemm(dflash_ctx *c, GemmArgs a, int R, hipStream_t s) {
  if (c->x16) return run_gemm_tc(c, a, R, s);
  a.sk_part = c->wsp<float>(c->L.skp);
  a.sk_cnt = c->wsp<int32_t>(c->L.skc);
  a.sk_max_wg = kSkMaxWg;
  a.sk_max_tiles = c->L.sk_tiles;
  if (c->profiling) c->recorded.push_back({a, R, false, TcPlan{}});
  return run_gemm(c->es(), c->dt(), a, R, s);
}

// A projection whose K ranges leave fp32 partial slices [range][R][N] for the consumer (qkv_post_kernel,
// norm_kernel) to add in order: *src, *stride and *n_part describe them.
dflash_status run_partial(dflash_ctx *c, GemmArgs a, int R, hipStream_t s, int *n_part, const float **src,
                          int64_t *stride) {
  a.epi = EPI_PARTIAL;
  if (c->x16) {  // several K ranges go to the range buffer, one range to L.part
    TcPlan p;
    dflash_status st = plan_tc(a, R, (int64_t)c->L.tcr_elems, &p);
    if (st != DFLASH_OK) return st;
    a.out_f32 = p.ranges > 1 ? c->wsp<float>(c->L.tcr) : c->wsp<float>(c->L.part);
    a.ld_out = a.N;
    if ((st = launch_tc(c, a, R, p, s)) != DFLASH_OK) return st;
    *n_part = p.ranges;
    *src = a.out_f32;
    *stride = (int64_t)R * a.N;
    return DFLASH_OK;
  }
  a.out_f32 = c->wsp<float>(c->L.part);
  a.ld_out = a.N;
  a.ksplit = R <= kGemmMaxRows ? std::min(kMaxKSplit, gemm_ksplit(R, a.N, a.K, c->dt(), c->L.part_elems)) : 1;
  a.part_stride = (int64_t)R * a.N;
  *n_part = a.ksplit;
  *src = a.out_f32;
  *stride = a.part_stride;
  return run_gemm(c, a, R, s);
}

// The RMSNorm that follows a residual update, deferred to the next projection: xn receives
// act(x * gain) for the selected rows (compacted), L.ss the sums of squares, and the projection that
// reads xn applies 1/rms to its outputs.
struct NextNorm {
  const void *gain;
  int take, stride, offset;
};
NextNorm all_rows(const void *gain, int R) { return NextNorm{gain, R, R, 0}; }

// Deferred RMSNorm of the fp32 rows x (after the embedding): one partial per row.
dflash_status prep_norm(dflash_ctx *c, int R, const void *gain, hipStream_t s) {
  NormArgs n;
  memset(&n, 0, sizeof n);
  n.x = c->wsp<float>(c->L.x);
  n.ld_x = c->cfg.hidden;
  n.gain = (const float *)gain;
  n.eps = c->cfg.rms_eps;
  n.hidden = c->cfg.hidden;
  n.out = c->wsp<void>(c->L.xn);
  n.ld_out = c->cfg.hidden;
  n.n_rows = R;
  n.take = R;
  n.stride = R;
  n.offset = 0;
  n.ss_out = c->x16 ? nullptr : c->wsp<float>(c->L.ss);  // x16 mode: normalised at once
  n.ss_ld = c->L.ss_ld;
  HIP_OK(launch_norm(n, c->dt(), s));
  return DFLASH_OK;
}

// A projection whose X rows are xn awaiting their 1/rms factor (ss_n partial sums per row in L.ss).
void with_norm(dflash_ctx *c, GemmArgs &a, int ss_n) {
  if (c->x16) return;  // its inputs are normalised already
  a.ss_in = c->wsp<float>(c->L.ss);
  a.ss_n = ss_n;
  a.ss_ld = c->L.ss_ld;
  a.norm_dim = c->cfg.hidden;
  a.eps = c->cfg.rms_eps;
}

// A hidden-width projection whose output is added to the residual (resid may be null: the output is
// the new row) and then RMS-normalised with the deferred scheme; returns ss_n for the consumer.
dflash_status run_resid_norm(dflash_ctx *c, GemmArgs a, int R, float *resid, void *feat, int ld_feat,
                             const NextNorm &nx, hipStream_t s, int *ss_n) {
  if (c->x16) {  // K-range partial sums, then one pass per row: residual add, feature tap, RMSNorm
    int np = 1;
    const float *part = nullptr;
    int64_t pstride = 0;
    dflash_status st = run_partial(c, a, R, s, &np, &part, &pstride);
    if (st != DFLASH_OK) return st;
    NormArgs n;
    memset(&n, 0, sizeof n);
    n.x = resid;
    n.ld_x = c->cfg.hidden;
    n.part = part;
    n.n_part = np;
    n.ld_part = a.N;
    n.part_stride = pstride;
    n.feat = feat;
    n.ld_feat = ld_feat;
    n.gain = (const float *)nx.gain;
    n.eps = c->cfg.rms_eps;
    n.hidden = c->cfg.hidden;
    n.out = c->wsp<void>(c->L.xn);
    n.ld_out = c->cfg.hidden;
    n.n_rows = R;
    n.take = nx.take;
    n.stride = nx.stride;
    n.offset = nx.offset;
    HIP_OK(launch_norm(n, c->dt(), s));
    *ss_n = 1;
    return DFLASH_OK;
  }
  a.epi = EPI_RESID_NORM;
  a.resid = resid;
  a.ld_resid = c->cfg.hidden;
  a.feat = feat;
  a.ld_feat = ld_feat;
  a.gain = (const float *)nx.gain;
  a.xg = c->wsp<void>(c->L.xn);
  a.ld_xg = c->cfg.hidden;
  a.ss_out = c->wsp<float>(c->L.ss);
  a.ss_out_ld = c->L.ss_ld;
  a.sel_take = nx.take;
  a.sel_stride = nx.stride;
  a.sel_offset = nx.offset;
  *ss_n = a.N / 32;
  return run_gemm(c, a, R, s);
}

QkvPostArgs post_base(dflash_ctx *c, const Rows &rows, int n_rows, bool drafter) {
  QkvPostArgs p;
  memset(&p, 0, sizeof p);
  p.src = c->wsp<float>(c->L.part);
  p.n_part = 1;
  p.n_rows = n_rows;
  p.rows = rows;
  p.block_table = drafter ? c->dbt() : c->bt();
  p.bt_stride = c->cap.max_pages_per_seq;
  p.kv = c->kvl;
  p.rope = c->wsp<float2>(c->L.rope);
  p.rope_rows = c->rope_rows();
  p.eps = c->cfg.rms_eps;
  p.err = c->err();
  return p;
}

// raw_qkv (optional, calls with one query tile per sequence): the layer's raw fp32 q/k/v rows, which the
// attention kernel normalises, rotates and writes to the pool itself (no separate post kernel).
dflash_status run_attention(dflash_ctx *c, const Rows &rows, int n_seq, int q_len, int mode, void *kv, int ctx_bound,
                            const int32_t *slots, const dflash_layer_weights *raw_w, hipStream_t s) {
  const dflash_model_cfg &m = c->cfg;
  AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = c->wsp<void>(c->L.qbuf);
  a.ldq = m.q_heads * m.head_dim;
  a.kv = kv;
  a.kvl = c->kvl;
  a.block_table = mode == 1 ? c->dbt() : c->bt();  // mode 1: the drafter's layers
  a.bt_stride = c->cap.max_pages_per_seq;
  a.rows = rows;
  a.n_seq = n_seq;
  a.q_len = q_len;
  a.q_heads = m.q_heads;
  a.mode = mode;
  a.window = c->dcfg.window;
  const int G = m.q_heads / m.kv_heads;
  // One 16-wide MFMA tile of query vectors per work-group (three work-groups per KV head and split at
  // G = 5, block 8): on MI355X this beats packing the whole block into one work-group by ~40% at
  // decode (more, lighter work-groups; each page's K/V is re-read from L2 by the tiles).
  // Larger calls (prefill) pack up to 64 query vectors per work-group.
  const char *qz = getenv("DFLASH_ATTN_QTILE");
  const int qt_env = qz ? atoi(qz) : 0;
  const bool decode = (size_t)n_seq * q_len <= c->L.att_rows;
  const int pt = c->cap.page_tokens;
  int key_span = ctx_bound + pt;  // keys of the widest work-group, rounded out to pages
  if (mode == 1 && c->dcfg.window > 0) key_span = std::min(key_span, c->dcfg.window + q_len + 2 * pt);
  const int pages = (key_span + pt - 1) / pt;
  // Batched calls (q/k/v post-processed separately) over long key ranges: one work-group per
  // (sequence, KV head) holds the whole block, so each K/V page is read once instead of once per
  // 16-wide query tile (at 6K keys and 32 sequences those re-reads bound the kernel: 47.0 -> 44.0 ms per
  // 27B step); at 1K keys the lighter one-tile work-groups stay faster.
  int qt = qt_env > 0 ? qt_env : 16 / G;
  if (decode && qt_env <= 0 && !raw_w && pages >= kAttnWholeBlockPages) qt = q_len;
  a.q_tile = std::max(1, std::min(q_len, !decode ? 64 / G : qt));
  const int ntile = (q_len + a.q_tile - 1) / a.q_tile;
  // Decode-sized calls split the keys into ranges of about nine pages (the fastest on MI355X at 1-2K
  // keys with one query tile per work-group; merged by attn_merge_kernel); larger calls keep one range.
  // Batched calls already have (sequences x KV heads x query tiles) work-groups: they split the keys
  // only as far as about kAttnWgTarget work-groups in all (more splits add merge work and rounds of
  // work-groups, not parallelism).
  int splits = 1;
  if ((size_t)n_seq * q_len <= c->L.att_rows) {
    const int wg_target = getenv("DFLASH_ATTN_WG") ? std::max(1, atoi(getenv("DFLASH_ATTN_WG"))) : kAttnWgTarget;
    const int gx = n_seq * m.kv_heads * ntile;
    splits = std::min({kAttnSplitMax, std::max(1, (pages + 8) / 9), std::max(1, (wg_target + gx - 1) / gx)});
  }
  int pps = (pages + splits - 1) / splits;
  const int env_pps = getenv("DFLASH_ATTN_PPS") ? atoi(getenv("DFLASH_ATTN_PPS")) : 0;
  if (env_pps > 0 && (pages + env_pps - 1) / env_pps <= kAttnSplitMax && (size_t)n_seq * q_len <= c->L.att_rows)
    pps = env_pps;
  // the last-arriver merge keeps m and l of every (query vector, split) in the head_dim-sized LDS tile
  const char *mz = getenv("DFLASH_ATTN_MERGE");
  const bool arrive = raw_w && mz && atoi(mz) == 1;
  if (arrive && (pages + pps - 1) / pps > m.head_dim / 2) pps = (pages + m.head_dim / 2 - 1) / (m.head_dim / 2);
  a.n_splits = (pages + pps - 1) / pps;
  a.split_tokens = pps * pt;
  a.part_o = c->wsp<float>(c->L.att_o);
  a.part_ml = c->wsp<float>(c->L.att_ml);
  a.out = c->wsp<void>(c->L.attn);
  a.ldo = m.q_heads * m.head_dim;
  a.err = c->err();
  for (int i = 0; i < n_seq; ++i) a.seq_slot[i] = slots[i];
  // klo = max(0, first_pos - window + 1) is 0 for every sequence when the allocation fits the window
  a.abs_range = mode == 0 || c->dcfg.window <= 0 || ctx_bound <= c->dcfg.window;
  if (raw_w) {
    a.raw = c->wsp<float>(c->L.part);
    a.ld_raw = (m.q_heads + 2 * m.kv_heads) * m.head_dim;
    a.q_gain = (const float *)raw_w->q_norm;
    a.k_gain = (const float *)raw_w->k_norm;
    a.eps = m.rms_eps;
    a.rope = c->wsp<float2>(c->L.rope);
    a.rope_rows = c->rope_rows();
    a.counters = arrive ? c->wsp<int32_t>(c->L.cnt) : nullptr;
  }
  // Prefill-sized causal calls: the flash-style kernel (one work-group per 128 query rows and query
  // head, keys staged once per work-group through LDS); DFLASH_ATTN_PREFILL=0 keeps the general kernel.
  static const bool flash_prefill = !getenv("DFLASH_ATTN_PREFILL") || atoi(getenv("DFLASH_ATTN_PREFILL")) != 0;
  if (flash_prefill && !decode && !raw_w && attn_prefill_fits(a, c->dt(), ctx_bound - 1)) {
    HIP_OK(launch_attn_prefill(a, s));
    return DFLASH_OK;
  }
  HIP_OK(launch_attention(a, c->dt(), s));
  return DFLASH_OK;
}

// One decoder layer over R rows.  On entry xn holds act(x * attn_norm) and L.ss its ss_n partial sums
// of squares (deferred RMSNorm); the residual x (fp32) is updated in place.  `next` is the RMSNorm that
// follows the layer (the next layer's attention norm, or the final norm over the rows that need
// logits); feat: optional tap of the layer's output.  Returns the ss_n of the deferred next norm.
dflash_status run_layer(dflash_ctx *c, const dflash_layer_weights &w, void *kv_layer, const Rows &rows,
                        const int32_t *slots, int n_seq, int q_len, int attn_mode, int ctx_bound, void *feat,
                        int ld_feat, const NextNorm &next, int *ss_n, hipStream_t s) {
  const dflash_model_cfg &m = c->cfg;
  const int R = n_seq * q_len, H = m.hidden, QD = m.q_heads * m.head_dim, KD = m.kv_heads * m.head_dim, F = m.ffn;
  float *x = c->wsp<float>(c->L.x);
  void *xn = c->wsp<void>(c->L.xn);
  dflash_status st;
  bool fused = false;
  const void *xq = xn;  // the q/k/v projections' input
  bool normed = false;  // xq is normalised already (no deferred 1/rms)
  if (attn_mode == 1 && c->dcfg.conv_kernel > 0) {
    // DFlash2 dynamic convolution along the block: tap logits u = W_conv x (with the deferred 1/rms),
    // then y_i = sum_t softmax_t(u_i)[group] x_{i-t} into L.xc
    const dflash_drafter_cfg &dc = c->dcfg;
    const int NU = dc.conv_kernel * H / dc.conv_group;
    GemmArgs u = gemm_base(xn, H, R, NU, H, EPI_STORE_F32);
    u.nseg = 1;
    u.seg[0] = GemmSeg{w.w_conv, NU};
    with_norm(c, u, *ss_n);
    u.out_f32 = c->wsp<float>(c->L.cu);
    u.ld_out = NU;
    if ((st = run_gemm(c, u, R, s)) != DFLASH_OK) return st;
    ConvArgs cv;
    memset(&cv, 0, sizeof cv);
    cv.x = xn;
    cv.ldx = H;
    cv.ss = c->x16 ? nullptr : c->wsp<float>(c->L.ss);
    cv.ss_n = *ss_n;
    cv.ss_ld = c->L.ss_ld;
    cv.eps = m.rms_eps;
    cv.u = u.out_f32;
    cv.ld_u = NU;
    cv.out = c->wsp<void>(c->L.xc);
    cv.ld_out = H;
    cv.rows = R;
    cv.hidden = H;
    cv.block = q_len;
    cv.taps = dc.conv_kernel;
    cv.group = dc.conv_group;
    HIP_OK(launch_dyn_conv(cv, c->dt(), s));
    xq = cv.out;
    normed = true;
  }
  {
    GemmArgs a = gemm_base(xq, H, R, QD + 2 * KD, H, EPI_PARTIAL);
    a.nseg = 3;
    a.seg[0] = GemmSeg{w.wq, QD};
    a.seg[1] = GemmSeg{w.wk, KD};
    a.seg[2] = GemmSeg{w.wv, KD};
    if (!normed) with_norm(c, a, *ss_n);
    int np = 1;
    const float *part = nullptr;
    int64_t part_stride = 0;
    if ((st = run_partial(c, a, R, s, &np, &part, &part_stride)) != DFLASH_OK) return st;
    // Decode-sized calls of up to kAttnFusedMaxSeqs sequences: the attention kernel post-processes
    // q / k / v itself (one query tile per work-group keeps that prologue short; 0.2 ms per 27B step
    // faster on MI355X than a separate post-processing launch at concurrency 1).  Larger batches take
    // the separate kernel: the plain attention kernel holds fewer registers (two work-groups per CU
    // instead of one), which measured 2-3% faster per step at concurrency 8 and 32.
    // DFLASH_ATTN_FUSED=0 / =1 selects the separate / fused kernel for every decode-sized call.
    // The fused kernel needs q_len <= 16 (the block's keys form one LDS page) and a 16-byte aligned
    // q gain.
    const char *fz = getenv("DFLASH_ATTN_FUSED");
    const bool want = fz ? atoi(fz) != 0 : n_seq <= kAttnFusedMaxSeqs;
    fused = want && np == 1 && (size_t)R <= c->L.att_rows && q_len <= 16 && ((uintptr_t)w.q_norm & 15) == 0;
    if (!fused) {
      QkvPostArgs p = post_base(c, rows, R, attn_mode == 1);
      p.src = part;
      p.ld_src = QD + 2 * KD;
      p.n_part = np;
      p.part_stride = part_stride;
      p.nseg = 3;
      p.seg[0] = PostSeg{m.q_heads, ROLE_Q, (const float *)w.q_norm, c->wsp<void>(c->L.qbuf), QD};
      p.seg[1] = PostSeg{m.kv_heads, ROLE_K, (const float *)w.k_norm, kv_layer, 0};
      p.seg[2] = PostSeg{m.kv_heads, ROLE_V, nullptr, kv_layer, 0};
      p.total_heads = m.q_heads + 2 * m.kv_heads;
      HIP_OK(launch_qkv_post(p, c->dt(), s));
    }
  }
  if ((st = run_attention(c, rows, n_seq, q_len, attn_mode, kv_layer, ctx_bound, slots, fused ? &w : nullptr, s)) !=
      DFLASH_OK)
    return st;
  {
    GemmArgs a = gemm_base(c->wsp<void>(c->L.attn), QD, R, H, QD, EPI_RESID_NORM);
    a.nseg = 1;
    a.seg[0] = GemmSeg{w.wo, H};
    if ((st = run_resid_norm(c, a, R, x, nullptr, 0, all_rows(w.ffn_norm, R), s, ss_n)) != DFLASH_OK)
      return st;
  }
  {
    GemmArgs a = gemm_base(xn, H, R, F, H, EPI_SWIGLU);
    a.nseg = 2;
    a.seg[0] = GemmSeg{w.w_gate, F};
    a.seg[1] = GemmSeg{w.w_up, F};
    a.out_act = c->wsp<void>(c->L.ffn);
    a.ld_out = F;
    with_norm(c, a, *ss_n);
    if ((st = run_gemm(c, a, R, s)) != DFLASH_OK) return st;
  }
  {
    GemmArgs a = gemm_base(c->wsp<void>(c->L.ffn), F, R, H, F, EPI_RESID_NORM);
    a.nseg = 1;
    a.seg[0] = GemmSeg{w.w_down, H};
    if ((st = run_resid_norm(c, a, R, x, feat, ld_feat, next, s, ss_n)) != DFLASH_OK) return st;
  }
  return DFLASH_OK;
}

dflash_status check_slots(dflash_ctx *c, int batch, const int32_t *slots, bool need_prefilled) {
  if (batch < 1 || batch > c->cap.max_slots) return fail(DFLASH_E_INVAL, "batch %d out of range", batch);
  if (!slots) return fail(DFLASH_E_INVAL, "slots is null");
  for (int b = 0; b < batch; ++b) {
    const int s = slots[b];
    if (s < 0 || s >= c->cap.max_slots) return fail(DFLASH_E_INVAL, "slot %d out of range", s);
    for (int q = 0; q < b; ++q)
      if (slots[q] == s) return fail(DFLASH_E_INVAL, "slot %d repeated", s);
    if (c->pages[s].empty()) return fail(DFLASH_E_STATE, "slot %d has no KV pages (call dflash_kv_alloc)", s);
    if (need_prefilled && !c->prefilled[s]) return fail(DFLASH_E_STATE, "slot %d has not been prefilled", s);
  }
  return DFLASH_OK;
}

bool same_slots(dflash_ctx *c, int batch, const int32_t *slots) {
  if (batch != c->last_batch) return false;
  for (int b = 0; b < batch; ++b)
    if (slots[b] != c->last_slots[b]) return false;
  return true;
}

dflash_status check_sampling(const dflash_sampling *sampling, int batch) {
  for (int b = 0; b < batch; ++b) {
    const dflash_sampling &sp = sampling[b];
    if (!(sp.temperature >= 0.f)) return fail(DFLASH_E_INVAL, "temperature must be >= 0");
    if (sp.temperature > 0.f) {
      if (sp.top_k < 1 || sp.top_k > DFLASH_MAX_TOPK) return fail(DFLASH_E_INVAL, "top_k must be in [1, %d]", DFLASH_MAX_TOPK);
      if (!(sp.top_p > 0.f) || sp.top_p > 1.f) return fail(DFLASH_E_INVAL, "top_p must be in (0, 1]");
    }
  }
  return DFLASH_OK;
}

// The candidate filter over `rows` logit rows, rows_per_seq of each request with its sampling.
void filter_setup(dflash_ctx *c, FilterArgs &f, const float *logits, int rows, int rows_per_seq,
                  const dflash_sampling *sampling, int batch, int32_t *cid, float *cp, int32_t *cn) {
  memset(&f, 0, sizeof f);
  f.logits = logits;
  f.rows = rows;
  f.vocab = c->cfg.vocab;
  f.rows_per_seq = rows_per_seq;
  for (int b = 0; b < batch; ++b) {
    f.temperature[b] = sampling[b].temperature;
    f.top_k[b] = sampling[b].top_k;
    f.top_p[b] = sampling[b].top_p;
  }
  f.cand_id = cid;
  f.cand_p = cp;
  f.cand_n = cn;
  f.stage_key = c->wsp<uint32_t>(c->L.skey);
  f.stage_idx = c->wsp<int32_t>(c->L.sidx);
  int kmax = 1;
  for (int b = 0; b < batch; ++b)
    if (sampling[b].temperature > 0.f) kmax = std::max(kmax, std::min(sampling[b].top_k, c->cfg.vocab));
  filter_plan(f, kmax);
}

}  // namespace

namespace df {

dflash_status set_error(dflash_status st, const char *msg) { return fail(st, "%s", msg); }

// The projection on the stream-K kernel with the scratch block at d_scratch (sk_scratch_bytes(N)
// bytes: partial tiles, then the tile counters, which are zeroed here before the launch).
dflash_status op_linear_sk(hipStream_t s, int32_t dtype, int32_t M, int32_t N, int32_t K, const void *d_x,
                           const void *d_w, float *d_y, void *d_scratch) {
  if (dtype != DFLASH_BF16 && dtype != DFLASH_F32) return fail(DFLASH_E_INVAL, "bad dtype");
  const int ksup = dtype == DFLASH_BF16 ? 128 : 64;  // K elements per 256-byte super-step
  if (M < 1 || M > 16 || N < 32 || N % 32 || K < ksup || K % ksup)
    return fail(DFLASH_E_INVAL, "stream-K shape: need 1 <= M <= 16, N a multiple of 32, K a multiple of %d", ksup);
  if (!d_x || !d_w || !d_y || !d_scratch) return fail(DFLASH_E_INVAL, "null pointer");
  if ((uintptr_t)d_scratch & 255) return fail(DFLASH_E_INVAL, "scratch must be 256-byte aligned");
  GemmArgs a = gemm_base(d_x, K, M, N, K, EPI_STORE_F32);
  a.nseg = 1;
  a.seg[0] = GemmSeg{d_w, N};
  a.out_f32 = d_y;
  a.ld_out = N;
  a.sk_part = (float *)d_scratch;
  a.sk_cnt = (int32_t *)((char *)d_scratch + kSkPartBytes);
  a.sk_max_wg = kSkMaxWg;
  a.sk_max_tiles = N / 16;
  a.sk_force = 1;
  HIP_OK(launch_zero_i32(a.sk_cnt, N / 16, s));
  HIP_OK(launch_gemm(a, dtype == DFLASH_BF16 ? 0 : 1, s));
  return DFLASH_OK;
}

}  // namespace df

extern "C" {

const char *dflash_last_error(void) { return g_err.c_str(); }

size_t dflash_kv_pool_bytes(const dflash_model_cfg *cfg, int32_t layers, const dflash_capacity *cap) {
  if (!cfg || !cap || layers < 1 || cap->num_pages < 1 || cap->page_tokens < 1) return 0;
  return (size_t)layers * cap->num_pages * 2 * cfg->kv_heads * cap->page_tokens * cfg->head_dim * esize(cfg);
}

size_t dflash_drafter_pool_bytes(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg,
                                 const dflash_capacity *cap) {
  if (!cfg || !dcfg || !cap || dcfg->layers < 1 || cap->max_slots < 1) return 0;
  const int r = drafter_ring_pages(dcfg, cap);
  if (!r) return dflash_kv_pool_bytes(cfg, dcfg->layers, cap);
  return (size_t)dcfg->layers * cap->max_slots * r * 2 * cfg->kv_heads * cap->page_tokens * cfg->head_dim *
         esize(cfg);
}

size_t dflash_workspace_bytes(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg, const dflash_capacity *cap) {
  if (check_cfg(cfg, dcfg, cap)) return 0;
  return make_layout(cfg, dcfg, cap).total;
}

dflash_status dflash_create(const dflash_model_cfg *cfg, const dflash_drafter_cfg *dcfg, const dflash_target_weights *tw,
                            const dflash_drafter_weights *dw, const dflash_capacity *cap, void *d_target_kv,
                            void *d_drafter_kv, void *d_workspace, hipStream_t stream, dflash_ctx **out) {
  if (!out) return fail(DFLASH_E_INVAL, "out is null");
  *out = nullptr;
  if (const char *why = check_cfg(cfg, dcfg, cap)) return fail(DFLASH_E_INVAL, "%s", why);
  if (!tw || !dw || !tw->layers || !dw->layers || !tw->embed || !tw->final_norm || !tw->lm_head || !dw->fc ||
      !dw->hidden_norm || !dw->final_norm)
    return fail(DFLASH_E_INVAL, "missing weight pointer");
  auto layer_ok = [](const dflash_layer_weights &w) {
    return w.attn_norm && w.wq && w.wk && w.wv && w.q_norm && w.k_norm && w.wo && w.ffn_norm && w.w_gate && w.w_up &&
           w.w_down;
  };
  for (int l = 0; l < cfg->layers; ++l)
    if (!layer_ok(tw->layers[l])) return fail(DFLASH_E_INVAL, "missing weight pointer in target layer %d", l);
  for (int l = 0; l < dcfg->layers; ++l) {
    if (!layer_ok(dw->layers[l])) return fail(DFLASH_E_INVAL, "missing weight pointer in drafter layer %d", l);
    if (dcfg->conv_kernel > 0 && !dw->layers[l].w_conv)
      return fail(DFLASH_E_INVAL, "missing w_conv in drafter layer %d (conv_kernel > 0)", l);
  }
  if (dcfg->selector_top_k > 0 && (!dw->sel_u || !dw->sel_v))
    return fail(DFLASH_E_INVAL, "missing selector factors sel_u / sel_v (selector_top_k > 0)");
  if (!d_target_kv || !d_drafter_kv || !d_workspace) return fail(DFLASH_E_INVAL, "null pool or workspace");
  if (((uintptr_t)d_target_kv | (uintptr_t)d_drafter_kv | (uintptr_t)d_workspace) & 255)
    return fail(DFLASH_E_INVAL, "pools and workspace must be 256-byte aligned");

  dflash_ctx *c = new dflash_ctx();
  c->cfg = *cfg;
  c->dcfg = *dcfg;
  c->cap = *cap;
  c->tl.assign(tw->layers, tw->layers + cfg->layers);
  c->dl.assign(dw->layers, dw->layers + dcfg->layers);
  c->embed = tw->embed;
  c->final_norm = tw->final_norm;
  c->lm_head = tw->lm_head;
  c->fc = dw->fc;
  c->hidden_norm = dw->hidden_norm;
  c->d_final_norm = dw->final_norm;
  c->sel_u = dw->sel_u;
  c->sel_v = dw->sel_v;
  c->tkv = (char *)d_target_kv;
  c->dkv = (char *)d_drafter_kv;
  c->ws = (char *)d_workspace;
  c->L = make_layout(cfg, dcfg, cap);
  c->kvl = KVLayout{cap->page_tokens, cfg->kv_heads, cfg->head_dim};
  c->layer_elems = (size_t)cap->num_pages * c->kvl.page_elems();
  c->dring = drafter_ring_pages(dcfg, cap);
  c->d_layer_elems = c->dring ? (size_t)cap->max_slots * c->dring * c->kvl.page_elems() : c->layer_elems;
  c->pages.assign(cap->max_slots, {});
  c->prefilled.assign(cap->max_slots, 0);
  for (int p = cap->num_pages - 1; p >= 0; --p) c->free_pages.push_back(p);
  // Pools start zeroed: unwritten key slots of a page are multiplied by zero probabilities in the
  // attention product, which is only exact for finite contents.  Only finite values are stored later.
  hipError_t e = hipMemsetAsync(c->tkv, 0, dflash_kv_pool_bytes(cfg, cfg->layers, cap), stream);
  if (e == hipSuccess) e = hipMemsetAsync(c->dkv, 0, dflash_drafter_pool_bytes(cfg, dcfg, cap), stream);
  if (e == hipSuccess) e = hipMemsetAsync(c->ws + c->L.state, 0, c->L.rows[0][0] - c->L.state, stream);
  if (e == hipSuccess)
    e = hipMemsetAsync(c->ws + c->L.bt, 0xff, sizeof(int32_t) * cap->max_slots * cap->max_pages_per_seq, stream);
  if (e == hipSuccess)
    e = hipMemsetAsync(c->ws + c->L.dbt, 0xff, sizeof(int32_t) * cap->max_slots * cap->max_pages_per_seq, stream);
  if (e == hipSuccess)
    e = launch_rope_table(c->wsp<float2>(c->L.rope), cfg->rope_theta, cfg->head_dim, c->rope_rows(), stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) {
    delete c;
    return fail(DFLASH_E_DEVICE, "workspace init: %s", hipGetErrorString(e));
  }
  *out = c;
  return DFLASH_OK;
}

dflash_status dflash_destroy(dflash_ctx *ctx) {
  delete ctx;
  return DFLASH_OK;
}

dflash_status dflash_kv_alloc(dflash_ctx *c, int32_t slot, int32_t n_tokens) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  if (slot < 0 || slot >= c->cap.max_slots) return fail(DFLASH_E_INVAL, "slot %d out of range", slot);
  if (n_tokens < 1) return fail(DFLASH_E_INVAL, "n_tokens must be positive");
  const int need = (n_tokens + c->cap.page_tokens - 1) / c->cap.page_tokens;
  if (need > c->cap.max_pages_per_seq)
    return fail(DFLASH_E_INVAL, "%d tokens exceed max_pages_per_seq", n_tokens);
  std::vector<int32_t> &pg = c->pages[slot];
  const int have = (int)pg.size();
  if (need <= have) return DFLASH_OK;
  if ((int)c->free_pages.size() < need - have)
    return fail(DFLASH_E_NOMEM, "KV pool exhausted: slot %d needs %d more pages, %zu free", slot, need - have,
                c->free_pages.size());
  for (int i = have; i < need; ++i) {
    pg.push_back(c->free_pages.back());
    c->free_pages.pop_back();
  }
  hipError_t e = hipMemcpy(c->bt() + (size_t)slot * c->cap.max_pages_per_seq + have, pg.data() + have,
                           sizeof(int32_t) * (need - have), hipMemcpyHostToDevice);
  if (e == hipSuccess && c->dring) {  // the drafter's ring: page index i of the slot -> slot * dring + i % dring
    std::vector<int32_t> ring(need - have);
    for (int i = have; i < need; ++i) ring[i - have] = slot * c->dring + i % c->dring;
    e = hipMemcpy(c->dbt() + (size_t)slot * c->cap.max_pages_per_seq + have, ring.data(), sizeof(int32_t) * ring.size(),
                  hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    // best effort: the new entries of both tables back to "no page", so that no kernel reaches pages
    // returned to the pool through this slot
    const std::vector<int32_t> neg(need - have, -1);
    for (int32_t *t : {c->bt(), c->dbt()})
      (void)hipMemcpy(t + (size_t)slot * c->cap.max_pages_per_seq + have, neg.data(), sizeof(int32_t) * neg.size(),
                      hipMemcpyHostToDevice);
    for (int i = need - 1; i >= have; --i) {
      c->free_pages.push_back(pg[i]);
      pg.pop_back();
    }
    return fail(DFLASH_E_DEVICE, "block-table upload: %s", hipGetErrorString(e));
  }
  return DFLASH_OK;
}

dflash_status dflash_kv_free(dflash_ctx *c, int32_t slot) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  if (slot < 0 || slot >= c->cap.max_slots) return fail(DFLASH_E_INVAL, "slot %d out of range", slot);
  std::vector<int32_t> &pg = c->pages[slot];
  if (!pg.empty()) {
    std::vector<int32_t> neg(pg.size(), -1);
    hipError_t e = hipMemcpy(c->bt() + (size_t)slot * c->cap.max_pages_per_seq, neg.data(), sizeof(int32_t) * neg.size(),
                             hipMemcpyHostToDevice);
    if (e == hipSuccess && c->dring)
      e = hipMemcpy(c->dbt() + (size_t)slot * c->cap.max_pages_per_seq, neg.data(), sizeof(int32_t) * neg.size(),
                    hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(DFLASH_E_DEVICE, "block-table clear: %s", hipGetErrorString(e));
    for (int i = (int)pg.size() - 1; i >= 0; --i) c->free_pages.push_back(pg[i]);
    pg.clear();
  }
  c->prefilled[slot] = 0;
  return DFLASH_OK;
}

dflash_status dflash_verify_block(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots,
                                  const int32_t *d_tokens, int32_t q_len, int32_t new_sequence, int32_t n_logit_rows,
                                  float *d_logits, void *d_feats) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  dflash_status st = check_slots(c, batch, slots, !new_sequence);
  if (st != DFLASH_OK) return st;
  if (q_len < 1 || (size_t)batch * q_len > (size_t)c->cap.max_rows)
    return fail(DFLASH_E_INVAL, "q_len %d with batch %d exceeds max_rows %d", q_len, batch, c->cap.max_rows);
  if (n_logit_rows < 1 || n_logit_rows > q_len) return fail(DFLASH_E_INVAL, "n_logit_rows out of range");
  if ((size_t)batch * n_logit_rows > (size_t)c->cap.max_rows)
    return fail(DFLASH_E_INVAL, "batch * n_logit_rows exceeds max_rows");
  if (!d_tokens || !d_logits) return fail(DFLASH_E_INVAL, "null tokens or logits");
  for (int b = 0; b < batch; ++b)
    if ((int)c->pages[slots[b]].size() * c->cap.page_tokens < q_len)
      return fail(DFLASH_E_NOMEM, "slot %d holds fewer KV pages than q_len", slots[b]);

  const dflash_model_cfg &m = c->cfg;
  const int R = batch * q_len, H = m.hidden;
  struct ModeScope {  // x16 mode for this call's projections; cleared on every exit
    dflash_ctx *c;
    ~ModeScope() { c->x16 = false; }
  } mode_scope{c};
  c->x16 = m.dtype == DFLASH_BF16 && R >= kTcMinRows;
  Rows rows = c->rows(0);
  PrepArgs p;
  memset(&p, 0, sizeof p);
  p.batch = batch;
  for (int b = 0; b < batch; ++b) p.slots[b] = slots[b];
  p.q_len = q_len;
  p.new_sequence = new_sequence;
  p.state = c->state();
  p.rows = rows;
  p.tokens = d_tokens;
  p.mode = 0;
  p.vocab = m.vocab;
  p.err = c->err();
  HIP_OK(launch_prep(p, s));
  HIP_OK(launch_embed(c->embed, c->dt(), rows, R, H, m.vocab, c->wsp<float>(c->L.x), c->err(), s));
  if ((st = prep_norm(c, R, c->tl[0].attn_norm, s)) != DFLASH_OK) return st;
  int ss_n = 1;
  const int ctx_bound = c->max_ctx(slots, batch);
  const int ld_feat = c->dcfg.n_taps * H;
  const int nl = n_logit_rows;
  for (int l = 0; l < m.layers; ++l) {
    void *feat = nullptr;
    for (int t = 0; t < c->dcfg.n_taps; ++t)
      if (c->dcfg.taps[t] == l && d_feats) feat = (char *)d_feats + (size_t)t * H * c->es();
    // after the last layer: the final norm over the last nl rows of every sequence, packed
    const NextNorm next = l + 1 < m.layers ? all_rows(c->tl[l + 1].attn_norm, R)
                                           : NextNorm{c->final_norm, nl, q_len, q_len - nl};
    st = run_layer(c, c->tl[l], c->tlayer(l), rows, slots, batch, q_len, 0, ctx_bound, feat, ld_feat, next,
                   &ss_n, s);
    if (st != DFLASH_OK) return st;
  }
  GemmArgs a = gemm_base(c->wsp<void>(c->L.xn), H, batch * nl, m.vocab, H, EPI_STORE_F32);
  a.nseg = 1;
  a.seg[0] = GemmSeg{c->lm_head, m.vocab};
  with_norm(c, a, ss_n);
  a.out_f32 = d_logits;
  a.ld_out = m.vocab;
  if ((st = run_gemm(c, a, batch * nl, s)) != DFLASH_OK) return st;

  for (int b = 0; b < batch; ++b)
    if (new_sequence) c->prefilled[slots[b]] = 1;
  c->last_qlen = q_len;
  c->last_nlogit = nl;
  c->last_nd = -1;
  c->last_batch = batch;
  c->last_slots.assign(slots, slots + batch);
  c->verified = true;
  return DFLASH_OK;
}

namespace {
dflash_status accept_impl(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots, const float *d_logits,
                          const int32_t *d_block, int32_t n_draft, const dflash_sampling *sampling, const int32_t *d_q_ids,
                          const float *d_q_p, int32_t *d_out, int32_t *d_n_out, int32_t *d_cand_ids, float *d_cand_p) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  dflash_status st = check_slots(c, batch, slots, true);
  if (st != DFLASH_OK) return st;
  if (!c->verified || !same_slots(c, batch, slots))
    return fail(DFLASH_E_STATE, "accept_resample must follow dflash_verify_block on the same slots");
  if (n_draft < 0 || n_draft + 1 != c->last_nlogit)
    return fail(DFLASH_E_INVAL, "n_draft + 1 must equal the n_logit_rows of the last verify (%d)", c->last_nlogit);
  if (n_draft > 0 && !d_block) return fail(DFLASH_E_INVAL, "null block");
  if (!d_logits || !d_out || !d_n_out || !sampling) return fail(DFLASH_E_INVAL, "null argument");
  if ((st = check_sampling(sampling, batch)) != DFLASH_OK) return st;
  const int rows = batch * (n_draft + 1);
  if ((size_t)rows > (size_t)c->cap.max_slots * std::max(1, c->dcfg.block_size))
    return fail(DFLASH_E_INVAL, "batch * (n_draft + 1) exceeds max_slots * block_size");
  FilterArgs f;
  filter_setup(c, f, d_logits, rows, n_draft + 1, sampling, batch, c->wsp<int32_t>(c->L.cid), c->wsp<float>(c->L.cp),
               c->wsp<int32_t>(c->L.cn));
  HIP_OK(launch_filter(f, s));
  DecideArgs d;
  memset(&d, 0, sizeof d);
  d.batch = batch;
  for (int b = 0; b < batch; ++b) {
    d.slots[b] = slots[b];
    d.seed[b] = sampling[b].seed;
  }
  d.n_draft = n_draft;
  d.block = d_block;
  d.cand_id = f.cand_id;
  d.cand_p = f.cand_p;
  d.cand_n = f.cand_n;
  d.state = c->state();
  d.out = d_out;
  d.n_out = d_n_out;
  d.err = c->err();
  d.q_id = n_draft > 0 ? d_q_ids : nullptr;
  d.q_p = n_draft > 0 ? d_q_p : nullptr;
  HIP_OK(launch_decide(d, s));
  if (d_cand_ids || d_cand_p) HIP_OK(launch_copy_cands(f.cand_id, f.cand_p, f.cand_n, rows, d_cand_ids, d_cand_p, s));
  c->verified = false;
  c->last_nd = n_draft;
  return DFLASH_OK;
}
}  // namespace

dflash_status dflash_accept_resample(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots,
                                     const float *d_logits, const int32_t *d_block, int32_t n_draft,
                                     const dflash_sampling *sampling, int32_t *d_out, int32_t *d_n_out,
                                     int32_t *d_cand_ids, float *d_cand_p) {
  return accept_impl(c, s, batch, slots, d_logits, d_block, n_draft, sampling, nullptr, nullptr, d_out, d_n_out,
                     d_cand_ids, d_cand_p);
}

dflash_status dflash_accept_resample_q(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots,
                                       const float *d_logits, const int32_t *d_block, int32_t n_draft,
                                       const dflash_sampling *sampling, const int32_t *d_q_ids, const float *d_q_p,
                                       int32_t *d_out, int32_t *d_n_out, int32_t *d_cand_ids, float *d_cand_p) {
  if (n_draft > 0 && (!d_q_ids || !d_q_p)) return fail(DFLASH_E_INVAL, "null draft candidate buffers");
  return accept_impl(c, s, batch, slots, d_logits, d_block, n_draft, sampling, d_q_ids, d_q_p, d_out, d_n_out,
                     d_cand_ids, d_cand_p);
}

namespace {

// DFlash2 selector over the drafter's logits [batch * (B-1)][V]: top-K candidates per row (the sampler's
// top-k stage in score mode, T = 1), their embedding rows and the anchor's gathered, projected by the
// rank-r factors (one GEMM over both), then a Viterbi pass per request writes the drafts into d_block.
dflash_status run_selector(dflash_ctx *c, hipStream_t s, int batch, const float *logits, int32_t *d_block) {
  const dflash_model_cfg &m = c->cfg;
  const dflash_drafter_cfg &dc = c->dcfg;
  const int B = dc.block_size, nd = B - 1, K = dc.selector_top_k, r = dc.selector_rank, H = m.hidden;
  FilterArgs f;
  memset(&f, 0, sizeof f);
  f.logits = logits;
  f.rows = batch * nd;
  f.vocab = m.vocab;
  f.rows_per_seq = nd;
  for (int b = 0; b < batch; ++b) {
    f.temperature[b] = 1.f;
    f.top_k[b] = K;
    f.top_p[b] = 1.f;
  }
  f.cand_id = c->wsp<int32_t>(c->L.sel_id);
  f.cand_s = c->wsp<float>(c->L.sel_s);
  f.stage_key = c->wsp<uint32_t>(c->L.skey);
  f.stage_idx = c->wsp<int32_t>(c->L.sidx);
  filter_plan(f, K);
  HIP_OK(launch_filter(f, s));
  SelArgs a;
  memset(&a, 0, sizeof a);
  a.batch = batch;
  a.nd = nd;
  a.K = K;
  a.rank = r;
  a.hidden = H;
  a.vocab = m.vocab;
  a.block = d_block;
  a.block_stride = B;
  a.cand_id = f.cand_id;
  a.cand_s = f.cand_s;
  a.cand_ld = kMaxTopK;
  a.embed = c->embed;
  a.x = c->wsp<void>(c->L.sel_x);
  a.proj = c->wsp<float>(c->L.sel_y);
  a.ld_proj = 2 * r;
  a.inv_sqrt_r = (float)(1.0 / std::sqrt((double)r));
  a.trans = c->wsp<float>(c->L.sel_t);
  a.out = d_block;
  HIP_OK(launch_sel_gather(a, c->dt(), s));
  const int rows = batch * (1 + nd * K);
  GemmArgs g = gemm_base(a.x, H, rows, 2 * r, H, EPI_STORE_F32);
  g.nseg = 2;
  g.seg[0] = GemmSeg{c->sel_u, r};
  g.seg[1] = GemmSeg{c->sel_v, r};
  g.out_f32 = c->wsp<float>(c->L.sel_y);
  g.ld_out = 2 * r;
  c->x16 = m.dtype == DFLASH_BF16 && rows >= kTcMinRows;
  dflash_status st = run_gemm(c, g, rows, s);
  if (st != DFLASH_OK) return st;
  HIP_OK(launch_sel_viterbi(a, s));
  c->sel_batch = batch;
  return DFLASH_OK;
}

// dflash_draft_block (sampling null: argmax drafts) and dflash_draft_block_sampled.
dflash_status draft_block_impl(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots, const void *d_feats,
                               int32_t *d_block, float *d_logits, const dflash_sampling *sampling, int32_t *d_q_ids,
                               float *d_q_p) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  dflash_status st = check_slots(c, batch, slots, true);
  if (st != DFLASH_OK) return st;
  if (!d_feats || !d_block) return fail(DFLASH_E_INVAL, "null features or block");
  if (sampling) {
    if (c->dcfg.selector_top_k > 0) return fail(DFLASH_E_INVAL, "stochastic drafts do not combine with the selector");
    if (!d_q_ids || !d_q_p) return fail(DFLASH_E_INVAL, "null draft candidate buffers");
    if ((st = check_sampling(sampling, batch)) != DFLASH_OK) return st;
  }
  if (c->last_qlen < 1 || !same_slots(c, batch, slots))
    return fail(DFLASH_E_STATE, "draft_block must use the slots of the last verified block");
  const dflash_model_cfg &m = c->cfg;
  const dflash_drafter_cfg &dc = c->dcfg;
  const int B = dc.block_size, H = m.hidden, KD = m.kv_heads * m.head_dim;
  if (B < 2) return fail(DFLASH_E_INVAL, "block_size 1 has no drafts");
  for (int b = 0; b < batch; ++b)
    if ((int)c->pages[slots[b]].size() * c->cap.page_tokens < B)
      return fail(DFLASH_E_NOMEM, "slot %d holds fewer KV pages than the block", slots[b]);

  // 1. KV injection of the rows committed by the last accept.  With a sliding window only the last rows
  // of a long verified block (a prefill) can ever be seen by a draft: the accept committed at least
  // Q - nd of its Q rows, the next draft starts right after the committed ones, and a query at p sees
  // context keys k > p - W; so rows before Q - nd - W are skipped (never computed, never stored).
  const int Q = c->last_qlen;
  const int skip = (dc.window > 0 && c->last_nd >= 0) ? std::max(0, Q - c->last_nd - dc.window) : 0;
  // With the drafter's page ring, the positions one call touches (injected rows from n - nd - W, reads
  // from n - W + 1, block rows and injected rows up to n + max(B, nd) - 1, where n >= n0 + Q - nd after an
  // accept of nd drafts of a block at n0) must not alias modulo the ring's R * pt positions.
  const int ring_pos = c->dring * c->cap.page_tokens;
  if (c->dring && (c->last_nd < 0 || dc.window + c->last_nd + std::max(B, c->last_nd) > ring_pos))
    return fail(DFLASH_E_STATE, "with a windowed drafter, draft_block must follow an accept of at most %d drafts",
                (ring_pos - dc.window) / 2);
  const int L = Q - skip, Ri = batch * L;
  Rows ri = c->rows(1);
  PrepArgs p;
  memset(&p, 0, sizeof p);
  p.batch = batch;
  for (int b = 0; b < batch; ++b) p.slots[b] = slots[b];
  p.q_len = L;
  p.row_skip = skip;
  p.state = c->state();
  p.rows = ri;
  p.mode = 1;
  p.mask_id = dc.mask_id;
  p.vocab = m.vocab;
  p.err = c->err();
  HIP_OK(launch_prep(p, s));
  int ss_n = 1;
  struct ModeScope {  // x16 mode for this call's projections; cleared on every exit
    dflash_ctx *c;
    ~ModeScope() { c->x16 = false; }
  } mode_scope{c};
  c->x16 = m.dtype == DFLASH_BF16 && Ri >= kTcMinRows;
  {
    GemmArgs a = gemm_base(d_feats, dc.n_taps * H, Ri, H, dc.n_taps * H, EPI_RESID_NORM);
    if (skip) {  // the last L of every Q feature rows
      a.x_take = L;
      a.x_stride = Q;
      a.x_off = skip;
    }
    a.nseg = 1;
    a.seg[0] = GemmSeg{c->fc, H};
    if ((st = run_resid_norm(c, a, Ri, nullptr, nullptr, 0, all_rows(c->hidden_norm, Ri), s, &ss_n)) !=
        DFLASH_OK)
      return st;
  }
  {
    GemmArgs a = gemm_base(c->wsp<void>(c->L.xn), H, Ri, dc.layers * 2 * KD, H, EPI_PARTIAL);
    a.nseg = 2 * dc.layers;
    QkvPostArgs p = post_base(c, ri, Ri, true);  // the drafter's K / V
    p.ld_src = dc.layers * 2 * KD;
    p.nseg = 2 * dc.layers;
    for (int j = 0; j < dc.layers; ++j) {
      a.seg[2 * j] = GemmSeg{c->dl[j].wk, KD};
      a.seg[2 * j + 1] = GemmSeg{c->dl[j].wv, KD};
      p.seg[2 * j] = PostSeg{m.kv_heads, ROLE_K, (const float *)c->dl[j].k_norm, c->dlayer(j), 0};
      p.seg[2 * j + 1] = PostSeg{m.kv_heads, ROLE_V, nullptr, c->dlayer(j), 0};
    }
    p.total_heads = dc.layers * 2 * m.kv_heads;
    with_norm(c, a, ss_n);
    int np = 1;
    const float *part = nullptr;
    int64_t part_stride = 0;
    if ((st = run_partial(c, a, Ri, s, &np, &part, &part_stride)) != DFLASH_OK) return st;
    p.src = part;
    p.n_part = np;
    p.part_stride = part_stride;
    HIP_OK(launch_qkv_post(p, c->dt(), s));
  }
  // 2. The block [anchor, MASK x (B-1)].
  c->x16 = m.dtype == DFLASH_BF16 && batch * B >= kTcMinRows;
  Rows rd = c->rows(2);
  p.rows = rd;
  p.q_len = B;
  p.row_skip = 0;
  p.mode = 2;
  p.block_out = d_block;
  HIP_OK(launch_prep(p, s));
  const int R = batch * B;
  HIP_OK(launch_embed(c->embed, c->dt(), rd, R, H, m.vocab, c->wsp<float>(c->L.x), c->err(), s));
  if ((st = prep_norm(c, R, c->dl[0].attn_norm, s)) != DFLASH_OK) return st;
  ss_n = 1;
  const int ctx_bound = c->max_ctx(slots, batch);
  const int nd = B - 1;
  for (int j = 0; j < dc.layers; ++j) {
    // after the last layer: the final norm over the B - 1 mask positions of every block, packed
    const NextNorm next = j + 1 < dc.layers ? all_rows(c->dl[j + 1].attn_norm, R) : NextNorm{c->d_final_norm, nd, B, 1};
    st = run_layer(c, c->dl[j], c->dlayer(j), rd, slots, batch, B, 1, ctx_bound, nullptr, 0, next, &ss_n, s);
    if (st != DFLASH_OK) return st;
  }
  float *logits = d_logits ? d_logits : c->wsp<float>(c->L.dlogits);
  const bool selector = dc.selector_top_k > 0;
  GemmArgs a = gemm_base(c->wsp<void>(c->L.xn), H, batch * nd, m.vocab, H, EPI_STORE_F32);
  a.nseg = 1;
  a.seg[0] = GemmSeg{c->lm_head, m.vocab};
  with_norm(c, a, ss_n);
  a.out_f32 = logits;
  a.ld_out = m.vocab;
  if ((st = run_gemm(c, a, batch * nd, s)) != DFLASH_OK) return st;
  if (selector) return run_selector(c, s, batch, logits, d_block);
  FilterArgs f;
  memset(&f, 0, sizeof f);
  f.logits = logits;
  f.rows = batch * nd;
  f.vocab = m.vocab;
  f.rows_per_seq = nd;
  f.stage_key = c->wsp<uint32_t>(c->L.skey);
  f.stage_idx = c->wsp<int32_t>(c->L.sidx);
  f.argmax_out = d_block;
  f.am_take = nd;
  f.am_stride = B;
  f.am_offset = 1;
  filter_plan(f, 1);
  if (sampling) {  // stochastic drafts: filter each row with the request's sampling, draw from it
    filter_setup(c, f, logits, batch * nd, nd, sampling, batch, d_q_ids, d_q_p, c->wsp<int32_t>(c->L.cn));
    HIP_OK(launch_filter(f, s));
    DraftSampleArgs ds;
    memset(&ds, 0, sizeof ds);
    ds.batch = batch;
    ds.nd = nd;
    ds.block = B;
    for (int b = 0; b < batch; ++b) {
      ds.slots[b] = slots[b];
      ds.seed[b] = sampling[b].seed;
    }
    ds.state = c->state();
    ds.q_id = d_q_ids;
    ds.q_p = d_q_p;
    ds.q_n = f.cand_n;
    ds.out = d_block;
    HIP_OK(launch_draft_sample(ds, s));
    return DFLASH_OK;
  }
  HIP_OK(launch_filter(f, s));
  return DFLASH_OK;
}

}  // namespace

dflash_status dflash_selector_state(dflash_ctx *c, hipStream_t s, int32_t batch, int32_t *d_ids, float *d_logits,
                                    float *d_trans) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  if (c->dcfg.selector_top_k < 1) return fail(DFLASH_E_STATE, "the drafter has no selector");
  if (batch < 1 || batch > c->sel_batch) return fail(DFLASH_E_STATE, "batch exceeds the last selector pass");
  if (!d_ids || !d_logits || !d_trans) return fail(DFLASH_E_INVAL, "null buffer");
  const size_t nd = c->dcfg.block_size - 1, K = c->dcfg.selector_top_k, rows = batch * nd;
  HIP_OK(hipMemcpy2DAsync(d_ids, K * sizeof(int32_t), c->wsp<int32_t>(c->L.sel_id), kMaxTopK * sizeof(int32_t),
                          K * sizeof(int32_t), rows, hipMemcpyDeviceToDevice, s));
  HIP_OK(hipMemcpy2DAsync(d_logits, K * sizeof(float), c->wsp<float>(c->L.sel_s), kMaxTopK * sizeof(float),
                          K * sizeof(float), rows, hipMemcpyDeviceToDevice, s));
  HIP_OK(hipMemcpyAsync(d_trans, c->wsp<float>(c->L.sel_t), rows * K * K * sizeof(float), hipMemcpyDeviceToDevice, s));
  return DFLASH_OK;
}

dflash_status dflash_draft_block(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots, const void *d_feats,
                                 int32_t *d_block, float *d_logits) {
  return draft_block_impl(c, s, batch, slots, d_feats, d_block, d_logits, nullptr, nullptr, nullptr);
}

dflash_status dflash_draft_block_sampled(dflash_ctx *c, hipStream_t s, int32_t batch, const int32_t *slots,
                                         const void *d_feats, const dflash_sampling *sampling, int32_t *d_block,
                                         int32_t *d_q_ids, float *d_q_p, float *d_logits) {
  if (!sampling) return fail(DFLASH_E_INVAL, "null sampling");
  return draft_block_impl(c, s, batch, slots, d_feats, d_block, d_logits, sampling, d_q_ids, d_q_p);
}

dflash_status dflash_op_linear(hipStream_t s, int32_t dtype, int32_t M, int32_t N, int32_t K, const void *d_x,
                               const void *d_w, float *d_y) {
  if (dtype != DFLASH_BF16 && dtype != DFLASH_F32) return fail(DFLASH_E_INVAL, "bad dtype");
  const int kstep = dtype == DFLASH_BF16 ? 32 : 16;
  if (M < 1 || N < 16 || N % 16 || K < kstep || K % kstep) return fail(DFLASH_E_INVAL, "bad GEMM shape");
  if (!d_x || !d_w || !d_y) return fail(DFLASH_E_INVAL, "null pointer");
  GemmArgs a = gemm_base(d_x, K, M, N, K, EPI_STORE_F32);
  a.nseg = 1;
  a.seg[0] = GemmSeg{d_w, N};
  a.out_f32 = d_y;
  a.ld_out = N;
  return run_gemm(dtype == DFLASH_BF16 ? 2 : 4, dtype == DFLASH_BF16 ? 0 : 1, a, M, s);
}

dflash_status dflash_op_linear_f16x(hipStream_t s, int32_t M, int32_t N, int32_t K, const void *d_x, const void *d_w,
                                    float *d_y, int32_t max_ranges, int32_t *ranges) {
  if (M < 1 || N < 32 || N % 32 || K < 64 || K % 64) return fail(DFLASH_E_INVAL, "bad GEMM shape");
  if (max_ranges < 1 || max_ranges > kTcMaxRanges || (max_ranges > 1 && !ranges))
    return fail(DFLASH_E_INVAL, "max_ranges out of range (or null ranges)");
  if (!d_x || !d_w || !d_y) return fail(DFLASH_E_INVAL, "null pointer");
  GemmArgs a = gemm_base(d_x, K, M, N, K, max_ranges > 1 ? EPI_PARTIAL : EPI_STORE_F32);
  a.nseg = 1;
  a.seg[0] = GemmSeg{d_w, N};
  a.out_f32 = d_y;
  a.ld_out = N;
  a.part_stride = (int64_t)M * N;
  TcPlan p;
  if (!gemm_tc_plan(a, (int64_t)max_ranges * M * N, &p)) return fail(DFLASH_E_INVAL, "shape not supported");
  HIP_OK(launch_gemm_tc(a, p, s));
  if (ranges) *ranges = p.ranges;
  return DFLASH_OK;
}

size_t dflash_op_linear_sk_scratch_bytes(int32_t N) { return N > 0 && N % 32 == 0 ? sk_scratch_bytes(N) : 0; }

dflash_status dflash_op_linear_sk(hipStream_t s, int32_t dtype, int32_t M, int32_t N, int32_t K, const void *d_x,
                                  const void *d_w, float *d_y, void *d_scratch, size_t scratch_bytes) {
  if (N > 0 && N % 32 == 0 && scratch_bytes < sk_scratch_bytes(N))
    return fail(DFLASH_E_INVAL, "scratch of %zu bytes, %zu needed", scratch_bytes, sk_scratch_bytes(N));
  return df::op_linear_sk(s, dtype, M, N, K, d_x, d_w, d_y, d_scratch);
}

dflash_status dflash_profile(dflash_ctx *c, int32_t enable) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  c->profiling = enable != 0;
  if (enable) c->recorded.clear();
  return DFLASH_OK;
}

dflash_status dflash_profile_replay(dflash_ctx *c, hipStream_t s, int32_t iters, double *ms, double *bytes,
                                    int32_t *launches) {
  if (!c || !ms || !bytes || !launches || iters < 1) return fail(DFLASH_E_INVAL, "bad argument");
  if (c->profiling) return fail(DFLASH_E_STATE, "disable profiling before replaying");
  double by = 0.0;
  int n = 0;
  for (const auto &r : c->recorded) {  // algorithmic bytes: every weight once per projection
    by += (double)r.a.N * (r.a.epi == EPI_SWIGLU ? 2 : 1) * r.a.K * c->es();
    ++n;
  }
  hipEvent_t e0, e1;
  HIP_OK(hipEventCreate(&e0));
  HIP_OK(hipEventCreate(&e1));
  HIP_OK(hipEventRecord(e0, s));
  for (int it = 0; it < iters; ++it)
    for (const auto &r : c->recorded) {
      if (r.x16) {
        HIP_OK(launch_gemm_tc(r.a, r.plan, s));
        continue;
      }
      dflash_status st = run_gemm(c->es(), c->dt(), r.a, r.rows, s);
      if (st != DFLASH_OK) return st;
    }
  HIP_OK(hipEventRecord(e1, s));
  HIP_OK(hipEventSynchronize(e1));
  float t = 0.f;
  HIP_OK(hipEventElapsedTime(&t, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *ms = t;
  *bytes = by;
  *launches = n;
  return DFLASH_OK;
}

dflash_status dflash_device_status(dflash_ctx *c, hipStream_t s) {
  if (!c) return fail(DFLASH_E_INVAL, "null context");
  HIP_OK(hipStreamSynchronize(s));
  int32_t flags[ERR_COUNT];
  HIP_OK(hipMemcpy(flags, c->err(), sizeof flags, hipMemcpyDeviceToHost));
  if (flags[ERR_TOKEN] || flags[ERR_PAGE] || flags[ERR_STATE]) {
    HIP_OK(hipMemset(c->err(), 0, sizeof flags));
    return fail(DFLASH_E_DEVICE, "device check failed:%s%s%s", flags[ERR_TOKEN] ? " token id out of range" : "",
                flags[ERR_PAGE] ? " position without a KV page" : "", flags[ERR_STATE] ? " inconsistent slot state" : "");
  }
  return DFLASH_OK;
}

}  // extern "C"
