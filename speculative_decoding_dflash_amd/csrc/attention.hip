// Paged attention on MFMA for the verify block (causal) and the draft block (bidirectional block +
// sliding-window injected context), gfx950.
//
// One work-group = (sequence, KV head, tile of query positions, key split); its 4 waves take the key
// pages of the split round-robin and merge through LDS at the end.  All query heads of the KV head's
// group and all positions of the tile are packed as "query vectors" (qv) into 16-wide MFMA tiles, so
// every K/V page is read once per work-group.
//   scores    S^T[key][qv] = K[key] . Q[qv]   (A = K page rows, B = Q^T held in registers)
//   output    O^T[dim][qv] += V^T[dim][key] P^T[key][qv]
// The accumulator layout of S^T (lane: qv = lane % 16, keys 4*(lane/16) + r) is exactly the B
// operand layout of the second product, so probabilities never leave registers.  K is stored
// token-major and V dim-major inside a page, so both A operands are contiguous loads.
// Softmax is online in fp32 (running max per qv, corrections applied to the accumulators); a split
// that sees no allowed key publishes m = -inf, l = 0.  Several splits are merged by a second kernel.
// Operand types: bf16 models keep q and the KV cache in fp16 and feed the probabilities to the PV
// product as fp16 (fp32 accumulation throughout); fp32 models run the fp32 MFMA on fp32 operands.  The
// output is the o projection's X operand (fp16 for bf16 models, like q and the KV cache).
#include "kernels.h"

namespace df {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));

constexpr float kAttnLazy = 8.f;  // see the softmax state of attn_kernel

template <typename T, int D> struct AttnFrag;

// K fragments: kSteps 16-byte vectors per lane (A operand of S^T = K Q^T, row = key = lane % 16).
// V fragments: D/16 vectors per lane (A operand of O^T += V^T P^T, row = dim, 4 keys per lane).
template <int D> struct AttnFrag<f16, D> {
  static constexpr int kSteps = D / 32;  // QK^T steps of 32 dims (8 per lane)
  static constexpr int kEPL = 8;         // dims per lane per step: ks * 32 + (lane / 16) * 8 + e
  using VF = u32x2;                      // 4 fp16 keys of one dim
  static DF_DEVICE u32x4 pack(const float *v) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (uint32_t)f32_to_f16(v[2 * j]) | ((uint32_t)f32_to_f16(v[2 * j + 1]) << 16);
    return r;
  }
  static DF_DEVICE u32x4 load_q(const f16 *qrow, int ks, int g) {
    return *reinterpret_cast<const u32x4 *>(qrow + ks * 32 + g * 8);
  }
  static DF_DEVICE void load_k(u32x4 *kf, const f16 *kblk, int key, int g) {
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) kf[ks] = *reinterpret_cast<const u32x4 *>(kblk + key * D + ks * 32 + g * 8);
  }
  static DF_DEVICE void load_v(VF *vf, const f16 *vblk, int l16, int g) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *reinterpret_cast<const u32x2 *>(vblk + (dt * 16 + l16) * 16 + 4 * g);
  }
  static DF_DEVICE void qk(f32x4 &acc, const u32x4 *kf, const u32x4 *q) {
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h16x8, kf[ks]), __builtin_bit_cast(h16x8, q[ks]),
                                                   acc, 0, 0, 0);
  }
  // element i (key 4g + i) of a V fragment, as raw bits
  static DF_DEVICE void set_v(VF &v, int i, uint32_t bits) {
    const int w = i >> 1, sh = (i & 1) * 16;
    v[w] = (v[w] & ~(0xFFFFu << sh)) | (bits << sh);
  }
  static DF_DEVICE uint32_t raw(const f16 &e) { return e.bits; }
  // p[r]: probability of key 4g + r for this lane's qv (in [0, 1]: fp16 keeps 11 significant bits of it).
  static DF_DEVICE void pv(f32x4 *o, const VF *vf, const float *p) {
    h16x4 pb;
    pb[0] = (_Float16)p[0];
    pb[1] = (_Float16)p[1];
    pb[2] = (_Float16)p[2];
    pb[3] = (_Float16)p[3];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h16x4, vf[dt]), pb, o[dt], 0, 0, 0);
  }
};

template <int D> struct AttnFrag<float, D> {
  static constexpr int kSteps = D / 16;  // 16 dims per step (4 per lane), as 4 K=4 slices
  static constexpr int kEPL = 4;         // dims per lane per step: ks * 16 + (lane / 16) * 4 + e
  using VF = u32x4;                      // 4 fp32 keys of one dim
  static DF_DEVICE u32x4 pack(const float *v) {
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = __builtin_bit_cast(uint32_t, v[j]);
    return r;
  }
  static DF_DEVICE u32x4 load_q(const float *qrow, int ks, int g) {
    return *reinterpret_cast<const u32x4 *>(qrow + ks * 16 + g * 4);
  }
  static DF_DEVICE void load_k(u32x4 *kf, const float *kblk, int key, int g) {
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) kf[ks] = *reinterpret_cast<const u32x4 *>(kblk + key * D + ks * 16 + g * 4);
  }
  static DF_DEVICE void load_v(VF *vf, const float *vblk, int l16, int g) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) vf[dt] = *reinterpret_cast<const u32x4 *>(vblk + (dt * 16 + l16) * 16 + 4 * g);
  }
  static DF_DEVICE void qk(f32x4 &acc, const u32x4 *kf, const u32x4 *q) {
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      const f32x4 k = __builtin_bit_cast(f32x4, kf[ks]);
      const f32x4 qf = __builtin_bit_cast(f32x4, q[ks]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(k[j], qf[j], acc, 0, 0, 0);
    }
  }
  static DF_DEVICE void set_v(VF &v, int i, uint32_t bits) { v[i] = bits; }
  static DF_DEVICE uint32_t raw(const float &e) { return __builtin_bit_cast(uint32_t, e); }
  static DF_DEVICE void pv(f32x4 *o, const VF *vf, const float *p) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 v = __builtin_bit_cast(f32x4, vf[dt]);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v[j], p[j], o[dt], 0, 0, 0);
    }
  }
};

// Loads through the vector memory path even where the address is uniform: a scalar load's wait
// (lgkmcnt, which has no order) would also be taken by every later kernel-argument load.
template <typename X>
DF_DEVICE X vload(const X *p, int i) {
  asm volatile("" : "+v"(i));
  return p[i];
}

template <typename T, int D, int NQT, bool FUSED>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  using F = AttnFrag<T, D>;
  using XT = T;  // output (X operand) type: the attention operands' storage type
  __shared__ __attribute__((aligned(16))) float so[4][16][D + 4];  // rows 16-byte aligned
  __shared__ float sm[4][NQT * 16], sl[4][NQT * 16];
  // fused calls: the block's own keys (K [16][D], V [D][16], row j = block row j), built here from raw k / v
  __shared__ __attribute__((aligned(16))) T s_bk[FUSED ? 16 * D : 1], s_bv[FUSED ? D * 16 : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  {
    // Touch the argument block's first four 64-byte lines together: each first touch misses the
    // scalar cache, and fetched as they are needed the misses would be waited for one after another.
    const int k0 = a.ldq, k1 = a.q_len, k2 = a.ld_raw, k3 = a.abs_range;
    asm volatile("" ::"s"(k0), "s"(k1), "s"(k2), "s"(k3));
  }
  const int kvh = a.kvl.kv_heads, G = a.q_heads / kvh;
  const int ntile = (a.q_len + a.q_tile - 1) / a.q_tile;
  // Work-groups are dealt to the 8 XCDs round-robin in launch order.  Renumbering them so that each
  // XCD gets a contiguous range of (query tile, KV head, sequence, split) puts the query tiles of one
  // (KV head, split) -- which read the same pages -- under one L2.
  int bx = blockIdx.x, split = blockIdx.y;
  const int gx = a.n_seq * kvh * ntile, n_wg = gx * a.n_splits;  // the launch grid, from the arguments
  if (n_wg % 8 == 0) {
    const int lin = blockIdx.x + gx * blockIdx.y;
    const int v = (lin % 8) * (n_wg / 8) + lin / 8;
    bx = v % gx;
    split = v / gx;
  }
  const int qt = bx % ntile;
  bx /= ntile;
  const int kh = bx % kvh;
  const int b = bx / kvh;
  const int p0 = qt * a.q_tile;
  const int np = min(a.q_tile, a.q_len - p0);
  const int nqv = np * G;
  const int rbase = b * a.q_len + p0;
  // scores are kept in log2 units (scaled by log2 e), so that every exponential is one v_exp_f32
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  const float NEG = -INFINITY;
  int err_page = 0;  // raised at the end (see below)

  // The prologue is ordered so that no load waits behind loads it does not need (a wave's loads return
  // in issue order): (A) loads addressed by the arguments alone; (B) loads addressed by positions from
  // (A): rotary rows and the block-table entries of the block's own keys; (C) the wave's first two K/V
  // pages, which stream while (D) q is normalised and rotated and the block's k / v are written.
  // Fused calls (raw q / k / v in, see AttnArgs) are a separate instantiation, so none of this is
  // behind a run-time branch.
  const int pt = a.kvl.page_tokens;
  const int32_t *bt = a.block_table + (size_t)a.seq_slot[b] * a.bt_stride;
  const int pps = a.split_tokens / pt;
  const bool pre = a.abs_range && pps <= 4 * 64;
  constexpr int EPL = F::kEPL, SD = 4 * EPL, KH = F::kSteps / 2, KHS = KH > 0 ? KH : 1;
  constexpr int kWR = 2;  // block rows per wave (rows wave + 4 w) whose k / v loads are hoisted
  // A wave can have at most 63 vector memory instructions outstanding; (A) issues ~30 (fused), so
  // none of it waits for an earlier load to return.  Fused calls (q_len <= 16, checked by the host)
  // read every block position once, lane j holding row j's, and share it by lane exchange.

  // (A) block-table entries of the split's pages when its key range is known on the host (lane i: the
  // wave's page i), the rows' positions, q (or raw q and its gain), the raw k / v of the block rows.
  int pre_bt = -1;
  if (pre) {
    const int pidx = split * pps + wave + 4 * lane;
    if (lane < (pps - wave + 3) / 4 && pidx < a.bt_stride) pre_bt = bt[pidx];
  }
  int first_pos_v = 0, last_pos_v = 0, nblk_v = 0;
  int bl_pos = 0, bl_val = 0;  // block row `lane` (fused): its position and validity
  if constexpr (FUSED) {
    const int row = b * a.q_len + (lane < a.q_len ? lane : 0);
    bl_pos = a.rows.pos[row];
    bl_val = a.rows.valid[row];
  } else {
    first_pos_v = vload(a.rows.pos, rbase);
    last_pos_v = vload(a.rows.pos, rbase + np - 1);
    nblk_v = vload(a.rows.pos, b * a.q_len);
  }
  int qpos[NQT];
  bool qok[NQT];
  u32x4 q[NQT][F::kSteps];
  float qraw[NQT][F::kSteps][EPL], qg[F::kSteps][EPL];
  const int wi = lane < D / 2 ? lane : 0;  // write rows: lane i < D/2 holds dims i and i + D/2
  float w_k[kWR][2], w_v[kWR][2], kg[2];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    const int qv = t * 16 + l16;
    qok[t] = qv < nqv;
    const int row = rbase + (qok[t] ? qv / G : 0);
    const int head = kh * G + (qok[t] ? qv % G : 0);
    if constexpr (!FUSED) {
      qpos[t] = a.rows.pos[row];
      const T *qrow = (const T *)a.q + (size_t)row * a.ldq + head * D;
#pragma unroll
      for (int ks = 0; ks < F::kSteps; ++ks) q[t][ks] = F::load_q(qrow, ks, g);
    } else {
      qpos[t] = row - b * a.q_len;  // the row's index in the block for now; its position below
      // this lane holds dims ks * SD + g * EPL + e of its query vector
      const float *src = a.raw + (size_t)row * a.ld_raw + head * D;
#pragma unroll
      for (int ks = 0; ks < F::kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const float4 u = *reinterpret_cast<const float4 *>(src + ks * SD + g * EPL + e);
          qraw[t][ks][e] = u.x;
          qraw[t][ks][e + 1] = u.y;
          qraw[t][ks][e + 2] = u.z;
          qraw[t][ks][e + 3] = u.w;
        }
    }
  }
  if constexpr (FUSED) {
#pragma unroll
    for (int ks = 0; ks < F::kSteps; ++ks)
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {  // 16-byte aligned (checked by the host)
        const float4 u = *reinterpret_cast<const float4 *>(a.q_gain + ks * SD + g * EPL + e);
        qg[ks][e] = u.x;
        qg[ks][e + 1] = u.y;
        qg[ks][e + 2] = u.z;
        qg[ks][e + 3] = u.w;
      }
    kg[0] = a.k_gain[wi];
    kg[1] = a.k_gain[wi + D / 2];
#pragma unroll
    for (int w = 0; w < kWR; ++w) {
      const int j = wave + 4 * w;
      const int row = b * a.q_len + (j < a.q_len ? j : 0);
      const float *kr = a.raw + (size_t)row * a.ld_raw + (size_t)(a.q_heads + kh) * D;
      const float *vr = a.raw + (size_t)row * a.ld_raw + (size_t)(a.q_heads + kvh + kh) * D;
      w_k[w][0] = kr[wi];
      w_k[w][1] = kr[wi + D / 2];
      w_v[w][0] = vr[wi];
      w_v[w][1] = vr[wi + D / 2];
    }
  }
  // (C, split range known up front) the wave's first two pool pages, which need only their
  // block-table entries: entries past the sequence's pages are -1 (loads of a dummy block) and pages
  // past the key range are loaded but never used.  Fused calls take the block's own keys from an LDS
  // copy (see `patch`), so no page has to wait for this call's K/V writes.
  const T *kvb = (const T *)a.kv;
  const T *dummy = kvb;
  u32x4 kf[2][F::kSteps];
  typename F::VF vf[2][D / 16];
  auto ring_loads = [&](int bts) {  // bts: lane p holds page p's block-table entry (-1: none)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int pg = __builtin_amdgcn_readlane(bts, p);
      F::load_k(kf[p], pg >= 0 ? kvb + a.kvl.block(pg, 0, kh) : dummy, l16, g);
      F::load_v(vf[p], pg >= 0 ? kvb + a.kvl.block(pg, 1, kh) : dummy, l16, g);
    }
  };
  // Unconditional (dummy blocks when the range is not known up front), like every global access up to
  // the page loop: a wave's outstanding-load count must be the same on every path, or later waits
  // fall back to waiting for everything, the K/V pages included.  For the same reason the kernel's
  // conditional global writes (the block's K/V to the pool, error flags) are issued at its end.
  ring_loads(pre ? pre_bt : -1);
  if constexpr (FUSED) {  // zero the LDS block page rows this wave owns (rows j = wave mod 4)
    for (int j = wave; j < 16; j += 4)
      for (int d = lane; d < D; d += 64) {
        Elem<T>::store(&s_bk[j * D + d], 0.f);
        Elem<T>::store(&s_bv[d * 16 + j], 0.f);
      }
  }

  int w_pos[kWR], w_val[kWR];
  if constexpr (FUSED) {  // positions from the block's lanes (waits for (A)'s first loads)
    first_pos_v = __builtin_amdgcn_readlane(bl_pos, p0);
    last_pos_v = __builtin_amdgcn_readlane(bl_pos, p0 + np - 1);
    nblk_v = __builtin_amdgcn_readlane(bl_pos, 0);
#pragma unroll
    for (int t = 0; t < NQT; ++t) qpos[t] = __shfl(bl_pos, qpos[t]);
#pragma unroll
    for (int w = 0; w < kWR; ++w) {
      const int j = wave + 4 * w;
      w_pos[w] = __builtin_amdgcn_readlane(bl_pos, j < a.q_len ? j : 0);
      w_val[w] = j < a.q_len && __builtin_amdgcn_readlane(bl_val, j < a.q_len ? j : 0);
    }
  }

  __builtin_amdgcn_sched_barrier(0);  // (B) addresses wait for (A): keep them after all of (A)'s loads
  // (B) rotary (cos, sin) of the query rows and of the write rows, and the write rows' pages
  float2 qcs[NQT][KHS][EPL];
  float2 w_cs[kWR];
  int w_page[kWR];
  if constexpr (FUSED) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int pos = qpos[t];
      const bool pos_ok = pos >= 0 && pos < a.rope_rows;
      const float2 *rp = a.rope + (size_t)(pos_ok ? pos : 0) * (D / 2);
#pragma unroll
      for (int ks = 0; ks < KHS; ++ks)
#pragma unroll
        for (int e = 0; e < EPL; ++e) qcs[t][ks][e] = rp[KH > 0 ? ks * SD + g * EPL + e : (g & 1) * EPL + e];
    }
#pragma unroll
    for (int w = 0; w < kWR; ++w) {
      const int pos = w_pos[w];
      const bool ok = pos >= 0 && pos < a.rope_rows && pos / pt < a.bt_stride;
      w_cs[w] = a.rope[(size_t)(ok ? pos : 0) * (D / 2) + wi];
      const int pg = vload(bt, ok ? pos / pt : 0);
      w_page[w] = ok ? pg : -1;
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // A block's rows hold consecutive positions, valid rows first (as the row preparation writes them):
  // the block's keys are positions [blk_lo, blk_lo + n_valid).
  int blk_lo = 0x7fffffff, n_valid = 0;
  if constexpr (FUSED) {
    n_valid = __popcll(__ballot(lane < a.q_len && bl_val));
    if (n_valid > 0) blk_lo = __builtin_amdgcn_readlane(bl_pos, 0);
  }
  // key range of the split (uniform; read back into scalar registers)
  int klo, khi;
  if (a.mode == 0) {
    klo = 0;
    khi = last_pos_v + 1;
  } else {
    khi = nblk_v + a.q_len;
    klo = a.window > 0 ? max(0, first_pos_v - a.window + 1) : 0;
  }
  const int kbase = pre ? 0 : __builtin_amdgcn_readfirstlane((klo / pt) * pt);  // 0 whenever pre holds
  const int kstart = kbase + split * a.split_tokens;
  // Wave w takes the split's pages w, w + 4, ..., in chunks of 64: lane i holds the block-table entry
  // of the chunk's page i (read once per chunk), and two pages' K/V fragments are in flight while one
  // is consumed.  Loads past the chunk's last page read a valid dummy block (the pool's first), so
  // that every load is unconditional.
  auto chunk_bt = [&](int c0, int n_my) {
    if (pre && c0 == 0) return pre_bt;  // same pages: kstart = split * split_tokens when the range is absolute
    int e = -1;
    if (lane < n_my) {
      const int pidx = (kstart + (wave + 4 * (c0 + lane)) * pt) / pt;
      e = pidx < a.bt_stride ? bt[pidx] : -1;
    }
    return e;
  };
  auto page_range = [&](int &kstop, int &n_all) {
    kstop = __builtin_amdgcn_readfirstlane(min(khi, kstart + a.split_tokens));
    const int npg = kstop > kstart ? (kstop - kstart + pt - 1) / pt : 0;
    n_all = wave < npg ? (npg - wave + 3) / 4 : 0;
  };
  int kstop = 0, n_all = 0;
  page_range(kstop, n_all);
  int n_my = min(64, n_all), my_bt = pre_bt;  // pre: -1 past the wave's pages, its pages in flight
  const int first_pos = first_pos_v;
  const int nblk = nblk_v;

  // (D) raw q -> RMSNorm (q_gain) -> rotate-half RoPE in the fragment layout: the rotation partner of
  // dim i < D/2 (step ks < kSteps / 2) is step ks + kSteps / 2 of the same lane; with a single step
  // (D == SD) it lives in lane ^ 32.
  if constexpr (FUSED) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      const int pos = qpos[t];
      err_page |= !(pos >= 0 && pos < a.rope_rows) && qok[t];
      float(&v)[F::kSteps][EPL] = qraw[t];
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < F::kSteps; ++ks)
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          ss += v[ks][e] * v[ks][e] + v[ks][e + 1] * v[ks][e + 1] + v[ks][e + 2] * v[ks][e + 2] + v[ks][e + 3] * v[ks][e + 3];
      ss += __shfl_xor(ss, 16);
      ss += __shfl_xor(ss, 32);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
      if constexpr (KH > 0) {
#pragma unroll
        for (int ks = 0; ks < KH; ++ks)
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            const float v1 = v[ks][e] * r * qg[ks][e], v2 = v[ks + KH][e] * r * qg[ks + KH][e];
            const float2 cs = qcs[t][ks][e];
            v[ks][e] = v1 * cs.x - v2 * cs.y;
            v[ks + KH][e] = v2 * cs.x + v1 * cs.y;
          }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const float own = v[0][e] * r * qg[0][e];
          const float other = __shfl_xor(own, 32);
          const float2 cs = qcs[t][0][e];
          v[0][e] = g < 2 ? own * cs.x - other * cs.y : own * cs.x + other * cs.y;
        }
      }
#pragma unroll
      for (int ks = 0; ks < F::kSteps; ++ks) q[t][ks] = F::pack(v[ks]);
    }
  }

  // Key range [lo, hi) of every query vector: causal (mode 0); block keys plus the sliding window of
  // context keys (mode 1, the drafter); empty for padding query vectors.
  int lo[NQT], hi[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    if (!qok[t]) {
      lo[t] = 1;
      hi[t] = 0;
    } else if (a.mode == 0) {
      lo[t] = klo;
      hi[t] = min(khi, qpos[t] + 1);
    } else {
      lo[t] = a.window > 0 ? max(klo, min(nblk, qpos[t] - a.window + 1)) : klo;
      hi[t] = khi;
    }
  }

  // Online softmax state per query vector: the reference maximum m (log2 units) moves only when a page's
  // scores exceed it by more than kAttnLazy, so the probabilities stay below 2^kAttnLazy, the lanes of a
  // query vector exchange their maxima only when one of them grows, and the accumulators are rescaled
  // only then; mb is m, or 0 while no key has been seen.  o / l (and the merges, which take any reference
  // maximum) are unchanged up to rounding.
  float m[NQT], l[NQT], mb[NQT];
  f32x4 o[NQT][D / 16];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    m[t] = NEG;
    mb[t] = 0.f;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[t][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }

  auto pool_row = [&](int pos, int page, float k1, float k2, float v1, float v2) {
    if (lane < D / 2) {
      const int tok = pos % pt;
      T *kd = (T *)a.kv + a.kvl.k_index(page, kh, tok, 0);
      T *vd = (T *)a.kv + a.kvl.v_index(page, kh, tok, 0);
      Elem<T>::store(kd + wi, k1);
      Elem<T>::store(kd + wi + D / 2, k2);
      Elem<T>::store(vd + (size_t)wi * pt, v1);
      Elem<T>::store(vd + (size_t)(wi + D / 2) * pt, v2);
    }
  };
  bool w_do[kWR] = {};  // hoisted block rows whose K/V go to the pool at the end
  if constexpr (FUSED) {
    // The block's own keys that fall in this split: RMSNorm (k_gain) + RoPE of k; k and v go to the
    // LDS page now and to the pool at the end (wave j % 4 takes block row j).  Every query tile's
    // work-group of the split writes the same values to the pool.
    auto norm_rope = [&](float &k1, float &k2, float2 cs) {
      float ss = lane < D / 2 ? k1 * k1 + k2 * k2 : 0.f;
      for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
      const float n1 = k1 * r * kg[0], n2 = k2 * r * kg[1];
      k1 = n1 * cs.x - n2 * cs.y;
      k2 = n2 * cs.x + n1 * cs.y;
    };
    auto lds_row = [&](int j, float k1, float k2, float v1, float v2) {
      if (lane < D / 2) {
        Elem<T>::store(&s_bk[j * D + wi], k1);
        Elem<T>::store(&s_bk[j * D + wi + D / 2], k2);
        Elem<T>::store(&s_bv[wi * 16 + j], v1);
        Elem<T>::store(&s_bv[(wi + D / 2) * 16 + j], v2);
      }
    };
#pragma unroll
    for (int w = 0; w < kWR; ++w) {
      const int pos = w_pos[w];
      w_do[w] = w_val[w] && pos >= kstart && pos < kstop;  // wave-uniform
      if (!w_do[w]) continue;
      norm_rope(w_k[w][0], w_k[w][1], w_cs[w]);
      lds_row(wave + 4 * w, w_k[w][0], w_k[w][1], w_v[w][0], w_v[w][1]);
      err_page |= w_page[w] < 0;
      w_do[w] = w_page[w] >= 0;
    }
    for (int j = wave + 4 * kWR; j < a.q_len; j += 4) {  // rows beyond the hoisted ones (q_len > 8)
      const int row = b * a.q_len + j, pos = a.rows.pos[row];
      if (!a.rows.valid[row] || pos < kstart || pos >= kstop) continue;  // wave-uniform
      const int pidx = pos / pt;
      const int page = (pidx < a.bt_stride && pos < a.rope_rows) ? bt[pidx] : -1;
      const float *kr = a.raw + (size_t)row * a.ld_raw + (size_t)(a.q_heads + kh) * D;
      const float *vr = a.raw + (size_t)row * a.ld_raw + (size_t)(a.q_heads + kvh + kh) * D;
      float k1 = kr[wi], k2 = kr[wi + D / 2];
      const float v1 = vr[wi], v2 = vr[wi + D / 2];
      norm_rope(k1, k2, a.rope[(size_t)(page >= 0 ? pos : 0) * (D / 2) + wi]);
      lds_row(j, k1, k2, v1, v2);
      if (page < 0) err_page = 1;
      else pool_row(pos, page, k1, k2, v1, v2);
    }
    __syncthreads();  // the LDS page is complete before any wave patches its fragments from it
  }

  // One page of 16 keys starting at position ps: scores, online softmax, P V.  Keys outside
  // [lo, hi) of a query vector, or outside [klim_lo, klim_hi), are masked.
  auto consume = [&](const u32x4 *kfp, const typename F::VF *vfp, int ps, int klim_lo, int klim_hi) {
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      F::qk(s, kfp, q[t]);  // lane holds S^T[key = 4g + r][qv = l16]
      float sv[4], mx = NEG;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = ps + 4 * g + r;
        sv[r] = (kp >= lo[t] && kp < hi[t] && kp >= klim_lo && kp < klim_hi) ? s[r] * scale : NEG;
        mx = __builtin_elementwise_max(mx, sv[r]);
      }
      if (__builtin_amdgcn_ballot_w64(mx > m[t] + kAttnLazy)) {  // some query vector's maximum moves
        mx = __builtin_elementwise_max(mx, __shfl_xor(mx, 16));
        mx = __builtin_elementwise_max(mx, __shfl_xor(mx, 32));
        const float mn = mx > m[t] + kAttnLazy ? mx : m[t];
        const float corr = mn == m[t] ? 1.f : __builtin_amdgcn_exp2f(m[t] - mn);  // 0 for the first keys
        l[t] *= corr;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[t][dt] *= corr;
        m[t] = mn;
        mb[t] = mn == NEG ? 0.f : mn;
      }
      float pr[4], ps_sum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(sv[r] - mb[t]);  // 0 for masked keys
        ps_sum += pr[r];
      }
      l[t] += ps_sum;
      F::pv(o[t], vfp, pr);
    }
  };
  if (!pre) {  // the first chunk's pages, now that the key range is known
    my_bt = chunk_bt(0, n_my);
    ring_loads(my_bt);
  }
  // Fused calls: a pool page holding block keys gets those keys' K/V from the LDS page (this call's
  // pool writes are not yet visible, and need not be); every key keeps its page, wave and position in
  // the online softmax, so the arithmetic is that of an all-pool read.
  auto patch = [&](u32x4 *kfp, typename F::VF *vfp, int ps) {
    const int off = ps - blk_lo;  // LDS row of the page's key 0
    const int jk = off + l16;     // this lane's K row
    const bool kin = jk >= 0 && jk < 16;
    u32x4 kt[F::kSteps];
    F::load_k(kt, s_bk, kin ? jk : 0, g);
#pragma unroll
    for (int ks = 0; ks < F::kSteps; ++ks)
      if (kin) kfp[ks] = kt[ks];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jv = off + 4 * g + i;
        if (jv >= 0 && jv < 16) F::set_v(vfp[dt], i, F::raw(s_bv[(dt * 16 + l16) * 16 + jv]));
      }
  };
  for (int c0 = 0; c0 < n_all; c0 += 64) {
    if (c0 > 0) {
      n_my = min(64, n_all - c0);
      my_bt = chunk_bt(c0, n_my);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int pg = p < n_my ? __builtin_amdgcn_readlane(my_bt, p) : -1;
        F::load_k(kf[p], pg >= 0 ? kvb + a.kvl.block(pg, 0, kh) : dummy, l16, g);
        F::load_v(vf[p], pg >= 0 ? kvb + a.kvl.block(pg, 1, kh) : dummy, l16, g);
      }
    }
    for (int i0 = 0; i0 < n_my; i0 += 2) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int ii = i0 + p;
        if (ii < n_my) {  // wave-uniform
          const int ps = kstart + (wave + 4 * (c0 + ii)) * pt;
          if (__builtin_amdgcn_readlane(my_bt, ii) < 0) {
            err_page = 1;
          } else {
            if (FUSED && ps + pt > blk_lo && ps < blk_lo + 16) patch(kf[p], vf[p], ps);  // wave-uniform
            consume(kf[p], vf[p], ps, 0, 0x7fffffff);
          }
        }
        const int nx = ii + 2;
        const int pg = nx < n_my ? __builtin_amdgcn_readlane(my_bt, nx) : -1;
        F::load_k(kf[p], pg >= 0 ? kvb + a.kvl.block(pg, 0, kh) : dummy, l16, g);
        F::load_v(vf[p], pg >= 0 ? kvb + a.kvl.block(pg, 1, kh) : dummy, l16, g);
      }
    }
  }

  // Merge the four waves, one 16-qv tile at a time: thread (qi = tid / 16, c = tid % 16) combines
  // dims [c * DPT, (c + 1) * DPT) of the tile's query vector qi, so all its LDS reads are independent.
  constexpr int DPT = D / 16;
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (g == 0) {
      sm[wave][t * 16 + l16] = m[t];
      sl[wave][t * 16 + l16] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) so[wave][l16][dt * 16 + 4 * g + r] = o[t][dt][r];
    __syncthreads();
    const int qi = tid >> 4, d0 = (tid & 15) * DPT;
    const int qv = t * 16 + qi;
    if (qv < nqv) {
      float mw[4], M = NEG;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mw[w] = sm[w][t * 16 + qi];
        M = fmaxf(M, mw[w]);
      }
      float f[4], L = 0.f, O[DPT];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = (mw[w] == NEG || M == NEG) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        L += f[w] * sl[w][t * 16 + qi];
      }
#pragma unroll
      for (int d = 0; d < DPT; ++d) {
        O[d] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) O[d] += f[w] * so[w][qi][d0 + d];
      }
      const int row = rbase + qv / G, head = kh * G + qv % G;
      if (a.n_splits == 1) {
        const size_t oi = (size_t)row * a.ldo + head * D + d0;
#pragma unroll
        for (int d = 0; d < DPT; ++d) store_x((XT *)a.out, oi + d, L > 0.f ? O[d] / L : 0.f);
      } else {
        const size_t pi = ((size_t)row * a.q_heads + head) * a.n_splits + split;
        float *po = a.part_o + pi * D + d0;
        if (a.counters) {  // written through to memory: the merging work-group may sit on another XCD
#pragma unroll
          for (int d = 0; d < DPT; ++d) __hip_atomic_store(po + d, O[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (d0 == 0) {
            __hip_atomic_store(&a.part_ml[pi * 2], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.part_ml[pi * 2 + 1], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          if constexpr (DPT % 4 == 0) {  // part_o rows are 16-byte aligned (D a multiple of 16)
#pragma unroll
            for (int d = 0; d < DPT; d += 4)
              *reinterpret_cast<float4 *>(po + d) = make_float4(O[d], O[d + 1], O[d + 2], O[d + 3]);
          } else {
#pragma unroll
            for (int d = 0; d < DPT; ++d) po[d] = O[d];
          }
          if (d0 == 0) {
            a.part_ml[pi * 2] = M;
            a.part_ml[pi * 2 + 1] = L;
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (FUSED) {
#pragma unroll
    for (int w = 0; w < kWR; ++w)
      if (w_do[w]) pool_row(w_pos[w], w_page[w], w_k[w][0], w_k[w][1], w_v[w][0], w_v[w][1]);
  }
  if (err_page) raise_err(a.err, ERR_PAGE);
  if (!a.counters || a.n_splits == 1) return;

  // Last-arriver merge of the splits of (sequence b, KV head kh).  Every thread's partial stores have
  // completed (vmcnt 0) before the work-group's arrival is counted; the work-group that sees all other
  // splits arrived reads their partials back (m, l through the coherent path; O blocks are whole cache
  // lines written only by their split and read only here) and writes the output.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores are done
  __syncthreads();
  int *cnt = a.counters + (b * kvh + kh) * ntile + qt;
  if (tid == 0) s_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.n_splits - 1;
  __syncthreads();
  if (!s_last) return;
  const int ns = a.n_splits;
  // LDS (the merge tile): m of every (qv, split), then l, then 1 / L per qv; ns <= D / 2 (host bound)
  float *wm = &so[0][0][0];
  float *wl = wm + nqv * ns;
  float *linv = wl + nqv * ns;
  for (int e = tid; e < nqv * ns; e += 256) {
    const int qv = e / ns, sp = e % ns;
    const int row = rbase + qv / G, head = kh * G + qv % G;
    const float *ml = a.part_ml + (((size_t)row * a.q_heads + head) * ns + sp) * 2;
    wm[e] = __hip_atomic_load(&ml[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wl[e] = __hip_atomic_load(&ml[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  for (int qv = tid; qv < nqv; qv += 256) {
    float M = NEG;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, wm[qv * ns + sp]);
    float L = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float ms = wm[qv * ns + sp];
      const float w = (ms == NEG || M == NEG) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      wm[qv * ns + sp] = w;  // now the split's weight
      L += w * wl[qv * ns + sp];
    }
    linv[qv] = L > 0.f ? 1.0f / L : 0.f;
  }
  __syncthreads();
  for (int e = tid; e < nqv * (D / 4); e += 256) {
    const int qv = e / (D / 4), d4 = (e % (D / 4)) * 4;
    const int row = rbase + qv / G, head = kh * G + qv % G;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + ((size_t)row * a.q_heads + head) * ns * D + d4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int sp = 0;
    for (; sp + 4 <= ns; sp += 4) {  // four splits' loads in flight at once
      float4 u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) u[k] = po[(size_t)(sp + k) * (D / 4)];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = wm[qv * ns + sp + k];
        acc.x += w * u[k].x;
        acc.y += w * u[k].y;
        acc.z += w * u[k].z;
        acc.w += w * u[k].w;
      }
    }
    for (; sp < ns; ++sp) {
      const float w = wm[qv * ns + sp];
      const float4 u = po[(size_t)sp * (D / 4)];
      acc.x += w * u.x;
      acc.y += w * u.y;
      acc.z += w * u.z;
      acc.w += w * u.w;
    }
    const float li = linv[qv];
    const size_t oi = (size_t)row * a.ldo + head * D + d4;
    store_x((XT *)a.out, oi + 0, acc.x * li);
    store_x((XT *)a.out, oi + 1, acc.y * li);
    store_x((XT *)a.out, oi + 2, acc.z * li);
    store_x((XT *)a.out, oi + 3, acc.w * li);
  }
  if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// out[row][head] = sum_s 2^{m_s - M} O_s / sum_s 2^{m_s - M} l_s  (splits in order; m in log2 units).
// One work-group per (row, head), thread d for dimension d.
template <typename XT>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a, int n_rows) {
  // Up to kR splits: every thread loads all (m, l) pairs (the same addresses across the work-group)
  // and its dimension's partial outputs at once, so the merge waits for one round of loads.
  constexpr int kR = 16;
  const int rh = blockIdx.x;  // row * q_heads + head
  const int D = a.kvl.head_dim, ns = a.n_splits;
  const int row = rh / a.q_heads, head = rh % a.q_heads;
  const float NEG = -INFINITY;
  const float *ml = a.part_ml + (size_t)rh * ns * 2;
  const float *po = a.part_o + (size_t)rh * ns * D;
  const int tid = threadIdx.x;
  if (ns <= kR) {
    const int dim = tid < D ? tid : 0;
    float mv[kR], lv[kR], pv[kR];
#pragma unroll
    for (int s = 0; s < kR; ++s) {
      const int sc = s < ns ? s : 0;  // loads stay unconditional
      mv[s] = ml[2 * sc];
      lv[s] = ml[2 * sc + 1];
      pv[s] = po[(size_t)sc * D + dim];
    }
    float M = NEG;
#pragma unroll
    for (int s = 0; s < kR; ++s)
      if (s < ns) M = fmaxf(M, mv[s]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int s = 0; s < kR; ++s)
      if (s < ns) {
        const float w = (mv[s] == NEG || M == NEG) ? 0.f : __builtin_amdgcn_exp2f(mv[s] - M);
        L += w * lv[s];
        O += w * pv[s];
      }
    if (tid < D) store_x((XT *)a.out, (size_t)row * a.ldo + head * D + tid, L > 0.f ? O / L : 0.f);
    return;
  }
  __shared__ float sw[64];
  __shared__ float s_L;
  const float ms = tid < ns ? ml[2 * tid] : NEG;
  float M = ms;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));  // wave 0 holds all splits
  if (tid < 64) sw[tid] = (tid < ns && ms != NEG && M != NEG) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
  __syncthreads();
  if (tid == 0) {
    float L = 0.f;
    for (int s = 0; s < ns; ++s) L += sw[s] * ml[2 * s + 1];
    s_L = L;
  }
  __syncthreads();
  const float L = s_L;
  for (int dim = tid; dim < D; dim += blockDim.x) {
    float O = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) O += sw[s] * po[(size_t)s * D + dim];
    store_x((XT *)a.out, (size_t)row * a.ldo + head * D + dim, L > 0.f ? O / L : 0.f);
  }
}

template <typename T, int D>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t s) {
  const int G = a.q_heads / a.kvl.kv_heads;
  const int nqt = (a.q_tile * G + 15) / 16;
  const int ntile = (a.q_len + a.q_tile - 1) / a.q_tile;
  dim3 grid(a.n_seq * a.kvl.kv_heads * ntile, a.n_splits), block(256);
  if (a.raw) {
    switch (nqt) {
      case 1: hipLaunchKernelGGL((attn_kernel<T, D, 1, true>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((attn_kernel<T, D, 2, true>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((attn_kernel<T, D, 3, true>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((attn_kernel<T, D, 4, true>), grid, block, 0, s, a); break;
    }
  } else {
    switch (nqt) {
      case 1: hipLaunchKernelGGL((attn_kernel<T, D, 1, false>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((attn_kernel<T, D, 2, false>), grid, block, 0, s, a); break;
      case 3: hipLaunchKernelGGL((attn_kernel<T, D, 3, false>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((attn_kernel<T, D, 4, false>), grid, block, 0, s, a); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1 || a.counters) return e;
  const int n_rows = a.n_seq * a.q_len;
  hipLaunchKernelGGL((attn_merge_kernel<T>), dim3(n_rows * a.q_heads), dim3(128), 0, s, a, n_rows);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int dtype, hipStream_t s) {
  const int D = a.kvl.head_dim;
  if (dtype == 0) {  // bf16 models: fp16 q and KV cache
    if (D == 128) return launch_attn_t<f16, 128>(a, s);
    if (D == 64) return launch_attn_t<f16, 64>(a, s);
    if (D == 32) return launch_attn_t<f16, 32>(a, s);
  } else {
    if (D == 128) return launch_attn_t<float, 128>(a, s);
    if (D == 64) return launch_attn_t<float, 64>(a, s);
    if (D == 32) return launch_attn_t<float, 32>(a, s);
  }
  return hipErrorInvalidValue;
}


// ------------------------------------------------------------------ prefill attention (flash-style)
// Causal attention of long query blocks (prefill) for bf16 models (fp16 q and KV cache), head_dim 128,
// 16-token pages.  One work-group per (block of 128 query rows, query head, sequence), heaviest blocks
// first, XCD by XCD per KV head; each of its 4 waves owns 32 rows (two 16-row MFMA tiles) outright, so
// no partial results cross waves.  Keys run in blocks of 64 (4 pages): the block's K ([key][dim]) and
// V^T ([dim][key]) are staged in swizzled, double-buffered LDS by the whole work-group, the next block's
// loads in registers while the current one is multiplied (one barrier per block); each thread stages 32
// bytes of each of the block's 4 pages, through buffer loads whose range is the page (empty for pages
// past the key range or without a block-table entry, whose reads return zeros).  Per block and wave:
// S^T = K Q^T (v_mfma 16x16x32, q held in registers), then an online softmax per query row in log2 units, then
// O^T += V^T P^T (v_mfma 16x16x32) with P^T taken from the S^T accumulators as they lie, all in fp32 with
// fp16 operands.  Only the blocks that reach past a wave's first query position are masked (key
// position > query position).  The running maximum of a row moves only when a block's maximum exceeds
// it by more than kPfLazy (log2 units): the probabilities then stay below 2^kPfLazy, the rescaling of
// the accumulators is skipped for most blocks, and o / l is unchanged up to rounding.  The sequence's
// block-table entries for its key range sit in LDS.  The waves raise their priority over their product
// sections (s_setprio), so that of the two waves sharing a SIMD the one with products ready issues them
// while the other works through its softmax.
constexpr int kPfBq = 128, kPfBk = 64, kPfMaxPages = 1024;
constexpr float kPfLazy = 8.f;
// LDS layouts.  The S^T tile kt of a 64-key block holds keys kidx(kt, i) (row i), chosen so that tiles
// 2 kk and 2 kk + 1 together give lane group g the 8 consecutive keys 32 kk + 8 g .. + 7: then the P^T
// operand of the PV product is the two tiles' accumulators as they lie, and its V^T operand is one 16-byte
// piece of a V^T row in key order (8 tokens of one page).  K rows (256 bytes, one per key) keep chunk c
// at c ^ ksw(key), where ksw(kidx(kt, i)) = i; V^T rows (128 bytes, one per dim) keep chunk c at
// c ^ (dim % 8).  Both fragment reads then run at the full LDS rate on gfx950 (measured: 4 cycles per
// 16-byte wave read; the swizzle (r % 8) ^ ((r / 8) % 2) on 128-byte rows takes twice that).
DF_DEVICE int pf_kidx(int kt, int i) { return 32 * (kt >> 1) + 8 * (i >> 2) + 4 * (kt & 1) + (i & 3); }
DF_DEVICE int pf_ksw(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }

__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(AttnArgs a) {
  constexpr int D = 128, PT = 16;
  constexpr int KS = D / 32;       // QK^T steps of 32 dims
  constexpr int DT = D / 16;       // 16-dim output tiles
  constexpr int KROW = D * 2;      // LDS bytes per K row: 16 16-byte chunks, chunk c at c ^ pf_ksw(key)
  constexpr int VROW = kPfBk * 2;  // LDS bytes per V^T row: 8 chunks, chunk c at c ^ (dim % 8)
  __shared__ __attribute__((aligned(16))) unsigned char sK[2][kPfBk * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char sV[2][D * VROW];
  __shared__ __attribute__((aligned(16))) int s_bt[kPfMaxPages + 8];
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  // Work-group order: heaviest query blocks (the longest key ranges) first.  Work-groups go to the 8 XCDs
  // round-robin (L mod 8); when the (sequence, KV head) units divide evenly, each XCD takes whole units,
  // so that a unit's K/V stays in one XCD's L2 for all its query heads and blocks.
  const int nqb = (a.q_len + kPfBq - 1) / kPfBq;
  const int kvh = a.kvl.kv_heads, G = a.q_heads / kvh, U = a.n_seq * kvh;
  const int L = blockIdx.x;
  int qb_rev, unit, gq;
  if (U % 8 == 0) {
    const int j = L >> 3, per = (U >> 3) * G;
    qb_rev = j / per;
    unit = (L & 7) + 8 * ((j % per) / G);
    gq = (j % per) % G;
  } else {
    const int per = U * G;
    qb_rev = L / per;
    unit = (L % per) / G;
    gq = (L % per) % G;
  }
  const int qb = nqb - 1 - qb_rev, b = unit / kvh, kh = unit % kvh, head = kh * G + gq;
  const int row0 = b * a.q_len;                    // the sequence's first row
  const int rlast = min(a.q_len, (qb + 1) * kPfBq) - 1;
  const int kmax = a.rows.pos[row0 + rlast];       // the work-group's last key position (rows are in order)
  const int nkb = kmax >= 0 ? kmax / kPfBk + 1 : 0;
  const int npg = nkb * (kPfBk / PT);
  if (npg > kPfMaxPages) {  // a position past what the host sized the call for (uniform exit)
    if (tid == 0) raise_err(a.err, ERR_PAGE);
    return;
  }
  const int32_t *bt = a.block_table + (size_t)a.seq_slot[b] * a.bt_stride;
  for (int i = tid; i < npg + 8; i += 256) s_bt[i] = i < npg && i < a.bt_stride ? bt[i] : -1;  // + 2 blocks past

  // this wave's query rows: tile t holds rows rw + 16 t + l16 (B operand: dims 8 g .. 8 g + 7 of each step)
  const int rw = qb * kPfBq + wave * 32;
  u32x4 q[2][KS];
  int qpos[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r = rw + 16 * t + l16;
    const bool ok = r < a.q_len;
    qpos[t] = ok ? a.rows.pos[row0 + r] : -1;
    const f16 *qr = (const f16 *)a.q + (size_t)(row0 + (ok ? r : 0)) * a.ldq + head * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[t][ks] = *reinterpret_cast<const u32x4 *>(qr + ks * 32 + g * 8);
  }
  // blocks whose last key is at or below the wave's first query position need no mask
  const int first_pos = __builtin_amdgcn_readfirstlane(qpos[0]);
  __syncthreads();  // s_bt

  // Staging from page i of the block (one buffer resource per page; a page past the key range or without
  // a block-table entry has an empty range, and its reads return zeros): thread tid loads K token tid / 16,
  // dims 8 (tid % 16) .. and V^T dim tid / 2, tokens 8 (tid % 2) .. (16 bytes each).
  const uint32_t page_bytes = (uint32_t)a.kvl.page_elems() * 2;
  const uint32_t k_off = ((uint32_t)kh * PT * D + (tid >> 4) * D + (tid & 15) * 8) * 2;
  const uint32_t v_off = ((uint32_t)(a.kvl.kv_heads + kh) * PT * D + (tid >> 1) * PT + (tid & 1) * 8) * 2;
  u32x4 rk[4], rv[4];
  auto load = [&](int4 pgs) {  // the block's 4 block-table entries
    const int pg[4] = {pgs.x, pgs.y, pgs.z, pgs.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = __builtin_amdgcn_readfirstlane(pg[i]);
      const char *base = (const char *)a.kv + (size_t)(e >= 0 ? e : 0) * page_bytes;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, e >= 0 ? (int)page_bytes : 0,
                                                                        0x00020000);
      rk[i] = __builtin_amdgcn_raw_buffer_load_b128(r, k_off, 0, 0);
      rv[i] = __builtin_amdgcn_raw_buffer_load_b128(r, v_off, 0, 0);
    }
  };
  int kst[4], vst[4];  // LDS byte offsets of the thread's pieces of page i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = 16 * i + (tid >> 4), d = tid >> 1;
    kst[i] = key * KROW + (((tid & 15) ^ pf_ksw(key)) << 4);
    vst[i] = d * VROW + (((2 * i + (tid & 1)) ^ (d & 7)) << 4);
  }
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<u32x4 *>(&sK[buf][kst[i]]) = rk[i];
      *reinterpret_cast<u32x4 *>(&sV[buf][vst[i]]) = rv[i];
    }
  };
  // a needed page (one holding a key at or below kmax) without a block-table entry is an error
  int err = 0;
  for (int i = tid; i <= kmax / PT && i < npg; i += 256) err |= s_bt[i] < 0;

  const float scale = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(D)
  const float NEG = -INFINITY;
  float m[2] = {NEG, NEG}, l[2] = {0.f, 0.f};  // running maximum (log2 units) and sum per query row
  float mb[2] = {0.f, 0.f};                     // m, or 0 while a row has seen no key
  f32x4 o[2][DT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto entries = [&](int kb) { return *reinterpret_cast<const int4 *>(&s_bt[kb * 4]); };
  load(entries(0));
  store(0);
  load(entries(1));
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int4 next = entries(kb + 2);  // read early: the loads at the end of the block use them
    const unsigned char *K = sK[buf], *V = sV[buf];
    // S^T[key pf_kidx(kt, 4 g + r)][query l16] of both query tiles
    __builtin_amdgcn_s_setprio(1);  // products first while both waves of the SIMD are ready
    // (dims step outermost: the 8 accumulators take turns, so no product waits on the one before it)
    f32x4 s[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[t][kt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        kf[kt] = *reinterpret_cast<const u32x4 *>(K + pf_kidx(kt, l16) * KROW + (((ks * 4 + g) ^ l16) << 4));
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          s[t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, kf[kt]), __builtin_bit_cast(h8, q[t][ks]),
                                                           s[t][kt], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    // mask (blocks reaching past the wave's first query position only) and each row's block maximum
    // (the row's 64 scores sit in the 4 lanes l16, l16 + 16, + 32, + 48)
    if (kb * kPfBk + kPfBk - 1 > first_pos) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kb * kPfBk + pf_kidx(kt, 4 * g + r) > qpos[t]) s[t][kt][r] = NEG;
    }
    // The grow test needs only each lane's own maximum (the row's maximum exceeds m + kPfLazy iff one of
    // its 4 lanes' does); the row's maximum itself is gathered only when some row of the wave grows.
    float mx[2];
    bool grow = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float v = NEG;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) v = __builtin_elementwise_max(v, s[t][kt][r]);
      mx[t] = v * scale;
      grow |= mx[t] > m[t] + kPfLazy;
    }
    if (__builtin_amdgcn_ballot_w64(grow)) {  // some row's maximum moves: rescale (wave-uniform branch)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float v = mx[t];
        v = __builtin_elementwise_max(v, __shfl_xor(v, 16));
        v = __builtin_elementwise_max(v, __shfl_xor(v, 32));
        const float mn = v > m[t] + kPfLazy ? v : m[t];
        const float corr = __builtin_amdgcn_exp2f(m[t] - mn);  // 0 for a row's first keys, 1 if unmoved
        m[t] = mn;
        mb[t] = mn == NEG ? 0.f : mn;  // a row with no key yet: every score is -inf
        l[t] *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] *= corr;
      }
    }
    h4 pf[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[t][kt][r], scale, -mb[t]));
          ps += p;
          pf[t][kt][r] = (_Float16)p;
        }
      l[t] += ps;
    }
    // O^T[dim 16 dt + 4 g + r][query l16] += V^T P^T over 32-key groups kk with 16x16x32 products: the
    // B operand of lane (query l16, g) is P^T of keys 32 kk + 8 g .. + 7, the accumulators of tiles 2 kk
    // and 2 kk + 1 as they lie; the A operand of lane (dim l16, g) is V^T of the same keys, chunk 4 kk + g
    // of the dim's row.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vf[dt] = *reinterpret_cast<const u32x4 *>(V + (16 * dt + l16) * VROW + (((4 * kk + g) ^ (l16 & 7)) << 4));
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const h8 pb = __builtin_shufflevector(pf[t][2 * kk], pf[t][2 * kk + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, vf[dt]), pb, o[t][dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (kb + 1 < nkb) store(buf ^ 1);
    load(next);  // past the key range: empty ranges, zeros, never used
    __syncthreads();
  }
  // normalise and store: lane holds dims 16 dt + 4 g + r of query row rw + 16 t + l16
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int r = rw + 16 * t + l16;
    if (r >= a.q_len) continue;
    f16 *out = (f16 *)a.out + (size_t)(row0 + r) * a.ldo + head * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Elem<f16>::store(out + 16 * dt + 4 * g + i, o[t][dt][i] * inv);
  }
  err = __any(err);
  if (err && lane == 0) raise_err(a.err, ERR_PAGE);
}

// Prefill attention through attn_prefill_kernel: causal calls of fp16 models at head_dim 128 with
// 16-token pages and at most kPfMaxPages pages of keys.
bool attn_prefill_fits(const AttnArgs &a, int dtype, int max_key_pos) {
  return dtype == 0 && a.mode == 0 && a.raw == nullptr && a.kvl.head_dim == 128 && a.kvl.page_tokens == 16 &&
         a.n_seq >= 1 && a.n_seq <= 64 && max_key_pos / kPfBk + 1 <= kPfMaxPages / (kPfBk / 16) &&
         a.q_heads % a.kvl.kv_heads == 0 && a.ldq % 8 == 0;
}

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t s) {
  if (a.q_len < 1) return hipSuccess;
  const dim3 grid((a.q_len + kPfBq - 1) / kPfBq * a.q_heads * a.n_seq);
  hipLaunchKernelGGL(attn_prefill_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace df
