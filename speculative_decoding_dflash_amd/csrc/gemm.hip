// Skinny GEMM Y[M, N] = X[M, K] W[N, K]^T on MFMA (gfx950), with fused column-local epilogues.
//
// The decode step is weight-streaming: M (block x batch rows) is small, so every weight byte is read
// once from HBM and the matrix cores are far from busy.  The kernel is shaped for that:
//   * a work-group owns 16 or 32 weight rows (one or two 16-row MFMA column tiles) over the whole K;
//     its NW waves take interleaved 256-byte K windows ("super-steps");
//   * weights are loaded in a layout that HBM streams well -- one wave instruction covers 4 rows x
//     256 contiguous bytes (16 bytes per lane) -- while the next super-step is already in flight;
//     each wave stages its rows in a private, padded LDS tile and reads the MFMA operand layout
//     (16 rows x 64 bytes per instruction, which streams ~25% slower from HBM) back from LDS;
//     a wave only ever reads what it wrote itself, so the main loop needs no barrier;
//   * X windows take the same path (quad-layout loads, wave-private LDS), which costs a few percent
//     where loading X directly in the MFMA layout cost a quarter of the bandwidth;
//   * bf16 models: X is fp16 and the weights are converted to fp16 (exactly) as they are staged, then
//     v_mfma_f32_16x16x32_f16 accumulates in fp32 (fp32 models: 4 x v_mfma_f32_16x16x4f32);
//   * the NW waves reduce their partial tiles through LDS in a fixed order, then the whole
//     work-group runs the epilogue on its columns.  No state crosses work-groups, so no device-scope
//     fences (which write back and invalidate the per-XCD L2s) are needed anywhere;
//   * gemm_sk_kernel, a stream-K variant for decode-sized M, spreads the items of projections whose
//     tile count fits the CUs badly evenly over one work-group per CU; tiles shared by two or three
//     work-groups are finished by the last to arrive, through write-through partial stores and one
//     arrival counter per tile (again no fences).
// Epilogues: fp32 store (logits), activation store, fp32 partial store of one K range (grid row y;
// the consumer sums the ranges in order: residual add + RMSNorm, q/k/v post-processing), and SwiGLU
// (gate and up rows of the same output column in one work-group).
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "kernels.h"

namespace df {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// MFMA operands per weight type: bf16 models multiply fp16 X (ActOf<bf16>) with their weights converted
// to fp16 as they are staged (w(): exact, see bf16x2_to_f16x2) on v_mfma_f32_16x16x32_f16; fp32 models
// use v_mfma_f32_16x16x4f32.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
  static constexpr int kEPL = 8;   // elements per lane per K step
  static constexpr int kStep = 32; // K per step
  static DF_DEVICE u32x4 w(u32x4 v) {
    return (u32x4){bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
  }
  static DF_DEVICE void mma(f32x4 &acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0,
                                                 0);
  }
};
template <> struct Frag<float> {
  static constexpr int kEPL = 4;
  static constexpr int kStep = 16;
  static DF_DEVICE u32x4 w(u32x4 v) { return v; }
  // Element j of every lane's 4-vector forms one K=4 slice (k = 4*(lane/16) + j), identically for A and B.
  static DF_DEVICE void mma(f32x4 &acc, u32x4 a, u32x4 b) {
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(af[j], bf[j], acc, 0, 0, 0);
  }
};

template <typename T> DF_DEVICE u32x4 ld16(const T *p) { return *reinterpret_cast<const u32x4 *>(p); }

// The X row that local row m (< M) reads: m itself, or with a row selection the selected row of global
// row row_off + m.
DF_DEVICE int x_src(const GemmArgs &a, int m) {
  if (!a.x_take) return m;
  const int r = a.row_off + m;
  return (r / a.x_take) * a.x_stride + a.x_off + r % a.x_take;
}

// Row v (< M) of the X operand.
template <typename T> DF_DEVICE const T *x_row(const GemmArgs &a, int v) { return (const T *)a.x + (size_t)x_src(a, v) * a.ldx; }

DF_DEVICE float silu(float g) { return g / (1.0f + expf(-g)); }

// Prefetch of the deferred RMSNorm's partial sums of squares: those of X row m sit at
// ss_in[(row_off + m) * ss_ld + p] (p < ss_n, ss_ld a multiple of 4).  Thread t loads the 4-vectors
// t + k * NT, k < kSS4, unconditionally (surplus loads read the first vector again) before the weight
// stream starts, and stores their sums to s_ssp[t + k * NT] once they are needed.  Beyond kSS4 * NT
// vectors the rows' sums are read from memory in the epilogue instead.
constexpr int kSS4 = 4;
template <int NT>
struct SsPrefetch {
  float4 v[kSS4];
  bool fast;
  DF_DEVICE void load(const GemmArgs &a) {
    const int ss_q = a.ss_ld / 4;  // 4-vectors per row
    fast = a.ss_in && a.M * ss_q <= kSS4 * NT;
    if (!fast) return;
    const float4 *base = reinterpret_cast<const float4 *>(a.ss_in + (size_t)a.row_off * a.ss_ld);
#pragma unroll
    for (int k = 0; k < kSS4; ++k) {
      const int idx = threadIdx.x + k * NT;
      v[k] = base[idx < a.M * ss_q ? idx : 0];
    }
  }
  DF_DEVICE void store(const GemmArgs &a, float *s_ssp) const {
    if (!fast) return;
    const int ss_q = a.ss_ld / 4;
#pragma unroll
    for (int k = 0; k < kSS4; ++k) {
      const int idx = threadIdx.x + k * NT;
      if (idx < a.M * ss_q) {
        const int p0 = (idx % ss_q) * 4;  // partials p0 .. p0 + 3 of row idx / ss_q
        s_ssp[idx] = (p0 < a.ss_n ? v[k].x : 0.f) + (p0 + 1 < a.ss_n ? v[k].y : 0.f) + (p0 + 2 < a.ss_n ? v[k].z : 0.f) +
                     (p0 + 3 < a.ss_n ? v[k].w : 0.f);
      }
    }
  }
};

// 1 / rms of X row m of the deferred RMSNorm: the row's ss_n partial sums of squares added in a fixed
// order (4-vector sums first, as prefetched into s_ssp, else read from memory the same way).
DF_DEVICE float gemm_rstd(const GemmArgs &a, int m, bool ss_fast, const float *s_ssp) {
  float tot = 0.f;
  if (ss_fast) {
    const int nq = (a.ss_n + 3) / 4;
    for (int i = 0; i < nq; ++i) tot += s_ssp[m * (a.ss_ld / 4) + i];
  } else {
    for (int pp = 0; pp < a.ss_n; pp += 4) {
      const float *q = a.ss_in + (size_t)(a.row_off + m) * a.ss_ld + pp;
      tot += (q[0] + (pp + 1 < a.ss_n ? q[1] : 0.f)) + (pp + 2 < a.ss_n ? q[2] : 0.f) + (pp + 3 < a.ss_n ? q[3] : 0.f);
    }
  }
  return 1.0f / sqrtf(tot / (float)a.norm_dim + a.eps);
}

// Epilogue of output tile c (K range `split`): lds[m * COLS + j] holds the tile's sums for rows m < M.
// Every thread of the work-group calls it (EPI_RESID_NORM synchronises the work-group).
template <typename T, int COLS, int NT>
DF_DEVICE void gemm_epilogue(const GemmArgs &a, int c, int split, float *lds, const float *s_rstd) {
  const int tid = threadIdx.x;
  const int M = a.M;
  const bool rs = a.ss_in != nullptr;
  switch (a.epi) {
    case EPI_STORE_F32:
      for (int e = tid; e < M * COLS; e += NT) {
        const int m = e / COLS, j = e % COLS;
        a.out_f32[(size_t)(a.row_off + m) * a.ld_out + COLS * c + j] = lds[m * COLS + j] * (rs ? s_rstd[m] : 1.f);
      }
      break;
    case EPI_PARTIAL: {
      float *o = a.out_f32 + (size_t)split * a.part_stride;
      for (int e = tid; e < M * COLS; e += NT) {
        const int m = e / COLS, j = e % COLS;
        o[(size_t)(a.row_off + m) * a.ld_out + COLS * c + j] = lds[m * COLS + j] * (rs ? s_rstd[m] : 1.f);
      }
      break;
    }
    case EPI_SWIGLU: {
      constexpr int HC = COLS / 2;  // output columns of the tile: gate in [0, HC), up in [HC, COLS)
      for (int e = tid; e < M * HC; e += NT) {
        const int m = e / HC, j = e % HC;
        const float r = rs ? s_rstd[m] : 1.f;
        const float gt = lds[m * COLS + j] * r, up = lds[m * COLS + HC + j] * r;
        store_x((ActOf<T> *)a.out_act, (size_t)(a.row_off + m) * a.ld_out + HC * c + j, silu(gt) * up);
      }
      break;
    }
    case EPI_RESID_NORM:
      if constexpr (COLS % 32 == 0) {
        for (int e = tid; e < M * COLS; e += NT) {
          const int m = e / COLS, j = e % COLS;
          const int r = a.row_off + m, n = COLS * c + j;
          float v = lds[m * COLS + j];
          if (a.resid) {
            const size_t idx = (size_t)r * a.ld_resid + n;
            v += a.resid[idx];
            a.resid[idx] = v;
          }
          if (a.feat) store_x((ActOf<T> *)a.feat, (size_t)r * a.ld_feat + n, v);
          const int jj = r % a.sel_stride - a.sel_offset;
          if (jj >= 0 && jj < a.sel_take)
            store_x((ActOf<T> *)a.xg, (size_t)((r / a.sel_stride) * a.sel_take + jj) * a.ld_xg + n, v * a.gain[n]);
          lds[m * COLS + j] = v * v;  // entry owned by this thread
        }
        __syncthreads();
        // one sum of squares per row and 32-column group (the tile's groups are COLS / 32 .. + COLS / 32 - 1)
        constexpr int NG = COLS / 32;
        if (tid < M * NG) {
          const int m = tid / NG, h = tid % NG;
          const int r = a.row_off + m, jj = r % a.sel_stride - a.sel_offset;
          if (jj >= 0 && jj < a.sel_take) {
            float t = 0.f;
            for (int j = 0; j < 32; ++j) t += lds[m * COLS + 32 * h + j];
            a.ss_out[(size_t)((r / a.sel_stride) * a.sel_take + jj) * a.ss_out_ld + NG * c + h] = t;
          }
        }
      }
      break;
  }
}

template <typename T, int MT, int CT, int NW, int PD, int XR>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GemmArgs a) {
  using F = Frag<T>;
  constexpr int COLS = 16 * CT;
  // XR: X operand rows staged per super-step (8 when there are at most 8, else padded to whole MFMA
  // tiles, 16 * MT)
  static_assert(XR == 16 * MT || (MT == 1 && XR == 8), "X staging rows");
  constexpr int NT = NW * 64;
  constexpr int ROWB = 256 + 16;           // LDS bytes per staged row (256 B of K plus padding)
  constexpr int NQ = COLS / 4;             // weight quad loads per super-step (4 rows x 256 B each)
  constexpr int NXQ = XR / 4;              // X quad loads per super-step (rows >= M skipped)
  constexpr int SK = 256 / sizeof(T);      // K elements per super-step (256 bytes of a row)
  constexpr int KS = SK / F::kStep;        // MFMA K steps per super-step (4)
  constexpr int kEnt = 16 * MT * COLS;     // entries of one wave's partial tile
  constexpr int kTileB = NW * (COLS + XR) * ROWB, kRedB = NW * kEnt * 4;
  // wave-private staging of weights and X during the main loop; the cross-wave reduction reuses it
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTileB > kRedB ? kTileB : kRedB];
  __shared__ float s_ssp[4 * NT], s_rstd[16 * MT];
  float *lds = reinterpret_cast<float *>(smem);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const bool swiglu = a.epi == EPI_SWIGLU;
  const int c = blockIdx.x;
  const int split = blockIdx.y;
  const int Kc = a.K / a.ksplit;  // this work-group's K range: [split * Kc, (split + 1) * Kc)
  const int k0 = split * Kc;

  const T *wbase[CT];  // row 16*ct of the tile
  if (swiglu) {  // CT == 2: a gate tile and an up tile of 16 rows each (CT == 1: see below)
    wbase[0] = (const T *)a.seg[0].w + (size_t)(16 * c) * a.K;
    wbase[CT - 1] = (const T *)a.seg[1].w + (size_t)(16 * c) * a.K;
  } else {
    const int r0 = COLS * c;
    int si = 0, base = 0;
    while (si + 1 < a.nseg && r0 >= base + a.seg[si].n) {
      base += a.seg[si].n;
      ++si;
    }
    const T *w = (const T *)a.seg[si].w;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) wbase[ct] = w + (size_t)(r0 - base + 16 * ct) * a.K;
  }
  // Quad layout: load q covers rows 4q .. 4q+3, lane (g = lane / 16) takes row 4q + g and bytes
  // 16 * r16 .. 16 * r16 + 15 of the 256-byte window.
  const T *qrow[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) qrow[q] = wbase[q / 4] + (size_t)(4 * (q % 4) + g) * a.K + k0 + r16 * F::kEPL;
  if constexpr (CT == 1) {
    if (swiglu) {  // one 16-column tile: gate rows 8c .. 8c + 7 (quads 0, 1), up rows 8c .. 8c + 7 (quads 2, 3)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        qrow[q] = (const T *)a.seg[q / 2].w + (size_t)(8 * c + 4 * (q % 2) + g) * a.K + k0 + r16 * F::kEPL;
    }
  }
  // X rows: rows >= M load row 0 (never read back: the operand read below masks them), so that every load
  // in the streaming loop is unconditional and the compiler can count outstanding loads exactly.
  const int Mv = a.M;
  const T *xrow[NXQ];
#pragma unroll
  for (int q = 0; q < NXQ; ++q) {
    const int m = 4 * q + g;
    xrow[q] = x_row<T>(a, m < Mv ? m : 0) + k0 + r16 * F::kEPL;
  }

  f32x4 acc[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  unsigned char *wt = smem + wave * (COLS + XR) * ROWB;
  unsigned char *xt = wt + COLS * ROWB;
  const int nsup = Kc / SK;  // streamed super-steps; wave w takes w, w + NW, ...
  // Deferred RMSNorm of the X rows: their partial sums of squares are loaded before the weight stream.
  SsPrefetch<NT> ssp;
  ssp.load(a);

  // PD register buffers per wave: PD super-steps are in flight while one is consumed.  Loads past the
  // wave's last super-step are redirected to X's first 256 bytes (cache-resident, never consumed),
  // which keeps them unconditional.
  const T *dummy = (const T *)a.x + r16 * F::kEPL;
  u32x4 buf[PD][NQ], bufx[PD][NXQ];
  if (nsup > 0) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int s0 = wave + p * NW;
      const bool ok = s0 < nsup;
#pragma unroll
      for (int q = 0; q < NQ; ++q) buf[p][q] = ld16(ok ? qrow[q] + (size_t)s0 * SK : dummy);
#pragma unroll
      for (int q = 0; q < NXQ; ++q) bufx[p][q] = ld16(ok ? xrow[q] + (size_t)s0 * SK : dummy);
      __builtin_amdgcn_sched_barrier(0);  // keep buffer p's loads ahead of buffer p + 1's
    }
  }
  ssp.store(a, s_ssp);
  for (int sup = wave; sup < nsup; sup += PD * NW) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int cs = sup + p * NW;
      if (cs < nsup) {  // wave-uniform
#pragma unroll
        for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4 *>(wt + (4 * q + g) * ROWB + 16 * r16) = F::w(buf[p][q]);
#pragma unroll
        for (int q = 0; q < NXQ; ++q) *reinterpret_cast<u32x4 *>(xt + (4 * q + g) * ROWB + 16 * r16) = bufx[p][q];
      }
      const int nxt = cs + PD * NW;
      const bool ok = nxt < nsup;
#pragma unroll
      for (int q = 0; q < NQ; ++q) buf[p][q] = ld16(ok ? qrow[q] + (size_t)nxt * SK : dummy);
#pragma unroll
      for (int q = 0; q < NXQ; ++q) bufx[p][q] = ld16(ok ? xrow[q] + (size_t)nxt * SK : dummy);
      if (cs < nsup) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 xv[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            xv[mt] = (mt * 16 + r16 < Mv)
                         ? *reinterpret_cast<const u32x4 *>(xt + (mt * 16 + (r16 < XR ? r16 : 0)) * ROWB + ks * 64 + 16 * g)
                         : zero;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const u32x4 wv = *reinterpret_cast<const u32x4 *>(wt + (16 * ct + r16) * ROWB + ks * 64 + 16 * g);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) F::mma(acc[mt][ct], xv[mt], wv);
          }
        }
      }
    }
  }
  // K tail (K not a multiple of the super-step): direct MFMA-layout loads
  for (int st = nsup * KS + wave; st < Kc / F::kStep; st += NW) {
    const int k = k0 + st * F::kStep + g * F::kEPL;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      const u32x4 xv = m < Mv ? ld16(x_row<T>(a, m) + k) : zero;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) F::mma(acc[mt][ct], xv, F::w(ld16(wbase[ct] + (size_t)r16 * a.K + k)));
    }
  }

  // Reduce the waves' partial tiles: C[m][n] sits at lane (n = lane % 16, m = 4 * (lane / 16) + r).
  __syncthreads();  // every wave is done with its staging tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) lds[wave * kEnt + (mt * 16 + g * 4 + r) * COLS + ct * 16 + r16] = acc[mt][ct][r];
  __syncthreads();
  // output row m < M: the waves' sums
  for (int e = tid; e < a.M * COLS; e += NT) {
    float v = lds[e];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += lds[w * kEnt + e];
    lds[e] = v;  // entry e < M * COLS is read and written by this thread only
  }
  if (a.ss_in && tid < a.M) s_rstd[tid] = gemm_rstd(a, tid, ssp.fast, s_ssp);
  __syncthreads();
  gemm_epilogue<T, COLS, NT>(a, c, split, lds, s_rstd);
}

// Stream-K variant (ksplit 1, K a whole number of super-steps, 8 waves, at most 16 X rows, 32 output
// columns per work item).
// With one tile per work-group, projections whose tile count is not a multiple of the CU count leave
// CUs idle while others stream (160 hidden-width tiles on 256 CUs).  Here the projection's items
// (tile, super-step), numbered tile-major, are cut into equal contiguous ranges, one per work-group
// and one work-group per CU.  A work-group walks its range tile by tile; its waves take interleaved
// items and their register prefetch runs on across tile boundaries.  At the end of each tile the waves'
// partial tiles are reduced through LDS.  A tile covered by one work-group gets its epilogue at once;
// a tile shared by several (only a range's first and last tile can be) is finished by whichever
// arrives last: the others write their partial tile through to memory (the finisher may sit on
// another XCD) and count their arrival on the tile's counter; the finisher adds the partials in
// work-group order -- a fixed order, so the result does not depend on who arrives last -- runs the
// epilogue and zeroes the counter for the next launch.  No work-group ever waits for another.
template <typename T, int XR>
__global__ __launch_bounds__(512) void gemm_sk_kernel(GemmArgs a, int per) {
  using F = Frag<T>;
  constexpr int NW = 8, NT = NW * 64;
  constexpr int COLS = 32, CT = COLS / 16, ROWS = 16;
  static_assert(XR == 8 || XR == 16, "X staging rows");
  constexpr int ROWB = 256 + 16;
  constexpr int NQ = COLS / 4, NXQ = XR / 4;
  constexpr int SK = 256 / sizeof(T);
  constexpr int KS = SK / F::kStep;
  constexpr int kEnt = ROWS * COLS;  // entries of one partial tile
  static_assert(kEnt <= kSkTileElems, "partial tile size");
  constexpr int kPer = (kEnt + NT - 1) / NT;
  constexpr int kTileB = NW * (32 + XR) * ROWB, kRedB = 2 * NW * kEnt * 4;
  // staging tiles (wave-private), then two reduction buffers (alternating tiles), then the tile sums
  __shared__ __attribute__((aligned(16))) unsigned char smem[kTileB + kRedB + kEnt * 4];
  __shared__ float s_ssp[kSS4 * NT], s_rstd[16];
  __shared__ int s_last;
  float *red = reinterpret_cast<float *>(smem + kTileB);
  float *fin = red + 2 * NW * kEnt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const bool swiglu = a.epi == EPI_SWIGLU;
  const int ntile = swiglu ? a.N / (COLS / 2) : a.N / COLS;
  const int nsup = a.K / SK, items = ntile * nsup;
  const int p = blockIdx.x;
  const int lo = p * per, hi = min(items, lo + per);

  // weight rows of tile t, as CT groups of 16 rows (accumulator ct = group ct): SWIGLU takes COLS / 2
  // gate rows (groups 0 .. CT/2-1) and the same up rows (groups CT/2 ..); otherwise COLS consecutive
  // rows of the concatenated segments (each segment a whole number of tiles)
  // (w0: groups 0 .. CT/2-1, w1: groups CT/2 .., each a run of COLS / 2 rows)
  // the first three segments' bases are held from the start: the cursor reaches a new tile every few
  // items, and a table read there (a vector load, as the wave index is not known to be uniform) would
  // wait for every weight load in flight
  const T *const sw0 = (const T *)a.seg[0].w, *const sw1 = (const T *)a.seg[1].w, *const sw2 = (const T *)a.seg[2].w;
  const int sn0 = a.seg[0].n, sn1 = a.seg[1].n;
  auto tile_base = [&](int t, const T *&w0, const T *&w1) {
    if (swiglu) {
      w0 = sw0 + (size_t)((COLS / 2) * t) * a.K;
      w1 = sw1 + (size_t)((COLS / 2) * t) * a.K;
      return;
    }
    if (a.nseg <= 3) {  // one segment, or q / k / v
      int r0 = COLS * t;
      const T *w = sw0;
      if (a.nseg > 1 && r0 >= sn0) {
        r0 -= sn0;
        w = sw1;
        if (a.nseg > 2 && r0 >= sn1) {
          r0 -= sn1;
          w = sw2;
        }
      }
      w0 = w + (size_t)r0 * a.K;
      w1 = w0 + (size_t)(COLS / 2) * a.K;
      return;
    }
    int r0 = COLS * t, si = 0;
    while (si + 1 < a.nseg && r0 >= a.seg[si].n) {
      r0 -= a.seg[si].n;
      ++si;
    }
    w0 = (const T *)a.seg[si].w + (size_t)r0 * a.K;
    w1 = w0 + (size_t)(COLS / 2) * a.K;
  };
  const size_t gstep = (size_t)16 * a.K;  // elements between consecutive 16-row groups of a run
  // quad layout as in gemm_kernel: quad q covers rows 4 (q % 4) .. + 3 of group q / 4
  size_t qoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) qoff[q] = (size_t)(4 * q + g) * a.K + r16 * F::kEPL;
  // X staging rows 0 .. XR-1 (rows >= M read row 0; their products are never read back)
  const T *xrow[NXQ];
#pragma unroll
  for (int q = 0; q < NXQ; ++q) {
    const int m = 4 * q + g;
    xrow[q] = (const T *)a.x + (size_t)x_src(a, m < a.M ? m : 0) * a.ldx + r16 * F::kEPL;
  }
  SsPrefetch<NT> ssp;
  ssp.load(a);

  unsigned char *wt = smem + wave * (32 + XR) * ROWB;
  unsigned char *xt = wt + 32 * ROWB;
  const T *dummy = (const T *)a.x + r16 * F::kEPL;
  // load cursor: item li = (tile lt, super-step ls); the use cursor ui trails it by one item
  int li = lo + wave;
  int lt = li / nsup, ls = li - lt * nsup;
  int ui = li;
  const T *w0, *w1;
  tile_base(lt < ntile ? lt : 0, w0, w1);
  u32x4 buf[NQ], bufx[NXQ];
  // loads of the item at the cursor: its weight quads and X rows
  auto issue = [&]() {
    const bool ok = li < hi;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int gi = q / 4;  // the quad's 16-row group
      const T *wq = (gi < CT / 2 ? w0 + (size_t)gi * gstep : w1 + (size_t)(gi - CT / 2) * gstep);
      buf[q] = ld16(ok ? wq + qoff[q % 4] + (size_t)ls * SK : dummy);
    }
#pragma unroll
    for (int q = 0; q < NXQ; ++q) bufx[q] = ld16(ok ? xrow[q] + (size_t)ls * SK : dummy);
  };
  auto advance = [&]() {
    li += NW;
    ls += NW;
    if (ls >= nsup) {
      while (ls >= nsup) {
        ls -= nsup;
        ++lt;
      }
      if (lt < ntile) tile_base(lt, w0, w1);
    }
  };
  issue();
  advance();
  ssp.store(a, s_ssp);
  __syncthreads();  // the rows' 1/rms before the stream (computed inside the tile loop, the kernel kept a stack frame)
  if (a.ss_in && tid < a.M) s_rstd[tid] = gemm_rstd(a, tid, ssp.fast, s_ssp);

  int seg = 0;
  for (int t = lo / nsup; t * nsup < hi; ++t, ++seg) {
    const int seg_hi = min(hi, (t + 1) * nsup);
    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (; ui < seg_hi; ui += NW) {
      // stage the item, then load the next one while it is multiplied
#pragma unroll
      for (int q = 0; q < NQ; ++q) *reinterpret_cast<u32x4 *>(wt + (4 * q + g) * ROWB + 16 * r16) = F::w(buf[q]);
#pragma unroll
      for (int q = 0; q < NXQ; ++q) *reinterpret_cast<u32x4 *>(xt + (4 * q + g) * ROWB + 16 * r16) = bufx[q];
      issue();
      advance();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 xv = r16 < a.M
                             ? *reinterpret_cast<const u32x4 *>(xt + (r16 < XR ? r16 : 0) * ROWB + ks * 64 + 16 * g)
                             : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const u32x4 wv = *reinterpret_cast<const u32x4 *>(wt + (16 * c2 + r16) * ROWB + ks * 64 + 16 * g);
          F::mma(acc[c2], xv, wv);
        }
      }
    }
    // C[m][n] of a wave's partial tile sits at lane (n % 16, 4 * (lane / 16) + r) of acc[n / 16]
    float *rb = red + (seg & 1) * NW * kEnt;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[wave * kEnt + (g * 4 + r) * COLS + ct * 16 + r16] = acc[ct][r];
    __syncthreads();
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * NT;
      v[i] = 0.f;
      if (e < a.M * COLS)
        for (int w = 0; w < NW; ++w) v[i] += rb[w * kEnt + e];
    }
    if (t * nsup < lo || (t + 1) * nsup > hi) {  // shared tile
      const int q0 = (t * nsup) / per, q1 = ((t + 1) * nsup - 1) / per;
      const int slot = t * nsup < lo ? 0 : 1;  // the range's first or last tile
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = tid + i * NT;
        if (e < a.M * COLS)
          __hip_atomic_store(&a.sk_part[((size_t)p * 2 + slot) * kEnt + e], v[i], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are done
      __syncthreads();
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(&a.sk_cnt[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == q1 - q0;
      __syncthreads();
      if (!s_last) continue;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = tid + i * NT;
        if (e >= a.M * COLS) continue;
        float tot = 0.f;
        for (int q = q0; q <= q1; ++q)
          tot += q == p ? v[i]
                        : __hip_atomic_load(&a.sk_part[((size_t)q * 2 + (t * nsup < q * per ? 0 : 1)) * kEnt + e],
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v[i] = tot;
      }
      if (tid == 0) __hip_atomic_store(&a.sk_cnt[t], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid + i * NT;
      if (e < kEnt) fin[e] = v[i];
    }
    __syncthreads();
    gemm_epilogue<T, COLS, NT>(a, t, 0, fin, s_rstd);
  }
}

namespace {
int env_int(const char *name, int dflt) {
  const char *e = getenv(name);
  return e ? atoi(e) : dflt;
}
}  // namespace

template <typename T, int MT, int CT, int NW, int XR>
static void launch_xr(const GemmArgs &a, int pd, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  // hipExtLaunchKernelGGL carries the optional timing events in the dispatch itself
  if constexpr (MT == 4) {
    if (pd >= 2) {
      hipExtLaunchKernelGGL((gemm_kernel<T, MT, CT, NW, 2, XR>), grid, dim3(NW * 64), 0, s, e0, e1, 0, a);
      return;
    }
  }
  if constexpr (MT == 1) {
    if (pd == 3) {
      hipExtLaunchKernelGGL((gemm_kernel<T, MT, CT, NW, 3, XR>), grid, dim3(NW * 64), 0, s, e0, e1, 0, a);
      return;
    }
    if (pd == 2) {
      hipExtLaunchKernelGGL((gemm_kernel<T, MT, CT, NW, 2, XR>), grid, dim3(NW * 64), 0, s, e0, e1, 0, a);
      return;
    }
  }
  hipExtLaunchKernelGGL((gemm_kernel<T, MT, CT, NW, 1, XR>), grid, dim3(NW * 64), 0, s, e0, e1, 0, a);
}

template <typename T, int MT, int CT, int NW>
static void launch_pd(const GemmArgs &a, int pd, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if constexpr (MT == 1) {
    if (a.M <= 8) {
      launch_xr<T, MT, CT, NW, 8>(a, pd, grid, s, e0, e1);
      return;
    }
  }
  launch_xr<T, MT, CT, NW, 16 * MT>(a, pd, grid, s, e0, e1);
}

template <typename T, int MT>
static void launch_mt(const GemmArgs &a, int ct, int nw, int pd, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const int tiles = a.epi == EPI_SWIGLU ? a.N / (8 * ct) : a.N / (16 * ct);
  dim3 grid(tiles, a.ksplit);
  if constexpr (MT == 4) {  // 8 waves would not fit their 64 staged X rows in LDS
    if (ct == 1) launch_pd<T, MT, 1, 4>(a, pd, grid, s, e0, e1);
    else launch_pd<T, MT, 2, 4>(a, pd, grid, s, e0, e1);
  } else {
    if (ct == 1) {
      if (nw == 8) launch_pd<T, MT, 1, 8>(a, pd, grid, s, e0, e1);
      else launch_pd<T, MT, 1, 4>(a, pd, grid, s, e0, e1);
    } else {
      if (nw == 8) launch_pd<T, MT, 2, 8>(a, pd, grid, s, e0, e1);
      else launch_pd<T, MT, 2, 4>(a, pd, grid, s, e0, e1);
    }
  }
}

struct TileCfg {
  int ct, nw, pd;
};

// Tile width and waves per work-group, from MI355X sweeps at M = 8 (one launch per shape, weights
// rotated through more memory than the memory-side cache holds): 32-row tiles with 8 waves stream best
// for hidden-width outputs (o / down / fc projections) and SwiGLU pairs; 16-row tiles with 4 waves for
// mid-sized outputs with short K (q/k/v, injected k/v: 448 tiles cover the CUs 1.75 times), 32-row tiles
// with 4 waves for the LM head.
static TileCfg pick_tiles(int epi, int N, int K) {
  static const int env_ct = env_int("DFLASH_GEMM_CT", 0), env_nw = env_int("DFLASH_GEMM_NW", 0),
                   env_pd = env_int("DFLASH_GEMM_PD", 0), env_pct = env_int("DFLASH_GEMM_PART_CT", 0),
                   env_pnw = env_int("DFLASH_GEMM_PART_NW", 0);
  TileCfg t{2, 8, 1};
  if (epi != EPI_SWIGLU && N >= 6144 && N <= 12288 && K <= 8192) {
    t.ct = 1;
    t.nw = 4;
  } else if (epi != EPI_SWIGLU && N >= 65536) {
    t.nw = 4;
  }
  if (epi == EPI_SWIGLU) {  // 8 gate + 8 up rows per 16-column tile
    t.ct = 1;
    t.nw = 8;
  }
  static const int env_sct = env_int("DFLASH_GEMM_SWIGLU_CT", 0);
  if (env_sct && epi == EPI_SWIGLU) t.ct = env_sct;
  if (env_ct && epi != EPI_SWIGLU) t.ct = env_ct;
  if (env_nw) t.nw = env_nw;
  if (env_pct && epi == EPI_PARTIAL) t.ct = env_pct;
  if (env_pnw && epi == EPI_PARTIAL) t.nw = env_pnw;
  if (env_pd) t.pd = env_pd;
  if (epi != EPI_SWIGLU && N % (16 * t.ct)) t.ct = 1;
  if (epi == EPI_RESID_NORM) t.ct = 2;  // its sums of squares are per 32 columns
  if (t.ct != 1 && t.ct != 2) t.ct = 1;
  if (t.nw != 4 && t.nw != 8) t.nw = 4;
  if (t.pd < 1 || t.pd > 3) t.pd = 1;
  return t;
}

int gemm_ksplit(int M, int N, int K, int dtype, size_t cap_elems) {
  // Splitting K did not pay at the 27B decode shapes on MI355X (more, shorter work-groups stream
  // no faster), so ranges are used only on request (DFLASH_GEMM_SPLIT).
  static const int env_split = env_int("DFLASH_GEMM_SPLIT", 1);
  if (M > 16 || env_split <= 1) return 1;
  const TileCfg t = pick_tiles(EPI_PARTIAL, N, K);
  const int tiles = N / (16 * t.ct);
  const int sk = 256 / (dtype == 0 ? 2 : 4);  // K elements per super-step
  (void)tiles;
  int split = 1;
  while (split < env_split && K % (2 * split * sk) == 0 && (size_t)2 * split * M * N <= cap_elems) split *= 2;
  return split;
}

// Stream-K launch: only with the caller's scratch, for shapes the kernel covers, and by default for the
// hidden-width (residual + norm) and SwiGLU projections, where it measured faster on MI355X at M = 8
// (o 15.0 -> 13.8 us, down 37.6 -> 33.7 us, gate/up 72 -> 64 us); q/k/v (448 16-column tiles) and the
// LM head (4748 tiles) stream as fast or faster with one tile per work-group.
// DFLASH_GEMM_SK=0 turns it off, =1 uses it wherever the shape allows.
static int sk_per(const GemmArgs &a, int dtype, int *n_wg) {
  const int env = env_int("DFLASH_GEMM_SK", -1);  // read per launch: tests switch it
  if (!a.sk_part || !a.sk_cnt || (env == 0 && !a.sk_force) || a.M < 1 || a.M > 16 || a.ksplit != 1) return 0;
  const int sk = dtype == 0 ? 128 : 64;  // K elements per super-step
  if (a.K < sk || a.K % sk) return 0;
  const bool swiglu = a.epi == EPI_SWIGLU;
  const int cols = 32;  // output columns per tile (SWIGLU: half gate, half up)
  if (swiglu ? a.N % (cols / 2) : a.N % cols) return 0;
  if (!swiglu)
    for (int i = 0; i < a.nseg; ++i)
      if (a.seg[i].n % cols) return 0;
  if (env != 1 && !a.sk_force && a.epi != EPI_RESID_NORM && !swiglu) return 0;
  const long ntile = swiglu ? a.N / (cols / 2) : a.N / cols;
  if (ntile > a.sk_max_tiles) return 0;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const long items = ntile * (a.K / sk);
  const int env_wg = env_int("DFLASH_GEMM_SK_WG", 0);  // work-groups of a stream-K launch, for tuning
  const long wg = std::min<long>(env_wg > 0 ? env_wg : cus[dev], a.sk_max_wg);
  if (wg < 1) return 0;
  const long per = (items + wg - 1) / wg;
  *n_wg = (int)((items + per - 1) / per);
  return (int)per;
}

hipError_t launch_gemm(const GemmArgs &a, int dtype, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (a.ksplit < 1 || a.K % a.ksplit || (a.ksplit > 1 && a.epi != EPI_PARTIAL)) return hipErrorInvalidValue;
  if (a.epi == EPI_RESID_NORM && (a.N % 32 || a.sel_stride < 1 || !a.gain || !a.xg || !a.ss_out))
    return hipErrorInvalidValue;
  if (a.ss_in && (a.ss_n < 1 || a.norm_dim < 1 || a.ss_ld % 4 || a.ss_n > a.ss_ld)) return hipErrorInvalidValue;
  if (a.epi == EPI_RESID_NORM && a.N / 32 > a.ss_out_ld) return hipErrorInvalidValue;
  int n_wg = 0;
  const int sk = sk_per(a, dtype, &n_wg);
  if (a.sk_force && !sk) return hipErrorInvalidValue;
  if (const int per = sk) {
    const dim3 grid(n_wg), block(512);
    const bool x8 = a.M <= 8;
    if (dtype == 0) {
      if (x8) hipExtLaunchKernelGGL((gemm_sk_kernel<bf16, 8>), grid, block, 0, s, e0, e1, 0, a, per);
      else hipExtLaunchKernelGGL((gemm_sk_kernel<bf16, 16>), grid, block, 0, s, e0, e1, 0, a, per);
    } else {
      if (x8) hipExtLaunchKernelGGL((gemm_sk_kernel<float, 8>), grid, block, 0, s, e0, e1, 0, a, per);
      else hipExtLaunchKernelGGL((gemm_sk_kernel<float, 16>), grid, block, 0, s, e0, e1, 0, a, per);
    }
    return hipGetLastError();
  }
  const TileCfg t = pick_tiles(a.epi, a.N, a.K);
  const int xr = a.M;
  if (xr > kGemmMaxRows) return hipErrorInvalidValue;  // the host chunks longer inputs
  const int MT = xr <= 16 ? 1 : (xr <= 32 ? 2 : 4);
  if (dtype == 0) {
    if (MT == 1) launch_mt<bf16, 1>(a, t.ct, t.nw, t.pd, s, e0, e1);
    else if (MT == 2) launch_mt<bf16, 2>(a, t.ct, t.nw, t.pd, s, e0, e1);
    else launch_mt<bf16, 4>(a, t.ct, t.nw, t.pd, s, e0, e1);
  } else {
    if (MT == 1) launch_mt<float, 1>(a, t.ct, t.nw, t.pd, s, e0, e1);
    else if (MT == 2) launch_mt<float, 2>(a, t.ct, t.nw, t.pd, s, e0, e1);
    else launch_mt<float, 4>(a, t.ct, t.nw, t.pd, s, e0, e1);
  }
  return hipGetLastError();
}

}  // namespace df
