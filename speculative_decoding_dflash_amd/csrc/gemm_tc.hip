// Tiled MFMA projection for many rows (decode batches of 32+ rows, prefill) of bf16 models:
// Y[M, N] = X[M, K] W[N, K]^T with X in fp16 (the activation type of bf16 models, see ActOf) and the bf16
// weights converted to fp16 as they are staged (exactly wherever fp16 is normal, see bf16x2_to_f16x2),
// accumulated in fp32 by v_mfma_f32_16x16x32_f16.  The row-chunked kernels of gemm.hip stream the
// weights past a handful of rows; here the product is compute-bound and the tiles are MFMA-shaped.
//
// Shape of the kernel:
//   * a work-group (4 waves, or 8 -- two per SIMD -- for 256-row tiles) computes a BM-row x (32 U)-
//     column tile, U <= UM "units" of 32 weight rows (SWIGLU: 16 output columns, as two 16-row fragments
//     of 8 gate rows and the same 8 up rows, paired in the epilogue by a lane exchange); each wave holds
//     64 rows of the tile and 1/WC of its 16-row fragments;
//   * the units of a projection are cut into `nch` contiguous chunks of as equal a size as possible
//     (grid x), so that a launch can have about one work-group per CU even when 32 UM does not divide
//     N into the CU count (the 27B gate/up's 1088 units make 256 chunks of 4 or 5);
//   * K runs in steps of 64 through a double-buffered LDS tile: the loads of step k + 2 are issued while
//     step k is multiplied out of LDS and step k + 1 waits in registers; every load is unconditional
//     (past the range, rows and steps are clamped onto valid memory and never used), so the waits count
//     outstanding loads exactly;
//   * grid z cuts K into ranges for projections with too few tiles to cover the CUs; each range writes
//     its raw fp32 sums to out_f32 + z * part_stride (EPI_PARTIAL), and the consumer adds the ranges in
//     order (qkv_post_kernel, norm_kernel);
//   * epilogues: fp32 store (EPI_STORE_F32, EPI_PARTIAL) and SwiGLU with an fp16 store of silu(g) u.
#include <hip/hip_ext.h>

#include <algorithm>

#include "kernels.h"

namespace df {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBK = 64;  // K per LDS step: one 128-byte LDS row per tile row

// LDS tiles hold 128-byte rows of eight 16-byte chunks; chunk c of row r sits at chunk c ^ sw(r).  With
// that swizzle the 16-byte fragment reads (16 rows, one chunk each) run at the full LDS rate on gfx950
// (measured: 4 cycles per 16-byte wave read, twice that with (r >> 3) & 1 added to the swizzle), and
// the staging writes (8 lanes per row) fill whole rows.
DF_DEVICE int sw(int r) { return r & 7; }
DF_DEVICE int lds_off(int r, int c) { return r * kBK + ((c ^ sw(r)) << 3); }

DF_DEVICE u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

DF_DEVICE u32x4 bf8_to_h8(u32x4 v) {
  return (u32x4){bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
}

DF_DEVICE void mma(f32x4 &acc, u32x4 a, u32x4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
}

DF_DEVICE float silu(float g) { return g / (1.0f + expf(-g)); }

// X row of local row m (< M): m itself, or with a row selection the selected row of global row row_off + m.
DF_DEVICE int tc_x_src(const GemmArgs &a, int m) {
  if (!a.x_take) return m;
  const int r = a.row_off + m;
  return (r / a.x_take) * a.x_stride + a.x_off + r % a.x_take;
}

template <int BM, int UM, int STG, int NWV, bool PIPE>
__global__ __launch_bounds__(NWV * 64, BM == 256 ? 1 : 2) void gemm_tc_kernel(GemmArgs a, int nch, int steps) {
  constexpr int NT = NWV * 64;
  constexpr int WR = BM / 64, WC = NWV / WR;  // waves across the tile's rows (64 each) and columns
  constexpr int BN = UM * 32;                 // weight rows of a full chunk
  constexpr int NJ = BN / 16 / WC;            // 16-row weight fragments per wave
  // 16-byte loads per thread and K step (chunks past the tile load a valid address and are not stored)
  constexpr int CA = (BM * 8 + NT - 1) / NT, CB = (BN * 8 + NT - 1) / NT;
  static_assert(WR * WC == NWV && NJ * WC * 16 == BN, "wave layout");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * kBK];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int wr = wave / WC, wc = wave % WC;
  const bool swiglu = a.epi == EPI_SWIGLU;
  const int units = swiglu ? a.N / 16 : a.N / 32;
  // XCD-aware order: work-group b runs on XCD b % 8 (round-robin dispatch); each XCD takes a contiguous
  // range of the (K range, row tile, chunk) items.  Within a K range the items run in blocks of up to
  // RB row tiles x CB chunks (chunk fastest, then row tile), so that the work-groups an XCD holds at
  // once share both their X row tiles and their weight chunks through the XCD's L2 (with chunk-fastest
  // order alone every row tile re-reads every weight chunk from memory).  8 x 8 measured best at 6400
  // rows (gate/up 13% faster than 4 x 8, 19% than chunk-fastest).
  int ch, ty, tz;
  {
    constexpr int RB = 8, CB = 8;
    const int rt = gridDim.y, T = nch * rt * gridDim.z;
    const int b = blockIdx.x + nch * (blockIdx.y + rt * blockIdx.z);
    const int per = T / 8, rem = T % 8, xcd = b % 8;
    const int l = xcd * per + min(xcd, rem) + b / 8;
    tz = l / (nch * rt);
    const int lz = l - tz * nch * rt;
    const int rg = lz / (RB * nch), rb = min(RB, rt - rg * RB);  // row group and its row tiles
    const int lr = lz - rg * RB * nch;
    const int cg = lr / (rb * CB), cb = min(CB, nch - cg * CB);  // chunk group and its chunks
    const int lc = lr - cg * rb * CB;
    ty = rg * RB + lc / cb;
    ch = cg * CB + lc % cb;
  }
  const int u0 = (int)((long)units * ch / nch), u1 = (int)((long)units * (ch + 1) / nch);
  const int nrows = (u1 - u0) * 32;  // weight rows of this chunk (<= BN)
  const int m0 = ty * BM;
  const int nk = a.K / kBK;
  const int kt0 = tz * steps, kt1 = min(nk, kt0 + steps);

  // this thread's 16-byte chunks of a K step: chunk c = tid + 256 i -> tile row c / 8, halfs 8 (c % 8) ..
  const uint16_t *pa[CA], *pb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + NT * i, row = min(c >> 3, BM - 1), kc = (c & 7) * 8;
    pa[i] = (const uint16_t *)a.x + (size_t)tc_x_src(a, min(m0 + row, a.M - 1)) * a.ldx + kc;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + NT * i, kc = (c & 7) * 8;
    const int lr = (c >> 3) < nrows ? (c >> 3) : 0;  // rows past the chunk (or the tile) reload its first row
    const uint16_t *w;
    if (swiglu) {  // unit u, half h (16-row fragment 2 u + h): rows 0-7 gate rows 16 u + 8 h .., 8-15 the same up rows
      const int u = u0 + lr / 32, h = (lr >> 4) & 1;
      w = (const uint16_t *)a.seg[(lr >> 3) & 1].w + (size_t)(16 * u + 8 * h + (lr & 7)) * a.K;
    } else {
      int nr = 32 * u0 + lr, si = 0;
      while (si + 1 < a.nseg && nr >= a.seg[si].n) {
        nr -= a.seg[si].n;
        ++si;
      }
      w = (const uint16_t *)a.seg[si].w + (size_t)nr * a.K;
    }
    pb[i] = w + kc;
  }

  f32x4 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // STG register stages: the loads of step k + STG are issued while step k is multiplied out of
  // LDS buffer (k - k0) % 2 and steps k + 1 .. k + STG - 1 are in flight; the stage index of step k is
  // (k - k0) % STG, a template constant in the unrolled loop so that the stages stay in registers.
  u32x4 ra[STG][CA], rb[STG][CB];
  auto load = [&](int st, int kt) {
    const int k = min(kt, kt1 - 1) * kBK;
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[st][i] = ld16(pa[i] + k);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[st][i] = ld16(pb[i] + k);
  };
  auto store = [&](int st, int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + NT * i;
      if ((BM * 8) % NT == 0 || c < BM * 8) *reinterpret_cast<u32x4 *>(&sA[buf][lds_off(c >> 3, c & 7)]) = ra[st][i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + NT * i;
      if ((BN * 8) % NT == 0 || c < BN * 8)
        *reinterpret_cast<u32x4 *>(&sB[buf][lds_off(c >> 3, c & 7)]) = bf8_to_h8(rb[st][i]);
    }
  };
  auto mult = [&](int buf) {
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      u32x4 fa[4], fb[NJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const u32x4 *>(&sA[buf][lds_off(wr * 64 + 16 * i + r16, 4 * s + g)]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[j] = *reinterpret_cast<const u32x4 *>(&sB[buf][lds_off((wc * NJ + j) * 16 + r16, 4 * s + g)]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mma(acc[i][j], fa[i], fb[j]);
    }
  };
#pragma unroll
  for (int st = 0; st < STG; ++st) load(st, kt0 + st);
  store(0, 0);
  __syncthreads();
  // PIPE: both K halves' fragments are read first (the second half's reads overlap the first half's
  // MFMAs) and the next step's LDS stores go between the halves, so that the MFMAs of a step are not
  // preceded by the wait for their own fragments and followed by the stores
  auto frags = [&](int buf, int s, u32x4 *fa, u32x4 *fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[i] = *reinterpret_cast<const u32x4 *>(&sA[buf][lds_off(wr * 64 + 16 * i + r16, 4 * s + g)]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[j] = *reinterpret_cast<const u32x4 *>(&sB[buf][lds_off((wc * NJ + j) * 16 + r16, 4 * s + g)]);
  };
  auto mmas = [&](const u32x4 *fa, const u32x4 *fb) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) mma(acc[i][j], fa[i], fb[j]);
  };
  auto kstep = [&](int kt, auto stc) {
    constexpr int st = decltype(stc)::value;
    const int buf = (kt - kt0) & 1;
    if constexpr (PIPE) {
      u32x4 fa0[4], fb0[NJ], fa1[4], fb1[NJ];
      frags(buf, 0, fa0, fb0);
      load(st, kt + STG);
      frags(buf, 1, fa1, fb1);
      mmas(fa0, fb0);
      if (kt + 1 < kt1) store((st + 1) % STG, buf ^ 1);
      mmas(fa1, fb1);
    } else {
      load(st, kt + STG);
      mult(buf);
      if (kt + 1 < kt1) store((st + 1) % STG, buf ^ 1);
    }
    __syncthreads();
  };
  int kt = kt0;
  for (; kt + STG <= kt1; kt += STG) {
    kstep(kt, std::integral_constant<int, 0>{});
    kstep(kt + 1, std::integral_constant<int, 1>{});
    if constexpr (STG == 3) kstep(kt + 2, std::integral_constant<int, 2>{});
  }
  if (kt < kt1) kstep(kt, std::integral_constant<int, 0>{});
  if (kt + 1 < kt1) kstep(kt + 1, std::integral_constant<int, 1>{});

  // acc[i][j][r] = Y[row m0 + 64 wr + 16 i + 4 g + r][weight row 32 u0 + 16 (wc NJ + j) + r16]
  if (swiglu) {  // a fragment's gate sums sit in lanes r16 < 8, the matching up sums 8 lanes further
    uint16_t *out = (uint16_t *)a.out_act;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int fl = wc * NJ + j;  // the fragment in the chunk
      if (fl * 16 >= nrows) continue;  // wave-uniform
      const int col = 16 * (u0 + fl / 2) + 8 * (fl & 1) + (r16 & 7);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gt = acc[i][j][r], up = __shfl_xor(gt, 8);
          const int m = m0 + 64 * wr + 16 * i + 4 * g + r;
          if (r16 < 8 && m < a.M) out[(size_t)(a.row_off + m) * a.ld_out + col] = f32_to_f16(silu(gt) * up);
        }
    }
    return;
  }
  float *out = a.out_f32 + (size_t)tz * a.part_stride;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int lr = (wc * NJ + j) * 16;
    if (lr >= nrows) continue;
    const int col = 32 * u0 + lr + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 64 * wr + 16 * i + 4 * g + r;
        if (m < a.M) out[(size_t)(a.row_off + m) * a.ld_out + col] = acc[i][j][r];
      }
  }
}

int env_int(const char *name, int dflt) {
  const char *e = getenv(name);
  return e ? atoi(e) : dflt;
}

int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus[dev] = 256;
  return cus[dev];
}

}  // namespace

// Tile height, units per chunk, chunk count and K ranges of a projection.  The choice minimises a
// simple model of the launch's time: rounds of work-groups (one per CU for 256-row tiles, two
// otherwise) times the longest chunk's units times its K steps, plus a fixed cost per work-group and
// the fp32 traffic of K-range partials.  DFLASH_TC_{BM,S,NCH} override it for sweeps.
bool gemm_tc_plan(const GemmArgs &a, int64_t range_cap, TcPlan *p) {
  const bool swiglu = a.epi == EPI_SWIGLU;
  if (a.M < 1 || a.K % kBK || a.ksplit != 1 || a.ss_in) return false;
  if (a.epi != EPI_STORE_F32 && a.epi != EPI_PARTIAL && !swiglu) return false;
  if (swiglu ? (a.N % 16 || a.nseg != 2) : a.N % 32) return false;
  if (!swiglu)
    for (int i = 0; i < a.nseg; ++i)
      if (a.seg[i].n % 32) return false;
  const int env_bm = env_int("DFLASH_TC_BM", 0);
  int bm = a.M <= 64 ? 64 : (a.M <= 128 ? 128 : 256);
  if (env_bm == 64 || env_bm == 128 || env_bm == 256) bm = env_bm;
  // 256-row tiles: eight waves (two per SIMD; DFLASH_TC_W8=0: four) with 5 or 6 units per chunk (6 only
  // where it saves a round of work-groups: a chunk of 6 runs a few per cent slower per unit); 64- and
  // 128-row tiles: four waves, 4 units.  DFLASH_TC_UM fixes the unit count.
  // The decode layers' projections on 64-row tiles (SwiGLU, and K-range partials) plan for one
  // work-group per CU with chunks of up to 6 units: two work-groups on one CU share its LDS and run at
  // about half speed each.  27B, 64 rows: gate/up in 363 chunks of 3 took 93 us against 78.5 us for 218
  // chunks of 5-6 alone on their CUs; down in 8 K ranges 42.3 against 36.8 us.  DFLASH_TC_STEP=0
  // switches this and the step cost below off.
  static const bool step_cost = env_int("DFLASH_TC_STEP", 1) != 0;
  const int env_um = env_int("DFLASH_TC_UM", 0);
  const bool glu64 = step_cost && bm == 64 && env_um == 0 && (swiglu || a.epi == EPI_PARTIAL);
  const int nwv = bm == 256 && env_int("DFLASH_TC_W8", 1) ? 8 : 4;
  const int um_lo = bm == 64 && env_um == 6 ? 6 : bm != 256 ? 4 : (env_um == 4 && nwv == 4) || (env_um == 6 && nwv == 8) ? env_um : 5;
  const int um_hi = glu64 ? 6 : bm == 256 && nwv == 8 && env_um == 0 ? 6 : um_lo;
  const int units = swiglu ? a.N / 16 : a.N / 32;
  const int rt = (a.M + bm - 1) / bm, nk = a.K / kBK;
  const int slots = cu_count() * (bm == 256 || glu64 ? 1 : 2);
  const int env_s = env_int("DFLASH_TC_S", 0), env_nch = env_int("DFLASH_TC_NCH", 0);
  // per-CU rate estimates (MI355X): ~60% of the dense fp16 MFMA peak, ~70% of an even share of HBM
  const double mfma_us = (double)bm * 32 * kBK * 2 / (0.6 * 2.5e15 / 256) * 1e6;  // one unit x one K step
  const double mem_us = (32.0 * kBK * 2) / (0.7 * 8e12 / 256) * 1e6;
  // 64-row tiles also pay a fixed ~0.6 us per K step (a fit to 64-row down / o / q-k-v launches: 1.24
  // us per step at 3 units of a chunk, 1.39 at 4, 1.08 at 2), so that fewer, longer-ranged steps win
  // there: 8 K ranges over 2 work-groups per CU measured 13% (down), 15% (q/k/v) and 6% (o) faster
  // than the plans without it.  Among equal estimates such calls take the most work-groups.
  const double step_us = step_cost && bm == 64 ? 0.6 : 0.0;
  const bool more_wgs = step_cost && bm == 64 && a.epi == EPI_PARTIAL;
  double best = 1e30;
  int best_wgs = 0;
  TcPlan bp{};
  const int smax = a.epi == EPI_PARTIAL ? kTcMaxRanges : 1;
  for (int s = 1; s <= smax; ++s) {
    if (env_s > 0 && s != env_s) continue;
    const int steps = (nk + s - 1) / s;
    if (s > 1 && (steps < 4 || (int64_t)s * a.M * a.N > range_cap)) continue;
    const int ranges = (nk + steps - 1) / steps;
    if (ranges != s) continue;
    for (int um = um_lo; um <= um_hi; ++um) {
      if (bm == 64 && um == 5) continue;  // 64-row tiles split a chunk over four waves: an even unit count
      const int nmin = (units + um - 1) / um;
      for (int nch = nmin; nch <= std::min(units, nmin * 4); ++nch) {
        if (env_nch > 0 && nch != env_nch) continue;
        const int wgs = nch * rt * s;
        const int rounds = (wgs + slots - 1) / slots;
        const int umax = (units + nch - 1) / nch;
        // a K step also stages BM X rows (from L2), worth about bm / 64 units of weight streaming
        const double per = (umax + bm / 64.0) * steps * std::max(mfma_us, mem_us) + steps * step_us + 1.5;
        const double t = rounds * per + (s > 1 ? (double)s * a.M * a.N * 8 / 5e12 * 1e6 : 0.0);
        if (t < best - 1e-9 || (more_wgs && t < best + 1e-9 && wgs > best_wgs)) {
          best = t;
          best_wgs = wgs;
          bp = TcPlan{bm, um, nch, s, steps, nwv};  // other ties keep the smaller unit count
        }
      }
    }
  }
  if (best >= 1e30) return false;
  *p = bp;
  return true;
}

template <int STG, bool PIPE>
static void launch_stg(const GemmArgs &a, const TcPlan &p, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const dim3 b4(256), b8(512);
  if (p.bm == 256) {
    if (p.nwv == 8 && p.um == 6)
      hipExtLaunchKernelGGL((gemm_tc_kernel<256, 6, STG, 8, PIPE>), grid, b8, 0, s, e0, e1, 0, a, p.nch, p.steps);
    else if (p.nwv == 8)
      hipExtLaunchKernelGGL((gemm_tc_kernel<256, 5, STG, 8, PIPE>), grid, b8, 0, s, e0, e1, 0, a, p.nch, p.steps);
    else if (p.um == 5)
      hipExtLaunchKernelGGL((gemm_tc_kernel<256, 5, STG, 4, PIPE>), grid, b4, 0, s, e0, e1, 0, a, p.nch, p.steps);
    else
      hipExtLaunchKernelGGL((gemm_tc_kernel<256, 4, STG, 4, PIPE>), grid, b4, 0, s, e0, e1, 0, a, p.nch, p.steps);
  } else if (p.bm == 128) {
    hipExtLaunchKernelGGL((gemm_tc_kernel<128, 4, STG, 4, PIPE>), grid, b4, 0, s, e0, e1, 0, a, p.nch, p.steps);
  } else {
    if (p.um == 6)
      hipExtLaunchKernelGGL((gemm_tc_kernel<64, 6, STG, 4, PIPE>), grid, b4, 0, s, e0, e1, 0, a, p.nch, p.steps);
    else
      hipExtLaunchKernelGGL((gemm_tc_kernel<64, 4, STG, 4, PIPE>), grid, b4, 0, s, e0, e1, 0, a, p.nch, p.steps);
  }
}

hipError_t launch_gemm_tc(const GemmArgs &a, const TcPlan &p, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (p.ranges > 1 && a.epi != EPI_PARTIAL) return hipErrorInvalidValue;
  const dim3 grid(p.nch, (a.M + p.bm - 1) / p.bm, p.ranges);
  // two register stages (three measured no faster, and with the pipelined step they spill); the
  // pipelined step by default, DFLASH_TC_PIPE=0 for the plain one
  static const bool pipe = env_int("DFLASH_TC_PIPE", 1) != 0;
  if (pipe) launch_stg<2, true>(a, p, grid, s, e0, e1);
  else launch_stg<2, false>(a, p, grid, s, e0, e1);
  return hipGetLastError();
}

}  // namespace df
