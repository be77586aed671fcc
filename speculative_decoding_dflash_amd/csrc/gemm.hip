// Skinny GEMM Y[M, N] = X[M, K] W[N, K]^T on MFMA (gfx950), with fused epilogues.
//
// The decode step is weight-streaming: M (block x batch rows) is small, so every weight byte is read
// once from HBM and the MFMA units are far from busy.  The kernel is built for that:
//   * a work-group (4 waves) owns 32 weight rows (two 16-row MFMA column tiles) over a K range; the
//     four waves take interleaved 32-element K steps, so at any moment the work-group reads 256
//     contiguous bytes of each of its rows, and each lane issues 16-byte loads;
//   * X fragments come straight from global memory (they stay in L2: X is at most 64 x K);
//   * v_mfma_f32_16x16x32_bf16 (or 4 x v_mfma_f32_16x16x4f32 for fp32 models) accumulates in fp32;
//   * the four waves reduce through LDS; when the K range is split over work-groups, or an epilogue
//     needs more than 32 columns (per-head RMSNorm + RoPE needs whole heads), partial tiles go to an
//     fp32 workspace and the last work-group to arrive (agent-scope counter) sums them in a fixed
//     order -- results do not depend on arrival order -- and runs the epilogue.
// Epilogues: fp32 store (logits), activation store, residual add (+ optional feature tap), SwiGLU
// (gate and up rows of the same output column in one work-group), and QKV (per-head q/k RMSNorm,
// rotate-half RoPE at each row's absolute position, paged K/V scatter).
#include "kernels.h"

namespace df {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> {
  static constexpr int kEPL = 8;   // elements per lane per K step
  static constexpr int kStep = 32; // K per step
  static DF_DEVICE void mma(f32x4 &acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
  }
};
template <> struct Frag<float> {
  static constexpr int kEPL = 4;
  static constexpr int kStep = 16;
  // Element j of every lane's 4-vector forms one K=4 slice (k = 4*(lane/16) + j), identically for A and B.
  static DF_DEVICE void mma(f32x4 &acc, u32x4 a, u32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.x), __builtin_bit_cast(float, b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.y), __builtin_bit_cast(float, b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.z), __builtin_bit_cast(float, b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, a.w), __builtin_bit_cast(float, b.w), acc, 0, 0, 0);
  }
};

template <typename T> DF_DEVICE u32x4 ld16(const T *p) { return *reinterpret_cast<const u32x4 *>(p); }

DF_DEVICE float silu(float g) { return g / (1.0f + expf(-g)); }

// Epilogue over a tile of M rows x G columns held in LDS (row stride ld).  col0: first column of the
// tile in weight-row space (for SwiGLU the tile holds 16 gate then 16 up columns of output col0/2).
template <typename T>
DF_DEVICE void epilogue(const GemmArgs &a, const float *tile, int ld, int G, int col0, int seg_i, int seg_base) {
  const int tid = threadIdx.x;
  const int M = a.M;
  switch (a.epi) {
    case EPI_STORE_F32:
      for (int e = tid; e < M * G; e += 256) {
        int m = e / G, j = e % G;
        a.out_f32[(size_t)(a.row_off + m) * a.ld_out + col0 + j] = tile[m * ld + j];
      }
      break;
    case EPI_STORE_ACT:
      for (int e = tid; e < M * G; e += 256) {
        int m = e / G, j = e % G;
        Elem<T>::store((T *)a.out_act + (size_t)(a.row_off + m) * a.ld_out + col0 + j, tile[m * ld + j]);
      }
      break;
    case EPI_RESID:
      for (int e = tid; e < M * G; e += 256) {
        int m = e / G, j = e % G;
        size_t idx = (size_t)(a.row_off + m) * a.ld_resid + col0 + j;
        float v = a.resid[idx] + tile[m * ld + j];
        a.resid[idx] = v;
        if (a.feat) Elem<T>::store((T *)a.feat + (size_t)(a.row_off + m) * a.ld_feat + col0 + j, v);
      }
      break;
    case EPI_SWIGLU:
      for (int e = tid; e < M * 16; e += 256) {
        int m = e / 16, j = e % 16;
        float g = tile[m * ld + j], u = tile[m * ld + 16 + j];
        Elem<T>::store((T *)a.out_act + (size_t)(a.row_off + m) * a.ld_out + col0 / 2 + j, silu(g) * u);
      }
      break;
    case EPI_QKV: {
      const GemmSeg &sg = a.seg[seg_i];
      const int d = a.kv.head_dim, half = d / 2;
      const int hpg = G / d;              // heads in this tile
      const int tpp = kWave / half;       // (row, head) tasks per wave pass
      const int wave = tid >> 6, lane = tid & 63;
      const int sub = lane / half, i = lane % half;
      const int cs = col0 - seg_base;     // first column of the tile inside its segment
      const int ntask = M * hpg;
      const double inv = pow((double)a.theta, -2.0 * (double)i / (double)d);
      for (int tb = wave * tpp; tb < ntask; tb += 4 * tpp) {
        const int task = tb + sub;
        const bool live = task < ntask;
        const int m = live ? task / hpg : 0, h = live ? task % hpg : 0;
        float v1 = tile[m * ld + h * d + i], v2 = tile[m * ld + h * d + i + half];
        const int grow = a.row_off + m;
        if (sg.role == ROLE_Q || sg.role == ROLE_K) {
          float ss = v1 * v1 + v2 * v2;
          for (int off = half / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
          const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
          v1 = v1 * r * sg.gain[i];
          v2 = v2 * r * sg.gain[i + half];
          const double ang = (double)a.rows.pos[grow] * inv;
          const float c = (float)cos(ang), s = (float)sin(ang);
          const float o1 = v1 * c - v2 * s, o2 = v2 * c + v1 * s;
          v1 = o1;
          v2 = o2;
        }
        if (!live) continue;
        const int head = cs / d + h;
        if (sg.role == ROLE_Q || sg.role == ROLE_PLAIN) {
          T *q = (T *)sg.dst + (size_t)grow * sg.ld_dst + head * d;
          Elem<T>::store(q + i, v1);
          Elem<T>::store(q + i + half, v2);
        } else if (a.rows.valid[grow]) {
          const int pos = a.rows.pos[grow], slot = a.rows.slot[grow];
          const int pidx = pos / a.kv.page_tokens;
          const int page = (pidx < a.bt_stride) ? a.block_table[(size_t)slot * a.bt_stride + pidx] : -1;
          if (page < 0) {
            raise_err(a.err, ERR_PAGE);
            continue;
          }
          const int tok = pos % a.kv.page_tokens;
          T *base = (T *)sg.dst;
          if (sg.role == ROLE_K) {
            Elem<T>::store(base + a.kv.k_index(page, head, tok, i), v1);
            Elem<T>::store(base + a.kv.k_index(page, head, tok, i + half), v2);
          } else {
            Elem<T>::store(base + a.kv.v_index(page, head, tok, i), v1);
            Elem<T>::store(base + a.kv.v_index(page, head, tok, i + half), v2);
          }
        }
      }
      break;
    }
  }
}

template <typename T, int MT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  using F = Frag<T>;
  __shared__ float lds[4 * 16 * MT * 32];
  __shared__ int s_last;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const bool swiglu = a.epi == EPI_SWIGLU;
  const int c = blockIdx.x, ks = blockIdx.y;

  // Weight rows of this lane in the two 16-row column tiles.
  const T *wp0, *wp1;
  int seg_i = 0, seg_base = 0;
  if (swiglu) {
    wp0 = (const T *)a.seg[0].w + (size_t)(16 * c + r16) * a.K;
    wp1 = (const T *)a.seg[1].w + (size_t)(16 * c + r16) * a.K;
  } else {
    const int r0 = 32 * c;
    while (seg_i + 1 < a.nseg && r0 >= seg_base + a.seg[seg_i].n) {
      seg_base += a.seg[seg_i].n;
      ++seg_i;
    }
    const T *w = (const T *)a.seg[seg_i].w;
    wp0 = w + (size_t)(r0 - seg_base + r16) * a.K;
    wp1 = w + (size_t)(r0 - seg_base + 16 + r16) * a.K;
  }
  const T *xp[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    xok[mt] = m < a.M;
    xp[mt] = (const T *)a.x + (size_t)(xok[mt] ? m : 0) * a.ldx;
  }

  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int kbeg = ks * a.kchunk;
  const int kend = min(a.K, kbeg + a.kchunk);
  const int nsteps = kend > kbeg ? (kend - kbeg) / F::kStep : 0;
  const int loff = kbeg + g * F::kEPL;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  int s = wave;
  for (; s + 12 < nsteps; s += 16) {
    u32x4 wv[4][2], xv[4][MT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = loff + (s + 4 * u) * F::kStep;
      wv[u][0] = ld16(wp0 + k);
      wv[u][1] = ld16(wp1 + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xv[u][mt] = xok[mt] ? ld16(xp[mt] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        F::mma(acc[mt][0], xv[u][mt], wv[u][0]);
        F::mma(acc[mt][1], xv[u][mt], wv[u][1]);
      }
  }
  for (; s < nsteps; s += 4) {
    const int k = loff + s * F::kStep;
    const u32x4 w0 = ld16(wp0 + k), w1 = ld16(wp1 + k);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 xv = xok[mt] ? ld16(xp[mt] + k) : zero;
      F::mma(acc[mt][0], xv, w0);
      F::mma(acc[mt][1], xv, w1);
    }
  }

  // Reduce the four waves' partial tiles: C[m][n] sits at lane (n = lane % 16, m = 4 * (lane / 16) + r).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lds[((wave * 16 * MT) + mt * 16 + g * 4 + r) * 32 + ct * 16 + r16] = acc[mt][ct][r];
  __syncthreads();
  constexpr int kEnt = 16 * MT * 32;
  float sums[kEnt / 256];
#pragma unroll
  for (int i = 0; i < kEnt / 256; ++i) {
    const int e = tid + 256 * i;
    sums[i] = ((lds[e] + lds[kEnt + e]) + lds[2 * kEnt + e]) + lds[3 * kEnt + e];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kEnt / 256; ++i) lds[tid + 256 * i] = sums[i];
  __syncthreads();

  const int arrivals = (a.group / 32) * a.split;
  if (arrivals == 1) {
    epilogue<T>(a, lds, 32, 32, 32 * c, seg_i, seg_base);
    return;
  }
  // Several work-groups meet in this epilogue group: publish the partial tile, count arrivals.
  const int NP = gridDim.x * 32;
  for (int e = tid; e < a.M * 32; e += 256) {
    const int m = e / 32, j = e % 32;
    a.partial[((size_t)ks * a.M + m) * NP + 32 * c + j] = lds[m * 32 + j];
  }
  __threadfence();
  __syncthreads();
  const int gi = (32 * c) / a.group;
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(a.counters + gi, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == arrivals - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int gc0 = gi * a.group;
  for (int e = tid; e < a.M * a.group; e += 256) {
    const int m = e / a.group, j = e % a.group;
    float v = 0.f;
    for (int q = 0; q < a.split; ++q)
      v += __builtin_nontemporal_load(a.partial + ((size_t)q * a.M + m) * NP + gc0 + j);
    lds[m * a.group + j] = v;
  }
  if (tid == 0) __hip_atomic_store(a.counters + gi, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  epilogue<T>(a, lds, a.group, a.group, gc0, seg_i, seg_base);
}

hipError_t launch_gemm(const GemmArgs &a, int dtype, hipStream_t s) {
  const int tiles = a.epi == EPI_SWIGLU ? a.N / 16 : a.N / 32;
  dim3 grid(tiles, a.split), block(256);
  const int MT = a.M <= 16 ? 1 : (a.M <= 32 ? 2 : 4);
  if (dtype == 0) {
    if (MT == 1) hipLaunchKernelGGL((gemm_kernel<bf16, 1>), grid, block, 0, s, a);
    else if (MT == 2) hipLaunchKernelGGL((gemm_kernel<bf16, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<bf16, 4>), grid, block, 0, s, a);
  } else {
    if (MT == 1) hipLaunchKernelGGL((gemm_kernel<float, 1>), grid, block, 0, s, a);
    else if (MT == 2) hipLaunchKernelGGL((gemm_kernel<float, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<float, 4>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace df
