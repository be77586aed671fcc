// Per-call row bookkeeping, embedding gather, RMSNorm, q/k/v post-processing and argmax (gfx950).
#include "kernels.h"

namespace df {

// One work-group.  Reads the slots' device state, fills the per-row arrays, then updates the state.
//   mode 0 (verify):  rows b*q_len + i at start + i (start = 0 for a new sequence, else seq_len);
//                     records the block as pending for the next accept.
//   mode 1 (inject):  rows b*q_len + i at inj_base + row_skip + i, valid for row_skip + i < inj_rows (the
//                     committed rows of the last verified block, whose features are to be injected;
//                     row_skip leading rows are left out); clears inj_rows.
//   mode 2 (draft):   rows b*q_len + i at seq_len + i; token = anchor for i = 0, mask id otherwise.
__global__ void prep_kernel(PrepArgs a) {
  __shared__ int s_start[64], s_lim[64], s_anchor[64];
  const int tid = threadIdx.x;
  if (tid < a.batch) {
    const SlotState &st = a.state[a.slots[tid]];
    if (a.mode == 0) {
      s_start[tid] = a.new_sequence ? 0 : st.seq_len;
      s_lim[tid] = a.q_len;
    } else if (a.mode == 1) {  // the verified rows row_skip .. row_skip + q_len - 1
      s_start[tid] = st.inj_base + a.row_skip;
      s_lim[tid] = st.inj_rows - a.row_skip;
    } else {
      s_start[tid] = st.seq_len;
      s_lim[tid] = a.q_len;
      s_anchor[tid] = st.anchor;
    }
  }
  __syncthreads();
  const int n = a.batch * a.q_len;
  for (int r = tid; r < n; r += blockDim.x) {
    const int b = r / a.q_len, i = r % a.q_len;
    a.rows.pos[r] = s_start[b] + i;
    a.rows.slot[r] = a.slots[b];
    a.rows.valid[r] = i < s_lim[b];
    if (a.mode == 0) {
      int t = a.tokens[r];
      if (t < 0 || t >= a.vocab) {
        raise_err(a.err, ERR_TOKEN);
        t = 0;
      }
      a.rows.tok[r] = t;
    } else if (a.mode == 2) {
      int t = (i == 0) ? s_anchor[b] : a.mask_id;
      if (t < 0 || t >= a.vocab) {
        raise_err(a.err, ERR_STATE);
        t = 0;
      }
      a.rows.tok[r] = t;
      if (i == 0 && a.block_out) a.block_out[r] = t;
    }
  }
  __syncthreads();
  if (tid < a.batch) {
    SlotState &st = a.state[a.slots[tid]];
    if (a.mode == 0) {
      st.pend_start = s_start[tid];
      st.pend_qlen = a.q_len;
      if (a.new_sequence) {
        st.seq_len = 0;
        st.inj_rows = 0;
        st.inj_base = 0;
      }
    } else if (a.mode == 1) {
      st.inj_rows = 0;
    }
  }
}

hipError_t launch_prep(const PrepArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
__global__ void embed_kernel(const T *embed, Rows rows, int hidden, int vocab, float *x, int32_t *err) {
  const int r = blockIdx.x;
  int t = rows.tok[r];
  if (t < 0 || t >= vocab) {
    if (threadIdx.x == 0) raise_err(err, ERR_TOKEN);
    t = 0;
  }
  const T *src = embed + (size_t)t * hidden;
  float *dst = x + (size_t)r * hidden;
  for (int h = threadIdx.x; h < hidden; h += blockDim.x) dst[h] = Elem<T>::load(src + h);
}

hipError_t launch_embed(const void *embed, int dtype, const Rows &rows, int32_t n_rows, int32_t hidden, int32_t vocab,
                        float *x, int32_t *err, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  if (dtype == 0) hipLaunchKernelGGL((embed_kernel<bf16>), dim3(n_rows), dim3(256), 0, s, (const bf16 *)embed, rows, hidden, vocab, x, err);
  else hipLaunchKernelGGL((embed_kernel<float>), dim3(n_rows), dim3(256), 0, s, (const float *)embed, rows, hidden, vocab, x, err);
  return hipGetLastError();
}

// Sum over the block in a fixed order (per-thread strided sums, then a fixed butterfly and a fixed
// cross-wave order), so results are reproducible run to run.
DF_DEVICE float block_sum(float v, float *red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

// One work-group per row: the row value is the fp32 residual plus the projection's K-range partial
// sums (added in range order), written back and optionally copied out as a feature tap; selected rows
// are then RMS-normalised.  Each of the NT threads keeps its VPT float4 slices (the row's, rounded up to
// a whole slice per thread) in registers between the passes; the partial ranges are read up to eight at
// a time with every load of a round issued before the first add, so that a row's loads overlap instead
// of waiting in turn.  The sum of squares is reduced in a fixed order.
template <typename T, int VPT, int NT>
__global__ __launch_bounds__(NT) void norm_kernel(NormArgs a) {
  __shared__ float red[NT / 64];
  const int r = blockIdx.x;
  const int j = r % a.stride - a.offset;
  const bool sel = a.out != nullptr && j >= 0 && j < a.take;
  if (!sel && !a.x && !a.feat) return;  // uniform over the work-group
  const int nv = a.hidden / 4;
  float4 *x = a.x ? reinterpret_cast<float4 *>(a.x + (size_t)r * a.ld_x) : nullptr;
  const float4 *p = a.part ? reinterpret_cast<const float4 *>(a.part + (size_t)r * a.ld_part) : nullptr;
  const size_t ps = (size_t)(a.part_stride / 4);
  // slice k of this thread: q = tid + NT k; past the row it reads slice 0 again and is never stored
  int qc[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int q = threadIdx.x + NT * k;
    qc[k] = q < nv ? q : 0;
  }
  float4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) v[k] = x ? x[qc[k]] : make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int kRound = 8;
  for (int sp = 0; sp < a.n_part; sp += kRound) {
    const int nr = min(kRound, a.n_part - sp);  // uniform
    float4 u[kRound][VPT];
#pragma unroll
    for (int i = 0; i < kRound; ++i)
      if (i < nr)
#pragma unroll
        for (int k = 0; k < VPT; ++k) u[i][k] = p[(sp + i) * ps + qc[k]];
#pragma unroll
    for (int i = 0; i < kRound; ++i)
      if (i < nr)
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
          v[k].x += u[i][k].x;
          v[k].y += u[i][k].y;
          v[k].z += u[i][k].z;
          v[k].w += u[i][k].w;
        }
  }
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int q = threadIdx.x + NT * k;
    if (q < nv) {
      if (x && a.n_part) x[q] = v[k];
      if (a.feat) {
        const size_t fi = (size_t)r * a.ld_feat + 4 * q;
        store_x((ActOf<T> *)a.feat, fi + 0, v[k].x);
        store_x((ActOf<T> *)a.feat, fi + 1, v[k].y);
        store_x((ActOf<T> *)a.feat, fi + 2, v[k].z);
        store_x((ActOf<T> *)a.feat, fi + 3, v[k].w);
      }
    } else {
      v[k] = make_float4(0.f, 0.f, 0.f, 0.f);  // outside the row: no part of the sum of squares
    }
  }
  if (!sel) return;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
  ss = block_sum(ss, red);
  const int o = (r / a.stride) * a.take + j;
  float rs = 1.0f / sqrtf(ss / (float)a.hidden + a.eps);
  if (a.ss_out) {  // deferred: the consumer applies 1/rms
    if (threadIdx.x == 0) a.ss_out[(size_t)o * a.ss_ld] = ss;
    rs = 1.f;
  }
  const size_t y = (size_t)o * a.ld_out;
  ActOf<T> *yh = (ActOf<T> *)a.out;
  const float4 *gv = reinterpret_cast<const float4 *>(a.gain);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int q = threadIdx.x + NT * k;
    if (q < nv) {
      const float4 gg = gv[q];
      store_x(yh, y + 4 * q + 0, v[k].x * rs * gg.x);
      store_x(yh, y + 4 * q + 1, v[k].y * rs * gg.y);
      store_x(yh, y + 4 * q + 2, v[k].z * rs * gg.z);
      store_x(yh, y + 4 * q + 3, v[k].w * rs * gg.w);
    }
  }
}

template <typename T>
static void launch_norm_t(const NormArgs &a, hipStream_t s) {
  // 512 threads a row (two waves per SIMD with one row per CU) while that leaves each at most 4 slices
  const int nv = a.hidden / 4;
  const dim3 g(a.n_rows);
  if (nv <= 512) hipLaunchKernelGGL((norm_kernel<T, 1, 512>), g, dim3(512), 0, s, a);
  else if (nv <= 1024) hipLaunchKernelGGL((norm_kernel<T, 2, 512>), g, dim3(512), 0, s, a);
  else if (nv <= 1536) hipLaunchKernelGGL((norm_kernel<T, 3, 512>), g, dim3(512), 0, s, a);
  else if (nv <= 2048) hipLaunchKernelGGL((norm_kernel<T, 4, 512>), g, dim3(512), 0, s, a);
  else hipLaunchKernelGGL((norm_kernel<T, 8, 512>), g, dim3(512), 0, s, a);
}

hipError_t launch_norm(const NormArgs &a, int dtype, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  if (a.hidden % 4 || a.hidden > 16384 || a.stride < 1 || (a.x && a.ld_x % 4) || (a.part && (a.ld_part % 4 || a.part_stride % 4)))
    return hipErrorInvalidValue;
  if (dtype == 0) launch_norm_t<bf16>(a, s);
  else launch_norm_t<float>(a, s);
  return hipGetLastError();
}

__global__ void zero_i32_kernel(int32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t *p, int32_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// Rotary table: the angle p * theta^(-2i/d) in fp64, then its cosine and sine rounded to fp32.
__global__ void rope_table_kernel(float2 *table, double theta, int half, int d, int n_pos) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n_pos * half) return;
  const int pos = e / half, i = e % half;
  const double inv = pow(theta, -2.0 * (double)i / (double)d);
  const double ang = (double)pos * inv;
  table[e] = make_float2((float)cos(ang), (float)sin(ang));
}

hipError_t launch_rope_table(float2 *table, float theta, int32_t head_dim, int32_t n_pos, hipStream_t s) {
  const int half = head_dim / 2, n = n_pos * half;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, table, (double)theta, half, head_dim,
                     n_pos);
  return hipGetLastError();
}

// ------------------------------------------------------------------ per-head q/k RMSNorm + RoPE + scatter
// One work-group per row and group of heads.  Lane i of a head's lane group holds elements i and
// i + d/2, exactly the pair that rotate-half RoPE rotates together.  T: the storage type of q and of
// the KV cache.
template <typename T>
__global__ __launch_bounds__(256) void qkv_post_kernel(QkvPostArgs a) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int d = a.kv.head_dim, half = d / 2;
  const int tpp = kWave / half;  // heads per wave
  const int sub = lane / half, i = lane % half;
  const int head_all = (blockIdx.y * 4 + wave) * tpp + sub;
  const bool live = head_all < a.total_heads;
  int si = 0, base = 0;
  if (live)
    while (si + 1 < a.nseg && head_all >= base + a.seg[si].heads) {
      base += a.seg[si].heads;
      ++si;
    }
  const PostSeg &sg = a.seg[si];
  const int head = head_all - base;
  const bool qk = sg.role == ROLE_Q || sg.role == ROLE_K;
  // every load that does not wait on another is issued first: the row's position, the norm gains and
  // the K-range partial sums (up to kR of them at once; they are added in range order below)
  const int pos = a.rows.pos[row];
  const float g1 = qk ? sg.gain[i] : 0.f, g2 = qk ? sg.gain[i + half] : 0.f;
  const float *src = a.src + (size_t)row * a.ld_src + (size_t)(live ? head_all : 0) * d;
  constexpr int kR = 8;
  float u1[kR], u2[kR];
#pragma unroll
  for (int sp = 0; sp < kR; ++sp)
    if (sp == 0 || sp < a.n_part) {
      u1[sp] = src[(size_t)sp * a.part_stride + i];
      u2[sp] = src[(size_t)sp * a.part_stride + i + half];
    }
  const float2 cr = (qk && pos >= 0 && pos < a.rope_rows) ? a.rope[(size_t)pos * half + i] : make_float2(1.f, 0.f);
  float v1 = u1[0], v2 = u2[0];
#pragma unroll
  for (int sp = 1; sp < kR; ++sp)
    if (sp < a.n_part) {
      v1 += u1[sp];
      v2 += u2[sp];
    }
  for (int sp = kR; sp < a.n_part; ++sp) {
    v1 += src[(size_t)sp * a.part_stride + i];
    v2 += src[(size_t)sp * a.part_stride + i + half];
  }
  if (qk) {
    float ss = v1 * v1 + v2 * v2;
    for (int off = half / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const float r = 1.0f / sqrtf(ss / (float)d + a.eps);
    v1 = v1 * r * g1;
    v2 = v2 * r * g2;
    // padding rows (a launch covering more rows than the call commits) are neither written nor checked
    if ((pos < 0 || pos >= a.rope_rows) && live && i == 0 && a.rows.valid[row]) raise_err(a.err, ERR_PAGE);
    const float cs = cr.x, sn = cr.y;
    const float o1 = v1 * cs - v2 * sn, o2 = v2 * cs + v1 * sn;
    v1 = o1;
    v2 = o2;
  }
  if (!live) return;
  if (sg.role == ROLE_Q) {
    T *q = (T *)sg.dst + (size_t)row * sg.ld_dst + head * d;
    Elem<T>::store(q + i, v1);
    Elem<T>::store(q + i + half, v2);
    return;
  }
  if (!a.rows.valid[row]) return;
  const int slot = a.rows.slot[row];
  const int pidx = pos / a.kv.page_tokens;
  const int page = (pidx < a.bt_stride) ? a.block_table[(size_t)slot * a.bt_stride + pidx] : -1;
  if (page < 0) {
    raise_err(a.err, ERR_PAGE);
    return;
  }
  const int tok = pos % a.kv.page_tokens;
  T *dst = (T *)sg.dst;
  if (sg.role == ROLE_K) {
    Elem<T>::store(dst + a.kv.k_index(page, head, tok, i), v1);
    Elem<T>::store(dst + a.kv.k_index(page, head, tok, i + half), v2);
  } else {
    Elem<T>::store(dst + a.kv.v_index(page, head, tok, i), v1);
    Elem<T>::store(dst + a.kv.v_index(page, head, tok, i + half), v2);
  }
}

hipError_t launch_qkv_post(const QkvPostArgs &a, int dtype, hipStream_t s) {
  if (a.n_rows == 0) return hipSuccess;
  const int tpp = kWave / (a.kv.head_dim / 2);
  dim3 grid(a.n_rows, (a.total_heads + 4 * tpp - 1) / (4 * tpp));
  // q and the KV cache hold the attention operands' storage type (fp16 for bf16 models)
  if (dtype == 0) hipLaunchKernelGGL((qkv_post_kernel<f16>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((qkv_post_kernel<float>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace df
