// Per-call row bookkeeping, embedding gather, RMSNorm and argmax (gfx950).
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
// are then RMS-normalised.  Every thread keeps its float4 slices in registers between the passes, and
// the sum of squares is reduced in a fixed order.
template <typename T, int VPT>
__global__ __launch_bounds__(256) void norm_kernel(NormArgs a) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int j = r % a.stride - a.offset;
  const bool sel = a.out != nullptr && j >= 0 && j < a.take;
  if (!sel && !a.x && !a.feat) return;  // uniform over the work-group
  const int nv = a.hidden / 4;
  float4 *x = a.x ? reinterpret_cast<float4 *>(a.x + (size_t)r * a.ld_x) : nullptr;
  const float4 *p = a.part ? reinterpret_cast<const float4 *>(a.part + (size_t)r * a.ld_part) : nullptr;
  const size_t ps = (size_t)(a.part_stride / 4);
  float4 v[VPT];
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    const int q = threadIdx.x + 256 * k;
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
    if (q < nv) {
      if (x) t = x[q];
      for (int sp = 0; sp < a.n_part; ++sp) {  // K-range partial sums, in order
        const float4 u = p[sp * ps + q];
        t.x += u.x;
        t.y += u.y;
        t.z += u.z;
        t.w += u.w;
      }
      if (x && a.n_part) x[q] = t;
      if (a.feat) {
        const size_t fi = (size_t)r * a.ld_feat + 4 * q;
        store_x((ActOf<T> *)a.feat, fi + 0, t.x);
        store_x((ActOf<T> *)a.feat, fi + 1, t.y);
        store_x((ActOf<T> *)a.feat, fi + 2, t.z);
        store_x((ActOf<T> *)a.feat, fi + 3, t.w);
      }
    }
    v[k] = t;
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
    const int q = threadIdx.x + 256 * k;
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
  const int vpt = (a.hidden / 4 + 255) / 256;
  dim3 g(a.n_rows), b(256);
  if (vpt <= 1) hipLaunchKernelGGL((norm_kernel<T, 1>), g, b, 0, s, a);
  else if (vpt <= 2) hipLaunchKernelGGL((norm_kernel<T, 2>), g, b, 0, s, a);
  else if (vpt <= 4) hipLaunchKernelGGL((norm_kernel<T, 4>), g, b, 0, s, a);
  else if (vpt <= 8) hipLaunchKernelGGL((norm_kernel<T, 8>), g, b, 0, s, a);
  else hipLaunchKernelGGL((norm_kernel<T, 16>), g, b, 0, s, a);
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

}  // namespace df
