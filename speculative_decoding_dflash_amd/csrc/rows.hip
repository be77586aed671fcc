// Per-call row bookkeeping, embedding gather, RMSNorm and argmax (gfx950).
#include "kernels.h"

namespace df {

// One work-group.  Reads the slots' device state, fills the per-row arrays, then updates the state.
//   mode 0 (verify):  rows b*q_len + i at start + i (start = 0 for a new sequence, else seq_len);
//                     records the block as pending for the next accept.
//   mode 1 (inject):  rows b*q_len + i at inj_base + i, valid for i < inj_rows (the committed rows of
//                     the last verified block, whose features are to be injected); clears inj_rows.
//   mode 2 (draft):   rows b*q_len + i at seq_len + i; token = anchor for i = 0, mask id otherwise.
__global__ void prep_kernel(PrepArgs a) {
  __shared__ int s_start[64], s_lim[64], s_anchor[64];
  const int tid = threadIdx.x;
  if (tid < a.batch) {
    const SlotState &st = a.state[a.slots[tid]];
    if (a.mode == 0) {
      s_start[tid] = a.new_sequence ? 0 : st.seq_len;
      s_lim[tid] = a.q_len;
    } else if (a.mode == 1) {
      s_start[tid] = st.inj_base;
      s_lim[tid] = st.inj_rows;
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

// out row i = act(in row (i / take) * stride + offset + i % take, normalised) * gain
template <typename T>
__global__ void rmsnorm_kernel(const float *in, int ld_in, int take, int stride, int offset, const float *gain,
                               float eps, int hidden, T *out, int ld_out) {
  __shared__ float red[16];
  const int i = blockIdx.x;
  const int src = (i / take) * stride + offset + (i % take);
  const float *x = in + (size_t)src * ld_in;
  float ss = 0.f;
  for (int h = threadIdx.x; h < hidden; h += blockDim.x) ss += x[h] * x[h];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)hidden + eps);
  T *y = out + (size_t)i * ld_out;
  for (int h = threadIdx.x; h < hidden; h += blockDim.x) Elem<T>::store(y + h, x[h] * r * gain[h]);
}

hipError_t launch_rmsnorm(const float *in, int32_t ld_in, int32_t take, int32_t stride, int32_t offset, int32_t n_rows,
                          const float *gain, float eps, int32_t hidden, void *out, int32_t ld_out, int dtype,
                          hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL((rmsnorm_kernel<bf16>), dim3(n_rows), dim3(256), 0, s, in, ld_in, take, stride, offset, gain, eps,
                       hidden, (bf16 *)out, ld_out);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<float>), dim3(n_rows), dim3(256), 0, s, in, ld_in, take, stride, offset, gain, eps,
                       hidden, (float *)out, ld_out);
  return hipGetLastError();
}

// Row argmax; ties resolve to the lowest index.
__global__ void argmax_kernel(const float *logits, int vocab, int take, int stride, int offset, int32_t *out) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const float *z = logits + (size_t)blockIdx.x * vocab;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int j = threadIdx.x; j < vocab; j += blockDim.x) {
    const float v = z[j];
    if (v > best) {  // strided scan visits increasing j, so '>' keeps the lowest index per thread
      best = v;
      bi = j;
    }
  }
  sv[threadIdx.x] = best;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      const float v = sv[threadIdx.x + off];
      const int i = si[threadIdx.x + off];
      if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && i < si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  const int r = blockIdx.x;
  if (threadIdx.x == 0) out[(r / take) * stride + offset + r % take] = si[0] == 0x7fffffff ? 0 : si[0];
}

hipError_t launch_argmax(const float *logits, int32_t rows, int32_t vocab, int32_t take, int32_t stride, int32_t offset,
                         int32_t *out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(256), 0, s, logits, vocab, take, stride, offset, out);
  return hipGetLastError();
}

}  // namespace df
