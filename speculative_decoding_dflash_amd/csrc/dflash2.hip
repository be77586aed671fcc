// DFlash2 drafter variants ([P3] "DFlash 2 的三个设计", which gives their configuration values only;
// definitions as read there): the dynamic convolution along the block that feeds each drafter layer's
// q/k/v projection, and the path selector that replaces argmax drafting.
//
// Dynamic convolution: for block row i (position i of its request's block) and channel c of group
// g = c / group, y_i[c] = sum_{t < taps, i - t >= 0} a_i[g][t] x_{i-t}[c], where x is the layer's
// normalised attention input and a_i[g][.] = softmax_t(u_i[g * taps + t]) with u_i = W_conv x_i (that
// projection runs on the GEMM kernels first).  One work-group per row.
//
// Selector: the K best candidates of every draft row (logit desc, id asc; the sampler's top-k stage),
// their shared-embedding rows gathered (with the anchor's) and projected by the rank-r factors U and V
// (a GEMM), transitions T(a -> b) = (U E[a]) . (V E[b]) / sqrt(r), then per request a Viterbi pass over
// the block: d_1(k) = z_1[k] + T(anchor -> c_1[k]); d_i(k) = z_i[k] + max_k' (d_{i-1}(k') + T(c_{i-1}[k']
// -> c_i[k])) in fp32, in that order (running score + transition, max, + emission); the last row's best
// and every predecessor that attained a max, the lowest index among equal values.
#include "kernels.h"

namespace df {

// 1 / rms of row r of a deferred RMSNorm (ss_n partial sums of squares at ss[r * ss_ld ..]), or 1.
DF_DEVICE float conv_rstd(const ConvArgs &a, int r) {
  if (!a.ss) return 1.f;
  float tot = 0.f;
  for (int p = 0; p < a.ss_n; p += 4) {
    const float *q = a.ss + (size_t)r * a.ss_ld + p;
    tot += (q[0] + (p + 1 < a.ss_n ? q[1] : 0.f)) + (p + 2 < a.ss_n ? q[2] : 0.f) + (p + 3 < a.ss_n ? q[3] : 0.f);
  }
  return 1.0f / sqrtf(tot / (float)a.hidden + a.eps);
}

template <typename A>
__global__ __launch_bounds__(256) void dyn_conv_kernel(ConvArgs a) {
  const int r = blockIdx.x, i = r % a.block;
  __shared__ float s_rstd[kConvMaxTaps];
  if (threadIdx.x < a.taps) s_rstd[threadIdx.x] = threadIdx.x <= i ? conv_rstd(a, r - threadIdx.x) : 0.f;
  __syncthreads();
  const A *x = (const A *)a.x;
  const float *u = a.u + (size_t)r * a.ld_u;
  for (int c = threadIdx.x; c < a.hidden; c += 256) {
    const int g = c / a.group;
    float m = u[g * a.taps];
    for (int t = 1; t < a.taps; ++t) m = fmaxf(m, u[g * a.taps + t]);
    float e[kConvMaxTaps], z = 0.f;
    for (int t = 0; t < a.taps; ++t) {
      e[t] = expf(u[g * a.taps + t] - m);
      z += e[t];
    }
    float y = 0.f;
    for (int t = 0; t < a.taps && t <= i; ++t)
      y += (e[t] / z) * (Elem<A>::load(x + (size_t)(r - t) * a.ldx + c) * s_rstd[t]);
    store_x((A *)a.out, (size_t)r * a.ld_out + c, y);
  }
}

hipError_t launch_dyn_conv(const ConvArgs &a, int dtype, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.taps < 1 || a.taps > kConvMaxTaps || a.group < 1 || a.hidden % a.group || a.block < 1) return hipErrorInvalidValue;
  if (dtype == 0) hipLaunchKernelGGL(dyn_conv_kernel<f16>, dim3(a.rows), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dyn_conv_kernel<float>, dim3(a.rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Row j of request b's selector input: j = 0 the anchor, j = 1 + (i - 1) K + k candidate k of draft
// row i; the embedding row in the activation type.  One work-group per row.
template <typename T>
__global__ __launch_bounds__(256) void sel_gather_kernel(SelArgs a) {
  const int per = 1 + a.nd * a.K;
  const int b = blockIdx.x / per, j = blockIdx.x % per;
  int id = j == 0 ? a.block[b * a.block_stride] : a.cand_id[(size_t)(b * a.nd + (j - 1) / a.K) * a.cand_ld + (j - 1) % a.K];
  if (id < 0 || id >= a.vocab) id = 0;  // a row with fewer candidates (vocabulary smaller than K) repeats id 0
  const T *e = (const T *)a.embed + (size_t)id * a.hidden;
  ActOf<T> *o = (ActOf<T> *)a.x + (size_t)blockIdx.x * a.hidden;
  for (int c = threadIdx.x; c < a.hidden; c += 256) store_x(o, c, Elem<T>::load(e + c));
}

// One work-group per request and draft row after row: the row's source and destination factors staged
// in LDS (rows padded by one float so that the 16 destinations of a wave sit in different banks), its
// transitions computed one per thread, then one Viterbi step by one wave (lane k: candidate k).
constexpr int kSelRankMax = 512;
__global__ __launch_bounds__(256) void sel_viterbi_kernel(SelArgs a) {
  __shared__ float s_t[kSelMaxK * kSelMaxK];
  __shared__ float s_phi[kSelMaxK * (kSelRankMax + 1)], s_psi[kSelMaxK * (kSelRankMax + 1)];
  __shared__ float s_delta[kSelMaxK];
  __shared__ int8_t s_back[kSelMaxSteps][kSelMaxK];
  const int b = blockIdx.x, tid = threadIdx.x, K = a.K, r = a.rank;
  const int per = 1 + a.nd * K;
  const float *y = a.proj + (size_t)b * per * a.ld_proj;  // [per][2 r]: phi then psi
  for (int i = 1; i <= a.nd; ++i) {
    const int nsrc = i == 1 ? 1 : K;
    const int src0 = i == 1 ? 0 : 1 + (i - 2) * K, dst0 = 1 + (i - 1) * K;
    const int rp = r + 1;
    for (int e = tid; e < nsrc * r; e += 256) s_phi[(e / r) * rp + e % r] = y[(size_t)(src0 + e / r) * a.ld_proj + e % r];
    for (int e = tid; e < K * r; e += 256) s_psi[(e / r) * rp + e % r] = y[(size_t)(dst0 + e / r) * a.ld_proj + r + e % r];
    __syncthreads();
    // T[k'][k] = phi(src k') . psi(dst k) / sqrt(r), summed in order over the rank
    for (int e = tid; e < K * K; e += 256) {
      const int kp = e / K, k = e % K;
      float t = 0.f;
      if (kp < nsrc) {
        const float *ph = s_phi + kp * rp, *ps = s_psi + k * rp;
        for (int q = 0; q < r; ++q) t += ph[q] * ps[q];
        t *= a.inv_sqrt_r;
      }
      s_t[e] = t;
      a.trans[((size_t)(b * a.nd + i - 1) * K + kp) * K + k] = t;
    }
    __syncthreads();
    if (tid < K) {
      const float z = a.cand_s[(size_t)(b * a.nd + i - 1) * a.cand_ld + tid];
      float best;
      int arg = 0;
      if (i == 1) {
        best = s_t[tid];  // d_1(k) = z_1[k] + T(anchor -> c_1[k])
      } else {
        best = s_delta[0] + s_t[tid];
        for (int kp = 1; kp < K; ++kp) {
          const float v = s_delta[kp] + s_t[kp * K + tid];
          if (v > best) {
            best = v;
            arg = kp;
          }
        }
      }
      s_back[i - 1][tid] = (int8_t)arg;
      __builtin_amdgcn_wave_barrier();
      s_delta[tid] = best + z;
    }
    __syncthreads();
  }
  if (tid == 0) {
    int k = 0;
    for (int q = 1; q < K; ++q)
      if (s_delta[q] > s_delta[k]) k = q;
    for (int i = a.nd; i >= 1; --i) {
      a.out[b * a.block_stride + i] = a.cand_id[(size_t)(b * a.nd + i - 1) * a.cand_ld + k];
      k = s_back[i - 1][k];
    }
  }
}

hipError_t launch_sel_gather(const SelArgs &a, int dtype, hipStream_t s) {
  if (a.K < 1 || a.K > kSelMaxK || a.nd < 1 || a.nd > kSelMaxSteps) return hipErrorInvalidValue;
  const dim3 grid(a.batch * (1 + a.nd * a.K));
  if (dtype == 0) hipLaunchKernelGGL(sel_gather_kernel<bf16>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(sel_gather_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sel_viterbi(const SelArgs &a, hipStream_t s) {
  if (a.K < 1 || a.K > kSelMaxK || a.nd < 1 || a.nd > kSelMaxSteps || a.rank > kSelRankMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sel_viterbi_kernel, dim3(a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace df
