// Candidate filter of the sampler, one work-group (1024 threads) per logits row (gfx950).
//
// For T > 0: s = z / T (IEEE division), keep the top_k scores ordered by (score desc, token id asc),
// softmax over them, keep the smallest prefix whose running sum reaches top_p (inclusive), and
// renormalise.  Sums run sequentially in sorted order in fp32 so that the accept / resample stage can
// reproduce them exactly.  For T = 0 the single candidate is the argmax (lowest id on ties).
//
// Top-k is an exact radix select over order-preserving 32-bit keys: three histogram passes (12, 12
// and 8 bits) find the k-th largest key; a fourth pass gathers every element whose key is at least
// that key (usually exactly k of them) into LDS, where a bitonic sort orders them by (key desc,
// id asc).  If ties at the threshold are so numerous that the gathered set would overflow LDS, an
// ordered scan takes the lowest-id ties instead.
#include "kernels.h"

namespace df {

constexpr int kFT = 1024;      // threads per row
constexpr int kGather = 1024;  // LDS capacity of the gathered set

DF_DEVICE uint32_t order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 are the same score
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DF_DEVICE float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

DF_DEVICE int block_excl_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < kFT / 64; ++w) {
    if (w < wave) before += wsum[w];
    all += wsum[w];
  }
  *total = all;
  return before + x - v;
}

// Among bins (descending), find the bin holding the need-th largest element; returns the bin and
// how many elements lie in higher bins.
DF_DEVICE void find_bin(const int *hist, int nbins, int need, int *wsum, int *s_bin, int *s_above) {
  const int per = nbins / kFT;  // bins per thread (>= 1)
  const int t = threadIdx.x;
  int local = 0;
  for (int j = 0; j < per; ++j) local += hist[nbins - 1 - (t * per + j)];
  int total;
  const int before = block_excl_scan(local, wsum, &total);
  if (before < need && need <= before + local) {
    int cum = before;
    for (int j = 0; j < per; ++j) {
      const int bin = nbins - 1 - (t * per + j);
      if (cum + hist[bin] >= need) {
        *s_bin = bin;
        *s_above = cum;
        break;
      }
      cum += hist[bin];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kFT) void filter_kernel(FilterArgs a) {
  __shared__ int hist[4096];
  __shared__ uint32_t gkey[kGather];
  __shared__ int gidx[kGather];
  __shared__ float ge[kMaxTopK];
  __shared__ int wsum[kFT / 64];
  __shared__ int s_bin, s_above, s_cnt, s_keep;
  __shared__ float s_kept;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int seq = row / a.rows_per_seq;
  const float T = a.temperature[seq];
  const float *z = a.logits + (size_t)row * a.vocab;
  int32_t *cid = a.cand_id + (size_t)row * kMaxTopK;
  float *cp = a.cand_p + (size_t)row * kMaxTopK;
  const int V = a.vocab;

  if (!(T > 0.0f)) {  // greedy: argmax, lowest id on ties
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int j = tid; j < V; j += kFT) {
      const float v = z[j];
      if (v > best) {
        best = v;
        bi = j;
      }
    }
    __shared__ float bv[kFT];
    __shared__ int bix[kFT];
    bv[tid] = best;
    bix[tid] = bi;
    __syncthreads();
    for (int off = kFT / 2; off > 0; off >>= 1) {
      if (tid < off) {
        const float v = bv[tid + off];
        const int i = bix[tid + off];
        if (v > bv[tid] || (v == bv[tid] && i < bix[tid])) {
          bv[tid] = v;
          bix[tid] = i;
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      cid[0] = bix[0] == 0x7fffffff ? 0 : bix[0];
      cp[0] = 1.0f;
      a.cand_n[row] = 1;
    }
    return;
  }

  const int K = min(a.top_k[seq], V);
  // ---- radix select of the K-th largest key
  uint32_t prefix = 0;
  int need = K;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int lvl = 0; lvl < 3; ++lvl) {
    const int nb = 1 << widths[lvl];
    for (int j = tid; j < nb; j += kFT) hist[j] = 0;
    __syncthreads();
    const int hi_shift = shifts[lvl] + widths[lvl];
    for (int j = tid; j < V; j += kFT) {
      const uint32_t k = order_key(__fdiv_rn(z[j], T));
      if (lvl == 0 || (k >> hi_shift) == prefix) atomicAdd(&hist[(k >> shifts[lvl]) & (nb - 1)], 1);
    }
    __syncthreads();
    if (nb >= kFT) {
      find_bin(hist, nb, need, wsum, &s_bin, &s_above);
    } else {
      if (tid == 0) {
        int cum = 0;
        for (int bin = nb - 1; bin >= 0; --bin) {
          if (cum + hist[bin] >= need) {
            s_bin = bin;
            s_above = cum;
            break;
          }
          cum += hist[bin];
        }
      }
      __syncthreads();
    }
    prefix = (prefix << widths[lvl]) | (uint32_t)s_bin;
    need -= s_above;
    __syncthreads();
  }
  const uint32_t kth = prefix;  // the K-th largest key; `need` elements equal to it are taken
  const int n_eq = hist[kth & 0xff];
  const int n_gt = K - need;

  // ---- gather
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  const bool all_fit = n_gt + n_eq <= kGather;
  for (int j = tid; j < V; j += kFT) {
    const uint32_t k = order_key(__fdiv_rn(z[j], T));
    if (k > kth || (all_fit && k == kth)) {
      const int slot = atomicAdd(&s_cnt, 1);
      gkey[slot] = k;
      gidx[slot] = j;
    }
  }
  __syncthreads();
  if (!all_fit) {
    // Ordered scan: each thread owns a contiguous chunk, so thread order is index order.
    const int chunk = (V + kFT - 1) / kFT;
    const int j0 = tid * chunk, j1 = min(V, j0 + chunk);
    int mine = 0;
    for (int j = j0; j < j1; ++j) mine += order_key(__fdiv_rn(z[j], T)) == kth;
    int total;
    int rank = block_excl_scan(mine, wsum, &total);
    for (int j = j0; j < j1 && rank < need; ++j) {
      if (order_key(__fdiv_rn(z[j], T)) == kth) {
        gkey[n_gt + rank] = kth;
        gidx[n_gt + rank] = j;
        ++rank;
      }
    }
    if (tid == 0) s_cnt = K;
    __syncthreads();
  }
  const int cnt = s_cnt;
  // ---- bitonic sort of the gathered set by (key desc, id asc); padding sorts last
  int n2 = 1;
  while (n2 < cnt) n2 <<= 1;
  for (int j = cnt + tid; j < n2; j += kFT) {
    gkey[j] = 0u;
    gidx[j] = 0x7fffffff;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kFT) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);  // first half of each merge runs in sorted ("greater first") order
        const uint32_t ka = gkey[lo], kb = gkey[hi];
        const int ia = gidx[lo], ib = gidx[hi];
        const bool a_first = (ka > kb) || (ka == kb && ia < ib);
        if (a_first != desc) {
          gkey[lo] = kb;
          gkey[hi] = ka;
          gidx[lo] = ib;
          gidx[hi] = ia;
        }
      }
      __syncthreads();
    }
  }
  // ---- softmax over the top K, nucleus cut, renormalisation
  const float s0 = key_value(gkey[0]);
  for (int j = tid; j < K; j += kFT) ge[j] = expf(key_value(gkey[j]) - s0);
  __syncthreads();
  if (tid == 0) {
    float Z = 0.f;
    for (int j = 0; j < K; ++j) Z = Z + ge[j];
    const float tp = a.top_p[seq];
    int keep = K;
    float acc = 0.f;
    if (tp < 1.0f) {
      for (int j = 0; j < K; ++j) {
        acc = acc + __fdiv_rn(ge[j], Z);
        if (acc >= tp) {
          keep = j + 1;
          break;
        }
      }
    }
    float kept = 0.f;
    for (int j = 0; j < keep; ++j) kept = kept + __fdiv_rn(ge[j], Z);
    s_keep = keep;
    s_kept = kept;
    for (int j = 0; j < K; ++j) ge[j] = __fdiv_rn(ge[j], Z);  // q_j
  }
  __syncthreads();
  const int keep = s_keep;
  for (int j = tid; j < kMaxTopK; j += kFT) {
    if (j < keep) {
      cid[j] = gidx[j];
      cp[j] = __fdiv_rn(ge[j], s_kept);
    } else {
      cid[j] = -1;
      cp[j] = 0.f;
    }
  }
  if (tid == 0) a.cand_n[row] = keep;
}

hipError_t launch_filter(const FilterArgs &a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(filter_kernel, dim3(a.rows), dim3(kFT), 0, s, a);
  return hipGetLastError();
}

__global__ void copy_cands_kernel(const int32_t *cid, const float *cp, const int32_t *cn, int rows, int32_t *oid, float *op) {
  const int r = blockIdx.x;
  const int n = cn[r];
  for (int j = threadIdx.x; j < kMaxTopK; j += blockDim.x) {
    const size_t i = (size_t)r * kMaxTopK + j;
    if (oid) oid[i] = j < n ? cid[i] : -1;
    if (op) op[i] = j < n ? cp[i] : 0.f;
  }
}

hipError_t launch_copy_cands(const int32_t *cid, const float *cp, const int32_t *cn, int32_t rows, int32_t *oid, float *op,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_cands_kernel, dim3(rows), dim3(256), 0, s, cid, cp, cn, rows, oid, op);
  return hipGetLastError();
}

}  // namespace df
