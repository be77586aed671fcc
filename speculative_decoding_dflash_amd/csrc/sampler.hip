// Candidate filter of the sampler and row argmax, in two stages (gfx950).
//
// For T > 0: s = z / T (IEEE division), keep the top_k scores ordered by (score desc, token id asc),
// softmax over them, keep the smallest prefix whose running sum reaches top_p (inclusive), and
// renormalise.  Sums run sequentially in sorted order in fp32 so that the accept / resample stage can
// reproduce them exactly.  For T = 0 the single candidate is the argmax (lowest id on ties).
//
// Stage 1: each row is cut into chunks of at most kChunkMax elements, one work-group per chunk.  The
// chunk's order-preserving 32-bit keys are cached in LDS and the chunk emits exactly its top k by
// (key desc, id asc).  For k <= 64 the keys at or above a lower bound of the k-th largest (from the
// waves' lane maxima) are usually few and are ranked directly; otherwise an 8-bit-digit radix select
// finds the k-th largest key and the chunk emits every key above it plus the lowest-id keys equal to
// it (ordered by an exclusive scan over contiguous sub-ranges).
// Stage 2: one work-group per row sorts the union of its chunks' candidates by (key desc, id asc) --
// the row's top k is the top k of that union -- and computes the distribution.
#include <algorithm>
#include <cstdlib>

#include "kernels.h"

namespace df {

constexpr int kChunkMax = 8192;  // elements per stage-1 chunk
constexpr int kMergeMax = kFilterScratch;  // stage-2 candidates per row (chunks * k)
constexpr int kT1 = 256;
constexpr int kT2 = 1024;

DF_DEVICE uint32_t order_key(float s) {
  if (s == 0.0f) s = 0.0f;  // -0 and +0 are the same score
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DF_DEVICE float key_value(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Exclusive prefix sum over the block (fixed order); *total receives the block sum.
template <int NT>
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
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) before += wsum[w];
    all += wsum[w];
  }
  *total = all;
  __syncthreads();
  return before + x - v;
}

// Histogram increment with wave-level aggregation: lanes holding the same bin add once per distinct
// bin, so a skewed digit (most logits share a sign and exponent) does not serialise the LDS atomics.
// Must be called by all lanes of the wave.
DF_DEVICE void hist_add(int *hist, int bin, bool active) {
  uint64_t todo = __ballot(active);
  while (todo) {
    const int leader = __ffsll((unsigned long long)todo) - 1;
    const int lbin = __shfl(bin, leader);
    const uint64_t same = __ballot(active && bin == lbin);
    if ((int)__lane_id() == leader) atomicAdd(&hist[lbin], (int)__popcll(same));
    todo &= ~same;
  }
}

DF_DEVICE void row_params(const FilterArgs &a, int row, float *T, int *K) {
  const int seq = row / a.rows_per_seq;
  const float t = a.temperature[seq];
  *T = t;
  *K = t > 0.0f ? a.top_k[seq] : 1;
}

__global__ __launch_bounds__(kT1) void topk_stage1(FilterArgs a) {
  __shared__ uint32_t skey[kChunkMax];
  __shared__ int hist[256];
  __shared__ int wsum[kT1 / 64];
  __shared__ int s_bin, s_above, s_cnt;
  const int row = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  float T;
  int K;
  row_params(a, row, &T, &K);
  const int c0 = chunk * a.chunk, c1 = min(a.vocab, c0 + a.chunk);
  const int n = c1 - c0;
  const float *z = a.logits + (size_t)row * a.vocab + c0;
  uint32_t tmax = 0u;  // the largest key of this thread's elements
  {
    // every load of the thread first (a loop of load -> convert -> LDS store waits for each load in
    // turn), then the keys
    constexpr int kPer = kChunkMax / kT1;
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tid + i * kT1;
      v[i] = z[j < n ? j : 0];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = tid + i * kT1;
      if (j < n) {
        const uint32_t k = order_key(T > 0.0f ? __fdiv_rn(v[i], T) : v[i]);
        skey[j] = k;
        tmax = max(tmax, k);
      }
    }
  }
  __syncthreads();
  const int Kc = min(K, n);
  uint32_t *okey = a.stage_key + ((size_t)row * a.n_chunks + chunk) * a.kmax;
  int32_t *oidx = a.stage_idx + ((size_t)row * a.n_chunks + chunk) * a.kmax;
  for (int j = Kc + tid; j < a.kmax; j += kT1) {
    okey[j] = 0u;
    oidx[j] = 0x7fffffff;
  }
  if (Kc == 1) {  // argmax: largest key, lowest index among equals
    uint32_t bk = 0u;
    int bi = 0x7fffffff;
    for (int j = tid; j < n; j += kT1)
      if (skey[j] > bk || bi == 0x7fffffff) {  // strided scan visits increasing j: '>' keeps the first
        bk = skey[j];
        bi = j;
      }
    __shared__ uint32_t rk[kT1];
    __shared__ int ri[kT1];
    rk[tid] = bk;
    ri[tid] = bi;
    __syncthreads();
    for (int off = kT1 / 2; off > 0; off >>= 1) {
      if (tid < off) {
        const uint32_t k2 = rk[tid + off];
        const int i2 = ri[tid + off];
        if (i2 != 0x7fffffff && (ri[tid] == 0x7fffffff || k2 > rk[tid] || (k2 == rk[tid] && i2 < ri[tid]))) {
          rk[tid] = k2;
          ri[tid] = i2;
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      okey[0] = rk[0];
      oidx[0] = c0 + ri[0];
    }
    return;
  }
  if (Kc <= 64) {
    // Candidates by a lower bound: the Kc largest lane maxima of a wave are Kc distinct keys of the
    // chunk, so the chunk's Kc-th largest key is at least the Kc-th largest lane maximum of every wave
    // (found by a bitonic sort across the wave, descending), hence at least tau, their largest.  Every
    // key of the chunk's top Kc is then >= tau; when few keys are, each is ranked directly by
    // (key desc, id asc) among them and the first Kc are emitted in rank order.
    __shared__ uint32_t s_tau[kT1 / 64];
    __shared__ uint32_t ck[kT1];
    __shared__ int ci[kT1];
    const int lane = tid & 63;
    uint32_t m = tmax;
    for (int k = 2; k <= 64; k <<= 1)
      for (int j = k >> 1; j > 0; j >>= 1) {
        const uint32_t o = __shfl_xor(m, j);
        m = (((lane & k) == 0) == ((lane & j) == 0)) ? max(m, o) : min(m, o);
      }
    const uint32_t tw = __shfl(m, Kc - 1);
    if (lane == 0) s_tau[tid >> 6] = tw;
    __syncthreads();
    uint32_t tau = s_tau[0];
#pragma unroll
    for (int w = 1; w < kT1 / 64; ++w) tau = max(tau, s_tau[w]);
    int mine = 0;
    for (int j = tid; j < n; j += kT1) mine += skey[j] >= tau;
    int total;
    int slot = block_excl_scan<kT1>(mine, wsum, &total);
    if (total <= kT1) {  // uniform; otherwise (many equal keys) the radix select below
      for (int j = tid; j < n; j += kT1)
        if (skey[j] >= tau) {
          ck[slot] = skey[j];
          ci[slot] = j;
          ++slot;
        }
      __syncthreads();
      if (tid < total) {
        const uint32_t k = ck[tid];
        const int ix = ci[tid];
        int rank = 0;
        for (int e = 0; e < total; ++e) {
          const uint32_t k2 = ck[e];
          rank += k2 > k || (k2 == k && ci[e] < ix);
        }
        if (rank < Kc) {
          okey[rank] = k;
          oidx[rank] = c0 + ix;
        }
      }
      return;
    }
  }
  // radix select of the Kc-th largest key, 8 bits at a time
  uint32_t prefix = 0;
  int need = Kc;
  for (int lvl = 0; lvl < 4; ++lvl) {
    const int shift = 24 - 8 * lvl;
    hist[tid] = 0;
    __syncthreads();
    for (int base = 0; base < n; base += kT1) {
      const int j = base + tid;
      const uint32_t k = j < n ? skey[j] : 0u;
      hist_add(hist, (int)((k >> shift) & 255), j < n && (lvl == 0 || (k >> (shift + 8)) == prefix));
    }
    __syncthreads();
    if (tid < 64) {
      // the bin holding the need-th largest key, found by wave 0: lane l holds bins 255 - 4l - i
      // (i = 0..3, descending), a prefix sum over the lanes gives the count of every higher bin, and
      // the one lane whose range reaches `need` walks its four bins (a single thread walking all 256
      // bins waited on each LDS read in turn)
      int c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * tid - i];
        sum += c[i];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (tid >= off) incl += y;
      }
      const int excl = incl - sum;
      if (excl < need && need <= incl) {
        int cum = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + c[i] >= need) {
            s_bin = 255 - 4 * tid - i;
            s_above = cum;
            break;
          }
          cum += c[i];
        }
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)s_bin;
    need -= s_above;
  }
  const uint32_t kth = prefix;  // `need` keys equal to it are taken, the lowest ids first
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  for (int j = tid; j < n; j += kT1) {
    if (skey[j] > kth) {
      const int slot = atomicAdd(&s_cnt, 1);
      okey[slot] = skey[j];
      oidx[slot] = c0 + j;
    }
  }
  const int n_gt = Kc - need;
  // ties in index order: contiguous sub-ranges per thread, exclusive scan of their counts
  const int per = (n + kT1 - 1) / kT1;
  const int j0 = tid * per, j1 = min(n, j0 + per);
  int mine = 0;
  for (int j = j0; j < j1; ++j) mine += skey[j] == kth;
  int total;
  int rank = block_excl_scan<kT1>(mine, wsum, &total);
  for (int j = j0; j < j1 && rank < need; ++j) {
    if (skey[j] == kth) {
      okey[n_gt + rank] = kth;
      oidx[n_gt + rank] = c0 + j;
      ++rank;
    }
  }
}

__global__ __launch_bounds__(kT2) void topk_stage2(FilterArgs a) {
  __shared__ uint32_t gkey[kMergeMax];
  __shared__ int gidx[kMergeMax];
  __shared__ float ge[kMaxTopK];
  __shared__ int s_keep;
  __shared__ float s_kept;
  const int row = blockIdx.x, tid = threadIdx.x;
  float T;
  int K;
  row_params(a, row, &T, &K);
  const int cnt = a.n_chunks * a.kmax;
  const uint32_t *ik = a.stage_key + (size_t)row * cnt;
  const int32_t *ii = a.stage_idx + (size_t)row * cnt;
  int n2 = 1;
  while (n2 < cnt) n2 <<= 1;
  for (int j = tid; j < n2; j += kT2) {
    gkey[j] = j < cnt ? ik[j] : 0u;
    gidx[j] = j < cnt ? ii[j] : 0x7fffffff;
  }
  __syncthreads();
  // bitonic sort by (key desc, id asc); padding (key 0, id max) sorts last
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n2 / 2; i += kT2) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0);
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
  if (a.argmax_out) {  // drafter argmax: the first entry
    if (tid == 0) a.argmax_out[(row / a.am_take) * a.am_stride + a.am_offset + row % a.am_take] = gidx[0];
    return;
  }
  int32_t *cid = a.cand_id + (size_t)row * kMaxTopK;
  if (a.cand_s) {  // score mode: the top K ids and their scores
    const int Kr = min(K, a.vocab);
    float *cs = a.cand_s + (size_t)row * kMaxTopK;
    for (int j = tid; j < Kr; j += kT2) {
      cid[j] = gidx[j];
      cs[j] = key_value(gkey[j]);
    }
    return;
  }
  float *cp = a.cand_p + (size_t)row * kMaxTopK;
  if (!(T > 0.0f)) {
    for (int j = tid; j < kMaxTopK; j += kT2) {
      cid[j] = j == 0 ? gidx[0] : -1;
      cp[j] = j == 0 ? 1.0f : 0.f;
    }
    if (tid == 0) a.cand_n[row] = 1;
    return;
  }
  const int Kr = min(K, a.vocab);
  const float s0 = key_value(gkey[0]);
  for (int j = tid; j < Kr; j += kT2) ge[j] = expf(key_value(gkey[j]) - s0);
  __syncthreads();
  if (tid == 0) {
    float Z = 0.f;
    for (int j = 0; j < Kr; ++j) Z = Z + ge[j];
    const float tp = a.top_p[row / a.rows_per_seq];
    int keep = Kr;
    float acc = 0.f;
    if (tp < 1.0f) {
      for (int j = 0; j < Kr; ++j) {
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
    for (int j = 0; j < Kr; ++j) ge[j] = __fdiv_rn(ge[j], Z);  // q_j
  }
  __syncthreads();
  const int keep = s_keep;
  for (int j = tid; j < kMaxTopK; j += kT2) {
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

// Chunking of a row: enough chunks to spread the row over the device, few enough that the stage-2
// union (chunks * kmax) fits in LDS.
void filter_plan(FilterArgs &a, int kmax) {
  a.kmax = kmax;
  static const int env_chunk = getenv("DFLASH_TOPK_CHUNK") ? atoi(getenv("DFLASH_TOPK_CHUNK")) : 0;
  const int target = env_chunk >= 256 && env_chunk <= kChunkMax ? env_chunk : 4000;  // elements per chunk
  int chunks = (a.vocab + target - 1) / target;
  chunks = std::max(1, std::min(chunks, kMergeMax / kmax));
  int chunk = (a.vocab + chunks - 1) / chunks;
  a.chunk = chunk;
  a.n_chunks = (a.vocab + chunk - 1) / chunk;
}

hipError_t launch_filter(const FilterArgs &a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (a.chunk > kChunkMax || a.n_chunks * a.kmax > kMergeMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_stage1, dim3(a.rows, a.n_chunks), dim3(kT1), 0, s, a);
  hipLaunchKernelGGL(topk_stage2, dim3(a.rows), dim3(kT2), 0, s, a);
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
