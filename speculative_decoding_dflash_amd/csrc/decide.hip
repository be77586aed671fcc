// Accept / resample and commit, one thread per request (gfx950).  Built with -ffp-contract=off: the
// stage uses only fp32 additions, one multiplication and comparisons, in a fixed order, so that its
// decisions are reproducible exactly from the candidate probabilities.
//
// Rule (lossless for deterministic drafts): draft x at position t is accepted iff u_acc(t) < p(x);
// at the first rejection the token is drawn by inverse CDF from p with x removed (threshold
// u_smp(t) * S, S = sum of the remaining probabilities in candidate order); if every draft is
// accepted the bonus token at the next position is drawn from the last row.  Uniforms are Philox4x64
// with 10 rounds (Salmon et al., SC 2011), key (seed, 0), counter (t, slot, 0, 0), using the top 24
// bits of words 0 (u_acc) and 1 (u_smp).
// Stochastic drafts (x drawn from the drafter's own distribution q, with the top 24 bits of word 0
// of counter (t, slot, 1, 0)): x is accepted iff u_acc(t) * q(x) < p(x), i.e. with probability
// min(1, p(x)/q(x)); the first rejected position is drawn from max(0, p - q) over p's candidates
// (from p should that vanish).  q a point mass at x gives exactly the deterministic rule.
#include "kernels.h"

namespace df {

struct U4 {
  uint64_t w[4];
};

DF_DEVICE U4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  U4 u;
  u.w[0] = c0;
  u.w[1] = c1;
  u.w[2] = c2;
  u.w[3] = c3;
  return u;
}

DF_DEVICE float u24(uint64_t w) { return (float)(uint32_t)(w >> 40) * 5.9604644775390625e-08f; }

// Inverse CDF over candidates (ids, p, n) with optional exclusion.
DF_DEVICE int inverse_cdf(const int32_t *ids, const float *p, int n, float u, int exclude) {
  float total = 0.f;
  for (int j = 0; j < n; ++j)
    if (ids[j] != exclude) total = total + p[j];
  const float thr = u * total;
  float acc = 0.f;
  int last = -1;
  for (int j = 0; j < n; ++j) {
    if (ids[j] == exclude) continue;
    acc = acc + p[j];
    if (thr < acc) return ids[j];
    if (p[j] > 0.f) last = ids[j];
  }
  return last;
}

// q(y) from a candidate row padded with -1
DF_DEVICE float q_of(const int32_t *qi, const float *qp, int y) {
  float v = 0.f;
  for (int j = 0; j < kMaxTopK && qi[j] >= 0; ++j)
    if (qi[j] == y) v = qp[j];
  return v;
}

// max(0, p - q) of candidate j
DF_DEVICE float resid(const int32_t *ids, const float *p, int j, const int32_t *qi, const float *qp) {
  const float d = p[j] - q_of(qi, qp, ids[j]);
  return d > 0.f ? d : 0.f;
}

// Inverse CDF over the residual max(0, p - q) (candidate order); -1 if the residual is all zero.
DF_DEVICE int inverse_cdf_resid(const int32_t *ids, const float *p, int n, const int32_t *qi, const float *qp, float u) {
  float total = 0.f;
  for (int j = 0; j < n; ++j) total = total + resid(ids, p, j, qi, qp);
  if (!(total > 0.f)) return -1;
  const float thr = u * total;
  float acc = 0.f;
  int last = -1;
  for (int j = 0; j < n; ++j) {
    const float r = resid(ids, p, j, qi, qp);
    acc = acc + r;
    if (thr < acc) return ids[j];
    if (r > 0.f) last = ids[j];
  }
  return last;
}

__global__ void decide_kernel(DecideArgs a) {
  const int b = threadIdx.x;
  if (b >= a.batch) return;
  const int slot = a.slots[b];
  SlotState &st = a.state[slot];
  const int nd = a.n_draft;
  const int anchor_pos = st.pend_start + st.pend_qlen - 1 - nd;
  int *out = a.out + (size_t)b * (nd + 1);
  int tau = 0;
  bool rejected = false;
  for (int i = 1; i <= nd; ++i) {
    const int row = b * (nd + 1) + (i - 1);
    const int32_t *ids = a.cand_id + (size_t)row * kMaxTopK;
    const float *p = a.cand_p + (size_t)row * kMaxTopK;
    const int n = a.cand_n[row];
    const int d = a.block[(size_t)b * (nd + 1) + i];
    const U4 w = philox4x64_10((uint64_t)(anchor_pos + i), (uint64_t)slot, 0, 0, a.seed[b], 0);
    float pd = 0.f;
    for (int j = 0; j < n; ++j)
      if (ids[j] == d) pd = p[j];
    if (!a.q_id) {
      if (u24(w.w[0]) < pd) {
        out[tau++] = d;
        continue;
      }
      out[tau++] = inverse_cdf(ids, p, n, u24(w.w[1]), d);
    } else {
      const int32_t *qi = a.q_id + (size_t)(b * nd + i - 1) * kMaxTopK;
      const float *qp = a.q_p + (size_t)(b * nd + i - 1) * kMaxTopK;
      if (u24(w.w[0]) * q_of(qi, qp, d) < pd) {
        out[tau++] = d;
        continue;
      }
      const int y = inverse_cdf_resid(ids, p, n, qi, qp, u24(w.w[1]));
      out[tau++] = y >= 0 ? y : inverse_cdf(ids, p, n, u24(w.w[1]), -1);
    }
    rejected = true;
    break;
  }
  if (!rejected) {
    const int row = b * (nd + 1) + nd;
    const U4 w = philox4x64_10((uint64_t)(anchor_pos + nd + 1), (uint64_t)slot, 0, 0, a.seed[b], 0);
    out[tau++] = inverse_cdf(a.cand_id + (size_t)row * kMaxTopK, a.cand_p + (size_t)row * kMaxTopK, a.cand_n[row],
                             u24(w.w[1]), -1);
  }
  for (int j = tau; j <= nd; ++j) out[j] = -1;
  a.n_out[b] = tau;
  const int committed = st.pend_qlen - 1 - nd + tau;
  st.inj_base = st.pend_start;
  st.inj_rows = committed;
  st.seq_len = st.pend_start + committed;
  st.anchor = out[tau - 1];
  if (out[tau - 1] < 0) raise_err(a.err, ERR_STATE);
}

__global__ void draft_sample_kernel(DraftSampleArgs a) {
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= a.batch * a.nd) return;
  const int b = row / a.nd, i = row % a.nd + 1;
  const int slot = a.slots[b];
  const int t = a.state[slot].seq_len + i;
  int32_t *ids = a.q_id + (size_t)row * kMaxTopK;
  float *p = a.q_p + (size_t)row * kMaxTopK;
  const int n = a.q_n[row];
  const U4 w = philox4x64_10((uint64_t)t, (uint64_t)slot, 1, 0, a.seed[b], 0);
  a.out[(size_t)b * a.block + i] = inverse_cdf(ids, p, n, u24(w.w[0]), -1);
  for (int j = n; j < kMaxTopK; ++j) {
    ids[j] = -1;
    p[j] = 0.f;
  }
}

hipError_t launch_draft_sample(const DraftSampleArgs &a, hipStream_t s) {
  const int rows = a.batch * a.nd;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(draft_sample_kernel, dim3((rows + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decide(const DecideArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(decide_kernel, dim3(1), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace df
