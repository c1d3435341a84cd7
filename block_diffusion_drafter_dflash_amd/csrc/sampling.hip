// Sampling kernels (DFlash explainer, section 4, "Sampling decoding"): inverse-CDF
// draws from tempered softmax rows, and speculative-sampling acceptance of a drafted
// block with the residual max(p_target - p_draft, 0) at the first rejection.
//
// A row of V logits is handled by one workgroup of kRowThreads threads. Thread t owns
// the contiguous ids [t * C, (t + 1) * C) (C = ceil(V / kRowThreads)). The weight of id
// k is w_k = exp2((l_k - max) * log2(e) / T) in fp32; chunk sums, their prefix scan
// and the draw are float64. A draw with uniform u returns the smallest id whose
// running sum exceeds u times the row total (ids in ascending order), and never an id
// of zero weight. Every reduction has a fixed order, so results are deterministic.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;

namespace {

// Workgroup maximum of one float per thread (every thread gets it).
__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < kRowWaves; ++i) r = fmaxf(r, sh[i]);
  return r;
}

// Exclusive prefix of one double per thread in thread order, plus the total. The
// waves' sums are combined in wave order; within a wave the scan is a fixed tree.
__device__ __forceinline__ double block_exclusive_scan(double v, double* sh, double& total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  double incl = v;
  for (int m = 1; m < kWave; m <<= 1) {
    const double o = __shfl_up(incl, m, kWave);
    if (lane >= m) incl += o;
  }
  __syncthreads();
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
  for (int i = 0; i < kRowWaves; ++i) {
    if (i < w) base += sh[i];
    tot += sh[i];
  }
  total = tot;
  return base + incl - v;
}

struct RowChunk {
  int k0, k1;
};
__device__ __forceinline__ RowChunk row_chunk(int V) {
  const int C = (V + kRowThreads - 1) / kRowThreads;
  const int k0 = min((int)threadIdx.x * C, V), k1 = min(k0 + C, V);
  return {k0, k1};
}

// The draw over weights w(k) (a functor, identical values on every call) given each
// thread's chunk sum and the workgroup's exclusive prefix and total. Returns the id
// on every thread.
template <typename Wf>
__device__ int block_draw(const Wf& w, RowChunk ch, double csum, double prefix, double total, double u,
                          int* sh_tok) {
  const double target = u * total;
  __syncthreads();
  if (threadIdx.x == 0) *sh_tok = 0x7fffffff;
  __syncthreads();
  // The owning chunk: prefix <= target < prefix + csum, with positive mass. Should
  // rounding let two neighbouring chunks both claim, the lower id wins.
  if (csum > 0.0 && prefix <= target && target < prefix + csum) {
    double run = prefix;
    int last = -1, tok = -1;
    for (int k = ch.k0; k < ch.k1; ++k) {
      const double x = w(k);
      if (x > 0.0) last = k;
      run += x;
      if (run > target && x > 0.0) {
        tok = k;
        break;
      }
    }
    atomicMin(sh_tok, tok >= 0 ? tok : last);   // LDS atomic; rounding may leave the crossing past the chunk
  }
  __syncthreads();
  int tok = *sh_tok;
  if (tok == 0x7fffffff) {
    __syncthreads();
    if (threadIdx.x == 0) *sh_tok = -1;
    // target at or past the total: the last id of positive weight
    __syncthreads();
    const int me = csum > 0.0 ? (int)threadIdx.x : -1;
    int best = me;
    for (int m = 1; m < kWave; m <<= 1) best = max(best, __shfl_xor(best, m, kWave));
    if ((threadIdx.x & 63) == 0) atomicMax(sh_tok, best);   // LDS atomic
    __syncthreads();
    const int owner = *sh_tok;
    __syncthreads();
    if ((int)threadIdx.x == owner) {
      int last = -1;
      for (int k = ch.k0; k < ch.k1; ++k)
        if (w(k) > 0.0) last = k;
      *sh_tok = last;
    }
    __syncthreads();
    tok = *sh_tok;
  }
  return tok;
}

}  // namespace

// One tempered softmax row: (max, total weight) as two doubles.
__global__ __launch_bounds__(kRowThreads) void k_row_stats(const float* logits, int V, int64_t ld, float scale,
                                                           double* stats) {
  __shared__ float shf[kRowWaves];
  __shared__ double shd[kRowWaves];
  const float* row = logits + (int64_t)blockIdx.x * ld;
  const RowChunk ch = row_chunk(V);
  float m = -INFINITY;
  for (int k = ch.k0; k < ch.k1; ++k) m = fmaxf(m, row[k]);
  m = block_max(m, shf);
  double cs = 0.0;
  for (int k = ch.k0; k < ch.k1; ++k) cs += (double)exp2f((row[k] - m) * scale);
  double total;
  (void)block_exclusive_scan(cs, shd, total);
  if (threadIdx.x == 0) {
    stats[2 * blockIdx.x] = (double)m;
    stats[2 * blockIdx.x + 1] = total;
  }
}

// One draw per row from softmax(row / T) with uniform u[row].
__global__ __launch_bounds__(kRowThreads) void k_sample_rows(const SampleParams p) {
  __shared__ float shf[kRowWaves];
  __shared__ double shd[kRowWaves];
  __shared__ int sh_tok;
  const float* row = p.logits + (int64_t)blockIdx.x * p.ld;
  const RowChunk ch = row_chunk(p.V);
  float m = -INFINITY;
  for (int k = ch.k0; k < ch.k1; ++k) m = fmaxf(m, row[k]);
  m = block_max(m, shf);
  const float sc = p.scale;
  auto w = [&](int k) { return (double)exp2f((row[k] - m) * sc); };
  double cs = 0.0;
  for (int k = ch.k0; k < ch.k1; ++k) cs += w(k);
  double total;
  const double prefix = block_exclusive_scan(cs, shd, total);
  const int tok = block_draw(w, ch, cs, prefix, total, (double)p.u[blockIdx.x], &sh_tok);
  if (threadIdx.x == 0) {
    p.token_out[blockIdx.x] = tok;
    if (p.prob_out) p.prob_out[blockIdx.x] = (float)(w(tok) / total);
  }
}

// Speculative-sampling acceptance of one stream's drafted block (one workgroup).
__global__ __launch_bounds__(kRowThreads) void k_verify_sampling(const SpecVerifyParams p) {
  __shared__ double shd[kRowWaves];
  __shared__ int sh_tok, sh_a;
  const int s = blockIdx.x, B = p.B, V = p.V;
  const float sc = p.scale;
  const int* d = p.draft + (int64_t)s * (B - 1);
  const float* dl = p.draft_logits + (int64_t)s * (B - 1) * p.ld;
  const float* tl = p.target_logits + (int64_t)s * B * p.ld;
  const double* ds = p.draft_stats + (int64_t)s * (B - 1) * 2;
  const double* ts = p.target_stats + (int64_t)s * B * 2;

  // accepted length: d_{j+1} is kept while u * p_draft(d) < p_target(d)
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < B - 1) {
      const int tok = d[a];
      if (tok < 0 || tok >= V) break;   // an id outside the vocabulary is rejected
      const float* drow = dl + (int64_t)a * p.ld;
      const float* trow = tl + (int64_t)a * p.ld;
      const double pd = (double)exp2f((drow[tok] - (float)ds[2 * a]) * sc) / ds[2 * a + 1];
      const double pt = (double)exp2f((trow[tok] - (float)ts[2 * a]) * sc) / ts[2 * a + 1];
      if (!((double)p.u_accept[(int64_t)s * (B - 1) + a] * pd < pt)) break;
      ++a;
    }
    sh_a = a;
  }
  __syncthreads();
  const int a = sh_a;
  const RowChunk ch = row_chunk(V);
  const double u = (double)p.u_sample[s];
  const float* trow = tl + (int64_t)a * p.ld;
  const float tm = (float)ts[2 * a];
  const double tz = ts[2 * a + 1];
  auto wt = [&](int k) { return (double)exp2f((trow[k] - tm) * sc) / tz; };
  int tok;
  if (a < B - 1) {
    // residual max(q - p, 0) at the rejected position; q itself if it has no mass
    const float* drow = dl + (int64_t)a * p.ld;
    const float dm = (float)ds[2 * a];
    const double dz = ds[2 * a + 1];
    auto wr = [&](int k) {
      const double r = wt(k) - (double)exp2f((drow[k] - dm) * sc) / dz;
      return r > 0.0 ? r : 0.0;
    };
    double cs = 0.0;
    for (int k = ch.k0; k < ch.k1; ++k) cs += wr(k);
    double total;
    const double prefix = block_exclusive_scan(cs, shd, total);
    if (total > 0.0) {
      tok = block_draw(wr, ch, cs, prefix, total, u, &sh_tok);
    } else {
      double cq = 0.0;
      for (int k = ch.k0; k < ch.k1; ++k) cq += wt(k);
      double tq;
      const double pq = block_exclusive_scan(cq, shd, tq);
      tok = block_draw(wt, ch, cq, pq, tq, u, &sh_tok);
    }
  } else {
    double cq = 0.0;
    for (int k = ch.k0; k < ch.k1; ++k) cq += wt(k);
    double tq;
    const double pq = block_exclusive_scan(cq, shd, tq);
    tok = block_draw(wt, ch, cq, pq, tq, u, &sh_tok);
  }
  if ((int)threadIdx.x < B) {
    const int j = threadIdx.x;
    p.committed[(int64_t)s * B + j] = j < a ? d[j] : (j == a ? tok : -1);
  }
  if (threadIdx.x == 0) {
    p.accept[s] = a;
    p.token[s] = tok;
    if (p.ctx_len) p.ctx_len[s] += a + 1;
  }
}

hipError_t launch_row_stats(const float* logits, int rows, int V, int64_t ld, float scale, double* stats,
                            hipStream_t st) {
  (void)launch_k(k_row_stats, dim3(rows), dim3(kRowThreads), st, logits, V, ld, scale, stats);
  return hipGetLastError();
}

hipError_t launch_sample_rows(const SampleParams& p, hipStream_t st) {
  (void)launch_k(k_sample_rows, dim3(p.rows), dim3(kRowThreads), st, p);
  return hipGetLastError();
}

hipError_t launch_verify_sampling(const SpecVerifyParams& p, hipStream_t st) {
  (void)launch_k(k_verify_sampling, dim3(p.S), dim3(kRowThreads), st, p);
  return hipGetLastError();
}

}  // namespace dfl
