// Sampling kernels (DFlash explainer, section 4, "Sampling decoding"): inverse-CDF
// draws from tempered softmax rows, and speculative-sampling acceptance of a drafted
// block with the residual max(p_target - p_draft, 0) at the first rejection.
//
// A row of V logits is handled by one workgroup of kRowThreads threads. The weight of
// id k is w_k = exp2((l_k - max) * log2(e) / T) in fp32 (for the residual, the
// difference of two normalised weights, in float64). Ids are cut into segments of
// kSeg consecutive ids; each wave sums batches of kBatch consecutive segments, all
// their loads in flight at once (lane l reads ids l, l + 64, ..., so every load is one
// contiguous 256-byte run), in float64, and the segment sums are kept in LDS. A draw with uniform u scans the segment sums in id
// order, picks the segment where the running total first exceeds u times the row
// total, and one wave scans that segment's ids in order: the smallest id whose
// running sum exceeds the target, never an id of zero weight. Every reduction has a
// fixed order, so results are deterministic.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / kWave;
constexpr int kSegPer = 4;                     // wave loads a segment
constexpr int kSeg = kSegPer * kWave;          // ids a segment
constexpr int kMaxSegs = kSampleVocabMax / kSeg;

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

// Loads of a strided pass go in batches of kBatch per thread, all in flight at once.
constexpr int kBatch = 8;

__device__ __forceinline__ float row_max(const float* row, int V, float* sh) {
  float m = -INFINITY;
  for (int k0 = threadIdx.x; k0 < V; k0 += kBatch * kRowThreads) {
    float x[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k = k0 + b * kRowThreads;
      x[b] = k < V ? row[k] : -INFINITY;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) m = fmaxf(m, x[b]);
  }
  return block_max(m, sh);
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Segment sums of the weights w(k) (0 past V) into seg[0 .. n_seg), then, in place,
// their exclusive prefix in id order; returns the row total (every thread).
template <typename Wf>
__device__ double segment_prefix(const Wf& w, int V, double* seg, double* sh) {
  const int n_seg = (V + kSeg - 1) / kSeg;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave wv sums segments wv * kBatch .. + kBatch - 1, then the next kRowWaves * kBatch
  for (int sg0 = wv * kBatch; sg0 < n_seg; sg0 += kRowWaves * kBatch) {
    double x[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      x[b] = 0.0;
#pragma unroll
      for (int i = 0; i < kSegPer; ++i) {
        const int k = (sg0 + b) * kSeg + i * kWave + lane;
        if (k < V) x[b] += w(k);
      }
    }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
#pragma unroll
      for (int b = 0; b < kBatch; ++b) x[b] += __shfl_xor(x[b], m, kWave);
    if (lane == 0)
#pragma unroll
      for (int b = 0; b < kBatch; ++b)
        if (sg0 + b < n_seg) seg[sg0 + b] = x[b];
  }
  __syncthreads();
  // exclusive prefix: thread t owns segments [t * per, (t + 1) * per)
  const int per = (n_seg + kRowThreads - 1) / kRowThreads;
  const int s0 = min((int)threadIdx.x * per, n_seg), s1 = min(s0 + per, n_seg);
  double own = 0.0;
  for (int sg = s0; sg < s1; ++sg) own += seg[sg];
  double incl = own;
  for (int m = 1; m < kWave; m <<= 1) {
    const double o = __shfl_up(incl, m, kWave);
    if (lane >= m) incl += o;
  }
  if (lane == kWave - 1) sh[wv] = incl;
  __syncthreads();
  double base = 0.0, total = 0.0;
  for (int i = 0; i < kRowWaves; ++i) {
    if (i < wv) base += sh[i];
    total += sh[i];
  }
  double run = base + incl - own;
  __syncthreads();   // every segment sum is read before it is overwritten
  for (int sg = s0; sg < s1; ++sg) {
    const double x = seg[sg];
    seg[sg] = run;
    run += x;
  }
  __syncthreads();
  return total;
}

// The draw with uniform u over the weights whose segment prefixes segment_prefix left
// in seg (total: the row total). Returns the id on every thread.
template <typename Wf>
__device__ int segment_draw(const Wf& w, int V, const double* seg, double total, double u, int* sh_tok) {
  const int n_seg = (V + kSeg - 1) / kSeg;
  const double target = u * total;
  if (threadIdx.x == 0) {
    // the last segment whose prefix is <= target (segments of zero mass share the
    // prefix of the next one and are skipped by taking the last)
    int lo = 0, hi = n_seg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg[mid] <= target) lo = mid;
      else hi = mid - 1;
    }
    *sh_tok = lo;
  }
  __syncthreads();
  const int sg = *sh_tok;
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    double run = seg[sg];
    int tok = -1, last = -1;
#pragma unroll
    for (int i = 0; i < kSegPer; ++i) {
      const int k = sg * kSeg + i * kWave + lane;
      const double x = k < V ? w(k) : 0.0;
      double incl = x;
      for (int m = 1; m < kWave; m <<= 1) {
        const double o = __shfl_up(incl, m, kWave);
        if (lane >= m) incl += o;
      }
      const unsigned long long hit = __ballot(x > 0.0 && run + incl > target);
      const unsigned long long pos = __ballot(x > 0.0);
      if (tok < 0 && hit) tok = sg * kSeg + i * kWave + __builtin_ctzll(hit);
      if (pos) last = sg * kSeg + i * kWave + 63 - __builtin_clzll(pos);
      run += __shfl(incl, kWave - 1, kWave);
    }
    // rounding left the crossing past this segment: its last id of positive weight
    if (lane == 0) *sh_tok = tok >= 0 ? tok : last;
  }
  __syncthreads();
  int tok = *sh_tok;
  if (tok < 0) {
    // a segment without mass (target at or past the total): the row's last id of
    // positive weight
    __syncthreads();
    if (threadIdx.x == 0) {
      int t = -1;
      for (int s = n_seg - 1; s >= 0 && t < 0; --s)
        for (int k = min(V, (s + 1) * kSeg) - 1; k >= s * kSeg; --k)
          if (w(k) > 0.0) {
            t = k;
            break;
          }
      *sh_tok = t;
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
  const float m = row_max(row, V, shf);
  double x = 0.0;
  for (int k0 = threadIdx.x; k0 < V; k0 += kBatch * kRowThreads) {
    float v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k = k0 + b * kRowThreads;
      v[b] = k < V ? row[k] : -INFINITY;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) x += (double)exp2f((v[b] - m) * scale);
  }
  x = wave_sum(x);
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) shd[wv] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int i = 0; i < kRowWaves; ++i) t += shd[i];
    stats[2 * blockIdx.x] = (double)m;
    stats[2 * blockIdx.x + 1] = t;
  }
}

// One draw per row from softmax(row / T) with uniform u[row].
__global__ __launch_bounds__(kRowThreads) void k_sample_rows(const SampleParams p) {
  __shared__ float shf[kRowWaves];
  __shared__ double shd[kRowWaves];
  __shared__ double seg[kMaxSegs];
  __shared__ int sh_tok;
  const float* row = p.logits + (int64_t)blockIdx.x * p.ld;
  const float m = row_max(row, p.V, shf);
  const float sc = p.scale;
  auto w = [&](int k) { return (double)exp2f((row[k] - m) * sc); };
  const double total = segment_prefix(w, p.V, seg, shd);
  const int tok = segment_draw(w, p.V, seg, total, (double)p.u[blockIdx.x], &sh_tok);
  if (threadIdx.x == 0) {
    p.token_out[blockIdx.x] = tok;
    if (p.prob_out) p.prob_out[blockIdx.x] = (float)(w(tok) / total);
  }
}

// Speculative-sampling acceptance of one stream's drafted block (one workgroup).
__global__ __launch_bounds__(kRowThreads) void k_verify_sampling(const SpecVerifyParams p) {
  __shared__ double shd[kRowWaves];
  __shared__ double seg[kMaxSegs];
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
  const double u = (double)p.u_sample[s];
  const float* trow = tl + (int64_t)a * p.ld;
  const float tm = (float)ts[2 * a];
  const double tz = ts[2 * a + 1];
  auto wt = [&](int k) { return (double)exp2f((trow[k] - tm) * sc) / tz; };
  int tok = -1;
  bool from_target = a == B - 1;
  if (!from_target) {
    // residual max(q - p, 0) at the rejected position; q itself if it has no mass
    const float* drow = dl + (int64_t)a * p.ld;
    const float dm = (float)ds[2 * a];
    const double dz = ds[2 * a + 1];
    auto wr = [&](int k) {
      const double r = wt(k) - (double)exp2f((drow[k] - dm) * sc) / dz;
      return r > 0.0 ? r : 0.0;
    };
    const double total = segment_prefix(wr, V, seg, shd);
    if (total > 0.0) tok = segment_draw(wr, V, seg, total, u, &sh_tok);
    else from_target = true;
  }
  if (from_target) {
    const double total = segment_prefix(wt, V, seg, shd);
    tok = segment_draw(wt, V, seg, total, u, &sh_tok);
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
