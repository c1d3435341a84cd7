// Sampling kernels (DFlash explainer, section 4, "Sampling decoding"): inverse-CDF
// draws from tempered softmax rows, and speculative-sampling acceptance of a drafted
// block with the residual max(p_target - p_draft, 0) at the first rejection.
//
// A row of V logits is cut into kSlices slices of whole segments (kSeg consecutive
// ids). The weight of id k is exp2((l_k - max) * log2(e) / T) in fp32; sums are
// float64. A first kernel gives every (row, slice) its max and its weight sum
// relative to that max, one workgroup each, so that a row's reductions spread over
// many CUs. A row's total is the slices' sums rescaled to the row max and added in
// slice order. A draw with uniform u takes the first slice whose running total
// exceeds u times the row total; inside it one workgroup sums the slice's segments
// (each wave a batch of consecutive segments, every load in flight, lane l reading
// ids l, l + 64, ...: contiguous 256-byte runs), scans the segment sums, binary-
// searches them and scans one segment with a wave: the smallest id whose running
// sum exceeds the target, never an id of zero weight (rounding that leaves the
// crossing past a slice or segment falls back to its last id of positive weight).
// Every reduction has a fixed order, so results are deterministic.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kDrawThreads = 1024;                 // the draw: one workgroup a row
constexpr int kDrawWaves = kDrawThreads / kWave;
constexpr int kSliceThreads = 256;                 // the per-slice kernels
constexpr int kSegPer = 4;                         // wave loads a segment
constexpr int kSeg = kSegPer * kWave;              // ids a segment
constexpr int kBatch = 8;                          // loads in flight a thread
constexpr int kMaxSliceSegs = (kSampleVocabMax / kSlices + kSeg - 1) / kSeg;

namespace {

// Slice s of a row of V ids: [lo, hi), whole segments (the last slices may be empty).
struct Slice {
  int lo, hi;
};
__device__ __forceinline__ Slice slice_of(int V, int s) {
  const int per = ((V + kSlices - 1) / kSlices + kSeg - 1) / kSeg * kSeg;
  const int lo = min(s * per, V);
  return {lo, min(lo + per, V)};
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Workgroup max / sum (every thread gets the result).
template <int NW>
__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = sh[0];
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  return r;
}
template <int NW>
__device__ __forceinline__ double block_sum(double v, double* sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < NW; ++i) r += sh[i];
  return r;
}

// Sum over ids [lo, hi) of w(k), strided over the workgroup, kBatch loads in flight.
template <int NT, typename Wf>
__device__ __forceinline__ double strided_sum(const Wf& w, int lo, int hi) {
  double x = 0.0;
  for (int k0 = lo + threadIdx.x; k0 < hi; k0 += kBatch * NT) {
    double v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k = k0 + b * NT;
      v[b] = k < hi ? w(k) : 0.0;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) x += v[b];
  }
  return x;
}

// A row's (max, total) from its slices' (max, sum): the total rescales each slice's
// sum to the row max (exp2 in fp32) and adds them in slice order. y[s] gets the
// rescaled slice sums when y is given.
__device__ __forceinline__ void combine_slices(const double* st, float scale, float& M, double& total, double* y) {
  float m = -INFINITY;
  for (int s = 0; s < kSlices; ++s) m = fmaxf(m, (float)st[2 * s]);
  double t = 0.0;
  for (int s = 0; s < kSlices; ++s) {
    const float ms = (float)st[2 * s];
    const double v = ms == -INFINITY ? 0.0 : st[2 * s + 1] * (double)exp2f((ms - m) * scale);
    if (y) y[s] = v;
    t += v;
  }
  M = m;
  total = t;
}

// The first slice whose running total exceeds target (the last slice of positive
// sum when rounding leaves none); base gets the running total before it.
__device__ __forceinline__ int pick_slice(const double* y, double target, double& base) {
  double run = 0.0;
  int last = -1;
  double last_base = 0.0;
  for (int s = 0; s < kSlices; ++s) {
    if (y[s] > 0.0) {
      if (run + y[s] > target) {
        base = run;
        return s;
      }
      last = s;
      last_base = run;
    }
    run += y[s];
  }
  base = last_base;
  return last;
}

// The draw inside ids [lo, hi) (one workgroup of kDrawThreads): the smallest id whose
// running sum of w exceeds target (relative to lo), falling back to the range's last
// id of positive weight. seg: LDS for the range's segment sums. Returns the id on
// every thread.
template <typename Wf>
__device__ int draw_in_range(const Wf& w, int lo, int hi, double target, double* seg, int* sh_tok) {
  const int n_seg = (hi - lo + kSeg - 1) / kSeg;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int sg0 = wv * kBatch; sg0 < n_seg; sg0 += kDrawWaves * kBatch) {
    double x[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      x[b] = 0.0;
#pragma unroll
      for (int i = 0; i < kSegPer; ++i) {
        const int k = lo + (sg0 + b) * kSeg + i * kWave + lane;
        if (k < hi) x[b] += w(k);
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
  if (threadIdx.x == 0) {
    // exclusive prefix in place, then the last segment whose prefix is <= target
    double run = 0.0;
    for (int sg = 0; sg < n_seg; ++sg) {
      const double v = seg[sg];
      seg[sg] = run;
      run += v;
    }
    int a = 0, b = n_seg - 1;
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (seg[mid] <= target) a = mid;
      else b = mid - 1;
    }
    *sh_tok = a;
  }
  __syncthreads();
  const int sg = *sh_tok;
  __syncthreads();
  if (threadIdx.x < kWave) {
    double run = seg[sg];
    int tok = -1, last = -1;
#pragma unroll
    for (int i = 0; i < kSegPer; ++i) {
      const int k = lo + sg * kSeg + i * kWave + lane;
      const double x = k < hi ? w(k) : 0.0;
      double incl = x;
      for (int m = 1; m < kWave; m <<= 1) {
        const double o = __shfl_up(incl, m, kWave);
        if (lane >= m) incl += o;
      }
      const unsigned long long hit = __ballot(x > 0.0 && run + incl > target);
      const unsigned long long pos = __ballot(x > 0.0);
      if (tok < 0 && hit) tok = lo + sg * kSeg + i * kWave + __builtin_ctzll(hit);
      if (pos) last = lo + sg * kSeg + i * kWave + 63 - __builtin_clzll(pos);
      run += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) *sh_tok = tok >= 0 ? tok : last;
  }
  __syncthreads();
  int tok = *sh_tok;
  if (tok < 0) {
    // the chosen segment has no mass: the range's last id of positive weight
    __syncthreads();
    if (threadIdx.x == 0) {
      int t = -1;
      for (int k = hi - 1; k >= lo; --k)
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

// (max, weight sum relative to that max) of slice blockIdx.x of row blockIdx.y.
// Rows [0, rows1) come from (logits, stats), the grid's rows past them from
// (logits2, stats2): one launch for the draft and the target rows of a verify.
__global__ __launch_bounds__(kSliceThreads) void k_slice_stats(const float* logits, int V, int64_t ld, float scale,
                                                               double* stats, int rows1, const float* logits2,
                                                               double* stats2) {
  __shared__ float shf[kSliceThreads / kWave];
  __shared__ double shd[kSliceThreads / kWave];
  const bool second = (int)blockIdx.y >= rows1;
  const int ry = second ? (int)blockIdx.y - rows1 : (int)blockIdx.y;
  const float* row = (second ? logits2 : logits) + (int64_t)ry * ld;
  const Slice sl = slice_of(V, blockIdx.x);
  float m = -INFINITY;
  for (int k0 = sl.lo + threadIdx.x; k0 < sl.hi; k0 += kBatch * kSliceThreads) {
    float v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int k = k0 + b * kSliceThreads;
      v[b] = k < sl.hi ? row[k] : -INFINITY;
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) m = fmaxf(m, v[b]);
  }
  m = block_max<kSliceThreads / kWave>(m, shf);
  double z = 0.0;
  if (m != -INFINITY)   // uniform: every thread holds the slice max
    z = block_sum<kSliceThreads / kWave>(
        strided_sum<kSliceThreads>([&](int k) { return (double)exp2f((row[k] - m) * scale); }, sl.lo, sl.hi), shd);
  if (threadIdx.x == 0) {
    double* o = (second ? stats2 : stats) + ((int64_t)ry * kSlices + blockIdx.x) * 2;
    o[0] = (double)m;
    o[1] = z;
  }
}

// One draw per row from softmax(row / T) with uniform u[row].
__global__ __launch_bounds__(kDrawThreads) void k_sample_rows(const SampleParams p) {
  __shared__ double seg[kMaxSliceSegs];
  __shared__ double y[kSlices];
  __shared__ float sh_m;
  __shared__ double sh_total, sh_base;
  __shared__ int sh_slice, sh_tok;
  const float* row = p.logits + (int64_t)blockIdx.x * p.ld;
  const double* st = p.slice_stats + (int64_t)blockIdx.x * kSlices * 2;
  const double u = (double)p.u[blockIdx.x];
  if (threadIdx.x == 0) {
    float M;
    double total, base;
    combine_slices(st, p.scale, M, total, y);
    sh_slice = pick_slice(y, u * total, base);
    sh_m = M;
    sh_total = total;
    sh_base = base;
  }
  __syncthreads();
  const float M = sh_m;
  const double total = sh_total;
  const float sc = p.scale;
  auto w = [&](int k) { return (double)exp2f((row[k] - M) * sc); };
  const Slice sl = slice_of(p.V, sh_slice);
  const int tok = draw_in_range(w, sl.lo, sl.hi, u * total - sh_base, seg, &sh_tok);
  if (threadIdx.x == 0) {
    p.token_out[blockIdx.x] = tok;
    if (p.prob_out) p.prob_out[blockIdx.x] = (float)(w(tok) / total);
  }
}

// Speculative-sampling acceptance (one wave a stream): lane j evaluates the test at
// position j (j < B - 1) and the (max, total) of target row j (j < B) in parallel; the
// accepted length is the first failing position (B - 1 when none fails), so the
// decisions are those of a walk that stops at the first rejection. For the draw that
// follows: the row max and total of the target row a and (on a rejection) of the
// draft row a.
__global__ __launch_bounds__(kWave) void k_spec_accept(const SpecVerifyParams p) {
  const int s = blockIdx.x, B = p.B, V = p.V, j = threadIdx.x;
  const float sc = p.scale;
  float tm = 0.f, dm = 0.f;
  double tz = 1.0, dz = 1.0;
  bool ok = false;   // the draft token at position j passes its test
  if (j < B) combine_slices(p.target_stats + ((int64_t)s * B + j) * kSlices * 2, sc, tm, tz, nullptr);
  if (j < B - 1) {
    combine_slices(p.draft_stats + ((int64_t)s * (B - 1) + j) * kSlices * 2, sc, dm, dz, nullptr);
    const int tok = p.draft[(int64_t)s * (B - 1) + j];
    if (tok >= 0 && tok < V) {   // an id outside the vocabulary is rejected
      const float* drow = p.draft_logits + ((int64_t)s * (B - 1) + j) * p.ld;
      const float* trow = p.target_logits + ((int64_t)s * B + j) * p.ld;
      const double pd = (double)exp2f((drow[tok] - dm) * sc) / dz;
      const double pt = (double)exp2f((trow[tok] - tm) * sc) / tz;
      ok = (double)p.u_accept[(int64_t)s * (B - 1) + j] * pd < pt;
    }
  }
  const uint64_t rejected = __ballot(j < B - 1 && !ok);
  const int a = rejected ? (int)__builtin_ctzll(rejected) : B - 1;
  const int ad = a < B - 1 ? a : B - 2;   // the draft row's values only matter on a rejection
  const float tma = __shfl(tm, a, kWave), dma = __shfl(dm, ad, kWave);
  const double tza = __shfl(tz, a, kWave), dza = __shfl(dz, ad, kWave);
  if (j == 0) {
    p.accept[s] = a;
    double* r = p.row_info + (int64_t)s * 4;
    r[0] = tma;
    r[1] = tza;
    r[2] = dma;
    r[3] = dza;
  }
}

// Per (slice, stream): the slice's sums of the residual max(q - p, 0) at the rejected
// position and of q itself (q alone after a full acceptance, at row B - 1).
__global__ __launch_bounds__(kSliceThreads) void k_spec_slices(const SpecVerifyParams p) {
  __shared__ double shd[kSliceThreads / kWave];
  const int s = blockIdx.y, B = p.B;
  const int a = p.accept[s];
  const double* ri = p.row_info + (int64_t)s * 4;
  const float tm = (float)ri[0], dm = (float)ri[2];
  const double tz = ri[1], dz = ri[3];
  const float sc = p.scale;
  const float* trow = p.target_logits + ((int64_t)s * B + a) * p.ld;
  const Slice sl = slice_of(p.V, blockIdx.x);
  auto wt = [&](int k) { return (double)exp2f((trow[k] - tm) * sc) / tz; };
  double rsum = 0.0;
  if (a < B - 1) {   // uniform over the workgroup
    const float* drow = p.draft_logits + ((int64_t)s * (B - 1) + a) * p.ld;
    auto wr = [&](int k) {
      const double v = wt(k) - (double)exp2f((drow[k] - dm) * sc) / dz;
      return v > 0.0 ? v : 0.0;
    };
    rsum = block_sum<kSliceThreads / kWave>(strided_sum<kSliceThreads>(wr, sl.lo, sl.hi), shd);
  }
  const double qsum = block_sum<kSliceThreads / kWave>(strided_sum<kSliceThreads>(wt, sl.lo, sl.hi), shd);
  if (threadIdx.x == 0) {
    double* o = p.slice_sums + ((int64_t)s * kSlices + blockIdx.x) * 2;
    o[0] = rsum;
    o[1] = qsum;
  }
}

// The draw that ends the stream's block (one workgroup a stream), and the outputs.
__global__ __launch_bounds__(kDrawThreads) void k_spec_draw(const SpecVerifyParams p) {
  __shared__ double seg[kMaxSliceSegs];
  __shared__ double y[kSlices];
  __shared__ double sh_target;
  __shared__ int sh_slice, sh_resid, sh_tok;
  const int s = blockIdx.x, B = p.B;
  const int a = p.accept[s];
  const double* ri = p.row_info + (int64_t)s * 4;
  const float tm = (float)ri[0], dm = (float)ri[2];
  const double tz = ri[1], dz = ri[3];
  const float sc = p.scale;
  const double u = (double)p.u_sample[s];
  if (threadIdx.x == 0) {
    const double* ss = p.slice_sums + (int64_t)s * kSlices * 2;
    double rt = 0.0;
    for (int i = 0; i < kSlices; ++i) rt += ss[2 * i];
    const int resid = a < B - 1 && rt > 0.0;   // else the target's own distribution
    double total = 0.0;
    for (int i = 0; i < kSlices; ++i) {
      y[i] = ss[2 * i + (resid ? 0 : 1)];
      total += y[i];
    }
    double base;
    sh_slice = pick_slice(y, u * total, base);
    sh_target = u * total - base;
    sh_resid = resid;
  }
  __syncthreads();
  const float* trow = p.target_logits + ((int64_t)s * B + a) * p.ld;
  auto wt = [&](int k) { return (double)exp2f((trow[k] - tm) * sc) / tz; };
  const Slice sl = slice_of(p.V, sh_slice);
  int tok;
  if (sh_resid) {
    const float* drow = p.draft_logits + ((int64_t)s * (B - 1) + a) * p.ld;
    auto wr = [&](int k) {
      const double v = wt(k) - (double)exp2f((drow[k] - dm) * sc) / dz;
      return v > 0.0 ? v : 0.0;
    };
    tok = draw_in_range(wr, sl.lo, sl.hi, sh_target, seg, &sh_tok);
  } else {
    tok = draw_in_range(wt, sl.lo, sl.hi, sh_target, seg, &sh_tok);
  }
  const int* d = p.draft + (int64_t)s * (B - 1);
  if ((int)threadIdx.x < B) {
    const int j = threadIdx.x;
    p.committed[(int64_t)s * B + j] = j < a ? d[j] : (j == a ? tok : -1);
  }
  if (threadIdx.x == 0) {
    p.token[s] = tok;
    if (p.ctx_len) p.ctx_len[s] += a + 1;
  }
}

hipError_t launch_slice_stats(const float* logits, int rows, int V, int64_t ld, float scale, double* stats,
                              hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  (void)launch_k(k_slice_stats, dim3(kSlices, rows), dim3(kSliceThreads), st, logits, V, ld, scale, stats, rows,
                 static_cast<const float*>(nullptr), static_cast<double*>(nullptr));
  return hipGetLastError();
}

hipError_t launch_sample_rows(const SampleParams& p, hipStream_t st) {
  hipError_t e = launch_slice_stats(p.logits, p.rows, p.V, p.ld, p.scale, p.slice_stats, st);
  if (e != hipSuccess) return e;
  (void)launch_k(k_sample_rows, dim3(p.rows), dim3(kDrawThreads), st, p);
  return hipGetLastError();
}

hipError_t launch_verify_sampling(const SpecVerifyParams& p, hipStream_t st) {
  const int rd = p.S * (p.B - 1), rt = p.S * p.B;   // draft rows, then target rows
  (void)launch_k(k_slice_stats, dim3(kSlices, rd + rt), dim3(kSliceThreads), st, p.draft_logits, p.V, p.ld, p.scale,
                 p.draft_stats, rd, p.target_logits, p.target_stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  (void)launch_k(k_spec_accept, dim3(p.S), dim3(kWave), st, p);
  (void)launch_k(k_spec_slices, dim3(kSlices, p.S), dim3(kSliceThreads), st, p);
  (void)launch_k(k_spec_draw, dim3(p.S), dim3(kDrawThreads), st, p);
  return hipGetLastError();
}

}  // namespace dfl
