// DFlash2 candidate path selector over drafted logits (gfx950).
//
// Each drafted position keeps its top-k tokens (largest logit first, ties to the lowest
// id) with node score log softmax(logits)(token); adjacent positions' candidates a, b
// add the pair score <U[a], W[b]> of two rank-r token codebooks (none at rank 0, where
// the path is each position's top-1). The best path maximises the sum of node and pair
// scores; a draft stops before the first position whose chosen token's probability is
// below min_p, and the positions past the stop get -1.
//
// k_select_topk: one workgroup a row. It forms the row's maximum and its float64
// partition sum (exponentials in float64, summed in a fixed order), then takes the
// candidates in k rounds, each the block-wide largest logit ordered after the previous
// round's (value descending, id ascending), so no candidate set is kept.
// k_select_path: one workgroup a stream: the pair scores of every adjacent pair of
// positions in float64 (the products of bf16 codebook entries are exact), then one
// wave runs the best-path recursion (a lane a candidate) and the walk back.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kPathThreads = 256;

// Ordered maximum: (v, i) before (w, j) when v > w, or v == w and i < j.
__device__ __forceinline__ bool before(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

}  // namespace

__global__ __launch_bounds__(kTopkThreads) void k_select_topk(const SelectParams p) {
  constexpr int NW = kTopkThreads / kWave;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW];
  __shared__ double s_d[NW];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* x = p.logits + (int64_t)row * p.ld;

  // maximum (ordered: the largest value, lowest id) = round 0's candidate
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = tid; i < p.V; i += kTopkThreads) {
    const float v = x[i];
    if (before(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  auto block_best = [&](float& v, int& i) {
    for (int m = 1; m < kWave; m <<= 1) {
      const float ov = __shfl_xor(v, m, kWave);
      const int oi = __shfl_xor(i, m, kWave);
      if (before(ov, oi, v, i)) {
        v = ov;
        i = oi;
      }
    }
    __syncthreads();
    if (lane == 0) {
      s_v[w] = v;
      s_i[w] = i;
    }
    __syncthreads();
    v = s_v[0];
    i = s_i[0];
    for (int k = 1; k < NW; ++k)
      if (before(s_v[k], s_i[k], v, i)) {
        v = s_v[k];
        i = s_i[k];
      }
  };
  block_best(bv, bi);
  const double m = (double)bv;

  // float64 partition sum: per-thread sums in index order, then lanes and waves in order
  double z = 0.0;
  for (int i = tid; i < p.V; i += kTopkThreads) z += exp((double)x[i] - m);
  for (int k = 1; k < kWave; k <<= 1) z += __shfl_xor(z, k, kWave);
  __syncthreads();
  if (lane == 0) s_d[w] = z;
  __syncthreads();
  z = s_d[0];
  for (int k = 1; k < NW; ++k) z += s_d[k];
  const double log_z = log(z);

  int* cidx = p.cand_idx + (int64_t)row * kSelectMaxK;
  double* cnode = p.cand_node + (int64_t)row * kSelectMaxK;
  if (tid == 0) {
    cidx[0] = bi;
    cnode[0] = (double)bv - m - log_z;
  }
  float lv = bv;
  int li = bi;
  for (int r = 1; r < p.k; ++r) {
    float cv = -INFINITY;
    int ci = 0x7fffffff;
    for (int i = tid; i < p.V; i += kTopkThreads) {
      const float v = x[i];
      if (before(lv, li, v, i) && before(v, i, cv, ci)) {   // after the last pick, best so far
        cv = v;
        ci = i;
      }
    }
    block_best(cv, ci);
    if (tid == 0) {
      cidx[r] = ci;
      cnode[r] = (double)cv - m - log_z;
    }
    lv = cv;
    li = ci;
  }
}

__global__ __launch_bounds__(kPathThreads) void k_select_path(const SelectParams p) {
  __shared__ int s_idx[kSelectMaxB][kSelectMaxK];
  __shared__ double s_node[kSelectMaxB][kSelectMaxK];
  __shared__ double s_edge[kSelectMaxB][kSelectMaxK][kSelectMaxK];
  __shared__ double s_best[kSelectMaxK];
  __shared__ int s_back[kSelectMaxB][kSelectMaxK];
  const int s = blockIdx.x, tid = threadIdx.x;
  const int P = p.B - 1, K = p.k;
  for (int e = tid; e < P * K; e += kPathThreads) {
    const int j = e / K, c = e % K;
    const int64_t row = (int64_t)s * P + j;
    s_idx[j][c] = p.cand_idx[row * kSelectMaxK + c];
    s_node[j][c] = p.cand_node[row * kSelectMaxK + c];
  }
  __syncthreads();
  // pair scores <U[a], W[b]> of candidates a at j and b at j + 1, float64, rank order
  for (int e = tid; e < (P - 1) * K * K; e += kPathThreads) {
    const int j = e / (K * K), a = (e / K) % K, b = e % K;
    double acc = 0.0;
    if (p.rank > 0) {
      const bf16_t* u = static_cast<const bf16_t*>(p.code_u) + (int64_t)s_idx[j][a] * p.rank;
      const bf16_t* wv = static_cast<const bf16_t*>(p.code_w) + (int64_t)s_idx[j + 1][b] * p.rank;
      for (int t = 0; t < p.rank; ++t) acc += (double)bf16_to_f32(u[t]) * (double)bf16_to_f32(wv[t]);
    }
    s_edge[j][a][b] = acc;
  }
  __syncthreads();
  // best-path recursion: lane b (b < k) of wave 0 holds the best score of paths ending at
  // candidate b; every thread stays for the barriers
  const int lane = tid;
  const bool on = lane < K;
  double best = on ? s_node[0][lane] : -INFINITY;
  for (int j = 1; j < P; ++j) {
    if (on) s_best[lane] = best;
    __syncthreads();
    if (on) {
      double mv = s_best[0] + s_edge[j - 1][0][lane];
      int ma = 0;
      for (int a = 1; a < K; ++a) {
        const double t = s_best[a] + s_edge[j - 1][a][lane];
        if (t > mv) {     // the first maximum: the earlier candidate
          mv = t;
          ma = a;
        }
      }
      s_back[j][lane] = ma;
      best = mv + s_node[j][lane];
    }
    __syncthreads();
  }
  if (on) s_best[lane] = best;
  __syncthreads();
  if (lane == 0) {
    int c = 0;
    for (int a = 1; a < K; ++a)
      if (s_best[a] > s_best[c]) c = a;
    int path[kSelectMaxB];
    path[P - 1] = c;
    for (int j = P - 1; j > 0; --j) {
      c = s_back[j][c];
      path[j - 1] = c;
    }
    int len = P;
    for (int j = 0; j < P; ++j)
      if (exp(s_node[j][path[j]]) < (double)p.min_p) {
        len = j;
        break;
      }
    for (int j = 0; j < P; ++j) p.draft_out[(int64_t)s * P + j] = j < len ? s_idx[j][path[j]] : -1;
    p.draft_len[s] = len;
  }
}

hipError_t launch_select(const SelectParams& p, hipStream_t st) {
  (void)launch_k(k_select_topk, dim3(p.S * (p.B - 1)), dim3(kTopkThreads), st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  (void)launch_k(k_select_path, dim3(p.S), dim3(kPathThreads), st, p);
  return hipGetLastError();
}

}  // namespace dfl
