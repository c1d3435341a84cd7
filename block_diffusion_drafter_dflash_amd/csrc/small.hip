// Small kernels of the draft round: block input gather, fused-row RMSNorm, greedy
// verify, workspace counter clearing (gfx950).
#include "common.hpp"
#include "kernels.h"

namespace dfl {

// Deterministic sum over a workgroup of 256 threads: butterfly inside each wave,
// then the four wave sums in wave order.
__device__ float block_sum_256(float v, float* red) {
  v = xor_sum(v, kWave);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

// Block rows: X[s*B] = embed[anchor[s]], X[s*B + j] = embed[mask] for j >= 1, and
// 1 / rms of each row for the first layer's input norm.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(const EmbedParams p) {
  constexpr int E = Elem<T>::E;
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int s = r / p.B, j = r % p.B;
  int tok = j == 0 ? p.anchor[s] : p.mask_token;
  tok = tok < 0 ? 0 : (tok >= p.vocab ? p.vocab - 1 : tok);
  const T* src = static_cast<const T*>(p.embed) + (int64_t)tok * p.hidden;
  T* dst = static_cast<T*>(p.x) + (int64_t)r * p.hidden;
  float ss = 0.f;
  for (int c = threadIdx.x * E; c < p.hidden; c += 256 * E) {
    uint4 v = ldg16(src + c);
    stg16(dst + c, v);
    float f[E];
    unpack(v, f, T());
#pragma unroll
    for (int e = 0; e < E; ++e) ss += f[e] * f[e];
  }
  ss = block_sum_256(ss, red);
  if (threadIdx.x == 0) p.inv[r] = (float)(1.0 / sqrt((double)ss / (double)p.hidden + (double)p.eps));
}

// Fused rows: out[r] = y[r] / sqrt(mean(y[r]^2) + eps) * gain, with the squares summed
// per 128-column tile by the fc GEMM and here over tiles in order.
template <typename T>
__global__ __launch_bounds__(256) void k_rownorm(const RowNormParams p) {
  constexpr int E = Elem<T>::E;
  __shared__ float s_inv;
  const int r = blockIdx.x;
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int t = 0; t < p.n_tiles; ++t) ss += p.ssq_part[(int64_t)r * p.n_tiles + t];
    s_inv = (float)(1.0 / sqrt((double)ss / (double)p.hidden + (double)p.eps));
  }
  __syncthreads();
  const float inv = s_inv;
  const float* y = p.y + (int64_t)r * p.hidden;
  const T* gn = static_cast<const T*>(p.gain);
  T* out = static_cast<T*>(p.out) + (int64_t)r * p.hidden;
  for (int c = threadIdx.x * E; c < p.hidden; c += 256 * E) {
    float f[E], gf[E];
    unpack(ldg16(gn + c), gf, T());
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = y[c + e] * inv * gf[e];
    stg16(out + c, pack(f, T()));
  }
}

// Greedy verify: one wave per stream; the accepted length is the index of the first
// mismatch (lowest set bit of the ballot), or B-1 when every drafted token matches.
__global__ __launch_bounds__(64) void k_verify(const VerifyParams p) {
  const int s = blockIdx.x, j = threadIdx.x;
  const int B = p.B;
  const int* d = p.draft + (int64_t)s * (B - 1);
  const int* t = p.target + (int64_t)s * B;
  const bool mismatch = (j < B - 1) && (d[j] != t[j]);
  const unsigned long long mask = __ballot(mismatch);
  const int a = mask ? __builtin_ctzll(mask) : B - 1;
  const int bonus = t[a];
  if (j < B) {
    int v = j < a ? d[j] : (j == a ? bonus : -1);
    p.committed[(int64_t)s * B + j] = v;
  }
  if (j == 0) {
    p.accept[s] = a;
    p.bonus[s] = bonus;
    if (p.ctx_len) p.ctx_len[s] += a + 1;
  }
}

__global__ void k_fill_zero(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

hipError_t launch_embed(int dtype, const EmbedParams& p, hipStream_t st) {
  if (dtype == 0) hipLaunchKernelGGL(k_embed<float>, dim3(p.S * p.B), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_embed<bf16_t>, dim3(p.S * p.B), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_rownorm(int dtype, const RowNormParams& p, hipStream_t st) {
  if (dtype == 0) hipLaunchKernelGGL(k_rownorm<float>, dim3(p.R), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_rownorm<bf16_t>, dim3(p.R), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& p, hipStream_t st) {
  hipLaunchKernelGGL(k_verify, dim3(p.S), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fill_zero(int* p, int64_t n, hipStream_t st) {
  int blocks = (int)((n + 255) / 256);
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace dfl
