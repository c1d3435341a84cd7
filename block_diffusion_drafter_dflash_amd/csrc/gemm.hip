// Skinny MFMA GEMMs of the draft round with fused epilogues (gfx950).
//
// Y[M, N] = A[M, K] . W[N, K]^T with M small (block rows x streams) and W streamed
// from HBM exactly once. A workgroup of 8 waves owns a tile of 16*NT output columns
// for 16*MT rows; the waves split K eight ways and each streams its slice of the
// tile's weight rows, every lane reading 64 contiguous bytes of a row per iteration
// with the next iteration's loads in flight. Every MFMA's partial (32 products per
// element for bf16) is added into a float64 accumulator, and the eight wave
// partials are summed in wave order, so the results sit much closer to the exact
// sums than a running fp32 accumulator would. No workgroup ever waits
// for another: row statistics (sums of squares for the next RMSNorm) leave as
// per-tile partials that the consuming kernel adds in tile order, so every result
// is independent of scheduling and of the batch (the per-row arithmetic never
// depends on how many rows share a workgroup).
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kKW = 8;                  // waves per workgroup, splitting K
constexpr int kGemmThreads = kKW * kWave;

template <typename T>
struct GemmCfg {
  static constexpr int E = Elem<T>::E;
  static constexpr int KF = Elem<T>::KF;
  static constexpr int U = 4;           // 16-byte fragments per lane per row per iteration
  static constexpr int KI = U * KF;     // k-elements per iteration
};

template <int EPI>
struct AModeOf {
  static constexpr int value = EPI == EPI_FC ? A_TAPS
                               : (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LMHEAD) ? A_NORMED
                                                                                            : A_PLAIN;
};

__device__ __forceinline__ void top_merge(float& v1, int& i1, float& v2, float bv1, int bi1, float bv2) {
  if (bv1 > v1 || (bv1 == v1 && bi1 < i1)) {
    v2 = fmaxf(v1, bv2);
    v1 = bv1;
    i1 = bi1;
  } else {
    v2 = fmaxf(v2, bv1);
  }
}

__device__ __forceinline__ void top_xor_merge(float& v1, int& i1, float& v2, int width) {
  for (int m = 1; m < width; m <<= 1) {
    float o1 = __shfl_xor(v1, m, kWave);
    int oi = __shfl_xor(i1, m, kWave);
    float o2 = __shfl_xor(v2, m, kWave);
    top_merge(v1, i1, v2, o1, oi, o2);
  }
}

// Weight row of output column n (tile-local column c) for each GEMM kind.
template <typename T, int NT, int EPI>
__device__ __forceinline__ const T* weight_row(const GemmParams& p, int tile, int c) {
  const int n = tile * (16 * NT) + c;
  if constexpr (EPI == EPI_SWIGLU) {
    // tile t: columns 0..15 are gate rows 16t.., columns 16..31 the matching up rows
    const int r = tile * 16 + (c & 15);
    return static_cast<const T*>(c < 16 ? p.w0 : p.w1) + (int64_t)r * p.K;
  } else if constexpr (EPI == EPI_QKV) {
    if (n < p.nq) return static_cast<const T*>(p.w0) + (int64_t)n * p.K;
    if (n < p.nq + p.nkv) return static_cast<const T*>(p.w1) + (int64_t)(n - p.nq) * p.K;
    return static_cast<const T*>(p.w2) + (int64_t)(n - p.nq - p.nkv) * p.K;
  } else if constexpr (EPI == EPI_INJECT) {
    const int l = n / (2 * p.nkv), rem = n % (2 * p.nkv);
    return static_cast<const T*>(rem < p.nkv ? p.wk_l[l] : p.wv_l[l]) + (int64_t)(rem % p.nkv) * p.K;
  } else {
    const int nn = n < p.N ? n : p.N - 1;   // ragged last tile: read a valid row, drop it later
    return static_cast<const T*>(p.w0) + (int64_t)nn * p.K;
  }
}

template <typename T, int MT, int NT, int EPI>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const GemmParams p) {
  using C = GemmCfg<T>;
  constexpr int E = C::E, U = C::U, KI = C::KI;
  constexpr int AM = AModeOf<EPI>::value;
  constexpr int ROWS = 16 * MT, COLS = 16 * NT;
  __shared__ float red[kKW][ROWS][COLS + 1];
  __shared__ double s_inv[ROWS];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so the row
  // groups of one column tile are placed on the same XCD and share its weight rows
  // in that XCD's L2.
  const int b = blockIdx.x, xcd = b & 7, jj = b >> 3;
  const int tile = 8 * (jj / p.mgroups) + xcd, mg = jj % p.mgroups;
  if (tile >= p.n_tiles) return;
  const int row0 = mg * ROWS;

  // ---- RMSNorm statistics of the A rows (sum of squares, added over parts in order)
  if constexpr (AM == A_NORMED) {
    constexpr int TPR = kGemmThreads / ROWS;   // threads per row: 32 (MT 1), 16, 8 (MT 4)
    const int rl = tid / TPR, j = tid % TPR;
    int r = row0 + rl;
    r = r < p.M ? r : p.M - 1;
    const int xr = p.a_rowmap_bm1 > 0 ? (r / p.a_rowmap_bm1) * (p.a_rowmap_bm1 + 1) + 1 + r % p.a_rowmap_bm1 : r;
    double ss = 0.0;
    for (int q = j; q < p.a_ssq_parts; q += TPR) ss += p.a_ssq[(int64_t)xr * p.a_ssq_ld + q];
    for (int m = 1; m < TPR; m <<= 1) ss += __shfl_xor(ss, m, kWave);
    if (j == 0) s_inv[rl] = 1.0 / sqrt(ss / (double)p.K + (double)p.eps);
    __syncthreads();
  }

  const T* brow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) brow[nt] = weight_row<T, NT, EPI>(p, tile, 16 * nt + lr);
  int64_t aoff[MT];
  double ainv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = row0 + 16 * mt + lr;
    r = r < p.M ? r : p.M - 1;
    const int xr = p.a_rowmap_bm1 > 0 ? (r / p.a_rowmap_bm1) * (p.a_rowmap_bm1 + 1) + 1 + r % p.a_rowmap_bm1 : r;
    aoff[mt] = AM == A_TAPS ? (int64_t)r * p.tap_stride : (int64_t)xr * p.lda;
    ainv[mt] = 1.0;
    if constexpr (AM == A_NORMED) ainv[mt] = s_inv[16 * mt + lr];
  }
  const T* abase = static_cast<const T*>(p.a);

  double acc[MT][NT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.0;

  const int it0 = (int)((int64_t)w * p.iters / kKW), it1 = (int)((int64_t)(w + 1) * p.iters / kKW);
  const int lane_k = lg * (U * E);

  auto load = [&](int it, uint4 (&a)[MT][U], uint4 (&g)[U], uint4 (&b)[NT][U]) {
    const int k = it * KI + lane_k;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < U; ++u) b[nt][u] = ldg16(brow[nt] + k + u * E);
    if constexpr (AM == A_TAPS) {
      // An iteration's KI columns never straddle two planes (hidden % KI == 0).
      const int plane = (it * KI) / p.tap_h;
      const T* tp = static_cast<const T*>(p.taps[plane]) + (k - plane * p.tap_h);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < U; ++u) a[mt][u] = ldg16(tp + aoff[mt] + u * E);
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int u = 0; u < U; ++u) a[mt][u] = ldg16(abase + aoff[mt] + k + u * E);
    }
    if constexpr (AM == A_NORMED) {
#pragma unroll
      for (int u = 0; u < U; ++u) g[u] = ldg16(static_cast<const T*>(p.a_gain) + k + u * E);
    }
  };

  if (it0 < it1) {
    uint4 a_c[MT][U], g_c[U], b_c[NT][U];
    load(it0, a_c, g_c, b_c);
    for (int it = it0; it < it1; ++it) {
      const int itn = it + 1 < it1 ? it + 1 : it;
      uint4 a_n[MT][U], g_n[U], b_n[NT][U];
      load(itn, a_n, g_n, b_n);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float gf[E];
        if constexpr (AM == A_NORMED) unpack(g_c[u], gf, T());
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint4 av = a_c[mt][u];
          if constexpr (AM == A_NORMED) {
            // a = round(x * inv_rms * gain), products in float64, one rounding
            float xf[E];
            double xd[E];
            unpack(av, xf, T());
#pragma unroll
            for (int e = 0; e < E; ++e) xd[e] = (double)xf[e] * ainv[mt] * (double)gf[e];
            av = pack_d(xd, T());
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            // each MFMA's partial (KF products) is added into the float64 accumulator
            floatx4 part = floatx4{0.f, 0.f, 0.f, 0.f};
            mma_frag(part, av, b_c[nt][u], T());
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] += (double)part[i];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        g_c[u] = g_n[u];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a_c[mt][u] = a_n[mt][u];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b_c[nt][u] = b_n[nt][u];
      }
    }
  }

  // ---- the eight K slices -> LDS, summed in wave order
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][16 * mt + 4 * lg + i][16 * nt + lr] = (float)acc[mt][nt][i];
  __syncthreads();

  // ---- epilogue: one element per thread and pass; COLS consecutive lanes per row
#pragma unroll
  for (int e0 = 0; e0 < ROWS * COLS; e0 += kGemmThreads) {
    const int e = e0 + tid;
    if (e >= ROWS * COLS) break;   // whole waves (ROWS * COLS is a multiple of 64)
    const int rl = e / COLS, c = e % COLS;
    double vd = 0.0;
#pragma unroll
    for (int ww = 0; ww < kKW; ++ww) vd += (double)red[ww][rl][c];
    const float v = (float)vd;
    const int r = row0 + rl;
    const bool rv = r < p.M;
    const int n = tile * COLS + c;

    if constexpr (EPI == EPI_FC) {
      double ss = vd * vd;
      for (int m = 1; m < COLS; m <<= 1) ss += __shfl_xor(ss, m, kWave);
      if (rv) {
        p.y_out[(int64_t)r * p.N + n] = vd;
        if (c == 0) p.ssq_out[(int64_t)r * p.ssq_ld + tile] = ss;
      }
    } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
      if (rv) p.y_out[(int64_t)r * p.N + n] = vd;   // raw projections; norms and RoPE follow
    } else if constexpr (EPI == EPI_RESID) {
      float xn = 0.f;
      if (rv) {
        T* x = static_cast<T*>(p.x_io) + (int64_t)r * p.N + n;
        xn = Elem<T>::round_d((double)Elem<T>::load1(x) + vd);
        if constexpr (sizeof(T) == 2) *x = (T)f32_to_bf16(xn);
        else *x = xn;
      }
      double ss = (double)xn * (double)xn;
      for (int m = 1; m < COLS; m <<= 1) ss += __shfl_xor(ss, m, kWave);
      if (rv && c == 0) p.ssq_out[(int64_t)r * p.ssq_ld + tile] = ss;
    } else if constexpr (EPI == EPI_SWIGLU) {
      const double up = __shfl_xor(vd, 16, kWave);
      if (rv && c < 16) {
        T* dst = static_cast<T*>(p.m_out) + (int64_t)r * p.ld_out + tile * 16 + c;
        Elem<T>::store_d(dst, vd / (1.0 + exp(-vd)) * up);
      }
    } else if constexpr (EPI == EPI_LMHEAD) {
      const bool cv = n < p.N;
      float v1 = cv ? v : -INFINITY, v2 = -INFINITY;
      int i1 = cv ? n : 0x7fffffff;
      if (rv && cv && p.logits_out) p.logits_out[(int64_t)r * p.N + n] = v;
      top_xor_merge(v1, i1, v2, COLS);
      if (rv && c == 0)
        reinterpret_cast<float4*>(p.tile_res)[(int64_t)r * p.n_tiles + tile] = make_float4(v1, __int_as_float(i1), v2, 0.f);
    }
  }
}

// Final argmax over the LM head's column tiles: one workgroup per mask row.
__global__ __launch_bounds__(256) void k_argmax_final(const float4* tile_res, int n_tiles, int* draft_out,
                                                      float* top2_out) {
  __shared__ float s1[4], s2[4];
  __shared__ int si[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff;
  for (int t = tid; t < n_tiles; t += 256) {
    const float4 x = tile_res[(int64_t)r * n_tiles + t];
    top_merge(v1, i1, v2, x.x, __float_as_int(x.y), x.z);
  }
  top_xor_merge(v1, i1, v2, kWave);
  if ((tid & 63) == 0) {
    s1[tid >> 6] = v1;
    si[tid >> 6] = i1;
    s2[tid >> 6] = v2;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k) top_merge(v1, i1, v2, s1[k], si[k], s2[k]);
    draft_out[r] = i1;
    if (top2_out) {
      top2_out[2 * r] = v1;
      top2_out[2 * r + 1] = v2;
    }
  }
}

// ------------------------------------------------------------------ host launchers

template <typename T, int MT, int NT, int EPI>
static hipError_t launch_t(const GemmParams& p, hipStream_t st) {
  const int blocks = 8 * p.mgroups * ((p.n_tiles + 7) / 8);
  hipLaunchKernelGGL((k_gemm<T, MT, NT, EPI>), dim3(blocks), dim3(kGemmThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T, int EPI, int NT>
static hipError_t launch_mt(const GemmParams& p, int mt, hipStream_t st) {
  if (mt == 1) return launch_t<T, 1, NT, EPI>(p, st);
  return launch_t<T, 2, NT, EPI>(p, st);
}

template <typename T>
static hipError_t launch_epi(const GemmParams& p, int epi, int mt, hipStream_t st) {
  switch (epi) {
    case EPI_FC: return launch_mt<T, EPI_FC, 1>(p, mt, st);
    case EPI_INJECT: return launch_mt<T, EPI_INJECT, 1>(p, mt, st);
    case EPI_QKV: return launch_mt<T, EPI_QKV, 1>(p, mt, st);
    case EPI_RESID: return launch_mt<T, EPI_RESID, 1>(p, mt, st);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU, 2>(p, mt, st);
    default: return launch_mt<T, EPI_LMHEAD, 2>(p, mt, st);
  }
}

int gemm_k_per_iter(int dtype) { return dtype == 0 ? GemmCfg<float>::KI : GemmCfg<bf16_t>::KI; }

int gemm_tile_cols(int epi) { return (epi == EPI_SWIGLU || epi == EPI_LMHEAD) ? 32 : 16; }

hipError_t launch_gemm(int dtype, int epi, const GemmParams& p, int mt, hipStream_t st) {
  if (dtype == 0) return launch_epi<float>(p, epi, mt, st);
  return launch_epi<bf16_t>(p, epi, mt, st);
}

hipError_t launch_argmax_final(const float* tile_res, int n_tiles, int rows, int* draft_out, float* top2_out,
                               hipStream_t st) {
  hipLaunchKernelGGL(k_argmax_final, dim3(rows), dim3(256), 0, st, reinterpret_cast<const float4*>(tile_res),
                     n_tiles, draft_out, top2_out);
  return hipGetLastError();
}

}  // namespace dfl
