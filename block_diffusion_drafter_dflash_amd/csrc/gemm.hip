// Skinny MFMA GEMMs of the draft round with fused epilogues (gfx950).
//
// Y[M, N] = A[M, K] . W[N, K]^T with M small (block rows x streams) and W streamed
// from HBM exactly once. A work item is a tile of 16*NT output columns for 16*MT
// rows; a workgroup of 8 waves takes a contiguous run of work items (row groups of
// one tile back to back, so a tile's weight rows are re-read from the same L2) and
// its waves split K eight ways. Each wave streams its slice of the tile's weight
// rows, every lane reading 64 contiguous bytes of a row per iteration; the loads of
// the next iteration - also across work items - are in flight while the current
// one is multiplied, so the next tile's reads overlap this tile's epilogue.
// Every MFMA's partial (32 products per element for bf16) is added into a float64
// accumulator and the eight wave partials are summed in wave order. No workgroup
// ever waits for another: row statistics (sums of squares for the next RMSNorm)
// leave as per-tile partials that the consuming kernel adds in tile order, so every
// result is independent of scheduling and of the batch.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

// Tuning of one GEMM kernel: KW waves per workgroup split K; each lane reads U
// 16-byte fragments (U * 16 contiguous bytes) of each of its rows per iteration.
template <int KW_, int U_>
struct GemmTune {
  static constexpr int KW = KW_;
  static constexpr int U = U_;
};
using DefaultTune = GemmTune<8, 4>;

template <typename T, typename Tune>
struct GemmCfg {
  static constexpr int E = Elem<T>::E;
  static constexpr int KF = Elem<T>::KF;
  static constexpr int KW = Tune::KW;
  static constexpr int U = Tune::U;
  static constexpr int KI = U * KF;     // k-elements per iteration
  static constexpr int THREADS = KW * kWave;
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

// Weight row of output column tile * (16 * NT) + c.
template <typename T, int NT, int EPI>
__device__ __forceinline__ const T* weight_row(const GemmParams& p, int tile, int c) {
  const int n = tile * (16 * NT) + c;
  if constexpr (EPI == EPI_SWIGLU) {
    // tile t: columns 0..15 are gate rows 16t.., columns 16..31 the matching up rows
    const int r = tile * 16 + (c & 15);
    return static_cast<const T*>(c < 16 ? p.w0 : p.w1) + (int64_t)r * p.K;
  } else if constexpr (EPI == EPI_RAW) {
    if (p.seg_layers > 0) {   // per layer [wk | wv]
      const int l = n / (2 * p.nkv), rem = n % (2 * p.nkv);
      return static_cast<const T*>(rem < p.nkv ? p.wk_l[l] : p.wv_l[l]) + (int64_t)(rem % p.nkv) * p.K;
    }
    if (n < p.nq) return static_cast<const T*>(p.w0) + (int64_t)n * p.K;
    if (n < p.nq + p.nkv) return static_cast<const T*>(p.w1) + (int64_t)(n - p.nq) * p.K;
    return static_cast<const T*>(p.w2) + (int64_t)(n - p.nq - p.nkv) * p.K;
  } else {
    const int nn = n < p.N ? n : p.N - 1;   // ragged last tile: read a valid row, drop it later
    return static_cast<const T*>(p.w0) + (int64_t)nn * p.K;
  }
}

template <typename T, int MT, int NT, int EPI, typename Tune = DefaultTune>
__global__ __launch_bounds__(Tune::KW * kWave) void k_gemm(const GemmParams p) {
  using C = GemmCfg<T, Tune>;
  constexpr int E = C::E, U = C::U, KI = C::KI, kKW = C::KW, kGemmThreads = C::THREADS;
  constexpr int AM = EPI == EPI_FC ? A_TAPS : A_PLAIN;
  constexpr int ROWS = 16 * MT, COLS = 16 * NT;
  __shared__ float red[kKW][ROWS][COLS + 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // contiguous run of work items (tile-major, row group fastest)
  const int G = gridDim.x, b = blockIdx.x;
  const int q0 = (int)((int64_t)b * p.n_work / G), q1 = (int)((int64_t)(b + 1) * p.n_work / G);
  if (q0 >= q1) return;

  const int it0 = (int)((int64_t)w * p.iters / kKW), it1 = (int)((int64_t)(w + 1) * p.iters / kKW);
  const bool has_k = it0 < it1;
  const int lane_k = lg * (U * E);
  const T* abase = static_cast<const T*>(p.a);

  // load cursor: work item, iteration and the item's row pointers
  int l_wi = q0, l_it = it0;
  const T* brow[NT];
  int64_t aoff[MT];
  auto setup = [&](int wi) {
    const int tile = wi / p.mgroups, mg = wi % p.mgroups;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) brow[nt] = weight_row<T, NT, EPI>(p, tile, 16 * nt + lr);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int r = mg * ROWS + 16 * mt + lr;
      r = r < p.M ? r : p.M - 1;
      aoff[mt] = AM == A_TAPS ? (int64_t)r * p.tap_stride : (int64_t)r * p.lda;
    }
  };
  auto load = [&](int it, uint4 (&a)[MT][U], uint4 (&bb)[NT][U]) {
    const int k = it * KI + lane_k;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int u = 0; u < U; ++u) bb[nt][u] = ldg16(brow[nt] + k + u * E);
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
  };

  setup(l_wi);
  uint4 a_c[MT][U], b_c[NT][U];
  if (has_k) load(l_it, a_c, b_c);

  for (int wi = q0; wi < q1; ++wi) {
    double acc[MT][NT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.0;

    for (int it = it0; it < it1; ++it) {
      // advance the load cursor and start the next iteration's reads
      if (++l_it == it1) {
        l_it = it0;
        if (++l_wi < q1) setup(l_wi);
      }
      uint4 a_n[MT][U], b_n[NT][U];
      const bool more = l_wi < q1;
      if (more) load(l_it, a_n, b_n);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            // each MFMA's partial (KF products) is added into the float64 accumulator
            floatx4 part = floatx4{0.f, 0.f, 0.f, 0.f};
            mma_frag(part, a_c[mt][u], b_c[nt][u], T());
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] += (double)part[i];
          }
      if (more) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) a_c[mt][u] = a_n[mt][u];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) b_c[nt][u] = b_n[nt][u];
        }
      }
    }

    // ---- the eight K slices -> LDS, summed in wave order
    const int tile = wi / p.mgroups, row0 = (wi % p.mgroups) * ROWS;
    __syncthreads();   // the previous item's epilogue has read red
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
      } else if constexpr (EPI == EPI_RAW) {
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

// Persistent grid: as many workgroups as the device holds at once (its CU count times
// the kernel's resident workgroups per CU), capped by the work items.
template <typename T, int MT, int NT, int EPI, typename Tune>
static int resident_grid(int n_work) {
  constexpr int kMaxDevices = 64;
  static int cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemm<T, MT, NT, EPI, Tune>,
                                                     GemmCfg<T, Tune>::THREADS, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cached[dev] = cus * per_cu;
  }
  return n_work < cached[dev] ? n_work : cached[dev];
}

// Tuning per GEMM kind, from a sweep over (waves, bytes per lane per row and
// iteration, grid) on the 9B round's shapes: the wide-N kinds run one workgroup per
// tile with 32-byte reads per lane and row, the fc GEMM (N = hidden, K = taps x
// hidden) keeps a resident grid with 128-byte reads when hidden allows it.
enum TuneId { TUNE_W8_U2 = 0, TUNE_W4_U2 = 1, TUNE_W4_U8 = 2, TUNE_W8_U4 = 3 };

static int tune_of(int epi, int K, int tap_h) {
  if (epi == EPI_LMHEAD) return TUNE_W4_U2;
  if (epi == EPI_FC) return tap_h % 256 == 0 && K % 256 == 0 ? TUNE_W4_U8 : TUNE_W8_U4;
  return TUNE_W8_U2;
}

template <typename T, int MT, int NT, int EPI, typename Tune>
static hipError_t launch_tuned(const GemmParams& p, bool persistent, hipStream_t st) {
  const int grid = persistent ? resident_grid<T, MT, NT, EPI, Tune>(p.n_work) : p.n_work;
  (void)launch_k(k_gemm<T, MT, NT, EPI, Tune>, dim3(grid), dim3(GemmCfg<T, Tune>::THREADS), st, p);
  return hipGetLastError();
}

template <typename T, int MT, int NT, int EPI>
static hipError_t launch_t(const GemmParams& p, hipStream_t st) {
  switch (tune_of(EPI, p.K, p.tap_h)) {
    case TUNE_W4_U2: return launch_tuned<T, MT, NT, EPI, GemmTune<4, 2>>(p, false, st);
    case TUNE_W4_U8: return launch_tuned<T, MT, NT, EPI, GemmTune<4, 8>>(p, true, st);
    case TUNE_W8_U4: return launch_tuned<T, MT, NT, EPI, GemmTune<8, 4>>(p, true, st);
    default: return launch_tuned<T, MT, NT, EPI, GemmTune<8, 2>>(p, false, st);
  }
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
    case EPI_RAW: return launch_mt<T, EPI_RAW, 1>(p, mt, st);
    case EPI_RESID: return launch_mt<T, EPI_RESID, 1>(p, mt, st);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU, 2>(p, mt, st);
    default: return launch_mt<T, EPI_LMHEAD, 2>(p, mt, st);
  }
}

int gemm_k_per_iter(int dtype, int epi, int K, int tap_h) {
  const int kf = dtype == 0 ? Elem<float>::KF : Elem<bf16_t>::KF;
  switch (tune_of(epi, K, tap_h)) {
    case TUNE_W4_U8: return 8 * kf;
    case TUNE_W8_U4: return 4 * kf;
    default: return 2 * kf;
  }
}

int gemm_tile_cols(int epi) { return (epi == EPI_SWIGLU || epi == EPI_LMHEAD) ? 32 : 16; }

hipError_t launch_gemm(int dtype, int epi, const GemmParams& p, int mt, hipStream_t st) {
  if (dtype == 0) return launch_epi<float>(p, epi, mt, st);
  return launch_epi<bf16_t>(p, epi, mt, st);
}

hipError_t launch_argmax_final(const float* tile_res, int n_tiles, int rows, int* draft_out, float* top2_out,
                               hipStream_t st) {
  (void)launch_k(k_argmax_final, dim3(rows), dim3(256), st, reinterpret_cast<const float4*>(tile_res),
                     n_tiles, draft_out, top2_out);
  return hipGetLastError();
}

}  // namespace dfl
