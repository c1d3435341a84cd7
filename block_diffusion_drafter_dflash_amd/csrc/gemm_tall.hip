// Tiled MFMA GEMM of the draft round for many rows (M > 64: batched streams), gfx950.
//
// Y[M, N] = A[M, K] . W[N, K]^T with the same epilogues and outputs as the skinny
// kernel (float64 K-range partials, SwiGLU, LM-head logits and per-32-column top-2).
// A workgroup of 4 waves owns a 128-row x 64-column output tile over one K range.
// Chunks of 64 k are copied from global memory into LDS (A: 128 x 64, W: 64 x 64,
// XOR-swizzled 16-byte pieces for conflict-free fragment reads), the next two
// chunks' reads in flight in registers while the current chunk is multiplied. Each wave
// computes 32 rows x 64 columns with v_mfma_f32_16x16x32_bf16; every two chunks
// (128 products per element) the fp32 MFMA sums are added into float64
// accumulators. The row tiles of one column share an XCD and run back to back, so a
// weight tile read from HBM serves all of them from L2. The summation order differs
// from the skinny kernel's (one K sweep per K range rather than eight wave slices),
// so a batch on this path is not bitwise equal to the same streams drafted alone.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

namespace {

constexpr int kTallThreads = 256;
constexpr int BM = 128, BN = 64, BK = 64;
constexpr int kFlushChunks = 2;
constexpr int ROWB = BK * 2;           // bytes of one tile row in LDS (bf16)
constexpr int NCH = ROWB / 16;         // 16-byte pieces per tile row

__device__ __forceinline__ int swz(int row) { return (row >> 1) & (NCH - 1); }

__device__ __forceinline__ void tall_top_merge(float& v1, int& i1, float& v2, float bv1, int bi1, float bv2) {
  if (bv1 > v1 || (bv1 == v1 && bi1 < i1)) {
    v2 = fmaxf(v1, bv2);
    v1 = bv1;
    i1 = bi1;
  } else {
    v2 = fmaxf(v2, bv1);
  }
}

// Weight row of local column c (0..63) of column tile t.
template <int EPI>
__device__ __forceinline__ const bf16_t* tall_wrow(const GemmParams& p, int t, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    // tile t: columns 0..31 are gate rows 32t.., columns 32..63 the matching up rows
    const int r = 32 * t + (c & 31);
    return static_cast<const bf16_t*>(c < 32 ? p.w0 : p.w1) + (int64_t)r * p.K;
  } else if constexpr (EPI == EPI_RAW) {
    const int n = t * BN + c;
    if (p.seg_layers > 0) {
      const int l = n / (2 * p.nkv), rem = n % (2 * p.nkv);
      return static_cast<const bf16_t*>(rem < p.nkv ? p.wk_l[l] : p.wv_l[l]) + (int64_t)(rem % p.nkv) * p.K;
    }
    if (p.nq == 0 || n < p.nq) return static_cast<const bf16_t*>(p.w0) + (int64_t)n * p.K;
    if (n < p.nq + p.nkv) return static_cast<const bf16_t*>(p.w1) + (int64_t)(n - p.nq) * p.K;
    return static_cast<const bf16_t*>(p.w2) + (int64_t)(n - p.nq - p.nkv) * p.K;
  } else {
    int n = t * BN + c;
    n = n < p.N ? n : p.N - 1;   // ragged last tile: read a valid row, drop it later
    return static_cast<const bf16_t*>(p.w0) + (int64_t)n * p.K;
  }
}

}  // namespace

template <int EPI, int AM>
__global__ __launch_bounds__(kTallThreads) void k_gemm_tall(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_a[BM * ROWB];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[BN * ROWB];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int n_ct = EPI == EPI_SWIGLU ? p.N / BN : (p.N + BN - 1) / BN;   // column tiles
  const int n_rt = (p.M + BM - 1) / BM;                                   // row tiles
  // (column tile, K range) columns; the row tiles of a column are 8 apart (one XCD)
  const int wi = blockIdx.x;
  const int col = (wi / (8 * n_rt)) * 8 + wi % 8, rt = (wi / 8) % n_rt;
  if (col >= n_ct * p.ksplit) return;
  const int ks = col % p.ksplit, ct = col / p.ksplit;
  const int n_chunks = p.K / BK;
  const int kb = (int)((int64_t)ks * n_chunks / p.ksplit), ke = (int)((int64_t)(ks + 1) * n_chunks / p.ksplit);

  // This thread's share of a chunk: A rows (tid >> 3) + 32 j, piece tid & 7; W rows
  // (tid >> 3) + 32 j, same piece.
  const int piece = tid & 7, trow = tid >> 3;
  const bf16_t* arow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = rt * BM + trow + 32 * j;
    r = r < p.M ? r : p.M - 1;
    arow[j] = AM == A_TAPS ? nullptr : static_cast<const bf16_t*>(p.a) + (int64_t)r * p.lda;
  }
  const bf16_t* wrow[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) wrow[j] = tall_wrow<EPI>(p, ct, trow + 32 * j);

  auto fetch = [&](int ch, uint4 (&ra)[4], uint4 (&rb)[2]) {
    const int k = ch * BK + piece * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (AM == A_TAPS) {
        // a chunk never straddles two planes (hidden % 64 == 0)
        const int plane = (ch * BK) / p.tap_h;
        int r = rt * BM + trow + 32 * j;
        r = r < p.M ? r : p.M - 1;
        ra[j] = ldg16(static_cast<const bf16_t*>(p.taps[plane]) + (int64_t)r * p.tap_stride + (k - plane * p.tap_h));
      } else {
        ra[j] = ldg16(arow[j] + k);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) rb[j] = ldg16(wrow[j] + k);
  };
  auto stage = [&](const uint4 (&ra)[4], const uint4 (&rb)[2]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = trow + 32 * j;
      *reinterpret_cast<uint4*>(lds_a + r * ROWB + ((piece ^ swz(r)) * 16)) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = trow + 32 * j;
      *reinterpret_cast<uint4*>(lds_b + r * ROWB + ((piece ^ swz(r)) * 16)) = rb[j];
    }
  };

  // wave w: rows 32w..32w+31 of the tile (2 row tiles), all 64 columns (4 column tiles)
  double acc[2][4][4];
  floatx4 part[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      part[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0;
    }

  auto compute = [&](int ch) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int pc = sub * 4 + lg;
      uint4 af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 32 * w + 16 * i + lr;
        af[i] = *reinterpret_cast<const uint4*>(lds_a + r * ROWB + ((pc ^ swz(r)) * 16));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * j + lr;
        bf[j] = *reinterpret_cast<const uint4*>(lds_b + r * ROWB + ((pc ^ swz(r)) * 16));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma_frag(part[i][j], af[i], bf[j], bf16_t());
    }
    if ((ch - kb) % kFlushChunks == kFlushChunks - 1 || ch + 1 == ke) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] += (double)part[i][j][e];
          part[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }
  };

  // Pipeline: chunk ch is in LDS while the reads of chunks ch + 1 and ch + 2 are in
  // flight in two register sets used alternately.
  if (kb < ke) {
    uint4 ra0[4], rb0[2], ra1[4], rb1[2];
    fetch(kb, ra0, rb0);
    if (kb + 1 < ke) fetch(kb + 1, ra1, rb1);
    stage(ra0, rb0);
    __syncthreads();
    // body(ch, next, free): `next` holds chunk ch + 1's reads; `free` takes ch + 2's
    auto body = [&](int ch, uint4 (&na)[4], uint4 (&nb)[2], uint4 (&fa)[4], uint4 (&fb)[2]) {
      if (ch + 2 < ke) fetch(ch + 2, fa, fb);
      compute(ch);
      __syncthreads();
      if (ch + 1 < ke) {
        stage(na, nb);
        __syncthreads();
      }
    };
    for (int ch = kb; ch < ke; ch += 2) {
      body(ch, ra1, rb1, ra0, rb0);
      if (ch + 1 < ke) body(ch + 1, ra0, rb0, ra1, rb1);
    }
  }

  // ---- epilogue: lane holds rows 32w + 16i + 4lg + e, columns 16j + lr
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt * BM + 32 * w + 16 * i + 4 * lg + e;
      const bool rv = r < p.M;
      if constexpr (EPI == EPI_RAW) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = ct * BN + 16 * j + lr;
          if (rv && n < p.N) p.y_out[((int64_t)ks * p.M + r) * p.N + n] = acc[i][j][e];
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const double g = acc[i][j][e], u = acc[i][j + 2][e];
          if (rv) Elem<bf16_t>::store_d(static_cast<bf16_t*>(p.m_out) + (int64_t)r * p.ld_out + 32 * ct + 16 * j + lr,
                                       g / (1.0 + exp(-g)) * u);
        }
      } else {   // EPI_LMHEAD: fp32 logits and top-2 of each 32-column group
#pragma unroll
        for (int jg = 0; jg < 2; ++jg) {
          float v1 = -INFINITY, v2 = -INFINITY;
          int i1 = 0x7fffffff;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = ct * BN + 32 * jg + 16 * jj + lr;
            const float v = (float)acc[i][2 * jg + jj][e];
            if (n < p.N) {
              if (rv && p.logits_out) p.logits_out[(int64_t)r * p.N + n] = v;
              tall_top_merge(v1, i1, v2, v, n, -INFINITY);
            }
          }
          for (int m = 1; m < 16; m <<= 1) {
            const float o1 = __shfl_xor(v1, m, kWave);
            const int oi = __shfl_xor(i1, m, kWave);
            const float o2 = __shfl_xor(v2, m, kWave);
            tall_top_merge(v1, i1, v2, o1, oi, o2);
          }
          const int grp = 2 * ct + jg;
          if (rv && lr == 0 && grp < p.n_tiles)
            reinterpret_cast<float4*>(p.tile_res)[(int64_t)r * p.n_tiles + grp] = make_float4(v1, __int_as_float(i1), v2, 0.f);
        }
      }
    }
}

int gemm_tall_column_tiles(int epi, int N) { return epi == EPI_SWIGLU ? N / BN : (N + BN - 1) / BN; }

// K ranges of the tiled GEMM: about 256 (column tile, K range) pairs, each range at
// least 8 chunks; a function of the weight's shape only, so that a row's arithmetic
// does not depend on how many rows the batch has.
int gemm_tall_ksplit(int epi, int N, int K) {
  if (epi != EPI_RAW) return 1;
  const int tiles = gemm_tall_column_tiles(epi, N);
  int ks = (256 + tiles / 2) / tiles;
  const int cap = K / BK / 8 > 1 ? K / BK / 8 : 1;
  ks = ks < cap ? ks : cap;
  return ks < 1 ? 1 : (ks > 8 ? 8 : ks);
}

hipError_t launch_gemm_tall(int epi, int am, const GemmParams& p, hipStream_t st) {
  const int n_ct = gemm_tall_column_tiles(epi, p.N), n_rt = (p.M + BM - 1) / BM;
  const int grid = (n_ct * p.ksplit + 7) / 8 * 8 * n_rt;
  if (epi == EPI_RAW && am == A_TAPS)
    (void)launch_k(k_gemm_tall<EPI_RAW, A_TAPS>, dim3(grid), dim3(kTallThreads), st, p);
  else if (epi == EPI_RAW)
    (void)launch_k(k_gemm_tall<EPI_RAW, A_PLAIN>, dim3(grid), dim3(kTallThreads), st, p);
  else if (epi == EPI_SWIGLU)
    (void)launch_k(k_gemm_tall<EPI_SWIGLU, A_PLAIN>, dim3(grid), dim3(kTallThreads), st, p);
  else
    (void)launch_k(k_gemm_tall<EPI_LMHEAD, A_PLAIN>, dim3(grid), dim3(kTallThreads), st, p);
  return hipGetLastError();
}

}  // namespace dfl
