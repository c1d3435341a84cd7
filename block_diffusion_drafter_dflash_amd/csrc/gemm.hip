// Skinny MFMA GEMMs of the draft round with fused epilogues (gfx950).
//
// Y[M, N] = A[M, K] . W[N, K]^T with M small (block rows x streams) and W streamed
// from HBM exactly once. A workgroup owns one work item: a tile of 32 output columns
// for 16*MT rows over one of the GEMM's ksplit ranges of K. W comes in the packed
// layout (dflash_pack_weights): the tile's rows as consecutive 4 KB chunks of 32 rows
// x 128 bytes, so a K range of a tile is one contiguous region, and inside a chunk the
// bytes stand in MFMA fragment order, so that each of a wave's four loads of a chunk
// is 1 KB contiguous. The KW waves take the range's chunks in turn, so the workgroup
// streams KW consecutive chunks at a time, with the wave's next chunk in flight; the
// loads are nontemporal (the weights are read once). Measured on the 9B shapes, this
// reads HBM at 5.7-6.7 TB/s where row-major chunks (each load 16 rows x 64 bytes of a
// 2 KB span) reach 5.0-6.0 and 32 rows read side by side 3.0-5.6. Every MFMA's partial (32 products per element for
// bf16) is added into a float64 accumulator and the KW wave partials are summed in
// wave order. With ksplit > 1 each range writes its own float64 partial and the
// consuming kernel adds the ranges in order (see kernels.h), so no workgroup ever
// waits for another and every result is independent of scheduling and of the
// batch: ksplit, KW and U depend only on the weight's shape, never on M.
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

// 16-byte load that bypasses the caches' retention (each weight is read once).
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// First byte of 4-bit packed tile `tile` (K / 64 chunks of kQ4Chunk bytes).
__device__ __forceinline__ const unsigned char* packed_tile_q4(const GemmParams& p, int tile) {
  const int64_t tile_bytes = (int64_t)(p.K / kQ4Group) * kQ4Chunk;
  if (p.wp_seg_tiles > 0)
    return static_cast<const unsigned char*>(p.wp_l[tile / p.wp_seg_tiles]) + (int64_t)(tile % p.wp_seg_tiles) * tile_bytes;
  return static_cast<const unsigned char*>(p.wp) + (int64_t)tile * tile_bytes;
}

// Eight 4-bit codes (nibble e = code e) -> eight bf16 values, exactly (0..15).
// The two masks leave each code in a byte of its own, so that every code is one
// byte-to-float conversion (v_cvt_f32_ubyte0..3 read any byte directly). The empty
// asm statements (no instruction) keep lo and hi opaque: otherwise the compiler
// folds each (lo >> 8k) & 0xff back into a bit-field extract from c, one more
// instruction a code.
__device__ __forceinline__ uint4 codes_to_bf16(uint32_t c) {
  uint32_t lo = c & 0x0F0F0F0Fu, hi = (c >> 4) & 0x0F0F0F0Fu;
  asm("" : "+v"(lo));
  asm("" : "+v"(hi));
  return make_uint4(f32x2_to_bf16x2((float)(lo & 0xffu), (float)(hi & 0xffu)),
                    f32x2_to_bf16x2((float)((lo >> 8) & 0xffu), (float)((hi >> 8) & 0xffu)),
                    f32x2_to_bf16x2((float)((lo >> 16) & 0xffu), (float)((hi >> 16) & 0xffu)),
                    f32x2_to_bf16x2((float)(lo >> 24), (float)(hi >> 24)));
}

// WQ = 1: B is the 4-bit packing (bf16 only). The MFMAs then run on the codes
// themselves (exact in bf16) and on all-ones, giving per 64-weight group g the sums
// P = sum_k x_k q_k and X = sum_k x_k; the group adds scale_g P + bias_g X, which is
// sum_k x_k (bias_g + scale_g q_k), the product with the dequantized weights.
template <typename T, int MT, int NT, int EPI, int AM, int WQ, typename Tune>
__global__ __launch_bounds__(Tune::KW * kWave) void k_gemm(const GemmParams p) {
  using C = GemmCfg<T, Tune>;
  constexpr int E = C::E, U = C::U, KI = C::KI, KW = C::KW, THREADS = C::THREADS;
  constexpr int ROWS = 16 * MT, COLS = 16 * NT;
  __shared__ float red[KW][ROWS][COLS + 1];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  // Work item: a column (tile, K range) and a row group. Workgroups are dealt to the
  // eight XCDs round-robin, so the row groups of one column are placed 8 apart: they
  // land on the same XCD back to back and share the column's weights in its L2.
  const int wi = blockIdx.x;
  const int col = (wi / (8 * p.mgroups)) * 8 + wi % 8, mg = (wi / 8) % p.mgroups;
  if (col >= p.n_tiles * p.ksplit) return;
  const int ks = col % p.ksplit, tile = col / p.ksplit;
  const int row0 = mg * ROWS;
  const int kb = (int)((int64_t)ks * p.iters / p.ksplit), ke = (int)((int64_t)(ks + 1) * p.iters / p.ksplit);
  const int lane_k = lg * (U * E);
  static_assert(16 * NT == kPackTileRows && KI * (int)sizeof(T) == 128, "a packed chunk is 32 rows of 128 bytes");

  // Packed weights: iteration `it` of this tile is the chunk at tw + it * 32 * KI, whose
  // fragment (nt, u) (1 KB at (2 nt + u) * 1 KB) holds at lane l's 16 bytes the piece
  // this lane multiplies: row 16 nt + lr, elements lane_k + u E .. of the chunk's KI.
  // The KW waves take the range's chunks in turn (wave w: kb + w, kb + w + KW, ...), so
  // at any time the workgroup streams KW consecutive 4 KB chunks of one region.
  const T* tw = packed_tile<T>(p, tile);
  const unsigned char* tq = WQ ? packed_tile_q4(p, tile) : nullptr;
  static_assert(!WQ || (sizeof(T) == 2 && KI == kQ4Group && U == 2 && NT == 2), "4-bit groups are one bf16 chunk");
  static_assert(U == 2 && NT == 2, "a chunk is four 1 KB fragments (nt, u)");
  int boff[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) boff[nt] = (2 * nt * kWave + lane) * E;
  int64_t aoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = row0 + 16 * mt + lr;
    r = r < p.M ? r : p.M - 1;
    aoff[mt] = AM == A_TAPS ? (int64_t)r * p.tap_stride : (int64_t)r * p.lda;
  }
  const T* abase = static_cast<const T*>(p.a);
  auto load = [&](int it, uint4 (&a)[MT][U], uint4 (&bb)[NT][U]) {
    const int k = it * KI + lane_k;
    if constexpr (WQ) {
      // the lane's 16 bytes of codes, then rows lr and 16 + lr's (scale, bias)
      const unsigned char* ch = tq + (int64_t)it * kQ4Chunk;
      bb[0][0] = ldg16(ch + 16 * lane);
      const uint2 sb = *reinterpret_cast<const uint2*>(ch + 1024 + 8 * lr);
      bb[0][1] = make_uint4(sb.x, sb.y, 0u, 0u);
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < U; ++u) bb[nt][u] = ldg16_nt(tw + (int64_t)it * (kPackTileRows * KI) + boff[nt] + u * kWave * E);
    }
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

  double acc[MT][NT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][nt][i] = 0.0;

  if (kb + w < ke) {
    uint4 a_c[MT][U], b_c[NT][U];
    load(kb + w, a_c, b_c);
    for (int it = kb + w; it < ke; it += KW) {
      uint4 a_n[MT][U], b_n[NT][U];
      const bool more = it + KW < ke;
      if (more) load(it + KW, a_n, b_n);
      if constexpr (WQ) {
        // codes of rows lr (dwords x, y) and 16 + lr (z, w), k = 16 lg + 8 u ..
        uint4 bq[NT][U];
        bq[0][0] = codes_to_bf16(b_c[0][0].x);
        bq[0][1] = codes_to_bf16(b_c[0][0].y);
        bq[1][0] = codes_to_bf16(b_c[0][0].z);
        bq[1][1] = codes_to_bf16(b_c[0][0].w);
        const uint32_t sbw[NT] = {b_c[0][1].x, b_c[0][1].y};
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          floatx4 xs = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < U; ++u) mma_frag(xs, a_c[mt][u], ones, T());
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            floatx4 part = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < U; ++u) mma_frag(part, a_c[mt][u], bq[nt][u], T());
            const float scale = bf16_to_f32(sbw[nt] & 0xffffu), bias = bf16_to_f32(sbw[nt] >> 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] += (double)fmaf(scale, part[i], bias * xs[i]);
          }
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            // an iteration's U MFMAs (U * KF products) are summed in fp32, then added
            // into the float64 accumulator
            floatx4 part = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < U; ++u) mma_frag(part, a_c[mt][u], b_c[nt][u], T());
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][nt][i] += (double)part[i];
          }
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
  }

  // ---- the KW K slices -> LDS, summed in wave order in float64. Each wave's float64
  // slice is stored as fp32 (one more rounding, of a slice about 1/sqrt(KW) of the
  // sum): a float64 array would double this LDS and cost the 9B round 0.5% and the
  // 4-bit round 5% for about a fifth fewer outputs rounded the other way in bf16.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[w][16 * mt + 4 * lg + i][16 * nt + lr] = (float)acc[mt][nt][i];
  __syncthreads();

  // ---- epilogue: one element per thread and pass; COLS consecutive lanes per row
#pragma unroll
  for (int e0 = 0; e0 < ROWS * COLS; e0 += THREADS) {
    const int e = e0 + tid;
    if (e >= ROWS * COLS) break;   // whole waves (ROWS * COLS is a multiple of 64)
    const int rl = e / COLS, c = e % COLS;
    double vd = 0.0;
#pragma unroll
    for (int ww = 0; ww < KW; ++ww) vd += (double)red[ww][rl][c];
    const float v = (float)vd;
    const int r = row0 + rl;
    const bool rv = r < p.M;
    const int n = tile * COLS + c;

    if constexpr (EPI == EPI_RAW) {
      // this K range's float64 partial; the consumer adds the ranges in order
      if (rv) p.y_out[((int64_t)ks * p.M + r) * p.N + n] = vd;
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

// Final argmax over the LM head's column tiles: one workgroup of 1024 threads per
// mask row. The (max, index, second max) merge is order-independent (largest value,
// lowest index among equals, largest remaining value), so the split over threads
// does not change the result.
constexpr int kArgmaxThreads = 1024;
__global__ __launch_bounds__(kArgmaxThreads) void k_argmax_final(const float4* tile_res, int n_tiles, int* draft_out,
                                                                 float* top2_out) {
  constexpr int NW = kArgmaxThreads / kWave;
  __shared__ float s1[NW], s2[NW];
  __shared__ int si[NW];
  const int r = blockIdx.x, tid = threadIdx.x;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff;
#pragma unroll 4
  for (int t = tid; t < n_tiles; t += kArgmaxThreads) {
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
    for (int k = 1; k < NW; ++k) top_merge(v1, i1, v2, s1[k], si[k], s2[k]);
    draft_out[r] = i1;
    if (top2_out) {
      top2_out[2 * r] = v1;
      top2_out[2 * r + 1] = v2;
    }
  }
}

// ------------------------------------------------------------------ host launchers

// Tuning per GEMM kind, from a sweep over (waves, bytes per lane per row and
// iteration, tile width, K ranges) on the 9B round's shapes: 32-column tiles
// everywhere, 8 waves reading 32 bytes per lane and row, 4 waves for the LM head.
enum TuneId { TUNE_W8_U2 = 0, TUNE_W4_U2 = 1 };

static int tune_of(int epi, int, int, int) { return epi == EPI_LMHEAD ? TUNE_W4_U2 : TUNE_W8_U2; }

template <typename T, int MT, int NT, int EPI, int AM, typename Tune>
static hipError_t launch_tuned(const GemmParams& p, hipStream_t st) {
  // columns padded to a multiple of 8 so that every column's row groups share an XCD
  const int grid = (p.n_tiles * p.ksplit + 7) / 8 * 8 * p.mgroups;
  if constexpr (sizeof(T) == 2) {
    if (p.q4) {
      (void)launch_k(k_gemm<T, MT, NT, EPI, AM, 1, Tune>, dim3(grid), dim3(GemmCfg<T, Tune>::THREADS), st, p);
      return hipGetLastError();
    }
  }
  (void)launch_k(k_gemm<T, MT, NT, EPI, AM, 0, Tune>, dim3(grid), dim3(GemmCfg<T, Tune>::THREADS), st, p);
  return hipGetLastError();
}

template <typename T, int MT, int NT, int EPI, int AM>
static hipError_t launch_t(const GemmParams& p, hipStream_t st) {
  if (tune_of(EPI, AM, p.K, p.tap_h) == TUNE_W4_U2) return launch_tuned<T, MT, NT, EPI, AM, GemmTune<4, 2>>(p, st);
  return launch_tuned<T, MT, NT, EPI, AM, GemmTune<8, 2>>(p, st);
}

template <typename T, int EPI, int NT, int AM>
static hipError_t launch_mt(const GemmParams& p, int mt, hipStream_t st) {
  if (mt == 1) return launch_t<T, 1, NT, EPI, AM>(p, st);
  if (mt == 2) return launch_t<T, 2, NT, EPI, AM>(p, st);
  return launch_t<T, 4, NT, EPI, AM>(p, st);
}

template <typename T>
static hipError_t launch_epi(const GemmParams& p, int epi, int am, int mt, hipStream_t st) {
  switch (epi) {
    case EPI_RAW:
      return am == A_TAPS ? launch_mt<T, EPI_RAW, 2, A_TAPS>(p, mt, st) : launch_mt<T, EPI_RAW, 2, A_PLAIN>(p, mt, st);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU, 2, A_PLAIN>(p, mt, st);
    default: return launch_mt<T, EPI_LMHEAD, 2, A_PLAIN>(p, mt, st);
  }
}

int gemm_k_per_iter(int dtype, int epi, int am, int K, int tap_h) {
  const int kf = dtype == 0 ? Elem<float>::KF : Elem<bf16_t>::KF;
  (void)epi;
  (void)am;
  (void)K;
  (void)tap_h;
  return 2 * kf;   // U = 2 for every tuning in use
}

int gemm_tile_cols(int) { return 32; }

// K ranges of a GEMM, a function of the weight's shape only. Preferred: the fewest
// ranges that give at least one workgroup per CU (two for K >= 16384) and deal the
// work items evenly over the MI355X's 256 CUs; otherwise about that many workgroups.
// Every range keeps at least 16 iterations.
constexpr int kCUs = 256;
int gemm_ksplit(int epi, int n_tiles, int iters, int K) {
  if (epi != EPI_RAW) return 1;
  const int target = K >= 16384 ? 2 * kCUs : kCUs;
  int cap = iters / 16 > 1 ? iters / 16 : 1;
  cap = cap < 8 ? cap : 8;
  for (int ks = 1; ks <= cap; ++ks)
    if (n_tiles * ks >= target && (n_tiles * ks) % kCUs == 0) return ks;
  int ks = (target + n_tiles / 2) / n_tiles;
  ks = ks < cap ? ks : cap;
  return ks < 1 ? 1 : ks;
}

hipError_t launch_gemm(int dtype, int epi, int am, const GemmParams& p, int mt, hipStream_t st) {
  if (dtype == 0) return launch_epi<float>(p, epi, am, mt, st);
  return launch_epi<bf16_t>(p, epi, am, mt, st);
}

hipError_t launch_argmax_final(const float* tile_res, int n_tiles, int rows, int* draft_out, float* top2_out,
                               hipStream_t st) {
  (void)launch_k(k_argmax_final, dim3(rows), dim3(kArgmaxThreads), st, reinterpret_cast<const float4*>(tile_res),
                     n_tiles, draft_out, top2_out);
  return hipGetLastError();
}

}  // namespace dfl
