// Skinny MFMA GEMMs of the draft round with fused epilogues (gfx950).
//
// Y[M, N] = A[M, K] . W[N, K]^T with M small (block rows x streams) and W streamed
// from HBM once. A workgroup (4 waves) owns a 128-column tile of Y for 16*MT rows
// over one K split; wave w owns columns [32w, 32w+32) of the tile (two 16x16 MFMA
// fragments per 16-row group). Each lane streams 64 contiguous bytes of a weight row
// per iteration. When K is split over several workgroups, each writes its fp32 partial
// in fragment order; the last one to arrive (an atomic counter, no waiting) sums the
// partials in split order, so results do not depend on arrival order. The summed tile
// goes through LDS into an epilogue chosen at compile time.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

template <typename T>
struct GemmCfg {
  static constexpr int E = Elem<T>::E;
  static constexpr int KF = Elem<T>::KF;
  static constexpr int U = 4;             // 16-byte fragments per lane per row per iteration
  static constexpr int KI = U * KF;       // k-elements per iteration
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

// How each epilogue's GEMM reads its A operand (fixed at compile time).
template <int EPI>
struct AModeOf {
  static constexpr int value = EPI == EPI_FC ? A_TAPS
                               : (EPI == EPI_QKV || EPI == EPI_SWIGLU || EPI == EPI_LMHEAD) ? A_NORMED
                                                                                            : A_PLAIN;
};

template <typename T, int MT, int EPI>
__global__ __launch_bounds__(kBlockThreads) void k_gemm(const GemmParams p) {
  using C = GemmCfg<T>;
  constexpr int AM = AModeOf<EPI>::value;
  constexpr int E = C::E, U = C::U, KI = C::KI;
  constexpr int ROWS = 16 * MT;
  constexpr int LDT = kTileN + 4;
  __shared__ float tile_s[ROWS][LDT];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int S = p.splits;
  const int tile = blockIdx.x / S, sp = blockIdx.x % S;
  const int mg = blockIdx.y;
  const int row0 = mg * ROWS;

  // ---------------- operand row pointers (fixed for the whole K loop)
  const T* brow[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    int c = 32 * w + 16 * nt + lr;            // column within the tile
    int n = tile * kTileN + c;
    const T* base;
    if constexpr (EPI == EPI_SWIGLU) {
      int r = tile * (kTileN / 2) + (c & 63);
      base = static_cast<const T*>(c < 64 ? p.w0 : p.w1) + (int64_t)r * p.K;
    } else if constexpr (EPI == EPI_QKV) {
      if (n < p.nq) base = static_cast<const T*>(p.w0) + (int64_t)n * p.K;
      else if (n < p.nq + p.nkv) base = static_cast<const T*>(p.w1) + (int64_t)(n - p.nq) * p.K;
      else base = static_cast<const T*>(p.w2) + (int64_t)(n - p.nq - p.nkv) * p.K;
    } else if constexpr (EPI == EPI_INJECT) {
      int l = n / (2 * p.nkv), rem = n % (2 * p.nkv);
      base = static_cast<const T*>(rem < p.nkv ? p.wk_l[l] : p.wv_l[l]) + (int64_t)(rem % p.nkv) * p.K;
    } else {
      int nn = n < p.N ? n : p.N - 1;          // ragged last tile: read a valid row, drop it later
      base = static_cast<const T*>(p.w0) + (int64_t)nn * p.K;
    }
    brow[nt] = base;
  }
  int64_t aoff[MT];   // element offset of each lane's A row in its source
  float ainv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = row0 + 16 * mt + lr;
    r = r < p.M ? r : p.M - 1;
    int xr = p.a_rowmap_bm1 > 0 ? (r / p.a_rowmap_bm1) * (p.a_rowmap_bm1 + 1) + 1 + r % p.a_rowmap_bm1 : r;
    aoff[mt] = AM == A_TAPS ? (int64_t)r * p.tap_stride : (int64_t)xr * p.lda;
    ainv[mt] = AM == A_NORMED ? p.a_inv[xr] : 1.0f;
  }
  const T* abase = static_cast<const T*>(p.a);

  floatx4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int it0 = (int)((int64_t)sp * p.iters / S), it1 = (int)((int64_t)(sp + 1) * p.iters / S);
  const int lane_k = lg * (U * E);

  auto load_a = [&](int it, uint4 (&a)[MT][U], uint4 (&g)[U]) {
    const int k = it * KI + lane_k;
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
  auto load_b = [&](int it, uint4 (&b)[2][U]) {
    const int k = it * KI + lane_k;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int u = 0; u < U; ++u) b[nt][u] = ldg16(brow[nt] + k + u * E);
  };

  if (it0 < it1) {
    uint4 a_c[MT][U], g_c[U], b_c[2][U];
    load_a(it0, a_c, g_c);
    load_b(it0, b_c);
    for (int it = it0; it < it1; ++it) {
      const int itn = it + 1 < it1 ? it + 1 : it;
      uint4 a_n[MT][U], g_n[U], b_n[2][U];
      load_b(itn, b_n);
      load_a(itn, a_n, g_n);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float gf[E];
        if constexpr (AM == A_NORMED) unpack(g_c[u], gf, T());
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          uint4 av = a_c[mt][u];
          if constexpr (AM == A_NORMED) {
            float xf[E];
            unpack(av, xf, T());
#pragma unroll
            for (int e = 0; e < E; ++e) xf[e] = xf[e] * ainv[mt] * gf[e];
            av = pack(xf, T());
          }
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) mma_frag(acc[mt][nt], av, b_c[nt][u], T());
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        g_c[u] = g_n[u];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a_c[mt][u] = a_n[mt][u];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) b_c[nt][u] = b_n[nt][u];
      }
    }
  }

  // ---------------- split-K: publish the partial, the last arrival reduces in split order
  if (S > 1) {
    const int64_t frag_stride = (int64_t)MT * 2 * kWave * 4;   // floats per wave
    const int64_t tile_id = (int64_t)mg * p.n_tiles + tile;
    const int64_t ntile_total = (int64_t)gridDim.y * p.n_tiles;
    float* mine = p.partials + ((sp * ntile_total + tile_id) * 4 + w) * frag_stride;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        *reinterpret_cast<floatx4*>(mine + ((mt * 2 + nt) * kWave + lane) * 4) = acc[mt][nt];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
      int old = atomicAdd(p.counters + tile_id, 1);
      s_last = (old == S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    // Loads of four splits are issued together, then added in split order.
    constexpr int SB = 4;
    for (int s0 = 0; s0 < S; s0 += SB) {
      floatx4 v[SB][MT][2];
#pragma unroll
      for (int i = 0; i < SB; ++i) {
        const int s2 = s0 + i < S ? s0 + i : S - 1;
        const float* src = p.partials + ((s2 * ntile_total + tile_id) * 4 + w) * frag_stride;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            v[i][mt][nt] = *reinterpret_cast<const floatx4*>(src + ((mt * 2 + nt) * kWave + lane) * 4);
      }
#pragma unroll
      for (int i = 0; i < SB; ++i)
        if (s0 + i < S) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[mt][nt] += v[i][mt][nt];
        }
    }
    if (tid == 0) p.counters[tile_id] = 0;   // every split has arrived: reset for the next use
  }

  // ---------------- fragments -> LDS tile [ROWS][128]
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) tile_s[16 * mt + 4 * lg + i][32 * w + 16 * nt + lr] = acc[mt][nt][i];
  __syncthreads();

  // ---------------- epilogue: thread -> (row, 8 columns); 16 threads per row
  const int er = tid >> 4, ec = (tid & 15) * 8;
#pragma unroll
  for (int pass = 0; pass < MT; ++pass) {
    const int rl = 16 * pass + er;
    const int r = row0 + rl;
    const bool rv = r < p.M;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tile_s[rl][ec + i];
    const int n = tile * kTileN + ec;

    if constexpr (EPI == EPI_FC) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
      ss = xor_sum(ss, 16);
      if (rv) {
        float* y = p.y_out + (int64_t)r * p.N + n;
        *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(y + 4) = make_float4(v[4], v[5], v[6], v[7]);
        if ((tid & 15) == 0) p.ssq_part[(int64_t)r * p.n_tiles + tile] = ss;
      }
    } else if constexpr (EPI == EPI_RESID) {
      float ss = 0.f;
      if (rv) {
        T* x = static_cast<T*>(p.x_io) + (int64_t)r * p.N + n;
        uint4 xv = ldg16(x);
        uint4 xv2 = xv;
        float xf[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if constexpr (E == 4) {
          xv2 = ldg16(x + 4);
          unpack(xv, xf, T());
          unpack(xv2, xf + 4, T());
        } else {
          unpack(xv, xf, T());
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xf[i] = Elem<T>::round(xf[i] + v[i]);
          ss += xf[i] * xf[i];
        }
        if constexpr (E == 4) {
          stg16(x, pack(xf, T()));
          stg16(x + 4, pack(xf + 4, T()));
        } else {
          stg16(x, pack(xf, T()));
        }
      }
      ss = xor_sum(ss, 16);
      if (rv && (tid & 15) == 0) p.ssq_part[(int64_t)r * p.n_tiles + tile] = ss;
    } else if constexpr (EPI == EPI_SWIGLU) {
      float up[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) up[i] = __shfl_xor(v[i], 8, kWave);
      if (rv && ec < 64) {
        float m[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float g = v[i];
          m[i] = g / (1.0f + expf(-g)) * up[i];
        }
        T* dst = static_cast<T*>(p.m_out) + (int64_t)r * p.ld_out + tile * (kTileN / 2) + ec;
        if constexpr (E == 4) {
          stg16(dst, pack(m, T()));
          stg16(dst + 4, pack(m + 4, T()));
        } else {
          stg16(dst, pack(m, T()));
        }
      }
    } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
      // Which tensor this tile belongs to, and the column inside it.
      int kind, col, layer = 0;
      const int d = p.head_dim;
      if constexpr (EPI == EPI_QKV) {
        if (n < p.nq) { kind = 0; col = n; }
        else if (n < p.nq + p.nkv) { kind = 1; col = n - p.nq; }
        else { kind = 2; col = n - p.nq - p.nkv; }
      } else {
        layer = n / (2 * p.nkv);
        int rem = n % (2 * p.nkv);
        kind = rem < p.nkv ? 1 : 2;
        col = rem % p.nkv;
      }
      const int dd = col % d;                 // first head-local dim of this thread
      float o[8];
      if (kind != 2) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
        ss = xor_sum(ss, d / 8);
        const float inv = 1.0f / sqrtf(ss / (float)d + p.eps);
        const T* gain;
        if constexpr (EPI == EPI_QKV) gain = static_cast<const T*>(kind == 0 ? p.qn_gain : p.kn_gain);
        else gain = static_cast<const T*>(p.kn_l[layer]);
        float xn[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xn[i] = v[i] * inv * Elem<T>::load1(gain + dd + i);
        float xp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) xp[i] = __shfl_xor(xn[i], d / 16, kWave);
        int pos = 0;
        if (rv) {
          if constexpr (EPI == EPI_QKV) {
            int s = r / p.block;
            int c = p.ctx_len[s];
            c = c < 0 ? 0 : (c > p.max_ctx ? p.max_ctx : c);
            pos = c + r % p.block;
          } else {
            pos = p.row_pos[r];
          }
        }
        const int half = d / 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = dd + i;
          float cs, sn;
          rope_cs(pos, j < half ? j : j - half, d, p.theta, cs, sn);
          o[i] = j < half ? xn[i] * cs - xp[i] * sn : xn[i] * cs + xp[i] * sn;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = v[i];
      }
      if (rv) {
        T* dst = nullptr;
        if constexpr (EPI == EPI_QKV) {
          T* base = static_cast<T*>(kind == 0 ? p.q_out : (kind == 1 ? p.k_out : p.v_out));
          const int ld = kind == 0 ? p.nq : p.nkv;
          dst = base + (int64_t)r * ld + col;
        } else {
          const int s = p.row_stream[r], pos = p.row_pos[r];
          const int span = p.pages_per_stream * p.page_size;
          if (s >= 0 && s < p.max_streams && pos >= 0 && pos < span) {
            const int page = p.page_table[(int64_t)s * p.pages_per_stream + pos / p.page_size];
            if (page >= 0 && page < p.pool_pages) {
              T* pool = static_cast<T*>(kind == 1 ? p.kpool_l[layer] : p.vpool_l[layer]);
              const int head = col / d;
              dst = pool + ((((int64_t)page * p.n_kv_heads + head) * p.page_size + pos % p.page_size) * d + dd);
            }
          }
        }
        if (dst) {
          if constexpr (E == 4) {
            stg16(dst, pack(o, T()));
            stg16(dst + 4, pack(o + 4, T()));
          } else {
            stg16(dst, pack(o, T()));
          }
        }
      }
    } else if constexpr (EPI == EPI_LMHEAD) {
      float v1 = -INFINITY, v2 = -INFINITY;
      int i1 = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (n + i < p.N) top_merge(v1, i1, v2, v[i], n + i, -INFINITY);
      if (rv && p.logits_out) {
        T* dst = static_cast<T*>(p.logits_out) + (int64_t)r * p.N + n;
        if (n + 8 <= p.N && (p.N % E) == 0) {
          if constexpr (E == 4) {
            stg16(dst, pack(v, T()));
            stg16(dst + 4, pack(v + 4, T()));
          } else {
            stg16(dst, pack(v, T()));
          }
        } else {
          for (int i = 0; i < 8; ++i)
            if (n + i < p.N) {
              if constexpr (E == 4) dst[i] = v[i];
              else dst[i] = (T)f32_to_bf16(v[i]);
            }
        }
      }
      top_xor_merge(v1, i1, v2, 16);
      if ((tid & 15) == 0) {
        float4* tr = reinterpret_cast<float4*>(p.tile_res) + ((int64_t)mg * p.n_tiles + tile) * ROWS + rl;
        *tr = make_float4(v1, __int_as_float(i1), v2, 0.f);
      }
    }
  }

  // ---------------- second level: per-row statistics over all column tiles
  if constexpr (EPI == EPI_RESID || EPI == EPI_LMHEAD) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
      int old = atomicAdd(p.counters2 + mg, 1);
      s_last = (old == p.n_tiles - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (tid == 0) p.counters2[mg] = 0;
    if constexpr (EPI == EPI_RESID) {
      for (int rl = tid; rl < ROWS; rl += kBlockThreads) {
        const int r = row0 + rl;
        if (r < p.M) {
          float ss = 0.f;
          for (int t = 0; t < p.n_tiles; ++t) ss += p.ssq_part[(int64_t)r * p.n_tiles + t];
          p.inv_out[r] = (float)(1.0 / sqrt((double)ss / (double)p.N + (double)p.eps));
        }
      }
    } else {
#pragma unroll
      for (int pass = 0; pass < MT; ++pass) {
        const int rl = 16 * pass + er;
        const int r = row0 + rl;
        float v1 = -INFINITY, v2 = -INFINITY;
        int i1 = 0x7fffffff;
        for (int t = (tid & 15); t < p.n_tiles; t += 16) {
          float4 tr = reinterpret_cast<const float4*>(p.tile_res)[((int64_t)mg * p.n_tiles + t) * ROWS + rl];
          top_merge(v1, i1, v2, tr.x, __float_as_int(tr.y), tr.z);
        }
        top_xor_merge(v1, i1, v2, 16);
        if (r < p.M && (tid & 15) == 0) {
          p.draft_out[r] = i1;
          if (p.top2_out) {
            p.top2_out[2 * r] = v1;
            p.top2_out[2 * r + 1] = v2;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ host launchers

template <typename T, int MT, int EPI>
static hipError_t launch_t(const GemmParams& p, int mgroups, hipStream_t st) {
  dim3 grid(p.n_tiles * p.splits, mgroups);
  hipLaunchKernelGGL((k_gemm<T, MT, EPI>), grid, dim3(kBlockThreads), 0, st, p);
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_mt(const GemmParams& p, int mt, int mgroups, hipStream_t st) {
  switch (mt) {
    case 1: return launch_t<T, 1, EPI>(p, mgroups, st);
    case 2: return launch_t<T, 2, EPI>(p, mgroups, st);
    default: return launch_t<T, 4, EPI>(p, mgroups, st);
  }
}

template <typename T>
static hipError_t launch_epi(const GemmParams& p, int epi, int mt, int mgroups, hipStream_t st) {
  switch (epi) {
    case EPI_FC: return launch_mt<T, EPI_FC>(p, mt, mgroups, st);
    case EPI_INJECT: return launch_mt<T, EPI_INJECT>(p, mt, mgroups, st);
    case EPI_QKV: return launch_mt<T, EPI_QKV>(p, mt, mgroups, st);
    case EPI_RESID: return launch_mt<T, EPI_RESID>(p, mt, mgroups, st);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU>(p, mt, mgroups, st);
    default: return launch_mt<T, EPI_LMHEAD>(p, mt, mgroups, st);
  }
}

int gemm_k_per_iter(int dtype) {
  return dtype == 0 ? GemmCfg<float>::KI : GemmCfg<bf16_t>::KI;
}

hipError_t launch_gemm(int dtype, int epi, const GemmParams& p, int mt, int mgroups, hipStream_t st) {
  if (dtype == 0) return launch_epi<float>(p, epi, mt, mgroups, st);
  return launch_epi<bf16_t>(p, epi, mt, mgroups, st);
}

}  // namespace dfl
