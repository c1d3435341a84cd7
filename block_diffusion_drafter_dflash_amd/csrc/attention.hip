// Non-causal block attention of the draft round (gfx950).
//
// Workgroup = (context chunk, kv head, stream) with QT waves; wave w owns 16 of the
// kv head's g * B queries (its g q-heads times the B block rows). Keys are the
// context rows in the layer's reach, read from the paged cache, plus all B block
// rows (added by the stream's last chunk). K and V^T tiles of 64 keys are staged in
// LDS, the next tile's cache reads already in flight while the current one is
// used. Scores are computed transposed (S^T = K Q^T) so that each lane owns one
// query: the softmax statistics are lane-local plus two cross-lane-group shuffles,
// and the probabilities feed the P.V MFMA without a transpose. P (fp32) enters the
// bf16 MFMA as three bf16 parts (hi, mid, lo) that hold all of its 24 bits, and the
// running output and denominator are kept in float64.
// A stream whose reach spans several chunks leaves per-chunk partials (max, sum,
// unnormalised output); k_attn_combine adds them in chunk order.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kKT = 64;       // keys per LDS tile
constexpr int kMaxBlock = 32; // block rows

template <typename T, int D>
struct AttnCfg {
  static constexpr int E = Elem<T>::E;
  static constexpr int PADK = 16 / sizeof(T);         // K rows padded by 16 bytes
  static constexpr int PADV = sizeof(T) == 2 ? 8 : 4; // V^T rows padded
  static constexpr int LDK = D + PADK;
  static constexpr int LDV = kKT + PADV;
  static constexpr int NF = D / 4 / E;                // 16-byte fragments per lane per query row
  static constexpr int CPK = D / E;                   // 16-byte chunks per key row
  static constexpr int NDT = D / 16;                  // 16-dim output tiles
};

template <typename T, int D, int QT>
__global__ __launch_bounds__(64 * QT) void k_attn(const AttnParams p) {
  using C = AttnCfg<T, D>;
  constexpr int E = C::E, NF = C::NF, CPK = C::CPK, NDT = C::NDT;
  constexpr int NTHR = 64 * QT;
  constexpr int NI = (kKT * CPK + NTHR - 1) / NTHR;   // cache chunks per thread per tile
  __shared__ __attribute__((aligned(16))) T ks[kKT][C::LDK];
  __shared__ __attribute__((aligned(16))) T vt[D][C::LDV];
  __shared__ double2 rope_tab[kMaxBlock][D / 2];      // (cos, sin) of the block positions

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = p.group, B = p.B, D_all_q = p.n_q_heads * D;
  const int nq_local = g * B;

  int Cs = p.ctx_len[s];
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int reach = Cs - lo;
  // Chunk length from this stream's own reach; its chunk count never exceeds the grid's.
  const int cl = reach > 0 ? attention_chunk_len(reach) : kKT;
  const int c_lo = lo + c * cl;
  const int c_hi = (c_lo + cl < Cs) ? c_lo + cl : Cs;
  const bool last_chunk = (c == p.n_chunks - 1);

  // Rotary angles of the block positions Cs + j (float64).
  for (int i = tid; i < B * (D / 2); i += NTHR) {
    const int j = i / (D / 2), f = i % (D / 2);
    const double inv_freq = pow((double)p.theta, -2.0 * (double)f / (double)D);
    double sn, cs;
    sincos((double)(Cs + j) * inv_freq, &sn, &cs);
    rope_tab[j][f] = make_double2(cs, sn);
  }
  __syncthreads();

  // Queries owned by this lane (MFMA column lr of wave w): q = RoPE(q_norm(raw q)),
  // rounded once to the MFMA input type. Lane group lg holds dims [lg*D/4, (lg+1)*D/4),
  // so the head's sum of squares is two shuffles away and each RoPE pair
  // (j, j + D/2) sits in lane groups lg and lg ^ 2.
  const int qi = 16 * w + lr;
  const bool q_valid = qi < nq_local;
  const int hl = q_valid ? qi / B : 0, jrow = q_valid ? qi % B : 0;
  const int qrow = s * B + jrow;
  const int qcol = (h * g + hl) * D;
  uint4 qf[NF];
  {
    constexpr int DL = D / 4;
    double x[DL];
    const double* qp = p.qkv_raw + (int64_t)qrow * p.ld_raw + qcol + lg * DL;
#pragma unroll
    for (int i = 0; i < DL; i += 2) {
      const double2 v = q_valid ? *reinterpret_cast<const double2*>(qp + i) : make_double2(0.0, 0.0);
      x[i] = v.x; x[i + 1] = v.y;
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < DL; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 16, kWave);
    ss += __shfl_xor(ss, 32, kWave);
    const double inv = 1.0 / sqrt(ss / (double)D + (double)p.eps);
    const T* gq = static_cast<const T*>(p.q_norm) + lg * DL;
#pragma unroll
    for (int i = 0; i < DL; ++i) x[i] = x[i] * inv * (double)Elem<T>::load1(gq + i);
    double o[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      const double xp = __shfl_xor(x[i], 32, kWave);
      const int j = lg * DL + i;
      const double2 cs = rope_tab[jrow][j < D / 2 ? j : j - D / 2];
      o[i] = q_valid ? (j < D / 2 ? x[i] * cs.x - xp * cs.y : x[i] * cs.x + xp * cs.y) : 0.0;
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) qf[f] = pack_d(o + f * E, T());
  }

  double oacc[NDT][4];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[dt][i] = 0.0;
  float m_run = -INFINITY;
  double l_run = 0.0;

  const int64_t head_stride = (int64_t)p.page_size * D;
  const int n_ctx_tiles = c_hi > c_lo ? (c_hi - c_lo + kKT - 1) / kKT : 0;
  const int n_tiles = n_ctx_tiles + (last_chunk ? 1 : 0);

  // Cache reads of one context tile into registers (invalid keys read as zero).
  uint4 kr[NI], vr[NI];
  auto fetch = [&](int t) {
    const int k0 = c_lo + t * kKT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ci = tid + i * NTHR;
      const int key = ci / CPK, part = ci % CPK;
      kr[i] = make_uint4(0, 0, 0, 0);
      vr[i] = make_uint4(0, 0, 0, 0);
      if (ci < kKT * CPK && k0 + key < c_hi) {
        const int pos = k0 + key;
        const int page = p.page_table[(int64_t)s * p.pages_per_stream + pos / p.page_size];
        if (page >= 0 && page < p.pool_pages) {
          const int64_t off = ((int64_t)page * p.n_kv_heads + h) * head_stride + (int64_t)(pos % p.page_size) * D + part * E;
          kr[i] = ldg16(static_cast<const T*>(p.kpool) + off);
          vr[i] = ldg16(static_cast<const T*>(p.vpool) + off);
        }
      }
    }
  };
  if (n_ctx_tiles > 0) fetch(0);

  for (int t = 0; t < n_tiles; ++t) {
    const bool blk = (t == n_ctx_tiles);
    const int nkeys = blk ? B : ((c_hi - (c_lo + t * kKT)) < kKT ? (c_hi - (c_lo + t * kKT)) : kKT);

    // ---- stage K rows and V^T into LDS
    if (blk) {
      // The block's own keys: k = RoPE(k_norm(raw k)), v = raw v, each rounded once.
      // D/8 consecutive threads own one key (8 dims each).
      constexpr int TPK = D / 8;
      for (int ci = tid; ci < kKT * TPK; ci += NTHR) {
        const int key = ci / TPK, part = ci % TPK;
        double kx[8], vx[8];
        const bool kvalid = key < nkeys;
        const double* kp = p.qkv_raw + (int64_t)(s * B + (kvalid ? key : 0)) * p.ld_raw + p.nq + h * D + part * 8;
        const double* vp = kp + p.nkv;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const double2 a = kvalid ? *reinterpret_cast<const double2*>(kp + i) : make_double2(0.0, 0.0);
          const double2 b = kvalid ? *reinterpret_cast<const double2*>(vp + i) : make_double2(0.0, 0.0);
          kx[i] = a.x; kx[i + 1] = a.y;
          vx[i] = b.x; vx[i + 1] = b.y;
        }
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += kx[i] * kx[i];
        for (int m = 1; m < TPK; m <<= 1) ss += __shfl_xor(ss, m, kWave);
        const double inv = 1.0 / sqrt(ss / (double)D + (double)p.eps);
        const T* gk = static_cast<const T*>(p.k_norm) + part * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) kx[i] = kx[i] * inv * (double)Elem<T>::load1(gk + i);
        double ko[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double kp2 = __shfl_xor(kx[i], TPK / 2, kWave);
          const int j = part * 8 + i;
          const double2 cs = rope_tab[kvalid ? key : 0][j < D / 2 ? j : j - D / 2];
          ko[i] = kvalid ? (j < D / 2 ? kx[i] * cs.x - kp2 * cs.y : kx[i] * cs.x + kp2 * cs.y) : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 8; i += E) *reinterpret_cast<uint4*>(&ks[key][part * 8 + i]) = pack_d(ko + i, T());
#pragma unroll
        for (int i = 0; i < 8; ++i) Elem<T>::store_d(&vt[part * 8 + i][key], kvalid ? vx[i] : 0.0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ci = tid + i * NTHR;
        if (ci < kKT * CPK) {
          const int key = ci / CPK, part = ci % CPK;
          *reinterpret_cast<uint4*>(&ks[key][part * E]) = kr[i];
          const T* ve = reinterpret_cast<const T*>(&vr[i]);
#pragma unroll
          for (int e = 0; e < E; ++e) vt[part * E + e][key] = ve[e];
        }
      }
    }
    __syncthreads();
    if (!blk && t + 1 < n_ctx_tiles) fetch(t + 1);   // next tile's reads overlap this tile's math

    // ---- S^T = K Q^T: lane holds query lr, keys 16 mt + 4 lg + i
    floatx4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      const T* krow = &ks[16 * mt + lr][lg * (D / 4)];
#pragma unroll
      for (int f = 0; f < NF; ++f) mma_frag(sacc[mt], *reinterpret_cast<const uint4*>(krow + f * E), qf[f], T());
    }

    // ---- online softmax (base 2); the denominator sums in float64
    float mx = -INFINITY;
    float pf[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * mt + 4 * lg + i;
        pf[mt][i] = key < nkeys ? sacc[mt][i] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, pf[mt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const double corr = (m_new == -INFINITY) ? 1.0 : (double)exp2f(m_run - m_new);
    double psum = 0.0;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[mt][i] = (m_new == -INFINITY || pf[mt][i] == -INFINITY) ? 0.f : exp2f(pf[mt][i] - m_new);
        psum += (double)pf[mt][i];
      }
    l_run = l_run * corr + psum;
    m_run = m_new;

    // ---- this tile's O^T = V^T P^T, added to the float64 running output
    floatx4 ot[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ot[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(T) == 2) {
      // P as hi + mid + lo bf16 parts: about 24 significant bits.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const float pv[8] = {pf[2 * kk][0], pf[2 * kk][1], pf[2 * kk][2], pf[2 * kk][3],
                             pf[2 * kk + 1][0], pf[2 * kk + 1][1], pf[2 * kk + 1][2], pf[2 * kk + 1][3]};
        float ph[8], pm[8], pl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ph[i] = Elem<T>::round(pv[i]);
          const float r1 = pv[i] - ph[i];     // exact: the leading 8 bits are gone
          pm[i] = Elem<T>::round(r1);
          pl[i] = Elem<T>::round(r1 - pm[i]);
        }
        const uint4 bh = pack(ph, T()), bm = pack(pm, T()), bl = pack(pl, T());
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* vrow = &vt[16 * dt + lr][0];
          const uint2 lo2 = *reinterpret_cast<const uint2*>(vrow + 32 * kk + 4 * lg);
          const uint2 hi2 = *reinterpret_cast<const uint2*>(vrow + 32 * kk + 16 + 4 * lg);
          const uint4 av = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
          mma_frag(ot[dt], av, bh, T());
          mma_frag(ot[dt], av, bm, T());
          mma_frag(ot[dt], av, bl, T());
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float pq[4] = {pf[mt][0], pf[mt][1], pf[mt][2], pf[mt][3]};
        const uint4 pb = pack(pq, T());
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint4 av = *reinterpret_cast<const uint4*>(&vt[16 * dt + lr][16 * mt + 4 * lg]);
          mma_frag(ot[dt], av, pb, T());
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] = oacc[dt][i] * corr + (double)ot[dt][i];
    __syncthreads();
  }

  double l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);

  if (p.n_chunks == 1) {
    if (!q_valid) return;
    T* op = static_cast<T*>(p.o) + (int64_t)qrow * D_all_q + qcol;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      double v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = oacc[dt][i] / l_tot;
      T* dst = op + 16 * dt + 4 * lg;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(bf16_from_double(v4[0]) | (bf16_from_double(v4[1]) << 16),
                                                    bf16_from_double(v4[2]) | (bf16_from_double(v4[3]) << 16));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4((float)v4[0], (float)v4[1], (float)v4[2], (float)v4[3]);
      }
    }
    return;
  }

  // ---- this chunk's (max, sum, unnormalised output) for k_attn_combine
  const int64_t sh = (int64_t)s * p.n_kv_heads + h;
  const int64_t chunk_id = sh * p.n_chunks + c;
  if (lg == 0) {
    float* ml = p.part_ml + (chunk_id * (QT * 16) + qi) * 2;
    ml[0] = m_run;
    ml[1] = (float)l_tot;
  }
  float* op = p.part_o + ((chunk_id * QT + w) * NDT) * (kWave * 4);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<float4*>(op + (dt * kWave + lane) * 4) =
        make_float4((float)oacc[dt][0], (float)oacc[dt][1], (float)oacc[dt][2], (float)oacc[dt][3]);
}

// Combine the chunks of one (stream, kv head, query tile, 16-dim slice) in chunk order.
template <typename T, int D>
__global__ __launch_bounds__(64) void k_attn_combine(const AttnParams p, int QT) {
  constexpr int NDT = D / 16;
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
  const int sh = blockIdx.x / QT, qt = blockIdx.x % QT, dt = blockIdx.y;
  const int s = sh / p.n_kv_heads, h = sh % p.n_kv_heads;
  const int qi = 16 * qt + lr;
  if (qi >= p.group * p.B) return;
  float M = -INFINITY;
  for (int cc = 0; cc < p.n_chunks; ++cc)
    M = fmaxf(M, p.part_ml[(((int64_t)sh * p.n_chunks + cc) * (QT * 16) + qi) * 2]);
  double L = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int cc = 0; cc < p.n_chunks; ++cc) {
    const int64_t chunk_id = (int64_t)sh * p.n_chunks + cc;
    const float* ml = p.part_ml + (chunk_id * (QT * 16) + qi) * 2;
    const double f = (ml[0] == -INFINITY) ? 0.0 : exp2((double)ml[0] - (double)M);
    L += (double)ml[1] * f;
    const float4 v =
        *reinterpret_cast<const float4*>(p.part_o + ((chunk_id * QT + qt) * NDT + dt) * (kWave * 4) + lane * 4);
    o[0] += (double)v.x * f;
    o[1] += (double)v.y * f;
    o[2] += (double)v.z * f;
    o[3] += (double)v.w * f;
  }
  const int hl = qi / p.B, jrow = qi % p.B;
  T* dst = static_cast<T*>(p.o) + (int64_t)(s * p.B + jrow) * (p.n_q_heads * D) + (h * p.group + hl) * D + 16 * dt + 4 * lg;
#pragma unroll
  for (int i = 0; i < 4; ++i) Elem<T>::store_d(dst + i, o[i] / L);
}

int attention_query_tiles(int group, int block) { return (group * block + 15) / 16; }

template <typename T, int D, int QT>
static void launch_qt(const AttnParams& p, hipStream_t st) {
  dim3 grid(p.n_chunks, p.n_kv_heads, p.S);
  hipLaunchKernelGGL((k_attn<T, D, QT>), grid, dim3(64 * QT), 0, st, p);
}

template <typename T, int D>
static hipError_t launch_td(const AttnParams& p, hipStream_t st) {
  const int qt = attention_query_tiles(p.group, p.B);
  switch (qt) {
    case 1: launch_qt<T, D, 1>(p, st); break;
    case 2: launch_qt<T, D, 2>(p, st); break;
    case 3: launch_qt<T, D, 3>(p, st); break;
    case 4: launch_qt<T, D, 4>(p, st); break;
    case 5: launch_qt<T, D, 5>(p, st); break;
    case 6: launch_qt<T, D, 6>(p, st); break;
    case 7: launch_qt<T, D, 7>(p, st); break;
    default: launch_qt<T, D, 8>(p, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_chunks == 1) return e;
  hipLaunchKernelGGL((k_attn_combine<T, D>), dim3(p.S * p.n_kv_heads * qt, D / 16), dim3(64), 0, st, p, qt);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st) {
  if (dtype == 0) return p.head_dim == 64 ? launch_td<float, 64>(p, st) : launch_td<float, 128>(p, st);
  return p.head_dim == 64 ? launch_td<bf16_t, 64>(p, st) : launch_td<bf16_t, 128>(p, st);
}

}  // namespace dfl
