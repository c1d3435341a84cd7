// Small kernels of the draft round (gfx950): block input gather, row RMSNorms, the
// block heads' norm + RoPE, injected K/V placement, greedy verify.
#include <type_traits>

#include "common.hpp"
#include "kernels.h"

namespace dfl {

// Deterministic sum over a workgroup of NT threads: butterfly inside each wave,
// then the wave sums in wave order.
template <int NT>
__device__ double block_sum(double v, double* red) {
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = red[0];
  for (int i = 1; i < NT / kWave; ++i) t += red[i];
  return t;
}

// E consecutive values, the in-order float64 sum of ksplit partials [ks][rows][ld]:
// ((P_0 + P_1) + P_2) + ..., the loads of up to four partials in flight at once. The
// partials are float64 (skinny GEMM) or float32 (tiled GEMM, whose sums are fp32 and
// convert to float64 exactly).
template <typename P, int E>
__device__ __forceinline__ void sum_parts_t(const P* parts, int ksplit, int64_t ks_stride, int64_t off,
                                            double (&out)[E]) {
  constexpr int KR = 4;
  using P2 = typename std::conditional<sizeof(P) == 8, double2, float2>::type;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = 0.0;
  for (int k0 = 0; k0 < ksplit; k0 += KR) {
    P2 v[KR][E / 2];
#pragma unroll
    for (int k = 0; k < KR; ++k)
      if (k0 + k < ksplit)
#pragma unroll
        for (int e = 0; e < E; e += 2) v[k][e / 2] = *reinterpret_cast<const P2*>(parts + (k0 + k) * ks_stride + off + e);
#pragma unroll
    for (int k = 0; k < KR; ++k)
      if (k0 + k < ksplit)
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          if (k0 + k == 0) {
            out[e] = (double)v[k][e / 2].x;
            out[e + 1] = (double)v[k][e / 2].y;
          } else {
            out[e] += (double)v[k][e / 2].x;
            out[e + 1] += (double)v[k][e / 2].y;
          }
        }
  }
}
template <int E>
__device__ __forceinline__ void sum_parts(const void* parts, int f32, int ksplit, int64_t ks_stride, int64_t off,
                                          double (&out)[E]) {
  if (f32) sum_parts_t<float, E>(static_cast<const float*>(parts), ksplit, ks_stride, off, out);
  else sum_parts_t<double, E>(static_cast<const double*>(parts), ksplit, ks_stride, off, out);
}

// Row kernels: kNormThreads threads a row, thread t owning the CH groups of E
// consecutive elements at (g * kNormThreads + t) * E, kept in registers between the
// sum of squares and the scaling (hidden <= kNormThreads * E * CH).
constexpr int kNormThreads = 512;

// Block rows: X[s*B] = embed[anchor[s]], X[s*B + j] = embed[mask] for j >= 1, and the
// first layer's normalised input a = round(X / sqrt(mean(X^2) + eps) * gain).
template <typename T, int CH>
__global__ __launch_bounds__(kNormThreads) void k_embed(const EmbedParams p) {
  constexpr int E = Elem<T>::E, NT = kNormThreads;
  __shared__ double red[NT / kWave];
  const int r = blockIdx.x;
  const int s = r / p.B, j = r % p.B;
  int tok = j == 0 ? p.anchor[s] : p.mask_token;
  tok = tok < 0 ? 0 : (tok >= p.vocab ? p.vocab - 1 : tok);
  const T* src = static_cast<const T*>(p.embed) + (int64_t)tok * p.hidden;
  T* dst = static_cast<T*>(p.x) + (int64_t)r * p.hidden;
  T* a = static_cast<T*>(p.a) + (int64_t)r * p.hidden;
  const T* gn = static_cast<const T*>(p.gain);
  if (threadIdx.x < p.head_dim / 2) {
    // this row's rotary table, for every layer of the round
    int Cs = p.ctx_len[s];
    Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
    const int i = threadIdx.x;
    const double inv_freq = pow((double)p.theta, -2.0 * (double)i / (double)p.head_dim);
    double sn, cs;
    sincos((double)(Cs + j) * inv_freq, &sn, &cs);
    p.rope[(int64_t)r * (p.head_dim / 2) + i] = make_double2(cs, sn);
  }
  uint4 v[CH], g[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      v[ch] = ldg16(src + c);
      g[ch] = ldg16(gn + c);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      stg16(dst + c, v[ch]);
      float f[E];
      unpack(v[ch], f, T());
#pragma unroll
      for (int e = 0; e < E; ++e) ss += (double)f[e] * (double)f[e];
    }
  }
  ss = block_sum<NT>(ss, red);
  const double inv = 1.0 / sqrt(ss / (double)p.hidden + (double)p.eps);
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      float f[E], gf[E];
      double y[E];
      unpack(v[ch], f, T());
      unpack(g[ch], gf, T());
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = (double)f[e] * inv * (double)gf[e];
      stg16(a + c, pack_d(y, T()));
    }
  }
}

// One row of the residual stream: x = round(x + branch) when the branch's partials
// are given, then a = round(x / sqrt(mean(x^2) + eps) * gain), the sum of squares
// taken over the stored (rounded) x in a fixed tree order.
template <typename T, int CH>
__global__ __launch_bounds__(kNormThreads) void k_norm(const NormParams p) {
  constexpr int E = Elem<T>::E, NT = kNormThreads;
  __shared__ double red[NT / kWave];
  const int r = blockIdx.x;
  const int bm1 = p.rowmap_bm1;
  const int xr = bm1 > 0 ? (r / bm1) * (bm1 + 1) + 1 + r % bm1 : r;
  T* x = static_cast<T*>(p.x) + (int64_t)xr * p.hidden;
  const T* gn = static_cast<const T*>(p.gain);
  const int64_t ks_stride = (int64_t)p.part_rows * p.hidden;
  uint4 v[CH], g[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      v[ch] = ldg16(x + c);
      g[ch] = ldg16(gn + c);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      float f[E];
      if (p.parts) {
        double br[E], xn[E];
        sum_parts<E>(p.parts, p.parts_f32, p.ksplit, ks_stride, (int64_t)xr * p.hidden + c, br);
        unpack(v[ch], f, T());
#pragma unroll
        for (int e = 0; e < E; ++e) xn[e] = (double)f[e] + br[e];
        v[ch] = pack_d(xn, T());
        stg16(x + c, v[ch]);
      }
      unpack(v[ch], f, T());
#pragma unroll
      for (int e = 0; e < E; ++e) ss += (double)f[e] * (double)f[e];
    }
  }
  ss = block_sum<NT>(ss, red);
  const double inv = 1.0 / sqrt(ss / (double)p.hidden + (double)p.eps);
  T* a = static_cast<T*>(p.a) + (int64_t)r * p.hidden;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      float f[E], gf[E];
      double y[E];
      unpack(v[ch], f, T());
      unpack(g[ch], gf, T());
#pragma unroll
      for (int e = 0; e < E; ++e) y[e] = (double)f[e] * inv * (double)gf[e];
      stg16(a + c, pack_d(y, T()));
    }
  }
}

// Block rows' heads: q = RoPE(q_norm(raw q)), k = RoPE(k_norm(raw k)), v = raw v,
// each rounded once. One wave per (row, head); lane l holds the rotary pair
// (l, l + D/2), rotated by the round's table (written by k_embed). k goes to the
// stream's block key page [32][D], v to its transposed value page [D][32]; the row-0
// wave of a head also clears slots B..31 of both.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_qkv_finish(const QkvFinishParams p) {
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int s = r / p.B, j = r % p.B;
  const int n_heads = p.n_q_heads + 2 * p.n_kv_heads;
  const int hi = blockIdx.y * 4 + (tid >> 6);
  const bool head_ok = hi < n_heads;
  const int nq = p.n_q_heads * D, ld = nq + 2 * p.n_kv_heads * D;
  const bool on = head_ok && lane < D / 2;
  const int64_t src_off = (int64_t)r * ld + (int64_t)(head_ok ? hi : 0) * D;
  const double* src = static_cast<const double*>(p.raw) + src_off;
  const float* srcf = static_cast<const float*>(p.raw) + src_off;
  const int64_t ks_stride = (int64_t)p.S * p.B * ld;
  double v0[8], v1[8];
  if (on) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < p.ksplit) {
        const int64_t o = k * ks_stride + lane;
        v0[k] = p.raw_f32 ? (double)srcf[o] : src[o];
        v1[k] = p.raw_f32 ? (double)srcf[o + D / 2] : src[o + D / 2];
      }
  }
  if (!head_ok) return;
  double x0 = 0.0, x1 = 0.0;
  if (on) {
    // ((P_0 + P_1) + P_2) + ...: the first eight from registers, the rest eight at a time
    for (int k0 = 0; k0 < p.ksplit; k0 += 8) {
      if (k0 > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k0 + k < p.ksplit) {
            const int64_t o = (k0 + k) * ks_stride + lane;
            v0[k] = p.raw_f32 ? (double)srcf[o] : src[o];
            v1[k] = p.raw_f32 ? (double)srcf[o + D / 2] : src[o + D / 2];
          }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k0 + k < p.ksplit) {
          x0 = k0 + k == 0 ? v0[k] : x0 + v0[k];
          x1 = k0 + k == 0 ? v1[k] : x1 + v1[k];
        }
    }
  }
  if (hi >= p.n_q_heads + p.n_kv_heads) {
    const int vh = hi - p.n_q_heads - p.n_kv_heads;
    T* vb = static_cast<T*>(p.vblk) + ((int64_t)s * p.n_kv_heads + vh) * (D * kBlockSlots);
    if (on) {
      Elem<T>::store_d(vb + lane * kBlockSlots + j, x0);
      Elem<T>::store_d(vb + (lane + D / 2) * kBlockSlots + j, x1);
      if (j == 0)
        for (int jj = p.B; jj < kBlockSlots; ++jj) {
          Elem<T>::store_d(vb + lane * kBlockSlots + jj, 0.0);
          Elem<T>::store_d(vb + (lane + D / 2) * kBlockSlots + jj, 0.0);
        }
    }
    return;
  }
  const bool is_q = hi < p.n_q_heads;
  double ss = x0 * x0 + x1 * x1;
  for (int m = 1; m < kWave; m <<= 1) ss += __shfl_xor(ss, m, kWave);
  if (!on) return;
  const double inv = 1.0 / sqrt(ss / (double)D + (double)p.eps);
  const T* gn = static_cast<const T*>(is_q ? p.q_norm : p.k_norm);
  const double y0 = x0 * inv * (double)Elem<T>::load1(gn + lane);
  const double y1 = x1 * inv * (double)Elem<T>::load1(gn + lane + D / 2);
  const double2 cs = p.rope[(int64_t)r * (D / 2) + lane];
  const double o0 = y0 * cs.x - y1 * cs.y, o1 = y1 * cs.x + y0 * cs.y;
  if (is_q) {
    T* q = static_cast<T*>(p.q) + (int64_t)r * nq + (int64_t)hi * D;
    Elem<T>::store_d(q + lane, o0);
    Elem<T>::store_d(q + lane + D / 2, o1);
  } else {
    const int kh = hi - p.n_q_heads;
    T* kb = static_cast<T*>(p.kblk) + ((int64_t)s * p.n_kv_heads + kh) * (kBlockSlots * D);
    Elem<T>::store_d(kb + j * D + lane, o0);
    Elem<T>::store_d(kb + j * D + lane + D / 2, o1);
    if (j == 0)
      for (int jj = p.B; jj < kBlockSlots; ++jj) {
        Elem<T>::store_d(kb + jj * D + lane, 0.0);
        Elem<T>::store_d(kb + jj * D + lane + D / 2, 0.0);
      }
  }
}

// Context K/V of injected rows: K = RoPE_pos(k_norm(raw k)) per kv head, V = raw v,
// rounded and written to the row's page slot (K pages [16][D], V pages [D][16]). One workgroup per (row, layer);
// D/8 consecutive threads own one head (8 dims each).
template <typename T, int D>
__global__ __launch_bounds__(256) void k_kv_finish(const KvFinishParams p) {
  __shared__ double2 tab[D / 2];
  const int r = blockIdx.x, l = blockIdx.y, tid = threadIdx.x;
  const int s = p.row_stream[r], pos = p.row_pos[r];
  const int span = p.pages_per_stream * p.page_size;
  if (s < 0 || s >= p.max_streams || pos < 0 || pos >= span) return;
  const int page = p.page_table[(int64_t)s * p.pages_per_stream + pos / p.page_size];
  if (page < 0 || page >= p.pool_pages) return;
  for (int i = tid; i < D / 2; i += 256) {
    const double inv_freq = pow((double)p.theta, -2.0 * (double)i / (double)D);
    double sn, cs;
    sincos((double)pos * inv_freq, &sn, &cs);
    tab[i] = make_double2(cs, sn);
  }
  __syncthreads();
  constexpr int TPH = D / 8;
  const int nkvd = p.n_kv_heads * D;
  const int64_t raw_off = (int64_t)r * (p.n_layers * 2 * nkvd) + (int64_t)l * 2 * nkvd;   // range 0
  const int items = 2 * p.n_kv_heads * TPH;
  for (int it = tid; it < items; it += 256) {
    const int kind = it / (p.n_kv_heads * TPH), rem = it % (p.n_kv_heads * TPH);
    const int head = rem / TPH, part = rem % TPH;
    double x[8];
    sum_parts<8>(p.raw, p.raw_f32, p.ksplit, (int64_t)p.R * p.n_layers * 2 * nkvd,
                 raw_off + (int64_t)kind * nkvd + head * D + part * 8, x);
    // norm and rotation are computed for every item (shuffles stay inside a head's
    // TPH lanes); only K items keep them
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
    for (int m = 1; m < TPH; m <<= 1) ss += __shfl_xor(ss, m, kWave);
    const double inv = 1.0 / sqrt(ss / (double)D + (double)p.eps);
    const T* gk = static_cast<const T*>(p.kn_l[l]) + part * 8;
    double xn[8], o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xn[i] = x[i] * inv * (double)Elem<T>::load1(gk + i);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double xp = __shfl_xor(xn[i], TPH / 2, kWave);
      const int j = part * 8 + i;
      const double2 cs = tab[j < D / 2 ? j : j - D / 2];
      const double rot = j < D / 2 ? xn[i] * cs.x - xp * cs.y : xn[i] * cs.x + xp * cs.y;
      o[i] = kind == 0 ? rot : x[i];
    }
    const int64_t ph = (int64_t)page * p.n_kv_heads + head;
    if (kind == 0) {   // K page [16][D]
      T* dst = static_cast<T*>(p.kpool_l[l]) + (ph * p.page_size + pos % p.page_size) * D + part * 8;
      constexpr int E = Elem<T>::E;
#pragma unroll
      for (int i = 0; i < 8; i += E) stg16(dst + i, pack_d(o + i, T()));
    } else {           // V page stored transposed, [D][16]
      T* dst = static_cast<T*>(p.vpool_l[l]) + (ph * D + part * 8) * p.page_size + pos % p.page_size;
#pragma unroll
      for (int i = 0; i < 8; ++i) Elem<T>::store_d(dst + i * p.page_size, o[i]);
    }
  }
}

// Fused rows: y = the fc GEMM's partials added in range order; out = round(y /
// sqrt(mean(y^2) + eps) * gain), the squares summed in a fixed tree order.
template <typename T, int CH>
__global__ __launch_bounds__(kNormThreads) void k_rownorm(const RowNormParams p) {
  constexpr int E = Elem<T>::E, NT = kNormThreads;
  __shared__ double red[NT / kWave];
  const int r = blockIdx.x;
  const int64_t ks_stride = (int64_t)p.R * p.hidden, off = (int64_t)r * p.hidden;
  const T* gn = static_cast<const T*>(p.gain);
  double y[CH][E];
  uint4 g[CH];
  double ss = 0.0;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      g[ch] = ldg16(gn + c);
      sum_parts<E>(p.parts, p.parts_f32, p.ksplit, ks_stride, off + c, y[ch]);
#pragma unroll
      for (int e = 0; e < E; ++e) ss += y[ch][e] * y[ch][e];
    }
  }
  ss = block_sum<NT>(ss, red);
  const double inv = 1.0 / sqrt(ss / (double)p.hidden + (double)p.eps);
  T* out = static_cast<T*>(p.out) + off;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int c = (ch * NT + threadIdx.x) * E;
    if (c < p.hidden) {
      float gf[E];
      double o[E];
      unpack(g[ch], gf, T());
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = y[ch][e] * inv * (double)gf[e];
      stg16(out + c, pack_d(o, T()));
    }
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

// Weights into the skinny GEMM's packed layout: one thread a 16-byte piece. Packed
// piece i is piece i % 8 of row (i / 8) % 32 of chunk (i / 256) % chunks of tile
// i / (256 chunks); its source is the same 16 bytes of output column 32 tile + row's
// weight row (zero past N).
__global__ __launch_bounds__(256) void k_pack(const PackJob j) {
  const int64_t chunks = (int64_t)j.K * j.esize / 128;
  const int64_t tiles = (j.N + kPackTileRows - 1) / kPackTileRows;
  const int64_t total = tiles * chunks * (kPackTileRows * 8);
  const int64_t row_bytes = (int64_t)j.K * j.esize;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    // 16-byte unit d of a chunk: fragment f = d / 64 (= 2 nt + u), lane l = d % 64
    // (= 16 lg + lr), holding piece 2 lg + u of tile row 16 nt + lr
    const int d = (int)(i % (8 * kPackTileRows)), f = d >> 6, l = d & 63;
    const int row = 16 * (f >> 1) + (l & 15), piece = 2 * (l >> 4) + (f & 1);
    const int64_t chunk = (i / (8 * kPackTileRows)) % chunks, tile = i / (8 * kPackTileRows * chunks);
    const int64_t n = tile * kPackTileRows + row;
    const char* src = nullptr;
    if (n < j.N) {
      if (j.kind == PACK_SWIGLU) {
        const int64_t r = tile * 16 + (row & 15);
        src = static_cast<const char*>(row < 16 ? j.w0 : j.w1) + r * row_bytes;
      } else if (j.kind == PACK_QKV) {
        src = n < j.nq ? static_cast<const char*>(j.w0) + n * row_bytes
                       : (n < j.nq + j.nkv ? static_cast<const char*>(j.w1) + (n - j.nq) * row_bytes
                                           : static_cast<const char*>(j.w2) + (n - j.nq - j.nkv) * row_bytes);
      } else {
        src = static_cast<const char*>(j.w0) + n * row_bytes;
      }
    }
    const uint4 v = src ? ldg16(src + chunk * 128 + piece * 16) : make_uint4(0, 0, 0, 0);
    stg16(static_cast<char*>(j.dst) + i * 16, v);
  }
}

// Source row of output column n of a pack job (nullptr past N).
__device__ __forceinline__ const char* pack_src_row(const PackJob& j, int64_t tile, int row) {
  const int64_t n = tile * kPackTileRows + row;
  if (n >= j.N) return nullptr;
  const int64_t row_bytes = (int64_t)j.K * j.esize;
  if (j.kind == PACK_SWIGLU)
    return static_cast<const char*>(row < 16 ? j.w0 : j.w1) + (tile * 16 + (row & 15)) * row_bytes;
  if (j.kind == PACK_QKV)
    return n < j.nq ? static_cast<const char*>(j.w0) + n * row_bytes
                    : (n < j.nq + j.nkv ? static_cast<const char*>(j.w1) + (n - j.nq) * row_bytes
                                        : static_cast<const char*>(j.w2) + (n - j.nq - j.nkv) * row_bytes);
  return static_cast<const char*>(j.w0) + n * row_bytes;
}

// 4-bit packing: one thread a (tile, chunk, row) group of 64 bf16 weights. The group's
// bias is its minimum, its scale (max - min) / 15 rounded once to bf16 and each code
// rint((w - bias) / scale) clamped to [0, 15], all in float64 (a zero scale gives
// codes 0); the codes and the (scale, bias) pair go to the places kQ4Chunk describes.
__global__ __launch_bounds__(256) void k_pack_q4(const PackJob j) {
  const int64_t chunks = j.K / kQ4Group;
  const int64_t tiles = (j.N + kPackTileRows - 1) / kPackTileRows;
  const int64_t total = tiles * chunks * kPackTileRows;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(i % kPackTileRows);
    const int64_t chunk = (i / kPackTileRows) % chunks, tile = i / (kPackTileRows * chunks);
    const char* src = pack_src_row(j, tile, row);
    float w[kQ4Group];
#pragma unroll
    for (int q = 0; q < kQ4Group / 8; ++q) {
      const uint4 v = src ? ldg16(src + chunk * kQ4Group * 2 + q * 16) : make_uint4(0, 0, 0, 0);
      unpack(v, w + 8 * q, bf16_t());
    }
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int k = 1; k < kQ4Group; ++k) {
      lo = fminf(lo, w[k]);
      hi = fmaxf(hi, w[k]);
    }
    const uint32_t sbits = bf16_from_double(((double)hi - (double)lo) / 15.0);
    const double scale = (double)bf16_to_f32(sbits);
    uint32_t codes[8];   // dword 2 lg + d: codes k = 16 lg + 8 d .. + 7, nibble e = code 16 lg + 8 d + e
#pragma unroll
    for (int dw = 0; dw < 8; ++dw) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        double q = scale > 0.0 ? rint(((double)w[8 * dw + e] - (double)lo) / scale) : 0.0;
        q = q < 0.0 ? 0.0 : (q > 15.0 ? 15.0 : q);
        c |= (uint32_t)q << (4 * e);
      }
      codes[dw] = c;
    }
    char* dst = static_cast<char*>(j.dst) + (tile * chunks + chunk) * kQ4Chunk;
    const int lr = row & 15, nt = row >> 4;
#pragma unroll
    for (int lg = 0; lg < 4; ++lg)
      *reinterpret_cast<uint2*>(dst + (16 * lg + lr) * 16 + 8 * nt) = make_uint2(codes[2 * lg], codes[2 * lg + 1]);
    *reinterpret_cast<uint32_t*>(dst + 1024 + 8 * lr + 4 * nt) = sbits | (f32_to_bf16(lo) << 16);
  }
}

hipError_t launch_pack(const PackJob& j, hipStream_t st) {
  if (j.q4) (void)launch_k(k_pack_q4, dim3(4096), dim3(256), st, j);
  else (void)launch_k(k_pack, dim3(4096), dim3(256), st, j);
  return hipGetLastError();
}

// Groups of E elements a thread needs for `hidden`: 1, 2 or 4 (hidden <= 4 * 512 * E).
static int row_groups(int dtype, int hidden) {
  const int per = kNormThreads * (dtype == 0 ? Elem<float>::E : Elem<bf16_t>::E);
  const int g = (hidden + per - 1) / per;
  return g <= 1 ? 1 : (g <= 2 ? 2 : 4);
}

hipError_t launch_embed(int dtype, const EmbedParams& p, hipStream_t st) {
  const int g = row_groups(dtype, p.hidden), rows = p.S * p.B;
  if (dtype == 0) {
    if (g == 1) (void)launch_k(k_embed<float, 1>, dim3(rows), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_embed<float, 2>, dim3(rows), dim3(kNormThreads), st, p);
    else (void)launch_k(k_embed<float, 4>, dim3(rows), dim3(kNormThreads), st, p);
  } else {
    if (g == 1) (void)launch_k(k_embed<bf16_t, 1>, dim3(rows), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_embed<bf16_t, 2>, dim3(rows), dim3(kNormThreads), st, p);
    else (void)launch_k(k_embed<bf16_t, 4>, dim3(rows), dim3(kNormThreads), st, p);
  }
  return hipGetLastError();
}

hipError_t launch_kv_finish(int dtype, const KvFinishParams& p, hipStream_t st) {
  dim3 grid(p.R, p.n_layers);
  if (dtype == 0) {
    if (p.head_dim == 64) (void)launch_k((k_kv_finish<float, 64>), grid, dim3(256), st, p);
    else (void)launch_k((k_kv_finish<float, 128>), grid, dim3(256), st, p);
  } else {
    if (p.head_dim == 64) (void)launch_k((k_kv_finish<bf16_t, 64>), grid, dim3(256), st, p);
    else (void)launch_k((k_kv_finish<bf16_t, 128>), grid, dim3(256), st, p);
  }
  return hipGetLastError();
}

hipError_t launch_norm(int dtype, const NormParams& p, hipStream_t st) {
  const int g = row_groups(dtype, p.hidden);
  if (dtype == 0) {
    if (g == 1) (void)launch_k(k_norm<float, 1>, dim3(p.R), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_norm<float, 2>, dim3(p.R), dim3(kNormThreads), st, p);
    else (void)launch_k(k_norm<float, 4>, dim3(p.R), dim3(kNormThreads), st, p);
  } else {
    if (g == 1) (void)launch_k(k_norm<bf16_t, 1>, dim3(p.R), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_norm<bf16_t, 2>, dim3(p.R), dim3(kNormThreads), st, p);
    else (void)launch_k(k_norm<bf16_t, 4>, dim3(p.R), dim3(kNormThreads), st, p);
  }
  return hipGetLastError();
}

hipError_t launch_qkv_finish(int dtype, const QkvFinishParams& p, hipStream_t st) {
  dim3 grid(p.S * p.B, (p.n_q_heads + 2 * p.n_kv_heads + 3) / 4);
  if (dtype == 0) {
    if (p.head_dim == 64) (void)launch_k((k_qkv_finish<float, 64>), grid, dim3(256), st, p);
    else (void)launch_k((k_qkv_finish<float, 128>), grid, dim3(256), st, p);
  } else {
    if (p.head_dim == 64) (void)launch_k((k_qkv_finish<bf16_t, 64>), grid, dim3(256), st, p);
    else (void)launch_k((k_qkv_finish<bf16_t, 128>), grid, dim3(256), st, p);
  }
  return hipGetLastError();
}

hipError_t launch_rownorm(int dtype, const RowNormParams& p, hipStream_t st) {
  const int g = row_groups(dtype, p.hidden);
  if (dtype == 0) {
    if (g == 1) (void)launch_k(k_rownorm<float, 1>, dim3(p.R), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_rownorm<float, 2>, dim3(p.R), dim3(kNormThreads), st, p);
    else (void)launch_k(k_rownorm<float, 4>, dim3(p.R), dim3(kNormThreads), st, p);
  } else {
    if (g == 1) (void)launch_k(k_rownorm<bf16_t, 1>, dim3(p.R), dim3(kNormThreads), st, p);
    else if (g == 2) (void)launch_k(k_rownorm<bf16_t, 2>, dim3(p.R), dim3(kNormThreads), st, p);
    else (void)launch_k(k_rownorm<bf16_t, 4>, dim3(p.R), dim3(kNormThreads), st, p);
  }
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& p, hipStream_t st) {
  (void)launch_k(k_verify, dim3(p.S), dim3(64), st, p);
  return hipGetLastError();
}

}  // namespace dfl
