// Non-causal block attention of the draft round (gfx950).
//
// Workgroup = (context chunk, kv head, stream); one wave per 16 queries, where the
// queries of a kv head are its g q-heads times the B block rows. Keys are the
// context rows in the layer's reach, read from the paged cache, plus all B block
// rows (added by the stream's last chunk). K and V^T tiles of 64 keys are staged in
// LDS; scores are computed transposed (S^T = K Q^T) so that each lane owns one query,
// which makes the softmax row statistics lane-local plus two cross-lane-group
// shuffles, and lets the probabilities feed the P.V MFMA without a transpose.
// Chunks of one (stream, kv head) are combined by the last chunk to finish, in chunk
// order, so the result does not depend on scheduling.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kKT = 64;  // keys per LDS tile

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

template <typename T, int D>
__global__ __launch_bounds__(512) void k_attn(const AttnParams p) {
  using C = AttnCfg<T, D>;
  constexpr int E = C::E, NF = C::NF, CPK = C::CPK, NDT = C::NDT;
  __shared__ __attribute__((aligned(16))) T ks[kKT][C::LDK];
  __shared__ __attribute__((aligned(16))) T vt[D][C::LDV];
  __shared__ int s_last;

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int QT = nthr >> 6;
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = p.group, B = p.B, D_all_q = p.n_q_heads * D, D_all_kv = p.n_kv_heads * D;
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

  // Queries owned by this lane (as MFMA column lr of wave w).
  const int qi = 16 * w + lr;
  const bool q_valid = qi < nq_local;
  const int hl = q_valid ? qi / B : 0, jrow = q_valid ? qi % B : 0;
  const int qrow = s * B + jrow;
  const int qcol = (h * g + hl) * D;
  uint4 qf[NF];
  {
    const T* qp = static_cast<const T*>(p.q) + (int64_t)qrow * D_all_q + qcol + lg * (D / 4);
#pragma unroll
    for (int f = 0; f < NF; ++f) qf[f] = q_valid ? ldg16(qp + f * E) : make_uint4(0, 0, 0, 0);
  }

  floatx4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t head_stride = (int64_t)p.page_size * D;
  const int n_ctx_tiles = c_hi > c_lo ? (c_hi - c_lo + kKT - 1) / kKT : 0;
  const int n_tiles = n_ctx_tiles + (last_chunk ? 1 : 0);

  for (int t = 0; t < n_tiles; ++t) {
    const bool blk = (t == n_ctx_tiles);
    const int k0 = blk ? 0 : c_lo + t * kKT;
    const int nkeys = blk ? B : ((c_hi - k0) < kKT ? (c_hi - k0) : kKT);

    // ---- stage K rows and V^T into LDS (invalid keys are zero)
    for (int ci = tid; ci < kKT * CPK; ci += nthr) {
      const int key = ci / CPK, part = ci % CPK;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < nkeys) {
        if (blk) {
          const int64_t off = (int64_t)(s * B + key) * D_all_kv + h * D + part * E;
          kv = ldg16(static_cast<const T*>(p.kb) + off);
          vv = ldg16(static_cast<const T*>(p.vb) + off);
        } else {
          const int pos = k0 + key;
          const int page = p.page_table[(int64_t)s * p.pages_per_stream + pos / p.page_size];
          if (page >= 0 && page < p.pool_pages) {
            const int64_t off = ((int64_t)page * p.n_kv_heads + h) * head_stride +
                                (int64_t)(pos % p.page_size) * D + part * E;
            kv = ldg16(static_cast<const T*>(p.kpool) + off);
            vv = ldg16(static_cast<const T*>(p.vpool) + off);
          }
        }
      }
      *reinterpret_cast<uint4*>(&ks[key][part * E]) = kv;
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int e = 0; e < E; ++e) vt[part * E + e][key] = ve[e];
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane holds query lr, keys 16 mt + 4 lg + i
    floatx4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      const T* krow = &ks[16 * mt + lr][lg * (D / 4)];
#pragma unroll
      for (int f = 0; f < NF; ++f) mma_frag(sacc[mt], *reinterpret_cast<const uint4*>(krow + f * E), qf[f], T());
    }

    // ---- online softmax (base 2)
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * mt + 4 * lg + i;
        float tv = key < nkeys ? sacc[mt][i] * p.scale_log2 : -INFINITY;
        sacc[mt][i] = tv;
        mx = fmaxf(mx, tv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = (m_new == -INFINITY) ? 0.f : exp2f(sacc[mt][i] - m_new);
        sacc[mt][i] = pv;
        psum += pv;
      }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] *= corr;

    // ---- O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
      // P enters the bf16 MFMA as hi + lo parts (P - hi rounded again), so the
      // probabilities keep ~16 significant bits instead of 8.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float ph[8], pl[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[i] = Elem<T>::round(sacc[2 * kk][i]);
          ph[4 + i] = Elem<T>::round(sacc[2 * kk + 1][i]);
          pl[i] = sacc[2 * kk][i] - ph[i];
          pl[4 + i] = sacc[2 * kk + 1][i] - ph[4 + i];
        }
        const uint4 pbh = pack(ph, T()), pbl = pack(pl, T());
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* vrow = &vt[16 * dt + lr][0];
          uint2 lo2 = *reinterpret_cast<const uint2*>(vrow + 32 * kk + 4 * lg);
          uint2 hi2 = *reinterpret_cast<const uint2*>(vrow + 32 * kk + 16 + 4 * lg);
          const uint4 av = make_uint4(lo2.x, lo2.y, hi2.x, hi2.y);
          mma_frag(oacc[dt], av, pbh, T());
          mma_frag(oacc[dt], av, pbl, T());
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        float pl[4] = {sacc[mt][0], sacc[mt][1], sacc[mt][2], sacc[mt][3]};
        const uint4 pb = pack(pl, T());
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint4 av = *reinterpret_cast<const uint4*>(&vt[16 * dt + lr][16 * mt + 4 * lg]);
          mma_frag(oacc[dt], av, pb, T());
        }
      }
    }
    __syncthreads();
  }

  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);

  auto store_o = [&](const floatx4* oa, float inv_l) {
    if (!q_valid) return;
    T* op = static_cast<T*>(p.o) + (int64_t)qrow * D_all_q + qcol;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float v4[4] = {oa[dt][0] * inv_l, oa[dt][1] * inv_l, oa[dt][2] * inv_l, oa[dt][3] * inv_l};
      T* dst = op + 16 * dt + 4 * lg;
      if constexpr (sizeof(T) == 2) {
        uint2 pk = make_uint2(f32_to_bf16(v4[0]) | (f32_to_bf16(v4[1]) << 16),
                              f32_to_bf16(v4[2]) | (f32_to_bf16(v4[3]) << 16));
        *reinterpret_cast<uint2*>(dst) = pk;
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]);
      }
    }
  };

  if (p.n_chunks == 1) {
    store_o(oacc, 1.0f / l_tot);
    return;
  }

  // ---- publish this chunk's (m, l, O); the last chunk to arrive combines in chunk order
  const int64_t sh = (int64_t)s * p.n_kv_heads + h;
  const int64_t qstride = (int64_t)QT * 16;
  float* mlp = p.part_ml + ((sh * p.n_chunks + c) * qstride + qi) * 2;
  if (lg == 0) {
    mlp[0] = m_run;
    mlp[1] = l_tot;
  }
  const int64_t ofrag = (int64_t)NDT * kWave * 4;   // floats per wave per chunk
  float* op = p.part_o + ((sh * p.n_chunks + c) * QT + w) * ofrag;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<floatx4*>(op + (dt * kWave + lane) * 4) = oacc[dt];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    int old = atomicAdd(p.counters + sh, 1);
    s_last = (old == p.n_chunks - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (tid == 0) p.counters[sh] = 0;

  float M = -INFINITY;
  for (int cc = 0; cc < p.n_chunks; ++cc)
    M = fmaxf(M, p.part_ml[((sh * p.n_chunks + cc) * qstride + qi) * 2]);
  float L = 0.f;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int cc = 0; cc < p.n_chunks; ++cc) {
    const float* ml = p.part_ml + ((sh * p.n_chunks + cc) * qstride + qi) * 2;
    const float mc = ml[0];
    const float f = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
    L += ml[1] * f;
    const float* src = p.part_o + ((sh * p.n_chunks + cc) * QT + w) * ofrag;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) oacc[dt] += *reinterpret_cast<const floatx4*>(src + (dt * kWave + lane) * 4) * f;
  }
  store_o(oacc, 1.0f / L);
}

int attention_query_tiles(int group, int block) { return (group * block + 15) / 16; }

hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st) {
  const int qt = attention_query_tiles(p.group, p.B);
  dim3 grid(p.n_chunks, p.n_kv_heads, p.S), block(64 * qt);
  if (dtype == 0) {
    if (p.head_dim == 64) hipLaunchKernelGGL((k_attn<float, 64>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_attn<float, 128>), grid, block, 0, st, p);
  } else {
    if (p.head_dim == 64) hipLaunchKernelGGL((k_attn<bf16_t, 64>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((k_attn<bf16_t, 128>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace dfl
