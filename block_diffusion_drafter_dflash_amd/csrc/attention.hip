// Non-causal block attention of the draft round (gfx950).
//
// Workgroup = (context chunk, kv head, stream) with QT waves; wave w owns 16 of the
// kv head's g * B queries (its g q-heads times the B block rows). Keys are the
// context rows in the layer's reach, read from the paged cache, plus all B block
// rows (added by the stream's last chunk). K pages are [16 keys][d] and V pages are
// stored transposed, [d][16 keys], so both MFMA operands are contiguous along the
// reduction. The chunk's pages are copied straight from HBM into LDS in batches
// (global_load_lds, 16 bytes a lane, every read of a batch in flight at once and no
// registers held), with an XOR swizzle of 16-byte pieces that keeps the fragment
// reads free of bank conflicts; each wave then reads its fragments from LDS.
// Scores are computed transposed (S^T = K Q^T) so that each lane owns one query:
// the softmax statistics are lane-local plus two cross-lane-group shuffles, and the
// probabilities feed the P.V MFMA without a transpose. P (fp32) enters the bf16
// MFMA as three bf16 parts (hi, mid, lo) that hold all of its 24 bits, and the
// running output and denominator are kept in float64.
// A stream whose reach spans several chunks leaves per-chunk partials (max, sum,
// unnormalised output); k_attn_combine adds them in chunk order.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kAttnLdsBytes = 64 * 1024;   // one batch of pages

template <typename T, int D>
struct AttnCfg {
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int E = Elem<T>::E;
  static constexpr int NF = D / 4 / E;                   // 16-byte K fragments per lane per 16-key tile
  static constexpr int NDT = D / 16;                     // 16-dim output tiles
  static constexpr int KROW = D * (int)sizeof(T);        // bytes of a key row
  static constexpr int NCK = KROW / 16;                  // 16-byte pieces of a key row
  static constexpr int VROW = 16 * (int)sizeof(T);       // bytes of a value dim row in a page
  static constexpr int NCV = VROW / 16;
  static constexpr int KBYTES = 16 * KROW;               // K part of a page in LDS
  static constexpr int SLOT = KBYTES + D * VROW;         // one page (K and V^T) in LDS
  static constexpr int NBP = kAttnLdsBytes / SLOT;       // pages per batch (even)
  static constexpr int NKI = KBYTES / 1024;              // wave-wide 16-byte loads per page: K
  static constexpr int NVI = D * VROW / 1024;            //   and V^T
  // XOR swizzles of 16-byte pieces: 16 lanes reading the same piece of 16 key rows,
  // or of 16 value dims, touch 16 distinct bank groups.
  __device__ static __forceinline__ int kswz(int row) {
    return (KROW >= 256 ? row : row / (256 / KROW)) % NCK;
  }
  __device__ static __forceinline__ int vswz(int d) { return (d / (256 / VROW)) % NCV; }
};

// Key (0..31 within the step's two pages) supplied as row r of S^T tile t. For bf16
// the rows are arranged so that lane group lg ends up holding the probabilities of
// keys 8lg..8lg+7, exactly the eight reduction slots it feeds to the 32-deep P.V MFMA.
template <bool BF>
__device__ __forceinline__ int key_of_row(int t, int r) {
  return BF ? 8 * (r >> 2) + 4 * t + (r & 3) : 16 * t + r;
}

struct StepSrc {
  const void* k[2];     // K page base ([16][D]) of each half, or null (no keys there)
  const void* v[2];     // V^T page base ([D][vld]) of each half, or null
  int vld;              // V^T row stride (16 for cache pages, 32 for the block)
  int key0;             // absolute position of the step's first key; -1 for the block
};

__device__ __forceinline__ void load_lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <typename T, int D, int QT>
__global__ __launch_bounds__(64 * QT, 2) void k_attn(const AttnParams p) {
  using C = AttnCfg<T, D>;
  constexpr bool BF = C::BF;
  constexpr int E = C::E, NF = C::NF, NDT = C::NDT, NBP = C::NBP, SLOT = C::SLOT;
  constexpr int KROW = C::KROW, VROW = C::VROW, KBYTES = C::KBYTES, NKI = C::NKI, NVI = C::NVI;
  static_assert(NBP >= 2 && NBP % 2 == 0, "a batch holds whole steps");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[NBP * SLOT];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int c = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int g = p.group, B = p.B;
  const int nq_local = g * B;

  int Cs = p.ctx_len[s];
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int pg_lo = lo / 16;
  const int n_pages = span_pages(lo, Cs);
  // This stream's own chunking; the grid's chunks past it are empty.
  const int n_own = attention_chunks(n_pages);
  const int cpp = n_pages > 0 ? attention_chunk_pages(n_pages) : 0;
  const int cp0 = c * cpp;
  const int cp1 = c < n_own ? ((c + 1) * cpp < n_pages ? (c + 1) * cpp : n_pages) : cp0;
  const bool has_block = (c == n_own - 1);
  const int n_ctx_steps = cp1 > cp0 ? (cp1 - cp0 + 1) / 2 : 0;
  const int n_steps = n_ctx_steps + (has_block ? 1 : 0);

  // Queries owned by this lane (column lr of wave w's MFMA tiles): dims
  // [lg*D/4, (lg+1)*D/4) of query row (hl, jrow), as NF 16-byte fragments.
  const int qi = 16 * w + lr;
  const bool q_valid = qi < nq_local;
  const int hl = q_valid ? qi / B : 0, jrow = q_valid ? qi % B : 0;
  const int qrow = s * B + jrow;
  const int qcol = (h * g + hl) * D;
  uint4 qf[NF];
  {
    const T* qp = static_cast<const T*>(p.q) + (int64_t)qrow * (p.n_q_heads * D) + qcol + lg * (D / 4);
#pragma unroll
    for (int f = 0; f < NF; ++f) qf[f] = q_valid ? ldg16(qp + f * E) : make_uint4(0, 0, 0, 0);
  }

  double oacc[NDT][4];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[dt][i] = 0.0;
  float m_run = -INFINITY;
  double l_run = 0.0;

  const int64_t kv_page = (int64_t)p.page_size * D;   // elements per (page, head)
  // Page ids of the current batch: lane i of every wave holds the id of the batch's
  // i-th page (one vector load per batch instead of a dependent read per step).
  int batch_pid = -1;
  auto load_batch_pids = [&](int b0) {
    const int i = cp0 + 2 * b0 + lane;   // chunk-relative page index
    batch_pid = -1;
    if (lane < NBP && i < cp1) batch_pid = p.page_table[(int64_t)s * p.pages_per_stream + pg_lo + i];
  };
  // step's sources; `b0` is the first step of the batch whose page ids are loaded
  auto source = [&](int step, int b0) {
    StepSrc src;
    if (step < n_ctx_steps) {
      const int pg = pg_lo + cp0 + 2 * step;
      src.vld = 16;
      src.key0 = pg * 16;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        src.k[hf] = nullptr;
        src.v[hf] = nullptr;
        if (cp0 + 2 * step + hf < cp1) {
          const int page = __shfl(batch_pid, 2 * (step - b0) + hf, kWave);
          if (page >= 0 && page < p.pool_pages) {
            const int64_t off = ((int64_t)page * p.n_kv_heads + h) * kv_page;
            src.k[hf] = static_cast<const T*>(p.kpool) + off;
            src.v[hf] = static_cast<const T*>(p.vpool) + off;
          }
        }
      }
    } else {
      const int64_t off = ((int64_t)s * p.n_kv_heads + h) * (kBlockSlots * D);
      src.vld = kBlockSlots;
      src.key0 = -1;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        src.k[hf] = static_cast<const T*>(p.kblk) + off + hf * 16 * D;
        src.v[hf] = static_cast<const T*>(p.vblk) + off + hf * 16;
      }
    }
    return src;
  };
  // A key's validity: on a page, and inside the reach (context) or a block row (block).
  auto key_ok = [&](const StepSrc& src, int kk) {
    if (!(kk < 16 ? src.k[0] : src.k[1])) return false;
    if (src.key0 < 0) return kk < B;
    const int pos = src.key0 + kk;
    return pos >= lo && pos < Cs;
  };
  // Copy page hf of step `step` into LDS slot `slot`: the wave-wide loads of the slot
  // are dealt to the workgroup's waves; lane l of load j fills bytes [j*1024 + 16 l,
  // + 16) of the slot's K part (then V part) from the piece that the swizzle puts there.
  auto issue = [&](const StepSrc& src, int hf, int slot, int& seq) {
    const T* kp = static_cast<const T*>(hf ? src.k[1] : src.k[0]);
    const T* vp = static_cast<const T*>(hf ? src.v[1] : src.v[0]);
    unsigned char* base = lds + slot * SLOT;
#pragma unroll
    for (int j = 0; j < NKI + NVI; ++j, ++seq) {
      if (seq % QT != w || !kp) continue;
      const int b = (j < NKI ? j : j - NKI) * 1024 + lane * 16;
      if (j < NKI) {
        const int row = b / KROW, pc = (b % KROW) / 16;
        const int piece = pc ^ C::kswz(row);
        load_lds16(kp + row * D + piece * (16 / (int)sizeof(T)), base + j * 1024);
      } else {
        const int d = b / VROW, ph = (b % VROW) / 16;
        const int piece = ph ^ C::vswz(d);
        load_lds16(vp + (int64_t)d * src.vld + piece * (16 / (int)sizeof(T)), base + KBYTES + (j - NKI) * 1024);
      }
    }
  };

  auto compute = [&](int step, int b0, const unsigned char* sb) {
    const StepSrc cur = source(step, b0);

    // ---- S^T = K Q^T: lane holds query lr; tile t row 4lg+i is key key_of_row(t, 4lg+i)
    floatx4 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int kk = key_of_row<BF>(t, lr), row = kk & 15;
      const unsigned char* krow = sb + (kk >> 4) * SLOT + row * KROW;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int piece = (lg * (D / 4) + f * E) * (int)sizeof(T) / 16;
        mma_frag(sacc[t], *reinterpret_cast<const uint4*>(krow + ((piece ^ C::kswz(row)) * 16)), qf[f], T());
      }
    }

    // ---- online softmax (base 2); the denominator sums in float64
    const bool edge = cur.key0 < 0 || !cur.k[0] || !cur.k[1] || cur.key0 < lo || cur.key0 + 32 > Cs;
    float pf[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = !edge || key_ok(cur, key_of_row<BF>(t, 4 * lg + i));
        pf[t][i] = ok ? sacc[t][i] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, pf[t][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const double corr = (m_new == -INFINITY) ? 1.0 : (double)exp2f(m_run - m_new);
    double psum = 0.0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[t][i] = (pf[t][i] == -INFINITY) ? 0.f : exp2f(pf[t][i] - m_new);
        psum += (double)pf[t][i];
      }
    l_run = l_run * corr + psum;
    m_run = m_new;

    // ---- this step's O^T = V^T P^T, added to the float64 running output. Values of
    // keys outside the reach (or of pages never loaded) may be stale or non-finite:
    // they are zeroed so that a zero probability times them cannot reach the output.
    floatx4 ot[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) ot[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF) {
      // P as hi + mid + lo bf16 parts (each remainder is exact in fp32): 24 bits.
      const float pv[8] = {pf[0][0], pf[0][1], pf[0][2], pf[0][3], pf[1][0], pf[1][1], pf[1][2], pf[1][3]};
      uint32_t hw[4], mw[4], lw[4], keep[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hw[q] = f32x2_to_bf16x2(pv[2 * q], pv[2 * q + 1]);
        const float r0 = pv[2 * q] - bf16_to_f32(hw[q] & 0xffffu);
        const float r1 = pv[2 * q + 1] - bf16_to_f32(hw[q] >> 16);
        mw[q] = f32x2_to_bf16x2(r0, r1);
        lw[q] = f32x2_to_bf16x2(r0 - bf16_to_f32(mw[q] & 0xffffu), r1 - bf16_to_f32(mw[q] >> 16));
        keep[q] = 0xffffffffu;
        if (edge)
          keep[q] = (key_ok(cur, 8 * lg + 2 * q) ? 0x0000ffffu : 0u) | (key_ok(cur, 8 * lg + 2 * q + 1) ? 0xffff0000u : 0u);
      }
      const uint4 bh = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      const uint4 bm = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      const uint4 bl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      // lane group lg: keys 8lg..8lg+7 = page lg/2, 16-byte piece lg&1 of each dim row
      const unsigned char* vbase = sb + (lg >> 1) * SLOT + KBYTES;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = 16 * dt + lr;
        uint4 vf = *reinterpret_cast<const uint4*>(vbase + d * VROW + (((lg & 1) ^ C::vswz(d)) * 16));
        vf.x &= keep[0];
        vf.y &= keep[1];
        vf.z &= keep[2];
        vf.w &= keep[3];
        mma_frag(ot[dt], vf, bh, T());
        mma_frag(ot[dt], vf, bm, T());
        mma_frag(ot[dt], vf, bl, T());
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 pb = make_uint4(__float_as_uint(pf[t][0]), __float_as_uint(pf[t][1]), __float_as_uint(pf[t][2]),
                                    __float_as_uint(pf[t][3]));
        const int k0 = 16 * t + 4 * lg;
        const bool ok0 = !edge || key_ok(cur, k0), ok1 = !edge || key_ok(cur, k0 + 1);
        const bool ok2 = !edge || key_ok(cur, k0 + 2), ok3 = !edge || key_ok(cur, k0 + 3);
        // page t, 16-byte piece lg (keys 4lg..4lg+3) of each dim row
        const unsigned char* vbase = sb + t * SLOT + KBYTES;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = 16 * dt + lr;
          uint4 vf = *reinterpret_cast<const uint4*>(vbase + d * VROW + ((lg ^ C::vswz(d)) * 16));
          vf.x = ok0 ? vf.x : 0u;
          vf.y = ok1 ? vf.y : 0u;
          vf.z = ok2 ? vf.z : 0u;
          vf.w = ok3 ? vf.w : 0u;
          mma_frag(ot[dt], vf, pb, T());
        }
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[dt][i] = oacc[dt][i] * corr + (double)ot[dt][i];
  };

  // Batches of NBP / 2 steps: copy every page of the batch into LDS, wait, compute.
  for (int b0 = 0; b0 < n_steps; b0 += NBP / 2) {
    const int b1 = b0 + NBP / 2 < n_steps ? b0 + NBP / 2 : n_steps;
    int seq = 0;
    load_batch_pids(b0);
    for (int st = b0; st < b1; ++st) {
      const StepSrc src = source(st, b0);
      issue(src, 0, 2 * (st - b0), seq);
      issue(src, 1, 2 * (st - b0) + 1, seq);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed in LDS
    __syncthreads();                 // and every other wave's
    for (int st = b0; st < b1; ++st) compute(st, b0, lds + 2 * (st - b0) * SLOT);
    __syncthreads();                 // the batch's slots are free again
  }

  double l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);

  if (p.n_chunks == 1) {
    // Same arithmetic as the combine of a single chunk (fp32 partials), so a stream's
    // output does not depend on how many chunks the batch's longest reach needs.
    if (!q_valid) return;
    const double L = (double)(float)l_tot;
    T* op = static_cast<T*>(p.o) + (int64_t)qrow * (p.n_q_heads * D) + qcol;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      double v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = (double)(float)oacc[dt][i] / L;
      T* dst = op + 16 * dt + 4 * lg;
      if constexpr (BF) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2(f32_round_odd(v4[0]), f32_round_odd(v4[1])),
                                                    f32x2_to_bf16x2(f32_round_odd(v4[2]), f32_round_odd(v4[3])));
      } else {
        *reinterpret_cast<float4*>(dst) = make_float4((float)v4[0], (float)v4[1], (float)v4[2], (float)v4[3]);
      }
    }
    return;
  }

  // ---- this chunk's (max, sum, unnormalised output) for k_attn_combine
  const int64_t sh = (int64_t)s * p.n_kv_heads + h;
  if (lg == 0) {
    float* ml = p.part_ml + ((sh * (QT * 16) + qi) * p.n_chunks + c) * 2;
    *reinterpret_cast<float2*>(ml) = make_float2(m_run, (float)l_tot);
  }
  float* op = p.part_o + (((sh * p.n_chunks + c) * QT + w) * NDT) * (kWave * 4);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
    *reinterpret_cast<float4*>(op + (dt * kWave + lane) * 4) =
        make_float4((float)oacc[dt][0], (float)oacc[dt][1], (float)oacc[dt][2], (float)oacc[dt][3]);
}

// Combine the chunks of one (stream, kv head, query tile, 16-dim slice): four waves
// take contiguous quarters of the stream's own chunks (its count depends only on its
// reach, so the grouping is the same in any batch). The maximum over all chunks comes
// first; then each wave sums its quarter in chunk order in float64, every chunk scaled
// by 2^(m_c - M) (fp32 exp2, as precise as the fp32 chunk partials it scales, and
// exactly 1 for the chunk holding the maximum), and the quarters are added in wave
// order. A lane's query has its chunks' (max, sum) pairs contiguous.
constexpr int kCombineWaves = 4;
template <typename T, int D>
__global__ __launch_bounds__(64 * kCombineWaves) void k_attn_combine(const AttnParams p, int QT) {
  constexpr int NDT = D / 16, NW = kCombineWaves;
  __shared__ float s_max[NW][16];
  __shared__ double s_sum[NW][64][5];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int sh = blockIdx.x / QT, qt = blockIdx.x % QT, dt = blockIdx.y;
  const int s = sh / p.n_kv_heads, h = sh % p.n_kv_heads;
  const int qi = 16 * qt + lr;
  const bool valid = qi < p.group * p.B;
  int Cs = p.ctx_len[s];
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int n_own = attention_chunks(span_pages(lo, Cs));
  const int c0 = (int)((int64_t)w * n_own / NW), c1 = (int)((int64_t)(w + 1) * n_own / NW);
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + ((int64_t)sh * (QT * 16) + (valid ? qi : 0)) * p.n_chunks;
  float M = -INFINITY;
  for (int cc = c0; cc < c1; ++cc) M = fmaxf(M, ml[cc].x);
  if (lg == 0) s_max[w][lr] = M;
  __syncthreads();
  M = s_max[0][lr];
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, s_max[ww][lr]);
  double L = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0};
  const float* po = p.part_o + (((int64_t)sh * p.n_chunks * QT + qt) * NDT + dt) * (kWave * 4) + lane * 4;
  const int64_t cstride = (int64_t)QT * NDT * (kWave * 4);
#pragma unroll 4
  for (int cc = c0; cc < c1; ++cc) {
    const float2 m = ml[cc];
    const float4 v = *reinterpret_cast<const float4*>(po + cc * cstride);
    const double f = (m.x == -INFINITY) ? 0.0 : (double)exp2f(m.x - M);
    L += (double)m.y * f;
    o[0] += (double)v.x * f;
    o[1] += (double)v.y * f;
    o[2] += (double)v.z * f;
    o[3] += (double)v.w * f;
  }
  s_sum[w][lane][0] = L;
#pragma unroll
  for (int i = 0; i < 4; ++i) s_sum[w][lane][1 + i] = o[i];
  __syncthreads();
  if (w != 0 || !valid) return;
#pragma unroll
  for (int ww = 1; ww < NW; ++ww) {
    L += s_sum[ww][lane][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] += s_sum[ww][lane][1 + i];
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
  (void)launch_k((k_attn<T, D, QT>), grid, dim3(64 * QT), st, p);
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
  (void)launch_k((k_attn_combine<T, D>), dim3(p.S * p.n_kv_heads * qt, D / 16), dim3(64 * kCombineWaves), st, p, qt);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st) {
  if (dtype == 0) return p.head_dim == 64 ? launch_td<float, 64>(p, st) : launch_td<float, 128>(p, st);
  return p.head_dim == 64 ? launch_td<bf16_t, 64>(p, st) : launch_td<bf16_t, 128>(p, st);
}

}  // namespace dfl
