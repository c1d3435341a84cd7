// Non-causal block attention of the draft round (gfx950).
//
// Workgroup = (context chunk, kv head, stream) with QT waves; wave w owns 16 of the
// kv head's g * B queries (its g q-heads times the B block rows). Keys are the
// context rows in the layer's reach, read from the paged cache, plus all B block
// rows (added by the stream's last chunk). K pages are [16 keys][d] and V pages are
// stored transposed, [d][16 keys], so both MFMA operands are contiguous along the
// reduction. A chunk's pages are copied straight from HBM into LDS in batches of
// BP pages (global_load_lds, 16 bytes a lane, no registers held), into two LDS
// buffers used alternately: batch b + 1 is in flight while the waves compute on
// batch b. An XOR swizzle of 16-byte pieces keeps the fragment reads free of bank
// conflicts. Scores are computed transposed (S^T = K Q^T) so that each lane owns
// one query: the softmax statistics are lane-local plus two cross-lane-group
// shuffles, and the probabilities feed the P.V MFMA without a transpose. The
// running maximum moves once per batch; P (fp32) enters the bf16 MFMA as three bf16
// parts that sum to it exactly, and a batch's P.V accumulates into the rescaled fp32
// running output. Which keys
// of a step are valid is one wave-uniform 32-bit mask, so steps without an edge
// (reach boundary, missing page, block padding) take no masking work at all.
// A stream whose reach spans several chunks leaves per-chunk partials (max, sum,
// unnormalised output); k_attn_combine adds them in chunk order.
#include <type_traits>

#include "common.hpp"
#include "kernels.h"

namespace dfl {

constexpr int kAttnBufBytes = 32 * 1024;   // one LDS buffer: a batch of pages

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
  static constexpr int BP = kAttnBufBytes / SLOT >= 4 ? 4 : 2;   // pages per batch
  static constexpr int NSB = BP / 2;                     // steps (two pages) per batch
  static constexpr int NKI = KBYTES / 1024;              // wave-wide 16-byte loads per page: K
  static constexpr int NVI = D * VROW / 1024;            //   and V^T
  static_assert(BP * SLOT <= kAttnBufBytes, "a batch fits one buffer");
  // XOR swizzles of 16-byte pieces: 16 lanes reading the same piece of 16 key rows,
  // or of 16 value dims, touch 16 distinct bank groups.
  __device__ static __forceinline__ int kswz(int row) {
    return (KROW >= 256 ? row : row / (256 / KROW)) % NCK;
  }
  __device__ static __forceinline__ int vswz(int d) { return (d / (256 / VROW)) % NCV; }
  static_assert(16 % (256 / VROW) == 0 && (16 / (256 / VROW)) % NCV == 0, "vswz(d + 16) == vswz(d)");
};

// Key (0..31 within the step's two pages) supplied as row r of S^T tile t. For bf16
// the rows are arranged so that lane group lg ends up holding the probabilities of
// keys 8lg..8lg+7, exactly the eight reduction slots it feeds to the 32-deep P.V MFMA.
template <bool BF>
__device__ __forceinline__ int key_of_row(int t, int r) {
  return BF ? 8 * (r >> 2) + 4 * t + (r & 3) : 16 * t + r;
}

__device__ __forceinline__ void load_lds16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Maximum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups), with the
// gfx950 lane-swap instructions: each swap leaves a lane holding its own value and its
// partner's (lane ^ 32, then lane ^ 16) in its two results.
__device__ __forceinline__ float xor_max_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Bits [a, e) of a 16-bit half (0 <= a, e <= 16).
__device__ __forceinline__ uint32_t bit_range16(int a, int e) {
  return e > a ? ((0xffffu >> (16 - (e - a))) << a) : 0u;
}

// The work item of this block: (chunk c, kv head h, stream s). Narrow and mid
// batches, and wide ones of more than 64 streams, take the grid's own order. Wide batches of up to
// 64 streams run their items longest first: a stream's chunks are cpp pages each but
// the last, which is shorter, and the streams' reaches differ, so in grid order the
// last workgroups to start can be whole chunks that finish long after the rest. The
// (stream, chunk) items are ranked by pages (descending), then stream, then chunk,
// with the kv heads innermost; block i takes item i (each lane of a wave holds one
// stream's two groups of equal-size chunks and finds their first ranks), and the
// blocks past the items return at once. An item's arithmetic does not depend on
// which block runs it.
__device__ __forceinline__ bool attn_item(const AttnParams& p, int& c, int& h, int& s) {
  if (p.cls != 2 || p.S > kWave) {
    c = blockIdx.x;
    h = blockIdx.y;
    s = blockIdx.z;
    return true;
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int i = (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
  // this lane's stream: groups (z1 pages x n1 chunks from chunk 0) and (z2 pages, the last)
  int z1 = -1, n1 = 0, z2 = -1, n_own = 0;
  if (lane < p.S) {
    int Cs = p.ctx_len[lane];
    Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
    const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
    const int pages = span_pages(lo, Cs);
    n_own = attention_chunks(pages, 2);
    const int cpp = pages > 0 ? attention_chunk_pages(pages, 2) : 0;
    z1 = cpp;
    n1 = n_own - 1;
    z2 = pages - (n_own - 1) * cpp;
  }
  // first rank of each group: the items of the groups ordered before it
  int r1 = 0, r2 = 0;
  for (int t = 0; t < p.S; ++t) {
    const int tz1 = __shfl(z1, t, kWave), tn1 = __shfl(n1, t, kWave), tz2 = __shfl(z2, t, kWave);
    // group (tz1, t, chunk 0) and group (tz2, t, chunk n_own(t) - 1)
    if (tn1 > 0) {
      if (tz1 > z1 || (tz1 == z1 && t < lane)) r1 += tn1;
      if (tz1 > z2 || (tz1 == z2 && t <= lane)) r2 += tn1;   // t == lane: chunks 0.. precede the last
    }
    if (tz2 > z1 || (tz2 == z1 && t < lane)) r1 += 1;
    if (tz2 > z2 || (tz2 == z2 && t < lane)) r2 += 1;
  }
  const int q = i / p.n_kv_heads;
  const bool in1 = lane < p.S && n1 > 0 && q >= r1 && q < r1 + n1;
  const bool in2 = lane < p.S && q == r2;
  const uint64_t m1 = __ballot(in1), m2 = __ballot(in2);
  if (m1 == 0 && m2 == 0) return false;
  const int src = m1 ? __builtin_ctzll(m1) : __builtin_ctzll(m2);
  const int cc = in1 ? q - r1 : n_own - 1;
  s = src;
  c = __shfl(cc, src, kWave);
  h = i % p.n_kv_heads;
  return true;
}

template <typename T, int D, int QT, int KG>
__device__ __forceinline__ void attn_body(const AttnParams& p) {
  using C = AttnCfg<T, D>;
  constexpr bool BF = C::BF;
  constexpr int E = C::E, NF = C::NF, NDT = C::NDT, BP = C::BP, NSB = C::NSB, SLOT = C::SLOT;
  constexpr int KROW = C::KROW, VROW = C::VROW, KBYTES = C::KBYTES, NKI = C::NKI, NVI = C::NVI;
  constexpr int NW = KG * QT;          // waves: KG key groups of QT query waves
  constexpr int NSG = NSB / KG;        // steps of a batch that one key group computes
  static_assert(KG >= 1 && NSB % KG == 0, "a batch's steps split evenly over the key groups");
  // Two separate buffers: the compiler then sees that a batch's copies into one
  // never alias the fragment reads of the other, and keeps them in flight.
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[BP * SLOT];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[BP * SLOT];
  // the second key group's (max, sum) handed to the first for the merge
  __shared__ float s_m[KG > 1 ? QT : 1][64];
  __shared__ double s_l[KG > 1 ? QT : 1][64];

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int kg = wv / QT, w = wv % QT;   // key group, query wave
  int c, h, s;
  if (!attn_item(p, c, h, s)) return;   // a block past the real work items: the whole workgroup leaves
  // The item and the stream's context length are the same in every lane; held as
  // scalars, the masks and branches that derive from them stay scalar too (no
  // exec-mask branches, and no copies of the running output between their paths).
  c = __builtin_amdgcn_readfirstlane(c);
  h = __builtin_amdgcn_readfirstlane(h);
  s = __builtin_amdgcn_readfirstlane(s);
  const int g = p.group, B = p.B;
  const int nq_local = g * B;

  int Cs = __builtin_amdgcn_readfirstlane(p.ctx_len[s]);
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int pg_lo = lo / 16;
  const int n_pages = span_pages(lo, Cs);
  // This stream's own chunking; the grid's chunks past it are empty.
  const int n_own = attention_chunks(n_pages, p.cls);
  const int cpp = n_pages > 0 ? attention_chunk_pages(n_pages, p.cls) : 0;
  const int cp0 = c * cpp;
  int n_cp = c < n_own ? ((c + 1) * cpp < n_pages ? (c + 1) * cpp : n_pages) - cp0 : 0;
  n_cp = n_cp > 0 ? n_cp : 0;   // the last chunks of a rounded-up split can be empty
  const bool has_block = (c == n_own - 1);
  const int nb_ctx = (n_cp + BP - 1) / BP;
  const int nb = nb_ctx + (has_block ? 1 : 0);

  // Page ids: lane i holds the id of the chunk's page i (a chunk has at most 64 pages).
  int pid = -1;
  if (lane < n_cp) pid = p.page_table[(int64_t)s * p.pages_per_stream + pg_lo + cp0 + lane];
  // Per chunk page i (lane i), computed once: the (page, kv head) index its keys and
  // values are copied from (a page that is absent, outside the pool or past the chunk
  // is copied from pool page 0 instead, valid memory whose keys are masked), and
  // whether all 16 of its keys are valid. A batch whose pages are all valid needs no
  // mask; the per-batch work is then a few scalar operations per page.
  const bool pg_ok = lane < n_cp && pid >= 0 && pid < p.pool_pages;
  const uint32_t src_page = (uint32_t)((pg_ok ? pid : 0) * p.n_kv_heads + h);
  const int pos_i = (pg_lo + cp0 + lane) * 16;
  const uint64_t full_pages = __ballot(pg_ok && pos_i >= lo && pos_i + 16 <= Cs);
  const uint64_t ok_pages = __ballot(pg_ok);

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

  floatx4 orun[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) orun[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  double l_run = 0.0;

  const int64_t blk_off = ((int64_t)s * p.n_kv_heads + h) * (kBlockSlots * D);
  const T* kblk = static_cast<const T*>(p.kblk) + blk_off;
  const T* vblk = static_cast<const T*>(p.vblk) + blk_off;

  // Copy batch b's pages into `buf`. Wave wv issues the wave-wide 16-byte loads
  // jj = wv, wv + NW, ... (< NKI + NVI) of every page of the batch: lane l of load jj
  // fills bytes [jj*1024 + 16 l, + 16) of the page's slot (K part, then V^T part)
  // from the piece that the swizzle puts there. The lane's source offset within a
  // page does not depend on the page (K rows [16][D]; V^T dim rows of stride 16 in
  // the cache, kBlockSlots in the block), so it is computed once.
  constexpr int LPP = NKI + NVI;
  constexpr int JW = (LPP + NW - 1) / NW;
  int src_pg[JW], src_blk[JW];
#pragma unroll
  for (int k = 0; k < JW; ++k) {
    const int jj = wv + NW * k;
    src_pg[k] = src_blk[k] = 0;
    if (jj >= LPP) continue;
    const int bo = (jj < NKI ? jj : jj - NKI) * 1024 + lane * 16;
    if (jj < NKI) {
      const int row = bo / KROW, pc = (bo % KROW) / 16;
      src_pg[k] = src_blk[k] = row * D + (pc ^ C::kswz(row)) * (16 / (int)sizeof(T));
    } else {
      const int d = bo / VROW, ph = (bo % VROW) / 16;
      const int piece = (ph ^ C::vswz(d)) * (16 / (int)sizeof(T));
      src_pg[k] = d * 16 + piece;
      src_blk[k] = d * kBlockSlots + piece;
    }
  }
  // Context batches copy BP pages each (the chunk's pages past its end come from the
  // stand-in page); the block batch copies the stream's two block pages.
  const T* kpool = static_cast<const T*>(p.kpool);
  const T* vpool = static_cast<const T*>(p.vpool);
  auto issue = [&](int b, unsigned char* buf) {
    if (b >= nb_ctx) {
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        unsigned char* slot = buf + pb * SLOT;
#pragma unroll
        for (int k = 0; k < JW; ++k) {
          const int jj = wv + NW * k;
          if (jj >= LPP) break;
          if (jj < NKI) load_lds16(kblk + pb * 16 * D + src_blk[k], slot + jj * 1024);
          else load_lds16(vblk + pb * 16 + src_blk[k], slot + KBYTES + (jj - NKI) * 1024);
        }
      }
      return;
    }
#pragma unroll
    for (int pb = 0; pb < BP; ++pb) {
      // b * BP + pb <= 63: a chunk has at most 64 pages and 64 % BP == 0
      const uint32_t sp = __builtin_amdgcn_readlane(src_page, b * BP + pb);
      const int64_t off = (int64_t)sp * (16 * D);   // pages of 16 keys
      const T* kp = kpool + off;
      const T* vp = vpool + off;
      unsigned char* slot = buf + pb * SLOT;
#pragma unroll
      for (int k = 0; k < JW; ++k) {
        const int jj = wv + NW * k;
        if (jj >= LPP) break;
        if (jj < NKI) load_lds16(kp + src_pg[k], slot + jj * 1024);
        else load_lds16(vp + src_pg[k], slot + KBYTES + (jj - NKI) * 1024);
      }
    }
  };
  // Context batch b has only valid keys.
  auto batch_full = [&](int b) {
    constexpr uint64_t all = (1ull << BP) - 1ull;
    return b < nb_ctx && ((full_pages >> (b * BP)) & all) == all;
  };

  // Valid keys of step st of batch b as a uniform 32-bit mask (bit k = key k).
  auto step_mask = [&](int b, int st) -> uint32_t {
    if (b >= nb_ctx) return st == 0 ? (B >= 32 ? 0xffffffffu : (1u << B) - 1u) : 0u;
    uint32_t m = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int i = b * BP + 2 * st + hf;
      if ((ok_pages >> i) & 1ull) {
        const int pos0 = (pg_lo + cp0 + i) * 16;
        const int a = lo - pos0 > 0 ? lo - pos0 : 0, e = Cs - pos0 < 16 ? Cs - pos0 : 16;
        m |= bit_range16(a, e) << (16 * hf);
      }
    }
    return m;
  };

  // Lane byte offsets of the fragments in a buffer (step 0; step st adds 2 st SLOT).
  // K: tile t row r is key key_of_row(t, r), whose 16-byte piece 4 lg + f (dims
  // [lg D/4 + f E, + E)) sits at the swizzled place. V^T: bf16 lane group lg reads
  // keys 8lg..8lg+7 = page lg/2, piece lg&1 of dim row lr (+16 dt); fp32 lane group
  // lg reads keys 4lg..4lg+3 = piece lg of page t. The swizzle of dim 16 dt + lr
  // equals that of dim lr. Every LDS address is one buffer plus one offset, so the
  // compiler can tell the two buffers apart.
  int koff[2][NF], voff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kk = key_of_row<BF>(t, lr), row = kk & 15;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int piece = (lg * (D / 4) + f * E) * (int)sizeof(T) / 16;
      koff[t][f] = (kk >> 4) * SLOT + row * KROW + (piece ^ C::kswz(row)) * 16;
    }
    voff[t] = BF ? (lg >> 1) * SLOT + KBYTES + lr * VROW + (((lg & 1) ^ C::vswz(lr)) * 16)
                 : t * SLOT + KBYTES + lr * VROW + ((lg ^ C::vswz(lr)) * 16);
  }

  // S^T tiles of step st: lane holds query lr; tile t row 4lg+i is key key_of_row(t, 4lg+i).
  auto qk_step = [&](const unsigned char* buf, int st, floatx4 (&sacc)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; ++f)
        mma_frag(sacc[t], *reinterpret_cast<const uint4*>(buf + (koff[t][f] + 2 * st * SLOT)), qf[f], T());
    }
  };
  // O^T += V^T P^T of step st (probabilities pr). With MASKED, the values of invalid
  // keys (outside the reach, absent pages, stale slots) are zeroed so that a zero
  // probability times them cannot reach the output.
  auto pv_step = [&](const unsigned char* buf, int st, const float (&pr)[2][4], uint32_t m, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    if constexpr (BF) {
      // P as three bf16 parts that sum to it exactly: hi = bf16(P); the remainder
      // P - hi is exact in fp32 and keeps at most 16 significant bits, mid = bf16 of
      // it; what is left, at most 8 bits, is exact in bf16 (lo). Two parts would leave
      // P off by up to 2^-18 (relative) per key, which alone moves about 2e-3 of the
      // stored bf16 outputs by one ulp; with three, only P's own fp32 rounding remains.
      const float pv[8] = {pr[0][0], pr[0][1], pr[0][2], pr[0][3], pr[1][0], pr[1][1], pr[1][2], pr[1][3]};
      uint32_t hw[4], mw[4], lw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hw[q] = f32x2_to_bf16x2(pv[2 * q], pv[2 * q + 1]);
        const float r0 = pv[2 * q] - bf16_to_f32(hw[q] & 0xffffu);
        const float r1 = pv[2 * q + 1] - bf16_to_f32(hw[q] >> 16);
        mw[q] = f32x2_to_bf16x2(r0, r1);
        lw[q] = f32x2_to_bf16x2(r0 - bf16_to_f32(mw[q] & 0xffffu), r1 - bf16_to_f32(mw[q] >> 16));
      }
      const uint4 bh = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      const uint4 bm = make_uint4(mw[0], mw[1], mw[2], mw[3]);
      const uint4 bl = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      uint32_t keep[4] = {~0u, ~0u, ~0u, ~0u};
      if constexpr (MASKED) {
        // lane group lg holds keys 8lg..8lg+7, two to a 32-bit word
        const uint32_t kb = m >> (8 * lg);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          keep[q] = ((kb >> (2 * q)) & 1u ? 0x0000ffffu : 0u) | ((kb >> (2 * q + 1)) & 1u ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        uint4 vf = *reinterpret_cast<const uint4*>(buf + (voff[0] + (2 * st * SLOT + dt * 16 * VROW)));
        if constexpr (MASKED) {
          vf.x &= keep[0];
          vf.y &= keep[1];
          vf.z &= keep[2];
          vf.w &= keep[3];
        }
        mma_frag(orun[dt], vf, bh, T());
        mma_frag(orun[dt], vf, bm, T());
        mma_frag(orun[dt], vf, bl, T());
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint4 pb = make_uint4(__float_as_uint(pr[t][0]), __float_as_uint(pr[t][1]), __float_as_uint(pr[t][2]),
                                    __float_as_uint(pr[t][3]));
        const uint32_t kb = m >> (16 * t + 4 * lg);   // page t, keys 4lg..4lg+3
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          uint4 vf = *reinterpret_cast<const uint4*>(buf + (voff[t] + (2 * st * SLOT + dt * 16 * VROW)));
          if constexpr (MASKED) {
            vf.x = (kb & 1u) ? vf.x : 0u;
            vf.y = (kb & 2u) ? vf.y : 0u;
            vf.z = (kb & 4u) ? vf.z : 0u;
            vf.w = (kb & 8u) ? vf.w : 0u;
          }
          mma_frag(orun[dt], vf, pb, T());
        }
      }
    }
  };

  // One batch. A batch whose keys are all valid (the common case) runs straight-line
  // code with no masking; otherwise steps without valid keys are skipped and edge
  // steps are masked (steps whose keys are all valid still take no masking work).
  auto compute = [&](int b, const unsigned char* buf) {
    // this key group's steps of the batch: kg * NSG + i
    uint32_t msk[NSG];
    bool full = batch_full(b);
#pragma unroll
    for (int i = 0; i < NSG; ++i) msk[i] = 0xffffffffu;
    if (!full) {
      bool f = true;
#pragma unroll
      for (int i = 0; i < NSG; ++i) {
        msk[i] = step_mask(b, kg * NSG + i);
        f = f && msk[i] == 0xffffffffu;
      }
      full = f;
    }
    // Workgroups of more than four query waves must fit three waves per SIMD; their
    // registers do not hold two steps' P.V in flight, so they go step by step.
    if constexpr (QT > 4 && NSG > 1) full = false;

    float sv[NSG][2][4];
    {
      floatx4 sacc[NSG][2];
      if (full) {
#pragma unroll
        for (int st = 0; st < NSG; ++st) qk_step(buf, kg * NSG + st, sacc[st]);
      } else {
#pragma unroll
        for (int st = 0; st < NSG; ++st) {
          if (msk[st]) qk_step(buf, kg * NSG + st, sacc[st]);
          else sacc[st][0] = sacc[st][1] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int st = 0; st < NSG; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[st][t][i] = sacc[st][t][i] * p.scale_log2;
    }
    if (!full) {
#pragma unroll
      for (int st = 0; st < NSG; ++st)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((msk[st] >> key_of_row<BF>(t, 4 * lg + i)) & 1u)) sv[st][t][i] = -INFINITY;
    }

    // ---- the batch's maximum, probabilities (base 2) and their sum; the running
    // output is rescaled to the new maximum before the batch's P.V accumulates.
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < NSG; ++st)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[st][t][i]);
    mx = xor_max_16_32(mx);
    const float m_new = fmaxf(m_run, mx);
    // A finite stand-in for the maximum: exp2(-inf - m_safe) is exactly 0, also while
    // no valid key has been seen (m_new = -inf, where the running sums are still 0).
    const float m_safe = m_new == -INFINITY ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_safe);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < NSG; ++st)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[st][t][i] = __builtin_amdgcn_exp2f(sv[st][t][i] - m_safe);
          psum += sv[st][t][i];
        }
    l_run = l_run * (double)corr + (double)psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) orun[dt][i] *= corr;

    if (full) {
#pragma unroll
      for (int st = 0; st < NSG; ++st) pv_step(buf, kg * NSG + st, sv[st], 0xffffffffu, std::false_type{});
    } else {
#pragma unroll
      for (int st = 0; st < NSG; ++st) {
        if (!msk[st]) continue;
        if (msk[st] == 0xffffffffu) pv_step(buf, kg * NSG + st, sv[st], msk[st], std::false_type{});
        else pv_step(buf, kg * NSG + st, sv[st], msk[st], std::true_type{});
      }
    }
  };

  // Pipeline: batch b + 1 is copied into the other buffer while batch b is computed.
  // Each wait covers only the batch about to be used (the next one is issued after
  // the barrier), and the barrier also frees the buffer that the next copy reuses.
  if (nb > 0) issue(0, buf0);
  for (int b = 0; b < nb; b += 2) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of batch b have landed
    __syncthreads();                 // everyone's; and buf1 is no longer read
    if (b + 1 < nb) issue(b + 1, buf1);
    compute(b, buf0);
    if (b + 1 >= nb) break;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (b + 2 < nb) issue(b + 2, buf0);
    compute(b + 1, buf1);
  }

  if constexpr (KG > 1) {
    // The second key group hands its running state to the first, which merges:
    // M = max(m0, m1), each side scaled by 2^(m_k - M) (exactly 1 for the side
    // holding M). The batch buffers are free once every wave is past the loop.
    __syncthreads();
    float* so0 = reinterpret_cast<float*>(buf0);
    float* so1 = reinterpret_cast<float*>(buf1);
    constexpr int HALF = NDT / 2;   // dims tiles 0..HALF-1 go through buf0, the rest buf1
    static_assert(QT * 64 * HALF * 4 * 4 <= BP * SLOT, "the hand-over fits the buffers");
    if (kg == 1) {
      s_m[w][lane] = m_run;
      s_l[w][lane] = l_run;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        float* dst = (dt < HALF ? so0 : so1) + ((w * HALF + dt % HALF) * 64 + lane) * 4;
        *reinterpret_cast<floatx4*>(dst) = orun[dt];
      }
    }
    __syncthreads();
    if (kg == 1) return;
    const float m1 = s_m[w][lane];
    const float M = fmaxf(m_run, m1);
    const float f0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
    const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    l_run = l_run * (double)f0 + s_l[w][lane] * (double)f1;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const floatx4 o1 = *reinterpret_cast<const floatx4*>((dt < HALF ? so0 : so1) + ((w * HALF + dt % HALF) * 64 + lane) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) orun[dt][i] = orun[dt][i] * f0 + o1[i] * f1;
    }
    m_run = M;
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
      for (int i = 0; i < 4; ++i) v4[i] = (double)orun[dt][i] / L;
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
    *reinterpret_cast<float4*>(op + (dt * kWave + lane) * 4) = make_float4(orun[dt][0], orun[dt][1], orun[dt][2], orun[dt][3]);
}

// KG key groups of QT query waves. Up to four query waves: registers for two waves a
// SIMD; more: three.
template <typename T, int D, int QT, int KG>
__global__ __launch_bounds__(64 * QT * KG, 2) void k_attn(const AttnParams p) {
  attn_body<T, D, QT, KG>(p);
}
template <typename T, int D, int QT, int KG>
__global__ __launch_bounds__(64 * QT * KG, 3) void k_attn_wide(const AttnParams p) {
  attn_body<T, D, QT, KG>(p);
}

// Combine the chunks of one (stream, kv head, query tile, 16-dim output slice).
// Only the stream's own chunks count (their number depends only on its reach, so
// the result is the same in any batch). Every wave first finds each query's maximum
// M over all chunk maxima. Then the four waves take contiguous quarters of the
// chunks; lane (lg, lr) owns dims 16 dt + 4 lg .. + 3 of query lr and adds, in chunk
// order in float64, each chunk's partial and sum scaled by 2^(m_c - M) (fp32 exp2,
// as precise as the fp32 chunk partials it scales, and exactly 1 for the chunk
// holding M); the quarters are added in wave order. Loads go in rounds of
// kCombineRound chunks a wave, all in flight at once (indices past the range are
// clamped to a valid chunk and their terms dropped).
constexpr int kCombineWaves = 4, kCombineRound = 8;
template <typename T, int D>
__global__ __launch_bounds__(64 * kCombineWaves) void k_attn_combine(const AttnParams p, int QT) {
  constexpr int NDT = D / 16, NW = kCombineWaves, RC = kCombineRound;
  __shared__ double s_sum[NW][64][5];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int sh = blockIdx.x / QT, qt = blockIdx.x % QT, dt = blockIdx.y;
  const int s = sh / p.n_kv_heads, h = sh % p.n_kv_heads;
  const int nq_local = p.group * p.B;
  const int qi = 16 * qt + lr;
  int Cs = p.ctx_len[s];
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int n_own = attention_chunks(span_pages(lo, Cs), p.cls);   // >= 1
  // (max, sum) of query qi, chunk c: mq[c]
  const float2* mq = reinterpret_cast<const float2*>(p.part_ml) + ((int64_t)sh * (QT * 16) + (qi < nq_local ? qi : 0)) * p.n_chunks;
  const float* po = p.part_o + (((int64_t)sh * p.n_chunks * QT + qt) * NDT + dt) * (kWave * 4) + lane * 4;
  const int64_t cstride = (int64_t)QT * NDT * (kWave * 4);

  // ---- M: lane group lg takes chunks lg, lg + 4, ...
  float M = -INFINITY;
  for (int c0 = 0; c0 < n_own; c0 += 4 * RC) {
    float m[RC];
#pragma unroll
    for (int k = 0; k < RC; ++k) {
      const int c = c0 + 4 * k + lg;
      const float x = mq[c < n_own ? c : n_own - 1].x;
      m[k] = c < n_own ? x : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < RC; ++k) M = fmaxf(M, m[k]);
  }
  M = fmaxf(M, __shfl_xor(M, 16, kWave));
  M = fmaxf(M, __shfl_xor(M, 32, kWave));

  // ---- this wave's quarter
  const int cb = (int)((int64_t)w * n_own / NW), ce = (int)((int64_t)(w + 1) * n_own / NW);
  double L = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = cb; c0 < ce; c0 += RC) {
    float4 v[RC];
    float2 ml[RC];
#pragma unroll
    for (int k = 0; k < RC; ++k) {
      const int c = c0 + k < ce ? c0 + k : ce - 1;
      v[k] = *reinterpret_cast<const float4*>(po + c * cstride);
      ml[k] = mq[c];
    }
#pragma unroll
    for (int k = 0; k < RC; ++k) {
      if (c0 + k < ce) {
        const double f = (ml[k].x == -INFINITY) ? 0.0 : (double)exp2f(ml[k].x - M);
        L += (double)ml[k].y * f;
        o[0] += (double)v[k].x * f;
        o[1] += (double)v[k].y * f;
        o[2] += (double)v[k].z * f;
        o[3] += (double)v[k].w * f;
      }
    }
  }
  s_sum[w][lane][0] = L;
#pragma unroll
  for (int i = 0; i < 4; ++i) s_sum[w][lane][1 + i] = o[i];
  __syncthreads();
  if (w != 0 || qi >= nq_local) return;
  L = s_sum[0][lane][0];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = s_sum[0][lane][1 + i];
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

// The same combine for grids of at most kCombineShort chunks: one workgroup per
// (stream, kv head, query tile), wave dt owning the 16-dim output slice dt. Each lane
// loads every chunk of its query and slice at once and forms exactly the sums above
// (the four quarters in chunk order, then added in quarter order), so the two kernels
// give identical results.
constexpr int kCombineShort = 8;
template <typename T, int D>
__global__ __launch_bounds__(64 * (D / 16)) void k_attn_combine_short(const AttnParams p, int QT) {
  constexpr int NDT = D / 16, RC = kCombineShort;
  const int tid = threadIdx.x, dt = tid >> 6, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int sh = blockIdx.x / QT, qt = blockIdx.x % QT;
  const int s = sh / p.n_kv_heads, h = sh % p.n_kv_heads;
  const int nq_local = p.group * p.B;
  const int qi = 16 * qt + lr;
  if (qi >= nq_local) return;   // whole lane groups of padding queries; no barrier follows
  int Cs = p.ctx_len[s];
  Cs = Cs < 0 ? 0 : (Cs > p.max_ctx ? p.max_ctx : Cs);
  const int lo = p.window > 0 ? (Cs - p.window > 0 ? Cs - p.window : 0) : 0;
  const int n_own = attention_chunks(span_pages(lo, Cs), p.cls);   // 1 <= n_own <= RC
  const float2* mq = reinterpret_cast<const float2*>(p.part_ml) + ((int64_t)sh * (QT * 16) + qi) * p.n_chunks;
  const float* po = p.part_o + (((int64_t)sh * p.n_chunks * QT + qt) * NDT + dt) * (kWave * 4) + lane * 4;
  const int64_t cstride = (int64_t)QT * NDT * (kWave * 4);
  float4 v[RC];
  float2 ml[RC];
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    const int cc = c < n_own ? c : n_own - 1;
    v[c] = *reinterpret_cast<const float4*>(po + cc * cstride);
    ml[c] = mq[cc];
  }
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < RC; ++c)
    if (c < n_own) M = fmaxf(M, ml[c].x);
  // One pass in chunk order; the running quarter sum is added into the total where
  // the next quarter starts (an empty quarter adds an exact zero).
  double L = 0.0, o[4] = {0.0, 0.0, 0.0, 0.0}, Lq = 0.0, oq[4] = {0.0, 0.0, 0.0, 0.0};
  const int e1 = n_own / kCombineWaves, e2 = 2 * n_own / kCombineWaves, e3 = 3 * n_own / kCombineWaves;
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    if (c < n_own) {
      if (c > 0 && (c == e1 || c == e2 || c == e3)) {
        L += Lq;
        Lq = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] += oq[i];
          oq[i] = 0.0;
        }
      }
      const double f = (ml[c].x == -INFINITY) ? 0.0 : (double)exp2f(ml[c].x - M);
      Lq += (double)ml[c].y * f;
      oq[0] += (double)v[c].x * f;
      oq[1] += (double)v[c].y * f;
      oq[2] += (double)v[c].z * f;
      oq[3] += (double)v[c].w * f;
    }
  }
  L += Lq;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] += oq[i];
  const int hl = qi / p.B, jrow = qi % p.B;
  T* dst = static_cast<T*>(p.o) + (int64_t)(s * p.B + jrow) * (p.n_q_heads * D) + (h * p.group + hl) * D + 16 * dt + 4 * lg;
#pragma unroll
  for (int i = 0; i < 4; ++i) Elem<T>::store_d(dst + i, o[i] / L);
}

int attention_query_tiles(int group, int block) { return (group * block + 15) / 16; }

template <typename T, int D, int QT>
static void launch_qt(const AttnParams& p, hipStream_t st) {
  dim3 grid(p.n_chunks, p.n_kv_heads, p.S);
  // Two key groups for five or six query waves: such workgroups run one to a CU (two
  // would put four waves on a SIMD), so the second group doubles the waves a batch is
  // computed with. Up to four query waves two workgroups share a CU already, each
  // with its own copies in flight; the doubled workgroup would run alone.
  constexpr int KG = (AttnCfg<T, D>::NSB % 2 == 0 && QT > 4 && QT <= 6) ? 2 : 1;
  if constexpr (QT > 4) (void)launch_k((k_attn_wide<T, D, QT, KG>), grid, dim3(64 * QT * KG), st, p);
  else (void)launch_k((k_attn<T, D, QT, KG>), grid, dim3(64 * QT * KG), st, p);
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
  if (p.n_chunks <= kCombineShort)
    (void)launch_k((k_attn_combine_short<T, D>), dim3(p.S * p.n_kv_heads * qt), dim3(64 * (D / 16)), st, p, qt);
  else
    (void)launch_k((k_attn_combine<T, D>), dim3(p.S * p.n_kv_heads * qt, D / 16), dim3(64 * kCombineWaves), st, p, qt);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st) {
  if (dtype == 0) return p.head_dim == 64 ? launch_td<float, 64>(p, st) : launch_td<float, 128>(p, st);
  return p.head_dim == 64 ? launch_td<bf16_t, 64>(p, st) : launch_td<bf16_t, 128>(p, st);
}

}  // namespace dfl
