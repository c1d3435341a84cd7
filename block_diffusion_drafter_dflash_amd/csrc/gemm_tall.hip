// Tiled MFMA GEMM of the draft round for many rows (M > 32: batched streams), gfx950.
//
// Y[M, N] = A[M, K] . W[N, K]^T with the same epilogues and outputs as the skinny
// kernel (float64 K-range partials, SwiGLU, LM-head logits and per-32-column top-2).
// A workgroup of 8 waves owns a 256-row x 128-column output tile over one K range, so
// a batch of up to 256 rows reads every weight tile from HBM exactly once (the LM head
// of up to 64 rows: a 64 x 128 tile, two waves); wave (wm, wn) computes a 64 x 64 piece
// as 4 x 4 v_mfma_f32_16x16x32_bf16 tiles (the largest piece whose accumulators fit,
// which keeps LDS reads at 0.5 per MFMA).
// K goes in chunks of 64: a chunk's A (256 x 64) and W (128 x 64, four 4 KB chunks of
// the packed weights) tiles are copied straight from global memory into LDS
// (buffer_load ... lds) through a ring of three buffers, two chunks in flight while
// one is multiplied. A's rows land XOR-swizzled by 16-byte pieces so that fragment
// reads are free of bank conflicts; W's chunks are copied as they are, since their
// bytes already stand in fragment order (each fragment read is 1 KB contiguous). A
// k-step of 32 takes pieces 2 lg + s of the 64 (lane group lg, step s), the order of
// the packed weights; A's fragments follow it. Each buffer is its own LDS
// object, so the compiler sees that copies into one never alias the fragment reads
// of another. The MFMAs accumulate in fp32 over the whole K range, and a K range's
// result is stored as a float32 partial (the consumers add the ranges in float64). Waves whose 64 rows lie past
// the batch (a batch of 33..64 rows uses one of the four row groups) copy their share
// of the tiles but skip the fragment reads and MFMAs; their results are never stored. The summation order differs from the skinny
// kernel's (one K sweep per K range rather than eight wave slices), so a batch on this
// path is not bitwise equal to the same streams drafted alone.
//
// Shapes: K is a multiple of 64 and every weight segment (q | k | v, a layer's k | v,
// SwiGLU halves) a multiple of 32 rows; the configuration checks (hidden,
// intermediate and head projections multiples of 128) guarantee both.
#include "common.hpp"
#include "kernels.h"

namespace dfl {

namespace {

constexpr int BN = 128, BK = 64;
constexpr int WN = 2;                        // waves along N: 64 columns each
constexpr int kRing = 3;                     // chunk buffers
constexpr int ROWB = BK * 2;                 // bytes of one tile row in LDS (bf16)
constexpr int WTILE = BN * ROWB;
constexpr int NPC = ROWB / 16;               // 16-byte pieces per tile row
constexpr int RPL = 1024 / ROWB;             // tile rows per wave-wide load

// Row tile of WM 64-row groups (WM x WN waves, each a 64 x 64 piece). The LM head of
// a batch of up to 64 rows takes WM = 1: a 64 x 128 tile, two waves and 72 KB of
// LDS, so two workgroups share a CU and keep twice the copies in flight of one
// 256-row workgroup whose other six waves would idle. An output element's arithmetic
// (its MFMAs over the K range, in order) does not depend on the tile, so both shapes
// give the same bits.
template <int WM_>
struct Tall {
  static constexpr int WM = WM_;
  static constexpr int kWaves = WM * WN, THREADS = 64 * kWaves;
  static constexpr int BM = 64 * WM;
  static constexpr int ATILE = BM * ROWB;
  static constexpr int QA = ATILE / 1024 / kWaves;   // A loads per wave per chunk
  static constexpr int QB = WTILE / 1024 / kWaves;   // W loads per wave per chunk
  static constexpr int LPW = QA + QB;                // loads per wave per chunk
  static_assert(WN * 64 == BN, "waves tile the output");
  static_assert(ATILE % (1024 * kWaves) == 0 && WTILE % (1024 * kWaves) == 0, "tiles split evenly over the waves");
};
// 16-byte piece p of tile row r sits at piece p ^ swz(r): the 16 rows one fragment
// read touches (128 bytes apart) land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & (NPC - 1); }

// Buffer resource over [base, base + 2 GiB): raw (stride 0) 32-bit accesses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
// Copy 16 bytes a lane from rsrc + lane_off + uniform_off straight into LDS at
// lds_wave_base + 16 lane (buffer_load ... lds: the lane offset register is not
// rewritten per copy, the uniform offset is a scalar). The destination is passed as
// a plain LDS address, so the copy carries no aliasing information and the compiler
// adds no waits of its own for it: the ring's explicit waits order copies and reads.
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, uint32_t uniform_off,
                                               void* lds_wave_base) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr)lds_wave_base);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(uintptr_t)dst, 16, lane_off, uniform_off, 0, 0);
}

__device__ __forceinline__ void tall_top_merge(float& v1, int& i1, float& v2, float bv1, int bi1, float bv2) {
  if (bv1 > v1 || (bv1 == v1 && bi1 < i1)) {
    v2 = fmaxf(v1, bv2);
    v1 = bv1;
    i1 = bi1;
  } else {
    v2 = fmaxf(v2, bv1);
  }
}

// Workgroup barrier for the copy ring: s_waitcnt vmcnt(VM) lgkmcnt(0) (gfx9 encoding),
// then s_barrier. __syncthreads() would also wait for every copy still in flight (its
// fence must cover LDS writes, and the copies write LDS), which would drain the ring.
// Here each wave has waited for its own copies of the chunk about to be read and for
// its own fragment reads, so after the barrier that chunk is complete and the buffer
// about to be refilled is no longer read. The asm's memory clobber keeps the compiler
// from moving memory accesses across it.
template <int VM>
__device__ __forceinline__ void ring_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

}  // namespace

template <int EPI, int AM, int WM_>
__global__ __launch_bounds__(Tall<WM_>::THREADS, 1) void k_gemm_tall(const GemmParams p) {
  using S = Tall<WM_>;
  constexpr int BM = S::BM, ATILE = S::ATILE, QA = S::QA, QB = S::QB, LPW = S::LPW;
  __shared__ __attribute__((aligned(1024))) unsigned char buf0[ATILE + WTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char buf1[ATILE + WTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char buf2[ATILE + WTILE];
  static_assert(kRing == 3, "three buffers");

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wm = w / WN, wn = w % WN;   // rows 64 wm .., columns 64 wn ..

  const int n_ct = EPI == EPI_SWIGLU ? p.N / BN : (p.N + BN - 1) / BN;   // column tiles
  const int n_rt = (p.M + BM - 1) / BM;                                   // row tiles
  // (column tile, K range) columns; the row tiles of a column are 8 apart (one XCD)
  const int wi = blockIdx.x;
  const int col = (wi / (8 * n_rt)) * 8 + wi % 8, rt = (wi / 8) % n_rt;
  if (col >= n_ct * p.ksplit) return;
  const int ks = col % p.ksplit, ct = col / p.ksplit;
  const int n_chunks = p.K / BK;
  const int kb = (int)((int64_t)ks * n_chunks / p.ksplit), ke = (int)((int64_t)(ks + 1) * n_chunks / p.ksplit);

  // ---- copies: wave w issues A loads q = QA w + k (k < QA) and W loads q = QB w + k.
  // Lane l of load q fills bytes [1024 q + 16 l, + 16) of the tile: row RPL q + l / NPC,
  // stored piece l % NPC, i.e. source piece (l % NPC) ^ swz(row). The uniform part of
  // a source address (matrix, first row of the load, chunk) is a scalar, the lane adds
  // a fixed offset. Rows past M (and LM-head rows past N) repeat the last row; their
  // results are never stored.
  // Each load's resource starts at its first row (a 64-bit base), so a lane's offset
  // spans at most RPL - 1 row strides: the host bounds the tap planes' row stride so
  // that this stays inside the resource's 31-bit range for any row count.
  int a_off[QA], w_off[QB];
  int64_t a_row0[QA];
  __amdgpu_buffer_rsrc_t a_rsrc[QA], w_rsrc[QB];
#pragma unroll
  for (int k = 0; k < QA; ++k) {
    const int q = QA * w + k;
    const int row = RPL * q + lane / NPC;
    const int piece = (lane % NPC) ^ swz(row);
    const int ar0 = min(rt * BM + RPL * q, p.M - 1), ar = min(rt * BM + row, p.M - 1);
    if constexpr (AM == A_TAPS) {
      a_row0[k] = (int64_t)ar0 * p.tap_stride;
      a_off[k] = (int)((int64_t)(ar - ar0) * p.tap_stride) + piece * 8;
    } else {
      a_rsrc[k] = rsrc_of(static_cast<const bf16_t*>(p.a) + (int64_t)ar0 * p.lda);
      a_off[k] = (ar - ar0) * (int)p.lda + piece * 8;
    }
  }
  // Weights come packed (dflash_pack_weights): column tile ct is packed tiles 4 ct ..
  // 4 ct + 3, whose chunk ch is 4 KB at ch * 4096 bytes, in fragment order: 1 KB
  // fragment f = 2 nt + u holds, at lane l's 16 bytes, piece 2 (l / 16) + u of row
  // 16 nt + l % 16. Copy q brings fragment q % 4 of packed tile 4 ct + q / 4 to LDS
  // offset q KB of the W tile, unchanged. Tiles past the matrix's last packed tile
  // repeat it (their results are never stored; packed rows past N are zero).
  const int n_ptiles = (p.N + kPackTileRows - 1) / kPackTileRows;
#pragma unroll
  for (int k = 0; k < QB; ++k) {
    const int q = QB * w + k;
    const int pt = min(4 * ct + q / 4, n_ptiles - 1);
    w_rsrc[k] = rsrc_of(packed_tile<bf16_t>(p, pt));
    w_off[k] = (q % 4) * 1024 + lane * 16;   // bytes
  }
  static_assert(BN == 4 * kPackTileRows && BK * 2 == 128 && WTILE == 16 * 1024,
                "a tile is four packed tiles; a chunk is one packed chunk of four 1 KB fragments");
  // Wave w copies A tile rows [RPL QA w, + RPL QA); when they all lie past the batch it
  // copies only its W share (their LDS rows are read by no live wave), and its ring
  // waits count only those copies.
  const bool a_live = RPL * QA * w < p.M - rt * BM;
  auto issue = [&](int ch, unsigned char* buf) {
    const int k0 = ch * BK;
#pragma unroll
    for (int k = 0; k < QA; ++k) {
      if (!a_live) break;
      const int q = QA * w + k;
      if constexpr (AM == A_TAPS) {
        // a chunk never straddles two planes (hidden % 64 == 0)
        const int plane = k0 / p.tap_h;
        buf_load_lds16(rsrc_of(static_cast<const bf16_t*>(p.taps[plane]) + a_row0[k] + (k0 - plane * p.tap_h)),
                       2u * (uint32_t)a_off[k], 0u, buf + q * 1024);
      } else {
        buf_load_lds16(a_rsrc[k], 2u * (uint32_t)a_off[k], 2u * (uint32_t)k0, buf + q * 1024);
      }
    }
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      const int q = QB * w + k;
      buf_load_lds16(w_rsrc[k], (uint32_t)w_off[k], (uint32_t)ch * (kPackTileRows * ROWB), buf + ATILE + q * 1024);
    }
  };

  // ---- fragments: A rows 64 wm + 16 i + lr, W rows 64 wn + 16 j + lr; for k-step s
  // of the chunk, lane group lg reads piece 2 lg + s (k = 16 lg + 8 s .. + 7): from A's
  // swizzled rows, and from W's fragment (nt, u) = (j % 2, s) of packed tile 2 wn +
  // j / 2, lane l at 16 l. One buffer plus one offset, so that every read stays
  // attributed to its buffer.
  constexpr int KS = BK / 32;
  int aoff[KS][4], boff[KS][4];
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = 64 * wm + 16 * i + lr;
      aoff[s][i] = ra * ROWB + (((2 * lg + s) ^ swz(ra)) * 16);
      boff[s][i] = ATILE + (2 * wn + i / 2) * 4096 + (2 * (i % 2) + s) * 1024 + lane * 16;
    }

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // A chunk's 16 fragments are read before its MFMAs; the schedule groups put the
  // second k-step's reads behind the first four MFMAs, so they overlap.
  const bool rows_live = 64 * wm < p.M - rt * BM;   // this wave's 64 rows hold any of the batch's
  auto compute = [&](const unsigned char* buf) {
    if (!rows_live) return;
    uint4 af[KS][4], bf[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[s][i] = *reinterpret_cast<const uint4*>(buf + aoff[s][i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[s][j] = *reinterpret_cast<const uint4*>(buf + boff[s][j]);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma_frag(acc[i][j], af[s][i], bf[s][j], bf16_t());
    static_assert(KS == 2, "the schedule groups below assume two k-steps a chunk");
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // DS reads of k-step 0
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);    // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // DS reads of k-step 1
    __builtin_amdgcn_sched_group_barrier(0x008, 28, 0);   // the remaining MFMAs
  };

  // ---- pipeline over the ring: chunk c lives in buffer (c - kb) % kRing. Before
  // chunk ch is multiplied, this wave's copies of it have landed (the kRing - 2 later
  // chunks may still be in flight) and, after the barrier, everyone's; no wave reads
  // the buffer of chunk ch - 1 any more, so chunk ch + kRing - 1 is copied into it.
  // Copies past the range repeat its last chunk (never read), so that every step has
  // the same number of copies in flight.
  auto step = [&](int ch, const unsigned char* cur, unsigned char* nxt) {
    if (a_live) ring_barrier<(kRing - 2) * LPW>();
    else ring_barrier<(kRing - 2) * QB>();
    issue(min(ch + kRing - 1, ke - 1), nxt);
    compute(cur);
  };
  if (kb < ke) {
    issue(kb, buf0);
    issue(min(kb + 1, ke - 1), buf1);
    for (int ch = kb; ch < ke; ch += kRing) {
      step(ch, buf0, buf2);
      if (ch + 1 >= ke) break;
      step(ch + 1, buf1, buf0);
      if (ch + 2 >= ke) break;
      step(ch + 2, buf2, buf1);
    }
    // the repeated copies must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- epilogue: lane holds rows 64 wm + 16 i + 4 lg + e, columns 64 wn + 16 j + lr
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = rt * BM + 64 * wm + 16 * i + 4 * lg + e;
      const bool rv = r < p.M;
      if constexpr (EPI == EPI_RAW) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = ct * BN + 64 * wn + 16 * j + lr;
          if (rv && n < p.N) reinterpret_cast<float*>(p.y_out)[((int64_t)ks * p.M + r) * p.N + n] = acc[i][j][e];
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
        // packed tile 4 ct + 2 wn + j (j = 0, 1): MFMA column tile 2 j holds its 16 gate
        // rows 64 ct + 32 wn + 16 j + lr, column tile 2 j + 1 the matching up rows
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const double g = acc[i][2 * j][e], u = acc[i][2 * j + 1][e];
          if (rv)
            Elem<bf16_t>::store_d(static_cast<bf16_t*>(p.m_out) + (int64_t)r * p.ld_out + 64 * ct + 32 * wn + 16 * j + lr,
                                  g / (1.0 + exp(-g)) * u);
        }
      } else {   // EPI_LMHEAD: fp32 logits and top-2 of each 32-column group
#pragma unroll
        for (int jg = 0; jg < 2; ++jg) {
          float v1 = -INFINITY, v2 = -INFINITY;
          int i1 = 0x7fffffff;
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = ct * BN + 64 * wn + 32 * jg + 16 * jj + lr;
            const float v = acc[i][2 * jg + jj][e];
            if (n < p.N) {
              if (rv && p.logits_out) p.logits_out[(int64_t)r * (p.ld_out > 0 ? p.ld_out : p.N) + n] = v;
              tall_top_merge(v1, i1, v2, v, n, -INFINITY);
            }
          }
          for (int m = 1; m < 16; m <<= 1) {
            const float o1 = __shfl_xor(v1, m, kWave);
            const int oi = __shfl_xor(i1, m, kWave);
            const float o2 = __shfl_xor(v2, m, kWave);
            tall_top_merge(v1, i1, v2, o1, oi, o2);
          }
          const int grp = 4 * ct + 2 * wn + jg;
          if (rv && lr == 0 && grp < p.n_tiles)
            reinterpret_cast<float4*>(p.tile_res)[(int64_t)r * p.n_tiles + grp] = make_float4(v1, __int_as_float(i1), v2, 0.f);
        }
      }
    }
}

// The SwiGLU product of the gate/up rows past a split (the tail): their ks K-range
// partials ([ks][M][2 tail] float32, in the packed column order of the tail's weights:
// packed tile j holds gate rows 16 j .. 16 j + 15, then the matching up rows) are added
// in range order in float64, as every consumer of K-range partials adds them, and
// silu(g) u is rounded once, as in the tiled kernel's own epilogue. Thread i of row r
// makes m[r][i].
__global__ __launch_bounds__(256) void k_swiglu_tail(const float* part, int ks, int M, int tail, int64_t ld_out,
                                                     bf16_t* m_out) {
  const int r = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= tail) return;
  const int64_t N = 2 * (int64_t)tail;
  const int cg = (i / 16) * 32 + i % 16, cu = cg + 16;
  double g = 0.0, u = 0.0;
  for (int k = 0; k < ks; ++k) {
    const float* pr = part + ((int64_t)k * M + r) * N;
    g += (double)pr[cg];
    u += (double)pr[cu];
  }
  Elem<bf16_t>::store_d(m_out + (int64_t)r * ld_out + i, g / (1.0 + exp(-g)) * u);
}

// The LM head's columns past a split (the tail): their ks K-range partials ([ks][M][tail]
// float32, in vocabulary order) are added in range order in float64 and rounded once
// to the fp32 logit; each 32-column group's largest and second largest logit and the
// largest one's id (lowest on a tie) go to the tile results, as the tiled kernel's own
// epilogue writes them. Block (x, r) takes row r's groups 8 x .. 8 x + 7, a half wave
// (32 lanes) each: lane i of group g, column col0 + 32 g + i.
__global__ __launch_bounds__(256) void k_lmhead_tail(const float* part, int ks, int M, int tail, int64_t N, int col0,
                                                     int n_tiles, float* logits, float4* tile_res) {
  const int r = blockIdx.y, g = blockIdx.x * 8 + (threadIdx.x >> 5), i = threadIdx.x & 31;
  const int c = 32 * g + i;
  float v1 = -INFINITY, v2 = -INFINITY;
  int i1 = 0x7fffffff;
  if (c < tail) {
    double s = 0.0;
    for (int k = 0; k < ks; ++k) s += (double)part[((int64_t)k * M + r) * tail + c];
    v1 = (float)s;
    i1 = col0 + c;
    if (logits) logits[(int64_t)r * N + i1] = v1;
  }
  for (int m = 1; m < 32; m <<= 1) {   // within the half wave
    const float o1 = __shfl_xor(v1, m, kWave);
    const int oi = __shfl_xor(i1, m, kWave);
    const float o2 = __shfl_xor(v2, m, kWave);
    tall_top_merge(v1, i1, v2, o1, oi, o2);
  }
  const int grp = col0 / 32 + g;
  if (i == 0 && 32 * g < tail && grp < n_tiles)
    tile_res[(int64_t)r * n_tiles + grp] = make_float4(v1, __int_as_float(i1), v2, 0.f);
}

hipError_t launch_lmhead_tail(const float* part, int ks, int M, int tail, int64_t N, int col0, int n_tiles,
                              float* logits, float* tile_res, hipStream_t st) {
  const int groups = (tail + 31) / 32;
  (void)launch_k(k_lmhead_tail, dim3((groups + 7) / 8, M), dim3(256), st, part, ks, M, tail, N, col0, n_tiles, logits,
                 reinterpret_cast<float4*>(tile_res));
  return hipGetLastError();
}

hipError_t launch_swiglu_tail(const float* part, int ks, int M, int tail_rows, int64_t ld_out, void* m_out,
                              hipStream_t st) {
  (void)launch_k(k_swiglu_tail, dim3((tail_rows + 255) / 256, M), dim3(256), st, part, ks, M, tail_rows, ld_out,
                 static_cast<bf16_t*>(m_out));
  return hipGetLastError();
}

int gemm_tall_column_tiles(int epi, int N) { return epi == EPI_SWIGLU ? N / BN : (N + BN - 1) / BN; }

// K ranges of the tiled GEMM, a function of the weight's shape only (so that a row's
// arithmetic does not depend on how many rows the batch has). Sized for one row tile
// (up to 256 rows) on 256 CUs, one workgroup each: the split with the shortest
// makespan, rounds(ks) / ks with rounds = ceil(tiles * ks / 256), each extra range
// charged a little for its float64 partial; every range at least 16 chunks.
int gemm_tall_ksplit(int epi, int N, int K) {
  if (epi != EPI_RAW) return 1;
  const int tiles = gemm_tall_column_tiles(epi, N);
  int cap = K / BK / 16 > 1 ? K / BK / 16 : 1;
  cap = cap < 8 ? cap : 8;
  int best = 1;
  double best_cost = 1e30;
  for (int ks = 1; ks <= cap; ++ks) {
    const int rounds = (tiles * ks + 255) / 256;
    const double cost = (double)rounds / ks + 0.02 * ks;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = ks;
    }
  }
  return best;
}

template <int WM>
static hipError_t launch_tall_shape(int epi, int am, const GemmParams& p, hipStream_t st) {
  using S = Tall<WM>;
  const int n_ct = gemm_tall_column_tiles(epi, p.N), n_rt = (p.M + S::BM - 1) / S::BM;
  const int grid = (n_ct * p.ksplit + 7) / 8 * 8 * n_rt;
  if (epi == EPI_RAW && am == A_TAPS)
    (void)launch_k(k_gemm_tall<EPI_RAW, A_TAPS, WM>, dim3(grid), dim3(S::THREADS), st, p);
  else if (epi == EPI_RAW)
    (void)launch_k(k_gemm_tall<EPI_RAW, A_PLAIN, WM>, dim3(grid), dim3(S::THREADS), st, p);
  else if (epi == EPI_SWIGLU)
    (void)launch_k(k_gemm_tall<EPI_SWIGLU, A_PLAIN, WM>, dim3(grid), dim3(S::THREADS), st, p);
  else
    (void)launch_k(k_gemm_tall<EPI_LMHEAD, A_PLAIN, WM>, dim3(grid), dim3(S::THREADS), st, p);
  return hipGetLastError();
}

// The 64-row tile for the LM head of batches of up to 64 rows: its ~1200 column tiles
// fill the GPU several times over, and two workgroups a CU stream it faster (4-stream
// long-context round: 318 -> 299 us). The projections have fewer column tiles than
// CUs; there the eight-wave workgroup, whose idle waves still issue copies, is faster.
hipError_t launch_gemm_tall(int epi, int am, const GemmParams& p, hipStream_t st) {
  if (p.M <= 64 && epi == EPI_LMHEAD) return launch_tall_shape<1>(epi, am, p, st);
  return launch_tall_shape<4>(epi, am, p, st);
}

}  // namespace dfl
