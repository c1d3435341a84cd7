// Kernel parameter blocks and launchers of the draft round (host + device).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace dfl {

enum AMode { A_PLAIN = 0, A_TAPS = 1 };
enum Epi { EPI_RAW = 1, EPI_SWIGLU = 3, EPI_LMHEAD = 4 };

constexpr int kMaxLayers = 64;
constexpr int kMaxTaps = 8;
constexpr int kBlockSlots = 32;   // block rows held by a stream's block K/V pages (block_size <= 32)

// One skinny GEMM launch: Y[M, N] = A[M, K] . W[N, K]^T. Every field not used by the
// epilogue stays zero.
//
// Split K: EPI_RAW launches cut the reduction into ksplit ranges (a function of the
// weight's shape only) and write one float64 partial per range,
// y_out[ks][M][N]. Every consumer forms the full sum as ((P_0 + P_1) + P_2) + ...
// in range order before using it, so results do not depend on scheduling.
struct GemmParams {
  int M, N, K;          // rows, output columns (all segments), reduction length
  int n_tiles;          // column tiles (16 or 32 columns each)
  int mgroups;          // row groups of 16 * MT rows
  int iters;            // K / k-elements per iteration
  int ksplit;           // K ranges (EPI_RAW only; 1 otherwise)
  int n_work;           // n_tiles * mgroups * ksplit work items, one per workgroup
  // A operand
  const void* a;        // A_PLAIN: [M, lda]
  int64_t lda;
  const void* taps[kMaxTaps];   // A_TAPS: plane t holds columns [t * tap_h, (t + 1) * tap_h)
  int tap_h;
  int64_t tap_stride;
  // B operand of the skinny kernel: the packed weights. Tile t (32 output columns) is
  // K / KI consecutive 4 KB chunks of 32 rows x KI elements (KI = 128 bytes of a row),
  // so a tile over a K range is one contiguous region; a chunk's 16-byte pieces are in
  // fragment order (1 KB fragment 2 nt + u: at 16 l, piece 2 (l / 16) + u of row
  // 16 nt + l % 16). wp_seg_tiles > 0 splits the tiles into per-layer segments with
  // their own bases (inject).
  const void* wp;
  int wp_seg_tiles;
  const void* wp_l[kMaxLayers];
  int q4;               // 1: wp holds 4-bit codes with per-group scale and bias (kQ4Chunk bytes a chunk)
  // B operand of the tiled kernel: one matrix, or segments picked by column
  const void* w0;       // single matrix; or wq / w_gate
  const void* w1;       // wk / w_up
  const void* w2;       // wv
  int nq, nkv;          // n_q*d, n_kv*d
  int seg_layers;       // > 0: columns are per layer [wk_l | wv_l] segments (inject)
  const void* wk_l[kMaxLayers];
  const void* wv_l[kMaxLayers];
  // epilogue outputs
  double* y_out;        // EPI_RAW: partials [ksplit, M, N], float64 (skinny kernel) or
                        // float32 (tiled kernel, whose sums are fp32) in the same buffer
  void* m_out;          // EPI_SWIGLU: [M, ld_out]
  int ld_out;           // also the tiled LM head's logits row stride when > 0 (else N)
  float* logits_out;    // EPI_LMHEAD (nullable), fp32
  float* tile_res;      // EPI_LMHEAD: [M, n_tiles] x (max, argmax bits, second max, -)
};

struct AttnParams {
  int S, B, n_q_heads, n_kv_heads, head_dim, group;
  int window;           // 0 = full
  int n_chunks;         // grid chunks per (stream, kv head): attention_chunks(max pages, cls)
  int cls;              // the batch's attention class (attn_class): 0 narrow, 1 mid, 2 wide
  int max_ctx;
  const int* ctx_len;
  const void* q;        // [S*B, n_q*d] rotated, normalised queries
  const void* kblk;     // [S, n_kv, 32, d]   block keys (rows >= B are zero)
  const void* vblk;     // [S, n_kv, d, 32]   block values, transposed
  const void* kpool;    // [pool_pages, n_kv, 16, d]
  const void* vpool;    // [pool_pages, n_kv, d, 16]
  const int* page_table;
  int pages_per_stream, page_size, pool_pages;
  void* o;              // [S*B, n_q*d]
  float* part_o;        // [S, n_kv, n_chunks, QT, d/16, 64 lanes, 4] fp32
  float* part_ml;       // [S, n_kv, n_chunks, QT*16, 2]
  float scale_log2;     // log2(e) / sqrt(d)
};

// Block rows' q | k | v projections -> rotated, normalised q and k, and v, in the
// layouts the attention kernel reads.
struct QkvFinishParams {
  int S, B, n_q_heads, n_kv_heads, head_dim;
  const void* raw;      // partials [ksplit, S*B, nq + 2 nkv]
  int ksplit;
  int raw_f32;          // 1: the partials are float32 (tiled GEMM), 0: float64
  const double2* rope;  // the round's rotary table (EmbedParams::rope)
  const void* q_norm;
  const void* k_norm;
  float eps;
  void* q;              // [S*B, nq]
  void* kblk;           // [S, n_kv, 32, d]
  void* vblk;           // [S, n_kv, d, 32]
};

struct KvFinishParams {
  int R, n_layers, n_kv_heads, head_dim;
  const void* raw;      // partials [ksplit, R, n_layers * 2 * n_kv * d]: per layer k | v
  int ksplit;
  int raw_f32;          // 1: the partials are float32 (tiled GEMM), 0: float64
  const int* row_stream;
  const int* row_pos;
  const void* kn_l[kMaxLayers];
  void* kpool_l[kMaxLayers];
  void* vpool_l[kMaxLayers];
  const int* page_table;
  int pages_per_stream, page_size, pool_pages, max_streams;
  float theta, eps;
};

struct EmbedParams {
  int S, B, hidden, vocab, mask_token;
  const int* anchor;
  const void* embed;
  const void* gain;     // first layer's input-norm gain
  float eps;
  void* x;              // [S*B, hidden] residual stream
  void* a;              // [S*B, hidden] round(RMSNorm(x) * gain)
  // the round's rotary table, shared by every layer: rope[r * head_dim / 2 + i] =
  // (cos, sin) of pos(r) * theta^(-2 i / head_dim) in float64, pos(r) = clamp(ctx_len[s],
  // 0, max_ctx) + j for block row r = s * B + j
  double2* rope;
  int head_dim, max_ctx;
  float theta;
  const int* ctx_len;
};

// Residual add and RMSNorm of one row: with partials,
//   x[src] = round(x[src] + ((P_0 + P_1) + ...)[src])     (written back),
// then a[r] = round(x[src] / sqrt(mean(x[src]^2) + eps) * gain). src(r) = r, or with
// rowmap_bm1 > 0 the r-th mask row: (r / bm1) * (bm1 + 1) + 1 + r % bm1.
struct NormParams {
  int R, hidden, rowmap_bm1;
  void* x;              // [rows, hidden] residual stream
  const void* parts;    // nullable: partials [ksplit, rows, hidden] of the branch
  int ksplit, part_rows;
  int parts_f32;        // 1: the partials are float32 (tiled GEMM), 0: float64
  const void* gain;
  float eps;
  void* a;              // [R, hidden]
};

// Fused rows: y = (P_0 + P_1) + ... (the fc GEMM's partials), out = round(y / rms(y) * gain).
struct RowNormParams {
  int R, hidden, ksplit;
  const void* parts;    // [ksplit, R, hidden]
  int parts_f32;        // 1: the partials are float32 (tiled GEMM), 0: float64
  const void* gain;
  void* out;            // [R, hidden]
  float eps;
};

// One weight matrix copied into the skinny kernel's packed layout (see GemmParams::wp):
// tile t holds output columns 32 t .. 32 t + 31 (zero rows past N) as K / KI chunks
// of 128 bytes a row, each chunk in fragment order. Kinds pick the source row of
// output column n.
enum PackKind { PACK_PLAIN = 0, PACK_QKV = 1, PACK_SWIGLU = 2 };
struct PackJob {
  int kind, N, K, esize;
  int q4;               // 1: quantize to the 4-bit packing (bf16 weights only)
  int nq, nkv;          // PACK_QKV: columns [0, nq) from w0, [nq, nq + nkv) from w1, the rest w2
  const void* w0;       // PACK_PLAIN: the matrix; PACK_SWIGLU: gate rows (tile t: 16 t ..)
  const void* w1;       //   and up rows (the tile's columns 16..31)
  const void* w2;
  void* dst;
};
constexpr int kPackTileRows = 32;
inline size_t packed_bytes(int N, int K, int esize) {
  return (size_t)((N + kPackTileRows - 1) / kPackTileRows) * kPackTileRows * (size_t)K * esize;
}
// 4-bit packing (PackJob::q4): every 64-weight group of a row (one chunk of K) as
// codes (w - bias) / scale, 4 bits each, with the group's bf16 scale and bias (bias the
// group minimum, scale (max - min) / 15 rounded to bf16, codes rounded to nearest even,
// all in float64). A chunk of a tile is 1024 bytes of codes, placed so that lane
// (lr, lg) of the GEMM's wave reads its 16 bytes at 16 (16 lg + lr): rows lr and
// 16 + lr (8 bytes each), k = 16 lg .. 16 lg + 15, two codes a byte (low nibble
// first); then 128 bytes of (scale, bias) pairs, rows lr and 16 + lr at 8 lr.
constexpr int kQ4Group = 64;
constexpr int kQ4Chunk = 1024 + 128;
inline size_t packed_q4_bytes(int N, int K) {
  return (size_t)((N + kPackTileRows - 1) / kPackTileRows) * (size_t)(K / kQ4Group) * kQ4Chunk;
}
hipError_t launch_pack(const PackJob& j, hipStream_t st);

// First element of bf16/fp32 packed tile `tile` of a GEMM (32 rows over all of K).
template <typename T>
__device__ __forceinline__ const T* packed_tile(const GemmParams& p, int tile) {
  const int64_t tile_elems = (int64_t)kPackTileRows * p.K;
  if (p.wp_seg_tiles > 0)
    return static_cast<const T*>(p.wp_l[tile / p.wp_seg_tiles]) + (int64_t)(tile % p.wp_seg_tiles) * tile_elems;
  return static_cast<const T*>(p.wp) + (int64_t)tile * tile_elems;
}

// DFlash2 candidate path selector over [S, B-1] rows of drafted fp32 logits.
constexpr int kSelectMaxK = 16;
constexpr int kSelectMaxB = 32;
struct SelectParams {
  int S, B, V, k, rank;
  int64_t ld;             // row stride of logits, in floats
  const float* logits;
  const void* code_u;     // bf16 [V, rank] (rank 0: unused)
  const void* code_w;
  float min_p;
  int* cand_idx;          // workspace [S * (B-1)][kSelectMaxK]
  double* cand_node;      // workspace [S * (B-1)][kSelectMaxK]: log softmax of each candidate
  int* draft_out;         // [S, B-1], -1 past the stop
  int* draft_len;         // [S]
};
hipError_t launch_select(const SelectParams& p, hipStream_t st);

struct VerifyParams {
  int S, B;
  const int* draft;
  const int* target;
  int* accept;
  int* bonus;
  int* committed;
  int* ctx_len;
};

// Largest vocabulary the sampling kernels take (a slice's segment sums live in LDS),
// and the slices a row is cut into for its reductions.
constexpr int kSampleVocabMax = 262144;
constexpr int kSlices = 32;

// Draws from tempered softmax rows: token_out[r] ~ softmax(logits[r] / T) by inverse
// CDF with uniform u[r]; prob_out (nullable) gets the drawn token's probability.
struct SampleParams {
  int rows, V;
  int64_t ld;           // row stride of logits, in floats
  const float* logits;
  float scale;          // log2(e) / T
  const float* u;
  int* token_out;
  float* prob_out;
  double* slice_stats;  // workspace [rows][kSlices][2]: each slice's (max, weight sum)
};

// Speculative-sampling acceptance. Rows of draft_logits [S, B-1] and target_logits
// [S, B] share the stride ld.
struct SpecVerifyParams {
  int S, B, V;
  int64_t ld;
  const int* draft;
  const float* draft_logits;
  const float* target_logits;
  double* draft_stats;          // workspace [S * (B - 1)][kSlices][2]
  double* target_stats;         // workspace [S * B][kSlices][2]
  double* row_info;             // workspace [S][4]: target row a (max, total), draft row a (max, total)
  double* slice_sums;           // workspace [S][kSlices][2]: residual and target sums of each slice
  float scale;                  // log2(e) / T
  const float* u_accept;        // [S, B - 1]
  const float* u_sample;        // [S]
  int* accept;
  int* token;
  int* committed;               // [S, B], -1 padded
  int* ctx_len;                 // nullable: += accept + 1
};

// Context chunking, in pages of 16 keys, of one stream's reach: a function of that
// reach and of the batch's class (attn_class), so a stream's result does not depend
// on the other streams of a batch of its class. Narrow and mid batches: chunks of
// `sp` pages (8 narrow, 16 mid: a mid batch's streams already give the grid more work
// items) while that makes at most kChunksShort of them; a longer reach is cut into
// chunks of 32 pages, at least kChunksShort and at most 2 * kChunksShort of them
// (up to 4096 pages: a single long stream still fills the GPU); beyond, chunks of
// at most 64 pages. Wide batches (many streams fill the GPU by themselves): chunks
// of up to 64 pages, which keeps the per-chunk partials few. No chunk ever exceeds 64
// pages (the attention kernel keeps a chunk's page ids one per lane), and the count
// never decreases as the reach grows, so a grid sized for the longest reach covers
// every stream.
constexpr int kChunkPagesNarrow = 8;
constexpr int kChunkPagesMid = 16;
constexpr int kChunkPagesLong = 32;
constexpr int kChunkPagesMax = 64;
constexpr int kChunksShort = 32;
__host__ __device__ inline int attention_chunks(int pages, int cls) {
  if (cls == 2 || pages > 2 * kChunksShort * kChunkPagesMax)
    return pages <= kChunkPagesMax ? 1 : (pages + kChunkPagesMax - 1) / kChunkPagesMax;
  const int sp = cls == 1 ? kChunkPagesMid : kChunkPagesNarrow;
  const int n = (pages + sp - 1) / sp;
  if (n <= kChunksShort) return n < 1 ? 1 : n;
  const int m = (pages + kChunkPagesLong - 1) / kChunkPagesLong;
  return m < kChunksShort ? kChunksShort : (m > 2 * kChunksShort ? 2 * kChunksShort : m);
}
__host__ __device__ inline int attention_chunk_pages(int pages, int cls) {
  const int n = attention_chunks(pages, cls);
  return (pages + n - 1) / n;
}
// Pages touched by the key range [lo, hi) (page-aligned span).
__host__ __device__ inline int span_pages(int lo, int hi) { return hi > lo ? (hi + 15) / 16 - lo / 16 : 0; }

// Launch timing for the library's own profiling: while a scope is active on this
// thread, the first launch records `start` as its dispatch begins and every launch
// records `stop` as it ends (the last one's time stands), both on the launch's stream.
struct ProfEvents {
  hipEvent_t start, stop;
  bool used;
};
extern thread_local ProfEvents* g_prof;

template <typename F, typename... Args>
inline hipError_t launch_k(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_prof) {
    if (!g_prof->used) a = g_prof->start;
    g_prof->used = true;
    b = g_prof->stop;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, 0, st, a, b, 0, args...);
  return hipGetLastError();
}

int gemm_k_per_iter(int dtype, int epi, int am, int K, int tap_h);
int gemm_ksplit(int epi, int n_tiles, int iters, int K);
// Batch classes, fixed functions of a batch's block rows (streams x block); a stream's
// results are bitwise the same in any batch of its class.
//  - From kTallMinRows rows on, the GEMMs (bf16) take the tiled kernel (same
//    parameters and outputs as the skinny one). The skinny kernel re-reads a work
//    item's A rows for every 32-column tile, so its L2 traffic grows with the row
//    groups; the tiled kernel copies each weight tile once for up to 256 rows and
//    skips the MFMAs of 64-row groups past the batch.
//  - Attention chunking (attention_chunks): up to 32 rows the narrow class, from
//    kTallMinRows rows the mid class (coarser short chunks), from kAttnWideMinRows
//    rows the wide class (64-page chunks: enough streams fill the GPU by themselves).
//    The mid class starts where the tiled GEMMs do, so it adds no class boundary.
constexpr int kTallMinRows = 33;
constexpr int kAttnWideMinRows = 65;
inline bool gemm_is_tiled(int rows) { return rows >= kTallMinRows; }
inline int attn_class(int rows) { return rows >= kAttnWideMinRows ? 2 : (rows >= kTallMinRows ? 1 : 0); }
int gemm_tall_ksplit(int epi, int N, int K);
int gemm_tall_column_tiles(int epi, int N);
constexpr int kTallRoundTiles = 256;   // column tiles of one round: one per CU
hipError_t launch_gemm_tall(int epi, int am, const GemmParams& p, hipStream_t st);
hipError_t launch_swiglu_tail(const float* part, int ks, int M, int tail_rows, int64_t ld_out, void* m_out,
                              hipStream_t st);   // m_out: bf16, the tail's first column
hipError_t launch_lmhead_tail(const float* part, int ks, int M, int tail, int64_t N, int col0, int n_tiles,
                              float* logits, float* tile_res, hipStream_t st);   // logits: nullable, row stride N
int gemm_tile_cols(int epi);
hipError_t launch_gemm(int dtype, int epi, int am, const GemmParams& p, int mt, hipStream_t st);
hipError_t launch_argmax_final(const float* tile_res, int n_tiles, int rows, int* draft_out, float* top2_out,
                               hipStream_t st);
hipError_t launch_kv_finish(int dtype, const KvFinishParams& p, hipStream_t st);
hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st);
int attention_query_tiles(int group, int block);
hipError_t launch_embed(int dtype, const EmbedParams& p, hipStream_t st);
hipError_t launch_rownorm(int dtype, const RowNormParams& p, hipStream_t st);
hipError_t launch_norm(int dtype, const NormParams& p, hipStream_t st);
hipError_t launch_qkv_finish(int dtype, const QkvFinishParams& p, hipStream_t st);
hipError_t launch_verify(const VerifyParams& p, hipStream_t st);
hipError_t launch_slice_stats(const float* logits, int rows, int V, int64_t ld, float scale, double* stats,
                              hipStream_t st);
hipError_t launch_sample_rows(const SampleParams& p, hipStream_t st);
hipError_t launch_verify_sampling(const SpecVerifyParams& p, hipStream_t st);

}  // namespace dfl
