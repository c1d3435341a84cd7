// Kernel parameter blocks and launchers of the draft round (host + device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

enum AMode { A_PLAIN = 0, A_NORMED = 1, A_TAPS = 2 };
enum Epi { EPI_FC = 0, EPI_INJECT = 1, EPI_QKV = 2, EPI_RESID = 3, EPI_SWIGLU = 4, EPI_LMHEAD = 5 };

constexpr int kMaxLayers = 64;
constexpr int kMaxTaps = 8;

// One skinny GEMM launch. Every field not used by the epilogue stays zero.
struct GemmParams {
  int M, N, K;          // rows, output columns (all segments), reduction length
  int n_tiles;          // column tiles (16 or 32 columns each)
  int mgroups;          // row groups of 16 * MT rows
  int iters;            // K / k-elements per iteration
  // A operand
  const void* a;        // A_PLAIN / A_NORMED: [rows, lda]
  int64_t lda;
  int a_rowmap_bm1;     // > 0: logical row r reads source row (r / bm1) * (bm1 + 1) + 1 + r % bm1
  const double* a_ssq;  // A_NORMED: per-row sum-of-squares partials of the source rows
  int a_ssq_parts, a_ssq_ld;
  const void* a_gain;   // A_NORMED: [K]
  float eps;
  const void* taps[kMaxTaps];   // A_TAPS
  int tap_h;
  int64_t tap_stride;
  // B operand
  const void* w0;       // single matrix; or wq / w_gate
  const void* w1;       // wk / w_up
  const void* w2;       // wv
  int nq, nkv;          // n_q*d, n_kv*d
  const void* wk_l[kMaxLayers];
  const void* wv_l[kMaxLayers];
  // epilogue outputs
  double* y_out;        // EPI_FC: y [M, N]; EPI_QKV / EPI_INJECT: raw projections [M, N] (float64)
  double* ssq_out;      // EPI_FC / EPI_RESID: [M, ssq_ld] per-tile sums of squares
  int ssq_ld;
  void* x_io;           // EPI_RESID: residual stream [M, N], updated in place
  void* m_out;          // EPI_SWIGLU: [M, ld_out]
  int ld_out;
  float* logits_out;    // EPI_LMHEAD (nullable), fp32
  float* tile_res;      // EPI_LMHEAD: [M, n_tiles] x (max, argmax bits, second max, -)
};

struct AttnParams {
  int S, B, n_q_heads, n_kv_heads, head_dim, group;
  int window;           // 0 = full
  int n_chunks;         // grid chunks per (stream, kv head): attention_chunks(max reach)
  int max_ctx;
  const int* ctx_len;
  const double* qkv_raw;  // [S*B, ld_raw]: raw q | k | v projections of the block rows
  int ld_raw, nq, nkv;
  const void* q_norm;   // [d]
  const void* k_norm;   // [d]
  float theta, eps;
  const void* kpool;
  const void* vpool;
  const int* page_table;
  int pages_per_stream, page_size, pool_pages;
  void* o;              // [S*B, n_q*d]
  float* part_o;        // [S, n_kv, n_chunks, QT, d/16, 64 lanes, 4] fp32
  float* part_ml;       // [S, n_kv, n_chunks, QT*16, 2]
  float scale_log2;     // log2(e) / sqrt(d)
};

struct KvFinishParams {
  int R, n_layers, n_kv_heads, head_dim;
  const double* raw;    // [R, n_layers * 2 * n_kv * d]: per layer k | v
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
  void* x;              // [S*B, hidden]
  double* ssq;          // [S*B]  sum of squares of each row (one part)
};

struct RowNormParams {
  int R, hidden, n_tiles;
  const double* y;      // [R, hidden]
  const double* ssq_part;  // [R, n_tiles]
  const void* gain;
  void* out;            // [R, hidden]
  float eps;
};

struct VerifyParams {
  int S, B;
  const int* draft;
  const int* target;
  int* accept;
  int* bonus;
  int* committed;
  int* ctx_len;
};

// Context chunking of one stream's reach, a function of that reach alone (so a
// stream's result does not depend on the other streams of the batch):
//   up to 4096 keys: chunks of ~256 keys; up to 65536: 16 chunks; beyond: ~4096 keys.
// The chunk count is non-decreasing in the reach, so a grid sized for the longest
// reach covers every stream.
__host__ __device__ inline int attention_chunks(int reach) {
  if (reach <= 4096) return reach <= 256 ? 1 : (reach + 255) / 256;
  if (reach <= 65536) return 16;
  return (reach + 4095) / 4096;
}
__host__ __device__ inline int attention_chunk_len(int reach) {
  const int n = attention_chunks(reach);
  int cl = (reach + n - 1) / n;
  return (cl + 63) / 64 * 64;
}

int gemm_k_per_iter(int dtype);
int gemm_tile_cols(int epi);
hipError_t launch_gemm(int dtype, int epi, const GemmParams& p, int mt, hipStream_t st);
hipError_t launch_argmax_final(const float* tile_res, int n_tiles, int rows, int* draft_out, float* top2_out,
                               hipStream_t st);
hipError_t launch_kv_finish(int dtype, const KvFinishParams& p, hipStream_t st);
hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st);
int attention_query_tiles(int group, int block);
hipError_t launch_embed(int dtype, const EmbedParams& p, hipStream_t st);
hipError_t launch_rownorm(int dtype, const RowNormParams& p, hipStream_t st);
hipError_t launch_verify(const VerifyParams& p, hipStream_t st);
hipError_t launch_fill_zero(int* p, int64_t n, hipStream_t st);

}  // namespace dfl
