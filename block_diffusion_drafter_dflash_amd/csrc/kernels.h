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
  int n_tiles;          // 128-column tiles
  int splits;           // K splits (workgroups per tile)
  int iters;            // K / k-elements per iteration
  // A operand
  int a_mode;
  const void* a;        // A_PLAIN / A_NORMED: [rows, lda]
  int64_t lda;
  const float* a_inv;   // A_NORMED: 1 / rms per source row
  const void* a_gain;   // A_NORMED: [K]
  int a_rowmap_bm1;     // > 0: logical row r reads source row (r / bm1) * (bm1 + 1) + 1 + r % bm1
  const void* taps[kMaxTaps];
  int tap_h;
  int64_t tap_stride;
  // B operand
  const void* w0;       // single matrix; or wq / w_gate
  const void* w1;       // wk / w_up
  const void* w2;       // wv
  int nq, nkv;          // n_q*d, n_kv*d
  const void* wk_l[kMaxLayers];
  const void* wv_l[kMaxLayers];
  // split-K and row statistics
  float* partials;
  int* counters;        // [mgroups * n_tiles]
  int* counters2;       // [mgroups]
  float* ssq_part;      // [rows, n_tiles]
  float eps;
  // epilogue outputs
  float* y_out;         // EPI_FC: [M, N] fp32
  void* x_io;           // EPI_RESID: residual stream [M, N], updated in place
  float* inv_out;       // EPI_RESID: [M]
  void* m_out;          // EPI_SWIGLU
  int ld_out;
  void *q_out, *k_out, *v_out;      // EPI_QKV
  const void *qn_gain, *kn_gain;    // EPI_QKV
  const void* kn_l[kMaxLayers];     // EPI_INJECT
  int head_dim;
  float theta;
  const int* ctx_len;   // EPI_QKV: positions ctx_len[s] + j
  int max_ctx, block;
  const int* row_stream;  // EPI_INJECT
  const int* row_pos;
  void* kpool_l[kMaxLayers];
  void* vpool_l[kMaxLayers];
  const int* page_table;
  int pages_per_stream, page_size, pool_pages, max_streams, n_kv_heads;
  void* logits_out;     // EPI_LMHEAD
  float* tile_res;      // EPI_LMHEAD: [mgroups, n_tiles, rows] x (v1, i1, v2, -)
  int* draft_out;
  float* top2_out;
};

struct AttnParams {
  int S, B, n_q_heads, n_kv_heads, head_dim, group;
  int window;           // 0 = full
  int n_chunks;         // grid chunks per (stream, kv head): attention_chunks(max reach)
  int max_ctx;
  const int* ctx_len;
  const void* q;        // [S*B, n_q*d]
  const void* kb;       // [S*B, n_kv*d]
  const void* vb;
  const void* kpool;
  const void* vpool;
  const int* page_table;
  int pages_per_stream, page_size, pool_pages;
  void* o;              // [S*B, n_q*d]
  float* part_o;        // [S, n_kv, n_chunks, QT, 64 lanes, d/4 dims...] fp32
  float* part_ml;       // [S, n_kv, n_chunks, QT*16, 2]
  int* counters;        // [S * n_kv]
  float scale_log2;     // log2(e) / sqrt(d)
};

struct EmbedParams {
  int S, B, hidden, vocab, mask_token;
  const int* anchor;
  const void* embed;
  void* x;              // [S*B, hidden]
  float* inv;           // [S*B]  1 / rms of each row
  float eps;
};

struct RowNormParams {
  int R, hidden, n_tiles;
  const float* y;       // [R, hidden]
  const float* ssq_part;// [R, n_tiles]
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
hipError_t launch_gemm(int dtype, int epi, const GemmParams& p, int mt, int mgroups, hipStream_t st);
hipError_t launch_attention(int dtype, const AttnParams& p, hipStream_t st);
int attention_query_tiles(int group, int block);
hipError_t launch_embed(int dtype, const EmbedParams& p, hipStream_t st);
hipError_t launch_rownorm(int dtype, const RowNormParams& p, hipStream_t st);
hipError_t launch_verify(const VerifyParams& p, hipStream_t st);
hipError_t launch_fill_zero(int* p, int64_t n, hipStream_t st);

}  // namespace dfl
