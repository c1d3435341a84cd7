// Host side of the DFlash draft-round library: config validation, weight binding,
// workspace planning and the launch sequence of each C-ABI call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dfl;

namespace {

thread_local std::string g_create_error = "";

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

namespace dfl {
thread_local ProfEvents* g_prof = nullptr;
}

struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};

struct dflash {
  dflash_config cfg;
  dflash_weights w;
  bool bound = false;
  std::string err;
  std::vector<std::pair<const void*, size_t>> ws_ready;
  bool profiling = false;
  std::vector<ProfRec> prof;
  void* trace = nullptr;        // stage copies of dflash_draft_block (instrumentation)
  size_t trace_cap = 0;
  // the skinny GEMMs' weights in their packed layout (dflash_pack_weights)
  bool packed = false;
  bool q4 = false;              // the packing is the 4-bit one (dflash_pack_weights_q4)
  struct {
    const void *fc, *lm;
    const void *qkv[DFLASH_MAX_LAYERS], *o[DFLASH_MAX_LAYERS], *gu[DFLASH_MAX_LAYERS], *down[DFLASH_MAX_LAYERS];
  } pk;
  std::vector<hipEvent_t> event_pool;

  ~dflash() {
    for (auto& r : prof) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (auto e : event_pool) (void)hipEventDestroy(e);
  }
  hipEvent_t take_event() {
    if (!event_pool.empty()) {
      hipEvent_t e = event_pool.back();
      event_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }

  int esize() const { return cfg.dtype == DFLASH_F32 ? 4 : 2; }
  int nq() const { return cfg.n_q_heads * cfg.head_dim; }
  int nkv() const { return cfg.n_kv_heads * cfg.head_dim; }
};

static int fail(dflash* h, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (h) h->err = buf;
  else g_create_error = buf;
  return code;
}

// ------------------------------------------------------------------ planning

namespace {

struct GemmPlan {
  int am, mt, mgroups, n_tiles, iters, ksplit, n_work;
  bool tall;   // many rows: the tiled kernel
  // Tiled GEMMs whose last round of column tiles would be mostly idle: the tiled kernel
  // takes the outputs before the split whole and the rest (the tail) in tail_ks K
  // ranges, whose float32 partials a finish kernel adds (tail_ks 0: no split).
  // SWIGLU: gate/up rows [0, tail_from) whole, the tail tail_rows gate and as many up
  // rows (k_swiglu_tail). LM head: columns [0, tail_from) whole, the tail tail_rows
  // columns (k_lmhead_tail: logits and each 32-column group's top two).
  int tail_from, tail_rows, tail_ks, tail_cols;   // tail_cols: columns of the tail's partials
  // K-range partials: float64 from the skinny kernel, float32 from the tiled one
  size_t part_bytes(int M, int N) const { return (size_t)ksplit * M * N * (tall ? 4 : 8); }
  size_t tail_part_bytes(int M) const { return (size_t)tail_ks * M * tail_cols * 4; }
};

// Rows are processed in groups of 16 * mt (mt = 1, 2 or 4), or by the tiled kernel
// when `tiled` (bf16 batches of kTallMinRows rows or more). The tiling of N, the K
// ranges and the wave split of each range depend only on the weight's shape, so a
// row's arithmetic depends on M only through the batch's class.
GemmPlan plan_gemm(int dtype, int epi, int am, int M, int N, int K, int tap_h, bool tiled, bool lm_tail = false) {
  GemmPlan g;
  g.am = am;
  g.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  g.mgroups = (M + 16 * g.mt - 1) / (16 * g.mt);
  const int cols = gemm_tile_cols(epi);
  g.n_tiles = (N + cols - 1) / cols;
  g.iters = K / gemm_k_per_iter(dtype, epi, am, K, tap_h);
  g.tall = dtype == DFLASH_BF16 && tiled;
  g.ksplit = g.tall ? gemm_tall_ksplit(epi, N, K) : gemm_ksplit(epi, g.n_tiles, g.iters, K);
  g.n_work = g.n_tiles * g.mgroups * g.ksplit;
  g.tail_from = g.tail_rows = g.tail_ks = g.tail_cols = 0;
  if (g.tall && epi == EPI_SWIGLU) {
    // One 128-column tile (64 gate + 64 up rows) per CU and round: a remainder of at
    // most a quarter round is split along K into as many ranges as fill half a round
    // (each range at least four 64-wide chunks; C4: 16 tiles x 8 ranges, against 16 or
    // 4 ranges: 119.8 against 120.2 and 124.4 us). A function of the weight's shape only.
    const int tiles = gemm_tall_column_tiles(epi, N), rem = tiles % kTallRoundTiles;
    if (tiles > kTallRoundTiles && rem > 0 && rem <= kTallRoundTiles / 4) {
      g.tail_from = (tiles - rem) * 64;
      g.tail_rows = N / 2 - g.tail_from;
      g.tail_ks = std::max(1, std::min(kTallRoundTiles / rem / 2, K / 64 / 4));
      g.tail_cols = 2 * g.tail_rows;
    }
  }
  if (g.tall && epi == EPI_LMHEAD && lm_tail) {
    // The vocabulary's last round of 128-column tiles (at the 9B vocabulary 163 of 1187)
    // costs close to a full round; in three K ranges its workgroups fill the GPU. Taken
    // for mid batches (33-64 block rows), whose float32 tail partials are small (C5: LM
    // head 302 -> 280 us); for wide ones (C4, 240 rows) they cost what the split saves.
    // A function of the weight's shape and the batch's class only.
    const int tiles = gemm_tall_column_tiles(epi, N), rem = tiles % kTallRoundTiles;
    if (tiles > kTallRoundTiles && rem > 0) {
      g.tail_from = (tiles - rem) * 128;
      g.tail_rows = g.tail_cols = N - g.tail_from;
      g.tail_ks = std::max(1, std::min(3, K / 64 / 4));
    }
  }
  return g;
}

struct AttnPlan {
  int n_chunks, qt, cls;
  size_t part_o_bytes, part_ml_bytes;
};

// The most pages any stream's reach can touch: all of [0, max_ctx) for a full layer;
// for a window W, W keys starting anywhere in a page (ceil((W + 15) / 16) pages).
int max_reach_pages(int max_ctx, int window) {
  const int all = (max_ctx + 15) / 16;
  return window > 0 ? std::min(all, (window + 30) / 16) : all;
}

AttnPlan plan_attn(const dflash_config& c, int S, int max_ctx, int window) {
  AttnPlan a;
  a.cls = attn_class(S * c.block_size);
  a.n_chunks = attention_chunks(max_reach_pages(max_ctx, window), a.cls);
  a.qt = attention_query_tiles(c.n_q_heads / c.n_kv_heads, c.block_size);
  const size_t sh = (size_t)S * c.n_kv_heads * a.n_chunks;
  a.part_o_bytes = a.n_chunks > 1 ? sh * a.qt * 64 * (c.head_dim / 16) * 4 * 4 : 0;
  a.part_ml_bytes = a.n_chunks > 1 ? sh * a.qt * 16 * 2 * 4 : 0;
  return a;
}

struct Region {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// Rows of one fuse or inject pass. A call of more than kRowPass rows runs as equal
// passes of at most kRowPass rows (each well above the tiled GEMM's first row count,
// whose per-row arithmetic depends only on the weight's shape), so the K-range
// partials stay bounded at any prompt length and a row's result is bitwise that of
// any other call of the tiled class.
constexpr int kRowPass = 8192;
int row_pass(int R) {
  if (R <= kRowPass) return R;
  const int n = (R + kRowPass - 1) / kRowPass;
  return (R + n - 1) / n;
}
// The largest tap-plane row stride (elements): the tiled kernel's lane offsets span up
// to seven row strides inside a 31-bit buffer range.
constexpr int64_t kMaxPlaneStride = int64_t(1) << 27;

struct FuseLayout {
  GemmPlan g;
  size_t y, end;
};
FuseLayout layout_fuse(const dflash& h, int R) {
  FuseLayout L;
  const auto& c = h.cfg;
  L.g = plan_gemm(c.dtype, EPI_RAW, A_TAPS, R, c.hidden, c.n_taps * c.hidden, c.hidden, gemm_is_tiled(R));
  Region r;
  L.y = r.take(L.g.part_bytes(R, c.hidden));
  L.end = r.off;
  return L;
}

struct InjectLayout {
  GemmPlan g;
  size_t raw, end;
};
InjectLayout layout_inject(const dflash& h, int R) {
  InjectLayout L;
  const auto& c = h.cfg;
  const int N = c.n_layers * 2 * h.nkv();
  L.g = plan_gemm(c.dtype, EPI_RAW, A_PLAIN, R, N, c.hidden, 0, gemm_is_tiled(R));
  Region r;
  L.raw = r.take(L.g.part_bytes(R, N));
  L.end = r.off;
  return L;
}

struct DraftLayout {
  GemmPlan qkv, o, gu, down, lm;
  std::vector<AttnPlan> attn;
  size_t x, a, rope, qkv_raw, o_parts, d_parts, q, kblk, vblk, o_buf, m, gu_tail, part_o, part_ml, tile_res, lm_tail, end;
};
DraftLayout layout_draft(const dflash& h, int S, int max_ctx) {
  DraftLayout L;
  const auto& c = h.cfg;
  const int M = S * c.block_size, Mm = S * (c.block_size - 1);
  const int es = h.esize();
  const bool tiled = gemm_is_tiled(M);   // the batch's class decides every GEMM path of the round
  L.qkv = plan_gemm(c.dtype, EPI_RAW, A_PLAIN, M, h.nq() + 2 * h.nkv(), c.hidden, 0, tiled);
  L.o = plan_gemm(c.dtype, EPI_RAW, A_PLAIN, M, c.hidden, h.nq(), 0, tiled);
  L.gu = plan_gemm(c.dtype, EPI_SWIGLU, A_PLAIN, M, 2 * c.intermediate, c.hidden, 0, tiled);
  L.down = plan_gemm(c.dtype, EPI_RAW, A_PLAIN, M, c.hidden, c.intermediate, 0, tiled);
  L.lm = plan_gemm(c.dtype, EPI_LMHEAD, A_PLAIN, Mm, c.vocab, c.hidden, 0, tiled, attn_class(M) == 1);
  size_t po = 0, pml = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    L.attn.push_back(plan_attn(c, S, max_ctx, c.layer_window[l]));
    po = std::max(po, L.attn.back().part_o_bytes);
    pml = std::max(pml, L.attn.back().part_ml_bytes);
  }
  Region r;
  L.x = r.take((size_t)M * c.hidden * es);
  L.a = r.take((size_t)M * c.hidden * es);
  L.rope = r.take((size_t)M * (c.head_dim / 2) * 16);
  L.qkv_raw = r.take(L.qkv.part_bytes(M, h.nq() + 2 * h.nkv()));
  L.o_parts = r.take(L.o.part_bytes(M, c.hidden));
  L.d_parts = r.take(L.down.part_bytes(M, c.hidden));
  L.q = r.take((size_t)M * h.nq() * es);
  L.kblk = r.take((size_t)S * c.n_kv_heads * kBlockSlots * c.head_dim * es);
  L.vblk = r.take((size_t)S * c.n_kv_heads * kBlockSlots * c.head_dim * es);
  L.o_buf = r.take((size_t)M * h.nq() * es);
  L.m = r.take((size_t)M * c.intermediate * es);
  L.gu_tail = r.take(L.gu.tail_part_bytes(M));
  L.part_o = r.take(po);
  L.part_ml = r.take(pml);
  L.tile_res = r.take((size_t)Mm * L.lm.n_tiles * 16);
  L.lm_tail = r.take(L.lm.tail_part_bytes(Mm));
  L.end = r.off;
  return L;
}

// Sampling: each row's per-slice (max, weight sum); for verify also each stream's
// draw rows (max, total) and per-slice residual and target sums.
struct SampleLayout {
  size_t stats, end;
};
SampleLayout layout_sample(int rows) {
  SampleLayout L;
  Region r;
  L.stats = r.take((size_t)rows * kSlices * 16);
  L.end = r.off;
  return L;
}
struct VerifyLayout {
  size_t draft_stats, target_stats, row_info, slice_sums, end;
};
VerifyLayout layout_verify(const dflash& h, int S) {
  VerifyLayout L;
  const int B = h.cfg.block_size;
  Region r;
  L.draft_stats = r.take((size_t)S * (B - 1) * kSlices * 16);
  L.target_stats = r.take((size_t)S * B * kSlices * 16);
  L.row_info = r.take((size_t)S * 4 * 8);
  L.slice_sums = r.take((size_t)S * kSlices * 16);
  L.end = r.off;
  return L;
}

// Stage copies of a draft (instrumentation): per layer x_in, a, q, block K, block V^T,
// o, x_attn, b, m; then the last residual stream and the final-normed mask rows.
// Offsets in elements of the activation dtype.
struct TraceLayout {
  size_t x_in, a, q, kblk, vblk, o, x_attn, b, m, per_layer, x_last, z, end;
};
TraceLayout layout_trace(const dflash& h, int S) {
  const auto& c = h.cfg;
  const size_t M = (size_t)S * c.block_size, Mm = (size_t)S * (c.block_size - 1), H = c.hidden;
  const size_t blk = (size_t)S * c.n_kv_heads * kBlockSlots * c.head_dim;
  TraceLayout t;
  t.x_in = 0;
  t.a = t.x_in + M * H;
  t.q = t.a + M * H;
  t.kblk = t.q + M * h.nq();
  t.vblk = t.kblk + blk;
  t.o = t.vblk + blk;
  t.x_attn = t.o + M * h.nq();
  t.b = t.x_attn + M * H;
  t.m = t.b + M * H;
  t.per_layer = t.m + M * c.intermediate;
  t.x_last = (size_t)c.n_layers * t.per_layer;
  t.z = t.x_last + M * H;
  t.end = t.z + Mm * H;
  return t;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The packed copies of the GEMM weights, one after another: fc, LM head, then per layer
// [wq | wk | wv], wo, [w_gate | w_up] (16 + 16 rows a tile), w_down.
struct PackLayout {
  size_t fc, lm, qkv[DFLASH_MAX_LAYERS], o[DFLASH_MAX_LAYERS], gu[DFLASH_MAX_LAYERS], down[DFLASH_MAX_LAYERS], end;
};
PackLayout layout_pack(const dflash& h, bool q4) {
  const auto& c = h.cfg;
  const int es = h.esize(), H = c.hidden;
  auto bytes = [&](int N, int K) { return q4 ? packed_q4_bytes(N, K) : packed_bytes(N, K, es); };
  PackLayout L;
  Region r;
  L.fc = r.take(bytes(H, c.n_taps * H));
  L.lm = r.take(bytes(c.vocab, H));
  for (int l = 0; l < c.n_layers; ++l) {
    L.qkv[l] = r.take(bytes(h.nq() + 2 * h.nkv(), H));
    L.o[l] = r.take(bytes(H, h.nq()));
    L.gu[l] = r.take(bytes(2 * c.intermediate, H));
    L.down[l] = r.take(bytes(H, c.intermediate));
  }
  L.end = r.off;
  return L;
}
// Bytes of one packed tile (32 output columns over all of K).
size_t packed_tile_bytes(const dflash& h, int K) {
  return h.q4 ? (size_t)(K / kQ4Group) * kQ4Chunk : (size_t)kPackTileRows * K * h.esize();
}

}  // namespace

// ------------------------------------------------------------------ device scratch

// Scratch for dflash_draft_block_noalloc: one file-scope array on every device the
// library runs on (each device holds its own copy until the process ends). Host code
// never passes the array's name to a kernel: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch_addr;   // (device, address of its scratch)
}  // namespace

static int scratch_of_current_device(dflash* h, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "scratch: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (auto& d : g_scratch_addr)
    if (d.first == dev) {
      *out = d.second;
      return DFLASH_OK;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(h, DFLASH_ERR_DEVICE, "scratch: hipGetSymbolAddress on device %d: %s", dev, hipGetErrorString(e));
  g_scratch_addr.push_back({dev, ptr});
  *out = ptr;
  return DFLASH_OK;
}

// ------------------------------------------------------------------ C-ABI

extern "C" {

const char* dflash_version(void) { return "dflash-mi355x 0.1"; }

void dflash_config_init(dflash_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof *cfg);
  cfg->dtype = DFLASH_BF16;
  cfg->rope_theta = 1.0e6f;
  cfg->rms_eps = 1.0e-6f;
  cfg->page_size = 16;
  cfg->max_streams = 1;
  cfg->pool_pages = 1;
}

int32_t dflash_tensor_count(const dflash_config* cfg) { return cfg ? 11 * cfg->n_layers + 3 : -1; }

static int validate(const dflash_config* c) {
#define REFUSE(...) return fail(nullptr, DFLASH_ERR_CONFIG, __VA_ARGS__)
  if (!c) return fail(nullptr, DFLASH_ERR_ARG, "config is NULL");
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) REFUSE("dtype %d is neither F32 nor BF16", c->dtype);
  if (c->n_layers < 1 || c->n_layers > DFLASH_MAX_LAYERS) REFUSE("n_layers %d outside 1..64", c->n_layers);
  if (c->head_dim != 64 && c->head_dim != 128) REFUSE("head_dim %d is not 64 or 128", c->head_dim);
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
    REFUSE("n_q_heads %d is not a multiple of n_kv_heads %d", c->n_q_heads, c->n_kv_heads);
  if (c->hidden < 128 || c->hidden % 128) REFUSE("hidden %d is not a positive multiple of 128", c->hidden);
  if (c->hidden > (c->dtype == DFLASH_F32 ? 8192 : 16384))
    REFUSE("hidden %d exceeds %d (the row kernels hold a row in registers)", c->hidden, c->dtype == DFLASH_F32 ? 8192 : 16384);
  if (c->intermediate < 128 || c->intermediate % 128) REFUSE("intermediate %d is not a positive multiple of 128", c->intermediate);
  if ((c->n_q_heads * c->head_dim) % 128 || (c->n_kv_heads * c->head_dim) % 128)
    REFUSE("head projections (n_q*d=%d, n_kv*d=%d) are not multiples of 128", c->n_q_heads * c->head_dim,
           c->n_kv_heads * c->head_dim);
  if (c->vocab < 2) REFUSE("vocab %d < 2", c->vocab);
  if (c->n_taps < 1 || c->n_taps > DFLASH_MAX_TAPS) REFUSE("n_taps %d outside 1..8", c->n_taps);
  if (c->target_n_layers < 1) REFUSE("target_n_layers %d < 1", c->target_n_layers);
  for (int i = 0; i < c->n_taps; ++i) {
    if (c->tap_layer_ids[i] < 0 || c->tap_layer_ids[i] >= c->target_n_layers)
      REFUSE("tap %d reads layer %d, past the target's %d layers", i, c->tap_layer_ids[i], c->target_n_layers);
    if (i > 0 && c->tap_layer_ids[i] == c->tap_layer_ids[i - 1]) REFUSE("tap layer %d is repeated", c->tap_layer_ids[i]);
    if (i > 0 && c->tap_layer_ids[i] < c->tap_layer_ids[i - 1])
      REFUSE("tap layer ids must be ascending (tap %d: %d after %d)", i, c->tap_layer_ids[i], c->tap_layer_ids[i - 1]);
  }
  if (c->block_size < 2 || c->block_size > 32) REFUSE("block_size %d outside 2..32", c->block_size);
  if ((c->n_q_heads / c->n_kv_heads) * c->block_size > 128)
    REFUSE("a kv head's block queries ((n_q/n_kv) * block = %d) exceed 128", (c->n_q_heads / c->n_kv_heads) * c->block_size);
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) REFUSE("mask_token_id %d outside the vocab", c->mask_token_id);
  if (c->causal != 0) REFUSE("a causal draft is refused: the block forward is non-causal");
  for (int l = 0; l < c->n_layers; ++l)
    if (c->layer_window[l] < 0) REFUSE("layer %d window %d < 0", l, c->layer_window[l]);
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) REFUSE("rope_theta must be positive");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps)) REFUSE("rms_eps must be >= 0");
  if (c->max_streams < 1) REFUSE("max_streams %d < 1", c->max_streams);
  if (c->page_size != 16) REFUSE("page_size %d is not 16", c->page_size);
  if (c->pool_pages < 1) REFUSE("pool_pages %d < 1", c->pool_pages);
  if ((int64_t)c->pool_pages * c->n_kv_heads > INT32_MAX)
    REFUSE("pool_pages * n_kv_heads = %lld exceeds 2^31 - 1", (long long)c->pool_pages * c->n_kv_heads);
#undef REFUSE
  return DFLASH_OK;
}

int dflash_create(const dflash_config* cfg, dflash** out) {
  if (!out) return fail(nullptr, DFLASH_ERR_ARG, "out is NULL");
  *out = nullptr;
  int rc = validate(cfg);
  if (rc != DFLASH_OK) return rc;
  dflash* h = new dflash();
  h->cfg = *cfg;
  std::memset(&h->w, 0, sizeof h->w);
  *out = h;
  g_create_error = "";
  return DFLASH_OK;
}

void dflash_destroy(dflash* h) { delete h; }

const char* dflash_last_error(const dflash* h) { return h ? h->err.c_str() : g_create_error.c_str(); }

int64_t dflash_fused_row_bytes(const dflash_config* cfg) {
  if (!cfg) return -1;
  return (int64_t)cfg->hidden * (cfg->dtype == DFLASH_F32 ? 4 : 2);
}

int64_t dflash_tap_row_bytes(const dflash_config* cfg, int32_t fusing) {
  if (!cfg) return -1;
  const int64_t row = (int64_t)cfg->hidden * (cfg->dtype == DFLASH_F32 ? 4 : 2);
  return fusing ? (2 * (int64_t)cfg->n_taps + 2) * row : (int64_t)cfg->n_taps * row;
}

int dflash_bind_weights(dflash* h, const dflash_weights* w, const int64_t* shapes) {
  if (!h) return DFLASH_ERR_ARG;
  if (!w || !shapes) return fail(h, DFLASH_ERR_ARG, "weights or shapes is NULL");
  const auto& c = h->cfg;
  const int64_t H = c.hidden, V = c.vocab, I = c.intermediate, d = c.head_dim;
  struct Want { const void* p; int64_t r, k; std::string name; };
  std::vector<Want> want = {
      {w->embed, V, H, "embed"}, {w->lm_head, V, H, "lm_head"}, {w->fc, H, (int64_t)c.n_taps * H, "fc"},
      {w->hidden_norm, H, 1, "hidden_norm"}, {w->norm, H, 1, "norm"}};
  for (int l = 0; l < c.n_layers; ++l) {
    std::string p = "layers." + std::to_string(l) + ".";
    want.push_back({w->in_norm[l], H, 1, p + "in_norm"});
    want.push_back({w->wq[l], h->nq(), H, p + "wq"});
    want.push_back({w->wk[l], h->nkv(), H, p + "wk"});
    want.push_back({w->wv[l], h->nkv(), H, p + "wv"});
    want.push_back({w->wo[l], H, h->nq(), p + "wo"});
    want.push_back({w->q_norm[l], d, 1, p + "q_norm"});
    want.push_back({w->k_norm[l], d, 1, p + "k_norm"});
    want.push_back({w->post_norm[l], H, 1, p + "post_norm"});
    want.push_back({w->w_gate[l], I, H, p + "w_gate"});
    want.push_back({w->w_up[l], I, H, p + "w_up"});
    want.push_back({w->w_down[l], H, I, p + "w_down"});
  }
  for (size_t i = 0; i < want.size(); ++i) {
    const Want& t = want[i];
    if (!t.p) return fail(h, DFLASH_ERR_ARG, "tensor %s: NULL pointer (nothing bound)", t.name.c_str());
    if (!aligned16(t.p)) return fail(h, DFLASH_ERR_ARG, "tensor %s: pointer not 16-byte aligned (nothing bound)", t.name.c_str());
    if (shapes[2 * i] != t.r || shapes[2 * i + 1] != t.k)
      return fail(h, DFLASH_ERR_SHAPE, "tensor %s: shape (%lld, %lld), expected (%lld, %lld) (nothing bound)",
                  t.name.c_str(), (long long)shapes[2 * i], (long long)shapes[2 * i + 1], (long long)t.r,
                  (long long)t.k);
  }
  h->w = *w;
  h->bound = true;
  h->packed = false;
  h->q4 = false;
  return DFLASH_OK;
}

size_t dflash_packed_weight_bytes(const dflash* h) { return h ? layout_pack(*h, false).end : 0; }

size_t dflash_q4_weight_bytes(const dflash* h) {
  return h && h->cfg.dtype == DFLASH_BF16 ? layout_pack(*h, true).end : 0;
}

static int pack_impl(dflash* h, void* buf, size_t bytes, void* stream, bool q4) {
  if (!h) return DFLASH_ERR_ARG;
  if (!h->bound) return fail(h, DFLASH_ERR_STATE, "weights are not bound");
  if (q4 && h->cfg.dtype != DFLASH_BF16) return fail(h, DFLASH_ERR_CONFIG, "4-bit weights are quantized from bf16 weights");
  if (!buf || ((uintptr_t)buf & 255)) return fail(h, DFLASH_ERR_ARG, "packed weight buffer is NULL or not 256-byte aligned");
  const PackLayout L = layout_pack(*h, q4);
  if (bytes < L.end) return fail(h, DFLASH_ERR_CAPACITY, "packed weights need %zu bytes, the buffer holds %zu", L.end, bytes);
  const auto& c = h->cfg;
  const int es = h->esize(), H = c.hidden;
  char* B = static_cast<char*>(buf);
  hipStream_t st = (hipStream_t)stream;
  h->packed = false;
  auto job = [&](int kind, int N, int K, const void* w0, const void* w1, const void* w2, size_t off) {
    PackJob j;
    std::memset(&j, 0, sizeof j);
    j.kind = kind;
    j.N = N;
    j.K = K;
    j.esize = es;
    j.nq = h->nq();
    j.nkv = h->nkv();
    j.w0 = w0;
    j.w1 = w1;
    j.w2 = w2;
    j.dst = B + off;
    j.q4 = q4 ? 1 : 0;
    return launch_pack(j, st);
  };
  hipError_t e = job(PACK_PLAIN, H, c.n_taps * H, h->w.fc, nullptr, nullptr, L.fc);
  if (e == hipSuccess) e = job(PACK_PLAIN, c.vocab, H, h->w.lm_head, nullptr, nullptr, L.lm);
  for (int l = 0; l < c.n_layers && e == hipSuccess; ++l) {
    e = job(PACK_QKV, h->nq() + 2 * h->nkv(), H, h->w.wq[l], h->w.wk[l], h->w.wv[l], L.qkv[l]);
    if (e == hipSuccess) e = job(PACK_PLAIN, H, h->nq(), h->w.wo[l], nullptr, nullptr, L.o[l]);
    if (e == hipSuccess) e = job(PACK_SWIGLU, 2 * c.intermediate, H, h->w.w_gate[l], h->w.w_up[l], nullptr, L.gu[l]);
    if (e == hipSuccess) e = job(PACK_PLAIN, H, c.intermediate, h->w.w_down[l], nullptr, nullptr, L.down[l]);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "pack weights: %s", hipGetErrorString(e));
  h->pk.fc = B + L.fc;
  h->pk.lm = B + L.lm;
  for (int l = 0; l < c.n_layers; ++l) {
    h->pk.qkv[l] = B + L.qkv[l];
    h->pk.o[l] = B + L.o[l];
    h->pk.gu[l] = B + L.gu[l];
    h->pk.down[l] = B + L.down[l];
  }
  h->q4 = q4;
  h->packed = true;
  return DFLASH_OK;
}

int dflash_pack_weights(dflash* h, void* buf, size_t bytes, void* stream) { return pack_impl(h, buf, bytes, stream, false); }

int dflash_pack_weights_q4(dflash* h, void* buf, size_t bytes, void* stream) { return pack_impl(h, buf, bytes, stream, true); }

size_t dflash_workspace_bytes(const dflash* h, int32_t max_rows, int32_t n_streams, int32_t max_ctx) {
  if (!h || max_rows < 0 || n_streams < 1 || n_streams > h->cfg.max_streams || max_ctx < 0) return 0;
  size_t b = 0;
  if (max_rows > 0) {
    // a call of up to max_rows rows runs passes of at most min(max_rows, kRowPass)
    // rows, on the skinny kernel (float64 partials) up to 32 rows, tiled from 33
    for (int r : {std::min(max_rows, kTallMinRows - 1), std::min(max_rows, kRowPass)}) {
      b = std::max(b, layout_fuse(*h, r).end);
      b = std::max(b, layout_inject(*h, r).end);
    }
  }
  b = std::max(b, layout_draft(*h, n_streams, max_ctx).end);
  b = std::max(b, layout_verify(*h, n_streams).end);
  b = std::max(b, layout_sample(std::max(max_rows, n_streams * h->cfg.block_size)).end);
  const size_t sel_rows = (size_t)n_streams * (h->cfg.block_size - 1);
  b = std::max(b, align_up(sel_rows * kSelectMaxK * 4) + sel_rows * kSelectMaxK * 8);
  return b;
}

int dflash_workspace_init(dflash* h, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  (void)stream;   // nothing is enqueued: no part of a workspace must start at zero
  if (!ws || !aligned16(ws)) return fail(h, DFLASH_ERR_ARG, "workspace is NULL or misaligned");
  if (ws_bytes == 0) return fail(h, DFLASH_ERR_CAPACITY, "workspace of 0 bytes");
  for (auto& r : h->ws_ready)
    if (r.first == ws) {
      r.second = ws_bytes;
      return DFLASH_OK;
    }
  h->ws_ready.push_back({ws, ws_bytes});
  return DFLASH_OK;
}

// Times the launches made inside it when profiling is on: the events are recorded by
// the dispatches themselves (start of the first, end of the last), so the interval
// is the kernels' own execution, free of event-packet overhead.
struct ProfScope {
  dflash* h;
  const char* name;
  ProfEvents ev{nullptr, nullptr, false};
  ProfEvents* prev = nullptr;
  bool active = false;
  ProfScope(dflash* h_, const char* n, hipStream_t) : h(h_), name(n) {
    if (!h->profiling) return;
    ev.start = h->take_event();
    ev.stop = h->take_event();
    if (!ev.start || !ev.stop) {
      if (ev.start) h->event_pool.push_back(ev.start);
      if (ev.stop) h->event_pool.push_back(ev.stop);
      return;
    }
    prev = g_prof;
    g_prof = &ev;
    active = true;
  }
  ~ProfScope() {
    if (!active) return;
    g_prof = prev;
    if (ev.used) {
      h->prof.push_back({name, ev.start, ev.stop});
    } else {
      h->event_pool.push_back(ev.start);
      h->event_pool.push_back(ev.stop);
    }
  }
};

static int check_ws(dflash* h, void* ws, size_t ws_bytes, size_t need) {
  if (!ws || !aligned16(ws)) return fail(h, DFLASH_ERR_ARG, "workspace is NULL or misaligned");
  bool ready = false;
  for (auto& r : h->ws_ready)
    if (r.first == ws && ws_bytes <= r.second) ready = true;
  if (!ready) return fail(h, DFLASH_ERR_STATE, "workspace was not initialised with dflash_workspace_init");
  if (ws_bytes < need) return fail(h, DFLASH_ERR_CAPACITY, "workspace holds %zu bytes, this call needs %zu", ws_bytes, need);
  return DFLASH_OK;
}

static GemmParams gemm_base(const GemmPlan& g, int M, int N, int K) {
  GemmParams p;
  std::memset(&p, 0, sizeof p);
  p.M = M;
  p.N = N;
  p.K = K;
  p.n_tiles = g.n_tiles;
  p.mgroups = g.mgroups;
  p.iters = g.iters;
  p.ksplit = g.ksplit;
  p.n_work = g.n_work;
  return p;
}

static_assert(sizeof(GemmParams) <= 4000, "kernel argument block too large");

static hipError_t run_gemm(int dtype, const GemmPlan& g, int epi, const GemmParams& p, hipStream_t st) {
  if (g.tall && g.tail_ks > 0 && epi == EPI_LMHEAD) {
    // LM head split by columns: [0, tail_from) tiled whole (logits at row stride N);
    // the tail's packed tiles (32 columns each) as a tiled GEMM in tail_ks K ranges into
    // the float32 partials at p.y_out, which k_lmhead_tail finishes.
    GemmParams a = p;
    a.N = g.tail_from;
    a.ld_out = p.N;
    hipError_t e = launch_gemm_tall(EPI_LMHEAD, g.am, a, st);
    if (e != hipSuccess) return e;
    GemmParams b = p;
    b.N = g.tail_rows;
    b.wp = static_cast<const char*>(p.wp) + (size_t)(g.tail_from / kPackTileRows) * kPackTileRows * p.K * 2;   // bf16 packing
    b.ksplit = g.tail_ks;
    e = launch_gemm_tall(EPI_RAW, g.am, b, st);
    if (e != hipSuccess) return e;
    return launch_lmhead_tail(reinterpret_cast<const float*>(p.y_out), g.tail_ks, p.M, g.tail_rows, p.N, g.tail_from,
                              p.n_tiles, p.logits_out, p.tile_res, st);
  }
  if (g.tall && g.tail_ks > 0) {
    // SWIGLU split by gate/up rows: [0, tail_from) tiled whole; the tail's packed tiles
    // (16 gate + 16 up rows each) as a tiled GEMM in tail_ks K ranges into the float32
    // partials at p.y_out, which k_swiglu_tail adds into m[:, tail_from:].
    GemmParams a = p;
    a.N = 2 * g.tail_from;
    hipError_t e = launch_gemm_tall(epi, g.am, a, st);
    if (e != hipSuccess) return e;
    GemmParams b = p;
    b.N = 2 * g.tail_rows;
    b.wp = static_cast<const char*>(p.wp) + (size_t)(g.tail_from / 16) * kPackTileRows * p.K * 2;   // bf16 packing
    b.ksplit = g.tail_ks;
    e = launch_gemm_tall(EPI_RAW, g.am, b, st);
    if (e != hipSuccess) return e;
    return launch_swiglu_tail(reinterpret_cast<const float*>(p.y_out), g.tail_ks, p.M, g.tail_rows, p.ld_out,
                              static_cast<char*>(p.m_out) + (size_t)g.tail_from * 2, st);   // bf16 m
  }
  if (g.tall) return launch_gemm_tall(epi, g.am, p, st);
  return launch_gemm(dtype, epi, g.am, p, g.mt, st);
}

int dflash_fuse_taps(dflash* h, const void* const* tap_planes, int64_t plane_row_stride, int32_t n_rows,
                     void* fused_out, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  const auto& c = h->cfg;
  if (!h->bound) return fail(h, DFLASH_ERR_STATE, "weights are not bound");
  if (n_rows < 0) return fail(h, DFLASH_ERR_ARG, "n_rows %d < 0", n_rows);
  if (n_rows == 0) return DFLASH_OK;
  if (!tap_planes || !fused_out || !aligned16(fused_out)) return fail(h, DFLASH_ERR_ARG, "tap_planes or fused_out invalid");
  for (int t = 0; t < c.n_taps; ++t)
    if (!tap_planes[t] || !aligned16(tap_planes[t])) return fail(h, DFLASH_ERR_ARG, "tap plane %d is NULL or misaligned", t);
  if (plane_row_stride < c.hidden || plane_row_stride % 8 || plane_row_stride > kMaxPlaneStride)
    return fail(h, DFLASH_ERR_ARG, "plane_row_stride %lld must be >= hidden, <= 2^27 and a multiple of 8",
                (long long)plane_row_stride);
  const int pass = row_pass(n_rows);
  int rc = check_ws(h, ws, ws_bytes, layout_fuse(*h, pass).end);
  if (rc) return rc;
  if (!h->packed) return fail(h, DFLASH_ERR_STATE, "weights are not packed (dflash_pack_weights)");
  if (h->q4 && gemm_is_tiled(pass))
    return fail(h, DFLASH_ERR_UNIMPLEMENTED, "4-bit weights run on calls of at most %d rows", kTallMinRows - 1);
  char* W = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  const size_t es = h->esize();
  for (int r0 = 0; r0 < n_rows; r0 += pass) {
    const int rows = std::min(pass, n_rows - r0);
    const FuseLayout L = layout_fuse(*h, rows);
    GemmParams p = gemm_base(L.g, rows, c.hidden, c.n_taps * c.hidden);
    for (int t = 0; t < c.n_taps; ++t)
      p.taps[t] = static_cast<const char*>(tap_planes[t]) + (size_t)r0 * plane_row_stride * es;
    p.tap_h = c.hidden;
    p.tap_stride = plane_row_stride;
    p.w0 = h->w.fc;
    p.wp = h->pk.fc;
    p.q4 = h->q4 ? 1 : 0;
    p.y_out = reinterpret_cast<double*>(W + L.y);
    hipError_t e;
    {
      ProfScope ps(h, "fuse_fc_gemm", st);
      e = run_gemm(c.dtype, L.g, EPI_RAW, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "fuse fc: %s", hipGetErrorString(e));
    RowNormParams rn;
    rn.R = rows;
    rn.hidden = c.hidden;
    rn.ksplit = L.g.ksplit;
    rn.parts = p.y_out;
    rn.parts_f32 = L.g.tall ? 1 : 0;   // the tiled kernel's partials are float32
    rn.gain = h->w.hidden_norm;
    rn.out = static_cast<char*>(fused_out) + (size_t)r0 * c.hidden * es;
    rn.eps = c.rms_eps;
    {
      ProfScope ps(h, "fuse_rownorm", st);
      e = launch_rownorm(c.dtype, rn, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "fuse norm: %s", hipGetErrorString(e));
  }
  return DFLASH_OK;
}

static int check_kv(dflash* h, const dflash_kv* kv) {
  const auto& c = h->cfg;
  if (!kv || !kv->page_table) return fail(h, DFLASH_ERR_ARG, "kv or its page table is NULL");
  if (kv->pages_per_stream < 1) return fail(h, DFLASH_ERR_ARG, "pages_per_stream %d < 1", kv->pages_per_stream);
  for (int l = 0; l < c.n_layers; ++l)
    if (!kv->k_pool[l] || !kv->v_pool[l] || !aligned16(kv->k_pool[l]) || !aligned16(kv->v_pool[l]))
      return fail(h, DFLASH_ERR_ARG, "layer %d K/V pool is NULL or misaligned", l);
  return DFLASH_OK;
}

// Injected K/V of the layers in layer_mask. The GEMM's K split is the one of the
// all-layer inject (a function of the weight's full shape), so a selected layer's
// K/V are bitwise those of an inject of every layer.
static int inject_impl(dflash* h, const void* fused, int32_t n_rows, const int32_t* row_stream,
                       const int32_t* row_pos, const dflash_kv* kv, uint64_t layer_mask, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  const auto& c = h->cfg;
  if (!h->bound) return fail(h, DFLASH_ERR_STATE, "weights are not bound");
  if (n_rows < 0) return fail(h, DFLASH_ERR_ARG, "n_rows %d < 0", n_rows);
  if (c.n_layers < 64 && (layer_mask >> c.n_layers) != 0)
    return fail(h, DFLASH_ERR_ARG, "layer_mask names a layer past n_layers (%d)", c.n_layers);
  int sel[DFLASH_MAX_LAYERS];
  int n_sel = 0;
  for (int l = 0; l < c.n_layers; ++l)
    if ((layer_mask >> l) & 1ull) sel[n_sel++] = l;
  if (n_rows == 0 || n_sel == 0) return DFLASH_OK;
  if (!fused || !aligned16(fused) || !row_stream || !row_pos) return fail(h, DFLASH_ERR_ARG, "fused, row_stream or row_pos invalid");
  int rc = check_kv(h, kv);
  if (rc) return rc;
  const int pass = row_pass(n_rows);
  rc = check_ws(h, ws, ws_bytes, layout_inject(*h, pass).end);
  if (rc) return rc;
  if (!h->packed) return fail(h, DFLASH_ERR_STATE, "weights are not packed (dflash_pack_weights)");
  if (h->q4 && gemm_is_tiled(pass))
    return fail(h, DFLASH_ERR_UNIMPLEMENTED, "4-bit weights run on calls of at most %d rows", kTallMinRows - 1);
  char* W = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  for (int r0 = 0; r0 < n_rows; r0 += pass) {
    const int rows = std::min(pass, n_rows - r0);
    const InjectLayout L = layout_inject(*h, rows);
    // the selected layers' [wk | wv] segments side by side; tiles of the all-layer plan
    GemmPlan g = L.g;
    const int N = n_sel * 2 * h->nkv();
    g.n_tiles = (N + gemm_tile_cols(EPI_RAW) - 1) / gemm_tile_cols(EPI_RAW);
    g.n_work = g.n_tiles * g.mgroups * g.ksplit;
    GemmParams p = gemm_base(g, rows, N, c.hidden);
    p.a = static_cast<const char*>(fused) + (size_t)r0 * c.hidden * h->esize();
    p.lda = c.hidden;
    p.nkv = h->nkv();
    p.seg_layers = n_sel;
    p.wp_seg_tiles = 2 * h->nkv() / kPackTileRows;
    p.q4 = h->q4 ? 1 : 0;
    for (int i = 0; i < n_sel; ++i) {
      p.wk_l[i] = h->w.wk[sel[i]];
      p.wv_l[i] = h->w.wv[sel[i]];
      // a layer's [wk | wv] tiles follow its wq tiles in the packed [wq | wk | wv]
      p.wp_l[i] = static_cast<const char*>(h->pk.qkv[sel[i]]) +
                  (size_t)(h->nq() / kPackTileRows) * packed_tile_bytes(*h, c.hidden);
    }
    p.y_out = reinterpret_cast<double*>(W + L.raw);
    hipError_t e;
    {
      ProfScope ps(h, "inject_kv_gemm", st);
      e = run_gemm(c.dtype, g, EPI_RAW, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "inject: %s", hipGetErrorString(e));
    KvFinishParams kf;
    std::memset(&kf, 0, sizeof kf);
    kf.R = rows;
    kf.n_layers = n_sel;
    kf.n_kv_heads = c.n_kv_heads;
    kf.head_dim = c.head_dim;
    kf.raw = p.y_out;
    kf.ksplit = g.ksplit;
    kf.raw_f32 = g.tall ? 1 : 0;
    kf.row_stream = row_stream + r0;
    kf.row_pos = row_pos + r0;
    for (int i = 0; i < n_sel; ++i) {
      kf.kn_l[i] = h->w.k_norm[sel[i]];
      kf.kpool_l[i] = kv->k_pool[sel[i]];
      kf.vpool_l[i] = kv->v_pool[sel[i]];
    }
    kf.page_table = kv->page_table;
    kf.pages_per_stream = kv->pages_per_stream;
    kf.page_size = c.page_size;
    kf.pool_pages = c.pool_pages;
    kf.max_streams = c.max_streams;
    kf.theta = c.rope_theta;
    kf.eps = c.rms_eps;
    {
      ProfScope ps(h, "inject_kv_finish", st);
      e = launch_kv_finish(c.dtype, kf, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "inject finish: %s", hipGetErrorString(e));
  }
  return DFLASH_OK;
}

int dflash_inject_kv(dflash* h, const void* fused, int32_t n_rows, const int32_t* row_stream,
                     const int32_t* row_pos, const dflash_kv* kv, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  const int nl = h->cfg.n_layers;
  const uint64_t all = nl >= 64 ? ~0ull : ((1ull << nl) - 1ull);
  return inject_impl(h, fused, n_rows, row_stream, row_pos, kv, all, ws, ws_bytes, stream);
}

int dflash_inject_kv_layers(dflash* h, const void* fused, int32_t n_rows, const int32_t* row_stream,
                            const int32_t* row_pos, const dflash_kv* kv, uint64_t layer_mask, void* ws,
                            size_t ws_bytes, void* stream) {
  return inject_impl(h, fused, n_rows, row_stream, row_pos, kv, layer_mask, ws, ws_bytes, stream);
}

uint64_t dflash_layers_reading(const dflash* h, int32_t pos, int32_t ctx_len) {
  if (!h || pos < 0 || pos >= ctx_len) return 0;
  const auto& c = h->cfg;
  uint64_t m = 0;
  for (int l = 0; l < c.n_layers; ++l) {
    const int w = c.layer_window[l];
    const int lo = w > 0 ? (ctx_len - w > 0 ? ctx_len - w : 0) : 0;
    if (pos >= lo) m |= 1ull << l;
  }
  return m;
}

// The draft with its workspace given by the caller (dflash_draft_block), or with the
// device's own file-scope scratch array (in_scratch: dflash_draft_block_noalloc).
static int draft_impl(dflash* h, int32_t n_streams, const int32_t* anchor, const int32_t* ctx_len,
                      int32_t max_ctx_len, const dflash_kv* kv, int32_t* draft_out, void* logits_out,
                      float* top2_out, void* ws, size_t ws_bytes, void* stream, bool in_scratch) {
  if (!h) return DFLASH_ERR_ARG;
  const auto& c = h->cfg;
  if (!h->bound) return fail(h, DFLASH_ERR_STATE, "weights are not bound");
  if (n_streams < 1 || n_streams > c.max_streams)
    return fail(h, DFLASH_ERR_CAPACITY, "n_streams %d outside 1..max_streams (%d)", n_streams, c.max_streams);
  if (!anchor || !ctx_len || !draft_out) return fail(h, DFLASH_ERR_ARG, "anchor, ctx_len or draft_out is NULL");
  if ((logits_out && !aligned16(logits_out)) || (top2_out && ((uintptr_t)top2_out & 7)))
    return fail(h, DFLASH_ERR_ARG, "logits_out / top2_out misaligned");
  int rc = check_kv(h, kv);
  if (rc) return rc;
  if (max_ctx_len < 0) return fail(h, DFLASH_ERR_ARG, "max_ctx_len %d < 0", max_ctx_len);
  if ((int64_t)max_ctx_len > (int64_t)kv->pages_per_stream * c.page_size)
    return fail(h, DFLASH_ERR_CAPACITY, "max_ctx_len %d is past the cache span of %d tokens", max_ctx_len,
                kv->pages_per_stream * c.page_size);
  DraftLayout L = layout_draft(*h, n_streams, max_ctx_len);
  if (in_scratch) {
    if (L.end > ws_bytes)
      return fail(h, DFLASH_ERR_CAPACITY, "this draft needs %zu bytes of scratch, the device array holds %zu", L.end,
                  ws_bytes);
  } else {
    rc = check_ws(h, ws, ws_bytes, L.end);
    if (rc) return rc;
  }
  if (!h->packed) return fail(h, DFLASH_ERR_STATE, "weights are not packed (dflash_pack_weights)");
  if (h->q4 && gemm_is_tiled(n_streams * c.block_size))
    return fail(h, DFLASH_ERR_UNIMPLEMENTED, "4-bit weights run on drafts of at most %d block rows", kTallMinRows - 1);

  const int B = c.block_size, M = n_streams * B, Mm = n_streams * (B - 1);
  char* W = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  const TraceLayout T = layout_trace(*h, n_streams);
  const size_t es = h->esize();
  if (h->trace && h->trace_cap < T.end * es)
    return fail(h, DFLASH_ERR_CAPACITY, "trace buffer holds %zu bytes, this draft needs %zu", h->trace_cap, T.end * es);
  // instrumentation: copy a stored tensor into the trace (no-op when tracing is off)
  auto trace = [&](size_t off, const void* src, size_t elems) -> hipError_t {
    if (!h->trace) return hipSuccess;
    return hipMemcpyAsync(static_cast<char*>(h->trace) + off * es, src, elems * es, hipMemcpyDeviceToDevice, st);
  };
  const size_t MH = (size_t)M * c.hidden, blk = (size_t)n_streams * c.n_kv_heads * kBlockSlots * c.head_dim;
  void* X = W + L.x;
  void* A = W + L.a;
  double* o_parts = reinterpret_cast<double*>(W + L.o_parts);   // wo . o, per K range
  double* d_parts = reinterpret_cast<double*>(W + L.d_parts);   // w_down . m, per K range
  double* qkv_raw = reinterpret_cast<double*>(W + L.qkv_raw);
  hipError_t e;

  EmbedParams ep;
  ep.S = n_streams;
  ep.B = B;
  ep.hidden = c.hidden;
  ep.vocab = c.vocab;
  ep.mask_token = c.mask_token_id;
  ep.anchor = anchor;
  ep.embed = h->w.embed;
  ep.gain = h->w.in_norm[0];
  ep.eps = c.rms_eps;
  ep.x = X;
  ep.a = A;
  ep.rope = reinterpret_cast<double2*>(W + L.rope);
  ep.head_dim = c.head_dim;
  ep.max_ctx = max_ctx_len;
  ep.theta = c.rope_theta;
  ep.ctx_len = ctx_len;
  {
    ProfScope ps(h, "embed", st);
    e = launch_embed(c.dtype, ep, st);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "embed: %s", hipGetErrorString(e));

  // x = round(x + branch) (the branch's K-range partials added in order), then the
  // next normalised input a = round(RMSNorm(x) * gain)
  auto norm = [&](const char* name, const double* parts, const GemmPlan& g, const void* gain, int rows,
                  int rowmap_bm1) {
    NormParams np;
    np.R = rows;
    np.hidden = c.hidden;
    np.rowmap_bm1 = rowmap_bm1;
    np.x = X;
    np.parts = parts;
    np.ksplit = g.ksplit;
    np.parts_f32 = g.tall ? 1 : 0;
    np.part_rows = M;
    np.gain = gain;
    np.eps = c.rms_eps;
    np.a = A;
    ProfScope ps(h, name, st);
    return launch_norm(c.dtype, np, st);
  };

  for (int l = 0; l < c.n_layers; ++l) {
    // X += w_down . m of the previous layer (residual add 2); a = round(RMSNorm(X) * in_norm)
    // (layer 0: a is written by embed)
    if (l > 0) {
      e = norm("norm_in", d_parts, L.down, h->w.in_norm[l], M, 0);
      if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d input norm: %s", l, hipGetErrorString(e));
    }
    const size_t tl = (size_t)l * T.per_layer;
    if ((e = trace(tl + T.x_in, X, MH)) != hipSuccess || (e = trace(tl + T.a, A, MH)) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));
    // raw q | k | v = a . [wq | wk | wv]^T
    GemmParams p = gemm_base(L.qkv, M, h->nq() + 2 * h->nkv(), c.hidden);
    p.a = A;
    p.lda = c.hidden;
    p.w0 = h->w.wq[l];
    p.w1 = h->w.wk[l];
    p.w2 = h->w.wv[l];
    p.wp = h->pk.qkv[l];
    p.q4 = h->q4 ? 1 : 0;
    p.nq = h->nq();
    p.nkv = h->nkv();
    p.y_out = qkv_raw;
    {
      ProfScope ps(h, "qkv_gemm", st);
      e = run_gemm(c.dtype, L.qkv, EPI_RAW, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d qkv: %s", l, hipGetErrorString(e));

    // q, k = RoPE(q_norm / k_norm(raw)), v = raw, into the attention layouts
    QkvFinishParams qf;
    qf.S = n_streams;
    qf.B = B;
    qf.n_q_heads = c.n_q_heads;
    qf.n_kv_heads = c.n_kv_heads;
    qf.head_dim = c.head_dim;
    qf.raw = qkv_raw;
    qf.ksplit = L.qkv.ksplit;
    qf.raw_f32 = L.qkv.tall ? 1 : 0;
    qf.rope = reinterpret_cast<const double2*>(W + L.rope);
    qf.q_norm = h->w.q_norm[l];
    qf.k_norm = h->w.k_norm[l];
    qf.eps = c.rms_eps;
    qf.q = W + L.q;
    qf.kblk = W + L.kblk;
    qf.vblk = W + L.vblk;
    {
      ProfScope ps(h, "qkv_finish", st);
      e = launch_qkv_finish(c.dtype, qf, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d qkv finish: %s", l, hipGetErrorString(e));
    if ((e = trace(tl + T.q, W + L.q, (size_t)M * h->nq())) != hipSuccess ||
        (e = trace(tl + T.kblk, W + L.kblk, blk)) != hipSuccess || (e = trace(tl + T.vblk, W + L.vblk, blk)) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));

    AttnParams ap;
    std::memset(&ap, 0, sizeof ap);
    ap.S = n_streams;
    ap.B = B;
    ap.n_q_heads = c.n_q_heads;
    ap.n_kv_heads = c.n_kv_heads;
    ap.head_dim = c.head_dim;
    ap.group = c.n_q_heads / c.n_kv_heads;
    ap.window = c.layer_window[l];
    ap.n_chunks = L.attn[l].n_chunks;
    ap.cls = L.attn[l].cls;
    ap.max_ctx = max_ctx_len;
    ap.ctx_len = ctx_len;
    ap.q = W + L.q;
    ap.kblk = W + L.kblk;
    ap.vblk = W + L.vblk;
    ap.kpool = kv->k_pool[l];
    ap.vpool = kv->v_pool[l];
    ap.page_table = kv->page_table;
    ap.pages_per_stream = kv->pages_per_stream;
    ap.page_size = c.page_size;
    ap.pool_pages = c.pool_pages;
    ap.o = W + L.o_buf;
    ap.part_o = reinterpret_cast<float*>(W + L.part_o);
    ap.part_ml = reinterpret_cast<float*>(W + L.part_ml);
    ap.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    {
      ProfScope ps(h, c.layer_window[l] > 0 ? "attention_sliding" : "attention_full", st);
      e = launch_attention(c.dtype, ap, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d attention: %s", l, hipGetErrorString(e));
    if ((e = trace(tl + T.o, W + L.o_buf, (size_t)M * h->nq())) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));

    // wo . o, per K range
    p = gemm_base(L.o, M, c.hidden, h->nq());
    p.a = W + L.o_buf;
    p.lda = h->nq();
    p.w0 = h->w.wo[l];
    p.wp = h->pk.o[l];
    p.q4 = h->q4 ? 1 : 0;
    p.y_out = o_parts;
    {
      ProfScope ps(h, "o_proj_gemm", st);
      e = run_gemm(c.dtype, L.o, EPI_RAW, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d o_proj: %s", l, hipGetErrorString(e));

    // X += wo . o (residual add 1); a = round(RMSNorm(X) * post_norm);
    // m = round(silu(w_gate . a) * (w_up . a))
    e = norm("norm_post", o_parts, L.o, h->w.post_norm[l], M, 0);
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d post norm: %s", l, hipGetErrorString(e));
    if ((e = trace(tl + T.x_attn, X, MH)) != hipSuccess || (e = trace(tl + T.b, A, MH)) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));
    p = gemm_base(L.gu, M, 2 * c.intermediate, c.hidden);
    p.a = A;
    p.lda = c.hidden;
    p.w0 = h->w.w_gate[l];
    p.w1 = h->w.w_up[l];
    p.wp = h->pk.gu[l];
    p.q4 = h->q4 ? 1 : 0;
    p.m_out = W + L.m;
    p.ld_out = c.intermediate;
    p.y_out = reinterpret_cast<double*>(W + L.gu_tail);   // the tail's K-range partials (if any)
    {
      ProfScope ps(h, "gate_up_gemm", st);
      e = run_gemm(c.dtype, L.gu, EPI_SWIGLU, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d gate/up: %s", l, hipGetErrorString(e));
    if ((e = trace(tl + T.m, W + L.m, (size_t)M * c.intermediate)) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));

    // w_down . m, per K range (added to X by the next norm: residual add 2)
    p = gemm_base(L.down, M, c.hidden, c.intermediate);
    p.a = W + L.m;
    p.lda = c.intermediate;
    p.w0 = h->w.w_down[l];
    p.wp = h->pk.down[l];
    p.q4 = h->q4 ? 1 : 0;
    p.y_out = d_parts;
    {
      ProfScope ps(h, "down_gemm", st);
      e = run_gemm(c.dtype, L.down, EPI_RAW, p, st);
    }
    if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "layer %d down: %s", l, hipGetErrorString(e));
  }

  // Last residual add and final norm of the mask rows (compacted), LM head, argmax
  // (lowest index on a tie).
  e = norm("norm_final", d_parts, L.down, h->w.norm, Mm, B - 1);
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "final norm: %s", hipGetErrorString(e));
  if ((e = trace(T.x_last, X, MH)) != hipSuccess || (e = trace(T.z, A, (size_t)Mm * c.hidden)) != hipSuccess)
    return fail(h, DFLASH_ERR_DEVICE, "trace: %s", hipGetErrorString(e));
  GemmParams p = gemm_base(L.lm, Mm, c.vocab, c.hidden);
  p.a = A;
  p.lda = c.hidden;
  p.w0 = h->w.lm_head;
  p.wp = h->pk.lm;
  p.q4 = h->q4 ? 1 : 0;
  p.logits_out = static_cast<float*>(logits_out);
  p.tile_res = reinterpret_cast<float*>(W + L.tile_res);
  p.y_out = reinterpret_cast<double*>(W + L.lm_tail);   // the tail's K-range partials (if any)
  {
    ProfScope ps(h, "lm_head_gemm", st);
    e = run_gemm(c.dtype, L.lm, EPI_LMHEAD, p, st);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "lm head: %s", hipGetErrorString(e));
  {
    ProfScope ps(h, "argmax_final", st);
    e = launch_argmax_final(p.tile_res, L.lm.n_tiles, Mm, draft_out, top2_out, st);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "argmax: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

int dflash_draft_block(dflash* h, int32_t n_streams, const int32_t* anchor, const int32_t* ctx_len,
                       int32_t max_ctx_len, const dflash_kv* kv, int32_t* draft_out, void* logits_out,
                       float* top2_out, void* ws, size_t ws_bytes, void* stream) {
  return draft_impl(h, n_streams, anchor, ctx_len, max_ctx_len, kv, draft_out, logits_out, top2_out, ws, ws_bytes,
                    stream, false);
}

int dflash_draft_block_noalloc(dflash* h, int32_t n_streams, const int32_t* anchor, const int32_t* ctx_len,
                               int32_t max_ctx_len, const dflash_kv* kv, int32_t* draft_out, void* logits_out,
                               float* top2_out, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(h, &ws);
  if (rc != DFLASH_OK) return rc;
  // no profiling events either: the call creates nothing
  const bool prof = h->profiling;
  h->profiling = false;
  const int out = draft_impl(h, n_streams, anchor, ctx_len, max_ctx_len, kv, draft_out, logits_out, top2_out, ws,
                             kScratchBytes, stream, true);
  h->profiling = prof;
  return out;
}

int dflash_verify_greedy(dflash* h, int32_t n_streams, const int32_t* draft, const int32_t* target_argmax,
                         int32_t* accept_len, int32_t* bonus, int32_t* committed, int32_t* ctx_len_inout,
                         void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  if (n_streams < 1) return fail(h, DFLASH_ERR_ARG, "n_streams %d < 1", n_streams);
  if (!draft || !target_argmax || !accept_len || !bonus || !committed)
    return fail(h, DFLASH_ERR_ARG, "a verify pointer is NULL");
  VerifyParams vp;
  vp.S = n_streams;
  vp.B = h->cfg.block_size;
  vp.draft = draft;
  vp.target = target_argmax;
  vp.accept = accept_len;
  vp.bonus = bonus;
  vp.committed = committed;
  vp.ctx_len = ctx_len_inout;
  hipError_t e;
  {
    ProfScope ps(h, "verify", (hipStream_t)stream);
    e = launch_verify(vp, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "verify: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

int dflash_sample_rows(dflash* h, int32_t n_rows, const float* logits, int64_t row_stride, float temperature,
                       const float* u, int32_t* token_out, float* prob_out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  if (n_rows < 0) return fail(h, DFLASH_ERR_ARG, "n_rows %d < 0", n_rows);
  if (n_rows == 0) return DFLASH_OK;
  if (!logits || !u || !token_out) return fail(h, DFLASH_ERR_ARG, "a sampling pointer is NULL");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(h, DFLASH_ERR_ARG, "temperature must be positive and finite");
  if (row_stride < h->cfg.vocab) return fail(h, DFLASH_ERR_ARG, "row_stride %lld < vocab", (long long)row_stride);
  if (h->cfg.vocab > kSampleVocabMax)
    return fail(h, DFLASH_ERR_CONFIG, "sampling takes a vocabulary of at most %d ids", kSampleVocabMax);
  const SampleLayout L = layout_sample(n_rows);
  int rc = check_ws(h, ws, ws_bytes, L.end);
  if (rc != DFLASH_OK) return rc;
  SampleParams sp;
  sp.rows = n_rows;
  sp.V = h->cfg.vocab;
  sp.ld = row_stride;
  sp.logits = logits;
  sp.scale = (float)(1.4426950408889634 / (double)temperature);
  sp.u = u;
  sp.token_out = token_out;
  sp.prob_out = prob_out;
  sp.slice_stats = reinterpret_cast<double*>(static_cast<char*>(ws) + L.stats);
  hipError_t e;
  {
    ProfScope ps(h, "sample_rows", (hipStream_t)stream);
    e = launch_sample_rows(sp, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "sample rows: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

int dflash_verify_sampling(dflash* h, int32_t n_streams, const int32_t* draft, const float* draft_logits,
                           const float* target_logits, int64_t row_stride, float temperature, const float* u_accept,
                           const float* u_sample, int32_t* accept_len, int32_t* token, int32_t* committed,
                           int32_t* ctx_len_inout, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  const auto& c = h->cfg;
  if (n_streams < 1 || n_streams > c.max_streams)
    return fail(h, DFLASH_ERR_ARG, "n_streams %d outside [1, %d]", n_streams, c.max_streams);
  if (!draft || !draft_logits || !target_logits || !u_accept || !u_sample || !accept_len || !token || !committed)
    return fail(h, DFLASH_ERR_ARG, "a verify pointer is NULL");
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(h, DFLASH_ERR_ARG, "temperature must be positive and finite");
  if (row_stride < c.vocab) return fail(h, DFLASH_ERR_ARG, "row_stride %lld < vocab", (long long)row_stride);
  if (c.vocab > kSampleVocabMax)
    return fail(h, DFLASH_ERR_CONFIG, "sampling takes a vocabulary of at most %d ids", kSampleVocabMax);
  const VerifyLayout L = layout_verify(*h, n_streams);
  int rc = check_ws(h, ws, ws_bytes, L.end);
  if (rc != DFLASH_OK) return rc;
  char* W = static_cast<char*>(ws);
  const int B = c.block_size;
  const float scale = (float)(1.4426950408889634 / (double)temperature);
  SpecVerifyParams vp;
  vp.S = n_streams;
  vp.B = B;
  vp.V = c.vocab;
  vp.ld = row_stride;
  vp.draft = draft;
  vp.draft_logits = draft_logits;
  vp.target_logits = target_logits;
  vp.draft_stats = reinterpret_cast<double*>(W + L.draft_stats);
  vp.target_stats = reinterpret_cast<double*>(W + L.target_stats);
  vp.row_info = reinterpret_cast<double*>(W + L.row_info);
  vp.slice_sums = reinterpret_cast<double*>(W + L.slice_sums);
  vp.scale = scale;
  vp.u_accept = u_accept;
  vp.u_sample = u_sample;
  vp.accept = accept_len;
  vp.token = token;
  vp.committed = committed;
  vp.ctx_len = ctx_len_inout;
  const hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  {
    ProfScope ps(h, "verify_sampling", st);
    e = launch_verify_sampling(vp, st);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "verify sampling: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

size_t dflash_trace_bytes(const dflash* h, int32_t n_streams) {
  if (!h || n_streams < 1 || n_streams > h->cfg.max_streams) return 0;
  return layout_trace(*h, n_streams).end * h->esize();
}

int dflash_set_trace(dflash* h, void* buf, size_t bytes) {
  if (!h) return DFLASH_ERR_ARG;
  if (buf && !aligned16(buf)) return fail(h, DFLASH_ERR_ARG, "trace buffer misaligned");
  h->trace = bytes ? buf : nullptr;
  h->trace_cap = buf ? bytes : 0;
  return DFLASH_OK;
}

int dflash_select_path(dflash* h, int32_t n_streams, const float* logits, int64_t row_stride, const void* code_u,
                       const void* code_w, int32_t rank, int32_t top_k, float min_p, int32_t* draft_out,
                       int32_t* draft_len, void* ws, size_t ws_bytes, void* stream) {
  if (!h) return DFLASH_ERR_ARG;
  const auto& c = h->cfg;
  if (n_streams < 1 || n_streams > c.max_streams)
    return fail(h, DFLASH_ERR_ARG, "n_streams %d outside [1, %d]", n_streams, c.max_streams);
  if (!logits || !draft_out || !draft_len) return fail(h, DFLASH_ERR_ARG, "logits, draft_out or draft_len is NULL");
  if (top_k < 1 || top_k > kSelectMaxK || top_k > c.vocab)
    return fail(h, DFLASH_ERR_ARG, "top_k %d outside [1, min(%d, vocab)]", top_k, kSelectMaxK);
  if (rank < 0) return fail(h, DFLASH_ERR_ARG, "rank %d < 0", rank);
  if (rank > 0 && (!code_u || !code_w)) return fail(h, DFLASH_ERR_ARG, "rank %d needs both codebooks", rank);
  if (row_stride < c.vocab) return fail(h, DFLASH_ERR_ARG, "row_stride %lld < vocab", (long long)row_stride);
  if (!(min_p >= 0.f) || !std::isfinite(min_p)) return fail(h, DFLASH_ERR_ARG, "min_p must be finite and >= 0");
  const size_t rows = (size_t)n_streams * (c.block_size - 1);
  const size_t need = align_up(rows * kSelectMaxK * 4) + rows * kSelectMaxK * 8;
  int rc = check_ws(h, ws, ws_bytes, need);
  if (rc != DFLASH_OK) return rc;
  char* W = static_cast<char*>(ws);
  SelectParams sp;
  sp.S = n_streams;
  sp.B = c.block_size;
  sp.V = c.vocab;
  sp.k = top_k;
  sp.rank = rank;
  sp.ld = row_stride;
  sp.logits = logits;
  sp.code_u = code_u;
  sp.code_w = code_w;
  sp.min_p = min_p;
  sp.cand_idx = reinterpret_cast<int*>(W);
  sp.cand_node = reinterpret_cast<double*>(W + align_up(rows * kSelectMaxK * 4));
  sp.draft_out = draft_out;
  sp.draft_len = draft_len;
  hipError_t e;
  {
    ProfScope ps(h, "select_path", (hipStream_t)stream);
    e = launch_select(sp, (hipStream_t)stream);
  }
  if (e != hipSuccess) return fail(h, DFLASH_ERR_DEVICE, "select path: %s", hipGetErrorString(e));
  return DFLASH_OK;
}

int dflash_set_profiling(dflash* h, int32_t enable) {
  if (!h) return DFLASH_ERR_ARG;
  h->profiling = enable != 0;
  return DFLASH_OK;
}

int dflash_profile_read(dflash* h, char* buf, size_t len) {
  if (!h || !buf || len == 0) return DFLASH_ERR_ARG;
  std::map<std::string, std::pair<long, double>> acc;
  for (auto& r : h->prof) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return fail(h, DFLASH_ERR_DEVICE, "profile: event wait failed");
    auto& a = acc[r.name];
    a.first += 1;
    a.second += ms;
    h->event_pool.push_back(r.a);
    h->event_pool.push_back(r.b);
  }
  h->prof.clear();
  std::string out;
  for (auto& kv : acc) {
    char line[256];
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  size_t n = std::min(out.size(), len - 1);
  std::memcpy(buf, out.data(), n);
  buf[n] = 0;
  return (int)n;
}

}  // extern "C"
