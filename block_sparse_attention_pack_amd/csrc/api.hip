// C ABI of the sparse decode-attention library: argument checks, error
// reporting and kernel launches. See include/bsa.h for the contract.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define BSA_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

// Checks shared by every entry point that takes a layout and a selection config.
int check_common(const bsa_kv_layout* L, const bsa_select_cfg* c, bsa::UnitGeom* g) {
  BSA_REQUIRE(L && c, BSA_ERR_INVALID_ARG, "layout and cfg must not be NULL");
  BSA_REQUIRE(L->head_dim == bsa::kHeadDim, BSA_ERR_UNSUPPORTED, "head_dim %d: only 128 is supported",
              L->head_dim);
  BSA_REQUIRE(L->block_size == bsa::kBlock, BSA_ERR_UNSUPPORTED,
              "block_size %d: only 128 is supported", L->block_size);
  BSA_REQUIRE(L->batch >= 1 && L->num_kv_heads >= 1 && L->num_q_heads >= 1, BSA_ERR_INVALID_ARG,
              "batch, num_kv_heads and num_q_heads must be >= 1");
  BSA_REQUIRE(L->num_q_heads % L->num_kv_heads == 0, BSA_ERR_INVALID_ARG,
              "num_q_heads %d is not a multiple of num_kv_heads %d", L->num_q_heads, L->num_kv_heads);
  const int G = L->num_q_heads / L->num_kv_heads;
  BSA_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, BSA_ERR_UNSUPPORTED,
              "query heads per KV head %d: supported 1, 2, 4, 8, 16", G);
  BSA_REQUIRE(L->max_tokens >= bsa::kBlock && L->max_tokens % bsa::kBlock == 0,
              BSA_ERR_INVALID_ARG, "max_tokens %d must be a positive multiple of 128",
              L->max_tokens);
  BSA_REQUIRE(L->max_tokens <= (1 << 26), BSA_ERR_UNSUPPORTED, "max_tokens %d above 2^26",
              L->max_tokens);
  BSA_REQUIRE(int64_t(L->batch) * L->num_kv_heads <= 65535, BSA_ERR_UNSUPPORTED,
              "batch * num_kv_heads above 65535");
  BSA_REQUIRE(L->kv_stride_t >= bsa::kHeadDim && L->kv_stride_t % 8 == 0 && L->kv_stride_h >= 0 &&
                  L->kv_stride_h % 8 == 0 && L->kv_stride_b >= 0 && L->kv_stride_b % 8 == 0,
              BSA_ERR_INVALID_ARG,
              "strides (b %lld, h %lld, t %lld): t >= 128, all non-negative multiples of 8",
              (long long)L->kv_stride_b, (long long)L->kv_stride_h, (long long)L->kv_stride_t);
  BSA_REQUIRE(L->kv_dtype == BSA_DTYPE_F16 || L->kv_dtype == BSA_DTYPE_BF16, BSA_ERR_UNSUPPORTED,
              "kv_dtype %d", L->kv_dtype);
  BSA_REQUIRE(L->value_dtype == BSA_VALUE_CACHE || L->value_dtype == BSA_VALUE_NVFP4,
              BSA_ERR_UNSUPPORTED, "value_dtype %d", L->value_dtype);
  BSA_REQUIRE(c->granularity == BSA_GRANULARITY_BLOCK || c->granularity == BSA_GRANULARITY_TOKEN ||
                  c->granularity == BSA_GRANULARITY_CLUSTER,
              BSA_ERR_INVALID_ARG, "granularity %d", c->granularity);
  BSA_REQUIRE(std::isfinite(c->softmax_scale) && c->softmax_scale > 0.0f, BSA_ERR_INVALID_ARG,
              "softmax_scale must be finite and > 0");
  const int NB = L->max_tokens / bsa::kBlock;
  if (c->granularity == BSA_GRANULARITY_CLUSTER) {
    BSA_REQUIRE(c->num_clusters >= 1 && c->num_clusters <= bsa::kMaxClusters, BSA_ERR_UNSUPPORTED,
                "num_clusters %d: supported 1 .. %d", c->num_clusters, bsa::kMaxClusters);
    BSA_REQUIRE(c->budget >= 1 && c->budget <= L->max_tokens, BSA_ERR_INVALID_ARG,
                "token budget %d must lie in [1, %d]", c->budget, L->max_tokens);
    BSA_REQUIRE(c->n_tail_pages == 0 && c->proj_dtype == 0 && c->query_dtype == 0 &&
                    c->top_p == 0.0f,
                BSA_ERR_INVALID_ARG,
                "cluster mode takes no tail pages, projection, query format or top_p");
  } else if (c->granularity == BSA_GRANULARITY_BLOCK) {
    BSA_REQUIRE(c->n_tail_pages >= 0 && c->n_tail_pages <= 2, BSA_ERR_INVALID_ARG,
                "n_tail_pages %d must be 0, 1 or 2", c->n_tail_pages);
    BSA_REQUIRE(c->budget >= 1 && c->budget >= c->n_tail_pages && c->budget <= NB,
                BSA_ERR_INVALID_ARG, "block budget %d must lie in [max(1, n_tail_pages), %d]",
                c->budget, NB);
  } else {
    BSA_REQUIRE(c->n_tail_pages == 0, BSA_ERR_INVALID_ARG, "token mode takes no tail pages");
    BSA_REQUIRE(c->budget >= 1 && c->budget <= L->max_tokens, BSA_ERR_INVALID_ARG,
                "token budget %d must lie in [1, %d]", c->budget, L->max_tokens);
    const int r = c->proj_rank;
    BSA_REQUIRE(r == 8 || r == 16 || r == 32 || r == 64 || r == 128, BSA_ERR_UNSUPPORTED,
                "proj_rank %d: supported 8, 16, 32, 64, 128", r);
    BSA_REQUIRE(c->proj_dtype == BSA_PROJ_BF16 || c->proj_dtype == BSA_PROJ_FP8,
                BSA_ERR_UNSUPPORTED, "proj_dtype %d", c->proj_dtype);
    BSA_REQUIRE(c->proj_dtype == BSA_PROJ_BF16 || r >= 16, BSA_ERR_UNSUPPORTED,
                "an FP8 projected cache needs proj_rank >= 16");
  }
  if (c->granularity == BSA_GRANULARITY_CLUSTER) {
    // checked above
  } else if (c->granularity == BSA_GRANULARITY_BLOCK) {
    BSA_REQUIRE(c->proj_dtype == BSA_PROJ_BF16, BSA_ERR_INVALID_ARG,
                "proj_dtype applies to token mode only (must be 0 in block mode)");
    BSA_REQUIRE(c->query_dtype == BSA_QUERY_F16 || c->query_dtype == BSA_QUERY_NVFP4,
                BSA_ERR_UNSUPPORTED, "query_dtype %d", c->query_dtype);
    BSA_REQUIRE(c->top_p == 0.0f, BSA_ERR_INVALID_ARG,
                "top_p applies to token mode only (must be 0 in block mode)");
  } else {
    BSA_REQUIRE(c->query_dtype == BSA_QUERY_F16, BSA_ERR_INVALID_ARG,
                "query_dtype applies to block mode only (must be 0 in token mode)");
    BSA_REQUIRE(std::isfinite(c->top_p) && c->top_p >= 0.0f && c->top_p <= 1.0f,
                BSA_ERR_INVALID_ARG, "top_p %g must lie in [0, 1]", double(c->top_p));
    BSA_REQUIRE(c->top_p == 0.0f || c->budget <= bsa::kTopPMaxBudget, BSA_ERR_UNSUPPORTED,
                "top_p needs a token budget <= %d (got %d)", bsa::kTopPMaxBudget, c->budget);
  }
  g->B = L->batch;
  g->Hkv = L->num_kv_heads;
  g->Hq = L->num_q_heads;
  g->G = G;
  g->Tmax = L->max_tokens;
  g->NBmax = NB;
  g->sb = L->kv_stride_b;
  g->sh = L->kv_stride_h;
  g->st = L->kv_stride_t;
  g->dtype = L->kv_dtype;
  g->vq = L->value_dtype == BSA_VALUE_NVFP4;
  return BSA_OK;
}

}  // namespace

namespace {

// Attention, then the merge: in the attention launch's last group of each unit
// up to bsa::kFusedMergeMaxSplits splits, in the row-parallel merge launch
// beyond. With sel_scores the attention launch also selects the blocks (block
// mode) into idx and count.
hipError_t attend_and_merge(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const void* q,
                            const void* k, const void* v, const int32_t* seq_lens,
                            int32_t* idx, int32_t* count, const uint16_t* tail_k,
                            const uint16_t* tail_v, int32_t num_splits, float* part_o,
                            float* part_lse, uint32_t* counters, float* out, float* out_lse,
                            hipStream_t s, const float* sel_scores = nullptr) {
  const bool merge_in_last_group = num_splits <= bsa::kFusedMergeMaxSplits;
  hipError_t e = bsa::launch_attention(
      g, cfg->granularity, cfg->budget, cfg->n_tail_pages, cfg->softmax_scale,
      static_cast<const _Float16*>(q), k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
      part_o, part_lse, merge_in_last_group ? counters : nullptr, out, out_lse, sel_scores,
      sel_scores ? idx : nullptr, sel_scores ? count : nullptr, s);
  if (e == hipSuccess && !merge_in_last_group)
    e = bsa::launch_combine(g.B * g.Hq, num_splits, part_o, part_lse, out, out_lse, s);
  return e;
}

// The calls that have no cluster-mode form.
int reject_cluster(const bsa_select_cfg* cfg, const char* what) {
  BSA_REQUIRE(cfg->granularity != BSA_GRANULARITY_CLUSTER, BSA_ERR_UNSUPPORTED,
              "%s has no cluster mode: use bsa_score_select_clusters and bsa_attend_combine",
              what);
  return BSA_OK;
}

// Argument checks of each stage, run before anything is enqueued (the combined
// calls run every stage's checks first).
int check_scan_args(const bsa_select_cfg* cfg, const void* q, const uint8_t* codes,
                    const uint8_t* scales, const float* global_scale, const void* kproj,
                    const float* proj, const int32_t* seq_lens, const float* scores) {
  BSA_REQUIRE(q && aligned16(q) && seq_lens && scores, BSA_ERR_INVALID_ARG,
              "q (16-byte aligned), seq_lens and scores are required");
  if (cfg->granularity == BSA_GRANULARITY_BLOCK)
    BSA_REQUIRE(codes && scales && global_scale && aligned16(codes) && aligned16(scales),
                BSA_ERR_INVALID_ARG,
                "block mode needs codes, scales (16-byte aligned) and global_scale");
  else
    BSA_REQUIRE(kproj && proj && aligned16(kproj) && aligned16(scores), BSA_ERR_INVALID_ARG,
                "token mode needs kproj and scores (16-byte aligned) and proj");
  return BSA_OK;
}

int check_select_args(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const float* scores,
                      const int32_t* seq_lens, const void* workspace, size_t workspace_bytes,
                      const int32_t* idx, const int32_t* count) {
  BSA_REQUIRE(scores && seq_lens && idx && count, BSA_ERR_INVALID_ARG,
              "scores, seq_lens, idx and count are required");
  if (cfg->granularity == BSA_GRANULARITY_TOKEN) {
    const size_t need = bsa::token_select_workspace(g, cfg->budget, cfg->top_p);
    BSA_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), BSA_ERR_WORKSPACE,
                "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  }
  return BSA_OK;
}

int check_attend_args(const bsa_select_cfg* cfg, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, const int32_t* idx, const int32_t* count,
                      const uint16_t* tail_k, const uint16_t* tail_v, int32_t num_splits,
                      const float* part_o, const float* part_lse) {
  BSA_REQUIRE(q && k && v && aligned16(q) && aligned16(k) && aligned16(v), BSA_ERR_INVALID_ARG,
              "q, k, v must be 16-byte aligned device pointers");
  BSA_REQUIRE(seq_lens && idx && count && part_o && part_lse, BSA_ERR_INVALID_ARG,
              "seq_lens, idx, count, part_o and part_lse are required");
  BSA_REQUIRE(num_splits >= 1 && num_splits <= cfg->budget && num_splits <= 1024,
              BSA_ERR_INVALID_ARG, "num_splits %d must lie in [1, min(budget, 1024)]",
              num_splits);
  if (cfg->n_tail_pages > 0)
    BSA_REQUIRE(tail_k && tail_v && aligned16(tail_k) && aligned16(tail_v), BSA_ERR_INVALID_ARG,
                "n_tail_pages > 0 needs 16-byte aligned tail_k and tail_v");
  return BSA_OK;
}

int check_merge_args(const float* out, const uint32_t* counters) {
  BSA_REQUIRE(out, BSA_ERR_INVALID_ARG, "out is required");
  BSA_REQUIRE(counters, BSA_ERR_WORKSPACE, "the arrival counters are required");
  return BSA_OK;
}

// select_ws (token mode, optional): the selection's workspace; the scan then
// also fills its histograms, and the selection that follows is launched with
// hist_ready.
hipError_t launch_scan(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const void* q,
                       const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                       const float* key_center, const void* kproj, const float* proj,
                       const int32_t* seq_lens, float* scores, hipStream_t s,
                       void* select_ws = nullptr) {
  const _Float16* qh = static_cast<const _Float16*>(q);
  if (cfg->granularity == BSA_GRANULARITY_BLOCK)
    return bsa::launch_scan_block(g, cfg->n_tail_pages, cfg->softmax_scale,
                                  cfg->query_dtype == BSA_QUERY_NVFP4, qh, codes, scales,
                                  global_scale, key_center, seq_lens, scores, s);
  return bsa::launch_scan_token(g, cfg->softmax_scale, cfg->proj_rank,
                                cfg->proj_dtype == BSA_PROJ_FP8, qh, kproj, proj, seq_lens,
                                scores, static_cast<uint32_t*>(select_ws),
                                bsa::token_unit_words(g), cfg->budget, s);
}

hipError_t launch_select(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const float* scores,
                         const int32_t* seq_lens, void* workspace, int32_t* idx, int32_t* count,
                         hipStream_t s, bool hist_ready = false) {
  if (cfg->granularity == BSA_GRANULARITY_BLOCK)
    return bsa::launch_select_block(g, cfg->budget, cfg->n_tail_pages, scores, seq_lens, idx,
                                    count, s);
  return bsa::launch_select_token(g, cfg->budget, scores, seq_lens, workspace, idx, count, s,
                                  hist_ready, cfg->top_p);
}

// The scan and the selection. Token mode: the scan fills the selection's
// first-digit histograms as it stores the scores, so the selection skips that
// pass.
hipError_t score_and_select(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const void* q,
                            const uint8_t* codes, const uint8_t* scales,
                            const float* global_scale, const float* key_center,
                            const void* kproj, const float* proj, const int32_t* seq_lens,
                            float* scores, void* workspace, int32_t* idx, int32_t* count,
                            hipStream_t s) {
  // (the one-group token select reads no histogram)
  const bool tok = cfg->granularity == BSA_GRANULARITY_TOKEN &&
                   !bsa::token_select_one_group(g, cfg->budget, cfg->top_p);
  hipError_t e = launch_scan(g, cfg, q, codes, scales, global_scale, key_center, kproj, proj,
                             seq_lens, scores, s, tok ? workspace : nullptr);
  if (e == hipSuccess) e = launch_select(g, cfg, scores, seq_lens, workspace, idx, count, s, tok);
  return e;
}

// The whole step: block mode (budget <= kFusedSelectMax) as the scan and the
// attention launch with the selection in its prologue; otherwise the scan, the
// selection and the attention.
hipError_t decode_step_launches(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, const void* q,
                                const uint8_t* codes, const uint8_t* scales,
                                const float* global_scale, const float* key_center,
                                const void* kproj, const float* proj, const void* k,
                                const void* v, const int32_t* seq_lens, const uint16_t* tail_k,
                                const uint16_t* tail_v, int32_t num_splits, float* scores,
                                void* workspace, int32_t* idx, int32_t* count, float* part_o,
                                float* part_lse, uint32_t* counters, float* out, float* out_lse,
                                hipStream_t s) {
  hipError_t e;
  if (cfg->granularity == BSA_GRANULARITY_BLOCK && cfg->budget <= bsa::kFusedSelectMax) {
    e = launch_scan(g, cfg, q, codes, scales, global_scale, key_center, kproj, proj, seq_lens,
                    scores, s);
    if (e == hipSuccess)
      e = attend_and_merge(g, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                           part_o, part_lse, counters, out, out_lse, s, scores);
  } else {
    e = score_and_select(g, cfg, q, codes, scales, global_scale, key_center, kproj, proj,
                         seq_lens, scores, workspace, idx, count, s);
    if (e == hipSuccess)
      e = attend_and_merge(g, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                           part_o, part_lse, counters, out, out_lse, s);
  }
  return e;
}

// --- the allocation-free step's scratch --------------------------------------
// One array per GPU, in device memory the library owns for the life of the
// process: the step's intermediates (scores, selection, split partials, merge
// counters, token selection workspace) for callers that cannot allocate. Host
// code never uses the array's name as an address: each device's address comes
// from hipGetSymbolAddress on the first call there.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  BSA_REQUIRE(dev >= 0 && dev < kMaxScratchDevices, BSA_ERR_UNSUPPORTED,
              "device %d: the scratch covers devices 0..%d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (es != hipSuccess || !p)
      return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(es));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

// Byte offsets of the step's buffers in the scratch (256-byte aligned); the
// arrival counters and the workspace are adjacent, so one fill clears both.
struct ScratchPlan {
  size_t counters, workspace, workspace_bytes, scores, idx, count, part_o, part_lse, total;
};

int plan_scratch(const bsa::UnitGeom& g, const bsa_select_cfg* cfg, int num_splits,
                 ScratchPlan* p) {
  const size_t U = size_t(g.B) * size_t(g.Hkv);
  const size_t rows = size_t(g.B) * size_t(g.Hq);
  const bool tok = cfg->granularity == BSA_GRANULARITY_TOKEN;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  p->counters = off;
  off = up(off + U * 4);
  p->workspace = off;
  p->workspace_bytes = tok ? bsa::token_select_workspace(g, cfg->budget, cfg->top_p) : 0;
  off = up(off + p->workspace_bytes);
  p->scores = off;
  off = up(off + U * size_t(tok ? g.Tmax : g.NBmax) * 4);
  p->idx = off;
  off = up(off + U * size_t(cfg->budget) * 4);
  p->count = off;
  off = up(off + U * 4);
  p->part_o = off;
  off = up(off + rows * size_t(num_splits) * bsa::kHeadDim * 4);
  p->part_lse = off;
  off = up(off + rows * size_t(num_splits) * 4);
  p->total = off;
  BSA_REQUIRE(off <= kScratchBytes, BSA_ERR_WORKSPACE,
              "this step needs %zu bytes of intermediates; the allocation-free step's scratch "
              "holds %zu",
              off, kScratchBytes);
  return BSA_OK;
}

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

#define BSA_CHECK(expr)   \
  do {                    \
    const int rc_ = (expr); \
    if (rc_) return rc_;  \
  } while (0)

}  // namespace

extern "C" {

int bsa_pack_kv_cache(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* k,
                      const float* key_center, const float* global_scale, const float* proj,
                      int32_t block_begin, int32_t block_end, uint8_t* codes, uint8_t* scales,
                      void* kproj, void* stream) {
  try {
    bsa::UnitGeom g;
    int rc = check_common(layout, cfg, &g);
    if (rc) return rc;
    BSA_CHECK(reject_cluster(cfg, "bsa_pack_kv_cache"));
    BSA_REQUIRE(k && aligned16(k), BSA_ERR_INVALID_ARG, "k must be a 16-byte aligned device pointer");
    BSA_REQUIRE(0 <= block_begin && block_begin <= block_end && block_end <= g.NBmax,
                BSA_ERR_INVALID_ARG, "block range [%d, %d) outside [0, %d]", block_begin,
                block_end, g.NBmax);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (cfg->granularity == BSA_GRANULARITY_BLOCK) {
      BSA_REQUIRE(global_scale && codes && scales && aligned16(codes), BSA_ERR_INVALID_ARG,
                  "block mode needs global_scale, codes (16-byte aligned) and scales");
      return hip_status(bsa::launch_pack_block(g, k, key_center, global_scale, block_begin,
                                               block_end, codes, scales, s),
                        "pack_nvfp4");
    }
    BSA_REQUIRE(proj && kproj, BSA_ERR_INVALID_ARG, "token mode needs proj and kproj");
    return hip_status(bsa::launch_pack_proj(g, k, proj, cfg->proj_rank,
                                            cfg->proj_dtype == BSA_PROJ_FP8, block_begin,
                                            block_end, kproj, s),
                      "pack_proj");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

size_t bsa_value_store_size(const bsa_kv_layout* layout) {
  if (!layout || layout->batch < 1 || layout->num_kv_heads < 1 || layout->max_tokens < 1)
    return 0;
  bsa::UnitGeom g;
  g.B = layout->batch;
  g.Hkv = layout->num_kv_heads;
  g.Tmax = layout->max_tokens;
  return bsa::value_store_bytes(g);
}

int bsa_pack_values(const bsa_kv_layout* layout, const void* v, const float* value_scale,
                    int32_t block_begin, int32_t block_end, void* store, void* stream) {
  try {
    BSA_REQUIRE(layout, BSA_ERR_INVALID_ARG, "layout must not be NULL");
    // the layout checks of every call (the selection rule plays no part here)
    bsa_select_cfg cfg{};
    cfg.granularity = BSA_GRANULARITY_BLOCK;
    cfg.budget = 1;
    cfg.softmax_scale = 1.0f;
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, &cfg, &g));
    BSA_REQUIRE(v && aligned16(v) && value_scale && store && aligned16(store),
                BSA_ERR_INVALID_ARG,
                "v and store (16-byte aligned device pointers) and value_scale are required");
    BSA_REQUIRE(0 <= block_begin && block_begin <= block_end && block_end <= g.NBmax,
                BSA_ERR_INVALID_ARG, "block range [%d, %d) outside [0, %d]", block_begin,
                block_end, g.NBmax);
    (void)hipGetLastError();
    return hip_status(bsa::launch_pack_values(g, v, value_scale, block_begin, block_end, store,
                                              static_cast<hipStream_t>(stream)),
                      "pack_values");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_append_token(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* k_new,
                     const void* v_new, const int32_t* seq_lens, void* k, void* v,
                     const float* key_center, const float* global_scale, const float* proj,
                     uint8_t* codes, uint8_t* scales, void* kproj, uint16_t* tail_k,
                     uint16_t* tail_v, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_append_token"));
    BSA_REQUIRE(k_new && v_new && aligned16(k_new) && aligned16(v_new) && k && v && seq_lens,
                BSA_ERR_INVALID_ARG,
                "k_new, v_new (16-byte aligned), k, v and seq_lens are required");
    const bool block = cfg->granularity == BSA_GRANULARITY_BLOCK;
    if (block)
      BSA_REQUIRE(codes && scales && global_scale, BSA_ERR_INVALID_ARG,
                  "block mode needs codes, scales and global_scale");
    else
      BSA_REQUIRE(proj && kproj, BSA_ERR_INVALID_ARG, "token mode needs proj and kproj");
    if (block && cfg->n_tail_pages > 0)
      BSA_REQUIRE(tail_k && tail_v && aligned16(tail_k) && aligned16(tail_v), BSA_ERR_INVALID_ARG,
                  "n_tail_pages > 0 needs 16-byte aligned tail_k and tail_v");
    (void)hipGetLastError();
    return hip_status(
        bsa::launch_append(g, block ? cfg->n_tail_pages : 0, block ? 0 : cfg->proj_rank,
                           cfg->proj_dtype == BSA_PROJ_FP8, k_new, v_new, seq_lens, k, v,
                           block ? key_center : nullptr, block ? global_scale : nullptr,
                           block ? codes : nullptr, block ? scales : nullptr,
                           block ? nullptr : proj, block ? nullptr : kproj,
                           block ? tail_k : nullptr, block ? tail_v : nullptr,
                           static_cast<hipStream_t>(stream)),
        "append_token");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_score_scan(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                   const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                   const float* key_center, const void* kproj, const float* proj,
                   const int32_t* seq_lens, float* scores, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_score_scan"));
    BSA_CHECK(check_scan_args(cfg, q, codes, scales, global_scale, kproj, proj, seq_lens, scores));
    (void)hipGetLastError();
    return hip_status(launch_scan(g, cfg, q, codes, scales, global_scale, key_center, kproj, proj,
                                  seq_lens, scores, static_cast<hipStream_t>(stream)),
                      "score_scan");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

size_t bsa_workspace_size(const bsa_kv_layout* layout, const bsa_select_cfg* cfg) {
  bsa::UnitGeom g;
  if (check_common(layout, cfg, &g)) return 0;
  return cfg->granularity == BSA_GRANULARITY_TOKEN ? bsa::token_select_workspace(g, cfg->budget, cfg->top_p) : 0;
}

int bsa_select_topk(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const float* scores,
                    const int32_t* seq_lens, void* workspace, size_t workspace_bytes,
                    int32_t* idx, int32_t* count, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_select_topk"));
    BSA_CHECK(check_select_args(g, cfg, scores, seq_lens, workspace, workspace_bytes, idx, count));
    (void)hipGetLastError();
    return hip_status(launch_select(g, cfg, scores, seq_lens, workspace, idx, count,
                                    static_cast<hipStream_t>(stream)),
                      "select_topk");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_sparse_decode_attn(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                           const void* k, const void* v, const int32_t* seq_lens,
                           const int32_t* idx, const int32_t* count, const uint16_t* tail_k,
                           const uint16_t* tail_v, int32_t num_splits, float* part_o,
                           float* part_lse, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(check_attend_args(cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                                part_o, part_lse));
    (void)hipGetLastError();
    return hip_status(bsa::launch_attention(g, cfg->granularity, cfg->budget, cfg->n_tail_pages,
                                            cfg->softmax_scale, static_cast<const _Float16*>(q),
                                            k, v, seq_lens, idx, count, tail_k, tail_v,
                                            num_splits, part_o, part_lse, nullptr, nullptr,
                                            nullptr, nullptr, nullptr, nullptr,
                                            static_cast<hipStream_t>(stream)),
                      "sparse_decode_attn");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_combine(int32_t rows, int32_t num_splits, int32_t head_dim, const float* part_o,
                const float* part_lse, float* out, float* out_lse, void* stream) {
  try {
    BSA_REQUIRE(head_dim == bsa::kHeadDim, BSA_ERR_UNSUPPORTED, "head_dim %d: only 128", head_dim);
    BSA_REQUIRE(rows >= 0 && num_splits >= 1 && num_splits <= 1024, BSA_ERR_INVALID_ARG,
                "rows %d >= 0 and num_splits %d in [1, 1024] required", rows, num_splits);
    BSA_REQUIRE(rows == 0 || (part_o && part_lse && out), BSA_ERR_INVALID_ARG,
                "part_o, part_lse and out are required");
    (void)hipGetLastError();
    return hip_status(bsa::launch_combine(rows, num_splits, part_o, part_lse, out, out_lse,
                                          static_cast<hipStream_t>(stream)),
                      "combine");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

size_t bsa_counters_size(const bsa_kv_layout* layout) {
  if (!layout || layout->batch < 1 || layout->num_kv_heads < 1) return 0;
  const int64_t units = int64_t(layout->batch) * layout->num_kv_heads;
  if (units > 65535) return 0;  // no call accepts such a layout
  return sizeof(uint32_t) * size_t(units);
}

int bsa_score_select(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                     const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                     const float* key_center, const void* kproj, const float* proj,
                     const int32_t* seq_lens, float* scores, void* workspace,
                     size_t workspace_bytes, int32_t* idx, int32_t* count, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_score_select"));
    BSA_CHECK(check_scan_args(cfg, q, codes, scales, global_scale, kproj, proj, seq_lens, scores));
    BSA_CHECK(check_select_args(g, cfg, scores, seq_lens, workspace, workspace_bytes, idx, count));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(score_and_select(g, cfg, q, codes, scales, global_scale, key_center, kproj,
                                       proj, seq_lens, scores, workspace, idx, count, s),
                      "score_select");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_attend_combine(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                       const void* k, const void* v, const int32_t* seq_lens,
                       const int32_t* idx, const int32_t* count, const uint16_t* tail_k,
                       const uint16_t* tail_v, int32_t num_splits, float* part_o,
                       float* part_lse, uint32_t* counters, float* out, float* out_lse,
                       void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(check_attend_args(cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                                part_o, part_lse));
    BSA_CHECK(check_merge_args(out, counters));
    (void)hipGetLastError();
    return hip_status(attend_and_merge(g, cfg, q, k, v, seq_lens, const_cast<int32_t*>(idx),
                                       const_cast<int32_t*>(count), tail_k, tail_v, num_splits,
                                       part_o, part_lse, counters, out, out_lse,
                                       static_cast<hipStream_t>(stream)),
                      "attend_combine");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_select_attend_combine(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                              const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, const float* scores, void* workspace,
                              size_t workspace_bytes, const uint16_t* tail_k,
                              const uint16_t* tail_v, int32_t num_splits, int32_t* idx,
                              int32_t* count, float* part_o, float* part_lse,
                              uint32_t* counters, float* out, float* out_lse, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_select_attend_combine"));
    BSA_CHECK(check_select_args(g, cfg, scores, seq_lens, workspace, workspace_bytes, idx, count));
    BSA_CHECK(check_attend_args(cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                                part_o, part_lse));
    BSA_CHECK(check_merge_args(out, counters));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t e;
    if (cfg->granularity == BSA_GRANULARITY_BLOCK && cfg->budget <= bsa::kFusedSelectMax) {
      e = attend_and_merge(g, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                           part_o, part_lse, counters, out, out_lse, s, scores);
    } else {
      e = launch_select(g, cfg, scores, seq_lens, workspace, idx, count, s);
      if (e == hipSuccess)
        e = attend_and_merge(g, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                             part_o, part_lse, counters, out, out_lse, s);
    }
    return hip_status(e, "select_attend_combine");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_decode_step(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                    const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                    const float* key_center, const void* kproj, const float* proj,
                    const void* k, const void* v, const int32_t* seq_lens,
                    const uint16_t* tail_k, const uint16_t* tail_v, int32_t num_splits,
                    float* scores, void* workspace, size_t workspace_bytes, int32_t* idx,
                    int32_t* count, float* part_o, float* part_lse, uint32_t* counters,
                    float* out, float* out_lse, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_decode_step"));
    BSA_CHECK(check_scan_args(cfg, q, codes, scales, global_scale, kproj, proj, seq_lens, scores));
    BSA_CHECK(check_select_args(g, cfg, scores, seq_lens, workspace, workspace_bytes, idx, count));
    BSA_CHECK(check_attend_args(cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                                part_o, part_lse));
    BSA_CHECK(check_merge_args(out, counters));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return hip_status(decode_step_launches(g, cfg, q, codes, scales, global_scale, key_center,
                                           kproj, proj, k, v, seq_lens, tail_k, tail_v,
                                           num_splits, scores, workspace, idx, count, part_o,
                                           part_lse, counters, out, out_lse, s),
                      "decode_step");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_decode_step_noalloc(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                            const void* q, const uint8_t* codes, const uint8_t* scales,
                            const float* global_scale, const float* key_center,
                            const void* kproj, const float* proj, const void* k, const void* v,
                            const int32_t* seq_lens, const uint16_t* tail_k,
                            const uint16_t* tail_v, int32_t num_splits, float* out,
                            float* out_lse, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_common(layout, cfg, &g));
    BSA_CHECK(reject_cluster(cfg, "bsa_decode_step_noalloc"));
    BSA_REQUIRE(num_splits >= 1 && num_splits <= cfg->budget && num_splits <= 1024,
                BSA_ERR_INVALID_ARG, "num_splits %d must lie in [1, min(budget, 1024)]",
                num_splits);
    ScratchPlan plan;
    BSA_CHECK(plan_scratch(g, cfg, num_splits, &plan));
    uint8_t* base = nullptr;
    BSA_CHECK(scratch_of_current_device(&base));
    float* scores = reinterpret_cast<float*>(base + plan.scores);
    int32_t* idx = reinterpret_cast<int32_t*>(base + plan.idx);
    int32_t* count = reinterpret_cast<int32_t*>(base + plan.count);
    float* part_o = reinterpret_cast<float*>(base + plan.part_o);
    float* part_lse = reinterpret_cast<float*>(base + plan.part_lse);
    uint32_t* counters = reinterpret_cast<uint32_t*>(base + plan.counters);
    void* workspace = plan.workspace_bytes ? base + plan.workspace : nullptr;
    BSA_CHECK(check_scan_args(cfg, q, codes, scales, global_scale, kproj, proj, seq_lens, scores));
    BSA_CHECK(check_select_args(g, cfg, scores, seq_lens, workspace, plan.workspace_bytes, idx,
                                count));
    BSA_CHECK(check_attend_args(cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                                part_o, part_lse));
    BSA_CHECK(check_merge_args(out, counters));
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    // the arrival counters and the selection's workspace start at zero: the
    // scratch keeps whatever the last call on this GPU left there
    hipLaunchKernelGGL(zero_words_kernel, dim3(256), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(base + plan.counters),
                       int64_t((plan.workspace + plan.workspace_bytes - plan.counters) / 4));
    hipError_t e = hipGetLastError();
    if (e == hipSuccess)
      e = decode_step_launches(g, cfg, q, codes, scales, global_scale, key_center, kproj, proj,
                               k, v, seq_lens, tail_k, tail_v, num_splits, scores, workspace,
                               idx, count, part_o, part_lse, counters, out, out_lse, s);
    return hip_status(e, "decode_step_noalloc");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

namespace {
int check_cluster_common(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                         bsa::UnitGeom* g) {
  BSA_CHECK(check_common(layout, cfg, g));
  BSA_REQUIRE(cfg->granularity == BSA_GRANULARITY_CLUSTER, BSA_ERR_INVALID_ARG,
              "the cluster calls need granularity BSA_GRANULARITY_CLUSTER");
  return BSA_OK;
}
}  // namespace

int bsa_build_cluster_index(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                            const void* k, const int32_t* assign, const int32_t* seq_lens,
                            float* centroids, int32_t* offsets, int32_t* members, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_cluster_common(layout, cfg, &g));
    BSA_REQUIRE(k && aligned16(k) && assign && seq_lens && centroids && aligned16(centroids) &&
                    offsets && members,
                BSA_ERR_INVALID_ARG,
                "k, centroids (16-byte aligned), assign, seq_lens, offsets and members are "
                "required");
    (void)hipGetLastError();
    return hip_status(bsa::launch_cluster_index(g, cfg->num_clusters, k, assign, seq_lens,
                                                centroids, offsets, members,
                                                static_cast<hipStream_t>(stream)),
                      "build_cluster_index");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_score_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg, const void* q,
                       const float* centroids, const int32_t* offsets, float* scores,
                       void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_cluster_common(layout, cfg, &g));
    BSA_REQUIRE(q && aligned16(q) && centroids && aligned16(centroids) && offsets && scores,
                BSA_ERR_INVALID_ARG,
                "q, centroids (16-byte aligned), offsets and scores are required");
    (void)hipGetLastError();
    return hip_status(bsa::launch_cluster_step(g, cfg->num_clusters, cfg->budget,
                                               cfg->softmax_scale, true, false,
                                               static_cast<const _Float16*>(q), centroids, offsets,
                                               nullptr, nullptr, scores, nullptr, nullptr,
                                               static_cast<hipStream_t>(stream)),
                      "score_clusters");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_select_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                        const float* scores, const int32_t* offsets, const int32_t* members,
                        int32_t* idx, int32_t* count, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_cluster_common(layout, cfg, &g));
    BSA_REQUIRE(scores && offsets && members && idx && count, BSA_ERR_INVALID_ARG,
                "scores, offsets, members, idx and count are required");
    (void)hipGetLastError();
    return hip_status(bsa::launch_cluster_step(g, cfg->num_clusters, cfg->budget,
                                               cfg->softmax_scale, false, true, nullptr, nullptr,
                                               offsets, members, scores, nullptr, idx, count,
                                               static_cast<hipStream_t>(stream)),
                      "select_clusters");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

int bsa_score_select_clusters(const bsa_kv_layout* layout, const bsa_select_cfg* cfg,
                              const void* q, const float* centroids, const int32_t* offsets,
                              const int32_t* members, float* scores, int32_t* idx,
                              int32_t* count, void* stream) {
  try {
    bsa::UnitGeom g;
    BSA_CHECK(check_cluster_common(layout, cfg, &g));
    BSA_REQUIRE(q && aligned16(q) && centroids && aligned16(centroids) && offsets && members &&
                    scores && idx && count,
                BSA_ERR_INVALID_ARG,
                "q, centroids (16-byte aligned), offsets, members, scores, idx and count are "
                "required");
    (void)hipGetLastError();
    return hip_status(bsa::launch_cluster_step(g, cfg->num_clusters, cfg->budget,
                                               cfg->softmax_scale, true, true,
                                               static_cast<const _Float16*>(q), centroids, offsets,
                                               members, nullptr, scores, idx, count,
                                               static_cast<hipStream_t>(stream)),
                      "score_select_clusters");
  } catch (...) {
    return fail(BSA_ERR_HIP, "unexpected exception");
  }
}

const char* bsa_last_error(void) { return g_err; }

const char* bsa_version(void) { return "bsa 0.1.0 (gfx950)"; }

}  // extern "C"
