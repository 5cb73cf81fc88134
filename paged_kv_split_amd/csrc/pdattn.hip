// C-ABI host layer: argument validation, the split planner and the launches.
// The operation, layouts and contracts are stated in include/pdattn.h.

#include "pdattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

constexpr uint32_t kPlanMagic = 0x70644131u;  // "pdA1"
// Target number of resident workgroups per compute unit that the adaptive
// planner sizes the split length for.
constexpr int kWorkgroupsPerCu = 4;
// Shortest adaptive split: one 16-token tile per wave of the workgroup.
constexpr int kMinSplitTokens = pdattn::kTileTokens * pdattn::kWaves;
// Upper bound on splits per sequence (workspace rows per (b, h)).
constexpr int kMaxSplits = 1024;

thread_local char g_last_error[512] = "";

pdattn_status fail(pdattn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
  int r = 0;
  while ((int64_t{1} << r) < x) ++r;
  return r;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }
bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

pdattn_status check_problem(const pdattn_problem* p) {
  if (p == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 0 || p->batch > 65535)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "batch %d outside [0, 65535]", p->batch);
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "head counts must be positive");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  const int g = p->num_q_heads / p->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(PDATTN_ERR_UNSUPPORTED, "group size %d not in {1, 2, 4, 8, 16}", g);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PDATTN_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", p->head_dim);
  if (!is_pow2(p->page_size) || p->page_size < 8 || p->page_size > 128)
    return fail(PDATTN_ERR_UNSUPPORTED, "page_size %d is not a power of two in [8, 128]", p->page_size);
  if (p->max_pages_per_seq < 0 || p->num_pages < 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "negative block table or pool size");
  if (p->kv_dtype != PDATTN_KV_BF16 && p->kv_dtype != PDATTN_KV_FP8_E4M3)
    return fail(PDATTN_ERR_UNSUPPORTED, "kv_dtype %d unknown", p->kv_dtype);
  if (!std::isfinite(p->scale)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "scale is not finite");
  return PDATTN_OK;
}

pdattn_status check_plan(const pdattn_plan_t* plan) {
  if (plan == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (plan->magic != kPlanMagic) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan was not produced by pdattn_plan");
  pdattn_status st = check_problem(&plan->problem);
  if (st != PDATTN_OK) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan holds an invalid problem: %s", g_last_error);
  const int64_t P = plan->problem.page_size;
  if (plan->split_tokens <= 0 || plan->split_tokens % pdattn::kTileTokens != 0 || plan->max_splits < 1 ||
      plan->max_splits > kMaxSplits || ceil_div(plan->split_tokens, P) + 1 > pdattn::kMaxPageList)
    return fail(PDATTN_ERR_PLAN_MISMATCH, "plan fields are inconsistent");
  const int64_t ws = plan->max_splits > 1 ? (int64_t)plan->problem.batch * plan->problem.num_q_heads *
                                                plan->max_splits * (plan->problem.head_dim + 2) * 4
                                          : 0;
  if ((int64_t)plan->workspace_bytes != ws) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan workspace size is inconsistent");
  return PDATTN_OK;
}

int64_t num_units(const pdattn_plan_t* plan) { return (int64_t)plan->problem.batch * plan->max_splits; }

// Workgroups of the partial kernel: Hkv per (sequence, split) unit, units
// padded to a multiple of the 8 XCDs.
int64_t partial_grid(const pdattn_plan_t* plan) {
  return 8 * (int64_t)plan->problem.num_kv_heads * ceil_div(num_units(plan), 8);
}

}  // namespace

extern "C" {

PDATTN_API const char* pdattn_status_string(pdattn_status status) {
  switch (status) {
    case PDATTN_OK: return "ok";
    case PDATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PDATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case PDATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case PDATTN_ERR_PLAN_MISMATCH: return "plan mismatch";
    case PDATTN_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

PDATTN_API const char* pdattn_last_error(void) { return g_last_error; }

PDATTN_API uint64_t pdattn_problem_size(void) { return sizeof(pdattn_problem); }
PDATTN_API uint64_t pdattn_plan_size(void) { return sizeof(pdattn_plan_t); }

PDATTN_API pdattn_status pdattn_plan(const pdattn_problem* problem, const int32_t* context_lens_host,
                                     int32_t num_cus, int32_t force_split_tokens, pdattn_plan_t* out) {
  g_last_error[0] = '\0';
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (out == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (problem->batch > 0 && context_lens_host == nullptr)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "context_lens_host is NULL");
  if (num_cus < 0 || force_split_tokens < 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_cus and force_split_tokens must be >= 0");

  const int64_t P = problem->page_size;
  const int64_t cap = (int64_t)problem->max_pages_per_seq * P;
  int64_t total = 0, max_len = 0;
  for (int b = 0; b < problem->batch; ++b) {
    const int64_t L = context_lens_host[b];
    if (L < 0 || L > cap)
      return fail(PDATTN_ERR_INVALID_ARGUMENT, "context_lens[%d] = %lld outside [0, max_pages_per_seq * page_size = %lld]",
                  b, (long long)L, (long long)cap);
    total += L;
    if (L > max_len) max_len = L;
  }
  if (max_len > 0 && problem->num_pages <= 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "empty page pool");

  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0)
      return fail(PDATTN_ERR_DEVICE, "cannot query the compute-unit count: %s", hipGetErrorString(e));
  }

  // Longest split whose block-table slice fits the LDS page list.
  const int64_t page_cap = ((pdattn::kMaxPageList - 1) * P) / pdattn::kTileTokens * pdattn::kTileTokens;
  int64_t split;
  if (force_split_tokens > 0) {
    split = round_up(force_split_tokens, pdattn::kTileTokens);
  } else if (total == 0) {
    split = pdattn::kTileTokens;
  } else {
    // Flash-decoding: cut the KV range only as far as needed to give every
    // compute unit kWorkgroupsPerCu work items of equal length.
    const int64_t slots = (int64_t)num_cus * kWorkgroupsPerCu;
    split = round_up(ceil_div(total * problem->num_kv_heads, slots), pdattn::kTileTokens);
    if (split < kMinSplitTokens) split = kMinSplitTokens;
    const int64_t whole = round_up(max_len, pdattn::kTileTokens);
    if (split > whole) split = whole;
  }
  if (split > page_cap) split = page_cap;
  if (split < pdattn::kTileTokens) split = pdattn::kTileTokens;
  if (max_len > 0 && ceil_div(max_len, split) > kMaxSplits) {
    split = round_up(ceil_div(max_len, kMaxSplits), pdattn::kTileTokens);
    if (split > page_cap)
      return fail(PDATTN_ERR_UNSUPPORTED, "context length %lld needs more than %d splits", (long long)max_len,
                  kMaxSplits);
  }
  const int64_t max_splits = max_len > 0 ? ceil_div(max_len, split) : 1;
  int64_t items = 0;
  for (int b = 0; b < problem->batch; ++b) {
    const int64_t L = context_lens_host[b];
    items += (L > 0 ? ceil_div(L, split) : 1) * problem->num_kv_heads;
  }

  pdattn_plan_t plan;
  std::memset(&plan, 0, sizeof plan);
  plan.problem = *problem;
  if (!(plan.problem.scale > 0.0f)) plan.problem.scale = 1.0f / std::sqrt((float)problem->head_dim);
  plan.split_tokens = (int32_t)split;
  plan.max_splits = (int32_t)max_splits;
  plan.num_cus = num_cus;
  plan.num_work_items = (int32_t)(items > INT32_MAX ? INT32_MAX : items);
  plan.max_context_len = max_len;
  plan.workspace_bytes = max_splits > 1 ? (uint64_t)problem->batch * problem->num_q_heads * max_splits *
                                              (problem->head_dim + 2) * 4
                                        : 0;
  plan.magic = kPlanMagic;
  if (partial_grid(&plan) > INT32_MAX) return fail(PDATTN_ERR_UNSUPPORTED, "grid too large");
  *out = plan;
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_decode(const pdattn_plan_t* plan, const void* q, const void* k_pages,
                                       const void* v_pages, const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       void* workspace, uint64_t workspace_bytes, float* out, float* lse,
                                       void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_plan(plan);
  if (st != PDATTN_OK) return st;
  const pdattn_problem& pr = plan->problem;
  if (pr.batch == 0) return PDATTN_OK;
  if (!q || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || (lse && !aligned(lse, 4)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "block_table, context_lens and lse must be 4-byte aligned");
  const bool fp8 = pr.kv_dtype == PDATTN_KV_FP8_E4M3;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "fp8 pools need 4-byte aligned k_scale and v_scale");
  if (!fp8 && (k_scale || v_scale))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "k_scale / v_scale must be NULL for bf16 pools");
  if (plan->workspace_bytes > 0) {
    if (!workspace || workspace_bytes < plan->workspace_bytes)
      return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes, got %llu at %p",
                  (unsigned long long)plan->workspace_bytes, (unsigned long long)workspace_bytes, workspace);
    if (!aligned(workspace, 16)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }

  pdattn::DecodeParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint8_t*>(k_pages);
  p.v = static_cast<const uint8_t*>(v_pages);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  const int64_t rows = (int64_t)pr.batch * pr.num_q_heads * plan->max_splits;
  p.part_acc = plan->workspace_bytes ? static_cast<float*>(workspace) : nullptr;
  p.part_ml = plan->workspace_bytes ? static_cast<float*>(workspace) + rows * pr.head_dim : nullptr;
  p.num_q_heads = pr.num_q_heads;
  p.num_kv_heads = pr.num_kv_heads;
  p.page_log2 = ilog2(pr.page_size);
  p.max_pages_per_seq = pr.max_pages_per_seq;
  p.num_pages = pr.num_pages;
  p.split_tokens = plan->split_tokens;
  p.max_splits = plan->max_splits;
  p.num_units = (int32_t)num_units(plan);
  p.qk_scale_log2 = pr.scale * 1.44269504088896340736f;

  hipError_t e = pdattn::launch_partial(p, pr.head_dim, pr.num_q_heads / pr.num_kv_heads, fp8,
                                        (uint32_t)partial_grid(plan), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "partial kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_reduce(const pdattn_plan_t* plan, const void* workspace,
                                       uint64_t workspace_bytes, const int32_t* context_lens, float* out,
                                       float* lse, void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_plan(plan);
  if (st != PDATTN_OK) return st;
  const pdattn_problem& pr = plan->problem;
  if (pr.batch == 0 || plan->max_splits == 1) return PDATTN_OK;
  if (!context_lens || !out) return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(context_lens, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "misaligned context_lens, out or lse");
  if (!workspace || workspace_bytes < plan->workspace_bytes)
    return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes", (unsigned long long)plan->workspace_bytes);
  if (!aligned(workspace, 16)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  pdattn::ReduceParams p;
  std::memset(&p, 0, sizeof p);
  const int64_t rows = (int64_t)pr.batch * pr.num_q_heads * plan->max_splits;
  p.part_acc = static_cast<const float*>(workspace);
  p.part_ml = static_cast<const float*>(workspace) + rows * pr.head_dim;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.num_q_heads = pr.num_q_heads;
  p.page_log2 = ilog2(pr.page_size);
  p.max_pages_per_seq = pr.max_pages_per_seq;
  p.split_tokens = plan->split_tokens;
  p.max_splits = plan->max_splits;
  hipError_t e = pdattn::launch_reduce(p, pr.head_dim, (uint32_t)((int64_t)pr.batch * pr.num_q_heads),
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "reduce kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

}  // extern "C"
