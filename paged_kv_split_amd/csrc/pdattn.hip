// C-ABI host layer: argument validation, the split planner and the launches.
// The operation, layouts and contracts are stated in include/pdattn.h.

#include "pdattn.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <vector>
#include <queue>
#include <limits>

#include "kernels.h"
#include "append.h"
#include "merge.h"
#include "prefill.h"
#include "tq4.h"

// The workspace of pdattn_decode_noalloc: one copy per device, held until the
// process ends. Host code never takes this name as an address: the device
// address comes from hipGetSymbolAddress (scratch_for_current_device).
static __device__ __align__(256) unsigned char scratch[PDATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr uint32_t kPlanMagic = 0x70644132u;  // "pdA2"
// Largest grid of the split reduce (its workgroups stride over the pairs).
constexpr int64_t kMaxMergeWorkgroups = 8192;

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
bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

// TQ4 problems are accepted only by the pdattn_tq4_* calls (allow_tq4).
pdattn_status check_problem(const pdattn_problem* p, bool allow_tq4 = false) {
  if (p == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "problem is NULL");
  if (p->batch < 0 || p->batch > 65535)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "batch %d outside [0, 65535]", p->batch);
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "head counts must be positive");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  const int g = p->num_q_heads / p->num_kv_heads;
  if (g > 16) return fail(PDATTN_ERR_UNSUPPORTED, "group size %d above 16", g);
  if (p->q_len < 0 || p->q_len > 16) return fail(PDATTN_ERR_INVALID_ARGUMENT, "q_len %d outside [0, 16]", p->q_len);
  const int cols = g * (p->q_len > 1 ? p->q_len : 1);
  if (cols > 16) return fail(PDATTN_ERR_UNSUPPORTED, "q_len * group size = %d above 16", cols);
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256)
    return fail(PDATTN_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", p->head_dim);
  if (!is_pow2(p->page_size) || p->page_size < 8 || p->page_size > 128)
    return fail(PDATTN_ERR_UNSUPPORTED, "page_size %d is not a power of two in [8, 128]", p->page_size);
  if (p->max_pages_per_seq < 0 || p->num_pages < 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "negative block table or pool size");
  if ((int64_t)p->max_pages_per_seq * p->page_size > INT32_MAX)
    return fail(PDATTN_ERR_UNSUPPORTED, "max_pages_per_seq * page_size exceeds 2^31 - 1 tokens");
  if (p->kv_dtype == PDATTN_KV_TQ4) {
    if (!allow_tq4) return fail(PDATTN_ERR_UNSUPPORTED, "TQ4 caches are served by the pdattn_tq4_* calls only");
  } else if (p->kv_dtype != PDATTN_KV_BF16 && p->kv_dtype != PDATTN_KV_FP8_E4M3 &&
             p->kv_dtype != PDATTN_KV_FP8_E4M3_INLINE) {
    return fail(PDATTN_ERR_UNSUPPORTED, "kv_dtype %d unknown", p->kv_dtype);
  }
  if (!std::isfinite(p->scale)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (p->kv_layout != PDATTN_LAYOUT_NHD && p->kv_layout != PDATTN_LAYOUT_HND)
    return fail(PDATTN_ERR_UNSUPPORTED, "kv_layout %d unknown", p->kv_layout);
  return PDATTN_OK;
}

int qlen_of(const pdattn_problem& p) { return p.q_len > 1 ? p.q_len : 1; }
// 0 bf16, 1 fp8 with separate scale arrays, 2 fp8 with inline scales
int kind_of(const pdattn_problem& p) {
  return p.kv_dtype == PDATTN_KV_FP8_E4M3_INLINE ? pdattn::kKindFp8Inline
                                                 : p.kv_dtype == PDATTN_KV_FP8_E4M3 ? pdattn::kKindFp8 : pdattn::kKindBf16;
}
// The decode instantiation of a problem: inline scales in head-major pools
// take the raw-row loads (a tile's rows are one contiguous block).
int decode_kind(const pdattn_problem& p) {
  const int k = kind_of(p);
  return k == pdattn::kKindFp8Inline && p.kv_layout == PDATTN_LAYOUT_HND ? pdattn::kKindFp8InlineRows : k;
}
// The scale arguments a dtype takes: both for fp8 with separate scales,
// none otherwise.
pdattn_status check_scales(const pdattn_problem& p, const float* k_scale, const float* v_scale) {
  if (kind_of(p) == pdattn::kKindFp8) {
    if (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4))
      return fail(PDATTN_ERR_INVALID_ARGUMENT, "fp8 pools need 4-byte aligned k_scale and v_scale");
  } else if (k_scale || v_scale) {
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "k_scale / v_scale must be NULL for %s pools",
                kind_of(p) == pdattn::kKindBf16 ? "bf16" : "inline-scale fp8");
  }
  return PDATTN_OK;
}
int heads_per_kv(const pdattn_problem& p) { return p.num_q_heads / p.num_kv_heads; }
// Valid columns: the (query row, head) pairs of one kv head; a kernel
// instantiation has the next power of two (the rest are padding).
int cols_of(const pdattn_problem& p) { return heads_per_kv(p) * qlen_of(p); }
int group_of(const pdattn_problem& p) {
  int c = 1;
  while (c < cols_of(p)) c <<= 1;
  return c;
}
bool pow2_heads(const pdattn_problem& p) { return is_pow2(heads_per_kv(p)); }

// Row strides of the pools: row index = page * P * Hkv + slot * slot_stride
// + kvh * head_stride.
int slot_stride_of(const pdattn_problem& p) { return p.kv_layout == PDATTN_LAYOUT_HND ? 1 : p.num_kv_heads; }
int head_stride_of(const pdattn_problem& p) { return p.kv_layout == PDATTN_LAYOUT_HND ? p.page_size : 1; }

bool balanced(int32_t flags) { return (flags & PDATTN_PLAN_BALANCED) != 0; }

// The streaming decode kernel serves bf16 pools and fp8 pools with separate
// scale arrays whose pages hold whole 16-token tiles, at batches whose tile
// prefix sums fit its workgroup's LDS, when every tile index it can meet
// (any device lengths the block table admits) fits in 31 bits; the general
// kernel (decode_kernels.hip) serves the rest.
bool use_stream(const pdattn_problem& p) {
  if (p.kv_dtype != PDATTN_KV_BF16 && p.kv_dtype != PDATTN_KV_FP8_E4M3) return false;
  if (p.page_size < pdattn::kTileTokens || p.batch > pdattn::kStreamMaxBatch) return false;
  const double cap_tiles = std::ceil((double)p.max_pages_per_seq * p.page_size / pdattn::kTileTokens);
  if ((double)p.batch * cap_tiles * p.num_kv_heads >= 2147483648.0) return false;
  // its output stores address the out array with 32-bit byte offsets
  if ((double)p.batch * qlen_of(p) * p.num_q_heads * p.head_dim * 4.0 >= 2147483648.0) return false;
  return pdattn::stream_built(p.head_dim, group_of(p), p.kv_dtype == PDATTN_KV_FP8_E4M3);
}
uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Default-mode workspace: 2 partial records per worker, then the tile
// prefix of the sequences (batch + 1 int64 words).
uint64_t records_bytes(const pdattn_problem& p, int64_t workers) {
  return (uint64_t)workers * 2 * pdattn::record_floats(p.head_dim, group_of(p)) * 4;
}

// Balanced-mode workspace: a 256-byte header (words 0..2: the initialisation
// stamp), the counters, the unit records, then (pairs longer than one unit)
// the pair-level records.
struct DynLayout {
  int64_t seg_max;     // units per pair at most
  int64_t units_max;   // batch * Hkv * seg_max
  uint64_t ctl_off, ctl_words;
  uint64_t rec_off, rec2_off, total;
};
DynLayout dyn_layout(const pdattn_problem& p, int64_t workers) {
  DynLayout d;
  const int64_t max_tiles = ceil_div((int64_t)p.max_pages_per_seq * p.page_size, pdattn::kTileTokens);
  d.seg_max = max_tiles > 0 ? ceil_div(max_tiles, pdattn::kUnitTiles) : 1;
  d.units_max = (int64_t)p.batch * p.num_kv_heads * d.seg_max;
  const uint64_t rec = (uint64_t)pdattn::record_floats(p.head_dim, group_of(p)) * 4;
  d.ctl_off = 256;
  d.ctl_words = 3 * (uint64_t)d.units_max + (uint64_t)p.batch * p.num_kv_heads;
  d.rec_off = d.ctl_off + round_up(d.ctl_words * 4, 256);
  d.rec2_off = d.rec_off + round_up(((uint64_t)d.units_max + 3 * (uint64_t)workers) * rec, 256);
  d.total = d.rec2_off + (d.seg_max > 1 ? (uint64_t)d.units_max * rec : 0);
  return d;
}

// Worker weights of a static plan's split (merge_ops.h), packed wa << 16 | wb.
int split_wa(const pdattn_plan_t* plan) { return (int)(plan->split_weights >> 16); }
int split_wb(const pdattn_plan_t* plan) { return (int)(plan->split_weights & 0xffffu); }
constexpr uint32_t kEqualWeights = (1u << 16) | 1u;
// fp8 pools: the CU serves its first resident workgroup before its second,
// and with half-size tiles the second one's waves alone do not keep the HBM
// busy once the first ones are done; the first half of the grid (each CU's
// first workgroup) takes 5 shares to the second half's 4 (measured on the
// FP8 KV step: decode 59.3-59.4 us against 61.1-61.4 with equal shares;
// bf16 steps gain nothing, their second workgroups alone still saturate).
constexpr uint32_t kFp8Weights = (5u << 16) | 4u;

// The streaming kernel for a plan with this many workers: it addresses its
// records with 32-bit buffer offsets (forced worker counts can exceed them).
bool use_stream_for(const pdattn_problem& p, int64_t workers) {
  return use_stream(p) && records_bytes(p, workers) < (1ull << 31);
}

uint64_t workspace_for(const pdattn_problem& p, int64_t workers, int32_t flags) {
  if (!balanced(flags)) return records_bytes(p, workers) + ((uint64_t)p.batch + 1) * 8;
  return dyn_layout(p, workers).total;
}

// Waves per workgroup of the kernel a plan launches.
int waves_of(const pdattn_problem& p, int32_t flags) {
  return !balanced(flags) && use_stream(p) ? pdattn::kStreamWaves : pdattn::kWaves;
}

// Occupancy-cache kinds: the general kernel's kinds (kernels.h) and the
// streaming kernel's two.
constexpr int kKindStreamBf16 = 4, kKindStreamFp8 = 5, kKindSlots = 6;
int engine_kind(const pdattn_problem& p) {
  if (!use_stream(p)) return decode_kind(p);
  return p.kv_dtype == PDATTN_KV_FP8_E4M3 ? kKindStreamFp8 : kKindStreamBf16;
}

// Resident workgroups per CU of one kernel instantiation on the current
// device, from the runtime's occupancy query (cached: the query costs
// milliseconds), 0 if it cannot be asked.
int wgs_per_cu_cached(int device, int head_dim, int group, int kind, bool dyn) {
  static std::atomic<int> cache[64][3][5][kKindSlots][2];
  if (device < 0 || device >= 64) return 0;
  const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : group == 8 ? 3 : 4;
  std::atomic<int>& slot = cache[device][head_dim == 256 ? 2 : head_dim == 128 ? 1 : 0][gi][kind][dyn];
  int v = slot.load(std::memory_order_relaxed);
  if (v > 0) return v;
  v = dyn                        ? pdattn::dynamic_wgs_per_cu(head_dim, group, kind != pdattn::kKindBf16)
      : kind == kKindStreamBf16 ? pdattn::stream_wgs_per_cu(head_dim, group, false)
      : kind == kKindStreamFp8  ? pdattn::stream_wgs_per_cu(head_dim, group, true)
                                : pdattn::decode_wgs_per_cu(head_dim, group, kind);
  if (v > 0) slot.store(v, std::memory_order_relaxed);
  return v;
}

pdattn_status check_plan(const pdattn_plan_t* plan) {
  if (plan == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (plan->magic != kPlanMagic) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan was not produced by pdattn_plan");
  pdattn_status st = check_problem(&plan->problem);
  if (st != PDATTN_OK) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan holds an invalid problem: %s", g_last_error);
  if (plan->num_workers < 1 || plan->num_workgroups < 1 ||
      (int64_t)plan->num_workgroups * waves_of(plan->problem, plan->flags) < plan->num_workers ||
      (plan->flags & ~PDATTN_PLAN_BALANCED) != 0 ||
      (balanced(plan->flags) &&
       (qlen_of(plan->problem) > 1 || plan->problem.head_dim == 256 || !pow2_heads(plan->problem))) ||
      plan->workspace_bytes != workspace_for(plan->problem, plan->num_workers, plan->flags) ||
      split_wa(plan) < 1 || split_wa(plan) > 16 || split_wb(plan) < 1 || split_wb(plan) > 16 ||
      (plan->split_weights != kEqualWeights &&
       (balanced(plan->flags) || !use_stream_for(plan->problem, plan->num_workers))))
    return fail(PDATTN_ERR_PLAN_MISMATCH, "plan fields are inconsistent");
  return PDATTN_OK;
}

// Pointer, alignment and scale checks shared by the decode entry points.
pdattn_status check_decode_args(const pdattn_plan_t* plan, const void* q, const void* k_pages, const void* v_pages,
                                const float* k_scale, const float* v_scale, const int32_t* block_table,
                                const int32_t* context_lens, const float* out, const float* lse) {
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
  return check_scales(pr, k_scale, v_scale);
}

// The default-mode decode launch on a checked workspace: records at its
// start, then the descriptors.
pdattn_status launch_static_decode(const pdattn_plan_t* plan, const void* q, const void* k_pages, const void* v_pages,
                                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                                   const int32_t* context_lens, void* workspace, float* out, float* lse,
                                   void* stream) {
  const pdattn_problem& pr = plan->problem;
  const bool fp8 = kind_of(pr) != pdattn::kKindBf16;
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
  p.rec = static_cast<float*>(workspace);
  p.pre = reinterpret_cast<int64_t*>(static_cast<unsigned char*>(workspace) + records_bytes(pr, plan->num_workers));
  p.batch = pr.batch;
  p.num_q_heads = pr.num_q_heads;
  p.num_kv_heads = pr.num_kv_heads;
  p.page_log2 = ilog2(pr.page_size);
  p.max_pages_per_seq = pr.max_pages_per_seq;
  p.num_pages = pr.num_pages;
  p.num_workers = plan->num_workers;
  p.split_wa = split_wa(plan);
  p.split_wb = split_wb(plan);
  p.q_len = qlen_of(pr);
  p.heads_per_kv = heads_per_kv(pr);
  p.num_cols = cols_of(pr);
  p.slot_stride = slot_stride_of(pr);
  p.head_stride = head_stride_of(pr);
  p.qk_scale_log2 = pr.scale * 1.44269504088896340736f;

  hipError_t e = use_stream_for(pr, plan->num_workers) ? pdattn::launch_decode_stream(p, pr.head_dim, group_of(pr), fp8,
                                                                (uint32_t)plan->num_workgroups,
                                                                static_cast<hipStream_t>(stream))
                                : pdattn::launch_decode(p, pr.head_dim, group_of(pr), decode_kind(pr),
                                                        (uint32_t)plan->num_workgroups, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "decode kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

// The default-mode reduce launch on a checked workspace.
pdattn_status launch_static_reduce(const pdattn_plan_t* plan, const void* workspace, float* out, float* lse,
                                   void* stream) {
  const pdattn_problem& pr = plan->problem;
  pdattn::MergeParams p;
  std::memset(&p, 0, sizeof p);
  p.rec = static_cast<const float*>(workspace);
  p.pre = reinterpret_cast<const int64_t*>(static_cast<const unsigned char*>(workspace) +
                                           records_bytes(pr, plan->num_workers));
  p.out = out;
  p.lse = lse;
  p.batch = pr.batch;
  p.num_kv_heads = pr.num_kv_heads;
  p.num_q_heads = pr.num_q_heads;
  p.num_workers = plan->num_workers;
  p.split_wa = split_wa(plan);
  p.split_wb = split_wb(plan);
  p.q_len = qlen_of(pr);
  p.heads_per_kv = heads_per_kv(pr);
  p.num_cols = cols_of(pr);
  // pieces of the longest pair under the host lengths: its tiles span at
  // most floor((nt - 1) NW / T) + 2 worker ranges
  const int64_t nt_max = ceil_div(plan->max_context_len, (int64_t)pdattn::kTileTokens);
  // (the lightest worker holds total_tiles * min(wa, wb) / W of them, W the
  // weight of all workers)
  const int64_t wa = split_wa(plan), wb = split_wb(plan);
  const int64_t wsum = wa * (plan->num_workers / 2) + wb * (plan->num_workers - plan->num_workers / 2);
  const int64_t max_pieces = plan->total_tiles > 0 && nt_max > 0
                                 ? (nt_max - 1) * wsum / (plan->total_tiles * std::min(wa, wb)) + 2
                                 : 1;
  const int waves = pdattn::merge_waves(pr.head_dim, group_of(pr), max_pieces);
  hipError_t e = pdattn::launch_merge(p, pr.head_dim, group_of(pr), waves, (uint32_t)kMaxMergeWorkgroups,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "reduce kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

// Device address of `scratch` on the current device, resolved once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pdattn_status scratch_for_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PDATTN_ERR_DEVICE, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || addr == nullptr)
      return fail(PDATTN_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = addr;
  }
  *ptr = g_scratch_ptr[dev];
  return PDATTN_OK;
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
PDATTN_API uint64_t pdattn_tq4_plan_size(void) { return sizeof(pdattn_tq4_plan_t); }

PDATTN_API pdattn_status pdattn_plan(const pdattn_problem* problem, const int32_t* context_lens_host,
                                     int32_t num_cus, int32_t force_workers, int32_t flags, pdattn_plan_t* out) {
  g_last_error[0] = '\0';
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (out == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (problem->batch > 0 && context_lens_host == nullptr)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "context_lens_host is NULL");
  if (num_cus < 0 || force_workers < 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_cus and force_workers must be >= 0");
  if ((flags & ~PDATTN_PLAN_BALANCED) != 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "unknown plan flags %d", flags);
  const bool dyn = balanced(flags);
  if (dyn && qlen_of(*problem) > 1)
    return fail(PDATTN_ERR_UNSUPPORTED, "multi-query decode (q_len > 1) needs a static plan");
  if (dyn && problem->head_dim == 256) return fail(PDATTN_ERR_UNSUPPORTED, "head_dim 256 needs a static plan");
  if (dyn && !pow2_heads(*problem))
    return fail(PDATTN_ERR_UNSUPPORTED, "a group size that is not a power of two needs a static plan");
  if (dyn && problem->kv_dtype == PDATTN_KV_FP8_E4M3_INLINE)
    return fail(PDATTN_ERR_UNSUPPORTED, "inline-scale fp8 pools need a static plan");

  const int64_t cap = (int64_t)problem->max_pages_per_seq * problem->page_size;
  int64_t tiles = 0, max_len = 0;
  for (int b = 0; b < problem->batch; ++b) {
    const int64_t L = context_lens_host[b];
    if (L < 0 || L > cap)
      return fail(PDATTN_ERR_INVALID_ARGUMENT,
                  "context_lens[%d] = %lld outside [0, max_pages_per_seq * page_size = %lld]", b, (long long)L,
                  (long long)cap);
    tiles += ceil_div(L, pdattn::kTileTokens);
    if (L > max_len) max_len = L;
  }
  tiles *= problem->num_kv_heads;
  if (max_len > 0 && problem->num_pages <= 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "empty page pool");

  const int kind = kind_of(*problem);
  const bool fp8 = kind != pdattn::kKindBf16;
  // resident workgroups per CU: the runtime's occupancy figure for this
  // instantiation when the device is asked, else a conservative estimate
  int per_cu = 0;
  if (num_cus == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0)
      return fail(PDATTN_ERR_DEVICE, "cannot query the compute-unit count: %s", hipGetErrorString(e));
    per_cu = wgs_per_cu_cached(dev, problem->head_dim, group_of(*problem), dyn ? kind : engine_kind(*problem), dyn);
  }
  if (per_cu <= 0) per_cu = pdattn::decode_wgs_per_cu_estimate(problem->head_dim, group_of(*problem), fp8, dyn);

  // Flash-decoding: as many worker waves as the device holds at once (the
  // grid is persistent: no workgroup waits for a free slot), each with at
  // least kMinTilesPerWorker tiles, so a small step is not spread thinner.
  const int64_t capacity = (int64_t)num_cus * per_cu * waves_of(*problem, flags);
  int64_t workers;
  if (force_workers > 0) {
    workers = force_workers;
  } else {
    workers = tiles / pdattn::kMinTilesPerWorker;
    if (workers > capacity) workers = capacity;
    if (workers < 1) workers = 1;
  }
  if (workers > (int64_t)1 << 20) return fail(PDATTN_ERR_UNSUPPORTED, "more than 2^20 workers");
  // the kernels form worker * total_tiles in 64-bit arithmetic, for any
  // device lengths the block table admits
  const double worst = (double)problem->batch * (double)ceil_div(cap, pdattn::kTileTokens) *
                       (double)problem->num_kv_heads * (double)(workers + 1);
  if (worst >= 4.0e18) return fail(PDATTN_ERR_UNSUPPORTED, "problem too large for 64-bit tile arithmetic");
  if (dyn && dyn_layout(*problem, workers).units_max > ((int64_t)1 << 24))
    return fail(PDATTN_ERR_UNSUPPORTED, "batch * num_kv_heads * units per pair exceeds 2^24");
  // the balanced kernel keeps tile positions in 31 bits, for any device
  // lengths the block table admits
  if (dyn && (double)problem->batch * problem->num_kv_heads * (double)ceil_div(cap, pdattn::kTileTokens) >= 2147483648.0)
    return fail(PDATTN_ERR_UNSUPPORTED, "batch * num_kv_heads * tiles per block-table row reaches 2^31");

  pdattn_plan_t plan;
  std::memset(&plan, 0, sizeof plan);
  plan.problem = *problem;
  if (!(plan.problem.scale > 0.0f)) plan.problem.scale = 1.0f / std::sqrt((float)problem->head_dim);
  plan.num_cus = num_cus;
  plan.num_workers = (int32_t)workers;
  plan.num_workgroups = (int32_t)ceil_div(workers, waves_of(*problem, flags));
  plan.total_tiles = tiles;
  plan.max_context_len = max_len;
  plan.flags = flags;
  plan.workspace_bytes = workspace_for(*problem, workers, flags);
  // fp8 pools on the streaming kernel at its full grid (two workgroups per
  // CU, blocks g and g + num_cus on CU g): the weighted split
  plan.split_weights = !dyn && force_workers == 0 && problem->kv_dtype == PDATTN_KV_FP8_E4M3 && per_cu == 2 &&
                               workers == capacity && use_stream_for(*problem, workers)
                           ? kFp8Weights
                           : kEqualWeights;
  plan.magic = kPlanMagic;
  *out = plan;
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_decode(const pdattn_plan_t* plan, const void* q, const void* k_pages,
                                       const void* v_pages, const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       void* workspace, uint64_t workspace_bytes, float* out, float* lse,
                                       void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_decode_args(plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, out, lse);
  if (st != PDATTN_OK) return st;
  const pdattn_problem& pr = plan->problem;
  if (pr.batch == 0) return PDATTN_OK;
  const bool fp8 = kind_of(pr) != pdattn::kKindBf16;
  if (!workspace || workspace_bytes < plan->workspace_bytes)
    return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes, got %llu at %p",
                (unsigned long long)plan->workspace_bytes, (unsigned long long)workspace_bytes, workspace);
  if (!aligned(workspace, 16)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  if (balanced(plan->flags)) {
    const DynLayout d = dyn_layout(pr, plan->num_workers);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    pdattn::DynParams p;
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
    p.rec = reinterpret_cast<float*>(ws + d.rec_off);
    p.rec2 = d.seg_max > 1 ? reinterpret_cast<float*>(ws + d.rec2_off) : nullptr;
    p.ctl = reinterpret_cast<uint32_t*>(ws + d.ctl_off);
    p.ws_magic = reinterpret_cast<const uint32_t*>(ws);
    p.batch = pr.batch;
    p.num_q_heads = pr.num_q_heads;
    p.num_kv_heads = pr.num_kv_heads;
    p.page_log2 = ilog2(pr.page_size);
    p.max_pages_per_seq = pr.max_pages_per_seq;
    p.num_pages = pr.num_pages;
    p.num_workers = plan->num_workers;
    p.seg_max = (int32_t)d.seg_max;
    p.units_max = (int32_t)d.units_max;
    p.slot_stride = slot_stride_of(pr);
    p.head_stride = head_stride_of(pr);
    p.qk_scale_log2 = pr.scale * 1.44269504088896340736f;
    hipError_t e = pdattn::launch_dynamic(p, pr.head_dim, group_of(pr), fp8, (uint32_t)plan->num_workgroups,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "decode kernel launch: %s", hipGetErrorString(e));
    return PDATTN_OK;
  }

  return launch_static_decode(plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, workspace, out,
                              lse, stream);
}

PDATTN_API pdattn_status pdattn_reduce(const pdattn_plan_t* plan, const void* workspace,
                                       uint64_t workspace_bytes, float* out, float* lse, void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_plan(plan);
  if (st != PDATTN_OK) return st;
  const pdattn_problem& pr = plan->problem;
  if (pr.batch == 0) return PDATTN_OK;
  if (!out) return fail(PDATTN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!aligned(out, 16) || (lse && !aligned(lse, 4)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "misaligned out or lse");
  if (!workspace || workspace_bytes < plan->workspace_bytes)
    return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes", (unsigned long long)plan->workspace_bytes);
  if (!aligned(workspace, 16)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (balanced(plan->flags)) return PDATTN_OK;  // merged inside pdattn_decode
  return launch_static_reduce(plan, workspace, out, lse, stream);
}

PDATTN_API pdattn_status pdattn_decode_noalloc(const pdattn_plan_t* plan, const void* q, const void* k_pages,
                                               const void* v_pages, const float* k_scale, const float* v_scale,
                                               const int32_t* block_table, const int32_t* context_lens, float* out,
                                               float* lse, void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_decode_args(plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, out, lse);
  if (st != PDATTN_OK) return st;
  if (plan->problem.batch == 0) return PDATTN_OK;
  if (balanced(plan->flags))
    return fail(PDATTN_ERR_UNSUPPORTED, "pdattn_decode_noalloc takes default-mode plans (balanced plans need a "
                                        "prepared workspace)");
  if (plan->workspace_bytes > PDATTN_NOALLOC_SCRATCH_BYTES)
    return fail(PDATTN_ERR_WORKSPACE, "plan needs %llu bytes of scratch; the static scratch holds %llu",
                (unsigned long long)plan->workspace_bytes, (unsigned long long)PDATTN_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != PDATTN_OK) return st;
  // every descriptor and every record the reduce reads is written by this
  // decode, so the scratch needs no clearing between calls
  st = launch_static_decode(plan, q, k_pages, v_pages, k_scale, v_scale, block_table, context_lens, ws, out, lse,
                            stream);
  if (st != PDATTN_OK) return st;
  return launch_static_reduce(plan, ws, out, lse, stream);
}

PDATTN_API pdattn_status pdattn_workspace_init(const pdattn_plan_t* plan, void* workspace, uint64_t workspace_bytes,
                                               void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_plan(plan);
  if (st != PDATTN_OK) return st;
  if (!balanced(plan->flags)) return PDATTN_OK;
  if (!workspace || workspace_bytes < plan->workspace_bytes)
    return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes, got %llu at %p",
                (unsigned long long)plan->workspace_bytes, (unsigned long long)workspace_bytes, workspace);
  if (!aligned(workspace, 16)) return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  const DynLayout d = dyn_layout(plan->problem, plan->num_workers);
  // words 3 .. end of the counters are zeroed; words 0..2 receive the stamp
  uint32_t* w = static_cast<uint32_t*>(workspace);
  const uint64_t words = d.ctl_off / 4 + d.ctl_words - 3;
  hipError_t e = pdattn::launch_workspace_init(
      w + 3, words, w, (uint32_t)d.units_max, (uint32_t)((int64_t)plan->problem.batch * plan->problem.num_kv_heads),
      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "workspace init launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_kv_append(const pdattn_problem* problem, int32_t num_tokens, const void* k_new,
                                          const void* v_new, const int32_t* token_seq, const int32_t* token_pos,
                                          const int32_t* block_table, void* k_pages, void* v_pages, float* k_scale,
                                          float* v_scale, int32_t flags, void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (num_tokens < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_tokens %d is negative", num_tokens);
  if ((flags & ~PDATTN_APPEND_POW2_SCALES) != 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "unknown append flags %d", flags);
  const int kind = kind_of(*problem);
  const bool fp8 = kind != pdattn::kKindBf16;
  if (!fp8 && (flags & PDATTN_APPEND_POW2_SCALES))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "PDATTN_APPEND_POW2_SCALES applies to fp8 pools only");
  if ((int64_t)problem->num_kv_heads * problem->head_dim > (1 << 19))
    return fail(PDATTN_ERR_UNSUPPORTED, "num_kv_heads * head_dim above 2^19");
  // nothing can resolve without a block-table column and a page
  if (num_tokens == 0 || problem->batch == 0 || problem->max_pages_per_seq == 0 || problem->num_pages == 0)
    return PDATTN_OK;
  if (!k_new || !v_new || !token_seq || !token_pos || !block_table || !k_pages || !v_pages)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "k_new, v_new, k_pages and v_pages must be 16-byte aligned");
  if (!aligned(token_seq, 4) || !aligned(token_pos, 4) || !aligned(block_table, 4))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "token_seq, token_pos and block_table must be 4-byte aligned");
  st = check_scales(*problem, k_scale, v_scale);
  if (st != PDATTN_OK) return st;

  pdattn::AppendParams p;
  std::memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.token_seq = token_seq;
  p.token_pos = token_pos;
  p.block_table = block_table;
  p.k_pages = k_pages;
  p.v_pages = v_pages;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_tokens = num_tokens;
  p.batch = problem->batch;
  p.num_kv_heads = problem->num_kv_heads;
  p.page_log2 = ilog2(problem->page_size);
  p.max_pages_per_seq = problem->max_pages_per_seq;
  p.num_pages = problem->num_pages;
  p.pow2_scales = (flags & PDATTN_APPEND_POW2_SCALES) ? 1 : 0;
  p.inline_scales = kind == pdattn::kKindFp8Inline ? 1 : 0;
  p.slot_stride = slot_stride_of(*problem);
  p.head_stride = head_stride_of(*problem);
  // one wave per token, four tokens per workgroup; a larger append is
  // covered by a grid-stride loop
  const int64_t wgs = ceil_div((int64_t)num_tokens, pdattn::kWaves);
  const uint32_t grid = (uint32_t)(wgs < ((int64_t)1 << 20) ? wgs : ((int64_t)1 << 20));
  hipError_t e = pdattn::launch_kv_append(p, problem->head_dim, fp8, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "append kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_merge(int32_t num_partials, int64_t num_rows, int32_t head_dim,
                                      const float* partial_out, const float* partial_lse, float* out, float* lse,
                                      void* stream) {
  g_last_error[0] = '\0';
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PDATTN_ERR_UNSUPPORTED, "head_dim %d not in {64, 128, 256}", head_dim);
  if (num_partials < 1) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_partials %d < 1", num_partials);
  if (num_rows < 0 || num_rows > ((int64_t)1 << 31))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_rows %lld outside [0, 2^31]", (long long)num_rows);
  if (num_rows == 0) return PDATTN_OK;
  if (!partial_out || !partial_lse || !out) return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(partial_out, 16) || !aligned(out, 16) || !aligned(partial_lse, 4) || (lse && !aligned(lse, 4)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "partial_out and out must be 16-byte aligned, the lse arrays 4-byte");
  pdattn::MergeStatesParams p;
  p.partial_out = partial_out;
  p.partial_lse = partial_lse;
  p.out = out;
  p.lse = lse;
  p.num_rows = num_rows;
  p.num_partials = num_partials;
  hipError_t e = pdattn::launch_merge_states(p, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "merge kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_fp8_conversion_check(uint64_t* mismatches, void* stream) {
  g_last_error[0] = '\0';
  if (!mismatches || !aligned(mismatches, 8))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "mismatches must be an 8-byte aligned device pointer");
  hipError_t e = pdattn::launch_fp8_conversion_check(reinterpret_cast<unsigned long long*>(mismatches),
                                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "conversion check launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_prefill_rows_per_tile(const pdattn_problem* problem, int32_t* rows_per_tile) {
  g_last_error[0] = '\0';
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (!rows_per_tile) return fail(PDATTN_ERR_INVALID_ARGUMENT, "rows_per_tile is NULL");
  *rows_per_tile = pdattn::prefill_columns(problem->head_dim) / heads_per_kv(*problem);
  return PDATTN_OK;
}

namespace {

// Positions a query tile reads: query tile j (rows j*rows .. of a request
// with n new rows and L context positions) sees t < L - n + i + 1 for its
// row i when causal, all t < L otherwise; `reach` is its last row's limit
// and `open` its first row's (positions below it are visible to every row),
// both clamped to [0, L].
void tile_limits(int64_t L, int64_t n, int64_t j, int64_t rows, bool causal, int64_t& reach, int64_t& open) {
  const int64_t last = std::min<int64_t>((j + 1) * rows, n) - 1;
  reach = causal ? L - n + last + 1 : L;
  reach = reach < 0 ? 0 : (reach > L ? L : reach);
  open = causal ? L - n + j * rows + 1 : L;
  open = open < 0 ? 0 : (open > L ? L : open);
}

}  // namespace

PDATTN_API pdattn_status pdattn_prefill_tiles(const int32_t* qo_indptr, const int32_t* context_lens, int32_t batch,
                                              int32_t rows_per_tile, int32_t causal, int32_t flags,
                                              int32_t* tile_batch, int32_t* tile_index, int32_t capacity,
                                              int32_t* num_tiles) {
  g_last_error[0] = '\0';
  if (!num_tiles) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_tiles is NULL");
  *num_tiles = 0;
  if (batch < 0 || batch > 65535) return fail(PDATTN_ERR_INVALID_ARGUMENT, "batch %d outside [0, 65535]", batch);
  if (rows_per_tile <= 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "rows_per_tile %d must be positive", rows_per_tile);
  if ((flags & ~PDATTN_TILES_LONGEST_FIRST) != 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "unknown tile flags %d", flags);
  if (causal != 0 && causal != 1) return fail(PDATTN_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (batch > 0 && !qo_indptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "qo_indptr is NULL");
  const bool longest = (flags & PDATTN_TILES_LONGEST_FIRST) != 0;
  if (longest && batch > 0 && !context_lens)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "PDATTN_TILES_LONGEST_FIRST needs the host context lengths");
  int64_t count = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    if (qo_indptr[b] < 0 || n < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "qo_indptr must start at >= 0 and not decrease (request %d)", b);
    count += ceil_div(n, rows_per_tile);
  }
  if (count > INT32_MAX) return fail(PDATTN_ERR_UNSUPPORTED, "more than 2^31 - 1 query tiles");
  *num_tiles = (int32_t)count;
  if (!tile_batch || !tile_index) return PDATTN_OK;  // count only
  if (capacity < count)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "%lld tiles do not fit in capacity %d", (long long)count, capacity);
  // request by request, tile by tile (the order of the pages' example)
  int64_t t = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    for (int64_t j = 0; j < ceil_div(n, rows_per_tile); ++j, ++t) {
      tile_batch[t] = b;
      tile_index[t] = (int32_t)j;
    }
  }
  if (longest && count > 1) {
    // most positions read first (the rows' reach into the context); equal
    // reaches keep their order
    struct Item { int64_t reach; int32_t b, j; };
    std::vector<Item> items;
    try {
      items.resize((size_t)count);
    } catch (...) {
      return fail(PDATTN_ERR_INVALID_ARGUMENT, "out of host memory for %lld tiles", (long long)count);
    }
    for (int64_t i = 0; i < count; ++i) {
      const int b = tile_batch[i];
      const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
      int64_t reach, open;
      tile_limits(context_lens[b], n, tile_index[i], rows_per_tile, causal != 0, reach, open);
      items[i] = Item{reach, tile_batch[i], tile_index[i]};
    }
    std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) { return x.reach > y.reach; });
    for (int64_t i = 0; i < count; ++i) {
      tile_batch[i] = items[i].b;
      tile_index[i] = items[i].j;
    }
  }
  return PDATTN_OK;
}

namespace {

// Fewest kernel tiles (K/V tiles) of one part of a split tile, and most parts.
constexpr int64_t kMinPartSteps = 4;
constexpr int64_t kMaxParts = 16;
// Positions per unit of a part boundary (a multiple of every kernel tile).
constexpr int64_t kPartUnit = 64;

int prefill_pool(const pdattn_problem& p) {
  return p.kv_dtype == PDATTN_KV_FP8_E4M3_INLINE ? pdattn::kPrefillFp8Inline
         : p.kv_dtype == PDATTN_KV_FP8_E4M3      ? pdattn::kPrefillFp8
                                                 : pdattn::kPrefillBf16;
}

uint64_t prefill_workspace_bytes(const pdattn_problem& problem, int64_t num_slots) {
  const uint64_t records = (uint64_t)num_slots * (uint64_t)problem.num_kv_heads;
  const uint64_t ctr = (records * 4 + 255) / 256 * 256;
  return ctr + records * (uint64_t)pdattn::prefill_record_floats(problem.head_dim) * 4;
}

pdattn_status prefill_launch(const pdattn_problem* problem, int32_t causal, const void* q, const int32_t* qo_indptr,
                             const int32_t* tile_batch, const int32_t* tile_index, const int32_t* tile_kv,
                             int32_t num_tiles, int32_t num_slots, void* workspace, uint64_t workspace_bytes,
                             const void* k_pages, const void* v_pages, const float* k_scale, const float* v_scale,
                             const int32_t* block_table, const int32_t* context_lens, float* out, float* lse,
                             void* stream) {
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(PDATTN_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (num_tiles < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_tiles %d is negative", num_tiles);
  if ((int64_t)num_tiles * problem->num_kv_heads > INT32_MAX)
    return fail(PDATTN_ERR_UNSUPPORTED, "num_tiles * num_kv_heads exceeds 2^31 - 1");
  if (num_slots < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_slots %d is negative", num_slots);
  if (num_slots > 0) {
    if (!workspace) return fail(PDATTN_ERR_WORKSPACE, "%d slots need a workspace", num_slots);
    if (!aligned(workspace, 256))
      return fail(PDATTN_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    const uint64_t need = prefill_workspace_bytes(*problem, num_slots);
    if (workspace_bytes < need)
      return fail(PDATTN_ERR_WORKSPACE, "workspace of %llu bytes; %d slots need %llu",
                  (unsigned long long)workspace_bytes, num_slots, (unsigned long long)need);
  }
  if (num_tiles == 0 || problem->batch == 0) return PDATTN_OK;
  if (!q || !qo_indptr || !tile_batch || !tile_index || !k_pages || !v_pages || !block_table || !context_lens || !out)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (!aligned(qo_indptr, 4) || !aligned(tile_batch, 4) || !aligned(tile_index, 4) || !aligned(block_table, 4) ||
      !aligned(context_lens, 4) || (lse && !aligned(lse, 4)) || (tile_kv && !aligned(tile_kv, 16)))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "index arrays and lse must be 4-byte aligned, tile_kv 16-byte");
  st = check_scales(*problem, k_scale, v_scale);
  if (st != PDATTN_OK) return st;

  pdattn::PrefillParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.qo_indptr = qo_indptr;
  p.tile_batch = tile_batch;
  p.tile_index = tile_index;
  p.k = static_cast<const uint8_t*>(k_pages);
  p.v = static_cast<const uint8_t*>(v_pages);
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.batch = problem->batch;
  p.num_q_heads = problem->num_q_heads;
  p.num_kv_heads = problem->num_kv_heads;
  p.heads_per_kv = heads_per_kv(*problem);
  p.rows_per_tile = pdattn::prefill_columns(problem->head_dim) / p.heads_per_kv;
  p.page_log2 = ilog2(problem->page_size);
  p.max_pages_per_seq = problem->max_pages_per_seq;
  p.num_pages = problem->num_pages;
  p.slot_stride = slot_stride_of(*problem);
  p.head_stride = head_stride_of(*problem);
  p.causal = causal;
  const float scale = problem->scale > 0.0f ? problem->scale : 1.0f / std::sqrt((float)problem->head_dim);
  p.qk_scale_log2 = scale * 1.44269504088896340736f;
  p.tile_kv = tile_kv;
  if (num_slots > 0) {
    const uint64_t records = (uint64_t)num_slots * (uint64_t)problem->num_kv_heads;
    p.part_ctr = static_cast<uint32_t*>(workspace);
    p.part_rec = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + (records * 4 + 255) / 256 * 256);
    p.num_slots = num_slots;
  }
  const uint32_t grid = (uint32_t)((int64_t)num_tiles * problem->num_kv_heads);
  hipError_t e = pdattn::launch_prefill(p, problem->head_dim, prefill_pool(*problem), grid,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "prefill kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

}  // namespace

PDATTN_API pdattn_status pdattn_prefill(const pdattn_problem* problem, int32_t causal, const void* q,
                                        const int32_t* qo_indptr, const int32_t* tile_batch,
                                        const int32_t* tile_index, int32_t num_tiles, const void* k_pages,
                                        const void* v_pages, const float* k_scale, const float* v_scale,
                                        const int32_t* block_table, const int32_t* context_lens, float* out,
                                        float* lse, void* stream) {
  g_last_error[0] = '\0';
  return prefill_launch(problem, causal, q, qo_indptr, tile_batch, tile_index, nullptr, num_tiles, 0, nullptr, 0,
                        k_pages, v_pages, k_scale, v_scale, block_table, context_lens, out, lse, stream);
}

PDATTN_API pdattn_status pdattn_prefill_split_tiles(const pdattn_problem* problem, const int32_t* qo_indptr,
                                                    const int32_t* context_lens, int32_t causal, int32_t slots,
                                                    int32_t* tile_batch, int32_t* tile_index, int32_t* tile_kv,
                                                    int32_t capacity, int32_t* num_tiles, int32_t* num_slots,
                                                    uint64_t* workspace_bytes) {
  g_last_error[0] = '\0';
  if (!num_tiles || !num_slots || !workspace_bytes)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_tiles, num_slots and workspace_bytes must not be NULL");
  *num_tiles = 0;
  *num_slots = 0;
  *workspace_bytes = 0;
  pdattn_status st = check_problem(problem);
  if (st != PDATTN_OK) return st;
  if (causal != 0 && causal != 1) return fail(PDATTN_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (slots < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "slots %d is negative", slots);
  const int batch = problem->batch;
  if (batch > 0 && (!qo_indptr || !context_lens))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "qo_indptr and context_lens (host arrays) are required");
  if (slots == 0) {
    int dev = 0, num_cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0)
      return fail(PDATTN_ERR_DEVICE, "cannot query the compute-unit count: %s", hipGetErrorString(e));
    const int per_cu = pdattn::prefill_wgs_per_cu(problem->head_dim, prefill_pool(*problem));
    slots = num_cus * (per_cu > 0 ? per_cu : 1);
  }
  const int64_t H = problem->num_kv_heads;
  const int64_t rows = pdattn::prefill_columns(problem->head_dim) / heads_per_kv(*problem);
  const int64_t nt = pdattn::prefill_kv_tile(problem->head_dim);
  const int64_t min_units = ceil_div(kMinPartSteps * nt, kPartUnit);  // smallest part, in 64-position units

  struct Tile {
    int64_t reach, open, steps;  // positions read; positions below every row's limit; kernel tiles
    int32_t b, j;
  };
  struct Piece {
    int64_t cost;
    int32_t b, j, kv0, kv1, base, pq;
  };
  // Costs in quarter kernel tiles: 4 per tile read, 1 more per tile at or
  // past the first row's causal limit (the masked loop), 20 per workgroup
  // for its start and end (the dependent loads before the first tile, the
  // output stores), 12 more per part for its record, counter and merge.
  auto piece_cost = [&](const Tile& t, int64_t kv0, int64_t kv1, bool part) {
    const int64_t i0 = kv0 / nt, i1 = ceil_div(kv1, nt);
    const int64_t masked = std::max<int64_t>(0, i1 - std::max(i0, t.open / nt));
    return 4 * (i1 - i0) + masked + 20 + (part ? 12 : 0);
  };
  std::vector<Tile> tiles;
  int64_t max_steps = 0;
  try {
    for (int b = 0; b < batch; ++b) {
      const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
      if (qo_indptr[b] < 0 || n < 0)
        return fail(PDATTN_ERR_INVALID_ARGUMENT, "qo_indptr must start at >= 0 and not decrease (request %d)", b);
      const int64_t L = context_lens[b];
      if (L < 0 || L > (int64_t)problem->max_pages_per_seq * problem->page_size)
        return fail(PDATTN_ERR_INVALID_ARGUMENT, "context_lens[%d] = %lld outside the block table", b, (long long)L);
      for (int64_t j = 0; j < ceil_div(n, rows); ++j) {
        int64_t reach, open;
        tile_limits(L, n, j, rows, causal != 0, reach, open);
        tiles.push_back(Tile{reach, open, ceil_div(reach, nt), b, (int32_t)j});
        max_steps = std::max(max_steps, tiles.back().steps);
        if ((int64_t)tiles.size() > INT32_MAX) return fail(PDATTN_ERR_UNSUPPORTED, "more than 2^31 - 1 query tiles");
      }
    }
  } catch (const std::bad_alloc&) {
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "out of host memory for the tile map");
  }

  // The device starts the workgroups in grid order as slots free up (each
  // entry's kv heads one after another): a list schedule. A tile of more
  // than `cap` kernel tiles is cut into ceil(steps / cap) parts (at most
  // 16, each of at least kMinPartSteps tiles, at multiples of 64
  // positions, as even as those allow); entries are listed by cost, most
  // first. The planner simulates that schedule on `slots` slots for no cut
  // and for caps of k / 16 of the longest tile (k = 3 .. 15), and keeps
  // the cap that ends first (the earlier candidate on a tie).
  std::vector<Piece> pieces, trial;
  int64_t slot_count = 0, best = -1;
  auto cut = [&](int64_t cap, std::vector<Piece>& out, int64_t& nslots) {
    out.clear();
    nslots = 0;
    for (const Tile& t : tiles) {
      const int64_t units = ceil_div(t.reach, kPartUnit);
      const int64_t parts =
          t.steps > cap ? std::min<int64_t>({ceil_div(t.steps, cap), kMaxParts, units / min_units}) : 1;
      if (parts < 2) {
        out.push_back(Piece{piece_cost(t, 0, t.reach, false), t.b, t.j, 0, (int32_t)t.reach, -1, 1 << 16});
        continue;
      }
      for (int64_t q = 0; q < parts; ++q) {
        const int64_t kv0 = q * units / parts * kPartUnit;
        const int64_t kv1 = q + 1 == parts ? t.reach : (q + 1) * units / parts * kPartUnit;
        out.push_back(Piece{piece_cost(t, kv0, kv1, true), t.b, t.j, (int32_t)kv0, (int32_t)kv1,
                            (int32_t)nslots, (int32_t)(q | (parts << 16))});
      }
      nslots += parts;
    }
    std::stable_sort(out.begin(), out.end(), [](const Piece& x, const Piece& y) { return x.cost > y.cost; });
  };
  auto makespan = [&](const std::vector<Piece>& list) {
    std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> free_at;
    for (int64_t i = 0; i < std::min<int64_t>(slots, (int64_t)list.size() * H); ++i) free_at.push(0);
    int64_t end = 0;
    for (const Piece& it : list)
      for (int64_t h = 0; h < H; ++h) {
        const int64_t t = free_at.top() + it.cost;
        free_at.pop();
        free_at.push(t);
        end = std::max(end, t);
      }
    return end;
  };
  try {
    std::vector<int64_t> caps = {std::numeric_limits<int64_t>::max()};
    for (int64_t k = 15; k >= 3; --k) caps.push_back(std::max<int64_t>(kMinPartSteps, ceil_div(max_steps * k, 16)));
    for (int64_t cap : caps) {
      int64_t nslots = 0;
      cut(cap, trial, nslots);
      if ((int64_t)trial.size() * H > INT32_MAX || nslots > INT32_MAX) continue;
      const int64_t span = makespan(trial);
      if (best < 0 || span < best) {
        best = span;
        pieces.swap(trial);
        slot_count = nslots;
      }
    }
  } catch (const std::bad_alloc&) {
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "out of host memory for the tile map");
  }
  if (!tiles.empty() && best < 0) return fail(PDATTN_ERR_UNSUPPORTED, "tiles * num_kv_heads exceeds 2^31 - 1");
  *num_tiles = (int32_t)pieces.size();
  *num_slots = (int32_t)slot_count;
  *workspace_bytes = slot_count > 0 ? prefill_workspace_bytes(*problem, slot_count) : 0;
  if (!tile_batch || !tile_index || !tile_kv) return PDATTN_OK;  // sizes only
  if (capacity < (int64_t)pieces.size())
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "%zu entries do not fit in capacity %d", pieces.size(), capacity);
  for (size_t i = 0; i < pieces.size(); ++i) {
    tile_batch[i] = pieces[i].b;
    tile_index[i] = pieces[i].j;
    tile_kv[4 * i + 0] = pieces[i].kv0;
    tile_kv[4 * i + 1] = pieces[i].kv1;
    tile_kv[4 * i + 2] = pieces[i].base;
    tile_kv[4 * i + 3] = pieces[i].pq;
  }
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_prefill_split(const pdattn_problem* problem, int32_t causal, const void* q,
                                              const int32_t* qo_indptr, const int32_t* tile_batch,
                                              const int32_t* tile_index, const int32_t* tile_kv, int32_t num_tiles,
                                              int32_t num_slots, void* workspace, uint64_t workspace_bytes,
                                              const void* k_pages, const void* v_pages, const float* k_scale,
                                              const float* v_scale, const int32_t* block_table,
                                              const int32_t* context_lens, float* out, float* lse, void* stream) {
  g_last_error[0] = '\0';
  if (num_tiles > 0 && !tile_kv) return fail(PDATTN_ERR_INVALID_ARGUMENT, "tile_kv is NULL");
  return prefill_launch(problem, causal, q, qo_indptr, tile_batch, tile_index, tile_kv, num_tiles, num_slots,
                        workspace, workspace_bytes, k_pages, v_pages, k_scale, v_scale, block_table, context_lens,
                        out, lse, stream);
}

PDATTN_API uint64_t pdattn_stream_read_sink_words(int32_t num_cus) {
  return (uint64_t)(num_cus > 0 ? num_cus : 0) * 2 * 256;
}

PDATTN_API pdattn_status pdattn_stream_read(const void* buffer, uint64_t bytes, uint32_t* sink, int32_t num_cus,
                                            void* stream) {
  g_last_error[0] = '\0';
  if (!buffer || !sink || num_cus <= 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "buffer, sink and num_cus required");
  if (!aligned(buffer, 16) || !aligned(sink, 4) || bytes % 4096 != 0)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "buffer must be 16-byte aligned and a multiple of 4096 bytes");
  hipError_t e = pdattn::launch_stream_read(buffer, bytes, sink, (uint32_t)num_cus * 2, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "stream-read kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

}  // extern "C"

// ---- TQ4 compressed cache ----------------------------------------------------

namespace {

constexpr uint32_t kTq4PlanMagic = 0x70645434u;  // "pdT4"

double std_normal_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }
double std_normal_pdf(double z) { return std::isinf(z) ? 0.0 : std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI); }

// Lloyd-Max quantiser of N(0, 1): start at the quantiles (i + 1/2) / 16
// (found by bisection on the cdf), then alternate midpoint boundaries and
// cell means until no centroid moves by more than 1e-13.
void lloyd_max16(double (&c)[16], double (&b)[15]) {
  for (int i = 0; i < 16; ++i) {
    const double u = (i + 0.5) / 16.0;
    double lo = -12.0, hi = 12.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      (std_normal_cdf(mid) < u ? lo : hi) = mid;
    }
    c[i] = 0.5 * (lo + hi);
  }
  for (int it = 0; it < 100000; ++it) {
    for (int i = 0; i < 15; ++i) b[i] = 0.5 * (c[i] + c[i + 1]);
    double moved = 0.0;
    for (int i = 0; i < 16; ++i) {
      const double a = i == 0 ? -INFINITY : b[i - 1];
      const double z = i == 15 ? INFINITY : b[i];
      // cell mass as a difference of upper tails (accurate in both tails)
      const double mass = 0.5 * (std::erfc(a / std::sqrt(2.0)) - std::erfc(z / std::sqrt(2.0)));
      const double m = (std_normal_pdf(a) - std_normal_pdf(z)) / mass;
      moved = std::max(moved, std::fabs(m - c[i]));
      c[i] = m;
    }
    if (moved <= 1e-13) break;
  }
  for (int i = 0; i < 15; ++i) b[i] = 0.5 * (c[i] + c[i + 1]);
}

pdattn_status check_tq4_problem(const pdattn_problem* p) {
  pdattn_status st = check_problem(p, true);
  if (st != PDATTN_OK) return st;
  if (p->kv_dtype != PDATTN_KV_TQ4) return fail(PDATTN_ERR_INVALID_ARGUMENT, "kv_dtype must be PDATTN_KV_TQ4");
  if (p->kv_layout != PDATTN_LAYOUT_HND) return fail(PDATTN_ERR_UNSUPPORTED, "TQ4 caches are head-major (HND) only");
  if (qlen_of(*p) != 1) return fail(PDATTN_ERR_UNSUPPORTED, "TQ4 decode takes one query row per sequence");
  return PDATTN_OK;
}

uint64_t tq4_qseq_bytes(const pdattn_problem& p) {
  return round_up((uint64_t)p.batch * p.num_q_heads * p.head_dim * 2, 256);
}
// workspace: rotated q (fp16), then the work items' records
uint64_t tq4_workspace(const pdattn_problem& p, int32_t max_chunks) {
  return tq4_qseq_bytes(p) + (uint64_t)max_chunks * p.batch * p.num_kv_heads *
                                 (uint64_t)pdattn::tq4_record_floats(heads_per_kv(p), p.head_dim) * 4;
}

pdattn_status check_tq4_plan(const pdattn_tq4_plan_t* plan) {
  if (plan == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (plan->magic != kTq4PlanMagic) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan was not produced by pdattn_tq4_plan");
  pdattn_status st = check_tq4_problem(&plan->problem);
  if (st != PDATTN_OK) return fail(PDATTN_ERR_PLAN_MISMATCH, "plan holds an invalid problem: %s", g_last_error);
  if (plan->num_workgroups < 0 || plan->chunk_tiles < 1 || plan->max_chunks < 1 ||
      plan->workspace_bytes != tq4_workspace(plan->problem, plan->max_chunks))
    return fail(PDATTN_ERR_PLAN_MISMATCH, "plan fields are inconsistent");
  return PDATTN_OK;
}

}  // namespace

extern "C" {

PDATTN_API pdattn_status pdattn_tq4_codebook(int32_t head_dim, float* centroids, float* boundaries) {
  g_last_error[0] = '\0';
  if (head_dim < 1) return fail(PDATTN_ERR_INVALID_ARGUMENT, "head_dim %d must be positive", head_dim);
  if (!centroids || !boundaries) return fail(PDATTN_ERR_INVALID_ARGUMENT, "centroids and boundaries required");
  double c[16], b[15];
  lloyd_max16(c, b);
  const double sigma = 1.0 / std::sqrt((double)head_dim);
  for (int i = 0; i < 16; ++i) centroids[i] = (float)(c[i] * sigma);
  for (int i = 0; i < 15; ++i) boundaries[i] = (float)(b[i] * sigma);
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_tq4_append(const pdattn_problem* problem, int32_t num_tokens, const void* k_new,
                                           const void* v_new, const int32_t* token_seq, const int32_t* token_pos,
                                           const int32_t* block_table, const float* rotation,
                                           const float* k_boundaries, const float* v_boundaries, void* cache,
                                           void* stream) {
  g_last_error[0] = '\0';
  pdattn_status st = check_problem(problem, true);
  if (st != PDATTN_OK) return st;
  if (problem->kv_dtype != PDATTN_KV_TQ4) return fail(PDATTN_ERR_INVALID_ARGUMENT, "kv_dtype must be PDATTN_KV_TQ4");
  if (problem->kv_layout != PDATTN_LAYOUT_HND) return fail(PDATTN_ERR_UNSUPPORTED, "TQ4 caches are head-major (HND) only");
  if (num_tokens < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_tokens %d is negative", num_tokens);
  if (num_tokens == 0 || problem->batch == 0 || problem->max_pages_per_seq == 0 || problem->num_pages == 0)
    return PDATTN_OK;
  if (!k_new || !v_new || !token_seq || !token_pos || !block_table || !rotation || !k_boundaries || !v_boundaries ||
      !cache)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(cache, 16) || !aligned(rotation, 16))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "k_new, v_new, cache and rotation must be 16-byte aligned");
  if (!aligned(token_seq, 4) || !aligned(token_pos, 4) || !aligned(block_table, 4) || !aligned(k_boundaries, 4) ||
      !aligned(v_boundaries, 4))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "index arrays and boundaries must be 4-byte aligned");
  pdattn::Tq4AppendParams p;
  std::memset(&p, 0, sizeof p);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.token_seq = token_seq;
  p.token_pos = token_pos;
  p.block_table = block_table;
  p.rotation = rotation;
  p.k_bounds = k_boundaries;
  p.v_bounds = v_boundaries;
  p.cache = static_cast<uint8_t*>(cache);
  p.num_tokens = num_tokens;
  p.batch = problem->batch;
  p.num_kv_heads = problem->num_kv_heads;
  p.page_log2 = ilog2(problem->page_size);
  p.max_pages_per_seq = problem->max_pages_per_seq;
  p.num_pages = problem->num_pages;
  // 16 row vectors (K and V of 8 (token, kv head) pairs) per workgroup,
  // grid-stride beyond 2^20 workgroups
  const int64_t wgs = ceil_div((int64_t)num_tokens * problem->num_kv_heads * 2, 16);
  const uint32_t grid = (uint32_t)std::min<int64_t>(wgs, (int64_t)1 << 20);
  hipError_t e = pdattn::launch_tq4_append(p, problem->head_dim, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "TQ4 append kernel launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_tq4_plan(const pdattn_problem* problem, const int32_t* context_lens_host,
                                         int32_t num_cus, int32_t chunk_tiles, pdattn_tq4_plan_t* out) {
  g_last_error[0] = '\0';
  pdattn_status st = check_tq4_problem(problem);
  if (st != PDATTN_OK) return st;
  if (out == nullptr) return fail(PDATTN_ERR_INVALID_ARGUMENT, "out is NULL");
  if (problem->batch > 0 && context_lens_host == nullptr)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "context_lens_host is NULL");
  if (num_cus < 0 || chunk_tiles < 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "num_cus and chunk_tiles must be >= 0");
  const int64_t cap = (int64_t)problem->max_pages_per_seq * problem->page_size;
  int64_t total = 0, max_len = 0, max_tiles = 0;
  for (int b = 0; b < problem->batch; ++b) {
    const int64_t L = context_lens_host[b];
    if (L < 0 || L > cap)
      return fail(PDATTN_ERR_INVALID_ARGUMENT, "context length %lld of sequence %d outside [0, %lld]", (long long)L, b,
                  (long long)cap);
    const int64_t nt = ceil_div(L, pdattn::kTileTokens);
    total += nt;
    max_len = std::max(max_len, L);
    max_tiles = std::max(max_tiles, nt);
  }
  total *= problem->num_kv_heads;
  if (max_len > 0 && problem->num_pages <= 0) return fail(PDATTN_ERR_INVALID_ARGUMENT, "empty page pool");
  int dev = 0;
  if (num_cus == 0) {
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || num_cus <= 0)
      return fail(PDATTN_ERR_DEVICE, "cannot query the compute-unit count: %s", hipGetErrorString(e));
  }
  int wpc = pdattn::tq4_decode_wgs_per_cu(problem->head_dim);
  if (wpc <= 0) wpc = problem->head_dim == 256 ? 1 : 2;
  const int64_t wgs = (int64_t)num_cus * wpc;
  const int64_t waves = wgs * pdattn::kTq4Waves;
  const int64_t pairs = (int64_t)problem->batch * problem->num_kv_heads;
  int64_t ct = chunk_tiles;
  if (ct == 0) {
    // about one work item per resident wave: a pair's item count rounds up,
    // so the pairs' rounding is taken off the waves first
    const int64_t slots = std::max<int64_t>(waves - pairs, waves / 2);
    ct = std::max<int64_t>(pdattn::kTq4MinChunkTiles, ceil_div(std::max<int64_t>(total, 1), slots));
  }
  ct = std::min<int64_t>(ct, 1 << 24);
  const int64_t mc = std::max<int64_t>(1, ceil_div(std::max<int64_t>(max_tiles, 1), ct));
  if (mc * pairs >= ((int64_t)1 << 31)) return fail(PDATTN_ERR_UNSUPPORTED, "too many work items");
  std::memset(out, 0, sizeof *out);
  out->problem = *problem;
  if (out->problem.scale <= 0.0f) out->problem.scale = 1.0f / std::sqrt((float)problem->head_dim);
  out->num_cus = num_cus;
  out->num_workgroups = (int32_t)std::min<int64_t>(wgs, std::max<int64_t>(1, ceil_div(mc * pairs, pdattn::kTq4Waves)));
  out->chunk_tiles = (int32_t)ct;
  out->max_chunks = (int32_t)mc;
  out->total_tiles = total;
  out->max_context_len = max_len;
  out->workspace_bytes = tq4_workspace(out->problem, out->max_chunks);
  out->magic = kTq4PlanMagic;
  return PDATTN_OK;
}

// Both TQ4 decode calls: model space (rotated = false: q rotated in, out
// rotated back) or the fused attention's own boundary (rotated = true: q
// arrives rotated as fp16, out stays rotated; no rotation matrix).
static pdattn_status tq4_decode_call(const pdattn_tq4_plan_t* plan, const void* q, const void* cache,
                                     const float* rotation, const float* k_centroids, const float* v_centroids,
                                     const int32_t* block_table, const int32_t* context_lens, void* workspace,
                                     uint64_t workspace_bytes, float* out, float* lse, void* stream, bool rotated) {
  g_last_error[0] = '\0';
  pdattn_status st = check_tq4_plan(plan);
  if (st != PDATTN_OK) return st;
  const pdattn_problem& pr = plan->problem;
  if (pr.batch == 0) return PDATTN_OK;
  if (!rotated && !rotation) return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!q || !out || !context_lens || !workspace || !block_table)
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (pr.num_pages > 0 && (!cache || !k_centroids || !v_centroids))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "cache and centroids required");
  if (!aligned(q, 16) || !aligned(cache, 16) || (!rotated && !aligned(rotation, 16)) || !aligned(out, 16) ||
      !aligned(workspace, 16))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "q, cache, rotation, out and workspace must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(context_lens, 4) || !aligned(lse, 4) || !aligned(k_centroids, 4) ||
      !aligned(v_centroids, 4))
    return fail(PDATTN_ERR_INVALID_ARGUMENT, "block_table, context_lens, lse and centroids must be 4-byte aligned");
  if (workspace_bytes < plan->workspace_bytes)
    return fail(PDATTN_ERR_WORKSPACE, "workspace needs %llu bytes, got %llu",
                (unsigned long long)plan->workspace_bytes, (unsigned long long)workspace_bytes);
  pdattn::Tq4DecodeParams p;
  std::memset(&p, 0, sizeof p);
  p.q = static_cast<const uint16_t*>(q);
  p.q_seq = static_cast<uint16_t*>(workspace);
  p.cache = static_cast<const uint8_t*>(cache);
  p.rotation = rotation;
  p.k_cent = k_centroids;
  p.v_cent = v_centroids;
  p.block_table = block_table;
  p.context_lens = context_lens;
  p.rec = reinterpret_cast<float*>(static_cast<char*>(workspace) + tq4_qseq_bytes(pr));
  p.out = out;
  p.lse = lse;
  p.batch = pr.batch;
  p.num_q_heads = pr.num_q_heads;
  p.num_kv_heads = pr.num_kv_heads;
  p.heads_per_kv = heads_per_kv(pr);
  p.page_log2 = ilog2(pr.page_size);
  p.max_pages_per_seq = pr.max_pages_per_seq;
  p.num_pages = pr.num_pages;
  p.chunk_tiles = plan->chunk_tiles;
  p.max_chunks = plan->max_chunks;
  const uint32_t grid = pr.num_pages > 0 && pr.max_pages_per_seq > 0 ? (uint32_t)plan->num_workgroups : 0;
  p.num_waves = (int32_t)(grid * pdattn::kTq4Waves);
  p.qk_scale_log2 = pr.scale * 1.44269504088896340736f;
  p.q_rotated = rotated ? 1 : 0;
  hipError_t e = pdattn::launch_tq4_decode(p, pr.head_dim, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PDATTN_ERR_DEVICE, "TQ4 decode launch: %s", hipGetErrorString(e));
  return PDATTN_OK;
}

PDATTN_API pdattn_status pdattn_tq4_decode(const pdattn_tq4_plan_t* plan, const void* q, const void* cache,
                                           const float* rotation, const float* k_centroids,
                                           const float* v_centroids, const int32_t* block_table,
                                           const int32_t* context_lens, void* workspace, uint64_t workspace_bytes,
                                           float* out, float* lse, void* stream) {
  return tq4_decode_call(plan, q, cache, rotation, k_centroids, v_centroids, block_table, context_lens, workspace,
                         workspace_bytes, out, lse, stream, false);
}

PDATTN_API pdattn_status pdattn_tq4_decode_rotated(const pdattn_tq4_plan_t* plan, const void* q_rot,
                                                   const void* cache, const float* k_centroids,
                                                   const float* v_centroids, const int32_t* block_table,
                                                   const int32_t* context_lens, void* workspace,
                                                   uint64_t workspace_bytes, float* out, float* lse, void* stream) {
  return tq4_decode_call(plan, q_rot, cache, nullptr, k_centroids, v_centroids, block_table, context_lens, workspace,
                         workspace_bytes, out, lse, stream, true);
}

}  // extern "C"
