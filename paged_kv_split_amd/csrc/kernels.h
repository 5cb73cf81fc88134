// Internal interface between the C-ABI host layer (pdattn.hip) and the
// gfx950 kernels (decode_kernels.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pdattn {

// Waves per workgroup of the decode kernel. Waves are independent workers;
// the workgroup only shares the length scan that places them.
constexpr int kWaves = 4;
// Tokens per tile: the M extent of one 16x16x32 MFMA.
constexpr int kTileTokens = 16;
// Stages of each wave's direct-to-LDS load ring (tiles in flight).
#ifndef PDATTN_STAGES
#define PDATTN_STAGES 2
#endif
constexpr int kStages = PDATTN_STAGES;
// Block-table entries a wave stages in LDS at a time.
constexpr int kPagesPerWave = 256;
// Fewest tiles the planner gives one worker wave.
constexpr int kMinTilesPerWorker = 4;
// Waves per workgroup of the streaming decode kernel.
constexpr int kStreamWaves = 4;
// Largest batch the streaming decode kernel takes (its workgroups hold the
// tile prefix sums of all sequences in LDS).
constexpr int kStreamMaxBatch = 512;
// Tiles of one balancing unit of the dynamic kernel (a pair longer than this
// is cut into several units, merged once more at the end).
constexpr int kUnitTiles = 512;
// Stamped into a dynamic-mode workspace by its initialisation.
constexpr uint32_t kWorkspaceMagic = 0x70645731u;

constexpr int kv_row_bytes(int head_dim, bool fp8) { return head_dim * (fp8 ? 1 : 2); }

// LDS bytes of one decode workgroup: per wave an S-stage ring (K tile, V
// tile, fp8 scales) and a block-table buffer, plus the length-scan scratch.
constexpr int decode_lds_bytes(int head_dim, bool fp8) {
  return kWaves * (kStages * (2 * kTileTokens * kv_row_bytes(head_dim, fp8) + (fp8 ? 256 : 0)) +
                   kPagesPerWave * 4) +
         512;
}

// LDS bytes of one dynamic-kernel workgroup: per wave the ring, a block-
// table buffer and the producer state; the scan and placement scratch.
constexpr int dynamic_lds_bytes(int head_dim, int group, bool fp8) {
  return kWaves * (kStages * (2 * kTileTokens * kv_row_bytes(head_dim, fp8) + (fp8 ? 256 : 0)) +
                   kPagesPerWave * 4 + 96 + 72) +
         64 + 0 * group;
}

// Resident decode workgroups per compute unit when no device can be asked
// (160 KB LDS; 512 VGPRs per SIMD lane, 4 SIMDs; one wave per SIMD per
// workgroup), from upper bounds of the builds' register counts.
constexpr int decode_wgs_per_cu_estimate(int head_dim, int group, bool fp8, bool dynamic) {
  const int by_lds = (160 * 1024) / (dynamic ? dynamic_lds_bytes(head_dim, group, fp8) : decode_lds_bytes(head_dim, fp8));
  const int vgprs = head_dim == 256 ? (group >= 16 ? 512 : 256) : (group >= 8 ? 256 : 168);
  const int by_vgpr = 512 / vgprs;
  const int n = by_lds < by_vgpr ? by_lds : by_vgpr;
  return n < 1 ? 1 : n;
}

// Floats of one worker's partial record: m[G], l[G], acc[G][D].
constexpr int64_t record_floats(int head_dim, int group) { return (int64_t)group * (head_dim + 2); }

struct DecodeParams {
  const uint16_t* q;          // bf16 bits [B][Hq][D]
  const uint8_t* k;           // pool bytes [num_pages][P][Hkv][D * esize]
  const uint8_t* v;
  const float* k_scale;       // fp8 pools: [num_pages][P][Hkv]
  const float* v_scale;
  const int32_t* block_table; // [B][max_pages_per_seq]
  const int32_t* context_lens;
  float* out;                 // [B][Hq][D]
  float* lse;                 // [B][Hq] or null
  float* rec;                 // [num_workers][2][record_floats]
  int64_t* pre;               // [batch + 1]: tiles per kv head before sequence b (workgroup 0 writes it)
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t num_workers;        // waves of the grid that own tile ranges
  int32_t split_wa, split_wb; // worker weights of the split (merge_ops.h): first half wa, the rest wb
  int32_t q_len;              // query rows per sequence (n)
  int32_t heads_per_kv;       // query heads per kv head (Gh)
  int32_t num_cols;           // valid columns n * Gh (<= the kernel's G; the rest is padding)
  int32_t slot_stride;        // row index = page * P * Hkv + slot * slot_stride + kvh * head_stride
  int32_t head_stride;        // (Hkv, 1): rows [page][slot][kvh]; (1, P): rows [page][kvh][slot]
  float qk_scale_log2;        // softmax scale * log2(e)
};

// The dynamic kernel: the same inputs, plus its workspace regions.
struct DynParams {
  const uint16_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* out;
  float* lse;
  float* rec;                 // unit records [units_max + 3 * num_workers][record_floats]
  float* rec2;                // pair-level records [units_max][record_floats] (seg_max > 1)
  uint32_t* ctl;              // counters: claims, records, done tiles [units_max] each; done units [B * Hkv]
  const uint32_t* ws_magic;   // header: kWorkspaceMagic, units_max, batch * num_kv_heads once initialised
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t page_log2;
  int32_t max_pages_per_seq;
  int32_t num_pages;
  int32_t num_workers;
  int32_t seg_max;            // units per pair at most
  int32_t units_max;          // batch * num_kv_heads * seg_max
  int32_t slot_stride;        // row strides as in DecodeParams
  int32_t head_stride;
  float qk_scale_log2;
};

struct MergeParams {
  const float* rec;           // the decode's records
  const int64_t* pre;         // the decode's tile prefix [batch + 1]
  float* out;
  float* lse;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t num_workers;
  int32_t split_wa, split_wb; // as in DecodeParams
  int32_t q_len;              // as in DecodeParams
  int32_t heads_per_kv;
  int32_t num_cols;
};

// KV kinds of the static decode kernel: bf16, fp8 with separate scale
// arrays, fp8 with each row's scale after its codes (4-byte loads, any row
// order; or, for head-major pools, 16-byte loads of the raw rows).
constexpr int kKindBf16 = 0, kKindFp8 = 1, kKindFp8Inline = 2, kKindFp8InlineRows = 3;

// Resident workgroups per compute unit of one decode instantiation, from the
// runtime's occupancy query; 0 when it cannot be asked.
int decode_wgs_per_cu(int head_dim, int group, int kind);

// The streaming decode kernel (decode_stream.hip): bf16 pools or fp8 pools
// with separate scale arrays, page_size >= 16, batch <= kStreamMaxBatch.
int stream_wgs_per_cu(int head_dim, int group, bool fp8);
bool stream_built(int head_dim, int group, bool fp8);  // instantiation within the LDS
hipError_t launch_decode_stream(const DecodeParams& p, int head_dim, int group, bool fp8, uint32_t grid,
                                hipStream_t stream);

// Returns hipErrorInvalidValue for an instantiation that is not built.
hipError_t launch_decode(const DecodeParams& p, int head_dim, int group, int kind, uint32_t grid,
                         hipStream_t stream);
// The split reduce: `waves` 1 (one pair per wave), 4 or 8 (one pair per
// workgroup of that many waves), from merge_waves; at most max_grid
// workgroups, striding over the pairs.
hipError_t launch_merge(const MergeParams& p, int head_dim, int group, int waves, uint32_t max_grid,
                        hipStream_t stream);
// The merge shape for pairs of at most max_pieces pieces.
int merge_waves(int head_dim, int group, int64_t max_pieces);
int dynamic_wgs_per_cu(int head_dim, int group, bool fp8);
hipError_t launch_dynamic(const DynParams& p, int head_dim, int group, bool fp8, uint32_t grid, hipStream_t stream);
hipError_t launch_workspace_init(uint32_t* ctl, uint64_t words, uint32_t* header, uint32_t units_max,
                                 uint32_t pairs, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, uint32_t grid, hipStream_t stream);

}  // namespace pdattn
