// Internal launch interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlav {

// Geometry shared by the host planner and the kernels.
constexpr int kDqk = 576;            // 512 latent + 64 rope dims
constexpr int kDv = 512;             // v = first 512 dims of a latent row
constexpr int kRowBytes = kDqk * 2;  // one bf16 latent row: 1152 B = 9 x 128-B lines
constexpr int kWaves = 4;            // waves per workgroup (one per SIMD)
constexpr int kRowsPerWave = 32;     // (token, head) rows owned by one wave
constexpr int kRowsPerGroup = kWaves * kRowsPerWave;  // rows per workgroup: 128
constexpr int kTileKeys = 32;        // keys gathered into LDS per step (one MFMA block)
constexpr int kRowsPerGroup2s = 2 * kRowsPerWave;  // rows per workgroup in the two-stream form: 64
constexpr int kRowsPerGroup4s = kRowsPerWave;      // rows per workgroup in the four-stream form: 32
constexpr int kRangeMaxBatch = 64;   // the range plan holds one request per lane of a wave

// Kernel 1: one workgroup per (request, split, row group of 128, 64 or 32 rows by form).
struct PartialArgs {
  const uint16_t* q;         // bf16 [T_q*H, 576]
  const uint16_t* kv;        // bf16 [num_slots, 576]
  const int32_t* slot_idx;   // [sum L]
  const int32_t* seq_lens;   // [B]
  const int32_t* q_lens;     // [B]
  uint16_t* o_part;          // fp16 [B, nsplit, rows_pad, 512], each row normalised within its split
  float* lse_part;           // fp32 [B, nsplit, rows_pad], natural log
  int32_t batch, heads, max_q_len, nsplit;
  int32_t row_groups;        // ceil(max_q_len*H / rows per workgroup of the form)
  int32_t rows_pad;          // workspace rows per partial (at least max_q_len*H)
  int32_t min_tiles;         // fewest 32-key tiles a split is given (caps the split count)
  int32_t streams;           // 1: 128-row workgroups; 2: 64-row workgroups over two key streams;
                             // 4: 32-row workgroups over four key streams
  int32_t plan_ranges;       // 1: range plan (128-row form, 2..kRangeMaxBatch requests); 0: splits per request
  int32_t workers;           // range plan: workers (each one workgroup per row group)
  float scale_log2;          // sm_scale * log2(e)
  int64_t num_slots;         // rows of kv; read only by the MLA_VERIFY_DEBUG build's slot check
  int32_t* debug_flags;      // MLA_VERIFY_DEBUG builds: device word the checks OR their bits into (or null)
};

// Kernel 2: one wave per (request, row); merges the row's split partials.
struct MergeArgs {
  const void* o_part;        // [B, nsplit, rows_stride, 512]: fp16 (the library's workspace) or fp32
  const float* lse_part;     // fp32 [B, nsplit, rows_stride]
  const int32_t* seq_lens;   // [B]; read only when use_all_splits == 0
  const int32_t* q_lens;     // [B]
  uint16_t* out;             // bf16 [T_q*H, 512]
  float* lse;                // fp32 [T_q*H]
  int32_t batch, heads, max_q_len, nsplit, rows_stride, min_tiles;
  int32_t use_all_splits;    // 1: merge all nsplit partials; 0: only the splits kernel 1 filled
  int32_t part_fp32;         // 1: o_part holds fp32 values; 0: fp16
  int32_t plan_ranges;       // 1: kernel 1 ran the range plan with `workers` workers (partials per request from it)
  int32_t workers;
  int32_t* debug_flags;      // as in PartialArgs
};

// Bits of the MLA_VERIFY_DEBUG build's device flag word (include/mla_verify.h, mla_verify_debug_flags).
constexpr int32_t kDebugSlotOutOfRange = 1;
constexpr int32_t kDebugNegativeLength = 2;
constexpr int32_t kDebugQLenOutOfRange = 4;

// KV compaction: dst[dst_first + j] = src[slot_idx[j]] (whole 1152-B rows), j < n_rows.
constexpr int kCompactThreads = 256;
struct CompactArgs {
  const uint16_t* src;       // bf16 [*, 576]
  const int32_t* slot_idx;   // [n_rows]
  uint16_t* dst;             // bf16 [dst_first + n_rows, 576] at least
  int32_t* new_slot_idx;     // [n_rows] or null: dst_first + j
  int64_t n_rows, dst_first;
};

// Step metadata: lengths and packed slot list of a verify call from a request-to-token table.
constexpr int kMetaThreads = 256;
constexpr int kMetaMaxBatch = 1024;
struct MetadataArgs {
  const int32_t* req_to_token;  // [table_rows, table_stride]; row r: slots of request r by position
  const int32_t* req_ids;       // [batch]
  const int32_t* prefix_lens;   // [batch]
  const int32_t* draft_lens;    // [batch]
  int32_t* slot_idx;            // [slot_capacity]
  int32_t* seq_lens;            // [batch]
  int32_t* q_lens;              // [batch]
  int32_t* status;              // [1]
  int64_t table_stride, slot_capacity;
  int32_t table_rows, table_width, batch;
};

hipError_t launch_partial(const PartialArgs& a, hipStream_t stream);
hipError_t launch_step_metadata(const MetadataArgs& a, hipStream_t stream);
hipError_t launch_compact(const CompactArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

}  // namespace mlav
