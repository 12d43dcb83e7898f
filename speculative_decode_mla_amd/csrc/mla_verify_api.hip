// C ABI of libmla_verify.so (declared in include/mla_verify.h): argument
// checks, workspace ownership and the two launches of a verify call.
#include "mla_verify.h"

#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>

#include "mla_verify_internal.h"

struct mla_verify_s {
  mla_verify_config cfg;
  int device;
  int32_t row_groups;
  int32_t rows_pad;
  int32_t streams;    // kernel 1 form: 1 (128-row workgroups) or 2 (64-row workgroups, two key streams)
  int32_t rows;       // max_q_len * H
  int32_t cus;        // compute units of the device
  int32_t plan_ranges;  // 1: batches of 2..64 requests in the 128-row form use the range plan
  int32_t workers;      // range plan: workers, one workgroup per row group each (CUs / row groups)
  uint16_t* o_part;  // fp16 [B, max_nsplit, rows_pad, 512]
  float* lse_part;  // [B, max_nsplit, rows_pad]
  int32_t* debug_flags;  // MLA_VERIFY_DEBUG builds: the device word of mla_verify_debug_flags (else null)
};

namespace {

// Splits are given at least this many 32-key tiles, so a short request does not
// fan out into many tiny partials (the result does not depend on the split count).
constexpr int32_t kMinTilesPerSplit = 8;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  return e == hipErrorOutOfMemory ? MLA_ERR_OUT_OF_MEMORY : MLA_ERR_HIP;
}

// Validate a config without any HIP call.
int validate_config(const mla_verify_config* cfg) {
  if (cfg == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (cfg->num_heads < 1 || cfg->batch < 1 || cfg->max_q_len < 1 || cfg->max_nsplit < 1 || cfg->num_slots < 1)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!(cfg->sm_scale > 0.f) || !std::isfinite(cfg->sm_scale)) return MLA_ERR_INVALID_ARGUMENT;
  if (cfg->d_qk != MLA_VERIFY_D_QK || cfg->d_v != MLA_VERIFY_D_V) return MLA_ERR_UNSUPPORTED;
  if (cfg->form != MLA_VERIFY_FORM_AUTO && cfg->form != MLA_VERIFY_FORM_128ROW &&
      cfg->form != MLA_VERIFY_FORM_TWO_STREAM && cfg->form != MLA_VERIFY_FORM_FOUR_STREAM)
    return MLA_ERR_INVALID_ARGUMENT;
  if ((cfg->flags & ~MLA_VERIFY_FLAG_BATCH_INVARIANT) != 0) return MLA_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)cfg->max_q_len * cfg->num_heads;
  const int64_t grid = (int64_t)cfg->batch * cfg->max_nsplit * ((rows + mlav::kRowsPerGroup4s - 1) / mlav::kRowsPerGroup4s);
  if (rows > INT32_MAX / 2 || grid > INT32_MAX || (int64_t)cfg->batch * rows > INT32_MAX)
    return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

// Kernel-1 form of a config before the per-call choice: 1 (128-row workgroups), 2 (two streams) or
// 4 (four streams).
int32_t config_streams(const mla_verify_config* cfg) {
  const int64_t rows = (int64_t)cfg->max_q_len * cfg->num_heads;
  // Requests of at most 64 rows (a q_len = 1 decode step with H <= 64) use the two-stream form of
  // kernel 1, whose workgroups hold 64 rows; larger ones the 128-row form (or, per call, a form of
  // fewer rows per workgroup when the call's workgroups would leave most CUs idle; see
  // launch_partials).
  return cfg->form == MLA_VERIFY_FORM_FOUR_STREAM ? 4
         : cfg->form == MLA_VERIFY_FORM_TWO_STREAM ? 2
         : cfg->form == MLA_VERIFY_FORM_128ROW     ? 1
         : rows <= mlav::kRowsPerGroup2s          ? 2 : 1;
}

// Rows per workgroup of a kernel-1 form.
int64_t form_rows(int32_t streams) {
  return streams == 4 ? mlav::kRowsPerGroup4s : streams == 2 ? mlav::kRowsPerGroup2s : mlav::kRowsPerGroup;
}

// Workspace rows per partial: rows past 64 are padded to a multiple of 128, which holds the row
// groups of any form.
int64_t config_rows_pad(const mla_verify_config* cfg) {
  const int64_t rows = (int64_t)cfg->max_q_len * cfg->num_heads;
  const int64_t group = config_streams(cfg) == 1 ? mlav::kRowsPerGroup : mlav::kRowsPerGroup2s;
  return rows <= mlav::kRowsPerGroup2s ? (rows + group - 1) / group * group
                                       : (rows + mlav::kRowsPerGroup - 1) / mlav::kRowsPerGroup * mlav::kRowsPerGroup;
}

// Fill every field of a handle but the workspace pointers (null) from a validated config and the
// device's CU count: the kernel-1 form, the row groups, the range plan.  No HIP call.
void fill_geometry(const mla_verify_config* cfg, int dev, int cus, mla_verify_s* h) {
  const int64_t rows = (int64_t)cfg->max_q_len * cfg->num_heads;
  const int32_t streams = config_streams(cfg);
  const int64_t group = form_rows(streams);
  const int64_t row_groups = (rows + group - 1) / group;
  h->cfg = *cfg;
  h->device = dev;
  h->row_groups = (int32_t)row_groups;
  h->rows_pad = (int32_t)config_rows_pad(cfg);
  h->streams = streams;
  h->rows = (int32_t)rows;
  h->cus = cus;
  // A batch in the 128-row form is spread over one workgroup per CU (one resident per CU), as
  // `workers` workers of row_groups workgroups each (the range plan of kernel 1), unless the
  // caller asked for results independent of the batch composition.
  h->plan_ranges = streams == 1 && cfg->batch >= 2 && cfg->batch <= mlav::kRangeMaxBatch && row_groups <= cus &&
                   (cfg->flags & MLA_VERIFY_FLAG_BATCH_INVARIANT) == 0;
  // (a multiple of 8 from 8 workers on, so that each XCD takes the same share and holds at most
  // 64 workers, one per lane of the planner's wave)
  const int64_t workers = cus / row_groups;
  h->workers = h->plan_ranges ? (int32_t)(workers >= 8 ? workers & ~int64_t(7) : workers) : 0;
  h->o_part = nullptr;
  h->lse_part = nullptr;
  h->debug_flags = nullptr;
}

// The current device and its CU count.
int current_device(int* dev, int* cus) {
  if (hipGetDevice(dev) != hipSuccess) return MLA_ERR_HIP;
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, *dev) != hipSuccess || *cus < 1)
    return MLA_ERR_HIP;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_verify_error_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_OUT_OF_MEMORY: return "MLA_ERR_OUT_OF_MEMORY";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_SCRATCH_TOO_SMALL: return "MLA_ERR_SCRATCH_TOO_SMALL";
    default: return "MLA_ERR_UNKNOWN";
  }
}

int mla_verify_create(const mla_verify_config* cfg, mla_verify_handle* out) {
  if (out == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  int st = validate_config(cfg);
  if (st != MLA_OK) return st;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != MLA_OK) return st;
  mla_verify_s geo;
  fill_geometry(cfg, dev, cus, &geo);
  const int64_t partial_rows = (int64_t)cfg->batch * cfg->max_nsplit * geo.rows_pad;
  mla_verify_s* h = new (std::nothrow) mla_verify_s(geo);
  if (h == nullptr) return MLA_ERR_OUT_OF_MEMORY;
  st = hip_status(hipMalloc((void**)&h->o_part, (size_t)partial_rows * mlav::kDv * sizeof(uint16_t)));
  if (st == MLA_OK) st = hip_status(hipMalloc((void**)&h->lse_part, (size_t)partial_rows * sizeof(float)));
#ifdef MLA_VERIFY_DEBUG
  if (st == MLA_OK) st = hip_status(hipMalloc((void**)&h->debug_flags, sizeof(int32_t)));
  if (st == MLA_OK) st = hip_status(hipMemset(h->debug_flags, 0, sizeof(int32_t)));
#endif
  if (st != MLA_OK) {
    (void)hipGetLastError();
    mla_verify_destroy(h);
    return st;
  }
  *out = h;
  return MLA_OK;
}

}  // extern "C"

namespace {

int check_run_args(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                   const int32_t* seq_lens, const int32_t* q_lens, int32_t nsplit) {
  if (h == nullptr || q == nullptr || kv_pool == nullptr || slot_idx == nullptr || seq_lens == nullptr ||
      q_lens == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (nsplit < 1 || nsplit > h->cfg.max_nsplit) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(slot_idx, 4) || !aligned(seq_lens, 4) ||
      !aligned(q_lens, 4))
    return MLA_ERR_INVALID_ARGUMENT;
  return MLA_OK;
}

int launch_partials(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                    const int32_t* seq_lens, const int32_t* q_lens, int32_t nsplit, hipStream_t s) {
  const mla_verify_config& c = h->cfg;
  mlav::PartialArgs pa;
  pa.q = static_cast<const uint16_t*>(q);
  pa.kv = static_cast<const uint16_t*>(kv_pool);
  pa.slot_idx = slot_idx;
  pa.seq_lens = seq_lens;
  pa.q_lens = q_lens;
  pa.o_part = h->o_part;
  pa.lse_part = h->lse_part;
  pa.batch = c.batch;
  pa.heads = c.num_heads;
  pa.max_q_len = c.max_q_len;
  pa.nsplit = nsplit;
  pa.row_groups = h->row_groups;
  pa.rows_pad = h->rows_pad;
  pa.min_tiles = kMinTilesPerSplit;
  pa.streams = h->streams;
  // A call whose 128-row workgroups would occupy at most half of the CUs (one request with few
  // splits, e.g. nsplit 16 with 8 row groups) takes the two-stream form instead: 64-row workgroups,
  // twice as many, over the same splits, so the partials (and the merge) are the same.  (Decided
  // from the call's shape alone; kernel 1 may still leave splits of short requests empty.)
  // With MLA_VERIFY_FLAG_BATCH_INVARIANT the choice is made as for one request, so that it does
  // not depend on the batch size either.
  const int64_t form_batch = (c.flags & MLA_VERIFY_FLAG_BATCH_INVARIANT) ? 1 : c.batch;
  if (c.form == MLA_VERIFY_FORM_AUTO && pa.streams == 1 && !h->plan_ranges &&
      2 * form_batch * nsplit * h->row_groups <= h->cus) {
    pa.streams = 2;
    pa.row_groups = (h->rows + mlav::kRowsPerGroup2s - 1) / mlav::kRowsPerGroup2s;  // rows_pad (a multiple of 128) holds them
  }
  // In the same way, a call whose 64-row workgroups would occupy at most half of the CUs (a short
  // context with few splits, a decode step with few splits) takes the four-stream form: 32-row
  // workgroups, twice as many again.
  if (c.form == MLA_VERIFY_FORM_AUTO && pa.streams == 2 && 2 * form_batch * nsplit * pa.row_groups <= h->cus) {
    pa.streams = 4;
    pa.row_groups = (h->rows + mlav::kRowsPerGroup4s - 1) / mlav::kRowsPerGroup4s;
  }
  pa.plan_ranges = h->plan_ranges;
  pa.workers = h->workers;
  pa.scale_log2 = c.sm_scale * 1.4426950408889634f;
  pa.num_slots = c.num_slots;
  pa.debug_flags = h->debug_flags;
  return mlav::launch_partial(pa, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_verify_partials(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                        const int32_t* seq_lens, const int32_t* q_lens, int32_t nsplit, void* stream) {
  int st = check_run_args(h, q, kv_pool, slot_idx, seq_lens, q_lens, nsplit);
  if (st != MLA_OK) return st;
  return launch_partials(h, q, kv_pool, slot_idx, seq_lens, q_lens, nsplit, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// ---- The entry point that allocates nothing (mla_verify_run_noalloc) --------------------------------
// Its split workspace is this file-scope device array: every GPU the library runs on holds its own
// copy (MLA_VERIFY_NOALLOC_SCRATCH_BYTES) from the first use until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory; the device address of the current GPU's
// copy comes from hipGetSymbolAddress, once per device, and only that address is handed to kernels.
static_assert(MLA_VERIFY_NOALLOC_SCRATCH_BYTES % 256 == 0, "lse partials start 256-B aligned");
static __device__ __align__(256) char scratch[MLA_VERIFY_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on device d (null until looked up)

// The current device's scratch address, looked up on the first call on that device.
int device_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MLA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MLA_OK;
}

// The two launches of a verify call on a handle whose arguments have been checked.
int enqueue_run(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                const int32_t* seq_lens, const int32_t* q_lens, void* out, float* lse, int32_t nsplit,
                hipStream_t s) {
  int st = launch_partials(h, q, kv_pool, slot_idx, seq_lens, q_lens, nsplit, s);
  if (st != MLA_OK) return st;

  const mla_verify_config& c = h->cfg;
  mlav::MergeArgs ma;
  ma.o_part = h->o_part;
  ma.lse_part = h->lse_part;
  ma.seq_lens = seq_lens;
  ma.q_lens = q_lens;
  ma.out = static_cast<uint16_t*>(out);
  ma.lse = lse;
  ma.batch = c.batch;
  ma.heads = c.num_heads;
  ma.max_q_len = c.max_q_len;
  ma.nsplit = nsplit;
  ma.rows_stride = h->rows_pad;
  ma.min_tiles = kMinTilesPerSplit;
  ma.use_all_splits = 0;
  ma.part_fp32 = 0;
  ma.plan_ranges = h->plan_ranges;
  ma.workers = h->workers;
  ma.debug_flags = h->debug_flags;
  return mlav::launch_merge(ma, s) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

int mla_verify_run(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                   const int32_t* seq_lens, const int32_t* q_lens, void* out, float* lse, int32_t nsplit,
                   void* stream) {
  int st = check_run_args(h, q, kv_pool, slot_idx, seq_lens, q_lens, nsplit);
  if (st != MLA_OK) return st;
  if (out == nullptr || lse == nullptr || !aligned(out, 16) || !aligned(lse, 4)) return MLA_ERR_INVALID_ARGUMENT;
  return enqueue_run(h, q, kv_pool, slot_idx, seq_lens, q_lens, out, lse, nsplit, static_cast<hipStream_t>(stream));
}

int mla_verify_run_noalloc(const mla_verify_config* cfg, const void* q, const void* kv_pool,
                           const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* q_lens, void* out,
                           float* lse, int32_t nsplit, void* stream) {
  int st = validate_config(cfg);
  if (st != MLA_OK) return st;
  if (q == nullptr || kv_pool == nullptr || slot_idx == nullptr || seq_lens == nullptr || q_lens == nullptr ||
      out == nullptr || lse == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (nsplit < 1 || nsplit > cfg->max_nsplit) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(slot_idx, 4) || !aligned(seq_lens, 4) ||
      !aligned(q_lens, 4) || !aligned(out, 16) || !aligned(lse, 4))
    return MLA_ERR_INVALID_ARGUMENT;
  // The call's partials, laid out as in a handle's workspace for this nsplit: fp16 rows, then fp32
  // LSEs from the next 256-B boundary.
  const int64_t partial_rows = (int64_t)cfg->batch * nsplit * config_rows_pad(cfg);
  const int64_t o_bytes = partial_rows * mlav::kDv * (int64_t)sizeof(uint16_t);
  const int64_t lse_offset = (o_bytes + 255) / 256 * 256;
  if (lse_offset + partial_rows * (int64_t)sizeof(float) > (int64_t)MLA_VERIFY_NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_SCRATCH_TOO_SMALL;
  int dev = 0, cus = 0;
  st = current_device(&dev, &cus);
  if (st != MLA_OK) return st;
  void* base = nullptr;
  st = device_scratch(dev, &base);
  if (st != MLA_OK) return st;
  mla_verify_s h;
  fill_geometry(cfg, dev, cus, &h);
  h.o_part = static_cast<uint16_t*>(base);
  h.lse_part = reinterpret_cast<float*>(static_cast<char*>(base) + lse_offset);
  return enqueue_run(&h, q, kv_pool, slot_idx, seq_lens, q_lens, out, lse, nsplit, static_cast<hipStream_t>(stream));
}

int mla_verify_merge(const float* o_part, const float* lse_part, const int32_t* q_lens, int32_t batch,
                     int32_t num_heads, int32_t max_q_len, int32_t nsplit, void* out, float* lse, void* stream) {
  if (o_part == nullptr || lse_part == nullptr || q_lens == nullptr || out == nullptr || lse == nullptr)
    return MLA_ERR_INVALID_ARGUMENT;
  if (batch < 1 || num_heads < 1 || max_q_len < 1 || nsplit < 1) return MLA_ERR_INVALID_ARGUMENT;
  if ((int64_t)max_q_len * num_heads * batch > INT32_MAX) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(o_part, 16) || !aligned(out, 16) || !aligned(lse_part, 4) || !aligned(lse, 4) ||
      !aligned(q_lens, 4))
    return MLA_ERR_INVALID_ARGUMENT;
  mlav::MergeArgs ma;
  ma.o_part = o_part;
  ma.lse_part = lse_part;
  ma.seq_lens = nullptr;
  ma.q_lens = q_lens;
  ma.out = static_cast<uint16_t*>(out);
  ma.lse = lse;
  ma.batch = batch;
  ma.heads = num_heads;
  ma.max_q_len = max_q_len;
  ma.nsplit = nsplit;
  ma.rows_stride = max_q_len * num_heads;
  ma.min_tiles = 1;
  ma.use_all_splits = 1;
  ma.part_fp32 = 1;
  ma.plan_ranges = 0;
  ma.workers = 0;
  ma.debug_flags = nullptr;
  return hip_status(mlav::launch_merge(ma, static_cast<hipStream_t>(stream))) == MLA_OK ? MLA_OK : MLA_ERR_HIP;
}

int mla_verify_compact(const void* kv_pool, const int32_t* slot_idx, int64_t n_rows, void* dst_pool,
                       int64_t dst_slots, int64_t dst_first, int32_t* new_slot_idx, void* stream) {
  if (n_rows < 0 || dst_slots < 0 || dst_first < 0 || n_rows > INT32_MAX) return MLA_ERR_INVALID_ARGUMENT;
  if (n_rows == 0) return MLA_OK;
  if (kv_pool == nullptr || slot_idx == nullptr || dst_pool == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  if (dst_first > dst_slots - n_rows) return MLA_ERR_INVALID_ARGUMENT;
  if (new_slot_idx != nullptr && dst_first + n_rows - 1 > INT32_MAX) return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(kv_pool, 16) || !aligned(dst_pool, 16) || !aligned(slot_idx, 4) ||
      (new_slot_idx != nullptr && !aligned(new_slot_idx, 4)))
    return MLA_ERR_INVALID_ARGUMENT;
  mlav::CompactArgs a;
  a.src = static_cast<const uint16_t*>(kv_pool);
  a.slot_idx = slot_idx;
  a.dst = static_cast<uint16_t*>(dst_pool);
  a.new_slot_idx = new_slot_idx;
  a.n_rows = n_rows;
  a.dst_first = dst_first;
  return mlav::launch_compact(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_verify_build_metadata(const int32_t* req_to_token, int32_t table_rows, int32_t table_width,
                              int64_t table_stride, const int32_t* req_ids, const int32_t* prefix_lens,
                              const int32_t* draft_lens, int32_t batch, int32_t* slot_idx, int64_t slot_capacity,
                              int32_t* seq_lens, int32_t* q_lens, int32_t* status, void* stream) {
  // the per-request arrays are read only for b < batch, slot_idx only below slot_capacity
  if (status == nullptr || (slot_capacity > 0 && slot_idx == nullptr) ||
      (batch > 0 && (req_to_token == nullptr || req_ids == nullptr || prefix_lens == nullptr ||
                     draft_lens == nullptr || seq_lens == nullptr || q_lens == nullptr)))
    return MLA_ERR_INVALID_ARGUMENT;
  if (table_rows < 1 || table_width < 0 || table_stride < table_width || batch < 0 ||
      batch > mlav::kMetaMaxBatch || slot_capacity < 0 || slot_capacity > INT32_MAX)
    return MLA_ERR_INVALID_ARGUMENT;
  if (!aligned(req_to_token, 4) || !aligned(req_ids, 4) || !aligned(prefix_lens, 4) || !aligned(draft_lens, 4) ||
      !aligned(slot_idx, 4) || !aligned(seq_lens, 4) || !aligned(q_lens, 4) || !aligned(status, 4))
    return MLA_ERR_INVALID_ARGUMENT;
  mlav::MetadataArgs a;
  a.req_to_token = req_to_token;
  a.req_ids = req_ids;
  a.prefix_lens = prefix_lens;
  a.draft_lens = draft_lens;
  a.slot_idx = slot_idx;
  a.seq_lens = seq_lens;
  a.q_lens = q_lens;
  a.status = status;
  a.table_stride = table_stride;
  a.slot_capacity = slot_capacity;
  a.table_rows = table_rows;
  a.table_width = table_width;
  a.batch = batch;
  return mlav::launch_step_metadata(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_verify_workspace(mla_verify_handle h, void** o_part, int64_t* o_part_bytes, void** lse_part,
                         int64_t* lse_part_bytes) {
  if (h == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  const int64_t rows = (int64_t)h->cfg.batch * h->cfg.max_nsplit * h->rows_pad;
  if (o_part != nullptr) *o_part = h->o_part;
  if (o_part_bytes != nullptr) *o_part_bytes = rows * mlav::kDv * (int64_t)sizeof(uint16_t);
  if (lse_part != nullptr) *lse_part = h->lse_part;
  if (lse_part_bytes != nullptr) *lse_part_bytes = rows * (int64_t)sizeof(float);
  return MLA_OK;
}

int mla_verify_debug_flags(mla_verify_handle h, int32_t* flags, int32_t clear) {
  if (h == nullptr || flags == nullptr) return MLA_ERR_INVALID_ARGUMENT;
  *flags = 0;
#ifdef MLA_VERIFY_DEBUG
  if (hipDeviceSynchronize() != hipSuccess) return MLA_ERR_HIP;
  if (hipMemcpy(flags, h->debug_flags, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return MLA_ERR_HIP;
  if (clear != 0 && hipMemset(h->debug_flags, 0, sizeof(int32_t)) != hipSuccess) return MLA_ERR_HIP;
  return hipDeviceSynchronize() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
#else
  (void)clear;
  return MLA_ERR_UNSUPPORTED;
#endif
}

int mla_verify_destroy(mla_verify_handle h) {
  if (h == nullptr) return MLA_OK;
  int st = MLA_OK;
  if (h->o_part != nullptr && hipFree(h->o_part) != hipSuccess) st = MLA_ERR_HIP;
  if (h->lse_part != nullptr && hipFree(h->lse_part) != hipSuccess) st = MLA_ERR_HIP;
  if (h->debug_flags != nullptr && hipFree(h->debug_flags) != hipSuccess) st = MLA_ERR_HIP;
  delete h;
  return st;
}

}  // extern "C"
