// gfx950 kernel that builds one verify step's metadata on the device: the
// "combined indices once per step" and "marshaling kernel" remedies of
// magik.net, "The Moment of Truth" ("Interpreting the Crossover: The
// Marshaling Tax", "Assumptions and Their Validity"), in static buffers so the
// step can be captured ("The Thinking Process").
//
//   seq_lens[b] = prefix_lens[b] + draft_lens[b],  q_lens[b] = draft_lens[b],
//   slot_idx    = first seq_lens[b] entries of table row req_ids[b], b in order.
//
// Every workgroup reads the (small) per-request arrays, validates them and
// forms the request offsets with a block scan in LDS; workgroup 0 writes the
// lengths and the status word; then all workgroups copy the slots over the
// concatenated token range in a grid-stride loop (consecutive lanes copy
// consecutive positions of one table row).  Bad input: status != 0, all
// lengths 0 and no slot written.
#include "mla_verify_internal.h"

namespace mlav {
namespace {

constexpr int kMetaPerThread = kMetaMaxBatch / kMetaThreads;  // requests per thread in the scan
static_assert(kMetaPerThread * kMetaThreads == kMetaMaxBatch, "");

__global__ __launch_bounds__(kMetaThreads) void mla_step_metadata_kernel(MetadataArgs a) {
  __shared__ int64_t off[kMetaMaxBatch + 1];  // exclusive prefix sums of the sequence lengths
  __shared__ int32_t seq[kMetaMaxBatch];
  __shared__ int32_t row_of[kMetaMaxBatch];
  __shared__ int64_t part[kMetaThreads];
  __shared__ int32_t bad;
  const int tid = threadIdx.x, B = a.batch;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kMetaThreads) {
    const int32_t r = a.req_ids[b], p = a.prefix_lens[b], d = a.draft_lens[b];
    int e = 0;
    if (r < 0 || r >= a.table_rows) e |= 1;
    if (p < 0 || d < 0) e |= 2;
    const int64_t s = (int64_t)p + d;
    if (s > a.table_width) e |= 4;
    seq[b] = e ? 0 : (int32_t)s;
    row_of[b] = r;
    if (e) atomicOr(&bad, e);
  }
  __syncthreads();
  // block scan: thread t sums requests [t*P, t*P + P), then an inclusive scan of those sums
  int64_t local = 0;
#pragma unroll
  for (int k = 0; k < kMetaPerThread; ++k) {
    const int b = tid * kMetaPerThread + k;
    if (b < B) local += seq[b];
  }
  part[tid] = local;
  __syncthreads();
  for (int d = 1; d < kMetaThreads; d <<= 1) {
    const int64_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int64_t run = part[tid] - local;  // exclusive prefix of this thread's first request
#pragma unroll
  for (int k = 0; k < kMetaPerThread; ++k) {
    const int b = tid * kMetaPerThread + k;
    if (b < B) {
      off[b] = run;
      run += seq[b];
    }
  }
  if (tid == kMetaThreads - 1) off[B] = part[tid];
  __syncthreads();
  if (tid == 0 && bad == 0 && off[B] > a.slot_capacity) bad = 8;
  __syncthreads();
  const int err = bad;
  if (blockIdx.x == 0) {
    for (int b = tid; b < B; b += kMetaThreads) {
      a.seq_lens[b] = err ? 0 : seq[b];
      a.q_lens[b] = err ? 0 : a.draft_lens[b];
    }
    if (tid == 0) *a.status = err;
  }
  if (err != 0 || B == 0) return;
  const int64_t total = off[B];
  const int64_t stride = (int64_t)gridDim.x * kMetaThreads;
  for (int64_t k = (int64_t)blockIdx.x * kMetaThreads + tid; k < total; k += stride) {
    int lo = 0, hi = B - 1;  // the last request whose range starts at or before k
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= k) lo = mid;
      else hi = mid - 1;
    }
    a.slot_idx[k] = a.req_to_token[(int64_t)row_of[lo] * a.table_stride + (k - off[lo])];
  }
}

}  // namespace

hipError_t launch_step_metadata(const MetadataArgs& a, hipStream_t stream) {
  int64_t blocks = (a.slot_capacity + 8 * kMetaThreads - 1) / (8 * kMetaThreads);
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(mla_step_metadata_kernel, dim3((unsigned)blocks), dim3(kMetaThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
