// gfx950 kernel for KV compaction of a page_size = 1 latent cache: the "KV
// defragmentation" that magik.net, "The Moment of Truth" (sections "The Broader
// Context: From Kernel to System" and "Conclusion") names as a next step.
//
// dst[dst_first + j] = src[slot_idx[j]] for each 1152-B row, bit for bit.  An
// HBM-bound gather copy: each workgroup moves 32 rows; its 256 threads walk the
// rows' 72 sixteen-byte chunks so that consecutive lanes touch consecutive
// chunks of one row (every row is 9 whole 128-B lines), and each thread keeps
// its nine loads in flight before it stores.
#include "mla_verify_internal.h"

namespace mlav {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kChunksPerRow = kRowBytes / 16;                                  // 72
constexpr int kCompactRows = 32;                                               // rows per workgroup
constexpr int kCompactPerThread = kCompactRows * kChunksPerRow / kCompactThreads;  // 9
static_assert(kCompactRows * kChunksPerRow == kCompactPerThread * kCompactThreads, "whole chunks per thread");

__global__ __launch_bounds__(kCompactThreads) void mla_kv_compact_kernel(CompactArgs a) {
  __shared__ int32_t slots[kCompactRows];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * kCompactRows;
  const int nrows = (int)(a.n_rows - row0 < kCompactRows ? a.n_rows - row0 : kCompactRows);
  if (tid < nrows) slots[tid] = a.slot_idx[row0 + tid];
  __syncthreads();
  const int nchunks = nrows * kChunksPerRow;
  const char* src = (const char*)a.src;
  char* dst = (char*)a.dst + (a.dst_first + row0) * kRowBytes;
  i32x4 v[kCompactPerThread];
#pragma unroll
  for (int k = 0; k < kCompactPerThread; ++k) {
    const int c = tid + kCompactThreads * k;
    if (c < nchunks) {
      const int r = c / kChunksPerRow, off = c - r * kChunksPerRow;
      v[k] = *(const i32x4*)(src + (int64_t)slots[r] * kRowBytes + off * 16);
    }
  }
#pragma unroll
  for (int k = 0; k < kCompactPerThread; ++k) {
    const int c = tid + kCompactThreads * k;
    if (c < nchunks) *(i32x4*)(dst + (int64_t)c * 16) = v[k];
  }
  if (a.new_slot_idx != nullptr && tid < nrows) a.new_slot_idx[row0 + tid] = (int32_t)(a.dst_first + row0 + tid);
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  const int64_t blocks = (a.n_rows + kCompactRows - 1) / kCompactRows;
  hipLaunchKernelGGL(mla_kv_compact_kernel, dim3((unsigned)blocks), dim3(kCompactThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
