// gfx950 (MI355X) kernels for MLA speculative-decoding verify attention.
//
// Kernel 1 (mla_verify_partial) computes, for one request, one chunk ("split")
// of its keys and 128 of its (draft token, head) rows, the softmax-attention
// partial of those rows over those keys: o_s (normalised within the chunk) and
// its natural-log LSE.  Kernel 2 (mla_verify_merge) reduces the partials of a
// row into the bf16 output and the fp32 LSE.  This is the partial + reduce
// ("KV-split flash-decode") scheme of magik.net "The Decisive A/B", sections
// "The Context" and "What This Reveals About the Bottleneck", laid out for
// CDNA4 rather than for the sm_120 part the page targets.
//
// Kernel 1 data flow (one workgroup = 4 waves, one per SIMD):
//   * Gather: 64 keys per step.  Each key's 1152-B latent row (9 whole 128-B
//     lines) is fetched through slot_idx straight into LDS with 16-B
//     direct-to-LDS loads, 8 lanes per 128-B line.  Two LDS buffers: the
//     next step's rows stream in while the current step computes.
//   * LDS tile layout: key k, 16-B chunk c of its row lives at
//       ((k/8)*9 + c/8)*1024 + (k%8)*128 + ((c%8) ^ (k%8))*16
//     so one load instruction fills one 1 KiB block (8 keys x 128 B), and the
//     XOR makes both the row reads for Q.K and the transposed reads for P.V
//     hit distinct banks.
//   * Q.K on MFMA 32x32x16 bf16 as S^T = K . Q^T: K (32 keys x 16 dims) is the
//     A operand read from LDS, the wave's 32 query rows are the B operand held
//     in registers for the whole split (36 fragments cover 576 dims).  The
//     C layout then gives each lane one row and 16 keys, so the softmax row
//     statistics need one cross-lane step (lane l and l^32 share a row).
//   * Online softmax in base 2 with the scale folded in; the running max is
//     only raised when a row's max grows by more than 2^8, so the rescale of
//     the 256 accumulator registers is rare.  Causal mask only on steps that
//     reach the draft block (keys >= L - Q + 1).
//   * P.V as O^T = V^T . P^T: the probabilities stay in registers as the B
//     operand (the S^T C layout is already a valid B layout after a fixed
//     permutation of the key order, which the V^T operand repeats), and V^T
//     fragments come from LDS with ds_read_b64_tr_b16, which transposes 4x16
//     blocks of bf16 across each 16-lane group.
#include "mla_verify_internal.h"

namespace mlav {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTileBytes = kTileKeys * kRowBytes;         // 73,728 B per LDS buffer
constexpr int kBlockBytes = 1024;                         // one direct-to-LDS instruction
constexpr int kKeyBlockBytes = 9 * kBlockBytes;           // 8 keys x 1152 B
constexpr int kKeyBlocksPerWave = kTileKeys / 8 / kWaves; // 2: key blocks each wave gathers
constexpr int kQkSteps = kDqk / 16;                       // 36 MFMA k-steps over 576 dims
constexpr int kColBlocks = kDv / 32;                      // 16 blocks of 32 output columns
constexpr int kPrefetch = 6;                              // LDS fragment reads in flight ahead of the MFMA
constexpr float kLn2 = 0.69314718055994530942f;

// Number of splits that carry keys for a request of L keys; both kernels use it.
__device__ __forceinline__ int split_count(int L, int nsplit, int min_tiles) {
  const int tiles = (L + kTileKeys - 1) / kTileKeys;
  if (tiles <= 0) return 0;
  int ns = (tiles + min_tiles - 1) / min_tiles;
  return ns < nsplit ? ns : nsplit;
}

// q_lens[b] clamped to [0, min(L, max_q_len)] (to [0, max_q_len] when seq_lens is null).
__device__ __forceinline__ int clamped_q(const int32_t* q_lens, const int32_t* seq_lens, int b, int max_q) {
  int q = q_lens[b];
  int lim = (seq_lens != nullptr && seq_lens[b] < max_q) ? seq_lens[b] : max_q;
  q = q < lim ? q : lim;
  return q > 0 ? q : 0;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// MFMA 32x32x16 bf16 issued through inline asm so that the accumulator stays in
// the register class chosen here: the 256-register output accumulator in
// AGPRs, the per-block scores in VGPRs.  The compiler does not look inside
// these statements, so the wait states it would otherwise insert are given
// explicitly: "s_nop 2" ahead of each MFMA covers a VALU write of an operand
// register just before it, and the s_nop blocks below cover an MFMA result
// read by VALU code.
__device__ __forceinline__ void mfma_acc_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
// 24 wait states: an MFMA result may now be read by VALU / accvgpr moves.
#define MLAV_MFMA_DRAIN "s_nop 7\n\ts_nop 7\n\ts_nop 7"

// 16-byte direct-to-LDS load: each lane moves 16 B from its global address to
// LDS at lds_addr + 16*lane (lds_addr is wave-uniform, carried in M0).  Issued
// through inline asm so the compiler does not fold these loads into its
// lgkmcnt bookkeeping for the ds_read stream; their completion is awaited
// explicitly (vmcnt) before the barrier that publishes a tile.  The s_nop is the
// wait state required between writing M0 and an LDS-DMA instruction reading it.
// M0 is a reserved register, hence the diagnostic push: nothing else in these
// kernels uses M0 (no LDS-DMA builtins, no GDS, no s_sendmsg).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// bf16 bits -> fp32
__device__ __forceinline__ float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// What one workgroup of kernel 1 works on: request b, split s of its keys,
// 128-row group g of its (draft token, head) rows.
struct WorkItem {
  int b, s, bs, g, L, Q, R, t_begin, t_end;
  int64_t ko, qo;
};

// Decode a workgroup id; false if the workgroup has nothing to do.  The row
// groups that read the same keys get ids that are equal mod 8: workgroups are
// dispatched round-robin over the 8 XCDs, so those groups share one XCD's L2.
__device__ __forceinline__ bool decode_work(const PartialArgs& p, int wg, WorkItem& wi) {
  const int nbs = p.batch * p.nsplit;
  if ((nbs & 7) == 0) {
    const int x = wg & 7, k = wg >> 3;
    wi.g = k % p.row_groups;
    wi.bs = 8 * (k / p.row_groups) + x;
  } else {
    wi.g = wg % p.row_groups;
    wi.bs = wg / p.row_groups;
  }
  wi.b = wi.bs / p.nsplit;
  wi.s = wi.bs - wi.b * p.nsplit;
  wi.L = p.seq_lens[wi.b];
  wi.Q = clamped_q(p.q_lens, p.seq_lens, wi.b, p.max_q_len);
  wi.R = wi.Q * p.heads;
  if (wi.Q <= 0 || wi.g * kRowsPerGroup >= wi.R) return false;
  const int ns = split_count(wi.L, p.nsplit, p.min_tiles);
  if (wi.s >= ns) return false;
  const int tiles = (wi.L + kTileKeys - 1) / kTileKeys;
  wi.t_begin = (int)((int64_t)wi.s * tiles / ns);
  wi.t_end = (int)((int64_t)(wi.s + 1) * tiles / ns);
  int64_t ko = 0, qo = 0;
  for (int i = 0; i < wi.b; ++i) {
    ko += p.seq_lens[i];
    qo += clamped_q(p.q_lens, p.seq_lens, i, p.max_q_len);
  }
  wi.ko = ko;
  wi.qo = qo;
  return true;
}

// Exact recomputation of rows whose scores rose more than kRefHeadroom above
// the row's reference max: one row at a time across the whole wave, with a
// running max and a rescale at every key, in fp32.  Overwrites the row's partial.
// Only reached for such rows, so its speed does not matter.
__device__ __forceinline__ void redo_rows_exact(const PartialArgs& p, const WorkItem& wi, int row_base, uint32_t rows) {
  const int lane = threadIdx.x & 63;
  const int key_begin = wi.t_begin * kTileKeys;
  const int key_end = min(wi.L, wi.t_end * kTileKeys);
  const int32_t* slots = p.slot_idx + wi.ko;
  while (rows != 0) {
    const int i = __builtin_ctz(rows);
    rows &= rows - 1;
    const int row = row_base + i;
    const int tok = row / p.heads;
    const int kend = min(key_end, wi.L - wi.Q + tok + 1);
    const uint16_t* qrow = p.q + (wi.qo * p.heads + row) * kDqk;
    float qv[9];
#pragma unroll
    for (int d = 0; d < 9; ++d) qv[d] = bf16f(qrow[d * 64 + lane]);
    float m = -INFINITY, l = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int key = key_begin; key < kend; ++key) {
      const uint16_t* krow = p.kv + (int64_t)slots[key] * kDqk;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < 9; ++d) dot += qv[d] * bf16f(krow[d * 64 + lane]);
      const float x = wave_sum(dot) * p.scale_log2;
      const float m_new = fmaxf(m, x);
      const float a = __builtin_amdgcn_exp2f(m - m_new);
      const float pw = __builtin_amdgcn_exp2f(x - m_new);
      l = l * a + pw;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = acc[j] * a + pw * bf16f(krow[lane * 8 + j]);
      m = m_new;
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t prow = (int64_t)wi.bs * p.rows_pad + row;
    float* dst = p.o_part + prow * kDv + lane * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = acc[j] * inv;
    if (lane == 0) p.lse_part[prow] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  }
}

}  // namespace

// Headroom (log2 units) above a row's reference max before exp2 could overflow
// the fp32 sums: p = 2^(x - m_ref) <= 2^64, times <= 2^31 keys, stays finite.
constexpr float kRefHeadroom = 64.0f;

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_verify_partial(PartialArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * kTileBytes];
  lds_char* smem = (lds_char*)smem_raw;

  WorkItem wi;
  if (!decode_work(p, blockIdx.x, wi)) return;
  const int L = wi.L, Q = wi.Q, H = p.heads, R = wi.R;
  const int t_begin = wi.t_begin, t_end = wi.t_end;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, lrow = lane & 31;
  const int myrow = wi.g * kRowsPerGroup + w * kRowsPerWave + lrow;  // (token, head) row in the request
  const bool row_valid = myrow < R;
  const int tok = row_valid ? myrow / H : 0;
  const int limit = L - Q + tok + 1;  // this row sees keys [0, limit)
  const int mask_from = L - Q + 1;    // first key that some draft row cannot see

  // ---- gather set-up --------------------------------------------------------------------------
  const int g_kr = lane >> 3;                   // key within an 8-key block
  const int g_byte = ((lane & 7) ^ g_kr) << 4;  // 16-B chunk of the 128-B line this lane moves
  const int32_t* slots = p.slot_idx + wi.ko;
  const char* kv = (const char*)p.kv;
  auto slot_of = [&](int tile, int e) {
    int key = tile * kTileKeys + (w * kKeyBlocksPerWave + e) * 8 + g_kr;
    key = key < L ? key : L - 1;  // ragged tail: repeat the last row (masked out below)
    return slots[key];
  };
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const int w_uniform = __builtin_amdgcn_readfirstlane(w);
  auto issue_tile = [&](int buf, int sl0, int sl1) {
    const uint32_t base = smem_base + buf * kTileBytes + w_uniform * kKeyBlocksPerWave * kKeyBlockBytes;
    const char* r0 = kv + (int64_t)sl0 * kRowBytes + g_byte;
    const char* r1 = kv + (int64_t)sl1 * kRowBytes + g_byte;
#pragma unroll
    for (int cg = 0; cg < 9; ++cg) dma16(r0 + cg * 128, base + cg * kBlockBytes);
#pragma unroll
    for (int cg = 0; cg < 9; ++cg) dma16(r1 + cg * 128, base + kKeyBlockBytes + cg * kBlockBytes);
  };

  int sl0 = slot_of(t_begin, 0), sl1 = slot_of(t_begin, 1);
  issue_tile(0, sl0, sl1);
  if (t_begin + 1 < t_end) {
    sl0 = slot_of(t_begin + 1, 0);
    sl1 = slot_of(t_begin + 1, 1);
  }

  // ---- the wave's 32 query rows, resident for the whole split ----------------------------------
  // lane holds row lrow, dims 16*ks + 8*hi .. +7 (MFMA B-operand layout)
  bf16x8 qf[kQkSteps];
  {
    const i32x4* qrow = (const i32x4*)(p.q + ((wi.qo * H + (row_valid ? myrow : 0)) * kDqk)) + hi;
    const int keep = row_valid ? -1 : 0;  // rows past the request are zero
#pragma unroll
    for (int ks = 0; ks < kQkSteps; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qrow[2 * ks] & keep);
  }

  // ---- per-lane LDS read addresses -----------------------------------------------------------
  // Q.K A operand: lane reads key (kb*32 + lrow), 16-B chunk (2*ks + hi).
  int kaddr[4];
  {
    const int base = (lrow >> 3) * kKeyBlockBytes + (lrow & 7) * 128;
    const int y = hi ^ (lrow & 7);
#pragma unroll
    for (int j = 0; j < 4; ++j) kaddr[j] = base + (((2 * j) ^ y) << 4);
  }
  // P.V A operand via the 4x16 transposing read: in 16-lane group G, lane j reads
  // key 4*(G>>1) + (j>>2) (+ 16*kk + 8*r) at columns 32*cb + 16*(G&1) + 4*(j&3) .. +3;
  // lane l then holds column 32*cb + (l&31) for keys 16*kk + 8*r + 4*(l>>5) .. +3.
  int vaddr[2];
  {
    const int G = lane >> 4, j = lane & 15;
    const int kr = 4 * (G >> 1) + (j >> 2);
    const int z = (2 * (G & 1) + ((j & 3) >> 1)) ^ kr;
#pragma unroll
    for (int e = 0; e < 2; ++e) vaddr[e] = kr * 128 + (((4 * e) ^ z) << 4) + (j & 1) * 8;
  }

  f32x16 o[kColBlocks];
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb) o[cb] = (f32x16){};
  // Softmax with a fixed per-row reference: m_ref is the row max of the split's
  // first block with a visible key; p = 2^(x - m_ref) is exact as long as no
  // later score exceeds m_ref by more than kRefHeadroom.  A row that does is
  // recomputed exactly at the end (redo_rows_exact).
  float m_ref = -INFINITY;
  float l_run = 0.f;    // this lane's share of the row sum of bf16-rounded P
  float l_exact = 0.f;  // ... and of P before rounding
  bool overflow = false;

  for (int it = t_begin; it < t_end; ++it) {
    const int buf = (it - t_begin) & 1;
    __builtin_amdgcn_s_waitcnt(0x0070 /* vmcnt(0) lgkmcnt(0) */);
    __syncthreads();
    if (it + 1 < t_end) {
      issue_tile(buf ^ 1, sl0, sl1);
      if (it + 2 < t_end) {
        sl0 = slot_of(it + 2, 0);
        sl1 = slot_of(it + 2, 1);
      }
    }
    const lds_char* tb = smem + buf * kTileBytes;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {  // two 32-key blocks per tile
      const int k0 = it * kTileKeys + kb * 32;
      const lds_char* kbp = tb + kb * 4 * kKeyBlockBytes;

      // S^T = K . Q^T: 32 keys x the wave's 32 rows.  K fragments are read
      // kPrefetch steps ahead of the MFMA that consumes them; the scheduling
      // barriers keep the compiler from sinking the reads next to their use.
      bf16x8 kf[kQkSteps];
      auto kread = [&](int ks) {
        kf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(kbp + kaddr[ks & 3] + (ks >> 2) * kBlockBytes);
      };
#pragma unroll
      for (int ks = 0; ks < kPrefetch; ++ks) kread(ks);
      f32x16 sacc;
#pragma unroll
      for (int ks = 0; ks < kQkSteps; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks + kPrefetch < kQkSteps) kread(ks + kPrefetch);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) mfma_first_v(sacc, kf[ks], qf[ks]);
        else mfma_acc_v(sacc, kf[ks], qf[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile(MLAV_MFMA_DRAIN : "+v"(sacc));

      // softmax numerators (base 2): lane holds row lrow, keys k0 + 8*(j>>2) + 4*hi + (j&3)
      sacc *= p.scale_log2;
      if (k0 + 32 > mask_from) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + 8 * (j >> 2) + 4 * hi + (j & 3);
          sacc[j] = key < limit ? sacc[j] : -INFINITY;
        }
      }
      float mx = sacc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sacc[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_ref = (m_ref == -INFINITY) ? mx : m_ref;
      overflow |= mx > m_ref + kRefHeadroom;
      const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
      // P is rounded to bf16 for the MFMA.  Two row sums: of the rounded values,
      // which normalises O (so o_s is a convex combination of the weights the
      // MFMA actually used), and of the unrounded values, which gives the LSE.
      bf16x8 pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float pv = __builtin_amdgcn_exp2f(sacc[kk * 8 + i] - mref);
          const __bf16 pb = (__bf16)pv;
          pf[kk][i] = pb;
          l_run += (float)pb;
          l_exact += pv;
        }

      // O^T += V^T . P^T over these 32 keys; V^T fragments read kPrefetch ahead
      bf16x8 vf[2 * kColBlocks];
      auto vread = [&](int i) {  // fragment i = (column block i/2, 16-key step i%2)
        const int cb = i >> 1, kk = i & 1;
        const lds_char* vb = tb + vaddr[cb & 1] + (cb >> 1) * kBlockBytes + (kb * 4 + 2 * kk) * kKeyBlockBytes;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)vb);
        const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(vb + kKeyBlockBytes));
        vf[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int i = 0; i < kPrefetch; ++i) vread(i);
#pragma unroll
      for (int i = 0; i < 2 * kColBlocks; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kPrefetch < 2 * kColBlocks) vread(i + kPrefetch);
        __builtin_amdgcn_sched_barrier(0);
        mfma_acc_a(o[i >> 1], vf[i], pf[i & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile(MLAV_MFMA_DRAIN : "+a"(o[kColBlocks - 1]));

  // ---- partial write: o_s = O / l, lse_s = ln2 * (m_ref + log2 l) -------------------------------
  if (!row_valid) return;
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float le = l_exact + __shfl_xor(l_exact, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  const int64_t prow = ((int64_t)wi.bs * p.rows_pad + myrow);
  float* dst = p.o_part + prow * kDv + 4 * hi;
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v = {o[cb][4 * q4 + 0] * inv, o[cb][4 * q4 + 1] * inv, o[cb][4 * q4 + 2] * inv, o[cb][4 * q4 + 3] * inv};
      *(f32x4*)(dst + cb * 32 + 8 * q4) = v;
    }
  if (hi == 0) p.lse_part[prow] = le > 0.f ? (m_ref + __builtin_amdgcn_logf(le)) * kLn2 : -INFINITY;

  // Rows whose scores outgrew the fixed reference are redone exactly by the wave.
  const uint64_t redo = __ballot(overflow && hi == 0);
  if (redo != 0) redo_rows_exact(p, wi, wi.g * kRowsPerGroup + w * kRowsPerWave, (uint32_t)redo);
}

__global__ __launch_bounds__(256) void mla_verify_merge_kernel(MergeArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t row_global = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int rows_per_b = p.max_q_len * p.heads;
  const int b = (int)(row_global / rows_per_b);
  const int r = (int)(row_global - (int64_t)b * rows_per_b);
  if (b >= p.batch) return;
  const int Q = clamped_q(p.q_lens, p.seq_lens, b, p.max_q_len);
  if (r >= Q * p.heads) return;
  const int ns = p.use_all_splits ? p.nsplit : split_count(p.seq_lens[b], p.nsplit, p.min_tiles);
  int64_t qo = 0;
  for (int i = 0; i < b; ++i) qo += clamped_q(p.q_lens, p.seq_lens, i, p.max_q_len);

  const int64_t base = (int64_t)b * p.nsplit * p.rows_stride + r;  // (b, s=0, r)
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float v = s < ns ? p.lse_part[base + (int64_t)s * p.rows_stride] : -INFINITY;
    M = fmaxf(M, wave_max(v));
  }
  const float Mref = (M == -INFINITY) ? 0.f : M;
  float Z = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float v = s < ns ? p.lse_part[base + (int64_t)s * p.rows_stride] : -INFINITY;
    Z += wave_sum(__expf(v - Mref));
  }
  const float invZ = Z > 0.f ? 1.0f / Z : 0.f;
  f32x4 a0 = {}, a1 = {};
  for (int s = 0; s < ns; ++s) {
    const int64_t off = base + (int64_t)s * p.rows_stride;
    const float ws = __expf(p.lse_part[off] - Mref) * invZ;
    const f32x4* src = (const f32x4*)(p.o_part + off * kDv) + 2 * lane;
    a0 += ws * src[0];
    a1 += ws * src[1];
  }
  const int64_t orow = qo * p.heads + r;
  bf16x8 ov;
  ov[0] = (__bf16)a0[0]; ov[1] = (__bf16)a0[1]; ov[2] = (__bf16)a0[2]; ov[3] = (__bf16)a0[3];
  ov[4] = (__bf16)a1[0]; ov[5] = (__bf16)a1[1]; ov[6] = (__bf16)a1[2]; ov[7] = (__bf16)a1[3];
  *((bf16x8*)(p.out + orow * kDv) + lane) = ov;
  if (lane == 0) p.lse[orow] = Z > 0.f ? Mref + __logf(Z) : -INFINITY;
}

hipError_t launch_partial(const PartialArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.batch * a.nsplit * a.row_groups;
  hipLaunchKernelGGL(mla_verify_partial, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.max_q_len * a.heads;
  const int64_t grid = (rows + 3) / 4;
  hipLaunchKernelGGL(mla_verify_merge_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
