// gfx950 (MI355X) kernels for MLA speculative-decoding verify attention.
//
// Kernel 1 (mla_verify_partial) computes, for one request, one chunk ("split")
// of its keys and 128 of its (draft token, head) rows, the softmax-attention
// partial of those rows over those keys: o_s (normalised within the chunk) and
// its natural-log LSE.  Two more layouts of it serve calls with few rows or few
// splits: mla_verify_partial_2s (64 rows, two key streams) and
// mla_verify_partial_4s (32 rows, four key streams), further below.  Kernel 2
// (mla_verify_merge) reduces the partials of a row into the bf16 output and the
// fp32 LSE.  This is the partial + reduce
// ("KV-split flash-decode") scheme of magik.net "The Decisive A/B", sections
// "The Context" and "What This Reveals About the Bottleneck", laid out for
// CDNA4 rather than for the sm_120 part the page targets.
//
// Kernel 1, one workgroup = 4 waves (one per SIMD), 32 (token, head) rows per wave:
//   * Slot indices: each lane holds one slot of each of the next 8 tiles; a
//     shuffle hands every gathering lane its key's slot.
//   * Gather: 32 keys per tile.  Each key's 1152-B latent row (9 whole 128-B
//     lines) goes straight from HBM into LDS with 16-B direct-to-LDS loads,
//     8 lanes per 128-B line, 8 keys per wave.  A ring of 4 tile buffers; the
//     load of tile i+3 is issued while tile i is being consumed.
//   * LDS tile layout: key k (0..31), 16-B chunk c (0..71) of its row lives at
//       ((k/8)*9 + c/8)*1024 + (k%8)*128 + ((c%8) ^ f(k))*16,  f(k) = (k%8) ^ ((k/8)%2)
//     so one load instruction fills one 1 KiB block (8 keys x 128 B), and the
//     XOR spreads both read patterns below over all banks.
//   * Q.K on MFMA 32x32x16 bf16 as S^T = K . Q^T: K (32 keys x 16 dims) is the
//     A operand read from LDS, the wave's 32 query rows are the B operand held
//     in registers for the whole split (36 fragments cover 576 dims).  In the C
//     layout each lane then holds one row and 16 keys; lanes l and l^32 share a
//     row.
//   * Softmax in base 2 with the scale folded in, against a per-row reference
//     max fixed at the split's first tile (no rescale of the accumulators; a
//     row whose sum outgrows it is redone exactly).  The exponentials of tile i
//     are computed between the Q.K MFMAs of tile i+1, its row sums between its
//     own P.V MFMAs.  Causal mask on the draft block (keys >= L - Q + 1).
//   * P.V as O^T = V^T . P^T: the probabilities stay in registers as the B
//     operand (the S^T C layout is a valid B layout after a fixed permutation
//     of the key order, which the V^T operand repeats), and V^T fragments come
//     from LDS with ds_read_b64_tr_b16, which transposes 4x16 blocks of bf16
//     across each 16-lane group.  Waves 2k and 2k+1 form a pair: each computes
//     256 of the 512 output columns for the pair's 64 rows, taking its
//     partner's P through LDS, so each wave reads only half of V.
#include <type_traits>

#include "mla_verify_internal.h"

namespace mlav {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTileBytes = kTileKeys * kRowBytes;  // 36,864 B per LDS tile buffer
constexpr int kRing = 4;                           // tile buffers
constexpr int kAhead = kRing - 1;                  // tiles in flight ahead of the one being consumed
constexpr int kXchgBytes = 2 * kWaves * 2048;      // bf16 P of every wave, two buffers
constexpr int kBlockBytes = 1024;                  // one direct-to-LDS instruction: 8 keys x 128 B
constexpr int kKeyBlockBytes = 9 * kBlockBytes;    // 8 keys x 1152 B
constexpr int kQkSteps = kDqk / 16;                // 36 MFMA k-steps over 576 dims
constexpr int kColBlocks = kDv / 32;               // 16 blocks of 32 output columns
constexpr int kHalfColBlocks = kColBlocks / 2;     // column blocks of one wave of a pair
constexpr int kPvFrags = 2 * kHalfColBlocks;       // V^T fragments per wave per tile (2 MFMAs each)
constexpr int kPrefetch = 4;                       // K fragment reads kept ahead of their MFMA
constexpr int kVPrefetch = 4;                      // V^T fragment reads kept ahead
constexpr int kDmaPerTile = 9;                     // direct-to-LDS loads per wave per tile
constexpr int kStageRowBytes = 528;                // epilogue: one fp16 row half (512 B) + 16 B of padding
constexpr int kStageBytes = 64 * kStageRowBytes;   // epilogue: one wave's 64 rows
constexpr float kLn2 = 0.69314718055994530942f;
static_assert(kTileKeys == 32 && kWaves * 8 == kTileKeys, "one 8-key block per wave per tile");
static_assert(kRing * kTileBytes + kXchgBytes <= 163840, "LDS budget");
static_assert(kWaves * kStageBytes <= kRing * kTileBytes, "epilogue staging fits in the ring");

// Number of splits that carry keys for a request of L keys; both kernels use it.
__device__ __forceinline__ int split_count(int L, int nsplit, int min_tiles) {
  const int tiles = (L + kTileKeys - 1) / kTileKeys;
  if (tiles <= 0) return 0;
  int ns = (tiles + min_tiles - 1) / min_tiles;
  return ns < nsplit ? ns : nsplit;
}

// Checks of device-visible arguments, compiled in only for the MLA_VERIFY_DEBUG build: a bad value
// is replaced before it is used for any access, and the check ORs its bit into *flags.  In the
// release build every one of them is the identity.
__device__ __forceinline__ void debug_flag(int32_t* flags, int32_t bit) {
#ifdef MLA_VERIFY_DEBUG
  if (flags != nullptr) atomicOr(flags, bit);
#else
  (void)flags;
  (void)bit;
#endif
}

// seq_lens[b]; the debug build reads a negative length as 0.
__device__ __forceinline__ int read_len(const int32_t* seq_lens, int b, int32_t* flags) {
  int L = seq_lens[b];
#ifdef MLA_VERIFY_DEBUG
  if (L < 0) {
    debug_flag(flags, kDebugNegativeLength);
    L = 0;
  }
#endif
  (void)flags;
  return L;
}

// A slot index read from slot_idx; the debug build clamps it into [0, num_slots).
__device__ __forceinline__ int checked_slot(int slot, int64_t num_slots, int32_t* flags) {
#ifdef MLA_VERIFY_DEBUG
  if (slot < 0 || (int64_t)slot >= num_slots) {
    debug_flag(flags, kDebugSlotOutOfRange);
    slot = slot < 0 ? 0 : (int)(num_slots - 1);
  }
#endif
  (void)num_slots;
  (void)flags;
  return slot;
}

// q_lens[b] clamped to [0, min(L, max_q_len)] (to [0, max_q_len] when seq_lens is null); the debug
// build also flags a value it had to clamp.
__device__ __forceinline__ int clamped_q(const int32_t* q_lens, const int32_t* seq_lens, int b, int max_q,
                                         int32_t* flags = nullptr) {
  const int q0 = q_lens[b];
  const int L = seq_lens != nullptr ? read_len(seq_lens, b, flags) : max_q;
  const int lim = L < max_q ? L : max_q;
  int q = q0 < lim ? q0 : lim;
  q = q > 0 ? q : 0;
  if (q != q0 && seq_lens != nullptr) debug_flag(flags, kDebugQLenOutOfRange);
  return q;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// max / sum of v over lanes l and l^32 (the two lanes that hold one row)
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// ... and over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one row of a 16x16 MFMA result); all four
// lanes get the same bits
__device__ __forceinline__ float quad_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return pair_max(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return pair_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

// MFMA 32x32x16 bf16 issued through inline asm so that the accumulator stays in
// the register class chosen here: the 256-register output accumulator in
// AGPRs, the per-tile scores in VGPRs.  The statements are volatile so that
// they keep their order relative to the softmax statements below, which sit
// between them on purpose.  The compiler does not look inside these statements,
// so it inserts no wait states for them.  Two hazards matter: a VALU write of
// an operand register just before an MFMA, and a VALU read of an MFMA result.
// The second is covered by MLAV_MFMA_DRAIN wherever scores or accumulators are
// read.  The first does not arise in the schedule below (operands come from LDS
// reads, which are waited on with lgkmcnt, from the resident q fragments, or
// from bf16 packs made many instructions earlier); tests/test_kernel_hazards.py
// checks the generated code for both.
__device__ __forceinline__ void mfma_acc_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_first_v(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
}
// MFMA 16x16x32 bf16 (the four-stream form's Q.K), accumulator in VGPRs
__device__ __forceinline__ void mfma16_acc_v(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_first_v(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

// Single VALU ops as volatile statements, so that each stays in the MFMA gap it
// is written in (the compiler would otherwise gather them into one block).
// None of them has a wait-state requirement towards its neighbours except the
// exp2: its result is read no earlier than after the next MFMA.
__device__ __forceinline__ float vfma(float x, float s, float c) {
  float r;
  asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(s), "v"(c));
  return r;
}
__device__ __forceinline__ float vexp2(float x) {
  float r;
  asm volatile("v_exp_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ int vpack_bf16(float lo, float hi) {  // round to nearest even
  int r;
  asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}
__device__ __forceinline__ void vadd_to(float& acc, float x) {
  asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(x));
}
// acc += lo + hi of a bf16 pair, widened exactly (a bf16 is the top half of an fp32).
// Four single-cycle ops: v_dot2c_f32_bf16 would do it in one but holds the wave
// for about eight cycles next to an MFMA.
__device__ __forceinline__ void vsum_pair_to(float& acc, int pair) {
  float lo, hi;
  asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(lo) : "v"(pair));
  asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(hi) : "v"(pair));
  asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(lo));
  asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc) : "v"(hi));
}
// 24 wait states: an MFMA result may now be read by VALU / accvgpr moves.
#define MLAV_MFMA_DRAIN "s_nop 7\n\ts_nop 7\n\ts_nop 7"

// One accumulator element out of its AGPR, as a volatile statement so that it keeps its
// place after the drain (the compiler would otherwise move such reads up to the last MFMA).
__device__ __forceinline__ float acc_read(float a) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(a));
  return r;
}

// 16-byte direct-to-LDS load: each lane moves 16 B from gsrc + OFF to LDS at
// m0 + OFF + 16*lane.  The immediate OFF applies to both addresses, so a caller
// that wants the data at lds_addr passes m0 = lds_addr - OFF: the nine loads of a
// key block then share one 64-bit row address and differ only in SALU-computed
// M0 values and the immediate, with no VALU work per load.  Issued through inline
// asm so the compiler does not fold these loads into its lgkmcnt bookkeeping for
// the ds_read stream; their completion is awaited explicitly (vmcnt) before the
// barrier that publishes a tile.  The s_nop is the wait state required between
// writing M0 and an LDS-DMA instruction reading it.  M0 is a reserved register,
// hence the diagnostic push: nothing else in these kernels uses M0 (no LDS-DMA
// builtins, no GDS, no s_sendmsg).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF>
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t m0_value) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               :
               : "v"(gsrc), "s"(m0_value), "i"(OFF)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// 16-byte store with the agent-coherence bit (sc1): written through to memory rather than left
// dirty in this XCD's L2, where the end of the kernel would have to write it back.
__device__ __forceinline__ void store16_through(void* dst, const i32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(dst), "v"(v) : "memory");
}
// ... at dst + OFF bytes (the instruction's immediate offset)
template <int OFF>
__device__ __forceinline__ void store16_through_at(void* dst, const i32x4& v) {
  static_assert(OFF >= 0 && OFF < 4096, "immediate offset range");
  asm volatile("global_store_dwordx4 %0, %1, off offset:%2 sc1" : : "v"(dst), "v"(v), "i"(OFF) : "memory");
}

// One wave's share of a tile: key block w (8 keys x 1152 B) as nine 1 KiB loads;
// load cg moves 16-B chunks [8cg, 8cg+8) of the eight rows (see the layout above).
// dma_chunk_group issues load cg alone (cg a compile-time constant after unrolling).
__device__ __forceinline__ void dma_chunk_group(const char* row, uint32_t lds_block, int cg) {
  switch (cg) {
    case 0: dma16<0 * 128>(row, lds_block + 0 * (kBlockBytes - 128)); break;
    case 1: dma16<1 * 128>(row, lds_block + 1 * (kBlockBytes - 128)); break;
    case 2: dma16<2 * 128>(row, lds_block + 2 * (kBlockBytes - 128)); break;
    case 3: dma16<3 * 128>(row, lds_block + 3 * (kBlockBytes - 128)); break;
    case 4: dma16<4 * 128>(row, lds_block + 4 * (kBlockBytes - 128)); break;
    case 5: dma16<5 * 128>(row, lds_block + 5 * (kBlockBytes - 128)); break;
    case 6: dma16<6 * 128>(row, lds_block + 6 * (kBlockBytes - 128)); break;
    case 7: dma16<7 * 128>(row, lds_block + 7 * (kBlockBytes - 128)); break;
    default: dma16<8 * 128>(row, lds_block + 8 * (kBlockBytes - 128)); break;
  }
}
__device__ __forceinline__ void dma_key_block(const char* row, uint32_t lds_block) {
  dma16<0 * 128>(row, lds_block + 0 * (kBlockBytes - 128));
  dma16<1 * 128>(row, lds_block + 1 * (kBlockBytes - 128));
  dma16<2 * 128>(row, lds_block + 2 * (kBlockBytes - 128));
  dma16<3 * 128>(row, lds_block + 3 * (kBlockBytes - 128));
  dma16<4 * 128>(row, lds_block + 4 * (kBlockBytes - 128));
  dma16<5 * 128>(row, lds_block + 5 * (kBlockBytes - 128));
  dma16<6 * 128>(row, lds_block + 6 * (kBlockBytes - 128));
  dma16<7 * 128>(row, lds_block + 7 * (kBlockBytes - 128));
  dma16<8 * 128>(row, lds_block + 8 * (kBlockBytes - 128));
}

// s_waitcnt vmcnt(n) with lgkmcnt/expcnt left alone.  gfx9 encoding: vmcnt[3:0] in
// bits 3:0, vmcnt[5:4] in bits 15:14, expcnt in 6:4, lgkmcnt in 11:8.
#define MLAV_WAIT_VMCNT(n)                                                                   \
  do {                                                                                       \
    static_assert((n) >= 0 && (n) < 64, "vmcnt is a 6-bit field");                          \
    __builtin_amdgcn_s_waitcnt(((n) & 0xF) | ((((n) >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8)); \
  } while (0)

// A load whose completion the compiler does not track (the prologue's slot indices).  The
// compiler counts only its own loads in the vmcnt waits it inserts, not the direct-to-LDS loads
// above, so a compiler-issued load followed by gathers would be awaited together with them.
// The loaded register is awaited explicitly by an asm s_waitcnt that names it as an in/out
// operand: every later use reads the wait's output, so none can be placed before it.
// tests/test_kernel_hazards.py checks the generated code: no instruction touches a register
// loaded here before a vmcnt wait that covers its load.
__device__ __forceinline__ int load_b32_untracked(const int32_t* p) {
  int v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p) : "memory");
  return v;
}

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
__device__ __forceinline__ bool decode_work(const PartialArgs& p, int wg, int rows_per_group, WorkItem& wi) {
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
  wi.L = read_len(p.seq_lens, wi.b, p.debug_flags);
  wi.Q = clamped_q(p.q_lens, p.seq_lens, wi.b, p.max_q_len, p.debug_flags);
  wi.R = wi.Q * p.heads;
  if (wi.Q <= 0 || wi.g * rows_per_group >= wi.R) return false;
  const int ns = split_count(wi.L, p.nsplit, p.min_tiles);
  if (wi.s >= ns) return false;
  const int tiles = (wi.L + kTileKeys - 1) / kTileKeys;
  wi.t_begin = (int)((int64_t)wi.s * tiles / ns);
  wi.t_end = (int)((int64_t)(wi.s + 1) * tiles / ns);
  int64_t ko = 0, qo = 0;
  for (int i = 0; i < wi.b; ++i) {
    ko += read_len(p.seq_lens, i, p.debug_flags);
    qo += clamped_q(p.q_lens, p.seq_lens, i, p.max_q_len, p.debug_flags);
  }
  wi.ko = ko;
  wi.qo = qo;
  return true;
}

// ---- Range plan for a batch of requests (2 .. kRangeMaxBatch requests) ------------------------------
// Splitting a ragged batch per request gives every request the same number of splits: a short
// request's workgroups finish early, a long one's late, and every split pays the fixed cost of
// staging q and writing a partial.  The range plan instead lays the 32-key tiles of all requests, in
// request order, out as one sequence of T tiles (a request without rows contributes none) and cuts
// it into chunks of C consecutive tiles, one per worker (a worker is one workgroup per 128-row
// group).  A chunk may end inside a request and carry on into the next ones: it holds one piece per
// request it touches, and each piece is one workgroup.  A request's partial s is its piece of chunk
// floor(J_b / C) + s (J_b: the request's first tile in the sequence), so every partial covers a
// contiguous key range.  C starts from an even share of T per worker and is raised only as far as
// needed to keep every request within nsplit chunks.
//
// Dispatch order does the balancing: the workers of XCD x are those with o = x (mod 8), and the
// workgroups of XCD x run its pieces in rounds, round k holding the k-th largest piece of each of
// its chunks; so every CU starts on the largest piece of a chunk, and the smaller pieces go to
// whichever CUs free up first.  The grid is sized for the most pieces a batch can have; workgroups
// past the actual pieces exit after the decode.  Kernel 1 and the merge both derive the plan from
// seq_lens and q_lens on the device, so it needs no host step and the call stays capture-safe.
// Tile counts are 32-bit: T stays below 2^31 for any batch whose slot list fits in memory.

struct RequestScan {  // lane b < batch holds request b; lanes past the batch hold zeros
  int L, Q, tiles;    // keys, clamped draft tokens, tiles with work (0 when the request has no rows)
  int J;              // first tile of the request in the batch's tile sequence
  int qo;             // first (draft token) row of the request: prefix sum of the clamped q_lens
  int64_t ko;         // first key of the request in slot_idx: prefix sum of seq_lens
};

__device__ __forceinline__ int wave_excl_scan(int v, int lane) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x - v;
}

__device__ __forceinline__ RequestScan scan_requests(const int32_t* seq_lens, const int32_t* q_lens, int batch,
                                                     int max_q, int32_t* flags) {
  const int lane = threadIdx.x & 63;
  RequestScan r;
  r.L = lane < batch ? read_len(seq_lens, lane, flags) : 0;
  r.Q = lane < batch ? clamped_q(q_lens, seq_lens, lane, max_q, flags) : 0;
  r.tiles = r.Q > 0 ? (r.L + kTileKeys - 1) / kTileKeys : 0;
  r.J = wave_excl_scan(r.tiles, lane);
  r.qo = wave_excl_scan(r.Q, lane);
  int64_t x = r.L;  // 64-bit prefix of seq_lens
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  r.ko = x - r.L;
  return r;
}

// Does every request lie within nsplit chunks of C tiles?
__device__ __forceinline__ bool chunks_fit(const RequestScan& r, int C, int nsplit) {
  const bool ok = r.tiles == 0 || (r.J + r.tiles - 1) / C - r.J / C + 1 <= nsplit;
  return __all(ok) != 0;
}

// The chunk length C (tiles per worker); the same value in every lane and every workgroup.
__device__ __forceinline__ int range_chunk(const RequestScan& r, int nsplit, int workers, int min_tiles) {
  const int T = __builtin_amdgcn_readlane(r.J + r.tiles, 63);
  if (T <= 0) return 1;
  int C = (T + workers - 1) / workers;
  if (C < min_tiles) C = min_tiles;
  if (chunks_fit(r, C, nsplit)) return C;
  int maxt = r.tiles;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) maxt = max(maxt, __shfl_xor(maxt, o));
  const int C1 = (maxt + nsplit - 1) / nsplit;  // the fewest tiles per chunk for the longest request
  if (C1 > C) {
    C = C1;
    if (chunks_fit(r, C, nsplit)) return C;
  }
  // A request of t tiles meets at most floor((t - 1) / C) + 2 chunks, so this always fits;
  // with one split per request, one chunk holds the whole batch.
  if (nsplit < 2) return T;
  const int C2 = (maxt + nsplit - 2) / (nsplit - 1);
  return C2 > C ? C2 : C;
}

// Requests (lanes) with tiles in chunk [lo, hi).
__device__ __forceinline__ uint64_t chunk_requests(const RequestScan& r, int lo, int hi) {
  return __ballot(r.tiles > 0 && r.J < hi && r.J + r.tiles > lo);
}

// Grid of the range plan: per pool (XCD), room for every worker's first piece plus one piece per
// request boundary, times the row groups.
__host__ __device__ __forceinline__ int range_pools(int workers) { return (workers & 7) == 0 ? 8 : 1; }
__host__ __device__ __forceinline__ int64_t range_grid(int workers, int row_groups, int batch) {
  const int pools = range_pools(workers);
  return (int64_t)pools * (workers / pools + batch - 1) * row_groups;
}

// Decode a workgroup id of the range plan; false if it has nothing to do.
__device__ __forceinline__ bool decode_piece(const PartialArgs& p, int wg, WorkItem& wi) {
  const int lane = threadIdx.x & 63;
  const RequestScan r = scan_requests(p.seq_lens, p.q_lens, p.batch, p.max_q_len, p.debug_flags);
  const int C = __builtin_amdgcn_readfirstlane(range_chunk(r, p.nsplit, p.workers, p.min_tiles));
  const int T = __builtin_amdgcn_readlane(r.J + r.tiles, 63);
  const int pools = range_pools(p.workers), per_pool = p.workers / pools;
  const int x = pools == 8 ? (wg & 7) : 0, kk = pools == 8 ? (wg >> 3) : wg;
  int j = kk / p.row_groups;
  const int g = kk - j * p.row_groups;
  // pieces of each of the pool's workers (worker x + pools*i in lane i; at most 64 workers per pool,
  // which the worker count chosen at create guarantees)
  int npieces = 0;
  for (int i = 0; i < per_pool; ++i) {
    const int o = x + pools * i;
    if ((int64_t)o * C >= T) break;
    const int lo = o * C, hi = lo + (C < T - lo ? C : T - lo);
    const int n = __popcll(chunk_requests(r, lo, hi));
    if (lane == i) npieces = n;
  }
  // round k holds the k-th largest piece of each chunk with more than k pieces, workers in order
  int o = -1, k = 0;
  for (;; ++k) {
    const uint64_t has = __ballot(lane < per_pool && npieces > k);
    if (has == 0) return false;
    const int cnt = __popcll(has);
    if (j < cnt) {
      uint64_t m = has;
      for (int t = 0; t < j; ++t) m &= m - 1;
      o = x + pools * __builtin_ctzll(m);
      break;
    }
    j -= cnt;
  }
  const int lo = o * C, hi = lo + (C < T - lo ? C : T - lo);
  const uint64_t reqs = chunk_requests(r, lo, hi);
  // the k-th largest piece of the chunk (ties in request order)
  const int size = min(hi, r.J + r.tiles) - max(lo, r.J);
  int rank = 0;
  for (uint64_t m = reqs; m != 0; m &= m - 1) {
    const int b2 = __builtin_ctzll(m);
    const int s2 = __builtin_amdgcn_readlane(size, b2);
    rank += (s2 > size || (s2 == size && b2 < lane)) ? 1 : 0;
  }
  const uint64_t pick = __ballot(((reqs >> lane) & 1) != 0 && rank == k);
  const int b = __builtin_ctzll(pick);
  wi.b = b;
  wi.g = g;
  wi.L = __builtin_amdgcn_readlane(r.L, b);
  wi.Q = __builtin_amdgcn_readlane(r.Q, b);
  wi.R = wi.Q * p.heads;
  if (g * kRowsPerGroup >= wi.R) return false;
  const int J = __builtin_amdgcn_readlane(r.J, b);
  const int tiles = __builtin_amdgcn_readlane(r.tiles, b);
  wi.s = o - J / C;
  wi.bs = b * p.nsplit + wi.s;
  wi.t_begin = (lo > J ? lo : J) - J;
  wi.t_end = (hi < J + tiles ? hi : J + tiles) - J;
  wi.qo = __builtin_amdgcn_readlane(r.qo, b);
  const uint32_t ko_lo = __builtin_amdgcn_readlane((int)(uint32_t)r.ko, b);
  const uint32_t ko_hi = __builtin_amdgcn_readlane((int)(r.ko >> 32), b);
  wi.ko = (int64_t)(((uint64_t)ko_hi << 32) | ko_lo);
  return true;
}

// Exact recomputation of rows whose fixed-reference row sum reached
// kRowSumLimit (scores far above the max of the split's first tile): one row at
// a time across the whole wave, with a running max and a rescale at every key,
// in fp32.  Overwrites the row's partial.  Only reached for such rows, so its
// speed does not matter.
// The partial's keys are the split's tiles tile_first, tile_first + tile_step, ...; it is stored as
// partial `part` (rows_pad rows each).
__device__ __forceinline__ void redo_rows_exact(const PartialArgs& p, const WorkItem& wi, int row_base, uint32_t rows,
                                                int tile_first, int tile_step, int64_t part) {
  const int lane = threadIdx.x & 63;
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
    for (int key = (wi.t_begin + tile_first) * kTileKeys; key < kend;
         key += (key + 1) % kTileKeys == 0 ? 1 + (tile_step - 1) * kTileKeys : 1) {  // skip the other stream's tiles
      const uint16_t* krow = p.kv + (int64_t)checked_slot(slots[key], p.num_slots, p.debug_flags) * kDqk;
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
    const int64_t prow = part * p.rows_pad + row;
    f16x8 ov;
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = (_Float16)(acc[j] * inv);
    *((f16x8*)(p.o_part + prow * kDv) + lane) = ov;
    if (lane == 0) p.lse_part[prow] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  }
}

// Per-row softmax state of one lane (row lrow; the lane pair l, l^32 agrees on
// m_ref and holds half of each row sum).
struct RowSoftmax {
  float m_ref;    // reference (log2 units): the row max of the split's first tile + kRefHeadroom; -inf if none is visible
  float l_run;    // this lane's share of the row sum of bf16-rounded P (normalises O)
  float l_exact;  // ... and of P before rounding (gives the LSE)
};

// p = 2^(x - m_ref) is used as is, with no rescale, as long as the row sums stay below 2^96:
// then every p is below 2^96 and, over at most 2^31 keys, neither the sums nor the output
// accumulators (|v| < 2^31) can overflow fp32.  A row whose sum reaches it (including +inf from
// an overflowing exp2) is redone exactly.
//
// The reference sits kRefHeadroom = 64 binades above the first tile's row max.  fp32 and bf16
// keep their relative precision from 2^-126 up, so scaling every p (and both row sums) by
// exactly 2^-64 changes no rounding, while a key may now score up to about 64 + 96 - log2(keys
// in the split) binades above the first tile's max (about 100 nats at 2,048 keys) before the
// sums reach the limit, instead of 64 - log2(keys).  The price is at the bottom: a p below
// 2^-126 is flushed, i.e. a key more than 62 binades below the first tile's max, whose weight
// next to that max key (which is in the same sum) is below 2^-62 -- far under fp32 precision.
constexpr float kRowSumLimit = 79228162514264337593543950336.0f;  // 2^96
constexpr float kRefHeadroom = 64.0f;

// Row max of a tile's raw scores: 16 values per lane, then the lane pair.
__device__ __forceinline__ float tile_row_max(const f32x16& s) {
  float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]);
  float m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
  float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]);
  m0 = fmaxf(fmaxf(m0, s[9]), s[10]);
  m1 = fmaxf(fmaxf(m1, s[11]), s[12]);
  m2 = fmaxf(fmaxf(m2, s[13]), s[14]);
  m0 = fmaxf(fmaxf(m0, m1), fmaxf(m2, s[15]));
  return pair_max(m0);
}

// Softmax of one tile.  First x_k = s_k * scale - m_ref for all 16 scores of the
// lane (scale_scores, 16 FMAs), issued while the first K reads of the next tile
// are in flight; they move the scores out of the registers the next tile's Q.K
// accumulates into, so no copy of them is needed.  Then, with one wave per SIMD
// an MFMA hides a few independent VALU ops of the same wave but not a long block
// of them, so the rest is spread thin between the Q.K MFMAs of the next tile
// (softmax_slot, slot k):
//   p_k = 2^(x_k)                                   (k < 16)
//   for even k >= 2: bf16 pack of (p_{k-2}, p_{k-1})  (both made in earlier slots)
// and the row sums sit between the P.V MFMAs of the same tile (sum_slot):
//   exact sum += p_n; for odd n, rounded sum += the packed pair.
// The causal mask is applied to the raw scores beforehand, on the tiles that
// reach the draft block only.
constexpr int kSoftmaxSlots = 17;
struct SoftmaxTile {
  f32x16 s;       // raw scores -> 2^(s*scale - m_ref)
  int pw[8];      // bf16 pairs; pw[0..3], pw[4..7] are the MFMA B operands of the two 16-key steps
                  // (kept as separate scalars: element inserts into a vector here were miscompiled)
  __device__ i32x4 operand(int kk) const { return (i32x4){pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]}; }
};

__device__ __forceinline__ void scale_scores(SoftmaxTile& t, const f32x16& raw, float nmref, float scale_log2) {
#pragma unroll
  for (int k = 0; k < 16; ++k) t.s[k] = vfma(raw[k], scale_log2, nmref);
}

__device__ __forceinline__ void softmax_slot(int k, SoftmaxTile& t) {
  if (k < 16) t.s[k] = vexp2(t.s[k]);
  if (k >= 2 && !(k & 1)) t.pw[(k - 2) >> 1] = vpack_bf16(t.s[k - 2], t.s[k - 1]);
}

__device__ __forceinline__ void sum_slot(int n, const SoftmaxTile& t, RowSoftmax& st) {
  vadd_to(st.l_exact, t.s[n]);
  if (n & 1) vsum_pair_to(st.l_run, t.pw[n >> 1]);
}

// Causal mask on the raw scores of a tile that reaches the draft block:
// lane holds keys key0 + 8*(j>>2) + (j&3) (key0 includes 4*hi); keys >= limit get -inf.
__device__ __forceinline__ void mask_tile(f32x16& s, int key0, int limit) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int key = key0 + 8 * (j >> 2) + (j & 3);
    s[j] = key < limit ? s[j] : -INFINITY;
  }
}

}  // namespace

// Kernel 1's work on one item: request wi.b, its tiles [t_begin, t_end), the rows of group wi.g;
// writes partial wi.bs of those rows.
__device__ __forceinline__ void partial_item(const PartialArgs& p, const WorkItem& wi) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRing * kTileBytes + kXchgBytes];
  lds_char* smem = (lds_char*)smem_raw;
  lds_char* xchg = smem + kRing * kTileBytes;  // [2][kWaves][2 KiB]: bf16 P of each wave, double-buffered

  const int L = wi.L, Q = wi.Q, H = p.heads, R = wi.R;
  const int ntiles = wi.t_end - wi.t_begin;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, lrow = lane & 31;
  const int half = w & 1;   // this wave computes output columns [256*half, 256*half + 256)
  const int partner = w ^ 1;
  const int row0 = wi.g * kRowsPerGroup;
  const int myrow = row0 + w * kRowsPerWave + lrow;        // own (token, head) row in the request
  const int parrow = row0 + partner * kRowsPerWave + lrow; // the partner wave's row in this lane
  const bool row_valid = myrow < R;
  const int tok = row_valid ? myrow / H : 0;
  const int limit = L - Q + tok + 1;  // this row sees keys [0, limit)
  const int mask_from = L - Q + 1;    // first key some draft row cannot see

  // ---- gather set-up: wave w moves keys 8w..8w+7 of every tile --------------------------------
  const int g_kr = lane >> 3;                             // key within the wave's 8-key block
  const int g_byte = ((lane & 7) ^ g_kr ^ (w & 1)) << 4;  // 16-B chunk of the 128-B line
  const char* kv = (const char*)p.kv;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const int w_uniform = __builtin_amdgcn_readfirstlane(w);
  // Slot index of the row this lane gathers in tile i of the split: key 8w + g_kr of the tile.
  // The prologue's gathers past a short split repeat its last tile (the buffer is never read),
  // and keys past the request's end use its last key's row (scores masked).
  const int32_t* slots_g = p.slot_idx + wi.ko;
  auto gather_key = [&](int i) {
    int key = (wi.t_begin + (i < ntiles ? i : ntiles - 1)) * kTileKeys + w * 8 + g_kr;
    return key < L ? key : L - 1;
  };
  auto issue_tile = [&](int buf, int slot) {
    const uint32_t base = smem_base + buf * kTileBytes + w_uniform * kKeyBlockBytes;
    dma_key_block(kv + (int64_t)slot * kRowBytes + g_byte, base);
  };

  // Q.K A operand: lane reads key lrow, 16-B chunk 2*ks + hi (relative to a tile buffer).
  int kaddr[4];
  {
    const int kr = lrow & 7, f = kr ^ ((lrow >> 3) & 1);
    const int base = (lrow >> 3) * kKeyBlockBytes + kr * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) kaddr[j] = base + (((2 * j) ^ hi ^ f) << 4);
  }

  // ---- prologue: slot indices, the q rows, then the first gathers --------------------------------
  // The slot indices of the first kAhead tiles are loaded first (untracked by the compiler,
  // awaited below).  The first kAhead tiles are always gathered (past a short split they repeat
  // its last tile into buffers that are never read), so the waits have fixed counts.
  static_assert(kAhead == 3, "the prologue loads three slot indices and gathers three tiles");
  int sl[kAhead];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) sl[i] = load_b32_untracked(slots_g + gather_key(i));

  // The wave's 32 query rows, resident in registers for the whole split: lane holds row lrow,
  // dims 16*ks + 8*hi .. +7 (MFMA B-operand layout).  Loads straight into that layout would make
  // every load touch 32 rows (32 partial 128-B lines), which costs microseconds of address
  // processing per workgroup; so wave w moves its rows into block w of the ring buffers in the
  // key-tile layout (row r of the wave as key r of block w of buffer r/8; 8 whole lines per load)
  // and reads them back with the Q.K read pattern.  A row past the request reads the request's first row instead: its scores are finite
  // and its output is never stored.
  {
    const uint32_t qbuf = smem_base + w_uniform * kKeyBlockBytes;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int r = row0 + w * kRowsPerWave + 8 * kb + g_kr;
      const int64_t qrow = wi.qo * H + (r < R ? r : 0);
      dma_key_block((const char*)(p.q + qrow * kDqk) + (((lane & 7) ^ g_kr ^ (kb & 1)) << 4), qbuf + kb * kTileBytes);
    }
  }
  // slot indices and q rows have landed; the memory clobber keeps the LDS reads below after it
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(sl[0]), "+v"(sl[1]), "+v"(sl[2]) : : "memory");
#pragma unroll
  for (int i = 0; i < kAhead; ++i) sl[i] = checked_slot(sl[i], p.num_slots, p.debug_flags);
  bf16x8 qf[kQkSteps];
  {
    // q row lrow of the wave sits in buffer lrow/8, block w: kaddr's key-block offset replaced
    const lds_char* qb = smem + w * kKeyBlockBytes + (lrow >> 3) * (kTileBytes - kKeyBlockBytes);
#pragma unroll
    for (int ks = 0; ks < kQkSteps; ++ks)
      qf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(qb + kaddr[ks & 3] + (ks >> 2) * kBlockBytes);
  }
  // Block w of every buffer held this wave's q rows only, so once its own reads are done the wave
  // gathers its eight keys of tile 0 into block w of buffer 0 without waiting for the other waves;
  // tiles 1 and 2 go between the Q.K MFMAs of tile 0 (each gather load takes the address unit for
  // a while, so issuing all three here would delay the first Q.K).
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  issue_tile(0, sl[0]);

  // ---- per-lane LDS read addresses for P.V (relative to a tile buffer) --------------------------
  // P.V A operand via the 4x16 transposing read: in 16-lane group G, lane j reads key
  // 16*kk + 8*r + 4*(G>>1) + (j>>2) at columns 32*cb + 16*(G&1) + 4*(j&3) .. +3; lane l then
  // holds column 32*cb + (l&31) for keys 16*kk + 8*r + 4*(l>>5) .. +3.  This wave's column
  // blocks are cb = 8*half + cbl; the half offset is folded into the base.
  int vaddr[2][2];
  {
    const int G = lane >> 4, j = lane & 15;
    const int kr = 4 * (G >> 1) + (j >> 2);
    const int u = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vaddr[e][r] = half * 4 * kBlockBytes + r * kKeyBlockBytes + kr * 128 + (((4 * e) ^ u ^ kr ^ r) << 4) +
                      (j & 1) * 8;
  }

  // O^T accumulators: columns [256*half, +256) for the wave's own 32 rows and the partner's 32 rows
  f32x16 o_own[kHalfColBlocks], o_par[kHalfColBlocks];
#pragma unroll
  for (int c = 0; c < kHalfColBlocks; ++c) {
    o_own[c] = (f32x16){};
    o_par[c] = (f32x16){};
  }
  // Softmax with a fixed per-row reference: m_ref is the row max of the split's
  // first tile plus kRefHeadroom (set after its Q.K below); p = 2^(x - m_ref) needs no rescale
  // while the row sum stays below kRowSumLimit.  A row that reaches it is
  // recomputed exactly at the end (redo_rows_exact).
  RowSoftmax st{-INFINITY, 0.f, 0.f};

  bf16x8 kf[kQkSteps];
  auto kread = [&](const lds_char* tb, int ks) {
    kf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(tb + kaddr[ks & 3] + (ks >> 2) * kBlockBytes);
  };

  // tile 0 published, Q.K of tile 0 with the gathers of tiles 1 and 2 between its MFMAs; then
  // tile 1 published for the first step
  MLAV_WAIT_VMCNT(0);  // tile 0 has arrived (nothing else is in flight)
  __syncthreads();
  const char* g_row1 = kv + (int64_t)sl[1] * kRowBytes + g_byte;
  const char* g_row2 = kv + (int64_t)sl[2] * kRowBytes + g_byte;
  const uint32_t g_lds1 = smem_base + 1 * kTileBytes + w_uniform * kKeyBlockBytes;
  const uint32_t g_lds2 = smem_base + 2 * kTileBytes + w_uniform * kKeyBlockBytes;
  static_assert(2 * 2 * kDmaPerTile <= kQkSteps, "two tiles of gathers fit in one Q.K, one per two MFMAs");
  f32x16 sacc;
#pragma unroll
  for (int ks = 0; ks < kPrefetch; ++ks) kread(smem, ks);
#pragma unroll
  for (int ks = 0; ks < kQkSteps; ++ks) {
    __builtin_amdgcn_sched_barrier(0);
    if (ks + kPrefetch < kQkSteps) kread(smem, ks + kPrefetch);
    __builtin_amdgcn_sched_barrier(0);
    if (ks == 0) mfma_first_v(sacc, kf[ks], qf[ks]);
    else mfma_acc_v(sacc, kf[ks], qf[ks]);
    __builtin_amdgcn_sched_barrier(0);
    if (!(ks & 1) && (ks >> 1) < 2 * kDmaPerTile) {
      const int j = ks >> 1;
      if (j < kDmaPerTile) dma_chunk_group(g_row1, g_lds1, j);
      else dma_chunk_group(g_row2, g_lds2, j - kDmaPerTile);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // The reference: the first tile's row max (masked).  If the row sees no key of
  // that tile it sees none of the split (later tiles hold later keys): m_ref
  // stays -inf, every p is 2^-inf = 0 and the partial is empty.
  float nmref;
  {
    asm volatile(MLAV_MFMA_DRAIN : "+v"(sacc));
    f32x16 s0 = sacc;
    if (wi.t_begin * kTileKeys + kTileKeys > mask_from) mask_tile(s0, wi.t_begin * kTileKeys + 4 * hi, limit);
    // (the scale is positive, so it commutes with the max; -inf stays -inf)
    st.m_ref = tile_row_max(s0) * p.scale_log2 + kRefHeadroom;
    nmref = (st.m_ref == -INFINITY) ? 0.f : -st.m_ref;
  }
  if (ntiles > 1) {
    MLAV_WAIT_VMCNT(kDmaPerTile);  // tile 1 has arrived
    __syncthreads();
  }
  // the first K fragments of tile 1 for the first step's Q.K (unused when there is no tile 1)
#pragma unroll
  for (int ks = 0; ks < kPrefetch; ++ks) kread(smem + kTileBytes, ks);
  // V^T fragment n of a tile: local column block n%8, 16-key step n/8.
  bf16x8 vf[kPvFrags];
  auto vread = [&](const lds_char* tb, int n) {
    const int cbl = n & (kHalfColBlocks - 1), kk = n >> 3;
    const lds_char* vb = tb + (cbl >> 1) * kBlockBytes + kk * 2 * kKeyBlockBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[cbl & 1][0]));
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[cbl & 1][1]));
    vf[n] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // One step; `refill` (a compile-time flag) says whether it gathers tile i+3, which the
  // last kAhead steps of a split do not: the loop runs in two parts, each with its own copy
  // of the step, so there is no branch inside a step.
  auto step = [&](const int i, auto refill) __attribute__((always_inline)) {
    constexpr bool kRefill = decltype(refill)::value;
    const int t = wi.t_begin + i;
    const lds_char* tb = smem + (i & (kRing - 1)) * kTileBytes;
    const int key0 = t * kTileKeys + 4 * hi;
    // Slot of the row this lane gathers for tile i+3, loaded now and awaited with the tile
    // loads before the barrier below.
    const int g_slot = kRefill ? checked_slot(slots_g[gather_key(i + kAhead)], p.num_slots, p.debug_flags) : 0;
    // (no drain: the last MFMA that wrote sacc is a whole P.V phase back)
    SoftmaxTile sm;
    if (t * kTileKeys + kTileKeys > mask_from) mask_tile(sacc, key0, limit);

    // this wave's P (B-operand layout) for its partner, written as soon as the last pair is packed
    lds_char* xw = xchg + (i & 1) * (kWaves * 2048) + w * 2048 + lane * 16;
    auto publish_p = [&]() {
      *(__attribute__((address_space(3))) i32x4*)(xw) = sm.operand(0);
      *(__attribute__((address_space(3))) i32x4*)(xw + 1024) = sm.operand(1);
    };

    // ---- phase A: Q.K of tile i+1 with the softmax of tile i between its MFMAs ----
    if (i + 1 < ntiles) {
      const lds_char* nb = smem + ((i + 1) & (kRing - 1)) * kTileBytes;
      f32x16 snext;
      // kf[0 .. kPrefetch) of this tile were read during the previous P.V phase
      __builtin_amdgcn_sched_barrier(0);
      scale_scores(sm, sacc, nmref, p.scale_log2);
#pragma unroll
      for (int ks = 0; ks < kQkSteps; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks + kPrefetch < kQkSteps) kread(nb, ks + kPrefetch);
        // the first V^T fragments of tile i, for the P.V phase after the barrier
        if (ks >= kQkSteps - kVPrefetch) vread(tb, ks - (kQkSteps - kVPrefetch));
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0) mfma_first_v(snext, kf[ks], qf[ks]);
        else mfma_acc_v(snext, kf[ks], qf[ks]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks < kSoftmaxSlots) softmax_slot(ks, sm);
        if (ks == kSoftmaxSlots) publish_p();
      }
      __builtin_amdgcn_sched_barrier(0);
      sacc = snext;
    } else {
      scale_scores(sm, sacc, nmref, p.scale_log2);
#pragma unroll
      for (int slot = 0; slot < kSoftmaxSlots; ++slot) softmax_slot(slot, sm);
      publish_p();
#pragma unroll
      for (int n = 0; n < kVPrefetch; ++n) vread(tb, n);
    }

    // tile i+2 complete and every wave's P written, then publish
    MLAV_WAIT_VMCNT(0);
    __syncthreads();

    // ---- phase B: P.V of tile i for the pair's 64 rows x this wave's 256 columns;
    //      the nine loads that refill the ring with tile i+3 (into the buffer of tile
    //      i-1, which every wave has finished) go between its MFMAs ----
    const bf16x8 pown[2] = {__builtin_bit_cast(bf16x8, sm.operand(0)), __builtin_bit_cast(bf16x8, sm.operand(1))};
    bf16x8 ppar[2];
    {
      const lds_char* xp = xchg + (i & 1) * (kWaves * 2048) + partner * 2048 + lane * 16;
      ppar[0] = *(const __attribute__((address_space(3))) bf16x8*)(xp);
      ppar[1] = *(const __attribute__((address_space(3))) bf16x8*)(xp + 1024);
    }
    const char* g_row = kv + (int64_t)g_slot * kRowBytes + g_byte;
    const uint32_t g_lds = smem_base + ((i + kAhead) & (kRing - 1)) * kTileBytes + w_uniform * kKeyBlockBytes;
    // tile i+2 (complete since the barrier above) is the next Q.K's: its first K fragments
    // are read in the last slots of this phase
    const lds_char* nb2 = smem + ((i + 2) & (kRing - 1)) * kTileBytes;
#pragma unroll
    for (int n = 0; n < kPvFrags; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      if (n + kVPrefetch < kPvFrags) vread(tb, n + kVPrefetch);
      if (n >= kPvFrags - kPrefetch) kread(nb2, n - (kPvFrags - kPrefetch));
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc_a(o_own[n & (kHalfColBlocks - 1)], vf[n], pown[n >> 3]);
      __builtin_amdgcn_sched_barrier(0);
      sum_slot(n, sm, st);
      if (kRefill && n < kDmaPerTile) dma_chunk_group(g_row, g_lds, n);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc_a(o_par[n & (kHalfColBlocks - 1)], vf[n], ppar[n >> 3]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int i = 0;
  for (; i < ntiles - kAhead; ++i) step(i, std::true_type{});
  for (; i < ntiles; ++i) step(i, std::false_type{});
  MLAV_WAIT_VMCNT(0);
  // The accumulators are read below only through acc_read (volatile), which stays behind this
  // drain.  It names no registers: tied operands here made the compiler move accumulators
  // between registers ahead of it.
  asm volatile(MLAV_MFMA_DRAIN);

  // ---- partial write: o_s = O / l (fp16), lse_s = ln2 * (m_ref + log2 l) -----------------------
  // The row sums live with the row's owner wave; swap them through LDS, together with
  // whether any row of the workgroup needs the exact redo.
  const float lt = pair_sum(st.l_run);
  const float le = pair_sum(st.l_exact);
  const bool overflow = !(le < kRowSumLimit);  // the row sum reached 2^96, or an exp2 overflowed to +inf
  const uint64_t redo = __ballot(overflow && hi == 0 && row_valid);
  __syncthreads();  // every wave is done with the ring and the P exchange buffers
  float* lsum = (float*)(smem_raw + kRing * kTileBytes);
  int* redo_flag = (int*)(lsum + kRowsPerGroup);
  if (hi == 0) lsum[w * 32 + lrow] = lt;
  if (lane == 0) redo_flag[w] = redo != 0;
  __syncthreads();
  const float lt_par = lsum[partner * 32 + lrow];
  const bool any_redo = (redo_flag[0] | redo_flag[1] | redo_flag[2] | redo_flag[3]) != 0;
  const float inv_own = lt > 0.f ? 1.0f / lt : 0.f;
  const float inv_par = lt_par > 0.f ? 1.0f / lt_par : 0.f;
  if (row_valid && hi == 0)
    // (le > 0 only if the reference is finite, and then m_ref = -nmref: one register less to keep)
    p.lse_part[(int64_t)wi.bs * p.rows_pad + myrow] = le > 0.f ? (__builtin_amdgcn_logf(le) - nmref) * kLn2 : -INFINITY;

  // The wave's 64 rows x 256 columns go through the free ring as fp16 rows (stride
  // kStageRowBytes, padded against bank conflicts), then out as whole 512-B row halves, two rows
  // per store instruction.  In the C layout the lane holds, per 32-column block c, columns
  // 32c + 8*q4 + 4*hi .. +3.  The wave's own rows (stage rows 0..31) are staged first and
  // stored while its partner's rows (stage rows 32..63) are converted, so the stores drain
  // under the conversion work.  Each half goes out as 16 LDS reads, one wait, then 16 stores:
  // a read, wait and store per row pair costs an LDS round trip per store (about 2 us a
  // workgroup).
  lds_char* stage = smem + w * kStageBytes;
  auto stage_block = [&](const f32x16& o, float inv, int row, int c, int q4) {
    const int cb = (32 * c + 8 * q4 + 4 * hi) * 2;
    const f16x4 v = {(_Float16)(acc_read(o[4 * q4]) * inv), (_Float16)(acc_read(o[4 * q4 + 1]) * inv),
                     (_Float16)(acc_read(o[4 * q4 + 2]) * inv), (_Float16)(acc_read(o[4 * q4 + 3]) * inv)};
    *(__attribute__((address_space(3))) f16x4*)(stage + row * kStageRowBytes + cb) = v;
  };
  // (the column half from the wave index in a scalar register: keeping `half` live this long spilled it)
  uint16_t* part_base = p.o_part + (int64_t)wi.bs * p.rows_pad * kDv + (w_uniform & 1) * (kDv / 2) + (lane & 31) * 8;
  // `between(k)` runs after the k-th store: the stores of the own rows go out between the
  // conversions of the partner's rows (the CU's store path and the VALU then work at once;
  // one after the other, the conversion and the store issue each took about 1 us).
  // (a row group with all 128 rows valid, as in every group of a request with a multiple of 128 rows,
  // stores without a per-row check, from one base address per two rows)
  const bool full_group = row0 + kRowsPerGroup <= R;
  auto store_half = [&](const int r0, const int grow0, auto between) {  // stage rows r0 .. r0+31 = rows grow0 ..
    i32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = *(const __attribute__((address_space(3))) i32x4*)(stage + (r0 + 2 * k + hi) * kStageRowBytes + (lane & 31) * 16);
    __builtin_amdgcn_sched_barrier(0);
    // (written through: the merge reads the partials from another XCD, not from this L2)
    if (full_group) {
      char* rowp = (char*)(part_base + (int64_t)(grow0 + hi) * kDv);
#pragma unroll
      for (int k = 0; k < 16; ++k) {  // row grow0 + 2k + hi: (k / 2) * 4 KiB + (k % 2) * 2 KiB from rowp
        if (k & 1) store16_through_at<2 * kDv * 2>(rowp + (k >> 1) * 4 * kDv * 2, v[k]);
        else store16_through_at<0>(rowp + (k >> 1) * 4 * kDv * 2, v[k]);
        between(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int grow = grow0 + 2 * k + hi;
        if (grow < R) store16_through(part_base + (int64_t)grow * kDv, v[k]);
        between(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
#pragma unroll
  for (int c = 0; c < kHalfColBlocks; ++c)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) stage_block(o_own[c], inv_own, lrow, c, q4);
  store_half(0, row0 + w * kRowsPerWave, [&](int k) {  // two of the 32 partner blocks per store
#pragma unroll
    for (int b = 2 * k; b < 2 * k + 2; ++b) stage_block(o_par[b >> 2], inv_par, 32 + lrow, b >> 2, b & 3);
  });
  store_half(32, row0 + partner * kRowsPerWave, [](int) {});

  // Rows whose sums outgrew the fixed reference are redone exactly by their owner wave,
  // once both halves of the row have been written.
  if (any_redo) {
    __syncthreads();  // (global writes of both halves are ordered by the barrier's release/acquire)
    if (redo != 0) redo_rows_exact(p, wi, row0 + w * kRowsPerWave, (uint32_t)redo, 0, 1, wi.bs);
  }
}

// Kernel 1, 128-row form.  kRanges = false: one workgroup per (request, split, row group), splits
// of equal length per request.  kRanges = true: the range plan above, one workgroup per (piece,
// row group).
// The arguments the workgroup's first loads depend on come first and separately (the lengths'
// addresses and the sizes the work decode reads): the build preloads the leading kernel arguments
// into scalar registers, so the lengths are requested without waiting for the argument block.
#define MLAV_LEAD_ARGS const int32_t *seq_lens, const int32_t *q_lens, int32_t batch, int32_t nsplit, \
                       int32_t row_groups, int32_t min_tiles, int32_t max_q_len
#define MLAV_LEAD_INTO(p)   \
  p.seq_lens = seq_lens;    \
  p.q_lens = q_lens;        \
  p.batch = batch;          \
  p.nsplit = nsplit;        \
  p.row_groups = row_groups; \
  p.min_tiles = min_tiles;  \
  p.max_q_len = max_q_len
#define MLAV_LEAD_OF(a) a.seq_lens, a.q_lens, a.batch, a.nsplit, a.row_groups, a.min_tiles, a.max_q_len

template <bool kRanges>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_verify_partial(MLAV_LEAD_ARGS, PartialArgs args) {
  PartialArgs p = args;
  MLAV_LEAD_INTO(p);
  if constexpr (!kRanges) {
    WorkItem wi;
    if (!decode_work(p, blockIdx.x, kRowsPerGroup, wi)) return;
    partial_item(p, wi);
  } else {
    WorkItem wi;
    if (!decode_piece(p, blockIdx.x, wi)) return;
    partial_item(p, wi);
  }
}

// Kernel 2: one workgroup of 256 threads per (request, row).  Thread t covers
// output columns 8*(t%64) .. +7 over the splits s = t/64, t/64 + 4, ...; the four
// partial sums are added through LDS.  Every thread keeps up to 8 loads in
// flight, so the partials stream at memory speed.  Each wave also forms the
// merge weights itself: M = max_s lse_s, w_s = exp(lse_s - M) / sum_s exp(lse_s - M).
// PartT is _Float16 for the library's own workspace, float for caller partials.
constexpr int kMergeUnroll = 8;
// Split groups per workgroup (64 threads each): 4 in general.  A call with few rows and many
// splits (a decode step has 64 rows) takes the column-sliced form below, which spreads a row over
// four workgroups, or, past the split count that form holds in LDS, 16 groups, so that a row's
// many partials are read with more loads in flight; with few splits or many rows either only
// costs launch and reduction time.
constexpr int kMergeGroupsFew = 16;
constexpr int kMergeFewRows = 512;      // fewer rows per call than this ...
constexpr int kMergeManySplits = 64;    // ... and at least this many splits: the forms for few rows
constexpr int kMergeWaveSplits = 32;    // up to this many splits: one wave per row

// Kernel 1, two-stream form, for requests of at most 64 (token, head) rows (a q_len = 1 decode
// step with H <= 64, or a few draft tokens with few heads).  A 128-row workgroup would spend half
// of its MFMA work on rows that do not exist; here the four waves form two streams of a wave pair,
// both over the same 64 rows (wave 2s + h: stream s, rows [32h, 32h + 32), all 512 output
// columns).  Stream s takes tiles s, s + 2, s + 4, ... of the split, so one step consumes two
// tiles.  Each stream's tiles are double-buffered in two of the four ring buffers: the next tile is
// gathered between the Q.K MFMAs of the current one, into the buffer every wave finished with at
// the step's barrier.  (The one-tile-ahead Q.K of the 128-row form would need three buffers per
// stream, which do not fit, so here the softmax sits between the two contractions of a tile.)
// Each wave's P.V covers its own rows only, so no wave waits for another's P: the half of the
// softmax that the first 16-key step needs runs before the P.V MFMAs, the other half between them.
// At the end the two streams are merged inside the workgroup and one partial per split is
// written, as in the 128-row form.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_verify_partial_2s(MLAV_LEAD_ARGS, PartialArgs args) {
  PartialArgs p = args;
  MLAV_LEAD_INTO(p);
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRing * kTileBytes + kXchgBytes];
  lds_char* smem = (lds_char*)smem_raw;

  WorkItem wi;
  if (!decode_work(p, blockIdx.x, kRowsPerGroup2s, wi)) return;
  const int L = wi.L, Q = wi.Q, H = p.heads, R = wi.R;
  const int ntiles = wi.t_end - wi.t_begin;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hi = lane >> 5, lrow = lane & 31;
  const int stream = __builtin_amdgcn_readfirstlane(w) >> 1;  // (wave-uniform: the step's branches are scalar)
  const int half = w & 1;
  const int row0 = wi.g * kRowsPerGroup2s;
  const int myrow = row0 + half * kRowsPerWave + lrow;
  const bool row_valid = myrow < R;
  const int tok = row_valid ? myrow / H : 0;
  const int limit = L - Q + tok + 1;  // this row sees keys [0, limit)
  const int mask_from = L - Q + 1;    // first key some draft row cannot see
  const int nst = (ntiles - stream + 1) / 2;  // this stream's tiles
  const int nsteps = (ntiles + 1) / 2;        // stream 0 has the most

  // ---- gather set-up: wave (s, h) moves key blocks 2h and 2h + 1 (keys 16h .. 16h + 15) of its
  // stream's tiles; keys past the request's end use its last key's row (scores masked) ----------
  const int g_kr = lane >> 3;
  const char* kv = (const char*)p.kv;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const int w_uniform = __builtin_amdgcn_readfirstlane(w);
  const int32_t* slots_g = p.slot_idx + wi.ko;
  auto buf_of = [&](int k) { return (w_uniform >> 1) + 2 * (k & 1); };  // ring buffer of the stream's tile k
  auto gather_key = [&](int k, int j) {
    const int kk = k < nst ? k : (nst > 0 ? nst - 1 : 0);
    const int key = (wi.t_begin + 2 * kk + stream) * kTileKeys + 16 * half + 8 * j + g_kr;
    return key < L ? key : L - 1;
  };
  auto g_row = [&](int slot, int j) { return kv + (int64_t)slot * kRowBytes + (((lane & 7) ^ g_kr ^ j) << 4); };
  auto g_lds = [&](int k, int j) {
    return smem_base + buf_of(k) * kTileBytes + (2 * (w_uniform & 1) + j) * kKeyBlockBytes;
  };

  // Q.K A operand: lane reads key lrow, 16-B chunk 2*ks + hi (relative to a tile buffer)
  int kaddr[4];
  {
    const int kr = lrow & 7, f = kr ^ ((lrow >> 3) & 1);
    const int base = (lrow >> 3) * kKeyBlockBytes + kr * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) kaddr[j] = base + (((2 * j) ^ hi ^ f) << 4);
  }

  // ---- prologue: slot indices of tile 0, the q rows, then tile 0 while the q rows land ----------
  // The two streams hold the same 64 rows, so the rows are staged once, through ring buffers 2 and 3
  // (rows of wave half h in buffer 2 + h, in the key-tile layout as in the 128-row form), and tile 0
  // of each stream (buffers 0 and 1) is gathered while they arrive.  The two waves of a half split
  // its 32 rows (wave (s, h) moves key blocks 2s, 2s + 1 of buffer 2 + h), so every wave issues the
  // same number of loads and the waits below have fixed counts; each wave reads all 32 rows of its
  // half after the barrier.  (With both waves moving all 32 rows, a workgroup moved 144 KiB for
  // its 72 KiB of q, and the q rows were the last to land.)  Tile 1 goes to buffers 2 and 3 in the
  // first step, after the barrier that follows every wave's q reads.
  int sl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) sl[j] = load_b32_untracked(slots_g + gather_key(0, j));
  static_assert(2 * kDmaPerTile == 18, "wait counts below");
  {
    const uint32_t qbuf = smem_base + (2 + (w_uniform & 1)) * kTileBytes;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int kb = 2 * (w_uniform >> 1) + k;
      const int r = row0 + half * kRowsPerWave + 8 * kb + g_kr;
      const int64_t qrow = wi.qo * H + (r < R ? r : 0);
      dma_key_block((const char*)(p.q + qrow * kDqk) + (((lane & 7) ^ g_kr ^ (kb & 1)) << 4), qbuf + kb * kKeyBlockBytes);
    }
  }
  // the slot indices have landed (the 18 q loads issued after them may still be in flight)
  asm volatile("s_waitcnt vmcnt(18)" : "+v"(sl[0]), "+v"(sl[1]) : : "memory");
#pragma unroll
  for (int j = 0; j < 2; ++j) sl[j] = checked_slot(sl[j], p.num_slots, p.debug_flags);
  if (nst > 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) dma_key_block(g_row(sl[j], j), g_lds(0, j));
    MLAV_WAIT_VMCNT(18);  // the q rows have landed (tile 0's 18 loads may still be in flight)
  } else {
    MLAV_WAIT_VMCNT(0);
  }
  __syncthreads();  // every wave's q rows are visible
  bf16x8 qf[kQkSteps];
  {
    const lds_char* qb = smem + (2 + (w_uniform & 1)) * kTileBytes;
#pragma unroll
    for (int ks = 0; ks < kQkSteps; ++ks)
      qf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(qb + kaddr[ks & 3] + (ks >> 2) * kBlockBytes);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // (the first step's barrier then frees buffers 2, 3)
  int sn[2];  // slots of the next tile to gather (compiler-tracked loads, awaited at the next step)
#pragma unroll
  for (int j = 0; j < 2; ++j) sn[j] = slots_g[gather_key(1, j)];

  // P.V A operand addresses, as in the 128-row form (the column block's offset is added per read)
  int vaddr[2][2];
  {
    const int G = lane >> 4, j = lane & 15;
    const int kr = 4 * (G >> 1) + (j >> 2);
    const int u = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vaddr[e][r] = r * kKeyBlockBytes + kr * 128 + (((4 * e) ^ u ^ kr ^ r) << 4) + (j & 1) * 8;
  }
  // O^T of the wave's 32 rows, all 512 columns (column block c: columns 32c .. 32c + 31)
  f32x16 o_acc[kColBlocks];
#pragma unroll
  for (int c = 0; c < kColBlocks; ++c) {
    o_acc[c] = (f32x16){};
    // zeroed here, in AGPRs: left alone, the compiler moved the zeroing down to just before the
    // first P.V MFMA inside the loop, with no wait states between the write and the MFMA
    asm volatile("" : "+a"(o_acc[c]));
  }
  RowSoftmax st{-INFINITY, 0.f, 0.f};
  float nmref = 0.f;
  bf16x8 kf[kQkSteps];
  auto kread = [&](const lds_char* tb, int ks) {
    kf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(tb + kaddr[ks & 3] + (ks >> 2) * kBlockBytes);
  };
  // V^T fragment n of a tile: column block n % 16, 16-key step n / 16
  constexpr int kPvFrags2s = 2 * kColBlocks;
  bf16x8 vf[kPvFrags2s];
  auto vread = [&](const lds_char* tb, int n) {
    const int cb = n & (kColBlocks - 1), kk = n >> 4;
    const lds_char* vb = tb + (cb >> 1) * kBlockBytes + kk * 2 * kKeyBlockBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[cb & 1][0]));
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[cb & 1][1]));
    vf[n] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  for (int k = 0; k < nsteps; ++k) {
    const bool active = k < nst;
    const lds_char* tb = smem + buf_of(k) * kTileBytes;
    MLAV_WAIT_VMCNT(0);  // this stream's tile k (and the slot loads for the next gather) have landed
    __syncthreads();     // every stream's tile k is visible; every wave is done with step k-1
    const bool refill = k + 1 < nst;
    const char* r0 = g_row(checked_slot(sn[0], p.num_slots, p.debug_flags), 0);
    const char* r1 = g_row(checked_slot(sn[1], p.num_slots, p.debug_flags), 1);
    if (refill) {
#pragma unroll
      for (int j = 0; j < 2; ++j) sn[j] = slots_g[gather_key(k + 2, j)];
    }
    const uint32_t l0 = g_lds(k + 1, 0), l1 = g_lds(k + 1, 1);
    if (active) {
      SoftmaxTile sm;
      // Q.K of tile k, the gathers of the stream's tile k+1 between its MFMAs (two copies of the loop,
      // with and without the gathers, so that no branch sits between its MFMAs)
      f32x16 sacc;
      auto qk = [&](auto gather_c) __attribute__((always_inline)) {
        constexpr bool kGather = decltype(gather_c)::value;
#pragma unroll
        for (int ks = 0; ks < kPrefetch; ++ks) kread(tb, ks);
#pragma unroll
        for (int ks = 0; ks < kQkSteps; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
          if (ks + kPrefetch < kQkSteps) kread(tb, ks + kPrefetch);
          // the first V^T fragments of the tile, for the P.V after the softmax
          if (ks >= kQkSteps - kVPrefetch) vread(tb, ks - (kQkSteps - kVPrefetch));
          __builtin_amdgcn_sched_barrier(0);
          if (ks == 0) mfma_first_v(sacc, kf[ks], qf[ks]);
          else mfma_acc_v(sacc, kf[ks], qf[ks]);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kGather) {
            if (!(ks & 1) && (ks >> 1) < 2 * kDmaPerTile) {
              const int j = ks >> 1;
              if (j < kDmaPerTile) dma_chunk_group(r0, l0, j);
              else dma_chunk_group(r1, l1, j - kDmaPerTile);
            }
          }
        }
      };
      if (refill) qk(std::true_type{});
      else qk(std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      asm volatile(MLAV_MFMA_DRAIN : "+v"(sacc));
      const int t = wi.t_begin + 2 * k + stream;
      if (t * kTileKeys + kTileKeys > mask_from) mask_tile(sacc, t * kTileKeys + 4 * hi, limit);
      if (k == 0) {  // the stream's reference: the row max of its first tile (see the 128-row form)
        st.m_ref = tile_row_max(sacc) * p.scale_log2 + kRefHeadroom;
        nmref = (st.m_ref == -INFINITY) ? 0.f : -st.m_ref;
      }
      // the first half of the softmax: the lane's scores 0..7 (keys 0..15 of the tile, what the
      // first 16 P.V MFMAs take)
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.s[j] = vfma(sacc[j], p.scale_log2, nmref);
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.s[j] = vexp2(sm.s[j]);
#pragma unroll
      for (int m = 0; m < 4; ++m) sm.pw[m] = vpack_bf16(sm.s[2 * m], sm.s[2 * m + 1]);
      asm volatile("s_nop 3");  // wait states between the last bf16 pair and the first MFMA reading it
      const bf16x8 p0 = __builtin_bit_cast(bf16x8, sm.operand(0));
      bf16x8 p1;
      // P.V of the wave's rows over all 32 column-block fragments: between the first 16 MFMAs the
      // second half of the softmax (scores 8..15: FMA and exp2 in slots 0..7, the bf16 pairs in
      // slots 8..11, four slots before the first MFMA that takes them), between the last 16 the
      // row sums
#pragma unroll
      for (int n = 0; n < kPvFrags2s; ++n) {
        __builtin_amdgcn_sched_barrier(0);
        if (n + kVPrefetch < kPvFrags2s) vread(tb, n + kVPrefetch);
        __builtin_amdgcn_sched_barrier(0);
        mfma_acc_a(o_acc[n & (kColBlocks - 1)], vf[n], n < kColBlocks ? p0 : p1);
        __builtin_amdgcn_sched_barrier(0);
        if (n < 8) {
          sm.s[8 + n] = vexp2(vfma(sacc[8 + n], p.scale_log2, nmref));
        } else if (n < 12) {
          sm.pw[n - 4] = vpack_bf16(sm.s[2 * n - 8], sm.s[2 * n - 7]);
          if (n == 11) p1 = __builtin_bit_cast(bf16x8, sm.operand(1));
        } else if (n >= kColBlocks) {
          sum_slot(n - kColBlocks, sm, st);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  MLAV_WAIT_VMCNT(0);  // the last slot loads
  // The accumulators are read below only through acc_read (volatile), which stays behind this drain.
  asm volatile(MLAV_MFMA_DRAIN);

  // ---- merge of the two streams, then the partial write (one partial per split, as in the
  // 128-row form).  Each stream's sums and accumulators are relative to its own reference m_s;
  // with m = max(m_0, m_1) and a_s = 2^(m_s - m), the split's are l = sum_s a_s l_s and
  // O = sum_s a_s O_s.  The per-row (m, l, l_exact) of every wave go through LDS; the
  // accumulators are combined column block by column block by both streams (below).  A row where
  // either stream's sum outgrew its reference is redone exactly over the whole split.
  const float lt = pair_sum(st.l_run);
  const float le = pair_sum(st.l_exact);
  __syncthreads();  // every wave is done with the ring
  float* stat = (float*)(smem_raw + kRing * kTileBytes);  // [wave][32 rows][3]: m_ref, l, l_exact
  if (hi == 0) {
    stat[(w * 32 + lrow) * 3 + 0] = st.m_ref;
    stat[(w * 32 + lrow) * 3 + 1] = lt;
    stat[(w * 32 + lrow) * 3 + 2] = le;
  }
  __syncthreads();
  // row 32*hh + lrow: stream 0 holds it in wave hh, stream 1 in wave 2 + hh
  struct Comb { float a0, a1, inv, lex, m; bool redo; };
  auto combine = [&](int hh) {
    const float* s0 = stat + (hh * 32 + lrow) * 3;
    const float* s1 = stat + ((hh + 2) * 32 + lrow) * 3;
    Comb c;
    c.m = fmaxf(s0[0], s1[0]);
    c.a0 = s0[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s0[0] - c.m);
    c.a1 = s1[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s1[0] - c.m);
    const float l = s0[1] * c.a0 + s1[1] * c.a1;
    c.lex = s0[2] * c.a0 + s1[2] * c.a1;
    c.inv = l > 0.f ? 1.0f / l : 0.f;
    c.redo = !(s0[2] < kRowSumLimit) || !(s1[2] < kRowSumLimit);  // incl. +inf / NaN
    return c;
  };
  const Comb co = combine(half);
  // (the other half's rows too, so that every wave sees the same answer for the barrier below)
  const bool any_redo = __ballot(co.redo || combine(1 - half).redo) != 0;
  const uint64_t redo = __ballot(co.redo && hi == 0 && row_valid);
  if (stream == 0 && row_valid && hi == 0)
    p.lse_part[(int64_t)wi.bs * p.rows_pad + myrow] =
        co.lex > 0.f ? (co.m + __builtin_amdgcn_logf(co.lex)) * kLn2 : -INFINITY;

  // Stream 0 writes columns 0..255 of the wave pair's rows (column blocks 0..7), stream 1 columns
  // 256..511.  Each stream first hands the other its contribution to the other's blocks, already
  // weighted (a_s / l) and rounded to fp16 (2^-12 of that contribution, far below the bf16 output's
  // own rounding), through LDS; one barrier; then each adds what it received to its own weighted
  // accumulators, stages its 32 rows x 256 columns as fp16 rows and stores them.
  constexpr int kStageRows2s = kRowsPerWave;
  constexpr int kStageBytes2s = kStageRows2s * kStageRowBytes;
  constexpr int kDumpBytes = 16 * 64 * 16;  // per wave: 16 x (two (block, quad) f16x4) x 64 lanes x 16 B
  static_assert(kWaves * (kStageBytes2s + kDumpBytes) <= kRing * kTileBytes, "staging and hand-over fit the ring");
  lds_char* stage = smem + w * kStageBytes2s;
  lds_char* dump_mine = smem + kWaves * kStageBytes2s + w * kDumpBytes;
  const lds_char* dump_other = smem + kWaves * kStageBytes2s + (w ^ 2) * kDumpBytes;
  // O = (O_0 a_0 + O_1 a_1) / l, with the division folded into the weights; a stream weighs its
  // own accumulators with `mine` for its own blocks and for the blocks it hands over alike
  const float mine = (stream == 0 ? co.a0 : co.a1) * co.inv;
  auto weighted = [&](int b, int q4) {  // column block b, quad q4 of the lane: 4 weighted fp16 values
    f16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (_Float16)(acc_read(o_acc[b][4 * q4 + e]) * mine);
    return v;
  };
  // (the blocks a wave hands over and keeps depend on its stream: a wave-uniform branch picks one
  // of two instantiations, so every accumulator index stays a compile-time constant)
  auto give = [&](auto b0_c) __attribute__((always_inline)) {
    constexpr int b0 = decltype(b0_c)::value;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {  // (block, quad) pairs 2jj, 2jj + 1 of the 32 handed over
      const int v0 = 2 * jj, v1 = 2 * jj + 1;
      const f16x4 a = weighted(b0 + (v0 >> 2), v0 & 3), b = weighted(b0 + (v1 >> 2), v1 & 3);
      *(__attribute__((address_space(3))) i32x4*)(dump_mine + (jj * 64 + lane) * 16) =
          __builtin_shufflevector(__builtin_bit_cast(i32x2, a), __builtin_bit_cast(i32x2, b), 0, 1, 2, 3);
    }
  };
  auto keep = [&](auto b0_c, const i32x4 (&dd)[16]) __attribute__((always_inline)) {
    constexpr int b0 = decltype(b0_c)::value;
#pragma unroll
    for (int v = 0; v < 32; ++v) {
      const int b = b0 + (v >> 2), q4 = v & 3;
      const i32x4 d = dd[v >> 1];
      const f16x4 r = __builtin_bit_cast(f16x4, (v & 1) ? (i32x2){d[2], d[3]} : (i32x2){d[0], d[1]});
      f16x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (_Float16)(acc_read(o_acc[b][4 * q4 + e]) * mine + (float)r[e]);
      const int cb = (32 * (v >> 2) + 8 * q4 + 4 * hi) * 2;  // byte column within the stream's 256
      *(__attribute__((address_space(3))) f16x4*)(stage + lrow * kStageRowBytes + cb) = o;
    }
  };
  if (stream == 0) give(std::integral_constant<int, kColBlocks / 2>{});
  else give(std::integral_constant<int, 0>{});
  __syncthreads();  // both streams' hand-overs are in LDS
  {
    i32x4 dd[16];  // all reads go out before any is used
#pragma unroll
    for (int j = 0; j < 16; ++j) dd[j] = *(const __attribute__((address_space(3))) i32x4*)(dump_other + (j * 64 + lane) * 16);
    __builtin_amdgcn_sched_barrier(0);
    if (stream == 0) keep(std::integral_constant<int, 0>{}, dd);
    else keep(std::integral_constant<int, kColBlocks / 2>{}, dd);
  }
  {
    // the wave's 32 staged rows (rows 32*half ..), two rows per store instruction; the wave reads
    // back only what it staged itself, so no barrier is needed here
    uint16_t* part_base = p.o_part + (int64_t)wi.bs * p.rows_pad * kDv + (w_uniform >> 1) * (kDv / 2) + (lane & 31) * 8;
    i32x4 sv[16];  // all staged rows read first, then all stores
#pragma unroll
    for (int k = 0; k < 16; ++k)
      sv[k] = *(const __attribute__((address_space(3))) i32x4*)(stage + (2 * k + hi) * kStageRowBytes + (lane & 31) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int grow = row0 + half * kRowsPerWave + 2 * k + hi;
      if (grow < R) store16_through(part_base + (int64_t)grow * kDv, sv[k]);
    }
  }
  if (any_redo) {
    __syncthreads();  // (the global writes of all four waves are ordered by the barrier's release/acquire)
    if (stream == 0 && redo != 0) redo_rows_exact(p, wi, row0 + half * kRowsPerWave, (uint32_t)redo, 0, 1, wi.bs);
  }
}

// ---- Kernel 1, four-stream form: 32-row workgroups ---------------------------------------------------
// For calls whose two-stream grid would still leave at least half of the CUs idle (a short context
// with few splits, a q_len = 1 decode step with few splits): the four waves hold the same 32 rows and
// run four key streams over the split, in 16-key half tiles, half tile j to wave j % 4.  Wave w
// gathers its stream's half tiles into two half-tile buffers (keys 0..15 and 16..31 of ring buffer
// w) and computes their Q.K and softmax; the probabilities of the four streams go through LDS, and
// wave w accumulates P.V over every stream's keys for its own 128 output columns (column blocks
// 4w .. 4w + 3).  So the streams share one softmax reference per row (the row max over the first
// half tiles of all four, plus the headroom), a wave holds 64 accumulators, and the partial needs
// no merge between the waves at the end.
//   * Q.K on MFMA 16x16x32 bf16 as S^T = K . Q^T, one MFMA per 16-row half of the rows: the A
//     operand (16 keys x 32 dims) comes from the half-tile buffer, the B operand (32 dims x 16 rows)
//     is resident (36 fragments: 18 dim steps x 2 row halves).  In the C layout lane l holds keys
//     4(l/16) .. 4(l/16) + 3 of row l % 16 (first half) and of row 16 + l % 16 (second half).
//   * P.V as in the other forms (MFMA 32x32x16, O^T = V^T . P^T, one 16-key step per half tile).  A
//     permlane16 swap and a permlane32 swap of the bf16-packed probabilities give lane l eight keys of
//     row l % 32 in the key order of the 32x32 S^T layout's first 16-key step, which the V^T
//     fragments already follow: keys 0-3, 8-11 in lanes 0..31 and 4-7, 12-15 in lanes 32..63.
//   * A step: wait for the own half tile; barrier (every stream's half tile k has landed, every wave
//     is done with step k - 1's buffers and probabilities); Q.K with the gathers of the next half
//     tile and the first V^T fragments between its MFMAs (two copies of that loop, with and without
//     the gathers); softmax, P to LDS, the stream's row sums; barrier; P.V over the four streams' P.
constexpr int kHalfTileBytes = 2 * kKeyBlockBytes;  // 16 keys
constexpr int kQkSteps16 = kDqk / 32;               // 18 dim steps of MFMA 16x16x32
constexpr int kOwnBlocks4s = kColBlocks / 4;        // output column blocks of a wave
constexpr int kPvFrags4s = 4 * kOwnBlocks4s;        // V^T fragments of a wave per step (four streams)
static_assert(kQkSteps16 == 2 * kDmaPerTile, "one gather load per Q.K dim step");
// beside the ring: every stream's P of the step, the first half tiles' row maxima, the row statistics
constexpr int kPBufOff4s = 0, kRowMaxOff4s = 4 * 1024, kStatOff4s = kRowMaxOff4s + 4 * 32 * 4;
static_assert(kStatOff4s + (4 * 32 * 2 + 32) * 4 <= kXchgBytes, "exchange areas fit");

__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void mla_verify_partial_4s(MLAV_LEAD_ARGS, PartialArgs args) {
  PartialArgs p = args;
  MLAV_LEAD_INTO(p);
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRing * kTileBytes + kXchgBytes];
  lds_char* smem = (lds_char*)smem_raw;

  WorkItem wi;
  if (!decode_work(p, blockIdx.x, kRowsPerGroup4s, wi)) return;
  const int L = wi.L, Q = wi.Q, H = p.heads, R = wi.R;
  const int nh = 2 * (wi.t_end - wi.t_begin);  // 16-key half tiles of the split
  const int nsteps = (nh + 3) / 4;             // (stream 0 has the most half tiles)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int w_uniform = __builtin_amdgcn_readfirstlane(w);
  const int g4 = lane >> 4, c16 = lane & 15, hi = lane >> 5, lrow = lane & 31;
  const int row0 = wi.g * kRowsPerGroup4s;
  // Q.K layout: the lane's rows c16 (x) and 16 + c16 (y) of the group; rows past R use token 0
  const int rx = row0 + c16, ry = row0 + 16 + c16;
  const int limx = L - Q + (rx < R ? rx / H : 0) + 1;  // row x sees keys [0, limx)
  const int limy = L - Q + (ry < R ? ry / H : 0) + 1;
  const int mask_from = L - Q + 1;  // first key some draft row cannot see
  auto nst_of = [&](int s) { return nh > s ? (nh - s + 3) / 4 : 0; };  // half tiles of stream s
  const int nst = nst_of(w_uniform);

  // ---- gather set-up: the wave moves both key blocks (keys 0..7, 8..15) of its half tile k (the
  // split's half tile 4k + w) into half-buffer k & 1 of ring buffer w; keys past the request's end
  // use its last key's row (scores masked) -------------------------------------------------------------
  const int g_kr = lane >> 3;
  const char* kv = (const char*)p.kv;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const int32_t* slots_g = p.slot_idx + wi.ko;
  auto gather_key = [&](int k, int j) {
    const int kk = k < nst ? k : (nst > 0 ? nst - 1 : 0);
    const int key = (2 * wi.t_begin + 4 * kk + w_uniform) * 16 + 8 * j + g_kr;
    return key < L ? key : L - 1;
  };
  auto g_row = [&](int slot, int j) { return kv + (int64_t)slot * kRowBytes + (((lane & 7) ^ g_kr ^ j) << 4); };
  auto g_lds = [&](int k, int j) {
    return smem_base + w_uniform * kTileBytes + (k & 1) * kHalfTileBytes + j * kKeyBlockBytes;
  };

  // Q.K operands of dim step ks (A: key c16 of a half-tile buffer; B: row c16 of a staged q half),
  // 16-B chunk 4 ks + g4 in the tile layout: kaddr16[ks & 1] + (ks >> 1) * 1 KiB from the buffer
  int kaddr16[2];
  {
    const int kr = c16 & 7, f = kr ^ (c16 >> 3);
    const int base = (c16 >> 3) * kKeyBlockBytes + kr * 128;
#pragma unroll
    for (int e = 0; e < 2; ++e) kaddr16[e] = base + (((4 * e + g4) ^ f) << 4);
  }

  // ---- prologue: slot indices of half tile 0; the q rows, staged as four key blocks (rows 8w ..
  // 8w + 7 moved by wave w) in the upper half-buffers of ring buffers 2 (rows 0..15) and 3 (rows
  // 16..31); half tile 0 of every stream (lower half-buffers) while they land.  Half tile 1 of
  // streams 2 and 3 goes to those upper halves after the barrier that follows every wave's q reads.
  int sl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) sl[j] = load_b32_untracked(slots_g + gather_key(0, j));
  static_assert(kDmaPerTile == 9, "wait counts below");
  {
    const uint32_t qblk =
        smem_base + (2 + (w_uniform >> 1)) * kTileBytes + kHalfTileBytes + (w_uniform & 1) * kKeyBlockBytes;
    const int r = row0 + 8 * w_uniform + g_kr;
    const int64_t qrow = wi.qo * H + (r < R ? r : 0);
    dma_key_block((const char*)(p.q + qrow * kDqk) + (((lane & 7) ^ g_kr ^ (w_uniform & 1)) << 4), qblk);
  }
  // the slot indices have landed (the 9 q loads issued after them may still be in flight)
  asm volatile("s_waitcnt vmcnt(9)" : "+v"(sl[0]), "+v"(sl[1]) : : "memory");
#pragma unroll
  for (int j = 0; j < 2; ++j) sl[j] = checked_slot(sl[j], p.num_slots, p.debug_flags);
  if (nst > 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) dma_key_block(g_row(sl[j], j), g_lds(0, j));
    MLAV_WAIT_VMCNT(18);  // the q block has landed (half tile 0's 18 loads may still be in flight)
  } else {
    MLAV_WAIT_VMCNT(0);
  }
  __syncthreads();  // every wave's q block is visible
  bf16x8 qf[2][kQkSteps16];
#pragma unroll
  for (int rh = 0; rh < 2; ++rh) {
    const lds_char* qb = smem + (2 + rh) * kTileBytes + kHalfTileBytes;
#pragma unroll
    for (int ks = 0; ks < kQkSteps16; ++ks)
      qf[rh][ks] = *(const __attribute__((address_space(3))) bf16x8*)(qb + kaddr16[ks & 1] + (ks >> 1) * kBlockBytes);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __syncthreads();  // every wave holds its q fragments: the upper halves of buffers 2 and 3 are free
  int sn[2];  // slots of the next half tile to gather (compiler-tracked loads, awaited at the next step)
#pragma unroll
  for (int j = 0; j < 2; ++j) sn[j] = slots_g[gather_key(1, j)];

  // P.V A operand addresses, as in the other forms (the column block's offset is added per read)
  int vaddr[2][2];
  {
    const int G = lane >> 4, j = lane & 15;
    const int kr = 4 * (G >> 1) + (j >> 2);
    const int u = 2 * (G & 1) + ((j & 3) >> 1);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vaddr[e][r] = r * kKeyBlockBytes + kr * 128 + (((4 * e) ^ u ^ kr ^ r) << 4) + (j & 1) * 8;
  }
  // O^T of the group's 32 rows over all the split's keys, the wave's 128 columns
  f32x16 o_acc[kOwnBlocks4s];
#pragma unroll
  for (int c = 0; c < kOwnBlocks4s; ++c) {
    o_acc[c] = (f32x16){};
    asm volatile("" : "+a"(o_acc[c]));  // zeroed here, in AGPRs (see the two-stream form)
  }
  // the reference of rows x and y (shared by the streams) and this stream's share of their row sums
  float m_x = -INFINITY, m_y = -INFINITY, nm_x = 0.f, nm_y = 0.f;
  float lr_x = 0.f, lr_y = 0.f, le_x = 0.f, le_y = 0.f;
  lds_char* xchg = smem + kRing * kTileBytes;
  float* rmax = (float*)(smem_raw + kRing * kTileBytes + kRowMaxOff4s);  // [stream][32 rows]: raw row max
  bf16x8 kf[kQkSteps16];
  auto kread = [&](const lds_char* hb, int ks) {
    kf[ks] = *(const __attribute__((address_space(3))) bf16x8*)(hb + kaddr16[ks & 1] + (ks >> 1) * kBlockBytes);
  };
  bf16x8 vf[kPvFrags4s];  // V^T fragment n: stream n / 4's half tile, column block 4w + n % 4
  // (a stream without a half tile in the step reads stream 0's, and its P is zero)
  auto vread = [&](int k, int n) {
    const int s = k < nst_of(n >> 2) ? (n >> 2) : 0;
    const lds_char* vb = smem + s * kTileBytes + (k & 1) * kHalfTileBytes +
                         (2 * w_uniform + ((n & 3) >> 1)) * kBlockBytes;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[n & 1][0]));
    const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(vb + vaddr[n & 1][1]));
    vf[n] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  for (int k = 0; k < nsteps; ++k) {
    const bool active = k < nst;
    const lds_char* hb = smem + w_uniform * kTileBytes + (k & 1) * kHalfTileBytes;
    MLAV_WAIT_VMCNT(0);  // this wave's half tile k (and the slot loads for the next gather) have landed
    __syncthreads();     // every stream's half tile k is visible; every wave is done with step k - 1
    f32x4 sx, sy;
    if (active) {
      const bool refill = k + 1 < nst;
      const char* r0 = g_row(checked_slot(sn[0], p.num_slots, p.debug_flags), 0);
      const char* r1 = g_row(checked_slot(sn[1], p.num_slots, p.debug_flags), 1);
      if (refill) {
#pragma unroll
        for (int j = 0; j < 2; ++j) sn[j] = slots_g[gather_key(k + 2, j)];
      }
      const uint32_t l0 = g_lds(k + 1, 0), l1 = g_lds(k + 1, 1);
      // Q.K of half tile k for both row halves, the gathers of half tile k + 1 between the MFMAs, the
      // first V^T fragments (stream 0's) in the last dim steps.  (Two copies of the loop, with and
      // without the gathers, so that no branch sits between its MFMAs.)
      auto qk = [&](auto gather_c) __attribute__((always_inline)) {
        constexpr bool kGather = decltype(gather_c)::value;
#pragma unroll
        for (int ks = 0; ks < kPrefetch; ++ks) kread(hb, ks);
#pragma unroll
        for (int ks = 0; ks < kQkSteps16; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
          if (ks + kPrefetch < kQkSteps16) kread(hb, ks + kPrefetch);
          if (ks >= kQkSteps16 - kVPrefetch) vread(k, ks - (kQkSteps16 - kVPrefetch));
          __builtin_amdgcn_sched_barrier(0);
          if (ks == 0) {
            mfma16_first_v(sx, kf[ks], qf[0][ks]);
            mfma16_first_v(sy, kf[ks], qf[1][ks]);
          } else {
            mfma16_acc_v(sx, kf[ks], qf[0][ks]);
            mfma16_acc_v(sy, kf[ks], qf[1][ks]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (kGather) {
            if (ks < kDmaPerTile) dma_chunk_group(r0, l0, ks);
            else dma_chunk_group(r1, l1, ks - kDmaPerTile);
          }
        }
      };
      if (refill) qk(std::true_type{});
      else qk(std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
      asm volatile(MLAV_MFMA_DRAIN : "+v"(sx), "+v"(sy));
      const int key0 = (2 * wi.t_begin + 4 * k + w_uniform) * 16 + 4 * g4;  // the lane's first key
      if (key0 - 4 * g4 + 16 > mask_from) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sx[r] = key0 + r < limx ? sx[r] : -INFINITY;
          sy[r] = key0 + r < limy ? sy[r] : -INFINITY;
        }
      }
    } else {
      // (a stream without a half tile in the split's last step: stream 0's V^T fragments without
      // prefetch, and a zero P for the others)
#pragma unroll
      for (int n = 0; n < kVPrefetch; ++n) vread(k, n);
      *(__attribute__((address_space(3))) i32x4*)(xchg + kPBufOff4s + (w * 64 + lane) * 16) = (i32x4){0, 0, 0, 0};
    }
    if (k == 0) {  // the shared references: the row maxima of the four streams' first half tiles
      const float mx = active ? quad_max(fmaxf(fmaxf(sx[0], sx[1]), fmaxf(sx[2], sx[3]))) : -INFINITY;
      const float my = active ? quad_max(fmaxf(fmaxf(sy[0], sy[1]), fmaxf(sy[2], sy[3]))) : -INFINITY;
      if (g4 == 0) {
        rmax[w * 32 + c16] = mx;
        rmax[w * 32 + 16 + c16] = my;
      }
      __syncthreads();
      float ax = rmax[c16], ay = rmax[16 + c16];
#pragma unroll
      for (int s = 1; s < 4; ++s) {
        ax = fmaxf(ax, rmax[s * 32 + c16]);
        ay = fmaxf(ay, rmax[s * 32 + 16 + c16]);
      }
      m_x = ax * p.scale_log2 + kRefHeadroom;
      m_y = ay * p.scale_log2 + kRefHeadroom;
      nm_x = (m_x == -INFINITY) ? 0.f : -m_x;
      nm_y = (m_y == -INFINITY) ? 0.f : -m_y;
    }
    if (active) {
      float ex[4], ey[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ex[r] = vfma(sx[r], p.scale_log2, nm_x);
#pragma unroll
      for (int r = 0; r < 4; ++r) ey[r] = vfma(sy[r], p.scale_log2, nm_y);
#pragma unroll
      for (int r = 0; r < 4; ++r) ex[r] = vexp2(ex[r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) ey[r] = vexp2(ey[r]);
      const int px0 = vpack_bf16(ex[0], ex[1]), px1 = vpack_bf16(ex[2], ex[3]);
      const int py0 = vpack_bf16(ey[0], ey[1]), py1 = vpack_bf16(ey[2], ey[3]);
      // lanes of rows 0..15 give their row 16.. keys to, and take their own row's next keys from, the
      // lanes 16 above (permlane16), then the halves swap (permlane32): see the layout note above
      const auto s0 = __builtin_amdgcn_permlane16_swap(px0, py0, false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(px1, py1, false, false);
      const auto t0 = __builtin_amdgcn_permlane32_swap(s0[0], s0[1], false, false);
      const auto t1 = __builtin_amdgcn_permlane32_swap(s1[0], s1[1], false, false);
      *(__attribute__((address_space(3))) i32x4*)(xchg + kPBufOff4s + (w * 64 + lane) * 16) =
          (i32x4){(int)t0[0], (int)t1[0], (int)t0[1], (int)t1[1]};
      // the stream's row sums (while the other streams reach the barrier)
#pragma unroll
      for (int r = 0; r < 4; ++r) vadd_to(le_x, ex[r]);
#pragma unroll
      for (int r = 0; r < 4; ++r) vadd_to(le_y, ey[r]);
      vsum_pair_to(lr_x, px0);
      vsum_pair_to(lr_x, px1);
      vsum_pair_to(lr_y, py0);
      vsum_pair_to(lr_y, py1);
    }
    __syncthreads();  // every active stream's P of the step is in LDS
    // P.V: the four streams' P (those with a half tile in this step) times their V^T fragments for the
    // wave's column blocks; stream s's P is read two MFMAs before its first one
    auto pread = [&](int s) {
      return *(const __attribute__((address_space(3))) bf16x8*)(xchg + kPBufOff4s + (s * 64 + lane) * 16);
    };
    bf16x8 pb[4];
    pb[0] = pread(0);
#pragma unroll
    for (int n = 0; n < kPvFrags4s; ++n) {
      __builtin_amdgcn_sched_barrier(0);
      if (n + kVPrefetch < kPvFrags4s) vread(k, n + kVPrefetch);
      if ((n & 3) == 2 && n + 2 < kPvFrags4s) pb[(n + 2) >> 2] = pread((n + 2) >> 2);
      __builtin_amdgcn_sched_barrier(0);
      mfma_acc_a(o_acc[n & 3], vf[n], pb[n >> 2]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  MLAV_WAIT_VMCNT(0);  // the last slot loads
  // The accumulators are read below only through acc_read (volatile), which stays behind this drain.
  asm volatile(MLAV_MFMA_DRAIN);

  // ---- the partial: the row sums of the four streams (one reference, so plain sums) through LDS,
  // then each wave normalises, stages and stores its 32 rows x 128 columns.  A row whose sum outgrew
  // the reference is redone exactly over the whole split.
  const float ltx = quad_sum(lr_x), lty = quad_sum(lr_y);
  const float lex = quad_sum(le_x), ley = quad_sum(le_y);
  float* stat = (float*)(smem_raw + kRing * kTileBytes + kStatOff4s);  // [stream][32 rows][2]: l, l_exact; then m[32]
  if (g4 == 0) {
    stat[(w * 32 + c16) * 2 + 0] = ltx;
    stat[(w * 32 + c16) * 2 + 1] = lex;
    stat[(w * 32 + 16 + c16) * 2 + 0] = lty;
    stat[(w * 32 + 16 + c16) * 2 + 1] = ley;
    if (w == 0) {
      stat[4 * 32 * 2 + c16] = m_x;
      stat[4 * 32 * 2 + 16 + c16] = m_y;
    }
  }
  __syncthreads();  // (also: every wave is done with the ring)
  float l = 0.f, lexact = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    l += stat[(s * 32 + lrow) * 2 + 0];
    lexact += stat[(s * 32 + lrow) * 2 + 1];
  }
  const float m = stat[4 * 32 * 2 + lrow];
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const bool redo_row = !(lexact < kRowSumLimit);  // incl. +inf / NaN
  const bool row_valid = row0 + lrow < R;
  const bool any_redo = __ballot(redo_row) != 0;
  const uint64_t redo = __ballot(redo_row && hi == 0 && row_valid);
  if (w_uniform == 0 && hi == 0 && row_valid)
    p.lse_part[(int64_t)wi.bs * p.rows_pad + row0 + lrow] =
        lexact > 0.f ? (m + __builtin_amdgcn_logf(lexact)) * kLn2 : -INFINITY;

  constexpr int kStageRowBytes4 = 256 + 16;  // one row's 128 fp16 columns + 16 B of padding
  constexpr int kStageBytes4 = 32 * kStageRowBytes4;
  static_assert(kWaves * kStageBytes4 <= kRing * kTileBytes, "staging fits the ring");
  lds_char* stage = smem + w_uniform * kStageBytes4;
#pragma unroll
  for (int v = 0; v < 4 * kOwnBlocks4s; ++v) {  // (block, quad) v: columns 32 (v / 4) + 8 (v % 4) + 4 hi ..
    const int b = v >> 2, q4 = v & 3;
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (_Float16)(acc_read(o_acc[b][4 * q4 + e]) * inv);
    *(__attribute__((address_space(3))) f16x4*)(stage + lrow * kStageRowBytes4 + (32 * b + 8 * q4 + 4 * hi) * 2) = o;
  }
  {
    // the wave's 32 staged rows, four rows per store instruction (16 lanes x 16 B per row); the wave
    // reads back only what it staged itself, so no barrier is needed here
    uint16_t* part_base = p.o_part + ((int64_t)wi.bs * p.rows_pad + row0) * kDv + w_uniform * (kDv / 4) + (lane & 15) * 8;
    i32x4 sv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      sv[k] = *(const __attribute__((address_space(3))) i32x4*)(stage + (4 * k + g4) * kStageRowBytes4 + (lane & 15) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + g4;
      if (row0 + r < R) store16_through(part_base + (int64_t)r * kDv, sv[k]);
    }
  }
  if (any_redo) {
    __syncthreads();  // (the global writes of all four waves are ordered by the barrier's release/acquire)
    if (w_uniform == 0 && redo != 0) redo_rows_exact(p, wi, row0, (uint32_t)redo, 0, 1, wi.bs);
  }
}

// Eight consecutive partial values: loaded raw (so that a batch of loads is in flight at
// once), widened to fp32 when used.
template <typename PartT>
struct Raw8;
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ void load(const float* src) { a = ((const f32x4*)src)[0]; b = ((const f32x4*)src)[1]; }
  __device__ float get(int j) const { return j < 4 ? a[j] : b[j - 4]; }
};
template <>
struct Raw8<_Float16> {
  f16x8 a;
  __device__ void load(const _Float16* src) { a = *(const f16x8*)src; }
  __device__ float get(int j) const { return (float)a[j]; }
};

// kRowsPerBlock > 1 (with one split group): one wave per row, kRowsPerBlock consecutive rows of a
// request per workgroup.  kRanges: the partials come from the range plan, whose requests have few
// partials each, so a row's work is one wave's few loads; the plan (the request's partial count
// and output offset) is derived once per workgroup, by its first wave.
template <typename PartT, int kMergeGroups, int kRowsPerBlock = 1, bool kRanges = false>
__global__ __launch_bounds__(64 * kMergeGroups * kRowsPerBlock) void mla_verify_merge_kernel(MergeArgs p) {
  static_assert(kMergeGroups == 1 || kRowsPerBlock == 1, "several rows per workgroup take one split group each");
  __shared__ float group_sum[kMergeGroups > 1 ? kMergeGroups - 1 : 1][64][8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int rows_per_b = p.max_q_len * p.heads;
  const int blocks_per_b = (rows_per_b + kRowsPerBlock - 1) / kRowsPerBlock;
  const int b = (int)(blockIdx.x / blocks_per_b);
  const int r = (int)(blockIdx.x - (int64_t)b * blocks_per_b) * kRowsPerBlock + (kRowsPerBlock > 1 ? tid >> 6 : 0);
  if (b >= p.batch) return;  // (uniform over the workgroup)
  int ns;
  int64_t qo = 0;
  if constexpr (kRanges) {
    __shared__ int plan[3];  // the request's partial count, first output row, rows
    if (tid < 64) {
      const RequestScan rq = scan_requests(p.seq_lens, p.q_lens, p.batch, p.max_q_len, p.debug_flags);
      const int C = range_chunk(rq, p.nsplit, p.workers, p.min_tiles);
      const int J = __builtin_amdgcn_readlane(rq.J, b), tiles = __builtin_amdgcn_readlane(rq.tiles, b);
      const int qo_b = __builtin_amdgcn_readlane(rq.qo, b), rows_b = __builtin_amdgcn_readlane(rq.Q, b) * p.heads;
      if (lane == 0) {
        plan[0] = tiles > 0 ? (J + tiles - 1) / C - J / C + 1 : 0;
        plan[1] = qo_b;
        plan[2] = rows_b;
      }
    }
    __syncthreads();
    if (r >= plan[2]) return;  // (no barrier follows)
    ns = plan[0];
    qo = plan[1];
  } else {
    const int Q = clamped_q(p.q_lens, p.seq_lens, b, p.max_q_len, p.debug_flags);
    if (r >= Q * p.heads) return;
    ns = p.use_all_splits ? p.nsplit : split_count(read_len(p.seq_lens, b, p.debug_flags), p.nsplit, p.min_tiles);
    for (int i = 0; i < b; ++i) qo += clamped_q(p.q_lens, p.seq_lens, i, p.max_q_len, p.debug_flags);
  }

  const int64_t base = (int64_t)b * p.nsplit * p.rows_stride + r;  // (b, s=0, r)
  const float* lse_s = p.lse_part + base;
  const int c8 = tid & 63, sg = kMergeGroups > 1 ? tid >> 6 : 0;
  const PartT* src = (const PartT*)p.o_part + base * kDv + 8 * c8;
  const int64_t sstride = (int64_t)p.rows_stride * kDv;

  // The LSEs of splits lane, lane + 64, ... go out first, then the first batch of partial
  // loads; the weights are formed while the partials are in flight.
  const float x0 = lane < ns ? lse_s[(int64_t)lane * p.rows_stride] : -INFINITY;
  Raw8<PartT> v[kMergeUnroll];
  auto load_batch = [&](int s0) {  // splits past ns re-read split 0 (weight 0 below)
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + kMergeGroups * u;
      v[u].load(src + (int64_t)(s < ns ? s : 0) * sstride);
    }
  };
  load_batch(sg);

  // M = max_s lse_s and Z = sum_s exp(lse_s - M): per lane (online), then across the wave.
  float m_l = x0, z_l = x0 > -INFINITY ? 1.f : 0.f;
  for (int s = lane + 64; s < ns; s += 64) {
    const float x = lse_s[(int64_t)s * p.rows_stride];
    const float m_new = fmaxf(m_l, x);
    if (m_new > -INFINITY) {
      z_l = z_l * __expf(m_l - m_new) + __expf(x - m_new);
      m_l = m_new;
    }
  }
  const float M = wave_max(m_l);
  const float Mref = (M == -INFINITY) ? 0.f : M;
  const float Z = wave_sum(m_l > -INFINITY ? z_l * __expf(m_l - Mref) : 0.f);
  const float invZ = Z > 0.f ? 1.0f / Z : 0.f;
  // weight of split s, exp(lse_s - M) / Z (wave-uniform): formed once by the lane that loaded its
  // LSE, or from memory past 64 splits
  const float w0 = lane < ns ? __expf(x0 - Mref) * invZ : 0.f;
  auto weight = [&](int s) {
    if (s < 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), s));
    return s < ns ? __expf(lse_s[(int64_t)s * p.rows_stride] - Mref) * invZ : 0.f;
  };

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg;;) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float ws = weight(s0 + kMergeGroups * u);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += ws * v[u].get(j);
    }
    s0 += kMergeGroups * kMergeUnroll;
    if (s0 >= ns) break;
    load_batch(s0);
  }
  if constexpr (kMergeGroups > 1) {
    if (sg > 0)
#pragma unroll
      for (int j = 0; j < 8; ++j) group_sum[sg - 1][c8][j] = acc[j];
    __syncthreads();
    if (sg == 0)
#pragma unroll
      for (int g = 0; g < kMergeGroups - 1; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += group_sum[g][c8][j];
  }
  if (sg == 0) {
    const int64_t orow = qo * p.heads + r;
    bf16x8 ov;
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = (__bf16)acc[j];
    *((bf16x8*)(p.out + orow * kDv) + c8) = ov;
    if (lane == 0) p.lse[orow] = Z > 0.f ? Mref + __logf(Z) : -INFINITY;
  }
}

// Kernel 2 for calls with few rows and many splits (a decode step: 64 rows, each with up to
// hundreds of partials): one workgroup of 256 threads per (request, row, 128-column slice), so
// that four times as many workgroups share the reads of a row.  The workgroup forms the merge
// weights once, from block-wide max and sum over the row's LSEs, and keeps them in LDS; thread t
// covers columns 8*(t%16) of its slice over the splits t/16, t/16 + 16, ...; the 16 partial sums
// are added through LDS.
constexpr int kSliceCols = 128;                          // output columns per workgroup
constexpr int kSliceThreads = kSliceCols / 8;            // threads per split group
constexpr int kSliceGroups = 256 / kSliceThreads;        // split groups per workgroup
constexpr int kSliceMaxSplits = 1024;                    // weights held in LDS
constexpr int kSliceLsePerThread = kSliceMaxSplits / 256;

template <typename PartT>
__global__ __launch_bounds__(256) void mla_verify_merge_sliced(MergeArgs p) {
  __shared__ float wts[kSliceMaxSplits];
  __shared__ float wred[2][4];
  __shared__ float gsum[kSliceGroups - 1][kSliceThreads][8];
  constexpr int kSlices = kDv / kSliceCols;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slice = (int)(blockIdx.x % kSlices);
  const int64_t row_id = blockIdx.x / kSlices;
  const int rows_per_b = p.max_q_len * p.heads;
  const int b = (int)(row_id / rows_per_b);
  const int r = (int)(row_id - (int64_t)b * rows_per_b);
  if (b >= p.batch) return;
  const int Q = clamped_q(p.q_lens, p.seq_lens, b, p.max_q_len, p.debug_flags);
  if (r >= Q * p.heads) return;  // uniform over the workgroup
  const int ns = p.use_all_splits ? p.nsplit : split_count(read_len(p.seq_lens, b, p.debug_flags), p.nsplit, p.min_tiles);
  int64_t qo = 0;
  for (int i = 0; i < b; ++i) qo += clamped_q(p.q_lens, p.seq_lens, i, p.max_q_len, p.debug_flags);

  const int64_t base = (int64_t)b * p.nsplit * p.rows_stride + r;  // (b, s=0, r)
  const float* lse_s = p.lse_part + base;
  const int c = tid % kSliceThreads, sg = tid / kSliceThreads;
  const PartT* src = (const PartT*)p.o_part + base * kDv + slice * kSliceCols + 8 * c;
  const int64_t sstride = (int64_t)p.rows_stride * kDv;

  // the row's LSEs (split tid + 256k), then the first batch of partial loads
  float x[kSliceLsePerThread];
#pragma unroll
  for (int k = 0; k < kSliceLsePerThread; ++k) {
    const int s = tid + 256 * k;
    x[k] = s < ns ? lse_s[(int64_t)s * p.rows_stride] : -INFINITY;
  }
  Raw8<PartT> v[kMergeUnroll];
  auto load_batch = [&](int s0) {  // splits past ns re-read split 0 (weight 0 below)
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + kSliceGroups * u;
      v[u].load(src + (int64_t)(s < ns ? s : 0) * sstride);
    }
  };
  load_batch(sg);

  // M = max_s lse_s, Z = sum_s exp(lse_s - M), w_s = exp(lse_s - M) / Z, while the partials load
  float m = x[0];
#pragma unroll
  for (int k = 1; k < kSliceLsePerThread; ++k) m = fmaxf(m, x[k]);
  m = wave_max(m);
  if (lane == 0) wred[0][wv] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  const float Mref = (M == -INFINITY) ? 0.f : M;
  float e[kSliceLsePerThread], z = 0.f;
#pragma unroll
  for (int k = 0; k < kSliceLsePerThread; ++k) {
    e[k] = x[k] > -INFINITY ? __expf(x[k] - Mref) : 0.f;
    z += e[k];
  }
  z = wave_sum(z);
  if (lane == 0) wred[1][wv] = z;
  __syncthreads();
  const float Z = (wred[1][0] + wred[1][1]) + (wred[1][2] + wred[1][3]);
  const float invZ = Z > 0.f ? 1.0f / Z : 0.f;
#pragma unroll
  for (int k = 0; k < kSliceLsePerThread; ++k) {
    const int s = tid + 256 * k;
    if (s < ns) wts[s] = e[k] * invZ;
  }
  __syncthreads();

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg;;) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int s = s0 + kSliceGroups * u;
      const float ws = s < ns ? wts[s] : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += ws * v[u].get(j);
    }
    s0 += kSliceGroups * kMergeUnroll;
    if (s0 >= ns) break;
    load_batch(s0);
  }
  if (sg > 0)
#pragma unroll
    for (int j = 0; j < 8; ++j) gsum[sg - 1][c][j] = acc[j];
  __syncthreads();
  if (sg == 0) {
#pragma unroll
    for (int g = 0; g < kSliceGroups - 1; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += gsum[g][c][j];
    const int64_t orow = qo * p.heads + r;
    bf16x8 ov;
#pragma unroll
    for (int j = 0; j < 8; ++j) ov[j] = (__bf16)acc[j];
    *(bf16x8*)(p.out + orow * kDv + slice * kSliceCols + 8 * c) = ov;
    if (slice == 0 && tid == 0) p.lse[orow] = Z > 0.f ? Mref + __logf(Z) : -INFINITY;
  }
}

hipError_t launch_partial(const PartialArgs& a, hipStream_t stream) {
  if (a.plan_ranges) {
    const int64_t grid = range_grid(a.workers, a.row_groups, a.batch);
    hipLaunchKernelGGL(mla_verify_partial<true>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, MLAV_LEAD_OF(a), a);
    return hipGetLastError();
  }
  const int64_t grid = (int64_t)a.batch * a.nsplit * a.row_groups;
  if (a.streams == 4)
    hipLaunchKernelGGL(mla_verify_partial_4s, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, MLAV_LEAD_OF(a), a);
  else if (a.streams == 2)
    hipLaunchKernelGGL(mla_verify_partial_2s, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, MLAV_LEAD_OF(a), a);
  else
    hipLaunchKernelGGL(mla_verify_partial<false>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, MLAV_LEAD_OF(a), a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.batch * a.max_q_len * a.heads;  // one workgroup per row below
  const bool few = rows < kMergeFewRows && a.nsplit >= kMergeManySplits;
  // The library's fp16 partials with at most kMergeWaveSplits per row (the range plan, or a call such
  // as ctx64k's 32 splits): one wave per row, four rows per workgroup (at ctx64k this took 0.7 us
  // less per call than 256 threads per row, measured on one box); after the range plan 16 rows per
  // workgroup, for which the plan is derived once.
  if (a.plan_ranges) {
    constexpr int kRowsPerBlock = 16;
    const int64_t blocks = (int64_t)a.batch * ((a.max_q_len * a.heads + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL((mla_verify_merge_kernel<_Float16, 1, kRowsPerBlock, true>), dim3((unsigned)blocks),
                       dim3(64 * kRowsPerBlock), 0, stream, a);
    return hipGetLastError();
  }
  if (!a.part_fp32 && !few && a.nsplit <= kMergeWaveSplits) {
    constexpr int kRowsPerBlock = 4;
    const int64_t blocks = (int64_t)a.batch * ((a.max_q_len * a.heads + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL((mla_verify_merge_kernel<_Float16, 1, kRowsPerBlock>), dim3((unsigned)blocks),
                       dim3(64 * kRowsPerBlock), 0, stream, a);
    return hipGetLastError();
  }
  if (few && a.nsplit <= kSliceMaxSplits) {
    const dim3 grid((unsigned)(rows * (kDv / kSliceCols)));
    if (a.part_fp32)
      hipLaunchKernelGGL(mla_verify_merge_sliced<float>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(mla_verify_merge_sliced<_Float16>, grid, dim3(256), 0, stream, a);
  } else if (a.part_fp32 && few)
    hipLaunchKernelGGL((mla_verify_merge_kernel<float, kMergeGroupsFew>), dim3((unsigned)rows), dim3(64 * kMergeGroupsFew), 0, stream, a);
  else if (a.part_fp32)
    hipLaunchKernelGGL((mla_verify_merge_kernel<float, 4>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  else if (few)
    hipLaunchKernelGGL((mla_verify_merge_kernel<_Float16, kMergeGroupsFew>), dim3((unsigned)rows), dim3(64 * kMergeGroupsFew), 0, stream, a);
  else
    hipLaunchKernelGGL((mla_verify_merge_kernel<_Float16, 4>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
