// Shared device helpers for the GQLA kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (v_mfma_f32_16x16x32_bf16), for a
// lane l = 16*q + c (q = l/16 in 0..3, c = l%16):
//   A (16 x 32, m x k):  lane holds A[m = c][k = 8q .. 8q+7]
//   B (32 x 16, k x n):  lane holds B[k = 8q .. 8q+7][n = c]
//   D (16 x 16, m x n):  lane holds D[m = 4q .. 4q+3][n = c]
// The k order inside an instruction is shared by A and B, so any consistent
// relabelling of k (e.g. of cache tokens) leaves the product unchanged.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even, by the
// hardware conversion (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf_bits2f(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// 16-byte global load straight into an MFMA operand register quad.
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Zero the bf16 elements j >= keep of an 8-element operand (0 <= keep <= 8).
__device__ __forceinline__ bf16x8 keep_first(const bf16x8& v, int keep) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int j = 2 * w;
    uint32_t m = (j < keep ? 0x0000ffffu : 0u) | (j + 1 < keep ? 0xffff0000u : 0u);
    u[w] &= m;
  }
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ float wave_max_xor16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Max / sum over the four lanes c, c+16, c+32, c+48 (the 4 lane groups q
// holding one MFMA column), with the gfx950 cross-lane swaps instead of an
// LDS permute: v_permlane16_swap a, b (a and b both holding x) leaves
// {x of lane l, x of lane l ^ 16} in {a, b} on every lane (likewise
// v_permlane32_swap with l ^ 32).  Written as asm on two distinct registers:
// the compiler's model of the builtin with equal inputs folds the two
// results into one.  The s_nops cover the VALU -> permlane -> VALU hazards
// the compiler cannot see inside asm.
__device__ __forceinline__ void swap_pairs16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_pairs32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float wave_max_q(float v) {
  float a = v, b = v;
  swap_pairs16(a, b);
  v = fmaxf(a, b);
  a = v;
  b = v;
  swap_pairs32(a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float wave_sum_q(float v) {
  float a = v, b = v;
  swap_pairs16(a, b);
  v = a + b;
  a = v;
  b = v;
  swap_pairs32(a, b);
  return a + b;
}

typedef __attribute__((address_space(3))) unsigned char lds_u8_t;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// i reads base + voff_bytes(i) and its 16 bytes land at lds_base + 16 * i.
// `base` and `lds_base` must be wave-uniform.  Issued from inline asm so that
// the compiler does not add its own conservative waits for it (it cannot tell
// which LDS buffer a copy targets and would wait for every copy in flight);
// callers wait with vm_wait<N>() before reading the buffer.  M0 is written in
// the same asm block; the one wait state between the M0 write and the copy is
// the s_nop.  There are no register outputs.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff_bytes, lds_u8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff_bytes), "s"(base), "s"(m0v) : "memory", "m0");
}

// The same copy with the non-temporal cache policy (nt): for data each
// workgroup reads once and no other one re-reads soon, so that it does not
// push shared data out of L2.  (Measured on the GQA path's K and V tiles:
// 175 us against 195 us per DSV3 call; on its shared rope tiles it costs.)
__device__ __forceinline__ void dma16_nt(const void* base, uint32_t voff_bytes, lds_u8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff_bytes), "s"(base), "s"(m0v) : "memory", "m0");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima),
// followed by a compiler barrier so LDS reads are not hoisted above it.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Scalar load of one wave-uniform int32 (e.g. a block-table entry).  Done in
// asm with its wait in the same block: a vector load here would make the wave
// wait on every vector-memory operation in flight (the in-order vmcnt),
// including the tile prefetches, while the scalar path only uses lgkmcnt.
// `ptr` must be wave-uniform and 4-byte aligned.
__device__ __forceinline__ int sload_i32(const int32_t* ptr) {
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}

// Scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier for LDS hand-offs: this wave's LDS reads and writes are
// complete before it arrives.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Swizzle of 16-byte chunk positions inside a token row (tokens 0..31 of a
// tile; requires 8 | chunks per row): the low three chunk bits are XOR-ed with
// f(t) = 4 ((t >> 1) & 1) + 2 ((t >> 2) & 1).  gfx950 LDS has 64 four-byte
// banks; a 16-byte read is served in four passes of 16 lanes (per half wave,
// the 4-lane quads of even bit parity and those of odd parity), an 8-byte or
// transposing read in two passes of 32 lanes.  With a 1152-byte token row
// (token t starts at 16-byte slot 8 (t & 1) mod 16) this f makes every pass of
// both readers hit 64 distinct banks: the QK reads (16 tokens x 4 consecutive
// chunks per instruction) and the PV transposing reads (4 consecutive tokens x
// 4 chunks per pass), checked exhaustively against that pass model over all
// chunk offsets.
__device__ __forceinline__ int tile_swz(int t) { return 4 * ((t >> 1) & 1) + 2 * ((t >> 2) & 1); }

// The sequence that owns unit u under a split plan: the last b with
// offs[b] <= u (the offsets are nondecreasing prefix sums from offs[0] = 0),
// its first unit offs[b] and its length lens[b].  One load per lane and 64
// sequences (lane j reads offs[j] and lens[j]; the owner's values come from
// its lane), rather than a chain of dependent loads.  u must be wave-uniform
// and below offs[batch]; every lane of the wave must be active.
struct UnitOwner {
  int b, first, len;
};
__device__ __forceinline__ UnitOwner unit_owner(const int32_t* __restrict__ offs, const int32_t* __restrict__ lens,
                                                int batch, int u) {
  const int lane = (int)(threadIdx.x & 63);
  UnitOwner r = {0, 0, 0};
  int cnt = 0;
  for (int c0 = 0; c0 < batch; c0 += 64) {
    const int j = c0 + lane;
    const bool in = j < batch;
    const int oj = in ? offs[j] : 0x7fffffff;
    const int lj = in ? lens[j] : 0;
    const int nb = __builtin_popcountll(__builtin_amdgcn_ballot_w64(oj <= u));
    if (nb > 0) {                                 // the last candidate so far is lane nb - 1
      r.first = __builtin_amdgcn_readlane(oj, nb - 1);
      r.len = __builtin_amdgcn_readlane(lj, nb - 1);
    }
    cnt += nb;
    if (nb < 64) break;                           // the prefix ends in this chunk
  }
  r.b = cnt - 1;
  return r;
}

}  // namespace gqla
