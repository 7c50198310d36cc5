// MQA-absorb decode over the shared latent cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "MQA-absorb path" and
// gist.science section 2 "MQA-Absorb-Pfad": W_UK[G] is folded into the query
// of every head, all h_q heads attend over the latent cache c^KV_t ++ k_rope_t
// (read once and shared by every query row), and W_UV[G] up-projects the
// latent output.  Per query row (head h in group G, MTP row i):
//   q_abs = W_UK[G] q_nope,   s_t = (q_abs . c_t + q_rope . k_rope_t) * scale,
//   o_lat = softmax(s) C,     out = o_lat W_UV[G].
//
// Three kernels per call:
//   1. absorb_prologue_kernel: q_abs for every query row of the batch (per
//      group a [rows x d_nope] x [d_nope x r] MFMA product), stored with
//      q_rope as one bf16 row of r + d_R in the workspace, and, in the same
//      launch, W_UV^T [g][d_v][r] (the up-projection's A operand is then one
//      16-byte load);
//   2. absorb_decode_kernel: attention over the latent cache, one workgroup
//      of four waves (one per SIMD, so each wave may hold 512 registers) per
//      (split of a sequence, block of 128 query rows); it writes the split's
//      normalised o_lat (bf16) and lse into the workspace;
//   3. absorb_merge_kernel: per (group, block of sequences), the log-sum-exp
//      merge of the splits' o_lat and the up-projection by W_UV[G].
// The up-projection runs once per sequence after the merge (exact by
// linearity) rather than once per split: every split of a sequence covers all
// g groups, so up-projecting per split would pull all of W_UV through each
// workgroup, as many bytes as its share of the cache.
//
// Decode kernel.  Each 32-token latent tile (36 KB for r + d_R = 576) is
// copied HBM -> LDS by direct DMA (global_load_lds_dwordx4; four tile buffers:
// tile it is multiplied by Q, tile it-1 by P, tiles it+1 and it+2 in flight)
// into an XOR-swizzled token-major layout.  Wave w owns 32 query rows end to
// end, on the 32x32x16 bf16 MFMA:
//   * its query rows (32 rows x the full r + d_R contraction) stay in
//     registers as B operands;
//   * S^T[32 tokens][32 rows] = C_tile Q^T: one 16-byte LDS read per MFMA;
//   * online softmax inside the wave: lane l holds row l%32 and 16 of the 32
//     tokens, so a row reduction is 16 in-lane values and one cross-half swap;
//     relabelling the tokens inside each 16-token k step makes the S^T
//     accumulators exactly the P^T B operands of the PV product;
//   * O^T[latent][row] += C^T P^T over all r latent dims: the O accumulators
//     (32 rows x 512 fp32) live in the accumulation registers; the C^T
//     operands come from the transposing LDS read ds_read_b64_tr_b16.
// One workgroup barrier per tile (copies landed, and the buffer refilled next
// has been read by every wave).  PV of tile it-1 runs after QK of tile it, so
// the softmax of tile it overlaps the PV MFMAs.
// Epilogue: o_lat is normalised, staged as bf16 in LDS and written out one
// full 1 KB row per store instruction.
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS hand-offs: this wave's LDS reads and writes are
// complete before it arrives.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Outstanding-copy counts are wave-uniform but not compile-time constants.
__device__ __forceinline__ void vm_wait_dyn(int n) {
  switch (n) {
#define GQLA_WV(N) case N: vm_wait<N>(); break;
    GQLA_WV(0) GQLA_WV(1) GQLA_WV(2) GQLA_WV(3) GQLA_WV(4) GQLA_WV(5) GQLA_WV(6) GQLA_WV(7)
    GQLA_WV(8) GQLA_WV(9) GQLA_WV(10) GQLA_WV(11) GQLA_WV(12) GQLA_WV(13) GQLA_WV(14) GQLA_WV(15)
    GQLA_WV(16) GQLA_WV(17) GQLA_WV(18) GQLA_WV(19) GQLA_WV(20) GQLA_WV(21) GQLA_WV(22) GQLA_WV(23)
#undef GQLA_WV
    default: vm_wait<0>(); break;
  }
}

template <int HPG, int SQ, int R, int DR, int DN, int DV>
struct AbsorbCfg {
  static constexpr int BS = 64;
  static constexpr int TILE = 32;                 // tokens per LDS tile
  static constexpr int NBUF = 4;                  // tile buffers (the copy of tile it+3 goes out at step it)
  static constexpr int ROW = R + DR;              // latent row (elements)
  static constexpr int CHR = ROW / 8;             // 16-byte chunks per token row
  static constexpr bool SWZ = (CHR % 8) == 0;     // XOR swizzle stays inside a row
  static constexpr int BUF_BYTES = TILE * ROW * 2;
  static constexpr int NI = TILE * CHR / 64;      // wave-wide DMA instructions per tile
  static constexpr int NW = 4;                    // waves per workgroup (one per SIMD)
  static constexpr int NIW = (NI + NW - 1) / NW;  // most DMA instructions of one wave per tile
  static constexpr int ROWS_W = 32;               // query rows per wave
  static constexpr int ROWS_WG = NW * ROWS_W;
  static constexpr int KQ = ROW / 16;             // k steps of S^T = C Q^T
  static constexpr int MT = R / 32;               // 32-dim tiles of O^T
  static constexpr int MD = DV / 16;              // 16-dim tiles of the output
  static constexpr int OL_STRIDE = 2 * R + 16;    // LDS row stride of the staged o_lat (bytes)
  static constexpr int OFF_VOTE = NBUF * BUF_BYTES;          // restart votes [2 slots][NW waves]
  static constexpr int LDS_BYTES = OFF_VOTE + 32;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(NW * ROWS_W * OL_STRIDE <= NBUF * BUF_BYTES, "o_lat staging fits in the tile buffers");
  static_assert((TILE * CHR) % 64 == 0, "tile must be whole DMA instructions");
  static_assert(ROW % 16 == 0 && R % 32 == 0 && DN % 32 == 0 && DV % 16 == 0, "unsupported dims");
  static_assert(NIW * 2 <= 63, "vmcnt budget");
};

// Swizzle of 16-byte chunk positions inside a token row (tokens 0..31 of a
// tile; requires 8 | chunks per row).  gfx950 LDS has 64 four-byte banks; a
// 16-byte read is served in four passes of 16 lanes (per half wave, the
// 4-lane quads of even bit parity and those of odd parity), an 8-byte or
// transposing read in two passes of 32 lanes.  With a 1152-byte token row,
// token t starts at bank slot 8 (t & 1) (16-byte slots mod 16).  XOR-ing the
// low three chunk bits with f(t) = 4 ((t >> 1) & 1) + ((t >> 3) & 3) gives:
//   * QK reads (one chunk of 16 tokens per pass): (t & 1, f(t)) is distinct
//     over the tokens of each pass, so the 16 slots are distinct;
//   * PV transposing reads (4 consecutive tokens x 4 chunks per pass): tokens
//     t and t + 2 differ in bit 2 of f, so their chunk quads land on disjoint
//     slots, and t, t + 1 differ in the slot's bit 3.
__device__ __forceinline__ int tile_swz(int t) { return 4 * ((t >> 1) & 1) + ((t >> 3) & 3); }

template <int HPG, int SQ, int R, int DR, int DN, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void absorb_decode_kernel(DecodeParams p) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KQ = C::KQ, MT = C::MT, MD = C::MD, NW = C::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  // Workgroups are dispatched round-robin over the 8 XCDs.  XCD x takes the
  // contiguous unit range [x * UPX, (x + 1) * UPX), so the splits of one
  // sequence (consecutive units) share an L2 for their query rows, and the
  // row blocks of one unit take consecutive slots on one XCD.
  const int UPX = (p.num_units + 7) / 8;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int u = xcd * UPX + k / RB;
  const int rb = k % RB;
  if (u >= p.num_units) return;                   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int hh = lane >> 5;                       // half wave
  int b, lo, hi;
  if (p.split_offsets) {
    b = split_owner(p.split_offsets, p.batch, u);
    const int j = u - p.split_offsets[b];
    lo = j * p.split_tokens;
    hi = min(lo + p.split_tokens, p.seqlens[b]);
  } else {
    b = u;
    lo = 0;
    hi = p.seqlens[b];
  }
  b = __builtin_amdgcn_readfirstlane(b);
  lo = __builtin_amdgcn_readfirstlane(lo);
  hi = __builtin_amdgcn_readfirstlane(hi);
  const int L = __builtin_amdgcn_readfirstlane(p.seqlens[b]);
  const int n_tiles = hi > lo ? (hi - lo + C::TILE - 1) / C::TILE : 0;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;     // wave-uniform

  // ---- HBM -> LDS tile copies: wave w issues instructions w, w+4, ... ----
  // Block-table entries are read through the scalar cache (constant address
  // space, wave-uniform index).  LDS position P (16-byte chunk index inside
  // the tile) holds token P / CHR, physical chunk P % CHR, i.e. logical chunk
  // (P % CHR) ^ f(token); the per-lane source offsets are the same for every
  // tile and are computed once.
  typedef const __attribute__((address_space(4))) int32_t cint32_t;
  const cint32_t* const cbt = (const cint32_t*)bt;
  constexpr bool kFixedCopies = (C::NI % NW) == 0;   // every wave issues NIW copies per tile
  const int niw = kFixedCopies ? C::NIW : (C::NI - w + NW - 1) / NW;
  uint32_t dvo[C::NIW];
#pragma unroll
  for (int kk = 0; kk < C::NIW; ++kk) {
    const int i = min(w + NW * kk, C::NI - 1);
    const int P = i * 64 + lane;
    const int t = P / CHR, pos = P % CHR;
    const int ch = C::SWZ ? (pos ^ tile_swz(t)) : pos;
    dvo[kk] = (uint32_t)(t * ROW + ch * 8) * 2u;
  }
  struct Copy {
    const uint16_t* src;
    lds_u8_t* dst;
  };
  auto copy_of = [&](int it) -> Copy {
    const int t0 = lo + C::TILE * it;
    const int page = cbt[t0 / BS];
    return Copy{p.cache + ((size_t)page * BS + (t0 % BS)) * ROW, lds + (it % C::NBUF) * C::BUF_BYTES};
  };
  auto copy_part = [&](const Copy& cp, int kk) {  // instruction kk of this wave (kk < niw)
    dma16(cp.src, dvo[kk], cp.dst + (w + NW * kk) * 1024);
  };

  // The copies of tiles 0, 1 and 2 go out first; the query loads follow.
  auto issue_head = [&]() {
    for (int i = 0; i < C::NBUF - 1 && i < n_tiles; ++i) {
      const Copy cp = copy_of(i);
      for (int kk = 0; kk < niw; ++kk) copy_part(cp, kk);
    }
  };
  issue_head();

  // ---- this wave's query rows: lane l holds row row0 + l%32 ----
  const int row0 = rb * C::ROWS_WG + C::ROWS_W * w;
  const bool active = row0 < rows_total;          // wave-uniform
  const int rq = row0 + (lane & 31);
  const bool rvalid = rq < rows_total;
  const int h_q = rvalid ? rq / SQ : 0, i_q = rvalid ? rq % SQ : 0;
  const int nvis = rvalid ? L - SQ + i_q + 1 : -1;  // tokens t < nvis are visible to this row
  bf16x8 qb[KQ];                                  // B operands: Q[row][16 ks + 8 hh .. +7]
  {
    const uint16_t* qrow = p.qcat + (((size_t)b * SQ + i_q) * H + h_q) * ROW;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) qb[ks] = rvalid ? ld_bf16x8(qrow + 16 * ks + 8 * hh) : zero_bf16x8();
  }

  // Per-lane LDS byte offsets of the MFMA operands inside a tile buffer.
  // QK A operand of k step ks: token lane%32, logical chunk 2 ks + hh, which
  // sits at 8 (ks >> 2) + ((2 (ks & 3) + hh) ^ f): one base per ks & 3, the
  // rest an immediate of 128 (ks >> 2) bytes.
  const int tq = lane & 31;
  int qkb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = C::SWZ ? ((2 * j + hh) ^ tile_swz(tq)) : (2 * j + hh);
    qkb[j] = tq * ROW * 2 + ch * 16;
  }
  auto qk_addr = [&](int ks) -> int {
    return C::SWZ ? qkb[ks & 3] + 128 * (ks >> 2) : qkb[0] + 32 * ks;
  };
  // PV A operand (C^T, 32 latent dims x 16 tokens) of tile mt, k step kk:
  // k index 8 hh + j stands for token 16 kk + 8 (j / 4) + 4 hh + j % 4, the
  // order in which the S^T accumulators hold the tokens.  Two transposing
  // reads (rd = j / 4); in read rd the 16-lane group gq = lane / 16 reads
  // tokens 16 kk + 8 rd + 4 (gq / 2) + s / 4 (s = lane % 16), dims
  // 32 mt + 16 (gq % 2) + 4 (s % 4) .. +3, so lane s receives dim
  // 32 mt + 16 (gq % 2) + s of four consecutive tokens.  Logical chunk
  // 4 mt + x (x = 2 (gq % 2) + (s % 4) / 2) sits at
  // 4 (mt ^ (s >> 3)) + (x ^ (rd + 2 kk)) under the swizzle: one base per
  // (rd, kk, mt & 1), the rest an immediate of 128 (mt >> 1) bytes.
  const int gq = lane >> 4, s16 = lane & 15;
  int pvb[2][2][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
        const int t = 16 * kk + 8 * rd + 4 * (gq >> 1) + (s16 >> 2);
        const int x = 2 * (gq & 1) + ((s16 & 3) >> 1);
        const int ch = C::SWZ ? 4 * (mp ^ ((s16 >> 3) & 1)) + (x ^ (rd + 2 * kk)) : 4 * mp + x;
        pvb[rd][kk][mp] = t * ROW * 2 + ch * 16 + 8 * (s16 & 1);
      }
  auto pv_operand = [&](const lds_u8_t* buf, int mt, int kk) -> bf16x8 {
    const int imm = C::SWZ ? 128 * (mt >> 1) : 128 * (mt >> 1);
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[0][kk][mt & 1] + imm));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[1][kk][mt & 1] + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Softmax reference.  A row's reference is the maximum of its first tile
  // and then stays fixed, so the O accumulators are only ever written by
  // MFMAs (a rescale of the accumulation registers by the vector ALU would
  // also make the compiler move them out of those registers).  Every
  // p = 2^(x - ref) is kept below 2^kSlack: a tile whose logits exceed
  // ref + kSlack on some row (an extreme logit spread, e.g. one dominant
  // token) makes the workgroup restart the split: pass 1 sweeps QK for the
  // exact row maxima, pass 2 reruns the attention with them as the
  // references (then p <= 1).
  constexpr float kSlack = 64.f;
  f32x16 o[MT];                                   // O^T: lane l = row l%32, latent 32 mt + 8 (i/4) + 4 hh + i%4
  float m_ref = -INFINITY, l_run = 0.f;
  bf16x8 pb[2];                                   // P^T operands of the previous tile (k steps 0, 1)
  typedef __attribute__((address_space(3))) int lds_i32_t;
  // Restart votes, two slots of one int per wave: the vote of the softmax of
  // tile it goes to slot (it + 1) & 1 (every wave stores its own entry every
  // tile, so nothing needs resetting) and is read after the barrier of
  // iteration it + 1; slot it & 1 is read right after the barrier of
  // iteration it, which every wave has passed before any wave writes that
  // slot again.
  lds_i32_t* const votes = (lds_i32_t*)(lds + C::OFF_VOTE);
  if (tid < 2 * NW) votes[tid] = 0;               // ordered before their reads by the first barrier

  // Query loads and the first copies complete before the tile loop, so the
  // compiler's own wait tracking has nothing pending inside it.
  vm_wait<0>();

  // Top of the step for tile it: tile it landed (the copies of tiles it+1
  // and it+2, issued after it, may still be in flight; copies complete in
  // order), then for every wave; the tail of the sequence's last tile is
  // zeroed (token rows past its end hold anything, and 0 * NaN would still be
  // NaN in the PV product).
  auto tile_top = [&](int it) {
    const int later = (it + 1 < n_tiles) + (it + 2 < n_tiles);
    if constexpr (kFixedCopies) {
      if (later == 2) vm_wait<2 * C::NIW>(); else if (later == 1) vm_wait<C::NIW>(); else vm_wait<0>();
    } else {
      vm_wait_dyn(later * niw);
    }
    block_sync_lds();
    if (it < n_tiles && lo + C::TILE * (it + 1) > L) {
      const int valid = L - (lo + C::TILE * it);
      lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
      for (int off = valid * ROW * 2 + tid * 16; off < C::BUF_BYTES; off += 64 * NW * 16)
        *(lds_u32x4_t*)(buf + off) = u32x4{0u, 0u, 0u, 0u};
      block_sync_lds();
    }
  };
  // The copies of tile it+3 go out into the buffer of tile it-1 as soon as
  // every wave is past its PV product (a barrier in the middle of step it),
  // so three tiles are in flight for most of a step.
  auto issue_ahead = [&](int it) {
    if (it + C::NBUF - 1 < n_tiles) {
      const Copy cp = copy_of(it + C::NBUF - 1);
      for (int kk = 0; kk < niw; ++kk) copy_part(cp, kk);
    }
  };
  // S^T of tile it over the full contraction
  auto qk_tile = [&](int it) -> f32x16 {
    f32x16 s = {};
    const lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
    auto qk_operand = [&](int ks) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + qk_addr(ks)));
    };
    constexpr int PD = 4;                         // operands read ahead
    bf16x8 a[PD + 1];
#pragma unroll
    for (int j = 0; j < PD && j < KQ; ++j) a[j] = qk_operand(j);
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
      if (j + PD < KQ) a[(j + PD) % (PD + 1)] = qk_operand(j + PD);
      s = mfma32(a[j % (PD + 1)], qb[j], s);
    }
    // schedule: the first PD operand reads, then per step the read of
    // operand j + PD followed by the MFMA of step j
    __builtin_amdgcn_sched_group_barrier(0x100, PD < KQ ? PD : KQ, 0);
#pragma unroll
    for (int j = 0; j < KQ; ++j) {
      if (j + PD < KQ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    return s;
  };
  // visibility of lane l's 16 logits of tile it (token t0 + 8 (i / 4) + 4 hh + i % 4)
  auto visible = [&](int it, int i) -> bool {
    return lo + C::TILE * it + 8 * (i >> 2) + 4 * hh + (i & 3) < nvis;
  };
  auto pack_p = [&](const float (&x)[16], bf16x8 (&pn)[2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      pn[kk] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(x[8 * kk + 0], x[8 * kk + 1]), pack_bf16x2(x[8 * kk + 2], x[8 * kk + 3]),
                        pack_bf16x2(x[8 * kk + 4], x[8 * kk + 5]), pack_bf16x2(x[8 * kk + 6], x[8 * kk + 7])});
  };
  float m_half = -INFINITY;                       // pass 1: running maximum of this lane's half row
  for (int pass = 0; pass < 3; ++pass) {          // 0: single pass; 1, 2: after a restart
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = f32x16{};
    l_run = 0.f;
    if (pass > 0) issue_head();                   // the first tiles again after a restart
    // ---- tile 0 of the split: sets each row's reference (pass 0) ----
    float ps_prev = 0.f;                          // P sum of the previous tile
    tile_top(0);
    issue_ahead(0);                               // buffer 3 is still unused
    if (active) {
      const f32x16 s = qk_tile(0);
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = visible(0, i) ? s[i] * p.scale_log2 : -INFINITY;
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
      m_half = fmaxf(m_half, mx);
      if (pass == 0) {
        float a0 = mx, a1 = mx;
        swap_pairs32(a0, a1);
        m_ref = fmaxf(a0, a1);                    // -inf for a row that sees none of it
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = __builtin_amdgcn_exp2f(x[i] - m_use);
        ps_prev += x[i];
      }
      pack_p(x, pb);
    }
    // ---- steps it = 1 .. n_tiles: S of tile it, the PV product of tile
    // it-1, then the softmax of tile it ----
    bool restart = false;
    for (int it = 1; it <= n_tiles; ++it) {
      tile_top(it);
      // restart votes raised before this barrier (pass 0 only)
      int flag = 0;
      if (pass == 0) {
        const u32x4 vt = *(volatile lds_u32x4_t*)(lds + C::OFF_VOTE + 16 * (it & 1));
        flag = (int)(vt[0] | vt[1] | vt[2] | vt[3]);
      }
      f32x16 s = {};
      if (it < n_tiles && active) s = qk_tile(it);
      if (__builtin_amdgcn_readfirstlane(flag)) { // uniform over the workgroup
        restart = true;
        break;
      }
      if (active && pass != 1) {
        l_run += ps_prev;
        // O^T += C^T P^T for tile it-1
        const lds_u8_t* buf = lds + ((it - 1) % C::NBUF) * C::BUF_BYTES;
        constexpr int NS = 2 * MT;                // (kk, mt) steps
        constexpr int PV = 4;
        bf16x8 v[PV + 1];
#pragma unroll
        for (int j = 0; j < PV && j < NS; ++j) v[j] = pv_operand(buf, j % MT, j / MT);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (j + PV < NS) v[(j + PV) % (PV + 1)] = pv_operand(buf, (j + PV) % MT, (j + PV) / MT);
          o[j % MT] = mfma32(v[j % (PV + 1)], pb[j / MT], o[j % MT]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV, 0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (j + PV < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      }
      if (it == n_tiles) break;
      block_sync_lds();                           // every wave is past PV of tile it-1
      issue_ahead(it);
      if (active) {
        // Softmax of tile it, branch-free: masking by select, every row's
        // reference fixed, no cross-lane step; each lane checks its own 16
        // logits against ref + kSlack (the vote).
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
        const float thr = m_ref + kSlack;
        float x[16], mx = -INFINITY, ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool vis = visible(it, i);
          const float xl = s[i] * p.scale_log2;
          mx = fmaxf(mx, vis ? xl : -INFINITY);
          x[i] = vis ? __builtin_amdgcn_exp2f(xl - m_use) : 0.f;
          ps += x[i];
        }
        m_half = fmaxf(m_half, mx);
        votes[NW * ((it + 1) & 1) + w] = __builtin_amdgcn_ballot_w64(mx > thr) != 0 ? 1 : 0;
        ps_prev = ps;
        pack_p(x, pb);
      }
    }
    if (pass == 0 && !restart) break;             // the common case: done in one pass
    if (pass == 1) {                              // the exact row maxima, for pass 2
      float a0 = m_half, a1 = m_half;
      swap_pairs32(a0, a1);
      m_ref = fmaxf(a0, a1);
    }
    // drain this pass's copies before the tile buffers are refilled
    vm_wait<0>();
    block_sync_lds();
    if (pass == 0) m_half = -INFINITY;
  }

  // ---- epilogue ----
  // Every wave is past its last read of the tile buffers before any o_lat
  // row is staged over them.
  block_sync_lds();
  if (!active) return;                            // no barrier follows
  float lt = l_run;
  {
    float a0 = lt, a1 = lt;
    swap_pairs32(a0, a1);
    lt = a0 + a1;                                 // lanes l, l ^ 32 hold the two token halves of a row
  }
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (hh == 0 && rvalid)
    p.olse[((size_t)u * SQ + i_q) * H + h_q] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
  // normalised o_lat rows of this wave as bf16 in LDS: row r (of 32) at
  // r * OL_STRIDE, latent-major; then one 1 KB row per store instruction
  lds_u8_t* const ol = lds + w * C::ROWS_W * C::OL_STRIDE;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int lat = 32 * mt + 8 * a + 4 * hh;
      const f32x16& om = o[mt];
      u32x2 pk = {pack_bf16x2(om[4 * a] * inv, om[4 * a + 1] * inv), pack_bf16x2(om[4 * a + 2] * inv, om[4 * a + 3] * inv)};
      *(__attribute__((address_space(3))) u32x2*)(ol + tq * C::OL_STRIDE + 2 * lat) = pk;
    }
  for (int j = 0; j < C::ROWS_W; ++j) {
    const int rho = row0 + j;                     // uniform
    if (rho >= rows_total) break;
    uint16_t* dst = p.olat + (((size_t)u * SQ + rho % SQ) * H + rho / SQ) * R;
    for (int e = lane; e < R / 8; e += 64)
      *reinterpret_cast<u32x4*>(dst + 8 * e) = *(const lds_u32x4_t*)(ol + j * C::OL_STRIDE + 16 * e);
  }
}

// Merge of the split partials and up-projection, per (group G, block of SB
// sequences): for each query row of the block,
//   m = max_s lse_s,  w_s = exp(lse_s - m),  o = sum_s w_s o_lat_s / sum_s w_s,
//   lse = m + ln sum_s w_s,  out = o W_UV[G].
// o is split into bf16 hi + lo (o - hi, rounded), both multiplied on the
// 16x16x32 MFMA, so the merge adds no bf16 rounding of its own.  W_UV^T[G] is
// read once per workgroup.  Without a split plan each sequence is one split
// (w = 1, lo = 0).
template <int HPG, int SQ, int R, int DV>
__global__ __launch_bounds__(512) void absorb_merge_kernel(DecodeParams p) {
  constexpr int NWM = 8;                            // waves
  constexpr int RG = HPG * SQ;                      // rows of one group per sequence
  constexpr int SB = RG >= 32 ? 1 : 32 / RG;        // sequences per workgroup
  constexpr int NR = SB * RG;                       // rows per workgroup
  constexpr int NT = NR / 16;                       // 16-row tiles
  constexpr int STR = 2 * R + 16;                   // LDS row stride (bytes)
  constexpr int MD = DV / 16;                       // 16-dim output tiles
  constexpr int RPW = NR / NWM;                     // rows per wave in the merge
  constexpr int SC = 4;                             // splits per load batch
  constexpr int NCH = (R / 8 + 63) / 64;            // 8-latent chunks per lane
  static_assert(NR <= 32 && NR % 16 == 0 && NR % NWM == 0, "merge tiling");
  static_assert(MD <= NWM, "one output tile per wave");
  __shared__ __attribute__((aligned(16))) unsigned char sm_raw[2 * NR * STR];
  lds_u8_t* const sm = (lds_u8_t*)sm_raw;
  const int G = blockIdx.y, b0 = blockIdx.x * SB;
  const int H = HPG * p.num_groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  // W_UV^T[G] operands of this wave's output tile md = w, loaded first so that
  // they arrive during the merge
  const uint16_t* WT = p.wuvT + (size_t)G * DV * R;
  const int md = w < MD ? w : 0;
  bf16x8 wa[R / 32];
#pragma unroll
  for (int kk = 0; kk < R / 32; ++kk) wa[kk] = ld_bf16x8(WT + (size_t)(16 * md + c) * R + 32 * kk + 8 * q);

  // ---- merge: wave w takes rows w, w + 8, ...; lane l holds latent 8l .. 8l+7
  // of the row (one coalesced 1 KB row per load instruction).  The loads (lse
  // and o_lat) of up to SC splits of all the wave's rows are issued
  // together, and the running maximum moves (acc, wsum rescaled) when a
  // batch raises it. ----
  int s0[RPW], ns[RPW], rowi[RPW], rowh[RPW];
  float m[RPW], wsum[RPW];
  float acc[RPW][NCH][8];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rr = w + NWM * j;
    const int b = b0 + rr / RG, lr = rr % RG;
    const bool bv = b < p.batch;
    const int bc = bv ? b : 0;                      // loads stay in bounds, no branch
    const int o0 = p.split_offsets ? p.split_offsets[bc] : bc;
    const int o1 = p.split_offsets ? p.split_offsets[bc + 1] : bc + 1;
    rowh[j] = G * HPG + lr / SQ;
    rowi[j] = lr % SQ;
    s0[j] = o0;
    ns[j] = bv ? o1 - o0 : 0;
    m[j] = -INFINITY;
    wsum[j] = 0.f;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][cc][e] = 0.f;
  }
  int smax = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) smax = max(smax, ns[j]);
  for (int sb = 0; sb < smax; sb += SC) {
    u32x4 v[RPW][SC][NCH];
    float ls[RPW][SC];
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int k = 0; k < SC; ++k) {
        const int s = sb + k;
        const bool have = s < ns[j];
        const size_t row = ((size_t)(s0[j] + (have ? s : 0)) * SQ + rowi[j]) * H + rowh[j];
        ls[j][k] = have ? p.olse[row] : -INFINITY;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          const int ch = lane + 64 * cc;
          v[j][k][cc] = (have && ch < R / 8) ? *reinterpret_cast<const u32x4*>(p.olat + row * R + 8 * ch)
                                             : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      float bm = ls[j][0];
#pragma unroll
      for (int k = 1; k < SC; ++k) bm = fmaxf(bm, ls[j][k]);
      const float mn = fmaxf(m[j], bm);
      if (mn == -INFINITY) continue;               // nothing visible yet (uniform)
      const float sc = m[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m[j] - mn) * kLog2e);
      m[j] = mn;
      wsum[j] *= sc;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][cc][e] *= sc;
#pragma unroll
      for (int k = 0; k < SC; ++k) {
        const float wt = ls[j][k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((ls[j][k] - mn) * kLog2e);
        wsum[j] += wt;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[j][cc][2 * e] += wt * bf_bits2f(v[j][k][cc][e] & 0xffffu);
            acc[j][cc][2 * e + 1] += wt * bf_bits2f(v[j][k][cc][e] >> 16);
          }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rr = w + NWM * j;
    const int b = b0 + rr / RG;
    if (lane == 0 && b < p.batch && p.lse)
      p.lse[((size_t)b * SQ + rowi[j]) * H + rowh[j]] = m[j] > -INFINITY ? m[j] + logf(wsum[j]) : -INFINITY;
    const float inv = wsum[j] > 0.f ? 1.f / wsum[j] : 0.f;
#pragma unroll
    for (int cc = 0; cc < NCH; ++cc) {
      const int ch = lane + 64 * cc;
      if (ch >= R / 8) break;
      u32x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = acc[j][cc][2 * e] * inv, x1 = acc[j][cc][2 * e + 1] * inv;
        const uint32_t hb = pack_bf16x2(x0, x1);
        hi[e] = hb;
        lo[e] = pack_bf16x2(x0 - bf_bits2f(hb & 0xffffu), x1 - bf_bits2f(hb >> 16));
      }
      *(lds_u32x4_t*)(sm + rr * STR + 16 * ch) = hi;
      *(lds_u32x4_t*)(sm + (NR + rr) * STR + 16 * ch) = lo;
    }
  }
  __syncthreads();
  // ---- out^T[d][row] = W_UV^T[G][d][:] . (hi + lo)[row][:], output tile md
  // of this wave (lane (q, c) = D[4q..][c]) ----
  if (w >= MD) return;
  f32x4 oacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < R / 32; ++kk)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int off = (16 * nt + c) * STR + 2 * (32 * kk + 8 * q);
      oacc[nt] = mfma16(wa[kk], __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(sm + off)), oacc[nt]);
      oacc[nt] = mfma16(wa[kk], __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(sm + NR * STR + off)), oacc[nt]);
    }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rr = 16 * nt + c;
    const int b = b0 + rr / RG, lr = rr % RG;
    if (b >= p.batch) continue;
    const int h = G * HPG + lr / SQ, i = lr % SQ;
    u32x2 pk = {pack_bf16x2(oacc[nt][0], oacc[nt][1]), pack_bf16x2(oacc[nt][2], oacc[nt][3])};
    *reinterpret_cast<u32x2*>(p.out + (((size_t)b * SQ + i) * H + h) * DV + 16 * md + 4 * q) = pk;
  }
}

// q_abs = W_UK[G] q_nope for every (sequence, MTP row, head), written next to
// q_rope as one [r + d_R] bf16 row per query row (the QK operand of the decode
// kernel).  Per group this is a [rows x d_nope] x [d_nope x r] product over all
// rows of the batch.  Workgroup = 4 waves x 32 query rows of one group and a
// chunk of up to 128 latent dims; D = q_abs^T (m = latent, n = row), so each
// W_UK operand feeds the wave's two 16-row tiles and each lane stores 4
// consecutive latent values of one row.  Every operand load is issued before
// the first product, so the wave waits for memory once.
template <int HPG, int SQ, int R, int DR, int DN>
__device__ __forceinline__ void absorb_q_block(const DecodeParams& p, int bx, int G, int bz) {
  constexpr int ROW = R + DR, KD = DN / 32, MT = R / 16;
  constexpr int MTC = MT < 8 ? MT : 8;               // latent tiles per workgroup (blockIdx.z)
  constexpr int NT = 2;                              // 16-row tiles per wave
  const int g = p.num_groups, H = HPG * g;
  const int rows_g = p.batch * SQ * HPG;             // query rows of one group
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int r0 = (bx * 4 + w) * 16 * NT;             // first group-row of this wave
  if (r0 >= rows_g) return;
  // group-row gr = (b * SQ + i) * HPG + hl  ->  head h = G*HPG + hl
  const uint16_t* W = p.w_uk + (size_t)G * R * DN;
  const int mt0 = bz * MTC;
  bf16x8 wa[MTC][KD];
#pragma unroll
  for (int m = 0; m < MTC; ++m)
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) wa[m][kd] = ld_bf16x8(W + (size_t)(16 * (mt0 + m) + c) * DN + 32 * kd + 8 * q);
  bf16x8 qn[NT][KD];
  size_t qrow[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int gr = r0 + 16 * nt + c;
    valid[nt] = gr < rows_g;
    const int hl = gr % HPG, bi = gr / HPG;          // bi = b * SQ + i
    qrow[nt] = (size_t)bi * H + G * HPG + hl;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      qn[nt][kd] = valid[nt] ? ld_bf16x8(p.q_nope + qrow[nt] * DN + 32 * kd + 8 * q) : zero_bf16x8();
  }
#pragma unroll
  for (int m = 0; m < MTC; ++m) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) acc = mfma16(wa[m][kd], qn[nt][kd], acc);
      // lane (q, c): latent 16 (mt0 + m) + 4q .. +3 of row (nt, c)
      if (valid[nt]) {
        u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
        *reinterpret_cast<u32x2*>(p.qcat + qrow[nt] * ROW + 16 * (mt0 + m) + 4 * q) = pk;
      }
    }
  }
  // rope part copied unchanged
  if (bz != 0) return;
  for (int id = lane; id < 16 * NT * DR / 8; id += 64) {
    const int rr = id / (DR / 8), part = id % (DR / 8);
    const int gr2 = r0 + rr;
    if (gr2 >= rows_g) continue;
    const size_t qr2 = ((size_t)(gr2 / HPG) * H + G * HPG + gr2 % HPG);
    *reinterpret_cast<u32x4*>(p.qcat + qr2 * ROW + R + part * 8) =
        *reinterpret_cast<const u32x4*>(p.q_rope + qr2 * DR + part * 8);
  }
}

// W_UV[G] (r x d_v) -> W_UV^T[G] (d_v x r), through an LDS tile of 64 latent
// rows x TD columns: 16-byte reads of W_UV rows, 2-byte transposed LDS
// writes, 16-byte reads of LDS rows and 16-byte writes of W_UV^T rows.
template <int R, int DV>
__device__ __forceinline__ void wuv_transpose_block(const DecodeParams& p, int bx, int by, int G) {
  constexpr int TD = DV < 64 ? DV : 64;              // columns per tile
  constexpr int TS = 64 + 8;                         // LDS row stride (elements), 16-byte aligned
  __shared__ __attribute__((aligned(16))) uint16_t t[TD * TS];
  const int l0 = bx * 64, d0 = by * TD;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * (TD / 8); e += 256) {   // (latent row, 8 columns)
    const int l = e / (TD / 8), dc = (e % (TD / 8)) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(p.w_uv + ((size_t)G * R + l0 + l) * DV + d0 + dc);
#pragma unroll
    for (int j = 0; j < 8; ++j) t[(dc + j) * TS + l] = (uint16_t)(v[j / 2] >> (16 * (j & 1)));
  }
  __syncthreads();
  for (int e = tid; e < TD * 8; e += 256) {          // (column, 8 latent rows)
    const int d = e / 8, lc = (e % 8) * 8;
    *reinterpret_cast<u32x4*>(p.wuvT + ((size_t)G * DV + d0 + d) * R + l0 + lc) =
        *reinterpret_cast<const u32x4*>(&t[d * TS + lc]);
  }
}

// The two prologue steps in one launch: workgroups [0, nq) compute q_abs
// (grid x-major over (row block, group, latent chunk)), the rest transpose
// W_UV tiles (over (latent tile, column tile, group)).
template <int HPG, int SQ, int R, int DR, int DN, int DV>
__global__ __launch_bounds__(256) void absorb_prologue_kernel(DecodeParams p, int qx, int qz) {
  const int g = p.num_groups;
  const int nq = qx * g * qz;
  int id = blockIdx.x;
  if (id < nq) {
    const int bx = id % qx;
    id /= qx;
    absorb_q_block<HPG, SQ, R, DR, DN>(p, bx, id % g, id / g);
  } else {
    id -= nq;
    constexpr int TD = DV < 64 ? DV : 64;
    const int bx = id % (R / 64);
    id /= R / 64;
    wuv_transpose_block<R, DV>(p, bx, id % (DV / TD), id / (DV / TD));
  }
}

template <int HPG, int SQ, int R, int DR, int DN, int DV>
hipError_t launch_absorb(const DecodeParams& p, hipStream_t stream) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  static_assert(R % 64 == 0 && (DV < 64 ? 64 % DV : DV % 64) == 0, "transpose tiling");
  {
    const int rows_g = p.batch * SQ * HPG;
    constexpr int MT = R / 16, MTC = MT < 8 ? MT : 8, TD = DV < 64 ? DV : 64;
    const int qx = (rows_g + 127) / 128, qz = MT / MTC;
    const int nq = qx * p.num_groups * qz, nt = (R / 64) * (DV / TD) * p.num_groups;
    hipLaunchKernelGGL((absorb_prologue_kernel<HPG, SQ, R, DR, DN, DV>), dim3((unsigned)(nq + nt)),
                       dim3(256), 0, stream, p, qx, qz);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int rows_total = HPG * p.num_groups * SQ;
    const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
    const unsigned grid = (unsigned)((p.num_units + 7) / 8) * 8u * (unsigned)RB;
    hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, DN, DV>), dim3(grid), dim3(64 * C::NW), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  constexpr int RG = HPG * SQ, SB = RG >= 32 ? 1 : 32 / RG;
  dim3 grid((unsigned)((p.batch + SB - 1) / SB), (unsigned)p.num_groups);
  hipLaunchKernelGGL((absorb_merge_kernel<HPG, SQ, R, DV>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t absorb_dispatch(int hpg, int sq, int r, int dn, int dv, int dr, const DecodeParams& p,
                           hipStream_t stream, bool* supported) {
  *supported = true;
#define GQLA_ABS_CASE(HPG, SQ, R, DR, DN, DV)                                     \
  if (hpg == HPG && sq == SQ && r == R && dr == DR && dn == DN && dv == DV) \
    return launch_absorb<HPG, SQ, R, DR, DN, DV>(p, stream);
  GQLA_ABS_CASE(16, 1, 512, 64, 128, 128)
  GQLA_ABS_CASE(16, 2, 512, 64, 128, 128)
  GQLA_ABS_CASE(4, 1, 512, 64, 128, 128)
  GQLA_ABS_CASE(4, 2, 512, 64, 128, 128)
  GQLA_ABS_CASE(8, 1, 64, 16, 32, 32)
  GQLA_ABS_CASE(8, 2, 64, 16, 32, 32)
#undef GQLA_ABS_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace gqla
