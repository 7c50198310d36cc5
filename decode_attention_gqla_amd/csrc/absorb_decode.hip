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
//      of eight waves per (split of a sequence, block of 64 query rows); it
//      writes the split's normalised o_lat (bf16) and lse into the workspace;
//   3. absorb_merge_kernel: per (group, block of sequences), the log-sum-exp
//      merge of the splits' o_lat and the up-projection by W_UV[G].
// The up-projection runs once per sequence after the merge (exact by
// linearity) rather than once per split: every split of a sequence covers all
// g groups, so up-projecting per split would pull all of W_UV through each
// workgroup, as many bytes as its share of the cache.
//
// Decode kernel.  Each 32-token latent tile (36 KB for r + d_R = 576) is
// copied HBM -> LDS by direct DMA (global_load_lds_dwordx4; four tile buffers:
// tile it in QK, tile it-1 in PV, tiles it+1 and it+2 in flight) into an
// XOR-swizzled token-major layout.  Two wave roles share every SIMD:
//   * QK waves (16 query rows each, 16x16x32 MFMA): their query rows stay in
//     registers as B operands; S^T = C_tile Q^T; the softmax against a fixed
//     per-row reference; P^T as bf16 into LDS;
//   * PV waves (32x32x16 MFMA): O^T[latent][row] += C^T P^T for their 4 of
//     the 16 latent dim tiles and all 64 rows, O in accumulation registers,
//     C^T from the transposing LDS read ds_read_b64_tr_b16; they also issue
//     the tile copies.
// One workgroup barrier per tile; phase it runs QK of tile it beside PV of
// tile it-1.  Epilogue: o_lat is normalised, staged as bf16 in LDS and
// written out one full 1 KB row per store instruction.
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

__device__ __forceinline__ f32x16 mfma16x32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
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
  static constexpr int NBUF = 4;                  // tile buffers
  static constexpr int ROW = R + DR;              // latent row (elements)
  static constexpr int CHR = ROW / 8;             // 16-byte chunks per token row
  static constexpr bool SWZ = (CHR % 8) == 0;     // XOR swizzle stays inside a row
  static constexpr int BUF_BYTES = TILE * ROW * 2;
  static constexpr int NI = TILE * CHR / 64;      // wave-wide DMA instructions per tile
  static constexpr int NQW = 4;                   // QK waves (one per SIMD)
  static constexpr int NPW = 4;                   // PV waves (one per SIMD); they also issue the copies
  static constexpr int NW = NQW + NPW;
  static constexpr int NIW = (NI + NPW - 1) / NPW;  // most copy instructions of one PV wave per tile
  static constexpr int ROWS_QW = 16;              // query rows per QK wave
  static constexpr int ROWS_WG = NQW * ROWS_QW;   // query rows per workgroup
  static constexpr int KQ = (ROW + 31) / 32;      // k steps of S^T = C Q^T (16x16x32)
  static constexpr int MT = R / 32;               // 32-dim tiles of O^T
  static constexpr int MTW = (MT + NPW - 1) / NPW;  // O tiles per PV wave (wave v: tiles v, v + NPW, ...)
  static constexpr int NTR = ROWS_WG / 32;        // 32-row tiles of O^T
  static constexpr int OL_STRIDE = 2 * R + 16;    // LDS row stride of the staged o_lat (bytes)
  static constexpr int P_BYTES = 2 * ROWS_WG * 32;           // P^T of one tile: [k step][row][16 tokens] bf16
  static constexpr int OFF_P = NBUF * BUF_BYTES;             // P^T, two tiles (double buffer)
  static constexpr int OFF_VOTE = OFF_P + 2 * P_BYTES;       // restart votes [2 slots][NQW]
  static constexpr int OFF_L = OFF_VOTE + 32;                // row sums [ROWS_WG] (fp32)
  static constexpr int LDS_BYTES = OFF_L + ROWS_WG * 4;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(ROWS_WG * OL_STRIDE <= NBUF * BUF_BYTES, "o_lat staging fits in the tile buffers");
  static_assert((TILE * CHR) % 64 == 0, "tile must be whole DMA instructions");
  static_assert(ROW % 16 == 0 && R % 32 == 0 && DN % 32 == 0 && DV % 16 == 0, "unsupported dims");
  static_assert(NIW <= 31, "vmcnt budget");
  static_assert(ROWS_WG % 32 == 0, "row tiles");
};


// Decode kernel, one workgroup of eight waves per (split of a sequence, block
// of 64 query rows); two waves per SIMD with complementary work, so one
// wave's memory and LDS latency is covered by the other's MFMAs:
//   * QK waves 0..3 (16 rows each, 16x16x32 MFMA): their query rows stay in
//     registers; S^T = C_tile Q^T per 32-token tile; the online softmax; the
//     bf16 P^T of the tile into LDS (double-buffered);
//   * PV waves 4..7: O^T += C^T P^T for the previous tile on the 32x32x16
//     MFMA, each wave over its 32-dim tiles of the latent and all 64 rows
//     (O in the accumulation registers; C^T by the transposing LDS read, P^T
//     from LDS); they also issue the HBM -> LDS copies of the tiles.
// One workgroup barrier per tile; phase it runs QK + softmax of tile it and
// PV of tile it-1.  The latent tiles go HBM -> LDS by direct DMA
// (global_load_lds_dwordx4, four buffers, two tiles in flight).
template <int HPG, int SQ, int R, int DR, int DN, int DV>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void absorb_decode_narrow_kernel(DecodeParams p) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KQ = C::KQ, MT = C::MT, NQW = C::NQW;
  constexpr int NPW = C::NPW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  // Workgroups are dispatched round-robin over the 8 XCDs.  XCD x takes the
  // contiguous unit range [x * UPX, (x + 1) * UPX), so the splits of one
  // sequence share an L2 for their query rows, and the row blocks of one unit
  // (which copy the same latent tiles) take consecutive slots on one XCD.
  const int UPX = (p.num_units + 7) / 8;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int u = xcd * UPX + k / RB;
  const int rb = k % RB;
  if (u >= p.num_units) return;                   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const bool is_qk = w < NQW;
  const int v = is_qk ? 0 : w - NQW;              // PV wave index
  const int hh = lane >> 5;                       // half wave
  const int c = lane & 15, qq = lane >> 4;        // 16x16 MFMA lane coordinates
  int b, lo, hi;
  if (p.split_offsets) {
    const UnitOwner own = unit_owner(p.split_offsets, p.seqlens, p.batch, u);
    b = own.b;
    lo = (u - own.first) * p.split_tokens;         // a multiple of BS
    hi = min(lo + p.split_tokens, own.len);
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

  // ---- HBM -> LDS tile copies by the PV waves: wave v issues instructions
  // v, v + NPW, ... of a tile.  LDS position P (16-byte chunk index inside the
  // tile) holds token P / CHR, physical chunk P % CHR, i.e. logical chunk
  // (P % CHR) ^ f(token); the per-lane source offsets are computed once.
  typedef const __attribute__((address_space(4))) int32_t cint32_t;
  const cint32_t* const cbt = (const cint32_t*)bt;
  constexpr bool kFixedCopies = (C::NI % NPW) == 0;  // every PV wave issues NIW copies per tile
  const int niw = kFixedCopies ? C::NIW : (C::NI - v + NPW - 1) / NPW;
  uint32_t dvo[C::NIW];
#pragma unroll
  for (int kk = 0; kk < C::NIW; ++kk) {
    const int i = min(v + NPW * kk, C::NI - 1);
    const int P = i * 64 + lane;
    const int t = P / CHR, pos = P % CHR;
    const int ch = C::SWZ ? (pos ^ tile_swz(t)) : pos;
    dvo[kk] = (uint32_t)(t * ROW + ch * 8) * 2u;
  }
  auto tile_page = [&](int it) -> int { return cbt[(lo + C::TILE * it) / BS]; };
  // Copy of tile it from page `page` (its block-table entry).  In the
  // sequence's last tile the rows past its end copy the last token's row
  // instead of the page's unused slots, which may hold anything: their logits
  // are masked, so their P is 0, and 0 times a finite row adds nothing to O
  // (0 times a NaN would).
  auto issue_tile = [&](int it, int page) {       // PV waves only
    const int t0 = lo + C::TILE * it;
    const uint16_t* src = p.cache + ((size_t)page * BS + (t0 % BS)) * ROW;
    lds_u8_t* dst = lds + (it % C::NBUF) * C::BUF_BYTES;
    if (t0 + C::TILE <= L) {
      for (int kk = 0; kk < niw; ++kk) dma16(src, dvo[kk], dst + (v + NPW * kk) * 1024);
    } else {
      const int last = L - t0 - 1;                // last valid row of the tile
      for (int kk = 0; kk < niw; ++kk) {
        const int t = (min(v + NPW * kk, C::NI - 1) * 64 + lane) / CHR;
        dma16(src, dvo[kk] - (uint32_t)(max(t - last, 0) * ROW * 2), dst + (v + NPW * kk) * 1024);
      }
    }
  };
  auto pv_wait_next = [&](int it) {               // PV waves: tile it + 1 landed (tile it + 2 may be in flight)
    if (it + 1 >= n_tiles) return;
    if (it + 2 < n_tiles) {
      if constexpr (kFixedCopies) vm_wait<C::NIW>(); else vm_wait_dyn(niw);
    } else {
      vm_wait<0>();
    }
  };

  // ---- QK waves: query rows rb * 64 + 16 w + c ----
  const int rl = C::ROWS_QW * w + c;              // row inside the workgroup (QK waves)
  const int rq = rb * C::ROWS_WG + rl;
  const bool rvalid = is_qk && rq < rows_total;
  const bool qk_active = is_qk && rb * C::ROWS_WG + C::ROWS_QW * w < rows_total;   // wave-uniform
  const int h_q = rvalid ? rq / SQ : 0, i_q = rvalid ? rq % SQ : 0;
  const int nvis = rvalid ? L - SQ + i_q + 1 : -1;  // tokens t < nvis are visible to this row
  const int ntv = min(C::NTR, (rows_total - rb * C::ROWS_WG + 31) / 32);   // row tiles with rows

  // QK A operand of token half st, k step ks: token 16 st + c, logical chunk
  // 4 ks + qq, at 8 (ks >> 1) + ((4 (ks & 1) + qq) ^ f): one base per
  // (st, ks & 1), the rest an immediate of 128 (ks >> 1) bytes.
  int qkb[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int t = 16 * st + c;
      const int ch = C::SWZ ? ((4 * kp + qq) ^ tile_swz(t)) : (4 * kp + qq);
      qkb[st][kp] = t * ROW * 2 + ch * 16;
    }
  auto qk_operand = [&](const lds_u8_t* buf, int st, int ks) -> bf16x8 {
    if (32 * ks + 8 * qq >= ROW) return zero_bf16x8();      // past the row (narrow shapes)
    const int addr = C::SWZ ? qkb[st][ks & 1] + 128 * (ks >> 1) : qkb[st][0] + 64 * ks;
    return __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + addr));
  };
  // PV A operand (C^T, 32 latent dims x 16 tokens) of dim tile mt = v + NPW m,
  // k step kk: k index 8 hh + j is token 16 kk + 8 hh + j.  Two transposing
  // reads (rd = j / 4); in read rd the 16-lane group gq = lane / 16 reads
  // tokens 16 kk + 8 (gq / 2) + 4 rd + s / 4 (s = lane % 16), dims
  // 32 mt + 16 (gq % 2) + 4 (s % 4) .. +3, so lane s receives dim
  // 32 mt + 16 (gq % 2) + s of four consecutive tokens.  Logical chunk
  // 4 mt + x (x = 2 (gq % 2) + (s % 4) / 2) sits at
  // 8 (mt >> 1) + ((4 (mt & 1) + x) ^ f); mt & 1 = v & 1 for every tile of the
  // wave, so one base per (rd, kk), plus 128 (mt >> 1) bytes.
  const int gq = lane >> 4, s16 = lane & 15;
  int pvb[2][2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int t = 16 * kk + 8 * (gq >> 1) + 4 * rd + (s16 >> 2);
      const int x = 2 * (gq & 1) + ((s16 & 3) >> 1);
      const int lowc = 4 * (v & 1) + x;
      const int ch = C::SWZ ? (lowc ^ tile_swz(t)) : lowc;
      pvb[rd][kk] = t * ROW * 2 + ch * 16 + 8 * (s16 & 1) + 128 * (v >> 1);
    }
  auto pv_operand = [&](const lds_u8_t* buf, int m, int kk) -> bf16x8 {
    const int imm = 256 * m;                      // mt >> 1 = (v >> 1) + 2 m
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[0][kk] + imm));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[1][kk] + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // P^T of tile it in LDS: [k step][row][16 tokens] bf16, 32 bytes per row
  // with its two 16-byte halves swapped on rows 8..15 of every 16 (so the PV
  // reads of 16 rows hit distinct banks).
  auto p_off = [&](int it, int kk, int row, int half) -> int {
    return C::OFF_P + (it & 1) * C::P_BYTES + (kk * C::ROWS_WG + row) * 32 + 16 * (half ^ ((row >> 3) & 1));
  };

  // Softmax reference: the maximum of a row's first tile, then fixed, so the
  // O accumulators are only ever written by MFMAs.  Every p = 2^(x - ref) is
  // kept below 2^kSlack: a tile whose logits exceed ref + kSlack on some row
  // (an extreme logit spread, e.g. one dominant token) makes the workgroup
  // restart the split before that tile's P is used: pass 1 sweeps QK for the
  // exact row maxima, pass 2 reruns the attention with them as the
  // references (then p <= 1).
  constexpr float kSlack = 64.f;
  typedef __attribute__((address_space(3))) int lds_i32_t;
  // restart votes of the QK waves, two slots: the softmax of tile it writes
  // slot it & 1 before the barrier that ends phase it, every wave reads it in
  // phase it + 1 (the PV waves first thing, the QK waves once their S reads
  // are in flight), and it is next written in phase it + 2
  lds_i32_t* const votes = (lds_i32_t*)(lds + C::OFF_VOTE);
  if (tid < 2 * NQW) votes[tid] = 0;
  // Every wave reads the same votes between the same two barriers, so both
  // roles take the same restart decision; their loops run the same barriers.
  auto restart_requested = [&](int pass, int it) -> bool {
    if (pass != 0 || it == 0) return false;       // votes of the softmax of tile it-1
    const u32x4 vt = *(volatile lds_u32x4_t*)(lds + C::OFF_VOTE + 16 * ((it - 1) & 1));
    return __builtin_amdgcn_readfirstlane((int)(vt[0] | vt[1] | vt[2] | vt[3])) != 0;
  };
  float* const l_lds = (float*)(lds_raw + C::OFF_L);
  f32x16 o[C::MTW][C::NTR];                       // PV waves: O^T tile (v + NPW m, nt): lane l = row 32 nt + l%32,
                                                  // latent 32 (v + NPW m) + 8 (i/4) + 4 hh + i%4
  const int mtw = is_qk ? 0 : (MT - v + NPW - 1) / NPW;   // this PV wave's dim tiles
  constexpr bool kAllDimTiles = (MT % NPW) == 0;  // every PV wave has MTW dim tiles

  if (is_qk) {
    // =================== QK waves ===================
    bf16x8 qb[KQ];                                // B operands: Q[row][32 ks + 8 qq .. +7]
    {
      const uint16_t* qrow = p.qcat + (((size_t)b * SQ + i_q) * H + h_q) * ROW;
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) {
        const int dim = 32 * ks + 8 * qq;
        qb[ks] = (rvalid && dim < ROW) ? ld_bf16x8(qrow + dim) : zero_bf16x8();
      }
    }
    float m_ref = -INFINITY, m_half = -INFINITY, l_run = 0.f;
    vm_wait<0>();
    block_sync_lds();                             // tiles 0 and 1 landed
    for (int pass = 0; pass < 3; ++pass) {        // 0: single pass; 1, 2: after a restart
      l_run = 0.f;
      if (pass > 0) block_sync_lds();             // the first tiles landed again
      bool restart = false;
      for (int it = 0; it <= n_tiles; ++it) {
        if (restart_requested(pass, it)) {
          restart = true;
          break;
        }
        f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        if (qk_active && it < n_tiles) {
          // ---- S^T of tile it, two 16-token halves over the full contraction ----
          const lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
          constexpr int NS = 2 * KQ, PD = 8;    // operands read ahead
          bf16x8 a[PD + 1];
#pragma unroll
          for (int j = 0; j < PD && j < NS; ++j) a[j] = qk_operand(buf, j & 1, j >> 1);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            if (j + PD < NS) a[(j + PD) % (PD + 1)] = qk_operand(buf, (j + PD) & 1, (j + PD) >> 1);
            s[j & 1] = mfma16(a[j % (PD + 1)], qb[j >> 1], s[j & 1]);
          }
          // schedule: the first PD operand reads, then per step the read of
          // operand j + PD and the MFMA of step j (left to itself the
          // compiler keeps only two reads in flight)
          __builtin_amdgcn_sched_group_barrier(0x100, PD < NS ? PD : NS, 0);
#pragma unroll
          for (int j = 0; j < NS; ++j) {
            if (j + PD < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
        }
        if (qk_active && it < n_tiles) {
          // ---- softmax (base 2); lane (qq, c): tokens t0 + 16 st + 4 qq + e of row c ----
          const int t0 = lo + C::TILE * it;
          float x[8], mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int st = e >> 2, ei = e & 3;
            x[e] = (t0 + 16 * st + 4 * qq + ei < nvis) ? s[st][ei] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, x[e]);
          }
          m_half = fmaxf(m_half, mx);
          if (it == 0 && pass == 0) m_ref = wave_max_q(mx);   // tile 0 sets each row's reference
          if (pass != 1) {
            // every row's reference is fixed from here on; each lane checks
            // its own logits against ref + kSlack (the vote)
            votes[4 * (it & 1) + w] = __builtin_amdgcn_ballot_w64(mx > m_ref + kSlack) != 0 ? 1 : 0;
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
              ps += x[e];
            }
            l_run += ps;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
              const u32x2 pk = {pack_bf16x2(x[4 * st], x[4 * st + 1]), pack_bf16x2(x[4 * st + 2], x[4 * st + 3])};
              *(__attribute__((address_space(3))) u32x2*)(lds + p_off(it, st, rl, qq >> 1) + 8 * (qq & 1)) = pk;
            }
          }
        }
        block_sync_lds();                         // end of phase it
      }
      if (pass == 0 && !restart) break;           // the common case: done in one pass
      if (pass == 1) m_ref = wave_max_q(m_half);  // the exact row maxima, for pass 2
      block_sync_lds();                           // end of the pass
      if (pass == 0) m_half = -INFINITY;
    }
    // row sums and the lse
    if (qk_active) {
      const float lt = wave_sum_q(l_run);         // the four lane groups hold a row's token quarters
      if (qq == 0) {
        l_lds[rl] = lt;
        if (rvalid) p.olse[((size_t)u * SQ + i_q) * H + h_q] = lt > 0.f ? (m_ref + log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  } else {
    // =================== PV waves ===================
    // Per phase it: the votes, the copy of tile it+2, then O^T += C^T P^T for
    // tile it-1 (P^T and the transposed latent operands read from LDS).
    bf16x8 ct[2][C::MTW];
    auto load_ct = [&](int it) {
      const lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int m = 0; m < C::MTW; ++m)
          ct[kk][m] = (kAllDimTiles || m < mtw) ? pv_operand(buf, m, kk) : zero_bf16x8();
    };
    for (int i = 0; i < 2 && i < n_tiles; ++i) issue_tile(i, tile_page(i));
    vm_wait<0>();
    block_sync_lds();                             // tiles 0 and 1 landed
    for (int pass = 0; pass < 3; ++pass) {
#pragma unroll
      for (int m = 0; m < C::MTW; ++m)
#pragma unroll
        for (int nt = 0; nt < C::NTR; ++nt) o[m][nt] = f32x16{};
      if (pass > 0) {                             // the first tiles again after a restart
        for (int i = 0; i < 2 && i < n_tiles; ++i) issue_tile(i, tile_page(i));
        vm_wait<0>();
        block_sync_lds();
      }
      bool restart = false;
      for (int it = 0; it <= n_tiles; ++it) {
        if (restart_requested(pass, it)) {
          restart = true;
          break;
        }
        if (it + 2 < n_tiles) issue_tile(it + 2, tile_page(it + 2));   // into the buffer of tile it-2
        const bool mult = it >= 1 && pass != 1 && mtw > 0;
        // Straight-line code, no per-MFMA guard: a row tile past the last
        // query row (nt >= ntv) multiplies whatever its P^T slots hold into
        // accumulators that are never stored, and a dim tile past the
        // latent (only when NPW does not divide MT) takes a zero operand.
        if (mult) {
          bf16x8 pt[2][C::NTR];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < C::NTR; ++nt)
              pt[kk][nt] = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(lds + p_off(it - 1, kk, 32 * nt + (lane & 31), hh)));
          load_ct(it - 1);
          // this wave's dim tiles x every row tile
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int m = 0; m < C::MTW; ++m)
#pragma unroll
              for (int nt = 0; nt < C::NTR; ++nt) o[m][nt] = mfma16x32(ct[kk][m], pt[kk][nt], o[m][nt]);
        }
        pv_wait_next(it);
        block_sync_lds();                         // end of phase it
      }
      if (pass == 0 && !restart) break;
      vm_wait<0>();                               // drain before the tile buffers are refilled
      block_sync_lds();                           // end of the pass
    }
  }

  // ---- epilogue ----
  block_sync_lds();                               // row sums in LDS; every tile buffer read
  // PV waves: normalised o_lat as bf16 in LDS over the tile buffers, row r at
  // r * OL_STRIDE, latent-major
  if (!is_qk) {
    const int tq = lane & 31;
#pragma unroll
    for (int nt = 0; nt < C::NTR; ++nt) {
      if (nt >= ntv) break;                       // uniform
      const float lt = l_lds[32 * nt + tq];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int m = 0; m < C::MTW; ++m) {
        if (m >= mtw) break;                      // uniform
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int lat = 32 * (v + NPW * m) + 8 * a + 4 * hh;
          const f32x16& om = o[m][nt];
          u32x2 pk = {pack_bf16x2(om[4 * a] * inv, om[4 * a + 1] * inv), pack_bf16x2(om[4 * a + 2] * inv, om[4 * a + 3] * inv)};
          *(__attribute__((address_space(3))) u32x2*)(lds + (32 * nt + tq) * C::OL_STRIDE + 2 * lat) = pk;
        }
      }
    }
  }
  block_sync_lds();
  // one 1 KB row per store instruction; wave w writes rows w, w + 8, ...
  for (int j = w; j < C::ROWS_WG; j += C::NW) {
    const int rho = rb * C::ROWS_WG + j;          // uniform
    if (rho >= rows_total) break;
    uint16_t* dst = p.olat + (((size_t)u * SQ + rho % SQ) * H + rho / SQ) * R;
    for (int e = lane; e < R / 8; e += 64)
      *reinterpret_cast<u32x4*>(dst + 8 * e) = *(const lds_u32x4_t*)(lds + j * C::OL_STRIDE + 16 * e);
  }
}

}  // namespace gqla

namespace gqla {
// The main decode kernel (512 + 64 latent rows, blocks of 64 query rows) lives
// in its own translation unit: it is built with MFMA accumulators in
// accumulation registers (absorb_wide.hip).
hipError_t absorb_wide_dispatch(int hpg, int sq, const DecodeParams& p, hipStream_t stream, bool* handled);

// Merge of the split partials and up-projection, per (group G, block of SB
// sequences, or a 32-row chunk of one sequence's group rows when a group has
// more than 32): for each query row of the block,
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
  constexpr int RCH = RG > 32 ? RG / 32 : 1;        // workgroups per (sequence, group)
  constexpr int NR = RG > 32 ? 32 : SB * RG;        // rows per workgroup
  static_assert(RG <= 32 || RG % 32 == 0, "row chunks of 32");
  constexpr int NT = NR / 16;                       // 16-row tiles
  constexpr int STR = 2 * R + 16;                   // LDS row stride (bytes)
  constexpr int MD = DV / 16;                       // 16-dim output tiles
  constexpr int RPW = NR / NWM;                     // rows per wave in the merge
  constexpr int SC = 4;                             // splits per load batch
  constexpr int NCH = (R / 8 + 63) / 64;            // 8-latent chunks per lane
  static_assert(NR <= 32 && NR % 16 == 0 && NR % NWM == 0, "merge tiling");
  static_assert(MD <= NWM, "one output tile per wave");
  static_assert(RPW * SC <= 64 && SB < 64, "plan and lse lanes");
  __shared__ __attribute__((aligned(16))) unsigned char sm_raw[2 * NR * STR];
  lds_u8_t* const sm = (lds_u8_t*)sm_raw;
  const int G = blockIdx.y, b0 = (blockIdx.x / RCH) * SB;
  const int lr0 = (blockIdx.x % RCH) * 32;          // first group row of this workgroup
  const int H = HPG * p.num_groups;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  // ---- merge: wave w takes rows w, w + 8, ...; lane l holds latent 8l .. 8l+7
  // of the row (one coalesced 1 KB row per load instruction).  The loads (lse
  // and o_lat) of up to SC splits of all the wave's rows are issued
  // together, and the running maximum moves (acc, wsum rescaled) when a
  // batch raises it. ----
  int s0[RPW], ns[RPW], rowi[RPW], rowh[RPW];
  float m[RPW], wsum[RPW];
  float acc[RPW][NCH][8];
  // The split plan of the workgroup's sequences in one vector load: lane i
  // (i <= SB) holds the first unit of sequence b0 + i (the end of the plan
  // past the batch).  Per-row values are then read from those lanes, so the
  // loads that depend on the plan wait for one memory round trip only.
  int offv;
  {
    const int bi = min(b0 + min(lane, SB), p.batch);
    offv = p.split_offsets ? p.split_offsets[bi] : bi;
  }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rr = w + NWM * j;
    const int b = b0 + rr / RG, lr = lr0 + rr % RG;
    const bool bv = b < p.batch;
    const int o0 = __builtin_amdgcn_readlane(offv, rr / RG);
    const int o1 = __builtin_amdgcn_readlane(offv, rr / RG + 1);
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
  // W_UV^T[G] operands of this wave's output tile md = w, issued after the
  // split-plan loads (so that waiting for those does not wait for these) and
  // before the partials' loads, so that they arrive during the merge (the
  // prologue stores W_UV^T[G] in operand order, so each load is one
  // contiguous 1 KB block)
  const uint16_t* WT = p.wuvT + (size_t)G * DV * R;
  const int md = w < MD ? w : 0;
  bf16x8 wa[R / 32];
#pragma unroll
  for (int kk = 0; kk < R / 32; ++kk) wa[kk] = ld_bf16x8(WT + ((size_t)(md * (R / 32) + kk) * 64 + lane) * 8);
  int smax = 0;
#pragma unroll
  for (int j = 0; j < RPW; ++j) smax = max(smax, ns[j]);
  for (int sb = 0; sb < smax; sb += SC) {
    u32x4 v[RPW][SC][NCH];
    float ls[RPW][SC];
    // the lse of every (row j, split sb + k) of the wave in one vector load:
    // lane j * SC + k
    float lsv;
    {
      const int jl = lane / SC, kl = lane % SC;
      int s0l = s0[0], nsl = 0, ril = rowi[0], rhl = rowh[0];
#pragma unroll
      for (int jj = 0; jj < RPW; ++jj)
        if (jl == jj) {
          s0l = s0[jj];
          nsl = ns[jj];
          ril = rowi[jj];
          rhl = rowh[jj];
        }
      const bool have = sb + kl < nsl;             // false on lanes past RPW * SC (nsl = 0)
      const size_t row = ((size_t)(s0l + (have ? sb + kl : 0)) * SQ + ril) * H + rhl;
      lsv = have ? p.olse[row] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int k = 0; k < SC; ++k) {
        const int s = sb + k;
        const bool have = s < ns[j];
        const size_t row = ((size_t)(s0[j] + (have ? s : 0)) * SQ + rowi[j]) * H + rowh[j];
        ls[j][k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lsv), j * SC + k));
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
    const int b = b0 + rr / RG, lr = lr0 + rr % RG;
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
// consecutive latent values of one row.  The chunk's W_UK rows are one
// contiguous block: the workgroup stages it in LDS once with 1 KB loads (each
// wave then reads its operands from there), and the query rows are loaded
// before the wait, so the workgroup waits for memory once.
template <int HPG, int SQ, int R, int DR, int DN>
__device__ __forceinline__ void absorb_q_block(const DecodeParams& p, int bx, int G, int bz) {
  constexpr int ROW = R + DR, KD = DN / 32, MT = R / 16;
  constexpr int MTC = MT < 8 ? MT : 8;               // latent tiles per workgroup (blockIdx.z)
  constexpr int NT = 2;                              // 16-row tiles per wave
  constexpr int WR = 16 * MTC;                       // W_UK rows staged
  constexpr int CPR = DN / 8;                        // 16-byte chunks per W_UK row
  constexpr int NCK = WR * CPR / 256;                // chunks per thread
  // row stride 2 DN + 32 bytes: the operand read of lane (q, c) starts at bank
  // 4 ((DN / 8 + 2) c + q) mod 64, which keeps every 16-lane pass of a 16-byte
  // read on 64 distinct banks
  constexpr int WSTR = 2 * DN + 32;
  static_assert(WR * CPR % 256 == 0, "staging tiling");
  __shared__ __attribute__((aligned(16))) unsigned char wl_raw[WR * WSTR];
  lds_u8_t* const wl = (lds_u8_t*)wl_raw;
  const int g = p.num_groups, H = HPG * g;
  const int rows_g = p.batch * SQ * HPG;             // query rows of one group
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int r0 = (bx * 4 + w) * 16 * NT;             // first group-row of this wave
  const int mt0 = bz * MTC;
  const uint16_t* W = p.w_uk + ((size_t)G * R + 16 * mt0) * DN;
  u32x4 wv[NCK];
#pragma unroll
  for (int i = 0; i < NCK; ++i) wv[i] = *reinterpret_cast<const u32x4*>(W + 8 * (tid + 256 * i));
  // group-row gr = (b * SQ + i) * HPG + hl  ->  head h = G*HPG + hl; rows past
  // the batch load row 0 and are not stored
  bf16x8 qn[NT][KD];
  size_t qrow[NT];
  bool valid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int gr = r0 + 16 * nt + c;
    valid[nt] = gr < rows_g;
    const int gc = valid[nt] ? gr : 0;
    const int hl = gc % HPG, bi = gc / HPG;          // bi = b * SQ + i
    qrow[nt] = (size_t)bi * H + G * HPG + hl;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) qn[nt][kd] = ld_bf16x8(p.q_nope + qrow[nt] * DN + 32 * kd + 8 * q);
  }
#pragma unroll
  for (int i = 0; i < NCK; ++i) {
    const int e = tid + 256 * i;
    *(lds_u32x4_t*)(wl + (e / CPR) * WSTR + 16 * (e % CPR)) = wv[i];
  }
  __syncthreads();
  if (r0 >= rows_g) return;
#pragma unroll
  for (int m = 0; m < MTC; ++m) {
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(wl + (16 * m + c) * WSTR + 64 * kd + 16 * q));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16(a, qn[nt][kd], acc[nt]);
    }
    // lane (q, c): latent 16 (mt0 + m) + 4q .. +3 of row (nt, c)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (valid[nt]) {
        u32x2 pk = {pack_bf16x2(acc[nt][0], acc[nt][1]), pack_bf16x2(acc[nt][2], acc[nt][3])};
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

// W_UV[G] (r x d_v) -> W_UV^T[G] (d_v x r) in the merge's MFMA operand order,
// through an LDS tile of 64 latent rows x TD columns: 16-byte reads of W_UV
// rows, 2-byte transposed LDS writes, 16-byte reads of LDS rows.  The 8
// latents l = 32 kk + 8 q .. +7 of output dim d = 16 md + c (the A operand of
// lane 16 q + c in k step kk of output tile md) are stored as one 16-byte
// chunk at element ((md * r / 32 + kk) * 64 + 16 q + c) * 8, so a wave's
// operand load for one k step is one contiguous 1 KB block.
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
    const int dd = d0 + d, ll = l0 + lc;            // output dim, first of 8 latents
    const size_t chunk = ((size_t)(dd / 16) * (R / 32) + ll / 32) * 64 + 16 * ((ll % 32) / 8) + dd % 16;
    *reinterpret_cast<u32x4*>(p.wuvT + (size_t)G * DV * R + chunk * 8) =
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

template <int HPG, int SQ, int R, int DV>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  constexpr int RG = HPG * SQ, SB = RG >= 32 ? 1 : 32 / RG, RCH = RG > 32 ? RG / 32 : 1;
  dim3 grid((unsigned)((p.batch + SB - 1) / SB * RCH), (unsigned)p.num_groups);
  hipLaunchKernelGGL((absorb_merge_kernel<HPG, SQ, R, DV>), grid, dim3(512), 0, stream, p);
  return hipGetLastError();
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
    hipError_t e = hipSuccess;
    bool wide = false;
    if constexpr (R == 512 && DR == 64 && DN == 128 && DV == 128) {
      if (rows_total % 64 == 0) e = absorb_wide_dispatch(HPG, SQ, p, stream, &wide);
    }
    if (!wide) {
      const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
      const unsigned grid = (unsigned)((p.num_units + 7) / 8) * 8u * (unsigned)RB;
      hipLaunchKernelGGL((absorb_decode_narrow_kernel<HPG, SQ, R, DR, DN, DV>), dim3(grid), dim3(64 * C::NW), 0,
                         stream, p);  // NW = 8 waves
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return launch_merge<HPG, SQ, R, DV>(p, stream);
}

// The merge and up-projection alone, over caller-provided latent partials
// (p.olat, p.olse, p.split_offsets): W_UV^T first (the prologue launch with
// no q_abs blocks), then the merge.
template <int HPG, int SQ, int R, int DR, int DN, int DV>
hipError_t launch_absorb_merge(const DecodeParams& p, hipStream_t stream) {
  constexpr int TD = DV < 64 ? DV : 64;
  const int nt = (R / 64) * (DV / TD) * p.num_groups;
  hipLaunchKernelGGL((absorb_prologue_kernel<HPG, SQ, R, DR, DN, DV>), dim3((unsigned)nt), dim3(256), 0, stream, p,
                     0, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge<HPG, SQ, R, DV>(p, stream);
}

// merge_only: the merge and up-projection of caller-provided partials.
hipError_t absorb_dispatch(int hpg, int sq, int r, int dn, int dv, int dr, const DecodeParams& p,
                           hipStream_t stream, bool* supported, bool merge_only) {
  *supported = true;
#define GQLA_ABS_CASE(HPG, SQ, R, DR, DN, DV)                                     \
  if (hpg == HPG && sq == SQ && r == R && dr == DR && dn == DN && dv == DV)  \
    return merge_only ? launch_absorb_merge<HPG, SQ, R, DR, DN, DV>(p, stream) \
                      : launch_absorb<HPG, SQ, R, DR, DN, DV>(p, stream);
  GQLA_ABS_CASE(16, 1, 512, 64, 128, 128)
  GQLA_ABS_CASE(16, 2, 512, 64, 128, 128)
  GQLA_ABS_CASE(32, 1, 512, 64, 128, 128)
  GQLA_ABS_CASE(32, 2, 512, 64, 128, 128)
  GQLA_ABS_CASE(4, 1, 512, 64, 128, 128)
  GQLA_ABS_CASE(4, 2, 512, 64, 128, 128)
  GQLA_ABS_CASE(8, 1, 64, 16, 32, 32)
  GQLA_ABS_CASE(8, 2, 64, 16, 32, 32)
#undef GQLA_ABS_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace gqla
