// MQA-absorb decode over the shared latent cache: the main kernel, for the
// 512 + 64 latent row in blocks of 64 query rows.
//
// GQLA pages: paperlayer.ai summary, section 4 "MQA-absorb path" (all query
// heads attend over one latent row per token, read once for every head) and
// gist.science section 2 "MQA-Absorb-Pfad".  Per query row:
//   s_t = (q_abs . c_t + q_rope . k_rope_t) * scale,   o_lat = softmax(s) C.
//
// One workgroup of eight waves (two per SIMD) per (split unit, block of 64
// query rows), in two roles, so that on every SIMD one wave's instruction
// issue (LDS reads, copy instructions, softmax arithmetic) runs while the
// other wave's MFMAs execute:
//   * QK waves 0..3.  Wave w takes query rows 32 (w & 1) .. +31 and the 16
//     tokens of token half (w >> 1) of every 32-token tile: S^T = C_half Q^T
//     on the 16x16x32 MFMA (each 16-byte operand read of the latent tile feeds
//     both 16-row tiles; the query rows stay in registers as B operands), the
//     softmax against a fixed per-row reference, and P^T as bf16 into LDS
//     (double-buffered).
//   * PV waves 4..7.  Wave 4 + v accumulates O^T[latent][row] += C^T P^T for
//     the latent dim tiles v, v + 4, v + 8, v + 12 and all 64 rows on the
//     32x32x16 MFMA (O in registers, C^T by the transposing LDS read), and
//     issues its share of the HBM -> LDS copies of every tile
//     (global_load_lds_dwordx4) between its MFMAs.
// Phase it runs QK and softmax of tile it beside PV of tile it - 1 and the
// copies of tile it + 2 (four tile buffers: it in QK, it - 1 in PV, it + 1 and
// it + 2 in flight), with one workgroup barrier per phase; both roles pass the
// same barriers in the same order.  Each latent tile is read from LDS twice by
// QK (once per 32-row half) and once by PV.
//
// Measured on this hardware (DeepSeek-V3-shaped batch, 64 phases per
// workgroup): a phase takes about 1700 clocks without the copies against 1088
// clocks of MFMA work per SIMD; the copies alone stream at about 5.9 TB/s with
// two tiles in flight per CU (about 52 B/clk per CU when the data is in L2).
// The QK chain is the longer one, so the copies go to the PV waves.
#pragma once

#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

// Direct HBM -> LDS copy of 4 bytes per lane (global_load_lds_dword); lane i's
// word lands at lds_base + 4 i.
__device__ __forceinline__ void dma4(const void* base, uint32_t voff_bytes, lds_u8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff_bytes), "s"(base), "s"(m0v) : "m0");
}

// The 16-byte copy without a memory clobber: it writes only an LDS buffer no
// wave reads before the next vm_wait + barrier (both of which are ordered
// against every LDS access), so LDS reads of other buffers may move across it.
// NT: the non-temporal policy, for a latent cache larger than the
// memory-side cache (each tile is read by the two row blocks of its unit,
// which run side by side on one XCD, and by no one else in the call).  A
// cache that fits keeps the default policy, so that it can stay resident
// from one decode step to the next.
template <bool NT>
__device__ __forceinline__ void dma16_free(const void* base, uint32_t voff_bytes, lds_u8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff_bytes), "s"(base), "s"(m0v) : "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff_bytes), "s"(base), "s"(m0v) : "m0");
}

template <int HPG, int SQ, int R, int DR, int QC>
struct WideCfg {
  static constexpr int BS = 64;
  static constexpr int TILE = 32;                  // tokens per LDS tile
  static constexpr int NBUF = 4;                   // tile buffers
  static constexpr int ROW = R + DR;               // latent row (elements)
  static constexpr int CHR = ROW / 8;              // 16-byte chunks per row
  static constexpr int BUF_BYTES = TILE * ROW * 2;
  static constexpr int NQW = 4;                    // QK waves
  static constexpr int NPW = 4;                    // PV waves (they also copy the tiles)
  static constexpr int NW = NQW + NPW;
  static constexpr int NI = TILE * CHR / 64;       // copy instructions per tile
  static constexpr int NQC = QC;                   // of them per QK wave
  static constexpr int NPC = (NI - NQW * QC) / NPW;  // per PV wave
  static constexpr int ROWS_WG = 64;               // query rows per workgroup
  static constexpr int NQI = ROWS_WG * CHR / 64;   // copy instructions of the query rows
  static constexpr int NQIW = NQI / NW;            // per wave
  static constexpr int KQ = ROW / 32;              // k steps of S^T (16x16x32)
  static constexpr int PD = 3;                     // QK operand reads in flight
  static constexpr int KA = 2;                     // S^T accumulators per 16-row tile
  static constexpr int MT = R / 32;                // 32-dim tiles of O^T
  static constexpr int MTW = MT / NPW;             // per PV wave (tiles v, v + NPW, ...)
  static constexpr int NTR = ROWS_WG / 32;         // 32-row tiles of O^T
  static constexpr int OL_STRIDE = 2 * R + 16;     // LDS row stride of the staged o_lat (bytes)
  static constexpr int P_BYTES = 2 * ROWS_WG * 32; // P^T of one tile: [token half][row][16 tokens] bf16
  static constexpr int OFF_Q = 2 * BUF_BYTES;      // query rows, staged once in buffers 2 and 3
  static constexpr int OFF_P = NBUF * BUF_BYTES;
  static constexpr int OFF_VOTE = OFF_P + 2 * P_BYTES;      // restart votes [2 slots][NQW]
  static constexpr int OFF_X = OFF_VOTE + 32;               // per-row exchange [2 token halves][64 rows] fp32
  static constexpr int PG_MAX = 1024;                       // block-table entries of one unit kept in LDS
  static constexpr int OFF_PG = OFF_X + 2 * ROWS_WG * 4;
  static constexpr int LDS_BYTES = OFF_PG + 4 * PG_MAX;
  static_assert(CHR % 8 == 0, "the chunk swizzle stays inside a row");
  static_assert(NQW * NQC + NPW * NPC == NI && NQI % NW == 0 && MT % NPW == 0, "work splits evenly over the waves");
  static_assert(2 * NQC <= KQ + 1, "QK copy slots between the QK MFMAs");
  static_assert(BUF_BYTES < 65536, "16-bit copy offsets");
  static_assert(KQ % KA == 0, "k steps per accumulator");
  static_assert(ROWS_WG * ROW * 2 <= 2 * BUF_BYTES, "query rows fit in two tile buffers");
  static_assert(ROWS_WG * OL_STRIDE <= NBUF * BUF_BYTES, "o_lat staging fits in the tile buffers");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(R % 32 == 0 && ROW % 32 == 0, "k steps");
};

// One wave's share of a tile copy: the tile's copy instructions k0 .. k0 + NC - 1.
// Instruction k fills LDS bytes 1024 k .. 1024 k + 1023 of the tile buffer:
// chunk position P = 64 k + lane holds token P / CHR, physical chunk
// P % CHR = logical chunk (P % CHR) ^ f(token).  The per-lane source offsets
// (bytes from the tile's first row, each below 2^16) are packed two per
// register.
template <int NC, int CHR, bool NT>
struct TileCopier {
  uint32_t dvp[NC > 0 ? (NC + 1) / 2 : 1];
  int k0;
  __device__ __forceinline__ void init(int first, int lane) {
    k0 = first;
#pragma unroll
    for (int kk = 0; kk < NC; ++kk) {
      const int P = (first + kk) * 64 + lane;
      const int t = P / CHR, pos = P % CHR;
      const uint32_t off = (uint32_t)(t * CHR * 8 + ((pos ^ tile_swz(t)) * 8)) * 2u;
      if (kk % 2 == 0) dvp[kk / 2] = off; else dvp[kk / 2] |= off << 16;
    }
  }
  __device__ __forceinline__ uint32_t off(int kk) const {
    return (kk % 2 == 0) ? (dvp[kk / 2] & 0xffffu) : (dvp[kk / 2] >> 16);
  }
  // copy instruction kk of this wave's share; tile = the tile's first row
  __device__ __forceinline__ void part(const uint16_t* tile, lds_u8_t* buf, int kk) const {
    dma16_free<NT>(tile, off(kk), buf + (k0 + kk) * 1024);
  }
  __device__ __forceinline__ void all(const uint16_t* tile, lds_u8_t* buf) const {
#pragma unroll
    for (int kk = 0; kk < NC; ++kk) part(tile, buf, kk);
  }
};

// Chunk positions inside a row use the swizzle tile_swz: both the 32 token
// rows of a tile and the 64 query rows of the staging block are read 16 rows
// x 4 consecutive chunks per instruction.

// QC: copy instructions of each tile issued by each QK wave (the PV waves
// issue the rest).
// PG_LDS: the unit's block-table entries (at most PG_MAX) are copied into LDS
// at the start and read from there (otherwise by scalar loads, whose waits
// also drain the LDS reads in flight).
template <int HPG, int SQ, int R, int DR, int QC, bool PG_LDS, bool NTC>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void absorb_decode_kernel(DecodeParams p) {
  using C = WideCfg<HPG, SQ, R, DR, QC>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KQ = C::KQ, NQC = C::NQC, NPC = C::NPC;
  constexpr int PD = C::PD, KA = C::KA, NQW = C::NQW, NPW = C::NPW, NW = C::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;                   // a multiple of 64 (checked by the launcher)
  const int RB = rows_total / C::ROWS_WG;
  // Workgroups are dispatched round-robin over the 8 XCDs.  XCD x takes the
  // contiguous unit range [x * UPX, (x + 1) * UPX), and the row blocks of one
  // unit (which copy the same latent tiles) take consecutive slots on one XCD.
  const int UPX = (p.num_units + 7) / 8;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, kx = wg >> 3;
  const int u = xcd * UPX + kx / RB;
  const int rb = kx % RB;
  if (u >= p.num_units) return;                    // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;
  const int c = lane & 15, qq = lane >> 4;
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
  auto tile_buf = [&](int it) -> lds_u8_t* { return lds + (it % C::NBUF) * C::BUF_BYTES; };
  float* const xch = (float*)(lds_raw + C::OFF_X); // [token half][row]
  typedef __attribute__((address_space(3))) int lds_i32_t;
  lds_i32_t* const votes = (lds_i32_t*)(lds + C::OFF_VOTE);
  auto votes_of = [&](int it) -> u32x4 {          // the votes of the softmax of tile it
    return *(volatile lds_u32x4_t*)(lds + C::OFF_VOTE + 16 * (it & 1));
  };
  auto any_vote = [&](const u32x4& vt) -> bool {
    return __builtin_amdgcn_readfirstlane((int)(vt[0] | vt[1] | vt[2] | vt[3])) != 0;
  };
  // copies of the query rows into buffers 2 and 3 (NQIW per wave): row r of
  // the block (head (rb * 64 + r) / SQ, MTP row (rb * 64 + r) % SQ) at LDS
  // position r * CHR + (logical chunk ^ f(r))
  auto copy_queries = [&]() {
    const uint16_t* qbase = p.qcat + (size_t)b * SQ * H * ROW;
#pragma unroll
    for (int kk = 0; kk < C::NQIW; ++kk) {
      const int P = (w + NW * kk) * 64 + lane;
      const int r = P / CHR, pos = P % CHR;
      const int rq = rb * C::ROWS_WG + r;
      const uint32_t off = (uint32_t)(((rq % SQ) * H + rq / SQ) * ROW + ((pos ^ tile_swz(r)) * 8)) * 2u;
      dma16_free<false>(qbase, off, lds + C::OFF_Q + (w + NW * kk) * 1024);
    }
  };
  // Block-table entries of the unit: with PG_LDS every wave copies all of them
  // into LDS (the same values to the same words) and reads them only after its
  // own copies landed; otherwise scalar loads.
  typedef const __attribute__((address_space(4))) int32_t cint32_t;
  const cint32_t* const cbt = (const cint32_t*)(p.block_table + (size_t)b * p.max_blocks);
  const lds_i32_t* const lpg = (const lds_i32_t*)(lds + C::OFF_PG);   // entry j: page of tokens lo + 64 j ..
  auto copy_pages = [&]() {
    if constexpr (PG_LDS) {
      const int np = n_tiles > 0 ? (hi - 1) / BS - lo / BS + 1 : 0;
      const int32_t* src = p.block_table + (size_t)b * p.max_blocks + lo / BS;
      for (int k = 0; k * 64 < np; ++k)
        dma4(src, (uint32_t)min(64 * k + lane, np - 1) * 4u, lds + C::OFF_PG + 256 * k);
    }
  };
  auto page_of = [&](int it) -> int {             // page of tile min(it, n_tiles - 1)
    const int tc = min(it, n_tiles - 1);
    if constexpr (PG_LDS) return __builtin_amdgcn_readfirstlane(lpg[(C::TILE * tc) / BS]);
    else return cbt[(lo + C::TILE * tc) / BS];
  };
  // first row of tile it in page `page`.  Rows past the sequence end are
  // copied as they are (the page's unused slots may hold anything): their
  // logits are masked, and before the PV product reads such a tile its rows
  // past the end are overwritten with zeros (0 times a NaN would not vanish).
  auto tile_src = [&](int it, int page) -> const uint16_t* {
    return p.cache + ((size_t)page * BS + ((lo + C::TILE * it) % BS)) * ROW;
  };

  // Softmax reference: the maximum of a row's first tile, then fixed, so the
  // O accumulators are only ever written by MFMAs.  Every p = 2^(x - ref) is
  // kept below 2^kSlack: a tile whose logits exceed ref + kSlack on some row
  // (an extreme logit spread, e.g. one dominant token) makes the workgroup
  // restart the split: a sweep of QK alone finds the exact row maxima, and the
  // attention reruns with them as the references (then p <= 1).  The votes of
  // the softmax of tile it are read by every wave after the barrier that ends
  // phase it and acted on at the end of phase it + 1; a restart discards O.
  constexpr float kSlack = 64.f;

  if (w < NQW) {
    // ================================ QK waves ================================
    const int rh = w & 1;                          // query rows 32 rh .. +31
    const int th = w >> 1;                         // tokens 16 th .. +15 of each tile
    // latent tile operand (A): token 16 th + c, logical chunk 4 ks + qq at
    // 8 (ks >> 1) + ((4 (ks & 1) + qq) ^ f(t)); one base per ks & 1, the rest
    // an immediate
    int qkb[2];
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const int t = 16 * th + c;
      qkb[kp] = t * ROW * 2 + ((4 * kp + qq) ^ tile_swz(t)) * 16;
    }
    auto qk_operand = [&](const lds_u8_t* buf, int ks) -> bf16x8 {
      return __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + qkb[ks & 1] + 128 * (ks >> 1)));
    };
    // P^T of tile it: [token half][row][16 tokens] bf16, 32 bytes per row, the
    // two 16-byte halves swapped on rows 8..15 of every 16 (so the PV reads of
    // 16 rows hit distinct banks); this lane's 4 tokens of row `row`
    auto p_off = [&](int it, int row) -> int {
      return C::OFF_P + (it & 1) * C::P_BYTES + (th * C::ROWS_WG + row) * 32 + 16 * ((qq >> 1) ^ ((row >> 3) & 1)) +
             8 * (qq & 1);
    };
    int nvis[2];                                   // tokens t < nvis[rt] are visible to row (rt, c)
    int qrow_h[2], qrow_i[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int rq = rb * C::ROWS_WG + 32 * rh + 16 * rt + c;
      qrow_h[rt] = rq / SQ;
      qrow_i[rt] = rq % SQ;
      nvis[rt] = L - SQ + qrow_i[rt] + 1;
    }
    float m_ref[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};                   // this lane's share of the sums of rows (rt, c)
    bf16x8 qb[2][KQ];                              // B operands: Q[row 32 rh + 16 rt + c][32 ks + 8 qq ..]
    TileCopier<NQC, CHR, NTC> cp_q;                     // this wave's copy instructions of every tile
    cp_q.init(w * NQC, lane);

    // S^T of tile it: s[rt][e] = logit of token 16 th + 4 qq + e of the tile
    // for row (rt, c).  Operand reads PD k steps ahead; KA accumulators per
    // row tile keep dependent MFMAs apart.  With cp, this wave's copies of a
    // later tile (first row csrc, into cbuf) go between the MFMAs.
    auto qk_tile = [&](const lds_u8_t* bq, f32x4 (&s)[2], bool cp, const uint16_t* csrc, lds_u8_t* cbuf) {
      bf16x8 a[PD + 1];
      f32x4 sp[2][KA];
#pragma unroll
      for (int j = 0; j < PD; ++j) a[j] = qk_operand(bq, j);
      sched_fence();
#pragma unroll
      for (int ks = 0; ks < KQ; ++ks) {
        if (ks + PD < KQ) a[(ks + PD) % (PD + 1)] = qk_operand(bq, ks + PD);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          sp[rt][ks % KA] = mfma16(a[ks % (PD + 1)], qb[rt][ks], ks < KA ? f32x4{0.f, 0.f, 0.f, 0.f} : sp[rt][ks % KA]);
        if (ks % 2 == 1 && ks / 2 < NQC && cp) cp_q.part(csrc, cbuf, ks / 2);
        sched_fence();
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        s[rt] = sp[rt][0];
#pragma unroll
        for (int j = 1; j < KA; ++j) s[rt] += sp[rt][j];
      }
    };
    // scaled logits in base 2 with the causal / sequence-end mask
    auto scaled = [&](int it, const f32x4 (&s)[2], float (&x)[2][4]) {
      const int t0 = lo + C::TILE * it + 16 * th + 4 * qq;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[rt][e] = (t0 + e < nvis[rt]) ? s[rt][e] * p.scale_log2 : -INFINITY;
    };
    // p = 2^(x - ref), its bf16 P^T into LDS, the row sums and the vote
    auto softmax_tile = [&](int it, const float (&x)[2][4], bool vote) {
      bool over = false;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float m_use = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt];
        const float lim = m_ref[rt] + kSlack;
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          over |= x[rt][e] > lim;
          pr[e] = __builtin_amdgcn_exp2f(x[rt][e] - m_use);
          l_run[rt] += pr[e];
        }
        const u32x2 pk = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3])};
        *(__attribute__((address_space(3))) u32x2*)(lds + p_off(it, 32 * rh + 16 * rt + c)) = pk;
      }
      if (vote) votes[4 * (it & 1) + w] = __builtin_amdgcn_ballot_w64(over) != 0 ? 1 : 0;
    };
    auto row_max = [&](const float (&x)[2][4], float (&mh)[2]) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        mh[rt] = fmaxf(mh[rt], fmaxf(fmaxf(x[rt][0], x[rt][1]), fmaxf(x[rt][2], x[rt][3])));
    };
    // the row maxima of the two token halves through LDS (one barrier, which
    // the PV waves match): the references of rows (rt, c)
    auto exchange_max = [&](float (&mh)[2]) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float mw = wave_max_q(mh[rt]);
        if (qq == 0) xch[th * C::ROWS_WG + 32 * rh + 16 * rt + c] = mw;
        mh[rt] = mw;
      }
      block_sync_lds();
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) m_ref[rt] = fmaxf(mh[rt], xch[(1 - th) * C::ROWS_WG + 32 * rh + 16 * rt + c]);
    };

    // start: the block-table entries, the query rows, this wave's share of
    // tiles 0 and 1; the query rows and tile 0 landed (every wave's: barrier);
    // the query rows into registers; buffers 2 and 3 free (barrier)
    copy_pages();
    copy_queries();
    vm_wait<C::NQIW>();                            // the block-table entries (copies complete in order)
    auto start_tiles = [&]() {
      if (n_tiles > 0) cp_q.all(tile_src(0, page_of(0)), tile_buf(0));
      if (n_tiles > 1) {
        cp_q.all(tile_src(1, page_of(1)), tile_buf(1));
        vm_wait<NQC>();
      } else {
        vm_wait<0>();
      }
    };
    start_tiles();
    block_sync_lds();
    {
      const lds_u8_t* qs = lds + C::OFF_Q;
      int qo[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const int r = 32 * rh + 16 * rt + c;
          qo[rt][kp] = r * ROW * 2 + ((4 * kp + qq) ^ tile_swz(r)) * 16;
        }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ks = 0; ks < KQ; ++ks)
          qb[rt][ks] = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(qs + qo[rt][ks & 1] + 128 * (ks >> 1)));
    }
    block_sync_lds();

    // one pass over the unit's tiles; check: pass 0 (tile 0 sets the
    // references, votes may ask for a restart, returned as true).  Every loop
    // has a single exit (a restart request ends the loop through its
    // condition): early exits would make the compiler keep extra copies of
    // long-lived registers.
    auto attend = [&](bool check) -> bool {
      l_run[0] = l_run[1] = 0.f;
      bool restart = false;
      if (n_tiles > 0) {
        // this wave's share of the copies of tile it + 2 in phase it (page pg,
        // read one phase ahead); at the end of the phase tile it + 1 landed
        int pg = page_of(2);
        {                                          // phase 0
          const int pn = page_of(3);
          const bool cp = n_tiles > 2;
          f32x4 s[2];
          float x[2][4];
          qk_tile(tile_buf(0), s, cp, tile_src(2, pg), tile_buf(2));
          scaled(0, s, x);
          if (check) {
            float mh[2] = {-INFINITY, -INFINITY};
            row_max(x, mh);
            exchange_max(mh);
          }
          softmax_tile(0, x, check);
          if (cp) vm_wait<NQC>(); else vm_wait<0>();
          block_sync_lds();
          pg = pn;
        }
        for (int it = 1; it < n_tiles && !restart; ++it) {
          u32x4 vt = {0u, 0u, 0u, 0u};
          if (check) vt = votes_of(it - 1);
          const int pn = page_of(it + 3);
          const bool cp = it + 2 < n_tiles;
          f32x4 s[2];
          float x[2][4];
          qk_tile(tile_buf(it), s, cp, tile_src(it + 2, pg), tile_buf(it + 2));
          scaled(it, s, x);
          softmax_tile(it, x, check);
          restart = check && any_vote(vt);
          if (cp && !restart) vm_wait<NQC>(); else vm_wait<0>();
          block_sync_lds();
          pg = pn;
        }
        if (!restart) {                            // the final phase: PV of the last tile only
          restart = check && any_vote(votes_of(n_tiles - 1));
          block_sync_lds();
        }
      }
      return restart;
    };
    // Pass 0; on a restart request, QK alone over every tile (the PV waves copy
    // each into buffer 0) for the exact row maxima, then the pass again with
    // them.
    if (attend(true)) {
      float mh[2] = {-INFINITY, -INFINITY};
      for (int it = 0; it < n_tiles; ++it) {
        cp_q.all(tile_src(it, page_of(it)), lds);
        vm_wait<0>();
        block_sync_lds();                          // tile it landed in buffer 0
        f32x4 s[2];
        float x[2][4];
        qk_tile(lds, s, false, nullptr, nullptr);
        scaled(it, s, x);
        row_max(x, mh);
        block_sync_lds();                          // buffer 0 read
      }
      exchange_max(mh);
      start_tiles();
      block_sync_lds();                            // tiles 0 and 1 of the new pass landed
      attend(false);
    }

    // epilogue: the row-sum halves into LDS (barrier), the lse; the PV waves
    // stage o_lat (barrier) and every wave stores it
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const float lw = wave_sum_q(l_run[rt]);      // this wave's token half of row (rt, c)
      if (qq == 0) xch[th * C::ROWS_WG + 32 * rh + 16 * rt + c] = lw;
    }
    block_sync_lds();
    if (th == 0 && qq == 0) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int r = 32 * rh + 16 * rt + c;
        const float lt = xch[r] + xch[C::ROWS_WG + r];
        p.olse[((size_t)u * SQ + qrow_i[rt]) * H + qrow_h[rt]] = lt > 0.f ? (m_ref[rt] + log2f(lt)) * kLn2 : -INFINITY;
      }
    }
    block_sync_lds();
  } else {
    // ================================ PV waves ================================
    const int v = w - NQW;
    TileCopier<NPC, CHR, NTC> cp_p;                     // this wave's copy instructions of every tile
    cp_p.init(NQW * NQC + v * NPC, lane);
    auto zero_tail = [&](int it) {                // latent part only: the PV product reads no rope
      const int valid = L - (lo + C::TILE * it);
      if (valid >= C::TILE) return;                // uniform
      lds_u8_t* buf = tile_buf(it);
      for (int e = tid - 64 * NQW; e < (C::TILE - valid) * (R / 8); e += 64 * NPW) {
        const int t = valid + e / (R / 8), lc = e % (R / 8);
        const int pc = 8 * (lc >> 3) + ((lc & 7) ^ tile_swz(t));
        *(lds_u32x4_t*)(buf + t * ROW * 2 + pc * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    };
    // PV A operand (C^T, 32 latent dims x 16 tokens) of dim tile mt = v + NPW m,
    // k step kk: two transposing reads; in read rd the 16-lane group gq reads
    // tokens 16 kk + 8 (gq / 2) + 4 rd + s / 4 (s = lane % 16), dims
    // 32 mt + 16 (gq % 2) + 4 (s % 4) .. +3.  mt & 1 = v & 1 for every tile
    // of the wave, so one base per (rd, kk), plus 128 (mt >> 1) bytes.
    const int gq = lane >> 4, s16 = lane & 15;
    int pvb[2][2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int t = 16 * kk + 8 * (gq >> 1) + 4 * rd + (s16 >> 2);
        const int x = 2 * (gq & 1) + ((s16 & 3) >> 1);
        const int ch = (4 * (v & 1) + x) ^ tile_swz(t);
        pvb[rd][kk] = t * ROW * 2 + ch * 16 + 8 * (s16 & 1) + 128 * (v >> 1);
      }
    auto pv_operand = [&](const lds_u8_t* buf, int m, int kk) -> bf16x8 {
      const int imm = 256 * m;                     // mt >> 1 = (v >> 1) + 2 m
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[0][kk] + imm));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[1][kk] + imm));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // P^T of tile it, k step kk (token half): rows 32 nt + lane % 32, tokens
    // 8 hh .. 8 hh + 7 of the half
    auto p_operand = [&](int it, int kk, int nt) -> bf16x8 {
      const int row = 32 * nt + (lane & 31);
      return __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(lds + C::OFF_P + (it & 1) * C::P_BYTES +
                                                              (kk * C::ROWS_WG + row) * 32 + 16 * (hh ^ ((row >> 3) & 1))));
    };
    f32x16 o[C::MTW][C::NTR];                      // O^T tile (v + NPW m, nt): lane l = row 32 nt + l % 32,
                                                   // latent 32 (v + NPW m) + 8 (i / 4) + 4 hh + i % 4
    // PV of tile it - 1 (FIRST: its accumulator operand is zero, so O is only
    // ever written by MFMAs), with this wave's copies of tile it + 2 (when cp;
    // page pg) placed between the MFMAs.
    auto pv_phase = [&](int it, auto first, bool cp, int pg) {
      constexpr bool FIRST = decltype(first)::value;
      const lds_u8_t* bp = tile_buf(it - 1);
      const uint16_t* csrc = tile_src(it + 2, pg);
      lds_u8_t* cbuf = tile_buf(it + 2);
      bf16x8 pt[2][C::NTR], ct[2][C::MTW];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int nt = 0; nt < C::NTR; ++nt) pt[kk][nt] = p_operand(it - 1, kk, nt);
#pragma unroll
        for (int m = 0; m < C::MTW; ++m) ct[kk][m] = pv_operand(bp, m, kk);
      }
      sched_fence();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int m = 0; m < C::MTW; ++m)
#pragma unroll
          for (int nt = 0; nt < C::NTR; ++nt) {
            o[m][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ct[kk][m], pt[kk][nt],
                                                               (FIRST && kk == 0) ? f32x16{} : o[m][nt], 0, 0, 0);
            const int j = (kk * C::MTW + m) * C::NTR + nt;
            if (j % 2 == 0 && j / 2 < NPC && cp) cp_p.part(csrc, cbuf, j / 2);
            sched_fence();
          }
#pragma unroll
      for (int kk = C::MTW * C::NTR; kk < NPC; ++kk)
        if (cp) cp_p.part(csrc, cbuf, kk);
    };
    using T = std::true_type;
    using F = std::false_type;

    // start (as the QK waves): block-table entries, query rows, this wave's
    // share of tiles 0 and 1; then tile 0 (and everything issued before it)
    // landed
    copy_pages();
    copy_queries();
    vm_wait<C::NQIW>();                            // the block-table entries (copies complete in order)
    auto start_tiles = [&]() {
      if (n_tiles > 0) cp_p.all(tile_src(0, page_of(0)), tile_buf(0));
      if (n_tiles > 1) {
        cp_p.all(tile_src(1, page_of(1)), tile_buf(1));
        vm_wait<NPC>();
      } else {
        vm_wait<0>();
      }
    };
    start_tiles();
    block_sync_lds();
    block_sync_lds();                              // (the QK waves read the query rows)

    // one pass (the same barriers as the QK waves', single-exit loops as
    // there); returns true on a restart request, with every copy waited for
    auto attend = [&](bool check) -> bool {
      bool restart = false;
      if (n_tiles == 0) {
#pragma unroll
        for (int m = 0; m < C::MTW; ++m)
#pragma unroll
          for (int nt = 0; nt < C::NTR; ++nt) o[m][nt] = f32x16{};
      } else {
        // Page of this phase's copies (pg), read one phase ahead.  Copies in
        // flight at the end of phase it after those of tile it + 1 (which must
        // have landed): this phase's.
        int pg = page_of(2);
        {                                          // phase 0: copies of tile 2
          const int pn = page_of(3);
          if (n_tiles > 2) cp_p.all(tile_src(2, pg), tile_buf(2));
          zero_tail(0);
          if (check) block_sync_lds();             // (the QK waves' exchange of the row maxima)
          if (n_tiles > 2) vm_wait<NPC>(); else vm_wait<0>();
          block_sync_lds();
          pg = pn;
        }
        // phases 1 .. n_tiles - 1; phase 1, whose PV product starts O, peeled
        auto steady = [&](int it, auto first) {
          u32x4 vt = {0u, 0u, 0u, 0u};
          if (check) vt = votes_of(it - 1);
          const int pn = page_of(it + 3);
          const bool cp = it + 2 < n_tiles;
          pv_phase(it, first, cp, pg);
          zero_tail(it);
          restart = check && any_vote(vt);
          if (cp && !restart) vm_wait<NPC>(); else vm_wait<0>();
          block_sync_lds();
          pg = pn;
        };
        if (n_tiles > 1) {
          steady(1, T{});
          for (int it = 2; it < n_tiles && !restart; ++it) steady(it, F{});
        }
        if (!restart) {
          restart = check && any_vote(votes_of(n_tiles - 1));
          if (!restart) {
            if (n_tiles == 1) pv_phase(1, T{}, false, 0); else pv_phase(n_tiles, F{}, false, 0);
          }
          block_sync_lds();
        }
      }
      return restart;
    };
    if (attend(true)) {
      for (int it = 0; it < n_tiles; ++it) {
        cp_p.all(tile_src(it, page_of(it)), lds);
        vm_wait<0>();
        block_sync_lds();                          // tile it landed in buffer 0
        block_sync_lds();                          // buffer 0 read
      }
      block_sync_lds();                            // (the QK waves' exchange of the row maxima)
      start_tiles();
      block_sync_lds();
      attend(false);
    }

    // epilogue: the row sums from LDS; normalised o_lat as bf16 in LDS over
    // the tile buffers, row r at r * OL_STRIDE, latent-major
    block_sync_lds();
    {
      const int tq = lane & 31;
#pragma unroll
      for (int nt = 0; nt < C::NTR; ++nt) {
        const int r = 32 * nt + tq;
        const float lt = xch[r] + xch[C::ROWS_WG + r];
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int m = 0; m < C::MTW; ++m) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int lat = 32 * (v + NPW * m) + 8 * a + 4 * hh;
            const f32x16& om = o[m][nt];
            const u32x2 pk = {pack_bf16x2(om[4 * a] * inv, om[4 * a + 1] * inv),
                              pack_bf16x2(om[4 * a + 2] * inv, om[4 * a + 3] * inv)};
            *(__attribute__((address_space(3))) u32x2*)(lds + r * C::OL_STRIDE + 2 * lat) = pk;
          }
        }
      }
    }
    block_sync_lds();
  }
  // one 1 KB row per store instruction; wave w writes rows w, w + NW, ...
  for (int j = w; j < C::ROWS_WG; j += NW) {
    const int rq = rb * C::ROWS_WG + j;
    uint16_t* dst = p.olat + (((size_t)u * SQ + rq % SQ) * H + rq / SQ) * R;
    for (int e = lane; e < R / 8; e += 64)
      *reinterpret_cast<u32x4*>(dst + 8 * e) = *(const lds_u32x4_t*)(lds + j * C::OL_STRIDE + 16 * e);
  }
}

// Memory-side (Infinity) cache of the MI355X.
constexpr double kMallBytes = 256.0 * 1024 * 1024;

template <int HPG, int SQ, int R, int DR, int QC>
hipError_t launch_absorb_wide(const DecodeParams& p, hipStream_t stream) {
  using C = WideCfg<HPG, SQ, R, DR, QC>;
  const int rows_total = HPG * p.num_groups * SQ;
  const int RB = rows_total / C::ROWS_WG;
  const unsigned grid = (unsigned)((p.num_units + 7) / 8) * 8u * (unsigned)RB;
  // block-table entries one unit can span: a split's share, else a whole row
  const long unit_pages = p.split_offsets ? (long)p.split_tokens / C::BS : (long)p.max_blocks;
  // latent bytes the call can read (units x their longest span): the
  // non-temporal copies when that exceeds the memory-side cache
  const double span_tokens = p.split_offsets ? (double)p.num_units * p.split_tokens
                                             : (double)p.batch * p.max_blocks * C::BS;
  const bool nt = span_tokens * C::ROW * 2.0 > kMallBytes;
  const dim3 g3(grid), b3(64 * C::NW);
  if (unit_pages <= C::PG_MAX) {
    if (nt) hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, QC, true, true>), g3, b3, 0, stream, p);
    else hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, QC, true, false>), g3, b3, 0, stream, p);
  } else {
    if (nt) hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, QC, false, true>), g3, b3, 0, stream, p);
    else hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, QC, false, false>), g3, b3, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace gqla
