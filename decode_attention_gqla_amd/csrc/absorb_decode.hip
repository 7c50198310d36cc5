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
//   1. absorb_q_kernel: q_abs for every query row of the batch (a per-group
//      [rows x d_nope] x [d_nope x r] MFMA product), stored with q_rope as one
//      bf16 row of r + d_R in the workspace;
//   2. wuv_transpose_kernel: W_UV^T into the workspace, its latent index
//      permuted inside each 32-wide block to the order in which the decode
//      kernel's accumulators hold o_lat (see the epilogue);
//   3. absorb_decode_kernel: attention + up-projection, one workgroup of four
//      waves (one per SIMD, so each wave may hold 512 registers) per (split
//      of a sequence, block of 128 query rows).
//
// Decode kernel.  Each 32-token latent tile (36 KB for r + d_R = 576) is
// copied HBM -> LDS by direct DMA (global_load_lds_dwordx4; four tile
// buffers, tiles it+1 and it+2 in flight while tile it is used) into a
// XOR-swizzled token-major layout.  Wave w owns 32 query rows end to end:
//   * its query rows (two 16-row tiles x the full 576-wide contraction) stay
//     in registers as MFMA B operands;
//   * S^T = C_tile . Q^T: each 16-token x 32-dim cache operand read from LDS
//     feeds two MFMAs (the two row tiles);
//   * online softmax inside the wave: the token order of a tile is relabelled
//     so that the S^T accumulators are exactly the P^T B operands of the PV
//     product, so P never leaves registers;
//   * O^T[latent][row] += C^T P^T over all 512 latent dims: the O
//     accumulators (32 rows x 512 fp32) live in the accumulation registers;
//     each C^T operand is read by the transposing LDS read ds_read_b64_tr_b16
//     and feeds two MFMAs.
// One workgroup barrier per tile (copies landed, and the buffer refilled next
// has been read by every wave).  The PV product of tile it-1 runs in the same
// iteration as QK of tile it, so the MFMA units see both streams, and the
// copies of tile it+2 are issued one instruction at a time between QK steps.
// Epilogue: o_lat is normalised, rounded to bf16 and fed straight from the
// accumulators into out^T = W_UV^T o_lat^T on MFMA (no LDS staging).
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

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
  static constexpr int NBUF = 4;                  // tile buffers
  static constexpr int ROW = R + DR;              // latent row (elements)
  static constexpr int CHR = ROW / 8;             // 16-byte chunks per token row
  static constexpr bool SWZ = (CHR % 8) == 0;     // XOR swizzle stays inside a row
  static constexpr int BUF_BYTES = TILE * ROW * 2;
  static constexpr int NI = TILE * CHR / 64;      // wave-wide DMA instructions per tile
  static constexpr int NW = 4;                    // waves per workgroup (one per SIMD)
  static constexpr int NIW = (NI + NW - 1) / NW;  // most DMA instructions of one wave per tile
  static constexpr int NTW = 1;                   // 16-row tiles per wave
  static constexpr int ROWS_W = 16 * NTW;         // query rows per wave
  static constexpr int ROWS_WG = NW * ROWS_W;
  static constexpr int KSL = R / 32;              // k steps over the latent
  static constexpr int KSR = (DR + 31) / 32;      // k steps over the rope key (zero padded)
  static constexpr int KS = KSL + KSR;
  static constexpr int MTL = R / 16;              // 16-dim tiles of o_lat
  static constexpr int MD = DV / 16;              // 16-dim tiles of the output
  static constexpr int OFF_FLAG = NBUF * BUF_BYTES;          // restart request (int)
  static constexpr int LDS_BYTES = OFF_FLAG + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert((TILE * CHR) % 64 == 0, "tile must be whole DMA instructions");
  static_assert(R % 32 == 0 && DN % 32 == 0 && DV % 16 == 0, "unsupported dims");
  static_assert(!SWZ || MTL % 4 == 0, "swizzled PV addressing takes latent tiles in fours");
  static_assert(NIW <= 23, "vmcnt budget");
};

// Swizzle of 16-byte chunk positions inside a token row (tokens 0..31 of a
// tile).  gfx950 LDS has 64 four-byte banks; a 16-byte read is served in four
// passes of 16 lanes (per half wave, the 4-lane quads of even and of odd bit
// parity), an 8-byte or transposing read in two passes of 32 lanes.  With a
// 1152-byte token row, XOR-ing chunk bits 1 and 2 with token bits 1 and 3
// gives every pass of the QK reads (16 tokens, one chunk) and of the
// transposing PV reads (8 tokens x 4 half-chunks) 64 distinct banks.
__device__ __forceinline__ int tile_swz(int t) { return 4 * ((t >> 3) & 1) + 2 * ((t >> 1) & 1); }

template <int HPG, int SQ, int R, int DR, int DN, int DV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void absorb_decode_kernel(DecodeParams p) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KSL = C::KSL, KS = C::KS;
  constexpr int MD = C::MD, MTL = C::MTL, NW = C::NW, NTW = C::NTW;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  // Workgroups are dispatched round-robin over the 8 XCDs; the row blocks of
  // one split unit take consecutive slots on one XCD (shared L2).
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int u = (k / RB) * 8 + xcd;
  const int rb = k % RB;
  if (u >= p.num_units) return;                   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int c = lane & 15, q = lane >> 4;
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
  // space, wave-uniform index).  The per-lane source offsets of this wave's
  // copy instructions are the same for every tile and are computed once.
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
    asm volatile("" : "+v"(dvo[kk]));             // keep, do not recompute per tile
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

  // ---- this wave's query rows: tiles nt < NTW of rows row0 + 16 nt + c ----
  const int row0 = rb * C::ROWS_WG + C::ROWS_W * w;
  const bool active = row0 < rows_total;          // wave-uniform
  const bool rows_all_valid = row0 + C::ROWS_W <= rows_total;
  bf16x8 qb[NTW][KS];
  int s_nvis[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int rho = row0 + 16 * nt + c;
    const bool valid = rho < rows_total;
    const int h = valid ? rho / SQ : 0, i = valid ? rho % SQ : 0;
    s_nvis[nt] = valid ? L - SQ + i + 1 : -1;
    const uint16_t* qrow = p.qcat + (((size_t)b * SQ + i) * H + h) * ROW;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dim = 32 * ks + 8 * q;
      qb[nt][ks] = (valid && dim < ROW) ? ld_bf16x8(qrow + dim) : zero_bf16x8();
    }
  }

  // Per-lane LDS byte offsets of the MFMA operands inside a tile buffer
  // (computed once; each read adds the buffer's offset and an immediate).
  // QK operand of token half st: token t = 8*(c/4) + 4*st + c%4, chunk
  // 4ks + q, which sits at 4*(ks ^ s2) + (q ^ (sw & 3)) with sw = tile_swz(t),
  // s2 = sw >> 2: one base per (st, ks parity), the rest is 64 ks bytes.
  int qkb[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int t = 8 * (c >> 2) + 4 * st + (c & 3);
      const int sw = C::SWZ ? tile_swz(t) : 0;
      const int lowq = q ^ (sw & 3), s2 = sw >> 2;
      qkb[st][par] = (t * CHR + lowq + 4 * (par == 0 ? s2 : -s2)) * 16;
      asm volatile("" : "+v"(qkb[st][par]));
    }
  // PV operand (transposing reads), half hh: tokens t = 8q + c/4 + 4hh, latent
  // 16mt + 4*(c%4), i.e. chunk 2mt + b1 (b1 = (c%4)/2), which the swizzle puts
  // at 2*((mt & ~3) | ((mt & 3) ^ (sw >> 1))) + (b1 ^ (sw & 1)): one base per
  // (hh, mt % 4), the rest is 128 (mt / 4) bytes; unswizzled, 32 mt bytes.
  constexpr int NPV = C::SWZ ? 4 : 1;
  int pvb[2][NPV];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int m3 = 0; m3 < NPV; ++m3) {
      const int t = 8 * q + (c >> 2) + 4 * hh;
      const int sw = C::SWZ ? tile_swz(t) : 0;
      const int b1 = (c & 3) >> 1, half = ((4 * (c & 3)) & 7) * 2;
      pvb[hh][m3] = (t * CHR + 2 * (m3 ^ (sw >> 1)) + (b1 ^ (sw & 1))) * 16 + half;
      asm volatile("" : "+v"(pvb[hh][m3]));
    }
  auto pv_operand = [&](const lds_u8_t* buf, int mt) -> bf16x8 {
    const int m3 = C::SWZ ? (mt & 3) : 0;
    const int imm = C::SWZ ? 128 * (mt >> 2) : 32 * mt;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[0][m3] + imm));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + pvb[1][m3] + imm));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Softmax reference.  A row's reference is its first finite tile maximum
  // and then stays fixed, so the O accumulators are only ever written by
  // MFMAs (an in-place rescale of the accumulation registers would need a
  // second register set).  Every p = 2^(x - ref) is kept below 2^kSlack; a
  // tile maximum above ref + kSlack (an extreme logit spread, e.g. one
  // dominant token) makes the workgroup restart the split: pass 1 sweeps QK
  // for the exact row maxima, pass 2 reruns the attention with them as the
  // references (then p <= 1).
  constexpr float kSlack = 64.f;
  f32x4 o[MTL][NTW];                              // O^T: lane (q, c) = latent 16mt + 4q.., row c
  float m_run[NTW], l_run[NTW];
  bf16x8 pb[NTW];                                 // P^T operands of the previous tile
  int* const restart_flag = (int*)(lds_raw + C::OFF_FLAG);
  if (tid == 0) *restart_flag = 0;                // ordered before its reads by the first barrier
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) m_run[nt] = -INFINITY;

  // The query loads complete before the first copy is issued, so the
  // compiler's own wait tracking has nothing pending inside the tile loop.
  vm_wait<0>();
  for (int pass = 0; pass < 3; ++pass) {          // 0: single pass; 1, 2: after a restart
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int mt = 0; mt < MTL; ++mt) o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run[nt] = 0.f;
      pb[nt] = zero_bf16x8();
    }
    for (int i = 0; i < 2 && i < n_tiles; ++i) {
      const Copy cp = copy_of(i);
      for (int kk = 0; kk < niw; ++kk) copy_part(cp, kk);
    }
    bool restart = false;
    for (int it = 0; it <= n_tiles; ++it) {
      // tile it landed (own copies; tile it+1 may still be in flight), then
      // for every wave; every wave is also past PV of tile it-2, whose buffer
      // takes tile it+2
      if (it + 1 < n_tiles) {
        if constexpr (kFixedCopies) vm_wait<C::NIW>(); else vm_wait_dyn(niw);
      } else {
        vm_wait<0>();
      }
      block_sync_lds();
      // a restart request posted before this barrier (pass 0 only)
      const int flag = pass == 0 ? *(volatile int*)restart_flag : 0;
      if (it < n_tiles && lo + C::TILE * (it + 1) > L) {
        // the sequence's last tile: token rows past its end hold anything
        // (the page's unused slots); zero them so the PV product needs no
        // mask (their logits are masked, but 0 * NaN would still be NaN)
        const int valid = L - (lo + C::TILE * it);
        lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
        for (int off = valid * ROW * 2 + tid * 16; off < C::BUF_BYTES; off += 64 * NW * 16)
          *(lds_u32x4_t*)(buf + off) = u32x4{0u, 0u, 0u, 0u};
        block_sync_lds();
      }
      const bool more = it + 2 < n_tiles;
      Copy cp = {nullptr, nullptr};
      if (more) cp = copy_of(it + 2);

      // ---- S^T of tile it: 2 token halves x NTW row tiles, full contraction ----
      // With a fixed copy count per wave, the copies of tile it+2 are issued
      // one at a time between QK steps (two copies of the unrolled QK body,
      // with and without them, so no runtime branch sits between the MFMAs);
      // otherwise they all go out after QK.
      f32x4 s[2][NTW];
      auto qk_tile = [&](auto with_copies) {
        constexpr bool WITH = decltype(with_copies)::value;
        const lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
        auto qk_operand = [&](int step) -> bf16x8 {  // step = 2 ks + st
          const int ks = step >> 1, st = step & 1;
          const bool have = ks < KSL || 32 * (ks - KSL) + 8 * q < DR;
          if (!have) return zero_bf16x8();
          return __builtin_bit_cast(bf16x8,
                                    *(const lds_u32x4_t*)(buf + qkb[st][C::SWZ ? (ks & 1) : 0] + 64 * ks));
        };
        constexpr int NS = 2 * KS, PD = 6;
        constexpr int GAP = NS / (C::NIW + 1) > 0 ? NS / (C::NIW + 1) : 1;   // QK steps between copies
        bf16x8 a[PD + 1];
#pragma unroll
        for (int j = 0; j < PD && j < NS; ++j) a[j] = qk_operand(j);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (j + PD < NS) a[(j + PD) % (PD + 1)] = qk_operand(j + PD);
          const int ks = j >> 1, st = j & 1;
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            s[st][nt] = mfma16(a[j % (PD + 1)], qb[nt][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[st][nt]);
          if (WITH && j % GAP == GAP - 1 && j / GAP < C::NIW) copy_part(cp, j / GAP);   // folded at compile time
        }
        // schedule: the first PD operand reads, then per step the read of
        // operand j + PD followed by the MFMA(s) of step j
        __builtin_amdgcn_sched_group_barrier(0x100, PD < NS ? PD : NS, 0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          if (j + PD < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NTW, 0);
        }
      };
      int issued = 0;
      if (it < n_tiles && active) {
        if (kFixedCopies && more) {
          qk_tile(std::true_type{});
          issued = niw;
        } else {
          qk_tile(std::false_type{});
        }
      }
      if (more)
        for (; issued < niw; ++issued) copy_part(cp, issued);
      if (__builtin_amdgcn_readfirstlane(flag)) { // uniform over the workgroup
        restart = true;
        break;
      }

      // ---- O^T += C^T P^T for tile it-1 ----
      if (pass != 1 && it > 0 && active) {
        const lds_u8_t* buf = lds + ((it - 1) % C::NBUF) * C::BUF_BYTES;
        constexpr int PV = 6;                     // operands read ahead
        bf16x8 v[PV + 1];
#pragma unroll
        for (int j = 0; j < PV && j < MTL; ++j) v[j] = pv_operand(buf, j);
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) {
          if (mt + PV < MTL) v[(mt + PV) % (PV + 1)] = pv_operand(buf, mt + PV);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) o[mt][nt] = mfma16(v[mt % (PV + 1)], pb[nt], o[mt][nt]);
        }
        // schedule: the first PV operands' reads, then per step the reads of
        // operand mt + PV followed by the MFMA(s) of step mt
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PV < MTL ? PV : MTL), 0);
#pragma unroll
        for (int mt = 0; mt < MTL; ++mt) {
          if (mt + PV < MTL) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NTW, 0);
        }
      }
      if (it == n_tiles) break;

      // ---- softmax of tile it (base 2), per row tile ----
      if (active) {
        const int t0 = lo + C::TILE * it;
        // masking is needed only on tiles that reach the first causal bound
        const bool masked = t0 + C::TILE > L - SQ + 1 || !rows_all_valid;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          // lane (q, c): tokens t0 + 8q + 4st + i of row c (st = 0, 1; i = 0..3)
          float x[8];
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[4 * st + i] = s[st][nt][i] * p.scale_log2;
          if (masked) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              x[j] = (t0 + 8 * q + 4 * (j >> 2) + (j & 3) < s_nvis[nt]) ? x[j] : -INFINITY;
          }
          float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
          mx = wave_max_q(mx);
          if (pass == 1) {                        // exact row maxima only
            m_run[nt] = fmaxf(m_run[nt], mx);
            continue;
          }
          if (pass == 0) {
            // a row takes its first finite tile maximum as its reference (its
            // O and l are still 0); a later maximum far above it restarts
            m_run[nt] = m_run[nt] == -INFINITY ? mx : m_run[nt];
            if (__any(mx > m_run[nt] + kSlack) && lane == 0) *restart_flag = 1;
          }
          const float m_use = (m_run[nt] == -INFINITY) ? 0.f : m_run[nt];
          float ps = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
            ps += x[j];
          }
          l_run[nt] += ps;
          pb[nt] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                                    pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])});
        }
      }
    }
    if (pass == 0 && !restart) break;             // the common case: done in one pass
    // drain this pass's copies before the tile buffers are refilled
    vm_wait<0>();
    block_sync_lds();
    if (pass == 0) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) m_run[nt] = -INFINITY;
    }
  }
  if (!active) return;                            // no barrier follows

  // ---- epilogue: lse, then out^T = W_UV^T o_lat^T straight from the accumulators ----
  // The B operand of k step kk (latent block 32kk .. 32kk+31) for row c is
  // lane (q, c): o_lat[16(2kk) + 4q + e] (e < 4) and o_lat[16(2kk+1) + 4q + e - 4]
  // (e >= 4), i.e. the lane's own accumulators o[2kk] and o[2kk+1]; the
  // workspace W_UV^T is stored with the latent index permuted the same way
  // inside each 32-block, so the A operand is one 16-byte load.
  const uint16_t* const wuvP = p.wuvT;
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float lt = wave_sum_q(l_run[nt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int r_first = row0 + 16 * nt;
    if (r_first >= rows_total) break;             // uniform
    const int rho = r_first + c;
    const bool valid = rho < rows_total;
    const int h = valid ? rho / SQ : 0, i = valid ? rho % SQ : 0;
    if (q == 0 && valid) {
      const float lse_v = lt > 0.f ? (m_run[nt] + log2f(lt)) * kLn2 : -INFINITY;
      if (p.split_offsets) p.part_lse[((size_t)u * SQ + i) * H + h] = lse_v;
      else if (p.lse) p.lse[((size_t)b * SQ + i) * H + h] = lse_v;
    }
    const int r_last = min(r_first + 15, rows_total - 1);
    const int g_lo = (r_first / SQ) / HPG, g_hi = (r_last / SQ) / HPG;
    const int myG = valid ? h / HPG : -1;
    // normalised o_lat of this row tile as bf16 B operands, built once
    bf16x8 bo[R / 32];
#pragma unroll
    for (int kk = 0; kk < R / 32; ++kk) {
      const f32x4 lo4 = o[2 * kk][nt] * inv, hi4 = o[2 * kk + 1][nt] * inv;
      bo[kk] = __builtin_bit_cast(bf16x8, u32x4{pack_bf16x2(lo4[0], lo4[1]), pack_bf16x2(lo4[2], lo4[3]),
                                                pack_bf16x2(hi4[0], hi4[1]), pack_bf16x2(hi4[2], hi4[3])});
    }
    for (int G = g_lo; G <= g_hi; ++G) {
      const uint16_t* WT = wuvP + (size_t)G * DV * R;
      f32x4 acc[MD];
#pragma unroll
      for (int md = 0; md < MD; ++md) acc[md] = f32x4{0.f, 0.f, 0.f, 0.f};
      // W_UV^T operands loaded one k step ahead (the compiler barrier keeps
      // the remaining loads from being hoisted into a register flood)
      bf16x8 wa[2][MD];
#pragma unroll
      for (int md = 0; md < MD; ++md) wa[0][md] = ld_bf16x8(WT + (size_t)(16 * md + c) * R + 8 * q);
#pragma unroll
      for (int kk = 0; kk < R / 32; ++kk) {
        if (kk + 1 < R / 32) {
#pragma unroll
          for (int md = 0; md < MD; ++md)
            wa[(kk + 1) & 1][md] = ld_bf16x8(WT + (size_t)(16 * md + c) * R + 32 * (kk + 1) + 8 * q);
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) acc[md] = mfma16(wa[kk & 1][md], bo[kk], acc[md]);
        asm volatile("" ::: "memory");
      }
      // acc[md] lane (q, c): output dims 16md + 4q .. +3 of row c
      if (myG != G) continue;
      if (p.split_offsets) {
        const size_t row = ((size_t)u * SQ + i) * H + h;
#pragma unroll
        for (int md = 0; md < MD; ++md)
          *reinterpret_cast<f32x4*>(p.part_out + row * DV + 16 * md + 4 * q) = acc[md];
      } else {
        const size_t row = ((size_t)b * SQ + i) * H + h;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          u32x2 pk = {pack_bf16x2(acc[md][0], acc[md][1]), pack_bf16x2(acc[md][2], acc[md][3])};
          *reinterpret_cast<u32x2*>(p.out + row * DV + 16 * md + 4 * q) = pk;
        }
      }
    }
  }
}

// q_abs = W_UK[G] q_nope for every (sequence, MTP row, head), written next to
// q_rope as one [r + d_R] bf16 row per query row (the QK operand of the decode
// kernel).  Per group this is a [rows x d_nope] x [d_nope x r] product over all
// rows of the batch, so each W_UK[G] is fetched by few workgroups.
// Workgroup = 4 waves x 16 query rows of one group; D = q_abs^T (m = latent,
// n = row) so each lane stores 4 consecutive latent values of one row.
template <int HPG, int SQ, int R, int DR, int DN>
__global__ __launch_bounds__(256) void absorb_q_kernel(DecodeParams p) {
  constexpr int ROW = R + DR, KD = DN / 32, MT = R / 16;
  constexpr int MTC = MT < 8 ? MT : 8;               // latent tiles per workgroup (blockIdx.z)
  const int g = p.num_groups, H = HPG * g;
  const int rows_g = p.batch * SQ * HPG;             // query rows of one group
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int G = blockIdx.y;
  const int r0 = (blockIdx.x * 4 + w) * 16;          // first group-row of this wave
  if (r0 >= rows_g) return;
  // group-row gr = (b * SQ + i) * HPG + hl  ->  head h = G*HPG + hl
  const int gr = r0 + c;
  const bool valid = gr < rows_g;
  const int hl = gr % HPG, bi = gr / HPG;            // bi = b * SQ + i
  const size_t qrow = ((size_t)bi * H + G * HPG + hl);
  bf16x8 qn[KD];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd)
    qn[kd] = valid ? ld_bf16x8(p.q_nope + qrow * DN + 32 * kd + 8 * q) : zero_bf16x8();
  const uint16_t* W = p.w_uk + (size_t)G * R * DN;
  uint16_t* dst = p.qcat + qrow * ROW;
  const int mt0 = blockIdx.z * MTC;
#pragma unroll
  for (int mt = mt0; mt < mt0 + MTC; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      acc = mfma16(ld_bf16x8(W + (size_t)(16 * mt + c) * DN + 32 * kd + 8 * q), qn[kd], acc);
    // lane (q, c): latent 16mt + 4q .. +3 of row c
    if (valid) {
      u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
      *reinterpret_cast<u32x2*>(dst + 16 * mt + 4 * q) = pk;
    }
  }
  // rope part copied unchanged
  if (blockIdx.z != 0) return;
  for (int id = lane; id < 16 * DR / 8; id += 64) {
    const int rr = id / (DR / 8), part = id % (DR / 8);
    const int gr2 = r0 + rr;
    if (gr2 >= rows_g) continue;
    const size_t qr2 = ((size_t)(gr2 / HPG) * H + G * HPG + gr2 % HPG);
    *reinterpret_cast<u32x4*>(p.qcat + qr2 * ROW + R + part * 8) =
        *reinterpret_cast<const u32x4*>(p.q_rope + qr2 * DR + part * 8);
  }
}

// W_UV[G] (r x d_v) -> W_UV^T[G] (d_v x r) with the latent index permuted
// inside each 32-wide block: position 8q + e holds latent 4q + e (e < 4) or
// 16 + 4q + e - 4 (e >= 4), the order in which lane q of the decode kernel's
// accumulators holds o_lat, so the up-projection's A operand (8 positions of
// one output column) is one contiguous 16-byte load.
template <int R, int DV>
__global__ __launch_bounds__(256) void wuv_transpose_kernel(DecodeParams p) {
  const int G = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;     // one latent row x 8 columns
  if (idx >= R * (DV / 8)) return;
  const int l = idx / (DV / 8), d0 = (idx % (DV / 8)) * 8;
  const int lb = l & 31;
  const int pos = (l & ~31) | (8 * ((lb & 15) >> 2) + 4 * (lb >> 4) + (lb & 3));
  const u32x4 v = *reinterpret_cast<const u32x4*>(p.w_uv + ((size_t)G * R + l) * DV + d0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t e = (uint16_t)(v[j / 2] >> (16 * (j & 1)));
    p.wuvT[((size_t)G * DV + d0 + j) * R + pos] = e;
  }
}

template <int HPG, int SQ, int R, int DR, int DN, int DV>
hipError_t launch_absorb(const DecodeParams& p, hipStream_t stream) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  {
    const int rows_g = p.batch * SQ * HPG;
    constexpr int MT = R / 16, MTC = MT < 8 ? MT : 8;
    dim3 grid((unsigned)((rows_g + 63) / 64), (unsigned)p.num_groups, (unsigned)(MT / MTC));
    hipLaunchKernelGGL((absorb_q_kernel<HPG, SQ, R, DR, DN>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    dim3 grid((unsigned)((R * (DV / 8) + 255) / 256), (unsigned)p.num_groups);
    hipLaunchKernelGGL((wuv_transpose_kernel<R, DV>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows_total = HPG * p.num_groups * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  const unsigned grid = (unsigned)((p.num_units + 7) / 8) * 8u * (unsigned)RB;
  hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, DN, DV>), dim3(grid), dim3(64 * C::NW), 0,
                     stream, p);
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
