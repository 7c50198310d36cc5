// MQA-absorb decode over the shared latent cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "MQA-absorb path" and
// gist.science section 2 "MQA-Absorb-Pfad": W_UK[G] is folded into the query
// of every head, all h_q heads attend over the latent cache c^KV_t ++ k^R_t
// (read once and shared by every query row), and W_UV[G] up-projects the
// latent output.  Per query row (head h in group G, MTP row i):
//   q_abs = W_UK[G] q_nope,   s_t = (q_abs . c_t + q_rope . k_rope_t) * scale,
//   o_lat = softmax(s) C,     out = o_lat W_UV[G].
//
// Three kernels per call:
//   1. absorb_q_kernel: q_abs for every query row of the batch (a per-group
//      [rows x d_nope] x [d_nope x r] MFMA product), stored with q_rope as one
//      bf16 row of r + d_R in the workspace;
//   2. wuv_transpose_kernel: W_UV^T into the workspace (so the up-projection
//      reads its operand rows contiguously);
//   3. absorb_decode_kernel: attention + up-projection, one workgroup of 8
//      waves per (split of a sequence, block of 64 query rows).  The row
//      blocks of one split run side by side on one XCD, so each cache byte is
//      fetched from HBM once and re-read from that XCD's L2.
//
// Inside the decode kernel each 32-token latent tile is copied HBM -> LDS by
// direct DMA (global_load_lds_dwordx4, three tiles in flight) into a
// XOR-swizzled token-major layout, and the 8 waves split the work so that
// the query operands (64 rows x 576) and the output accumulators
// (64 rows x 512 fp32) sit in registers with room to spare:
//   QK      wave (16-row tile rt, half kh): S^T over half of the 576-wide
//           contraction; the two halves are summed through LDS;
//   softmax waves 0..3 own one 16-row tile each: online softmax, P (bf16)
//           to LDS;
//   PV      wave w owns latent dims [64w, 64w + 64) of all 64 rows:
//           O^T[latent][row] += C^T . P^T, with C^T read by the LDS
//           transposing read ds_read_b64_tr_b16 once and reused for the 4
//           16-row tiles.
// Epilogue: o_lat (bf16) staged in LDS; wave w up-projects half of the
// output dims of one 16-row tile: out^T = W_UV^T o_lat^T on MFMA.
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Outstanding-copy counts are wave-uniform but not compile-time constants.
__device__ __forceinline__ void vm_wait_dyn(int n) {
  switch (n) {
#define GQLA_WV(N) case N: vm_wait<N>(); break;
    GQLA_WV(0) GQLA_WV(1) GQLA_WV(2) GQLA_WV(3) GQLA_WV(4) GQLA_WV(5) GQLA_WV(6) GQLA_WV(7)
    GQLA_WV(8) GQLA_WV(9) GQLA_WV(10) GQLA_WV(11) GQLA_WV(12) GQLA_WV(13) GQLA_WV(14) GQLA_WV(15)
#undef GQLA_WV
    default: vm_wait<0>(); break;
  }
}

template <int HPG, int SQ, int R, int DR, int DN, int DV>
struct AbsorbCfg {
  static constexpr int BS = 64;
  static constexpr int TILE = 32;                 // tokens per LDS tile
  static constexpr int NBUF = 3;
  static constexpr int ROW = R + DR;              // latent row (elements)
  static constexpr int CHR = ROW / 8;             // 16-byte chunks per token row
  static constexpr bool SWZ = (CHR % 8) == 0;     // XOR swizzle stays inside a row
  static constexpr int BUF_BYTES = TILE * ROW * 2;
  static constexpr int NI = TILE * CHR / 64;      // wave-wide DMA instructions per tile
  static constexpr int NW = 8;                    // waves per workgroup
  static constexpr int ROWS_WG = 64;              // query rows per workgroup (4 n-tiles)
  static constexpr int NTW = ROWS_WG / 16;        // 16-row tiles per workgroup
  static constexpr int KSL = R / 32;              // k steps over the latent
  static constexpr int KSR = (DR + 31) / 32;      // k steps over the rope key (zero padded)
  static constexpr int KS = KSL + KSR;
  static constexpr int KSH = (KS + 1) / 2;        // k steps per half
  static constexpr int MTL = R / 16;              // 16-dim tiles of o_lat
  static constexpr int MTW = MTL >= NW ? MTL / NW : 1;   // latent tiles per wave in PV
  static constexpr int MD = DV / 16;              // 16-dim tiles of the output
  // LDS map (bytes)
  static constexpr int OFF_SP = NBUF * BUF_BYTES;            // partial S: [2][NTW][2][64] f32x4
  static constexpr int OFF_PB = OFF_SP + 2 * NTW * 2 * 64 * 16;     // P: [NTW][64] bf16x8
  static constexpr int OFF_AL = OFF_PB + NTW * 64 * 16;      // alpha per row [ROWS_WG] f32
  static constexpr int OFF_FL = OFF_AL + ROWS_WG * 4;        // rescale flag per n-tile i32
  static constexpr int OFF_IL = OFF_FL + 64;                 // 1/l per row [ROWS_WG] f32
  static constexpr int LDS_BYTES = OFF_IL + ROWS_WG * 4;
  static constexpr int OLAT_BYTES = ROWS_WG * R * 2;         // epilogue staging (overlaps KV/SP)
  static constexpr int OSWZ = (R / 8) >= 16 ? 15 : (R / 8) - 1;   // o_lat chunk swizzle mask
  static_assert(OLAT_BYTES <= OFF_AL, "o_lat staging must not overlap the row arrays");
  static_assert((TILE * CHR) % 64 == 0, "tile must be whole DMA instructions");
  static_assert(R % 32 == 0 && DN % 32 == 0 && DV % 16 == 0, "unsupported dims");
  static_assert(MTL % NW == 0 || MTL < NW, "latent tiles must split evenly over waves");
  static_assert(!SWZ || MTW % 4 == 0, "swizzled PV addressing needs 4 tiles per wave");
  static_assert((NI + NW - 1) / NW <= 15, "vmcnt budget");
  static_assert(NW == 2 * NTW, "one QK wave per (n-tile, contraction half)");
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
__global__ __launch_bounds__(512, 1) void absorb_decode_kernel(DecodeParams p) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KSL = C::KSL, KS = C::KS;
  constexpr int KSH = C::KSH, MTW = C::MTW, MD = C::MD, MTL = C::MTL;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
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
  const int row_base = rb * C::ROWS_WG;           // first query row of this workgroup

  // ---- HBM -> LDS tile copy (each wave issues instructions w, w+8, ...) ----
  const int niw = (C::NI - w + C::NW - 1) / C::NW;
  auto issue_tile = [&](int it) {
    const int t0 = lo + C::TILE * it;
    const uint16_t* src = p.cache + ((size_t)sload_i32(bt + t0 / BS) * BS + (t0 % BS)) * ROW;
    lds_u8_t* dst = lds + (it % C::NBUF) * C::BUF_BYTES;
    for (int i = w; i < C::NI; i += C::NW) {
      const int P = i * 64 + lane;
      const int t = P / CHR, pos = P % CHR;
      const int ch = C::SWZ ? (pos ^ tile_swz(t)) : pos;
      dma16(src, (uint32_t)(t * ROW + ch * 8) * 2u, dst + i * 1024);
    }
  };

  // ---- QK role: 16-row tile rt, k steps [kh*KSH, kh*KSH + KSH) ----
  const int rt = w >> 1, kh = w & 1;
  bf16x8 qb[KSH];
  {
    const int rho = row_base + 16 * rt + c;
    const bool valid = rho < rows_total;
    const int h = valid ? rho / SQ : 0, i = valid ? rho % SQ : 0;
    const uint16_t* qrow = p.qcat + (((size_t)b * SQ + i) * H + h) * ROW;
#pragma unroll
    for (int j = 0; j < KSH; ++j) {
      const int dim = 32 * (kh * KSH + j) + 8 * q;
      qb[j] = (valid && kh * KSH + j < KS && dim < ROW) ? ld_bf16x8(qrow + dim) : zero_bf16x8();
    }
  }
  // ---- softmax role (waves 0 .. NTW-1): rows 16*w .. 16*w+15 of the block ----
  const bool smax_wave = w < C::NTW;
  const int srow = 16 * (w % C::NTW) + c;         // block-local row of this lane
  const int srho = row_base + srow;
  const bool svalid = smax_wave && srho < rows_total;
  const int s_nvis = svalid ? L - SQ + (srho % SQ) + 1 : -1;
  float m_run = -INFINITY, l_run = 0.f;

  // Per-lane LDS byte offsets of the MFMA operands inside a tile buffer,
  // recomputed each tile from an opaque zero (cheaper than keeping a dozen
  // loop-invariant registers live across the tile loop).
  // QK: token t = 8*(c/4) + 4*st + c%4, chunk 4ks + q, which sits at
  // 4*(ks ^ s2) + (q ^ (sw & 3)) with sw = tile_swz(t), s2 = sw >> 2: one base
  // per ks parity, the rest an immediate offset.
  auto qk_base = [&](int z, int st, int par) -> int {
    const int t = 8 * (c >> 2) + 4 * st + (c & 3) + z;
    const int sw = C::SWZ ? tile_swz(t) : 0;
    const int lowq = q ^ (sw & 3), s2 = sw >> 2;
    return (t * CHR + lowq + 4 * (par == 0 ? s2 : -s2)) * 16;
  };
  // PV (transposing reads): tokens t = 8q + c/4 (+4), latent 16mt + 4*(c%4),
  // chunk 2mt + b1 at 2*((mt & ~3) | ((mt & 3) ^ s1)) + (b1 ^ (sw & 1)).
  auto pv_base = [&](int z, int hh, int m3) -> int {
    const int t = 8 * q + (c >> 2) + 4 * hh + z;
    const int sw = C::SWZ ? tile_swz(t) : 0;
    const int b1 = (c & 3) >> 1, half = ((4 * (c & 3)) & 7) * 2;
    return (t * CHR + 2 * (m3 ^ (sw >> 1)) + (b1 ^ (sw & 1))) * 16 + half;
  };
  const int mt0 = w * MTW;                        // first latent tile of this wave (PV)
  const bool pv_active = mt0 < MTL;

  constexpr int NTW = C::NTW;
  f32x4 o[MTW][NTW];
#pragma unroll
  for (int j = 0; j < MTW; ++j)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) o[j][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The query loads complete before the first tile copy is issued, so the
  // compiler's own wait tracking has nothing pending inside the tile loop.
  vm_wait<0>();
  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  lds_u8_t* const sp = lds + C::OFF_SP;
  lds_u8_t* const pbuf = lds + C::OFF_PB;
  float* const al = (float*)(lds_raw + C::OFF_AL);
  int* const fl = (int*)(lds_raw + C::OFF_FL);

  for (int it = 0; it < n_tiles; ++it) {
    // tile it landed (own copies), then for every wave
    if (it + 1 < n_tiles) vm_wait_dyn(niw); else vm_wait<0>();
    block_sync_lds();
    const lds_u8_t* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
    const int t0 = lo + C::TILE * it;
    int z;                                        // opaque 0: keeps per-lane offsets in the loop
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));

    // ---- QK (half of the contraction), partial S^T to LDS ----
    {
      auto qk_operand = [&](int st, int j) -> bf16x8 {
        const int ks = kh * KSH + j;              // wave-uniform
        const bool have = ks < KS && (ks < KSL || 32 * (ks - KSL) + 8 * q < DR);
        if (!have) return zero_bf16x8();
        const int off = qk_base(z, st, C::SWZ ? (ks & 1) : 0) + 64 * ks;
        return __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + off));
      };
      // one token subtile at a time, operands read three steps ahead; the
      // compiler barrier per step keeps the remaining reads from being hoisted
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
        constexpr int PD = 3;
        bf16x8 a[PD + 1];
#pragma unroll
        for (int j = 0; j < PD && j < KSH; ++j) a[j] = qk_operand(st, j);
#pragma unroll
        for (int j = 0; j < KSH; ++j) {
          if (j + PD < KSH) a[(j + PD) % (PD + 1)] = qk_operand(st, j + PD);
          s0 = mfma16(a[j % (PD + 1)], qb[j], s0);
          asm volatile("" ::: "memory");
        }
        *(__attribute__((address_space(3))) f32x4*)(sp + (((kh * NTW + rt) * 2 + st) * 64 + lane) * 16) = s0;
      }
    }
    block_sync_lds();
    // every wave is past PV of tile it-1: its buffer can be refilled
    if (it + 2 < n_tiles) issue_tile(it + 2);

    // ---- softmax for rows 16w .. 16w+15 (waves 0 .. NTW-1) ----
    if (smax_wave) {
      // masking is needed only on tiles that reach the first causal bound
      const bool masked = t0 + C::TILE > L - SQ + 1 || !svalid;
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int base = (w * 2 + st) * 64 + lane;            // half 0 of (n-tile w, st)
        const f32x4 a0 = *(const __attribute__((address_space(3))) f32x4*)(sp + base * 16);
        const f32x4 a1 = *(const __attribute__((address_space(3))) f32x4*)(sp + (base + NTW * 2 * 64) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = (a0[i] + a1[i]) * p.scale_log2;
          if (masked) v = (t0 + 8 * q + 4 * st + i < s_nvis) ? v : -INFINITY;
          x[4 * st + i] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = wave_max_xor16_32(mx);
      // lazily moved reference max: rescale only when it grows by more than 8
      // (so every p <= 2^8), which after the first tiles is rare
      const bool resc = __any(mx > m_run + 8.f);
      if (resc) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        if (q == 0) al[srow] = alpha;
      }
      if (lane == 0) fl[w] = resc ? 1 : 0;
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
        ps += x[j];
      }
      l_run += ps;
      u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                  pack_bf16x2(x[6], x[7])};
      *(lds_u32x4_t*)(pbuf + (w * 64 + lane) * 16) = pk;
    }
    block_sync_lds();

    // ---- PV for latent tiles mt0 .. mt0+MTW-1 of all the block's rows ----
    if (pv_active) {
      int flags[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; nt += 4) {
        const u32x4 f4 = *(const lds_u32x4_t*)(lds + C::OFF_FL + nt * 4);
#pragma unroll
        for (int k2 = 0; k2 < 4 && nt + k2 < NTW; ++k2) flags[nt + k2] = (int)f4[k2];
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (flags[nt]) {                          // rows of n-tile nt moved their reference
          const float a = al[16 * nt + c];
#pragma unroll
          for (int j = 0; j < MTW; ++j) o[j][nt] *= a;
        }
      }
      const bool tail = t0 + C::TILE > L;
      const int keep = min(max(L - (t0 + 8 * q), 0), 8);
      // latent tiles two at a time (8 operand registers), P tiles re-read per pair
      constexpr int JP = MTW >= 2 ? 2 : 1;
#pragma unroll
      for (int j0 = 0; j0 < MTW; j0 += JP) {
        bf16x8 v[JP];
#pragma unroll
        for (int jj = 0; jj < JP; ++jj) {
          const int j = j0 + jj, mt = mt0 + j;
          if constexpr (C::SWZ) {
            const int off_lo = pv_base(z, 0, j & 3) + 128 * (mt >> 2);
            const int off_hi = pv_base(z, 1, j & 3) + 128 * (mt >> 2);
            s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + off_lo));
            s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + off_hi));
            v[jj] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            const int n = 16 * mt + 4 * (c & 3);
            const int ch = n >> 3, half = (n & 7) * 2;
            const int t_lo = 8 * q + (c >> 2), t_hi = t_lo + 4;
            s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + (t_lo * CHR + ch) * 16 + half));
            s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + (t_hi * CHR + ch) * 16 + half));
            v[jj] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          }
          if (tail) v[jj] = keep_first(v[jj], keep);   // tokens past the sequence end hold anything
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const bf16x8 pbv = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(pbuf + (nt * 64 + lane) * 16));
#pragma unroll
          for (int jj = 0; jj < JP; ++jj) o[j0 + jj][nt] = mfma16(v[jj], pbv, o[j0 + jj][nt]);
        }
        asm volatile("" ::: "memory");
      }
    }
  }

  // ---- epilogue ----
  float* const il = (float*)(lds_raw + C::OFF_IL);
  if (smax_wave) {
    const float lt = wave_sum_xor16_32(l_run);
    if (q == 0) il[srow] = lt > 0.f ? 1.f / lt : 0.f;
    if (q == 0 && svalid) {
      const float lse_v = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
      const int h = srho / SQ, i = srho % SQ;
      if (p.split_offsets) p.part_lse[((size_t)u * SQ + i) * H + h] = lse_v;
      else if (p.lse) p.lse[((size_t)b * SQ + i) * H + h] = lse_v;
    }
  }
  block_sync_lds();                               // 1/l ready; KV, S and P buffers free
  // o_lat (normalised, bf16) -> LDS [row][R], 16-byte chunks swizzled by row
  lds_u8_t* const olat = lds;
  if (pv_active) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int r = 16 * nt + c;
      const float inv = il[r];
#pragma unroll
      for (int j = 0; j < MTW; ++j) {
        const f32x4 v = o[j][nt] * inv;
        const int ch = 2 * (mt0 + j) + (q >> 1);
        const int pos = (ch & ~C::OSWZ) | ((ch ^ r) & C::OSWZ);
        u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *(__attribute__((address_space(3))) u32x2*)(olat + (r * (R / 8) + pos) * 16 + (q & 1) * 8) = pk;
      }
    }
  }
  block_sync_lds();
  // up-projection: wave w takes 16-row tile et = w / 2 and output dims
  // [half * DV/2, (half + 1) * DV/2), half = w % 2:
  // out^T[d][row] = sum_l W_UV^T[d][l] o_lat[row][l]
  constexpr int MDH = MD >= 2 ? MD / 2 : 1;      // output tiles per wave
  const int et = w >> 1, half = w & 1;
  if (half * MDH >= MD) return;
  const int erow = 16 * et + c;                   // block-local row of this lane
  const int erho = row_base + erow;
  const int r_first = row_base + 16 * et;
  if (r_first >= rows_total) return;
  const int r_last = min(r_first + 15, rows_total - 1);
  const int g_lo = (r_first / SQ) / HPG, g_hi = (r_last / SQ) / HPG;
  const bool evalid = erho < rows_total;
  const int myG = evalid ? (erho / SQ) / HPG : -1;
  for (int G = g_lo; G <= g_hi; ++G) {
    const uint16_t* WT = p.wuvT + (size_t)G * DV * R;
    f32x4 acc[MDH];
#pragma unroll
    for (int m = 0; m < MDH; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int kk = 0; kk < R / 32; ++kk) {
      const int ch = 4 * kk + q;
      const int pos = (ch & ~C::OSWZ) | ((ch ^ erow) & C::OSWZ);
      const bf16x8 bo = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(olat + (erow * (R / 8) + pos) * 16));
#pragma unroll
      for (int m = 0; m < MDH; ++m) {
        const int md = half * MDH + m;
        acc[m] = mfma16(ld_bf16x8(WT + (size_t)(16 * md + c) * R + 32 * kk + 8 * q), bo, acc[m]);
      }
    }
    // acc[m] lane (q, c): dims 16md + 4q .. +3 of row erow
    if (myG != G) continue;
    const int h = erho / SQ, i = erho % SQ;
    if (p.split_offsets) {
      const size_t row = ((size_t)u * SQ + i) * H + h;
#pragma unroll
      for (int m = 0; m < MDH; ++m)
        *reinterpret_cast<f32x4*>(p.part_out + row * DV + 16 * (half * MDH + m) + 4 * q) = acc[m];
    } else {
      const size_t row = ((size_t)b * SQ + i) * H + h;
#pragma unroll
      for (int m = 0; m < MDH; ++m) {
        u32x2 pk = {pack_bf16x2(acc[m][0], acc[m][1]), pack_bf16x2(acc[m][2], acc[m][3])};
        *reinterpret_cast<u32x2*>(p.out + row * DV + 16 * (half * MDH + m) + 4 * q) = pk;
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

// W_UV[G] (r x d_v) -> W_UV^T[G] (d_v x r), so the up-projection operand (8
// consecutive latent rows of one output column) is one contiguous load.
template <int R, int DV>
__global__ __launch_bounds__(256) void wuv_transpose_kernel(DecodeParams p) {
  const int G = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;     // one latent row x 8 columns
  if (idx >= R * (DV / 8)) return;
  const int l = idx / (DV / 8), d0 = (idx % (DV / 8)) * 8;
  const u32x4 v = *reinterpret_cast<const u32x4*>(p.w_uv + ((size_t)G * R + l) * DV + d0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint16_t e = (uint16_t)(v[j / 2] >> (16 * (j & 1)));
    p.wuvT[((size_t)G * DV + d0 + j) * R + l] = e;
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
  hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, DN, DV>), dim3(grid), dim3(512), 0,
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
