// GQA-path decode over the per-group expanded cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "GQA path" and gist.science
// section 2 "GQA-Pfad": the latent is materialised once into g K/V groups and
// decode runs conventional grouped-query attention, h_q/g heads x s_q query
// rows per group, with the decoupled rope key shared by all groups.
//
// Work decomposition: one workgroup per (split unit, group), one wave per
// 16-row tile of the group's query rows (h_q/g heads x s_q tokens, padded),
// which stay in registers.  Each 32-token tile of the group's K and V blocks
// (both token-major) and of the shared rope key is copied HBM -> LDS by direct
// DMA (global_load_lds_dwordx4, three tiles ahead, no VGPR staging; the waves
// share the copy instructions and the tile), then read as bf16 MFMA operands
// (the copies are waited for explicitly with vmcnt, see dma16):
//   S^T[token][row] = K[token][:] . Q[row][:]        (A = cache rows, B = Q^T)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// The token order inside a tile is relabelled so that the S^T accumulator lane
// layout is exactly the P^T B-operand layout of the PV product (lane group q
// holds tokens 8q..8q+7); the V^T A operand (8 tokens of one dim per lane) is
// read from the token-major V rows with ds_read_b64_tr_b16.  The LDS copies
// are XOR-swizzled in 16-byte chunks so every operand read is bank-conflict
// free.
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {


template <int HPG, int SQ, int DN, int DV, int DR>
struct GqaCfg {
  static constexpr int BS = 64;
  static constexpr int TILE = 32;
  static constexpr int NBUF = 4;                  // tile buffers
  static constexpr int LA = NBUF - 1;             // tiles in flight ahead of the one in use
  static constexpr int ROWS = HPG * SQ;
  static constexpr int NT = (ROWS + 15) / 16;     // 16-row tiles
  static constexpr int KSN = DN / 32;             // 32-wide k steps over d_nope
  static constexpr int KSR = (DR + 31) / 32;      // over d_rope (zero padded)
  static constexpr int MT = DV / 16;              // 16-dim output tiles
  static constexpr int KCH = DN / 8;              // 16-byte chunks per K row
  static constexpr int RCH = DR / 8;              // 16-byte chunks per rope row
  static constexpr int VCH = DV / 8;              // 16-byte chunks per V row
  static constexpr int K_BYTES = TILE * DN * 2;
  static constexpr int V_BYTES = DV * TILE * 2;
  static constexpr int R_BYTES = TILE * DR * 2;
  static constexpr int TILE_BYTES = K_BYTES + V_BYTES + R_BYTES;
  static constexpr int NI_K = K_BYTES / 1024, NI_V = V_BYTES / 1024;
  static constexpr int NI_R = (R_BYTES + 1023) / 1024;
  static constexpr int NI = NI_K + NI_V + NI_R;   // DMA instructions per tile
  static constexpr int NW = NT;                   // waves per workgroup, one per 16-row tile
  static constexpr int NIW = NI / NW;             // DMA instructions per wave per tile
  static_assert(DN % 32 == 0 && DV % 16 == 0 && DR % 8 == 0, "unsupported head dims");
  static_assert(K_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "whole DMA instructions");
  static_assert(NI % NW == 0, "the waves share the copies evenly");
  static_assert(NW <= 4, "launch bound of 256 threads");
  static_assert(LA * NIW < 64, "vmcnt budget");
  static_assert(LA <= 3, "the in-flight wait covers up to two later tiles");
  static_assert((KCH & (KCH - 1)) == 0 && (RCH & (RCH - 1)) == 0, "power-of-two rows");
  static_assert(DV == 32 || DV == 64 || DV == 128, "V rows of 64, 128 or 256 bytes");
};

// Token swizzles (tile-local token t in 0..31).  The QK reads touch 16 tokens
// {8a + 4st + b} (a, b in 0..3) at one chunk: kswz is distinct over them.
__device__ __forceinline__ int kswz(int t) { return (t & 3) | ((t >> 3) << 2); }
__device__ __forceinline__ int rswz(int t) { return ((t >> 1) & 1) | ((t >> 3) << 1); }
// V rows (token-major, DV dims): a transposing 8-byte read is served in two
// passes of 32 lanes over 64 four-byte banks.  One pass of a PV read touches
// tokens 8q + 4h + r (q of one parity, r in 0..3) at the chunk pair of its
// 16-dim output tile.  128 / DV rows share a bank period, which separates the
// low bits of r; the remaining bits of r and the parity of q select the chunk
// pair, so every pass hits 64 distinct banks.  The swizzle is even: a pair
// of chunks stays adjacent.
template <int DV>
__device__ __forceinline__ int vswz(int t) {
  constexpr int LRP = DV == 128 ? 0 : (DV == 64 ? 1 : 2);   // log2 rows per bank period
  return 2 * (((t & 3) >> LRP) | (((t >> 3) & 1) << (2 - LRP)));
}

template <int HPG, int SQ, int DN, int DV, int DR>
__global__ __launch_bounds__(256) void gqa_decode_kernel(DecodeParams p) {
  using C = GqaCfg<HPG, SQ, DN, DV, DR>;
  constexpr int BS = C::BS, NW = C::NW, KSN = C::KSN, KSR = C::KSR, MT = C::MT;
  constexpr int KCH = C::KCH, RCH = C::RCH, VCH = C::VCH;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::NBUF * C::TILE_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;

  const int g = p.num_groups;
  const int H = HPG * g;
  // Workgroups are dispatched round-robin over the 8 XCDs; give the g groups
  // of one split unit consecutive slots on the same XCD so the shared rope
  // key is fetched from HBM once and re-read from that XCD's L2.
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int u = (k / g) * 8 + xcd;
  const int G = k % g;
  if (u >= p.num_units) return;

  int b, lo, hi;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // this wave's 16-row tile
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
  const int L = p.seqlens[b];
  const int c = lane & 15, q = lane >> 4;
  const size_t page_elems = (size_t)BS * (g * (DN + DV) + DR);
  const int n_tiles = hi > lo ? (hi - lo + C::TILE - 1) / C::TILE : 0;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;     // wave-uniform

  // ---- DMA of tile `it` into `dst` (the buffer of tile it % NBUF) ----
  auto issue_tile = [&](int it) {
    lds_u8_t* dst = lds + (it % C::NBUF) * C::TILE_BYTES;
    const int t0 = lo + C::TILE * it;
    const uint16_t* page = p.cache + (size_t)sload_i32(bt + t0 / BS) * page_elems;
    const int slot0 = t0 % BS;
    const uint16_t* kblk = page + (size_t)G * BS * (DN + DV) + slot0 * DN;
    const uint16_t* vblk = page + (size_t)G * BS * (DN + DV) + BS * DN + slot0 * DV;
    const uint16_t* rope = page + (size_t)g * BS * (DN + DV) + slot0 * DR;
    // copy instruction j of the tile (K, then V, then rope) is issued by
    // wave j % NW
#pragma unroll
    for (int i = 0; i < C::NI_K; ++i) {        // K rows: token-major, chunk swizzled
      if (i % NW != w) continue;
      const int P = i * 64 + lane, t = P / KCH, pos = P % KCH;
      const int ch = pos ^ (kswz(t) & (KCH - 1));
      dma16(kblk, (uint32_t)(t * DN + ch * 8) * 2u, dst + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::NI_V; ++i) {        // V rows: token-major, chunk swizzled
      if ((C::NI_K + i) % NW != w) continue;
      const int P = i * 64 + lane, t = P / VCH, pos = P % VCH;
      const int ch = pos ^ vswz<DV>(t);
      dma16(vblk, (uint32_t)(t * DV + ch * 8) * 2u, dst + C::K_BYTES + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < C::NI_R; ++i) {        // rope rows: token-major, chunk swizzled
      if ((C::NI_K + C::NI_V + i) % NW != w) continue;
      int P = i * 64 + lane;
      if (P >= C::TILE * RCH) P = C::TILE * RCH - 1;   // partial last instruction: duplicate
      const int t = P / RCH, pos = P % RCH;
      const int ch = pos ^ (rswz(t) & (RCH - 1));
      dma16(rope, (uint32_t)(t * DR + ch * 8) * 2u, dst + C::K_BYTES + C::V_BYTES + i * 1024);
    }
  };

  // Query rows of this wave's tile as B operands (Q^T): lane (q, c) holds 8
  // dims of row 16 w + c.
  const int rho = 16 * w + c;
  const bool rvalid = rho < C::ROWS;
  bf16x8 qb[KSN + KSR];
  {
    const int hl = rvalid ? rho / SQ : 0, iq = rvalid ? rho % SQ : 0;
    const size_t qrow = ((size_t)b * SQ + iq) * H + G * HPG + hl;
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks)
      qb[ks] = rvalid ? ld_bf16x8(p.q_nope + qrow * DN + 32 * ks + 8 * q) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < KSR; ++ks) {
      const int dim = 32 * ks + 8 * q;
      qb[KSN + ks] = (rvalid && dim < DR) ? ld_bf16x8(p.q_rope + qrow * DR + dim) : zero_bf16x8();
    }
  }

  // The query loads complete before the first tile copy is issued, so the
  // compiler's own wait tracking has nothing pending inside the tile loop.
  vm_wait<0>();
  for (int i = 0; i < C::LA && i < n_tiles; ++i) issue_tile(i);

  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int nvis = L - SQ + (rvalid ? rho % SQ : SQ - 1) + 1;   // tokens t < nvis are visible

  // One tile: S^T, the online softmax, O^T += V^T P^T.  EDGE: the tile
  // reaches the causal bound or the sequence end, so logits are masked and
  // the V rows of tokens past the end (which may hold anything) are zeroed.
  auto tile_step = [&](const lds_u8_t* buf, int t0, auto edge) {
    constexpr bool EDGE = decltype(edge)::value;
    f32x4 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int t = 8 * (c >> 2) + 4 * st + (c & 3);     // token held by MFMA row c
      s[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSN; ++ks) {
        const int pos = (4 * ks + q) ^ (kswz(t) & (KCH - 1));
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + (t * KCH + pos) * 16));
        s[st] = mfma16(a, qb[ks], s[st]);
      }
#pragma unroll
      for (int ks = 0; ks < KSR; ++ks) {
        const int ch = 4 * ks + q;
        bf16x8 a = zero_bf16x8();
        if (8 * ch < DR) {
          const int pos = ch ^ (rswz(t) & (RCH - 1));
          a = __builtin_bit_cast(bf16x8, *(const lds_u32x4_t*)(buf + C::K_BYTES + C::V_BYTES + (t * RCH + pos) * 16));
        }
        s[st] = mfma16(a, qb[KSN + ks], s[st]);
      }
    }
    // Online softmax (base 2) with a lazily moved reference max: the
    // accumulators are rescaled only when the row's max exceeds its reference
    // by more than 8 (so every p <= 2^8), which is rare after the first tile.
    float x[8], mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[st][i] * p.scale_log2;
        if constexpr (EDGE) v = (t0 + 8 * q + 4 * st + i < nvis) ? v : -INFINITY;
        x[4 * st + i] = v;
        mx = fmaxf(mx, v);
      }
    mx = wave_max_q(mx);
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
    }
    bf16x8 pb;
    {
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
        ps += x[j];
      }
      l_run += ps;
      u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      pb = __builtin_bit_cast(bf16x8, pk);
    }
    const int keep = EDGE ? min(max(L - (t0 + 8 * q), 0), 8) : 8;
    // transposing reads: source lane (q, c) of read h addresses dims
    // 16 mt + 4 (c & 3) .. +3 of token 8 q + 4 h + c / 4, so lane (q, c)
    // receives dim 16 mt + c of tokens 8 q + 4 h .. +3
    const int tv0 = 8 * q + (c >> 2), tv1 = tv0 + 4;
    const lds_u8_t* vr0 = buf + C::K_BYTES + tv0 * (DV * 2) + 8 * (c & 1);
    const lds_u8_t* vr1 = buf + C::K_BYTES + tv1 * (DV * 2) + 8 * (c & 1);
    const int sw0 = vswz<DV>(tv0), sw1 = vswz<DV>(tv1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int lch = 2 * mt + ((c >> 1) & 1);          // logical 16-byte chunk
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr0 + (lch ^ sw0) * 16));
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vr1 + (lch ^ sw1) * 16));
      bf16x8 v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      if constexpr (EDGE) v = keep_first(v, keep);
      o[mt] = mfma16(v, pb, o[mt]);
    }
  };

  for (int it = 0; it < n_tiles; ++it) {
    // this wave's copies of tile it landed (those of the next LA-1 tiles may
    // be in flight); after the barrier every wave's copies of tile it landed
    // and every wave is done with tile it-1, whose buffer takes tile it+LA
    const int ahead = min(C::LA - 1, n_tiles - 1 - it);     // later tiles in flight
    if (ahead == 2) vm_wait<2 * C::NIW>();
    else if (ahead == 1) vm_wait<C::NIW>();
    else vm_wait<0>();
    if constexpr (NW > 1) __syncthreads();
    if (it + C::LA < n_tiles) issue_tile(it + C::LA);
    const lds_u8_t* buf = lds + (it % C::NBUF) * C::TILE_BYTES;
    const int t0 = lo + C::TILE * it;
    // only tiles that reach the first causal bound (L - s_q + 1), the last
    // one or two of the sequence, mask logits and V rows
    if (t0 + C::TILE > L - SQ + 1) tile_step(buf, t0, std::true_type{});
    else tile_step(buf, t0, std::false_type{});
  }

  // Epilogue: lane (q, c) holds dims 16*mt + 4q .. +3 of row 16 w + c.
  const float lt = wave_sum_q(l_run);
  if (!rvalid) return;
  const int hl = rho / SQ, iq = rho % SQ;
  const int h = G * HPG + hl;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  if (p.split_offsets) {
    const size_t row = ((size_t)u * SQ + iq) * H + h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 v = o[mt] * inv;
      *reinterpret_cast<f32x4*>(p.part_out + row * DV + 16 * mt + 4 * q) = v;
    }
    if (q == 0) p.part_lse[row] = lse_v;
  } else {
    const size_t row = ((size_t)b * SQ + iq) * H + h;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const f32x4 v = o[mt] * inv;
      u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      *reinterpret_cast<u32x2*>(p.out + row * DV + 16 * mt + 4 * q) = pk;
    }
    if (q == 0 && p.lse) p.lse[row] = lse_v;
  }
}

// Host-side launcher: returns hipError_t of the launch.
template <int HPG, int SQ, int DN, int DV, int DR>
hipError_t launch_gqa(const DecodeParams& p, hipStream_t stream) {
  const int g = p.num_groups;
  const int rounds = (p.num_units + 7) / 8;
  const unsigned grid = (unsigned)rounds * 8u * (unsigned)g;
  hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR>), dim3(grid), dim3(64 * GqaCfg<HPG, SQ, DN, DV, DR>::NW), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t gqa_dispatch(int hpg, int sq, int dn, int dv, int dr, const DecodeParams& p,
                        hipStream_t stream, bool* supported) {
  *supported = true;
#define GQLA_GQA_CASE(HPG, SQ, DN, DV, DR) \
  if (hpg == HPG && sq == SQ && dn == DN && dv == DV && dr == DR) return launch_gqa<HPG, SQ, DN, DV, DR>(p, stream);
  GQLA_GQA_CASE(16, 1, 128, 128, 64)
  GQLA_GQA_CASE(16, 2, 128, 128, 64)
  GQLA_GQA_CASE(32, 1, 128, 128, 64)
  GQLA_GQA_CASE(32, 2, 128, 128, 64)
  GQLA_GQA_CASE(4, 1, 128, 128, 64)
  GQLA_GQA_CASE(4, 2, 128, 128, 64)
  GQLA_GQA_CASE(8, 1, 32, 32, 16)
  GQLA_GQA_CASE(8, 2, 32, 32, 16)
#undef GQLA_GQA_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace gqla
