// GQA-path decode over the per-group expanded cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "GQA path" and gist.science
// section 2 "GQA-Pfad": the latent is materialised once into g K/V groups and
// decode runs conventional grouped-query attention, h_q/g heads x s_q query
// rows per group, with the decoupled rope key shared by all groups.
//
// Work decomposition: one workgroup per (split unit, group), one wave per
// 16-row tile of the group's query rows (h_q/g heads x s_q tokens, padded),
// which stay in registers.  When the group's rows take one or two waves, the
// workgroup holds two such wave groups that take alternate tiles, each with
// its own running softmax state, merged through LDS at the end (the
// log-sum-exp merge of split-KV inside the workgroup): a CU then keeps about
// eight waves busy, with no second launch.  Each 32-token tile of the group's
// K and V blocks (both token-major) and of the shared rope key is copied
// HBM -> LDS by direct DMA (global_load_lds_dwordx4 into a ring of 4, 6 or 8
// tile buffers, no VGPR staging; the waves of a wave group share the copy
// instructions of its tiles; K and V, read once, with the non-temporal
// policy, the rope tile shared by the g group workgroups through L2 without
// it), then read as bf16 MFMA operands (the copies are waited for explicitly
// with vmcnt, see dma16):
//   S^T[token][row] = K[token][:] . Q[row][:]        (A = cache rows, B = Q^T)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// The token order inside a tile is relabelled so that the S^T accumulator lane
// layout is exactly the P^T B-operand layout of the PV product (lane group q
// holds tokens 8q..8q+7); the V^T A operand (8 tokens of one dim per lane) is
// read from the token-major V rows with ds_read_b64_tr_b16.  The LDS copies
// are XOR-swizzled in 16-byte chunks so every operand read is bank-conflict
// free.
#include <algorithm>
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {


// NB tile buffers; HV wave groups ("halves"), each of NW waves, taking the
// tiles it with it % HV == its index and keeping its own softmax state,
// merged in LDS at the end.
template <int HPG, int SQ, int DN, int DV, int DR, int NB = 4, int HV = 1>
struct GqaCfg {
  static constexpr int BS = 64;
  static constexpr int TILE = 32;
  static constexpr int NBUF = NB;                 // tile buffers
  static constexpr int PF = NBUF / HV - 1;        // rounds of HV tiles in flight ahead of the one in use
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
  static constexpr int NW = NT;                   // waves per wave group, one per 16-row tile
  static constexpr int NWT = NW * HV;             // waves per workgroup
  static constexpr int NIW = NI / NW;             // DMA instructions per wave per tile of its group
  static_assert(DN % 32 == 0 && DV % 16 == 0 && DR % 8 == 0, "unsupported head dims");
  static_assert(K_BYTES % 1024 == 0 && V_BYTES % 1024 == 0, "whole DMA instructions");
  static_assert(NI % NW == 0, "the waves share the copies evenly");
  static_assert(NWT <= 4, "launch bound of 256 threads");
  static_assert(NBUF % HV == 0 && PF >= 1, "whole rounds of tiles in the ring");
  static_assert(PF * NIW < 64, "vmcnt budget");
  static_assert(NBUF * TILE_BYTES <= 160 * 1024, "LDS budget");
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

// Row code of one entry of a sparse selection (built by sparse_codes_kernel):
// bits 0..27 the cache row page * 64 + slot of the listed token, bits 28..30
// the first query row index that may see it (0 .. s_q - 1), or 7 for an entry
// no row sees (outside [0, L), or padding), whose row is then 0.
constexpr uint32_t kRowMask = (1u << 28) - 1;
constexpr uint32_t kInvalidEntry = 7u << 28;

// The 32 row codes of tile `it` of a sparse unit, read through the scalar
// path (constant address space, wave-uniform address): the vector-memory
// counter stays reserved for the tile copies.
struct TileCodes {
  uint32_t v[32];
};
// Lane e (< 32) of the result holds v[e]; lanes 32..63 hold 0.  One
// v_writelane_b32 per entry (a register-only VALU op with an immediate lane
// select; this compiler has no builtin for it).
__device__ __forceinline__ uint32_t spread_codes(const TileCodes& t) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(r) : "s"(t.v[e]), "i"(e));
  return r;
}
__device__ __forceinline__ TileCodes load_codes(const uint32_t* unit_codes, int it) {
  const __attribute__((address_space(4))) uint32_t* cs =
      (const __attribute__((address_space(4))) uint32_t*)(unit_codes + 32 * it);
  TileCodes t;
#pragma unroll
  for (int e = 0; e < 32; ++e) t.v[e] = cs[e];
  return t;
}

// Direct HBM -> LDS copy of 16 bytes per lane from a per-lane 64-bit address
// (the gather form of dma16; same waiting rules); NT: non-temporal policy,
// as dma16_nt.
template <bool NT>
__device__ __forceinline__ void dma16_gather(const void* addr, lds_u8_t* lds_base) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(addr), "s"(m0v) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(addr), "s"(m0v) : "memory", "m0");
}

// SPARSE = false: dense decode of a sequence or split.  SPARSE = true: the
// unit is (sequence, group) and its tiles are 32 consecutive entries of the
// group's row codes (sparse GQLA: gist.science section 2, subsection "Sparse
// GQLA"; every query row of the group shares the selection, so the group's
// rows stay one dense MFMA tile).  Entries are gathered row by row into the
// same LDS tile layout, so the tile step is the same apart from its masks.
// Wait until at most `ahead` tiles of NIW copies each are still in flight
// (ahead in 0 .. MAXA, wave-uniform).
template <int NIW, int MAXA>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      vm_wait<MAXA * NIW>();
      return;
    }
    wait_tiles_ahead<NIW, MAXA - 1>(ahead);
  } else {
    vm_wait<0>();
  }
}

// NB: tile buffers (NB - 1 tiles in flight ahead of the one in use).  Four
// when two workgroups share a CU; more when a launch has one workgroup per CU,
// so that a CU keeps about as many bytes in flight either way.
template <int HPG, int SQ, int DN, int DV, int DR, bool SPARSE, int NB, int HV>
__global__ __launch_bounds__(256) void gqa_decode_kernel(DecodeParams p) {
  using C = GqaCfg<HPG, SQ, DN, DV, DR, NB, HV>;
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
  const int wid = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int w = wid % NW;                         // this wave's 16-row tile
  const int hv = wid / NW;                        // its wave group: tiles it with it % HV == hv
  if constexpr (SPARSE) {                         // units: (sequence, entry range) x group
    if (p.split_offsets) {
      b = unit_owner(p.split_offsets, p.seqlens, p.batch, u).b;
      lo = (u - p.split_offsets[b]) * p.split_tokens;
      hi = min(lo + p.split_tokens, p.topk_pad);
    } else {
      b = u;
      lo = 0;
      hi = p.topk_pad;
    }
    if (p.seqlens[b] <= 0) hi = lo;               // no entry is visible in an empty sequence
  } else if (p.split_offsets) {
    const UnitOwner own = unit_owner(p.split_offsets, p.seqlens, p.batch, u);
    b = own.b;
    lo = (u - own.first) * p.split_tokens;
    hi = min(lo + p.split_tokens, own.len);
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
  const uint32_t* unit_codes = SPARSE ? p.codes + ((size_t)b * g + G) * p.topk_pad + lo : nullptr;
  uint32_t edge_bits = 0;                         // sparse: tiles in the ring that need masks
  uint32_t code_ring[C::NBUF];                    // sparse: lane e < 32 holds entry e's code, per buffer
#pragma unroll
  for (int r = 0; r < C::NBUF; ++r) code_ring[r] = 0;

  // ---- DMA of tile `it` into `dst` (the buffer of tile it % NBUF) ----
  auto issue_tile = [&](int it, const TileCodes& tc) {
    lds_u8_t* dst = lds + (it % C::NBUF) * C::TILE_BYTES;
    if constexpr (SPARSE) {
      // lanes 0..31 hold the cache rows of the tile's entries; each copy lane
      // fetches the row of its entry with a cross-lane read
      const uint32_t cv = spread_codes(tc);
      const uint32_t rows = cv & kRowMask;
      uint32_t any = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) any |= tc.v[e];
      const int slot = it % C::NBUF;
#pragma unroll
      for (int r = 0; r < C::NBUF; ++r) code_ring[r] = r == slot ? cv : code_ring[r];
      const int bit = 1 << slot;
      edge_bits = (any >> 28) ? (edge_bits | bit) : (edge_bits & ~bit);
      // Wave w issues copies w, w + NW, ... of the tile (the same ones as in
      // the dense case); each region (K, V, rope) holds a multiple of NW
      // copies, so copy k of this wave lies in a region known at compile
      // time.  First every copy lane's entry row (cross-lane reads, one wait),
      // then the copies.
      static_assert(C::NI_K % NW == 0 && C::NI_V % NW == 0 && C::NI_R % NW == 0, "copies per region");
      constexpr int KW = C::NI_K / NW, VW = C::NI_V / NW;
      auto entry_of = [&](int k) {                // tile entry copied by this lane in copy k, and its chunk
        int P, chunks;
        if (k < KW) {
          P = (k * NW + w) * 64 + lane;
          chunks = KCH;
        } else if (k < KW + VW) {
          P = ((k - KW) * NW + w) * 64 + lane;
          chunks = VCH;
        } else {
          P = min(((k - KW - VW) * NW + w) * 64 + lane, C::TILE * RCH - 1);   // partial last copy: duplicate
          chunks = RCH;
        }
        return int2{P / chunks, P % chunks};
      };
      uint32_t r[C::NIW];
#pragma unroll
      for (int k = 0; k < C::NIW; ++k) r[k] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * entry_of(k).x, (int)rows);
#pragma unroll
      for (int k = 0; k < C::NIW; ++k) {
        const int2 tp = entry_of(k);
        const int t = tp.x, pos = tp.y;
        const uint16_t* page = p.cache + (size_t)(r[k] >> 6) * page_elems;
        const int slot = (int)(r[k] & 63u);
        if (k < KW) {                              // K rows: token-major, chunk swizzled
          const int ch = pos ^ (kswz(t) & (KCH - 1));
          dma16_gather<true>(page + (size_t)G * BS * (DN + DV) + slot * DN + ch * 8, dst + (k * NW + w) * 1024);
        } else if (k < KW + VW) {                  // V rows
          const int ch = pos ^ vswz<DV>(t);
          dma16_gather<true>(page + (size_t)G * BS * (DN + DV) + BS * DN + slot * DV + ch * 8,
                             dst + C::K_BYTES + ((k - KW) * NW + w) * 1024);
        } else {                                   // rope rows
          const int ch = pos ^ (rswz(t) & (RCH - 1));
          dma16_gather<false>(page + (size_t)g * BS * (DN + DV) + slot * DR + ch * 8,
                              dst + C::K_BYTES + C::V_BYTES + ((k - KW - VW) * NW + w) * 1024);
        }
      }
    } else {
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
        dma16_nt(kblk, (uint32_t)(t * DN + ch * 8) * 2u, dst + i * 1024);
      }
#pragma unroll
      for (int i = 0; i < C::NI_V; ++i) {        // V rows: token-major, chunk swizzled
        if ((C::NI_K + i) % NW != w) continue;
        const int P = i * 64 + lane, t = P / VCH, pos = P % VCH;
        const int ch = pos ^ vswz<DV>(t);
        dma16_nt(vblk, (uint32_t)(t * DV + ch * 8) * 2u, dst + C::K_BYTES + i * 1024);
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
    }
  };
  auto codes_of = [&](int it) {
    if constexpr (SPARSE) return load_codes(unit_codes, it);
    else return TileCodes{};
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
  constexpr int PF = C::PF;
  // this group's tiles: it = HV j + hv, j < n_my; round k holds tiles HV k .. HV k + HV - 1
  const int n_my = n_tiles > hv ? (n_tiles - hv + HV - 1) / HV : 0;
  const int n_rounds = (n_tiles + HV - 1) / HV;
  for (int j = 0; j < PF && j < n_my; ++j) issue_tile(HV * j + hv, codes_of(HV * j + hv));

  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int nvis = L - SQ + (rvalid ? rho % SQ : SQ - 1) + 1;   // tokens t < nvis are visible
  const int iq_row = rvalid ? rho % SQ : SQ - 1;  // this lane's query row index

  // One tile: S^T, the online softmax, O^T += V^T P^T.  EDGE: the tile
  // reaches the causal bound or the sequence end, so logits are masked and
  // the V rows of tokens past the end (which may hold anything) are zeroed.
  auto tile_step = [&](const lds_u8_t* buf, int t0, auto edge) {
    constexpr bool EDGE = decltype(edge)::value;
    // sparse edge tiles: the codes of this lane's 8 entries 8q .. 8q+7
    uint32_t ecode[8];
    if constexpr (SPARSE && EDGE) {
      const int slot = ((t0 - lo) / C::TILE) % C::NBUF;
      uint32_t cv = 0;
#pragma unroll
      for (int r = 0; r < C::NBUF; ++r) cv = r == slot ? code_ring[r] : cv;
#pragma unroll
      for (int j = 0; j < 8; ++j) ecode[j] = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (8 * q + j), (int)cv);
    }
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
        if constexpr (EDGE && SPARSE) v = ((int)(ecode[4 * st + i] >> 28) <= iq_row) ? v : -INFINITY;
        else if constexpr (EDGE) v = (t0 + 8 * q + 4 * st + i < nvis) ? v : -INFINITY;
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
    const int keep = (EDGE && !SPARSE) ? min(max(L - (t0 + 8 * q), 0), 8) : 8;
    // sparse: V elements of entries no row sees are zeroed (their rows may hold anything)
    u32x4 vkeep = {~0u, ~0u, ~0u, ~0u};
    if constexpr (EDGE && SPARSE) {
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2)
        vkeep[w2] = (ecode[2 * w2] >= kInvalidEntry ? 0u : 0x0000ffffu) |
                    (ecode[2 * w2 + 1] >= kInvalidEntry ? 0u : 0xffff0000u);
    }
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
      if constexpr (EDGE && SPARSE) v = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, v) & vkeep);
      else if constexpr (EDGE) v = keep_first(v, keep);
      o[mt] = mfma16(v, pb, o[mt]);
    }
  };

  for (int k = 0; k < n_rounds; ++k) {
    const int it = HV * k + hv;                   // this group's tile of round k (none past the end)
    const int itn = HV * (k + PF) + hv;           // its tile whose copies this round issues
    // sparse: the row codes of tile itn, read before the wait so their
    // latency overlaps it (clamped to a real tile; unused past the end)
    const TileCodes nxt = codes_of(min(itn, n_tiles - 1));
    // this wave's copies of tile it landed (those of its next PF - 1 tiles
    // may be in flight); after the barrier every wave's copies of round k
    // landed and every wave is done with round k - 1, whose buffers take
    // round k + PF
    wait_tiles_ahead<C::NIW, PF - 1>(max(0, min(PF - 1, n_my - 1 - k)));   // later tiles in flight
    if constexpr (C::NWT > 1) __syncthreads();
    if (itn < n_tiles) issue_tile(itn, nxt);
    if (it < n_tiles) {
      const lds_u8_t* buf = lds + (it % C::NBUF) * C::TILE_BYTES;
      const int t0 = lo + C::TILE * it;
      // only tiles that reach the first causal bound (L - s_q + 1), the last
      // one or two of the sequence, mask logits and V rows; sparse tiles do
      // when an entry is invalid or visible to later query rows only
      const bool edge = SPARSE ? ((edge_bits >> (it % C::NBUF)) & 1) != 0 : (t0 + C::TILE > L - SQ + 1);
      if (edge) tile_step(buf, t0, std::true_type{});
      else tile_step(buf, t0, std::false_type{});
    }
  }

  // The wave groups' states of the same rows meet in LDS (over the tile
  // ring): group 0 merges them by their row maxima, as the split merge does.
  if constexpr (HV > 1) {
    constexpr int NF = 4 * MT + 2;                // floats per lane: o, m_run, l_run
    __syncthreads();                              // every tile read
    typedef __attribute__((address_space(3))) float lds_f32_t;
    lds_f32_t* const xs = (lds_f32_t*)lds;        // [group - 1][wave][field][lane]
    if (hv > 0) {
      lds_f32_t* dst = xs + ((hv - 1) * NW + w) * NF * 64 + lane;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(4 * mt + i) * 64] = o[mt][i];
      dst[(4 * MT) * 64] = m_run;
      dst[(4 * MT + 1) * 64] = l_run;
    }
    __syncthreads();
    if (hv > 0) return;
#pragma unroll
    for (int h2 = 1; h2 < HV; ++h2) {
      const lds_f32_t* src = xs + ((h2 - 1) * NW + w) * NF * 64 + lane;
      const float m2 = src[(4 * MT) * 64];
      const float mn = fmaxf(m_run, m2);
      if (mn == -INFINITY) continue;              // neither state saw a token of these rows
      const float a = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
      const float b2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
      l_run = l_run * a + src[(4 * MT + 1) * 64] * b2;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[mt][i] = o[mt][i] * a + src[(4 * mt + i) * 64] * b2;
      m_run = mn;
    }
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

hipError_t cu_count(int* n);   // compute units of the current device (expand.hip)

// Host-side launcher: returns hipError_t of the launch.
template <int HPG, int SQ, int DN, int DV, int DR, bool SPARSE>
hipError_t launch_gqa(const DecodeParams& p, hipStream_t stream) {
  const int g = p.num_groups;
  const int rounds = (p.num_units + 7) / 8;
  const unsigned grid = (unsigned)rounds * 8u * (unsigned)g;
  using C4 = GqaCfg<HPG, SQ, DN, DV, DR, 4, 1>;
  constexpr int NW = C4::NW;
  int cus = 0;
  const hipError_t e = cu_count(&cus);
  if (e != hipSuccess) return e;
  // Two wave groups over alternate tiles per workgroup when the row tiles
  // take at most two waves, so that a CU runs about eight waves:
  //   * at most one workgroup per CU: one-wave row tiles in an eight-buffer
  //     ring (three rounds in flight), two-wave row tiles in a six-buffer ring;
  //   * more: a four-buffer ring (one round in flight), two workgroups per CU.
  if constexpr (NW <= 2 && 2 * C4::NIW < 64) {
    if (grid <= (unsigned)cus) {
      if constexpr (NW == 1 && 8 * C4::TILE_BYTES <= 160 * 1024 && 3 * C4::NIW < 64) {
        hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR, SPARSE, 8, 2>), dim3(grid), dim3(128), 0, stream,
                           p);
        return hipGetLastError();
      } else if constexpr (6 * C4::TILE_BYTES <= 160 * 1024) {
        hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR, SPARSE, 6, 2>), dim3(grid), dim3(128 * NW), 0,
                           stream, p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR, SPARSE, 4, 2>), dim3(grid), dim3(128 * NW), 0, stream,
                       p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR, SPARSE, 4, 1>), dim3(grid), dim3(64 * NW), 0, stream,
                     p);
  return hipGetLastError();
}

hipError_t gqa_dispatch(int hpg, int sq, int dn, int dv, int dr, const DecodeParams& p,
                        hipStream_t stream, bool* supported) {
  *supported = true;
  const bool sparse = p.codes != nullptr;
#define GQLA_GQA_CASE(HPG, SQ, DN, DV, DR)                                            \
  if (hpg == HPG && sq == SQ && dn == DN && dv == DV && dr == DR)                     \
    return sparse ? launch_gqa<HPG, SQ, DN, DV, DR, true>(p, stream)                  \
                  : launch_gqa<HPG, SQ, DN, DV, DR, false>(p, stream);
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

// Row codes of a sparse selection: one thread per (sequence, group, entry)
// of the padded lists (the format is described with kRowMask above).
__global__ __launch_bounds__(256) void sparse_codes_kernel(SparseCodeParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_seq = (int64_t)p.num_groups * p.topk_pad;
  if (p.split_offsets && i <= p.batch) p.split_offsets[i] = (int32_t)(i * p.splits_per_seq);
  if (i >= (int64_t)p.batch * per_seq) return;
  const int b = (int)(i / per_seq);
  const int G = (int)((i % per_seq) / p.topk_pad);
  const int e = (int)(i % p.topk_pad);
  uint32_t code = kInvalidEntry;
  if (e < p.topk) {
    const int t = p.indices[((int64_t)b * p.num_groups + G) * p.topk + e];
    const int L = p.seqlens[b];
    if (t >= 0 && t < L && t / p.block_size < p.max_blocks) {
      const int32_t page = p.block_table[(int64_t)b * p.max_blocks + t / p.block_size];
      if (page >= 0 && page < p.num_pages)
        code = ((uint32_t)page * (uint32_t)p.block_size + (uint32_t)(t % p.block_size)) |
               ((uint32_t)max(t - (L - p.s_q), 0) << 28);
    }
  }
  p.codes[i] = code;
}

hipError_t sparse_codes_launch(const SparseCodeParams& p, hipStream_t stream) {
  const int64_t n = std::max<int64_t>((int64_t)p.batch * p.num_groups * p.topk_pad, (int64_t)p.batch + 1);
  hipLaunchKernelGGL(sparse_codes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqla
