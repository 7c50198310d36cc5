// GQA-path decode over the per-group expanded cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "GQA path" and gist.science
// section 2 "GQA-Pfad": the latent is materialised once into g K/V groups and
// decode runs conventional grouped-query attention, h_q/g heads x s_q query
// rows per group, with the decoupled rope key shared by all groups.
//
// Work decomposition: one wave (one 64-lane workgroup) per (split unit, group).
// The wave's query rows (h_q/g heads x s_q tokens, padded to 16-row tiles)
// stay in registers; the wave streams its group's K block, dim-major V block
// and the shared rope key straight from HBM into MFMA operand registers, two
// 32-token tiles in flight, so nothing is staged through LDS.
//
//   S^T[token][row] = K[token][:] . Q[row][:]        (A = cache rows, B = Q^T)
//   O^T[dim][row]  += V^T[dim][token] . P^T[token][row]
// The token order inside a 32-token tile is relabelled so that the S^T
// accumulator lane layout is exactly the P^T B-operand layout of the PV
// product (lane group q holds tokens 8q..8q+7), and V^T is stored dim-major
// so its A operand is one contiguous 16-byte load per lane.
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

template <int HPG, int SQ, int DN, int DV, int DR>
struct GqaCfg {
  static constexpr int BS = 64;
  static constexpr int ROWS = HPG * SQ;
  static constexpr int NT = (ROWS + 15) / 16;     // 16-row tiles
  static constexpr int KSN = DN / 32;             // 32-wide k steps over d_nope
  static constexpr int KSR = (DR + 31) / 32;      // over d_rope (zero padded)
  static constexpr int MT = DV / 16;              // 16-dim output tiles
  static_assert(DN % 32 == 0 && DV % 16 == 0, "unsupported head dims");
};

template <class C>
struct GqaTile {
  bf16x8 k[2][C::KSN];
  bf16x8 r[2][C::KSR];
  bf16x8 v[C::MT];
};

template <class C, int DN, int DV, int DR>
__device__ __forceinline__ void gqa_load_tile(GqaTile<C>& T, const uint16_t* __restrict__ page,
                                              int G, int g, int slot0, int lane) {
  constexpr int BS = C::BS;
  const int c = lane & 15, q = lane >> 4;
  const uint16_t* kblk = page + (size_t)G * BS * (DN + DV);
  const uint16_t* vblk = kblk + BS * DN;
  const uint16_t* rope = page + (size_t)g * BS * (DN + DV);
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const int slot = slot0 + 8 * (c >> 2) + 4 * st + (c & 3);
#pragma unroll
    for (int ks = 0; ks < C::KSN; ++ks) T.k[st][ks] = ld_bf16x8(kblk + slot * DN + 32 * ks + 8 * q);
#pragma unroll
    for (int ks = 0; ks < C::KSR; ++ks) {
      const int dim = 32 * ks + 8 * q;
      T.r[st][ks] = (dim < DR) ? ld_bf16x8(rope + slot * DR + dim) : zero_bf16x8();
    }
  }
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) T.v[mt] = ld_bf16x8(vblk + (16 * mt + c) * BS + slot0 + 8 * q);
}

template <int HPG, int SQ, int DN, int DV, int DR>
__global__ __launch_bounds__(64) void gqa_decode_kernel(DecodeParams p) {
  using C = GqaCfg<HPG, SQ, DN, DV, DR>;
  constexpr int BS = C::BS, NT = C::NT, KSN = C::KSN, KSR = C::KSR, MT = C::MT;
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
  const int lane = threadIdx.x;
  if (p.split_offsets) {
    b = split_owner(p.split_offsets, p.batch, u);
    const int j = u - p.split_offsets[b];
    const int L = p.seqlens[b];
    lo = j * p.split_tokens;
    hi = min(lo + p.split_tokens, L);
  } else {
    b = u;
    lo = 0;
    hi = p.seqlens[b];
  }
  const int L = p.seqlens[b];
  const int c = lane & 15, q = lane >> 4;
  const size_t page_elems = (size_t)BS * (g * (DN + DV) + DR);

  // Query rows of this group as B operands (Q^T): lane (q, c) holds 8 dims of row c.
  bf16x8 qb[NT][KSN + KSR];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rho = 16 * nt + c;
    const bool valid = rho < C::ROWS;
    const int hl = valid ? rho / SQ : 0, iq = valid ? rho % SQ : 0;
    const int h = G * HPG + hl;
    const size_t qrow = ((size_t)b * SQ + iq) * H + h;
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks)
      qb[nt][ks] = valid ? ld_bf16x8(p.q_nope + qrow * DN + 32 * ks + 8 * q) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < KSR; ++ks) {
      const int dim = 32 * ks + 8 * q;
      qb[nt][KSN + ks] = (valid && dim < DR) ? ld_bf16x8(p.q_rope + qrow * DR + dim) : zero_bf16x8();
    }
  }

  f32x4 o[MT][NT];
  float m_run[NT], l_run[NT];
  int nvis[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
    const int rho = 16 * nt + c;
    nvis[nt] = L - SQ + (rho < C::ROWS ? rho % SQ : SQ - 1) + 1;
  }

  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  auto page_of = [&](int t0) -> const uint16_t* {
    return p.cache + (size_t)bt[t0 / BS] * page_elems;
  };

  auto compute = [&](GqaTile<C>& T, int t0) {
    f32x4 s[2][NT];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSN; ++ks) acc = mfma16(T.k[st][ks], qb[nt][ks], acc);
#pragma unroll
        for (int ks = 0; ks < KSR; ++ks) acc = mfma16(T.r[st][ks], qb[nt][KSN + ks], acc);
        s[st][nt] = acc;
      }
    // tokens past the end of the sequence may hold anything: keep their V at 0
    if (t0 + 32 > L) {
      const int keep = min(max(L - (t0 + 8 * q), 0), 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) T.v[mt] = keep_first(T.v[mt], keep);
    }
    bf16x8 pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 8 * q + 4 * st + i;
          const float v = s[st][nt][i] * p.scale_log2;
          x[4 * st + i] = (t < nvis[nt]) ? v : -INFINITY;
          mx = fmaxf(mx, x[4 * st + i]);
        }
      mx = wave_max_xor16_32(mx);
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run[nt] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        x[j] = exp2f(x[j] - m_use);
        ps += x[j];
      }
      l_run[nt] = l_run[nt] * alpha + ps;
      m_run[nt] = m_new;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt][nt] *= alpha;
      u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                  pack_bf16x2(x[6], x[7])};
      pb[nt] = __builtin_bit_cast(bf16x8, pk);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[mt][nt] = mfma16(T.v[mt], pb[nt], o[mt][nt]);
  };

  const int n_tiles = (hi - lo + 31) / 32;
  GqaTile<C> ta, tb;
  if (n_tiles > 0) gqa_load_tile<C, DN, DV, DR>(ta, page_of(lo), G, g, lo % BS, lane);
  for (int it = 0; it < n_tiles; it += 2) {
    const int t0 = lo + 32 * it;
    if (it + 1 < n_tiles) gqa_load_tile<C, DN, DV, DR>(tb, page_of(t0 + 32), G, g, (t0 + 32) % BS, lane);
    compute(ta, t0);
    if (it + 1 < n_tiles) {
      if (it + 2 < n_tiles) gqa_load_tile<C, DN, DV, DR>(ta, page_of(t0 + 64), G, g, (t0 + 64) % BS, lane);
      compute(tb, t0 + 32);
    }
  }

  // Epilogue: lane (q, c) holds dims 16*mt + 4q .. +3 of row 16*nt + c.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = wave_sum_xor16_32(l_run[nt]);
    const int rho = 16 * nt + c;
    if (rho >= C::ROWS) continue;
    const int hl = rho / SQ, iq = rho % SQ;
    const int h = G * HPG + hl;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m_run[nt] + log2f(lt)) * kLn2 : -INFINITY;
    if (p.split_offsets) {
      const size_t row = ((size_t)u * SQ + iq) * H + h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = o[mt][nt] * inv;
        *reinterpret_cast<f32x4*>(p.part_out + row * DV + 16 * mt + 4 * q) = v;
      }
      if (q == 0) p.part_lse[row] = lse_v;
    } else {
      const size_t row = ((size_t)b * SQ + iq) * H + h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 v = o[mt][nt] * inv;
        u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(p.out + row * DV + 16 * mt + 4 * q) = pk;
      }
      if (q == 0 && p.lse) p.lse[row] = lse_v;
    }
  }
}

// Host-side launcher: returns hipError_t of the launch.
template <int HPG, int SQ, int DN, int DV, int DR>
hipError_t launch_gqa(const DecodeParams& p, hipStream_t stream) {
  const int g = p.num_groups;
  const int rounds = (p.num_units + 7) / 8;
  const unsigned grid = (unsigned)rounds * 8u * (unsigned)g;
  hipLaunchKernelGGL((gqa_decode_kernel<HPG, SQ, DN, DV, DR>), dim3(grid), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t gqa_dispatch(int hpg, int sq, int dn, int dv, int dr, const DecodeParams& p,
                        hipStream_t stream, bool* supported) {
  *supported = true;
#define GQLA_GQA_CASE(HPG, SQ, DN, DV, DR) \
  if (hpg == HPG && sq == SQ && dn == DN && dv == DV && dr == DR) return launch_gqa<HPG, SQ, DN, DV, DR>(p, stream);
  GQLA_GQA_CASE(16, 1, 128, 128, 64)
  GQLA_GQA_CASE(16, 2, 128, 128, 64)
  GQLA_GQA_CASE(4, 1, 128, 128, 64)
  GQLA_GQA_CASE(4, 2, 128, 128, 64)
  GQLA_GQA_CASE(8, 1, 32, 32, 16)
  GQLA_GQA_CASE(8, 2, 32, 32, 16)
#undef GQLA_GQA_CASE
  *supported = false;
  return hipSuccess;
}

}  // namespace gqla
