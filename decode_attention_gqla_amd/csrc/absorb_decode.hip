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
// One workgroup = 4 waves x 32 query rows (all 128 heads of a DeepSeek-V3
// shaped sequence at s_q = 1) for one split of one sequence, so every cache
// byte is fetched from HBM once.  32-token latent tiles are copied
// HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging), three buffers
// deep, into a XOR-swizzled token-major layout; waves then read
//   - QK operands with ds_read_b128 (8 latent dims of one token per lane),
//   - PV operands with ds_read_b64_tr_b16 (8 tokens of one latent dim per
//     lane, transposed by the LDS unit),
// and run bf16 MFMA 16x16x32 with fp32 accumulation:
//   S^T[token][row] = C_tile . [q_abs | q_rope]^T,   O^T[latent][row] += C_tile^T . P^T.
// Prologue: q_abs = W_UK[G] q_nope on MFMA, laid out directly as the QK B
// operand.  Epilogue: out^T = W_UV[G]^T o_lat^T on MFMA, W_UV staged per wave
// in LDS and read transposed.
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vm_dyn(int n) {
  switch (n) {
#define GQLA_WV(N) case N: wait_vm<N>(); break;
    GQLA_WV(0) GQLA_WV(1) GQLA_WV(2) GQLA_WV(3) GQLA_WV(4) GQLA_WV(5) GQLA_WV(6) GQLA_WV(7)
    GQLA_WV(8) GQLA_WV(9) GQLA_WV(10) GQLA_WV(11) GQLA_WV(12) GQLA_WV(13) GQLA_WV(14) GQLA_WV(15)
    GQLA_WV(16) GQLA_WV(17) GQLA_WV(18) GQLA_WV(19) GQLA_WV(20) GQLA_WV(21) GQLA_WV(22) GQLA_WV(23)
#undef GQLA_WV
    default: wait_vm<0>(); break;
  }
}

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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
  static constexpr int KSL = R / 32;              // k steps over the latent
  static constexpr int KSR = (DR + 31) / 32;      // k steps over the rope key (zero padded)
  static constexpr int KS = KSL + KSR;
  static constexpr int KD = DN / 32;              // k steps of the absorption product
  static constexpr int MTL = R / 16;              // 16-dim tiles of o_lat
  static constexpr int MD = DV / 16;              // 16-dim tiles of the output
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int ROWS_WG = NW * 32;
  static constexpr int WCH = 64;                  // W_UV rows staged per wave per step
  static constexpr int WSTRIDE = DV + 16;         // padded staged row (elements)
  static constexpr int WSTAGE_BYTES = WCH * WSTRIDE * 2;
  static constexpr int LDS_BYTES = NBUF * BUF_BYTES > NW * WSTAGE_BYTES ? NBUF * BUF_BYTES
                                                                        : NW * WSTAGE_BYTES;
  static_assert((TILE * CHR) % 64 == 0, "tile must be whole DMA instructions");
  static_assert(R % 32 == 0 && DN % 32 == 0 && DV % 16 == 0, "unsupported dims");
  static_assert(NI <= 4 * 11, "vmcnt budget");
};

// Swizzle of 16-byte chunk positions inside a token row (tokens 0..31 of a
// tile): conflict-free for both the QK reads (16 tokens, one chunk) and the
// transposed PV reads (4 tokens x 2 chunks per 16-lane group).
__device__ __forceinline__ int tile_swz(int t) { return 4 * ((t >> 1) & 1) + (t >> 3); }

template <int HPG, int SQ, int R, int DR, int DN, int DV>
__global__ __launch_bounds__(256, 1) void absorb_decode_kernel(DecodeParams p) {
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  constexpr int BS = C::BS, ROW = C::ROW, CHR = C::CHR, KSL = C::KSL, KSR = C::KSR, KS = C::KS;
  constexpr int KD = C::KD, MTL = C::MTL, MD = C::MD;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];

  const int g = p.num_groups;
  const int H = HPG * g;
  const int rows_total = H * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int u = (k / RB) * 8 + xcd;
  const int rb = k % RB;
  if (u >= p.num_units) return;                   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int L = p.seqlens[b];
  const int n_tiles = hi > lo ? (hi - lo + C::TILE - 1) / C::TILE : 0;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;

  // ---- HBM -> LDS tile copy (each wave issues instructions w, w+4, ...) ----
  const int niw = (C::NI - w + 3) / 4;            // DMA instructions of this wave per tile
  auto issue_tile = [&](int it) {
    const int t0 = lo + C::TILE * it;
    const uint16_t* src = p.cache + ((size_t)bt[t0 / BS] * BS + (t0 % BS)) * ROW;
    unsigned char* dst = lds + (it % C::NBUF) * C::BUF_BYTES;
    for (int i = w; i < C::NI; i += 4) {
      const int P = i * 64 + lane;
      const int t = P / CHR, pos = P % CHR;
      const int ch = C::SWZ ? (pos ^ tile_swz(t)) : pos;
      __builtin_amdgcn_global_load_lds((const void*)(src + t * ROW + ch * 8),
                                       (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
  };
  if (n_tiles > 0) issue_tile(0);
  if (n_tiles > 1) issue_tile(1);

  // ---- rows of this wave: rho = 128*rb + 32*w + 16*nt + c (head-major: rho = h*SQ + i) ----
  const int row0 = rb * C::ROWS_WG + 32 * w;
  const bool wave_has_rows = row0 < rows_total;
  int nvis[2], grp[2];
  bool rvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int rho = row0 + 16 * nt + c;
    rvalid[nt] = rho < rows_total;
    const int h = rvalid[nt] ? rho / SQ : 0, i = rvalid[nt] ? rho % SQ : SQ - 1;
    nvis[nt] = L - SQ + i + 1;
    grp[nt] = h / HPG;
  }

  // ---- Q operands [q_abs | q_rope] (written by absorb_q_kernel) in the QK B layout ----
  // lane (q, c) of qb[nt][ks] holds 8 consecutive dims 32ks + 8q.. of row c.
  bf16x8 qb[2][KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int rho = row0 + 16 * nt + c;
    const int h = rvalid[nt] ? rho / SQ : 0, i = rvalid[nt] ? rho % SQ : 0;
    const uint16_t* qrow = p.qcat + (((size_t)b * SQ + i) * H + h) * ROW;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int dim = 32 * ks + 8 * q;
      qb[nt][ks] = (rvalid[nt] && dim < ROW) ? ld_bf16x8(qrow + dim) : zero_bf16x8();
    }
  }

  // ---- main loop over 32-token tiles ----
  f32x4 o[MTL][2];
#pragma unroll
  for (int mt = 0; mt < MTL; ++mt) o[mt][0] = o[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  for (int it = 0; it < n_tiles; ++it) {
    block_sync_lds();                             // everyone is done with tile it-1
    if (it + 2 < n_tiles) issue_tile(it + 2);
    wait_vm_dyn(niw * (min(it + 2, n_tiles - 1) - it));
    block_sync_lds();                             // tile it is in LDS for every wave
    if (!wave_has_rows) continue;
    const unsigned char* buf = lds + (it % C::NBUF) * C::BUF_BYTES;
    const int t0 = lo + C::TILE * it;

    // S^T: token-subtile st holds tokens 8*(c/4) + 4*st + c%4 in MFMA row c, so the
    // accumulator lane (q, c) holds tokens 8q + 4st + 0..3 of query row c.
    f32x4 s[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st][0] = s[st][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = 8 * (c >> 2) + 4 * st + (c & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = 4 * ks + q;
        const int pos = C::SWZ ? (ch ^ tile_swz(t)) : ch;
        bf16x8 a;
        if (ks >= KSL && 32 * (ks - KSL) + 8 * q >= DR) {
          a = zero_bf16x8();                      // rope padding
        } else {
          a = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(buf + (t * CHR + pos) * 16));
        }
        s[st][0] = mfma16(a, qb[0][ks], s[st][0]);
        s[st][1] = mfma16(a, qb[1][ks], s[st][1]);
      }
    }
    // online softmax (base 2); masked tokens -> -inf, never added
    bf16x8 pb[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 8 * q + 4 * st + i;
          const float v = s[st][nt][i] * p.scale_log2;
          x[4 * st + i] = (tok < nvis[nt]) ? v : -INFINITY;
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
      for (int mt = 0; mt < MTL; ++mt) o[mt][nt] *= alpha;
      u32x4 pk = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                  pack_bf16x2(x[6], x[7])};
      pb[nt] = __builtin_bit_cast(bf16x8, pk);
    }
    // PV: A = C^T tile (latent 16mt + c, tokens 8q + j) via transposing LDS reads.
    const bool tail = t0 + C::TILE > L;
    const int keep = min(max(L - (t0 + 8 * q), 0), 8);
#pragma unroll
    for (int mt = 0; mt < MTL; ++mt) {
      const int n = 16 * mt + 4 * (c & 3);        // latent column of this source lane
      const int ch = n >> 3, half = (n & 7) * 2;
      bf16x8 v;
      {
        const int t_lo = 8 * q + (c >> 2), t_hi = t_lo + 4;
        const int p_lo = C::SWZ ? (ch ^ tile_swz(t_lo)) : ch;
        const int p_hi = C::SWZ ? (ch ^ tile_swz(t_hi)) : ch;
        s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + (t_lo * CHR + p_lo) * 16 + half));
        s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(buf + (t_hi * CHR + p_hi) * 16 + half));
        v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      if (tail) v = keep_first(v, keep);
      o[mt][0] = mfma16(v, pb[0], o[mt][0]);
      o[mt][1] = mfma16(v, pb[1], o[mt][1]);
    }
  }

  // ---- epilogue: normalise, up-project by W_UV[G], write ----
  block_sync_lds();                               // KV buffers are free from here on
  if (!wave_has_rows) return;
  float inv[2], lse_v[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = wave_sum_xor16_32(l_run[nt]);
    inv[nt] = lt > 0.f ? 1.f / lt : 0.f;
    lse_v[nt] = lt > 0.f ? (m_run[nt] + log2f(lt)) * kLn2 : -INFINITY;
  }
  unsigned char* stage = lds + w * C::WSTAGE_BYTES;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r_first = row0 + 16 * nt;
    if (r_first >= rows_total) continue;
    const int r_last = min(r_first + 15, rows_total - 1);
    const int g_lo = (r_first / SQ) / HPG, g_hi = (r_last / SQ) / HPG;
    const int rho = r_first + c;
    const int h = rvalid[nt] ? rho / SQ : 0, i = rvalid[nt] ? rho % SQ : 0;
    for (int G = g_lo; G <= g_hi; ++G) {
      const uint16_t* W = p.w_uv + (size_t)G * R * DV;
      f32x4 acc[MD];
#pragma unroll
      for (int md = 0; md < MD; ++md) acc[md] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r0 = 0; r0 < R; r0 += C::WCH) {
        // stage rows r0 .. r0+WCH-1 of W_UV[G] (wave-private)
        constexpr int PIECES = C::WCH * DV / 8;
        __builtin_amdgcn_wave_barrier();
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        for (int id = lane; id < PIECES; id += 64) {
          const int rr = id / (DV / 8), cc = (id % (DV / 8)) * 8;
          *(lds_u32x4*)(stage + (rr * C::WSTRIDE + cc) * 2) =
              *reinterpret_cast<const u32x4*>(W + (size_t)(r0 + rr) * DV + cc);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < C::WCH / 32; ++kk) {
          // B operand: o_lat of row c, k slot j <-> latent 32*kk' + 16*(j/4) + 4q + j%4
          const int kg = r0 / 32 + kk;              // global 32-latent step
          const f32x4 o0 = o[2 * kg][nt] * inv[nt], o1 = o[2 * kg + 1][nt] * inv[nt];
          u32x4 pk = {pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3]),
                      pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
          const bf16x8 bo = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
          for (int md = 0; md < MD; ++md) {
            // A operand: W_UV^T, lane (q, i) slot 4hh + r <-> W rows 32kk + 16hh + 4q + r, col 16md + i
            const int col = 16 * md + 4 * (c & 3);
            const int rlo = 32 * kk + 4 * q + (c >> 2);
            s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(stage + (rlo * C::WSTRIDE + col) * 2));
            s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(stage + ((rlo + 16) * C::WSTRIDE + col) * 2));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[md] = mfma16(a, bo, acc[md]);
          }
        }
      }
      // acc[md] lane (q, c): dims 16md + 4q .. +3 of row c
      if (!(rvalid[nt] && grp[nt] == G)) continue;
      if (p.split_offsets) {
        const size_t row = ((size_t)u * SQ + i) * H + h;
#pragma unroll
        for (int md = 0; md < MD; ++md)
          *reinterpret_cast<f32x4*>(p.part_out + row * DV + 16 * md + 4 * q) = acc[md];
        if (q == 0) p.part_lse[row] = lse_v[nt];
      } else {
        const size_t row = ((size_t)b * SQ + i) * H + h;
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          u32x2 pk = {pack_bf16x2(acc[md][0], acc[md][1]), pack_bf16x2(acc[md][2], acc[md][3])};
          *reinterpret_cast<u32x2*>(p.out + row * DV + 16 * md + 4 * q) = pk;
        }
        if (q == 0 && p.lse) p.lse[row] = lse_v[nt];
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
#pragma unroll 4
  for (int mt = 0; mt < MT; ++mt) {
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
  for (int id = lane; id < 16 * DR / 8; id += 64) {
    const int rr = id / (DR / 8), part = id % (DR / 8);
    const int gr2 = r0 + rr;
    if (gr2 >= rows_g) continue;
    const size_t qr2 = ((size_t)(gr2 / HPG) * H + G * HPG + gr2 % HPG);
    *reinterpret_cast<u32x4*>(p.qcat + qr2 * ROW + R + part * 8) =
        *reinterpret_cast<const u32x4*>(p.q_rope + qr2 * DR + part * 8);
  }
}

template <int HPG, int SQ, int R, int DR, int DN, int DV>
hipError_t launch_absorb(const DecodeParams& p, hipStream_t stream) {
  {
    const int rows_g = p.batch * SQ * HPG;
    dim3 grid((unsigned)((rows_g + 63) / 64), (unsigned)p.num_groups);
    hipLaunchKernelGGL((absorb_q_kernel<HPG, SQ, R, DR, DN>), grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  using C = AbsorbCfg<HPG, SQ, R, DR, DN, DV>;
  const int rows_total = HPG * p.num_groups * SQ;
  const int RB = (rows_total + C::ROWS_WG - 1) / C::ROWS_WG;
  const unsigned grid = (unsigned)((p.num_units + 7) / 8) * 8u * (unsigned)RB;
  hipLaunchKernelGGL((absorb_decode_kernel<HPG, SQ, R, DR, DN, DV>), dim3(grid), dim3(256), 0,
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
