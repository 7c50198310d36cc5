// One-shot cache expansion: latent pages -> per-group K/V pages.
//
// GQLA pages: paperlayer.ai summary, section 3 "Methods", bullet "Two
// equivalent decoding paths" (deployment switches paths by a one-shot cache
// compression or expansion) and pwwt.cn section 3 (expansion is a one-time
// deployment step, not per decode step).  Per token t and group G:
//   K[t, G] = bf16(c_t W_UK[G]),  V[t, G] = bf16(c_t W_UV[G]),  rope copied.
//
// Each workgroup (4 waves) computes one (group, K-or-V) product for 4 pages
// (256 tokens): a [256 x r] x [r x d] GEMM on bf16 MFMA with fp32
// accumulation.  The weight slice for a 32-row k step is staged in LDS and
// read with ds_read_b64_tr_b16 (transposing read), because the MFMA A
// operand needs 8 consecutive latent rows of one weight column per lane; the
// latent rows come straight from HBM as 16-byte operand loads.  Both K and V
// are produced transposed, K^T = W_UK^T C^T and V^T = W_UV^T C^T, so every
// lane writes 4 consecutive dims of one token (both blocks token-major).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

template <int R, int DH, int DR, bool KIND_V>
__device__ __forceinline__ void expand_body(const ExpandParams& p, int64_t tile, int G, uint16_t* wl);

template <int R, int DH, int DR>
__global__ __launch_bounds__(256) void expand_kernel(ExpandParams p) {
  constexpr int LDS_STRIDE = DH + 16;   // padded weight row (elements)
  __shared__ __attribute__((aligned(16))) uint16_t wl[32 * LDS_STRIDE];
  const int g = p.num_groups;
  const int64_t n_tiles = (p.n_expand + 3) / 4;
  const int wg = blockIdx.x;
  const int xcd = wg & 7, k = wg >> 3;
  const int64_t tile = (int64_t)(k / (2 * g)) * 8 + xcd;
  const int gk = k % (2 * g);
  if (tile >= n_tiles) return;          // uniform over the workgroup
  if (gk & 1) expand_body<R, DH, DR, true>(p, tile, gk >> 1, wl);
  else expand_body<R, DH, DR, false>(p, tile, gk >> 1, wl);
}

template <int R, int DH, int DR, bool KIND_V>
__device__ __forceinline__ void expand_body(const ExpandParams& p, int64_t tile, int G, uint16_t* wl) {
  constexpr bool kind_v = KIND_V;
  constexpr int BS = 64;
  constexpr int KS = R / 32;            // k steps
  constexpr int MT = DH / 16;           // 16-dim tiles of the output
  constexpr int NT = BS / 16;           // 16-slot tiles (one page per wave)
  constexpr int LDS_STRIDE = DH + 16;
  constexpr int CHUNKS = 32 * DH / 8;   // 16-byte pieces of one weight k step
  static_assert(R % 32 == 0 && DH % 16 == 0, "unsupported dims");
  const int g = p.num_groups;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int64_t idx = tile * 4 + wave;
  const bool active = idx < p.n_expand;
  const int64_t pidx = active ? idx : 0;
  const int64_t page = p.page_ids ? (int64_t)p.page_ids[pidx] : pidx;
  constexpr int ROW = R + DR;                                   // latent row length
  const uint16_t* lat = p.latent + (size_t)page * BS * ROW;
  const size_t page_elems = (size_t)BS * (g * 2 * DH + DR);
  uint16_t* dst = p.expanded + (size_t)page * page_elems;
  const uint16_t* W = (kind_v ? p.w_uv : p.w_uk) + (size_t)G * R * DH;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int WPT = (CHUNKS + 255) / 256;   // weight pieces per thread per k step
  constexpr bool WFULL = CHUNKS % 256 == 0;
  // Rows of inactive waves (past the last page) alias the first listed page:
  // they are loaded and multiplied but never stored.
  const uint16_t* crow = lat + (size_t)c * ROW + 8 * q;
  u32x4 wreg[WPT];
  bf16x8 cb[2][NT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int ch = tid + 256 * i;
    if (WFULL || ch < CHUNKS)
      wreg[i] = *reinterpret_cast<const u32x4*>(W + (size_t)(ch / (DH / 8)) * DH + (ch % (DH / 8)) * 8);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) cb[0][nt] = ld_bf16x8(crow + (size_t)16 * nt * ROW);

#pragma unroll 2
  for (int ks = 0; ks < KS; ++ks) {
    __syncthreads();                    // all waves done reading the previous slice
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int ch = tid + 256 * i;
      if (WFULL || ch < CHUNKS)
        *reinterpret_cast<u32x4*>(wl + (ch / (DH / 8)) * LDS_STRIDE + (ch % (DH / 8)) * 8) = wreg[i];
    }
    __syncthreads();
    if (ks + 1 < KS) {
#pragma unroll
      for (int i = 0; i < WPT; ++i) {
        const int ch = tid + 256 * i;
        if (WFULL || ch < CHUNKS)
          wreg[i] = *reinterpret_cast<const u32x4*>(W + (size_t)(32 * (ks + 1) + ch / (DH / 8)) * DH +
                                                    (ch % (DH / 8)) * 8);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        cb[(ks + 1) & 1][nt] = ld_bf16x8(crow + (size_t)16 * nt * ROW + 32 * (ks + 1));
    }
    const int cur = ks & 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // transposing read: lane (q, i) gets W[32ks + 8q + j][16mt + i], j = 0..7
      const uint16_t* a0 = wl + (8 * q + (c >> 2)) * LDS_STRIDE + 16 * mt + 4 * (c & 3);
      const uint16_t* a1 = a0 + 4 * LDS_STRIDE;
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a0);
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a1);
      bf16x8 wt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16(wt, cb[cur][nt], acc[mt][nt]);
    }
  }

  if (!active) return;
  uint16_t* kblk = dst + (size_t)G * BS * 2 * DH;
  uint16_t* vblk = kblk + BS * DH;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const f32x4 v = acc[mt][nt];
      u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      // lane holds dims 16mt + 4q .. +3 of slot 16nt + c
      *reinterpret_cast<u32x2*>((kind_v ? vblk : kblk) + (16 * nt + c) * DH + 16 * mt + 4 * q) = pk;
    }
  if (G == 0 && !kind_v) {
    uint16_t* rope = dst + (size_t)g * BS * 2 * DH;
    constexpr int PIECES = BS * DR / 8;
    for (int id = lane; id < PIECES; id += 64) {
      const int slot = id / (DR / 8), part = id % (DR / 8);
      *reinterpret_cast<u32x4*>(rope + slot * DR + part * 8) =
          *reinterpret_cast<const u32x4*>(lat + (size_t)slot * ROW + R + part * 8);
    }
  }
}

// ---------------------------------------------------------------------------
// The 512 + 64 latent row with d_nope = d_v = 128: one workgroup of four waves
// (one per SIMD, 512 registers each) per 4 pages; wave w owns page 4 wg + w
// (64 tokens) for every (group, K or V) block.
//   * The page's latent rows stay in accumulation registers for the whole
//     workgroup as the B operands of K^T = W^T C^T (lane (q, c) holds
//     C[token 16 nt + c][32 kc + 8 q .. +7]: 4 token tiles x 16 k chunks,
//     256 registers), read from HBM once instead of once per block.
//   * Each block W[G] (512 x 128 bf16, shared by every workgroup from L2) is
//     taken in two 64-dim halves; a phase covers one half over 256 k rows, a
//     32 KB slice copied into LDS by direct copy (global_load_lds_dwordx4):
//     four slice buffers, three slices in flight, one workgroup barrier per
//     phase.  The A operand (8 consecutive k of one output dim per lane) is a
//     transposing read (ds_read_b64_tr_b16) of the slice's 128-byte rows;
//     16-byte chunk x of row r sits at x ^ s(r),
//     s(r) = 2 (((r >> 1) & 1) + 2 ((r >> 3) & 1)), which puts each 32-lane
//     pass of the read on 64 distinct banks (checked exhaustively against the
//     measured pass structure).  Each A operand feeds four MFMAs (the four
//     token tiles).
//   * The same MFMA (16x16x32) over the same 32-wide k chunks in the same
//     order as gqla_append_tokens, so both write bit-identical K and V.
//   * A finished half-block (64 tokens x 64 dims) is rounded to bf16 and
//     staged in LDS (the wave's 8 KB, token rows of 128 bytes, chunk x of
//     token t at x ^ ((t >> 1) & 7): conflict-free writes and reads), then
//     stored during the next two phases with one store instruction per 8
//     whole rows (full 128-byte lines), so that the output writes of all
//     workgroups (which run in step) spread over the run instead of meeting
//     in one burst per block.
//   * The copy and store instructions of a phase sit between its MFMAs (one
//     every four), where their issue overlaps the matrix work.
//   * The latent rows (read once) and the output rows (written once, 1.1 GB
//     for the DeepSeek-V3-shaped pool) use the non-temporal policy; the weight
//     slices, shared by every workgroup through L2, the default one.
template <int R, int DH, int DR>
struct ExpandPagesCfg {
  static constexpr int BS = 64;
  static constexpr int ROW = R + DR;
  static constexpr int NW = 4;                     // waves = pages per workgroup
  static constexpr int DHH = 64;                   // output dims per pass (half a block)
  static constexpr int NH = DH / DHH;              // passes per block
  static constexpr int KH = 256;                   // weight rows per phase
  static constexpr int NKH = R / KH;               // phases per pass
  static constexpr int SBYTES = KH * DHH * 2;      // one slice in LDS
  static constexpr int NBUF = 4;
  static constexpr int NI = SBYTES / 1024;         // copy instructions per slice
  static constexpr int NIW = NI / NW;              // per wave
  static constexpr int KC = R / 32;                // k chunks of the product
  static constexpr int KCP = KH / 32;              // per phase
  static constexpr int MT = DHH / 16;              // 16-dim output tiles per pass
  static constexpr int NT = BS / 16;               // 16-token tiles of a page
  static constexpr int NPART = 2;                  // store parts of a finished pass
  static constexpr int STAGE = BS * DHH * 2;       // a wave's staged pass (bytes)
  static constexpr int NSI = STAGE / 1024;         // its store instructions (8 token rows each)
  static constexpr int NSP = NSI / NPART;          // per part
  static constexpr int OFF_STAGE = NBUF * SBYTES;
  static constexpr int LDS_BYTES = OFF_STAGE + NW * STAGE;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(DHH == 64 && DH % DHH == 0, "128-byte slice rows: the chunk swizzle covers 8 chunks");
  static_assert(R % KH == 0 && NI % NW == 0 && KH * DH * 2 <= 65536, "slice tiling, 16-bit copy offsets");
  static_assert(NKH >= NPART && NSI % NPART == 0, "a pass's stores fit in the next pass's phases");
};

__device__ __forceinline__ int ex_swz(int r) { return 2 * (((r >> 1) & 1) + 2 * ((r >> 3) & 1)); }

template <int R, int DH, int DR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void expand_pages_kernel(ExpandParams p) {
  using C = ExpandPagesCfg<R, DH, DR>;
  constexpr int BS = C::BS, ROW = C::ROW, NW = C::NW, NIW = C::NIW, KCP = C::KCP, NKH = C::NKH, NH = C::NH;
  constexpr int MT = C::MT, NT = C::NT, KC = C::KC, DHH = C::DHH, NPART = C::NPART, NSP = C::NSP;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_raw[C::LDS_BYTES];
  lds_u8_t* const lds = (lds_u8_t*)lds_raw;
  const int g = p.num_groups;
  const int npass = 2 * g * NH;                    // (group, K or V, half) passes
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, q = lane >> 4;
  // This workgroup's segment: page quad `quad` (wave w: page 4 quad + w),
  // passes ps0 .. ps1 - 1.  The first whole_quads workgroups take a quad
  // whole; each later one takes one of `pieces` pass ranges of a quad, so the
  // last, partial round of quads is spread over many CUs.
  const int64_t wi = blockIdx.x;
  int64_t quad = wi;
  int ps0 = 0, ps1 = npass;
  if (wi >= p.whole_quads) {
    const int r = (int)(wi - p.whole_quads);     // below CUs * passes: 32-bit division
    const int j = r % p.pieces;
    quad = p.whole_quads + r / p.pieces;
    ps0 = j * npass / p.pieces;
    ps1 = (j + 1) * npass / p.pieces;
  }
  __builtin_assume(ps0 >= 0);                      // (so the k step of a phase, pi % NKH, is known)
  const int nph = ps1 * NKH;                       // end of the segment's phases
  const int64_t idx = quad * NW + w;
  const bool active = idx < p.n_expand;            // inactive waves compute on page 0 and store nothing
  const int64_t pidx = active ? idx : 0;
  const int64_t page = p.page_ids ? (int64_t)p.page_ids[pidx] : pidx;
  const uint16_t* lat = p.latent + (size_t)page * BS * ROW;
  const size_t page_elems = (size_t)BS * (g * 2 * DH + DR);
  uint16_t* dst = p.expanded + (size_t)page * page_elems;

  // Phase pi: pass ps = pi / NKH (block blk = ps / NH, half h = ps % NH),
  // weight rows KH (pi % NKH) .. +KH-1, dims DHH h .. +DHH-1.
  // This wave's copy instructions of every slice: instruction k (of the
  // slice's NI) fills LDS bytes 1024 k ..; position P = 64 k + lane holds
  // row P / 8, physical chunk P % 8 = logical chunk (P % 8) ^ s(row).
  // Source offsets (bytes from the slice's first row and dim) packed two per
  // register.
  uint32_t cpo[(NIW + 1) / 2];
#pragma unroll
  for (int kk = 0; kk < NIW; ++kk) {
    const int P = (w * NIW + kk) * 64 + lane;
    const int r = P / 8, pc = P % 8;
    const uint32_t off = (uint32_t)(r * DH * 2 + ((pc ^ ex_swz(r)) * 16));
    if (kk % 2 == 0) cpo[kk / 2] = off; else cpo[kk / 2] |= off << 16;
  }
  auto slice_src = [&](int pi) -> const uint16_t* {
    const int ps = pi / NKH, blk = ps / NH, h = ps % NH, kh = pi % NKH;
    const uint16_t* W = ((blk & 1) ? p.w_uv : p.w_uk) + (size_t)(blk >> 1) * R * DH;
    return W + (size_t)kh * C::KH * DH + h * DHH;
  };
  auto copy_part = [&](const uint16_t* src, int pi, int kk) {   // copy instruction kk of slice pi
    const uint32_t off = (kk % 2 == 0) ? (cpo[kk / 2] & 0xffffu) : (cpo[kk / 2] >> 16);
    dma16(src, off, lds + (pi % C::NBUF) * C::SBYTES + (w * NIW + kk) * 1024);
  };
  auto copy_slice = [&](int pi) {
    const uint16_t* src = slice_src(pi);
#pragma unroll
    for (int kk = 0; kk < NIW; ++kk) copy_part(src, pi, kk);
  };

  // ---- start: the page's latent rows into accumulation registers; slices
  // 0, 1, 2 ----
  bf16x8 cb[NT][KC];
  {
    const uint16_t* crow = lat + (size_t)c * ROW + 8 * q;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        cb[nt][kc] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                                    crow + (size_t)16 * nt * ROW + 32 * kc)));
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (ps0 * NKH + j < nph) copy_slice(ps0 * NKH + j);
  vm_wait<0>();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) asm volatile("" : "+a"(cb[nt][kc]));
  block_sync_lds();

  // transposing-read bases of output tile mt: row 8 q + (c >> 2) of the
  // k chunk, dims 16 mt + 4 (c & 3) .. +3 of the half; + (32 kc + 4 rd) rows
  int ab[MT];
  {
    const int r0 = 8 * q + (c >> 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      ab[mt] = r0 * DHH * 2 + (((2 * mt + ((c & 3) >> 1)) ^ ex_swz(r0)) * 16) + 8 * (c & 1);
  }
  auto a_operand = [&](const lds_u8_t* buf, int kc, int mt) -> bf16x8 {
    const int imm = 32 * kc * DHH * 2;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + ab[mt] + imm));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(buf + ab[mt] + imm + 4 * DHH * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x4 acc[MT][NT];
  lds_u8_t* const stage = lds + C::OFF_STAGE + w * C::STAGE;
  // staged byte offset of 16-byte chunk x of token t
  auto stage_off = [&](int t, int x) -> int { return t * DHH * 2 + ((x ^ ((t >> 1) & 7)) * 16); };
  // the output rows of pass ps (token-major, DH elements apart)
  auto pass_dst = [&](int ps) -> uint16_t* {
    const int blk = ps / NH, h = ps % NH;
    return dst + (size_t)(blk >> 1) * BS * 2 * DH + (blk & 1) * BS * DH + h * DHH;
  };
  // store instruction i of a staged pass: tokens 8 i .. 8 i + 7, lane l writes
  // chunk l % 8 of token 8 i + l / 8
  auto staged = [&](int i) -> u32x4 {
    return *(const lds_u32x4_t*)(stage + stage_off(8 * i + lane / 8, lane % 8));
  };
  auto store_row8 = [&](uint16_t* ob, int i, const u32x4& v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(ob + (size_t)(8 * i + lane / 8) * DH + 8 * (lane % 8)));
  };
  // Phase pi (k step kh of pass ps): the MFMAs of slice pi, with the copies
  // of slice pi + 3 (cpy; its buffer was last read in phase pi - 1) and part
  // kh of the previous pass's stores (st) between them; after the pass's last
  // phase the pass is staged.  FIRST: the pass's first phase (its first k
  // chunk starts the accumulators from zero).
  auto mfmas = [&](int pi, auto first, bool cpy, bool st) {
    constexpr bool FIRST = decltype(first)::value;
    const int kh = pi % NKH;
    const lds_u8_t* buf = lds + (pi % C::NBUF) * C::SBYTES;
    const uint16_t* csrc = slice_src(pi + 3);
    uint16_t* ob = pass_dst(pi / NKH - 1);
    u32x4 sv[NSP];
    if (st) {
#pragma unroll
      for (int i = 0; i < NSP; ++i) sv[i] = staged(kh * NSP + i);
    }
    constexpr int NS = KCP * MT;                   // A operands
    constexpr int PD = 2;
    static_assert(NS >= 4 * NIW && NS >= 4 * NSP, "copy and store slots");
    bf16x8 a[PD + 1];
#pragma unroll
    for (int j = 0; j < PD; ++j) a[j] = a_operand(buf, j / MT, j % MT);
    sched_fence();
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int kc = j / MT, mt = j % MT;
      if (j + PD < NS) a[(j + PD) % (PD + 1)] = a_operand(buf, (j + PD) / MT, (j + PD) % MT);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 bq = cb[nt][KCP * kh + kc];
        acc[mt][nt] = mfma16(a[j % (PD + 1)], bq, (FIRST && kc == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt][nt]);
      }
      if (j % 4 == 0 && j / 4 < NIW && cpy) copy_part(csrc, pi + 3, j / 4);
      if (j % 4 == 2 && j / 4 < NSP && st) store_row8(ob, kh * NSP + j / 4, sv[j / 4]);
      // the step's four MFMAs interleaved with its two operand reads and its
      // address arithmetic (measured: 2796 against 2849 clocks per phase)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x006, 2, 0);   // VALU / SALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      sched_fence();
    }
  };
  auto stage_pass = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int t = 16 * nt + c, d = 16 * mt + 4 * q;     // 4 dims of token t
        const u32x2 pk = {pack_bf16x2(acc[mt][nt][0], acc[mt][nt][1]), pack_bf16x2(acc[mt][nt][2], acc[mt][nt][3])};
        *(__attribute__((address_space(3))) u32x2*)(stage + stage_off(t, d / 8) + (d % 8) * 2) = pk;
      }
  };
  // Phase pi, then slice pi + 1 landed (barrier).  The wait counts only the
  // copies issued after slice pi + 1's; stores among them at worst make it
  // wait longer.  Every wave reads only its own staged rows.
  auto phase = [&](int pi, auto first) {
    const int ps = pi / NKH, kh = pi % NKH;
    mfmas(pi, first, pi + 3 < nph, active && ps > ps0 && kh < NPART);
    if (kh == NKH - 1) stage_pass();
    if (pi + 3 < nph) vm_wait<2 * NIW>();
    else if (pi + 2 < nph) vm_wait<NIW>();
    else vm_wait<0>();
    block_sync_lds();
  };
  using T = std::true_type;
  using F = std::false_type;
  for (int ps = ps0; ps < ps1; ++ps) {
    phase(ps * NKH, T{});
#pragma unroll
    for (int kh = 1; kh < NKH; ++kh) phase(ps * NKH + kh, F{});
  }
  if (active) {                                    // the segment's last pass
    uint16_t* ob = pass_dst(ps1 - 1);
#pragma unroll
    for (int i = 0; i < C::NSI; ++i) store_row8(ob, i, staged(i));
  }

  // the shared rope key, copied unchanged (by the segment that starts the page)
  if (active && ps0 == 0) {
    uint16_t* rope = dst + (size_t)g * BS * 2 * DH;
    for (int id = lane; id < BS * DR / 8; id += 64) {
      const int slot = id / (DR / 8), part = id % (DR / 8);
      *reinterpret_cast<u32x4*>(rope + slot * DR + part * 8) =
          *reinterpret_cast<const u32x4*>(lat + (size_t)slot * ROW + R + part * 8);
    }
  }
}

// Compute units of the current device, looked up once per device.
hipError_t cu_count(int* n) {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = v > 0 ? v : 1;
  }
  *n = cached[dev];
  return hipSuccess;
}

hipError_t expand_dispatch(int r, int dn, int dv, int dr, const ExpandParams& p, hipStream_t stream,
                           bool* supported) {
  *supported = true;
  const int64_t n_tiles = (p.n_expand + 3) / 4;
  const int64_t rounds = (n_tiles + 7) / 8;
  const int64_t grid64 = rounds * 8 * 2 * p.num_groups;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > 0x7fffffff) { *supported = false; return hipSuccess; }
  const unsigned grid = (unsigned)grid64;
  if (r == 512 && dn == 128 && dv == 128 && dr == 64) {
    using C = ExpandPagesCfg<512, 128, 64>;
    // One workgroup per CU at a time (it takes all of a CU's LDS).  The quads
    // of the last, partial round (quads mod CUs) are each cut into up to
    // CUs / leftover pass ranges, so that round takes about one pass instead
    // of a whole quad on a few CUs.
    int cus = 0;
    const hipError_t e = cu_count(&cus);
    if (e != hipSuccess) return e;
    const int64_t quads = (p.n_expand + C::NW - 1) / C::NW;
    const int64_t left = quads % cus;
    const int npass = 2 * p.num_groups * C::NH;
    const int pieces = left > 0 ? (int)std::min<int64_t>(npass, cus / left) : 1;
    ExpandParams q = p;
    q.whole_quads = quads - left;
    q.pieces = pieces;
    const int64_t nwg = q.whole_quads + left * pieces;
    if (nwg > 0x7fffffff) { *supported = false; return hipSuccess; }
    hipLaunchKernelGGL((expand_pages_kernel<512, 128, 64>), dim3((unsigned)nwg), dim3(64 * C::NW), 0, stream, q);
  } else if (r == 64 && dn == 32 && dv == 32 && dr == 16) {
    hipLaunchKernelGGL((expand_kernel<64, 32, 16>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    *supported = false;
    return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace gqla
