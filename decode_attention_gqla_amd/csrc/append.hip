// Incremental append of new tokens: their latent rows into the paged latent
// cache and, for the GQA path, their per-group K/V into the expanded cache.
//
// GQLA pages: paperlayer.ai summary, section 4 "GQA path" (after the one-shot
// conversion the GQA path decodes with no per-step latent expansion: the
// latent pages stay the stored state) and section 3 "Methods" (the latent
// row of a token is c_t ++ k_rope_t; K = c W_UK[G], V = c W_UV[G]).  Each
// decode step adds n_new tokens per sequence at positions L_b - n_new ..
// L_b - 1 (page block_table[b][t / 64], slot t % 64).
//
// append_kernel: one wave per (sequence, new token) copies the row.
// expand_tokens_kernel: one workgroup per (16-token tile of the new tokens of
// the whole batch, group, K or V, half of the output dims), its column slice
// of W[G] copied into LDS by direct DMA, four waves over the output dims; the
// workgroups of group 0 also write the tile's latent rows.  The new rows are
// read from the caller's buffer, so nothing orders the copy before the
// products.  It multiplies exactly as the one-shot
// expansion kernel does for those tokens -- the same 16x16x32 MFMA in the same
// orientation (K^T = W_UK^T C^T, V^T = W_UV^T C^T), the same 32-row k steps in the same
// order, the same rounding -- so every written value is bit-identical to a
// full expansion of the updated pages; only the new tokens' slots are
// written.
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

__global__ __launch_bounds__(64) void append_kernel(AppendParams p) {
  const int b = blockIdx.x / p.n_new, j = blockIdx.x % p.n_new;
  const int lane = threadIdx.x;
  const int t = p.seqlens[b] - p.n_new + j;       // position of new token j
  const int64_t row_elems = p.row_elems;
  const int chunks = (int)(row_elems / 8);        // 16-byte pieces per row
  if (t < 0 || t / p.bs >= p.max_blocks) return;  // precondition violated: write nothing
  const int32_t page = p.block_table[(size_t)b * p.max_blocks + t / p.bs];
  const u32x4* src = reinterpret_cast<const u32x4*>(p.new_rows + ((size_t)b * p.n_new + j) * row_elems);
  u32x4* dst = reinterpret_cast<u32x4*>(p.latent + ((size_t)page * p.bs + t % p.bs) * row_elems);
  for (int c = lane; c < chunks; c += 64) dst[c] = src[c];
}

template <int R, int DH, int DR>
__global__ __launch_bounds__(256) void expand_tokens_kernel(AppendParams p) {
  constexpr int BS = 64, ROW = R + DR, KS = R / 32;
  constexpr int NH = DH >= 64 ? 2 : 1;            // column halves of W[G] (one per workgroup)
  constexpr int DC = DH / NH;                     // output dims of this workgroup
  constexpr int MTC = DC / 16, NWV = 4, MTW = (MTC + NWV - 1) / NWV;
  constexpr int PR = DC / 8;                      // 16-byte pieces per W row slice
  constexpr int NI = R * PR / 64;                 // copy instructions for the slice
  static_assert((R * PR) % 64 == 0, "whole copy instructions");
  __shared__ __attribute__((aligned(1024))) uint16_t wl[R * DC];   // W[G][:, slice], row stride DC
  const int g = p.num_groups;
  int id = blockIdx.x;
  const int hsel = id % NH;
  id /= NH;
  const int tile = id / (2 * g), gk = id % (2 * g);
  const int G = gk >> 1;
  const bool kind_v = gk & 1;                     // uniform
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int n_tok = p.batch * p.n_new;
  // position of new token `tok` of the batch: its page and slot; false when
  // the position breaks the precondition (t < 0 or past the block table), and
  // then nothing is written for the token
  auto locate = [&](int tok, int& page, int& slot) -> bool {
    const int b = tok / p.n_new, j = tok % p.n_new;
    const int t = p.seqlens[b] - p.n_new + j;
    if (t < 0 || t / BS >= p.max_blocks) return false;
    page = p.block_table[(size_t)b * p.max_blocks + t / BS];
    slot = t % BS;
    return true;
  };
  // this workgroup's column slice of W[G] into LDS by direct copy: piece
  // i * 64 + lane is row (i * 64 + lane) / PR, 16-byte piece % PR of the slice
  const uint16_t* W = (kind_v ? p.w_uv : p.w_uk) + (size_t)G * R * DH + hsel * DC;
  lds_u8_t* const wlds = (lds_u8_t*)wl;
  for (int i = w; i < NI; i += NWV) {
    const int pc = i * 64 + lane;
    dma16(W, (uint32_t)((pc / PR) * DH + (pc % PR) * 8) * 2u, wlds + i * 1024);
  }
  // MFMA column / row c of the tile is new token tile*16 + c (its row read
  // from new_rows); past the last token it repeats the last one (multiplied,
  // never stored)
  const int tok_c = min(tile * 16 + c, n_tok - 1);
  const uint16_t* crow = p.new_rows + (size_t)tok_c * ROW + 8 * q;
  bf16x8 cb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) cb[ks] = ld_bf16x8(crow + 32 * ks);
  vm_wait<0>();
  __syncthreads();                                // every wave's part of the slice landed

  f32x4 acc[MTW];
#pragma unroll
  for (int m = 0; m < MTW; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const int mt = w * MTW + m;
      if (mt >= MTC) break;                       // uniform
      // transposing read: lane (q, i) gets W[32 ks + 8 q + j][slice col 16 mt + i], j = 0..7
      const uint16_t* a0 = wl + (32 * ks + 8 * q + (c >> 2)) * DC + 16 * mt + 4 * (c & 3);
      const uint16_t* a1 = a0 + 4 * DC;
      s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a0);
      s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a1);
      const bf16x8 wt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[m] = mfma16(wt, cb[ks], acc[m]);
    }
  }

  const size_t page_elems = (size_t)BS * (g * 2 * DH + DR);
  const int d0 = hsel * DC;                       // first output dim of this workgroup
  // lane (q, c) holds dims d0 + 16 mt + 4 q .. +3 of token c (K and V token-major)
  int page_c = 0, slot_c = 0;
  if (tile * 16 + c < n_tok && locate(tok_c, page_c, slot_c)) {
    uint16_t* orow = p.expanded + (size_t)page_c * page_elems + (size_t)G * BS * 2 * DH + (kind_v ? BS * DH : 0) +
                     (size_t)slot_c * DH + d0;
#pragma unroll
    for (int m = 0; m < MTW; ++m) {
      const int mt = w * MTW + m;
      if (mt >= MTC) break;
      u32x2 pk = {pack_bf16x2(acc[m][0], acc[m][1]), pack_bf16x2(acc[m][2], acc[m][3])};
      *reinterpret_cast<u32x2*>(orow + 16 * mt + 4 * q) = pk;
    }
    if (G == 0 && !kind_v && hsel == 0 && w == 0) {   // the token's latent row and shared rope key
      uint16_t* rope = p.expanded + (size_t)page_c * page_elems + (size_t)g * BS * 2 * DH + (size_t)slot_c * DR;
      const uint16_t* src = p.new_rows + (size_t)tok_c * ROW;
      uint16_t* lat = p.latent + ((size_t)page_c * BS + slot_c) * ROW;
      for (int part = q; part < DR / 8; part += 4)
        *reinterpret_cast<u32x4*>(rope + 8 * part) = *reinterpret_cast<const u32x4*>(src + R + 8 * part);
      for (int part = q; part < ROW / 8; part += 4)
        *reinterpret_cast<u32x4*>(lat + 8 * part) = *reinterpret_cast<const u32x4*>(src + 8 * part);
    }
  }
}

hipError_t append_launch(const AppendParams& p, int r, int dn, int dv, int dr, hipStream_t stream, bool* supported) {
  *supported = true;
  if (!p.expanded) {                              // latent rows only
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)(p.batch * p.n_new)), dim3(64), 0, stream, p);
    return hipGetLastError();
  }
  // one launch: the expansion workgroups of group 0 also write the latent rows
  const unsigned tiles = (unsigned)((p.batch * p.n_new + 15) / 16);
  if (r == 512 && dn == 128 && dv == 128 && dr == 64) {
    hipLaunchKernelGGL((expand_tokens_kernel<512, 128, 64>), dim3(tiles * 2u * (unsigned)p.num_groups * 2u),
                       dim3(256), 0, stream, p);
  } else if (r == 64 && dn == 32 && dv == 32 && dr == 16) {
    hipLaunchKernelGGL((expand_tokens_kernel<64, 32, 16>), dim3(tiles * 2u * (unsigned)p.num_groups),
                       dim3(256), 0, stream, p);
  } else {
    *supported = false;
    return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace gqla
