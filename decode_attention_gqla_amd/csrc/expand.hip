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
    hipLaunchKernelGGL((expand_kernel<512, 128, 64>), dim3(grid), dim3(256), 0, stream, p);
  } else if (r == 64 && dn == 32 && dv == 32 && dr == 16) {
    hipLaunchKernelGGL((expand_kernel<64, 32, 16>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    *supported = false;
    return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace gqla
