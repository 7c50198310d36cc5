// Split-KV log-sum-exp merge.
//
// The GQLA pages do not discuss splitting the context; the merge is the exact
// decomposition of a softmax over disjoint token ranges: with per-split
// normalised outputs o_s and log-sum-exps lse_s,
//   m = max_s lse_s,  w_s = exp(lse_s - m),
//   out = sum_s w_s o_s / sum_s w_s,   lse = m + log(sum_s w_s).
// Splits with lse = -inf (no visible token) carry weight 0.
//
// One thread per 4 consecutive output dims of one (sequence, row); a row of
// d_v dims is d_v/4 adjacent threads, so every split partial row is read with
// fully coalesced 16-byte loads.  The lse values and partial rows of up to SC
// splits are loaded together (one memory latency per batch of splits, not one
// per split); a later batch with a larger maximum rescales what is summed.
// With at most SC splits the sums are formed in split order exactly as in
// the formula above.
#include "common.hip.h"
#include "params.hip.h"

namespace gqla {

template <int DV>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int TPR = DV / 4;                      // threads per row
  constexpr int SC = 8;                            // splits per load batch
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const int gr = tid / TPR;                         // global row = b * rows + r
  const int part = tid % TPR;
  if (gr >= p.batch * p.rows) return;
  const int b = gr / p.rows, r = gr % p.rows;
  const int s0 = p.split_offsets[b], s1 = p.split_offsets[b + 1];

  float m = -INFINITY, z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sb = s0; sb < s1; sb += SC) {
    float ls[SC];
    f32x4 v[SC];
#pragma unroll
    for (int k = 0; k < SC; ++k) {
      const bool have = sb + k < s1;
      const size_t row = (size_t)(have ? sb + k : s0) * p.rows + r;
      ls[k] = have ? p.part_lse[row] : -INFINITY;
      v[k] = have ? *reinterpret_cast<const f32x4*>(p.part_out + row * DV + 4 * part) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bm = ls[0];
#pragma unroll
    for (int k = 1; k < SC; ++k) bm = fmaxf(bm, ls[k]);
    const float mn = fmaxf(m, bm);
    if (mn == -INFINITY) continue;                  // no visible token so far
    if (m != -INFINITY && m != mn) {
      const float sc = expf(m - mn);
      acc *= sc;
      z *= sc;
    }
    m = mn;
#pragma unroll
    for (int k = 0; k < SC; ++k) {
      if (ls[k] == -INFINITY) continue;             // empty split (its partial row may hold anything)
      const float w = expf(ls[k] - m);
      acc += w * v[k];
      z += w;
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const f32x4 o = acc * inv;
  u32x2 pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
  *reinterpret_cast<u32x2*>(p.out + (size_t)gr * DV + 4 * part) = pk;
  if (part == 0 && p.lse) p.lse[gr] = z > 0.f ? m + logf(z) : -INFINITY;
}

hipError_t combine_dispatch(int dv, const CombineParams& p, hipStream_t stream, bool* supported) {
  *supported = true;
  const long threads_per_row = dv / 4;
  const long total = (long)p.batch * p.rows * threads_per_row;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (grid == 0) return hipSuccess;
  if (dv == 128) {
    hipLaunchKernelGGL(combine_kernel<128>, dim3(grid), dim3(256), 0, stream, p);
  } else if (dv == 32) {
    hipLaunchKernelGGL(combine_kernel<32>, dim3(grid), dim3(256), 0, stream, p);
  } else {
    *supported = false;
    return hipSuccess;
  }
  return hipGetLastError();
}

}  // namespace gqla
