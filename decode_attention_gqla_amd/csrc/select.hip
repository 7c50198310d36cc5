// Path selector: the pages' roofline model applied to one decode call of each
// path (host code only).
//
// GQLA pages: paperlayer.ai summary, section 4 "Roofline analysis" (time =
// max(bytes / BW, FLOPs / peak); intensities of the absorb and GQA paths) and
// "Hardware operating points" (the path whose intensity sits at or below the
// ridge wins); gist.science section 2 "Pfadauswahl".  Counting convention:
// bf16 operands (2 bytes), each moved once; 2 FLOPs per multiply-accumulate;
// QK over d_nope + d_rope (GQA) or d_latent + d_rope (absorb) and PV over d_v
// or d_latent; query row i of a sequence of length L sees L - s_q + i + 1
// tokens.
#include <cmath>

#include "gqla.h"

namespace {

struct Counts {
  double cache = 0, bytes = 0, flops = 0;
};

// Total visible (row, token) pairs of one head over the batch.
double visible_pairs(const int32_t* lens, int batch, int s_q) {
  double n = 0;
  for (int b = 0; b < batch; ++b)
    for (int i = 0; i < s_q; ++i) n += (double)(lens[b] - s_q + i + 1);
  return n;
}

Counts count_absorb(const gqla_dims& d, const int32_t* lens, int batch, int s_q, bool cache_only) {
  const double H = d.num_heads, g = d.num_groups, r = d.d_latent, dr = d.d_rope, dn = d.d_nope, dv = d.d_v;
  double tokens = 0;
  for (int b = 0; b < batch; ++b) tokens += lens[b];
  Counts c;
  c.cache = tokens * (r + dr) * 2;
  c.flops = visible_pairs(lens, batch, s_q) * H * 2 * (2 * r + dr);
  c.bytes = c.cache;
  if (!cache_only) {
    c.bytes += batch * s_q * H * (dn + dr) * 2      // q_nope, q_rope
             + g * r * (dn + dv) * 2                // W_UK, W_UV
             + batch * s_q * H * dv * 2;            // out
    c.flops += 2.0 * batch * s_q * H * r * (dn + dv);   // q absorption and up-projection
  }
  return c;
}

Counts count_gqa(const gqla_dims& d, const int32_t* lens, int batch, int s_q, bool cache_only) {
  const double H = d.num_heads, g = d.num_groups, dr = d.d_rope, dn = d.d_nope, dv = d.d_v;
  double tokens = 0;
  for (int b = 0; b < batch; ++b) tokens += lens[b];
  Counts c;
  c.cache = tokens * (g * (dn + dv) + dr) * 2;
  c.flops = visible_pairs(lens, batch, s_q) * H * 2 * (dn + dr + dv);
  c.bytes = c.cache;
  if (!cache_only) c.bytes += batch * s_q * H * (dn + dr) * 2 + batch * s_q * H * dv * 2;
  return c;
}

gqla_path_estimate estimate(const Counts& c, const gqla_hw& hw, double frac, int batch, int s_q) {
  gqla_path_estimate e;
  e.bytes = c.bytes;
  e.flops = c.flops;
  e.t_hbm_us = c.bytes / (hw.hbm_gbps * 1e9) * 1e6;
  e.t_mfma_us = c.flops / (hw.mfma_tflops * 1e12) * 1e6;
  e.bound = e.t_mfma_us > e.t_hbm_us ? 1 : 0;
  e.t_roofline_us = e.bound ? e.t_mfma_us : e.t_hbm_us;
  e.t_expected_us = e.t_roofline_us / frac;
  e.tokens_per_s = (double)batch * s_q / (e.t_expected_us * 1e-6);
  return e;
}

}  // namespace

extern "C" int gqla_select_path(const gqla_dims* d, int32_t batch, const int32_t* lens,
                                int32_t s_q_absorb, int32_t s_q_gqa, const gqla_hw* hw,
                                gqla_path_estimate* absorb, gqla_path_estimate* gqa) {
  if (!d || !hw || !lens || batch < 1) return GQLA_ERR_INVALID_ARG;
  if (s_q_absorb < 1 || s_q_absorb > 2 || s_q_gqa < 1 || s_q_gqa > 2) return GQLA_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || d->num_groups <= 0 || d->num_heads % d->num_groups != 0 || d->d_latent <= 0 ||
      d->d_rope < 0 || d->d_nope <= 0 || d->d_v <= 0)
    return GQLA_ERR_INVALID_ARG;
  if (!(hw->hbm_gbps > 0) || !(hw->mfma_tflops > 0) || !(hw->frac_absorb > 0) || !(hw->frac_absorb <= 1) ||
      !(hw->frac_gqa > 0) || !(hw->frac_gqa <= 1))
    return GQLA_ERR_INVALID_ARG;
  const int smax = s_q_absorb > s_q_gqa ? s_q_absorb : s_q_gqa;
  for (int b = 0; b < batch; ++b)
    if (lens[b] < smax) return GQLA_ERR_INVALID_ARG;
  const bool co = hw->cache_only != 0;
  const gqla_path_estimate ea = estimate(count_absorb(*d, lens, batch, s_q_absorb, co), *hw, hw->frac_absorb, batch, s_q_absorb);
  const gqla_path_estimate eg = estimate(count_gqa(*d, lens, batch, s_q_gqa, co), *hw, hw->frac_gqa, batch, s_q_gqa);
  if (absorb) *absorb = ea;
  if (gqa) *gqa = eg;
  return eg.tokens_per_s > ea.tokens_per_s ? GQLA_PATH_GQA : GQLA_PATH_ABSORB;
}
