// Translation unit of the main MQA-absorb decode kernel (absorb_wide.hip.h).
#include "absorb_wide.hip.h"

namespace gqla {

// Copy instructions of each tile issued by each QK wave; the PV waves issue
// the rest.  Measured on the DeepSeek-V3-shaped batch (64 x 4096 tokens,
// 2048-token splits): 76.6 us with all copies in the PV waves, 83.4 us with 5
// of 9 per QK wave, 85.5 us with all in the QK waves (their MFMA chain is the
// longer one).
#ifndef GQLA_ABSORB_QK_COPIES
#define GQLA_ABSORB_QK_COPIES 0
#endif
constexpr int kAbsorbQkCopies = GQLA_ABSORB_QK_COPIES;

// The shapes with 512 + 64 latent rows and nope = v = 128 whose query rows per
// sequence are a multiple of 64; *handled = false for the others.
hipError_t absorb_wide_dispatch(int hpg, int sq, const DecodeParams& p, hipStream_t stream, bool* handled) {
  *handled = true;
#define GQLA_WIDE_CASE(HPG, SQ) \
  if (hpg == HPG && sq == SQ) return launch_absorb_wide<HPG, SQ, 512, 64, kAbsorbQkCopies>(p, stream);
  GQLA_WIDE_CASE(16, 1)
  GQLA_WIDE_CASE(16, 2)
  GQLA_WIDE_CASE(32, 1)
  GQLA_WIDE_CASE(32, 2)
  GQLA_WIDE_CASE(4, 2)
#undef GQLA_WIDE_CASE
  *handled = false;
  return hipSuccess;
}

}  // namespace gqla
