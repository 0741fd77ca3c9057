// The gate_up and down launches with full double-buffered stages (items of
// more than 16 tokens of blocks below 8 bits; every 128-token gate_up item
// below 8 bits). Kernels and launcher: k_ffn_kernels.h.
#include "k_ffn_kernels.h"

namespace mpb {

hipError_t launch_gate_up_df(const FfnParams& p, int qmax, int tc, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  switch (tc) {
    case 1: return launch_tc<1, true, true, true>(p, qmax, s, ev0, ev1);
    case 4: return launch_tc<4, true, false, true>(p, qmax, s, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_down_df(const FfnParams& p, int qmax, bool nt, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
  return nt ? launch_tc<1, false, true, true>(p, qmax, s, ev0, ev1) : launch_tc<1, false, false, true>(p, qmax, s, ev0, ev1);
}

}  // namespace mpb
