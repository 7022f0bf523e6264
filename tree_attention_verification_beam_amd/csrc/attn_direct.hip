// attn_direct.hip -- the direct-to-LDS plan of the bf16 tree attention (wide
// GQA groups at D = 128: 128-row blocks of 4 waves, K/V tiles loaded straight
// into LDS, the next tile's scores beside this tile's softmax).  It has a
// compile unit of its own because the build compiles this one with the
// backend's max-ilp scheduling strategy, which orders this kernel's loop
// better than the default and the register-staged plans' loops worse.
#include "attn_bf16.hpp"

namespace spec {
namespace attn {

int launch_direct(bool once, int n_slots, const AttnArgs& args, hipStream_t s) {
  return once ? launch_main<128, 4, 2, 1, 2, 2, true>(n_slots, args, s)
              : launch_main<128, 4, 2, 1, 2, 2, false>(n_slots, args, s);
}

}  // namespace attn
}  // namespace spec
