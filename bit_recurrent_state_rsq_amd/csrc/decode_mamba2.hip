// Decode-step kernel instances for the mamba2 row of Table 1.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_mamba2(int cl, int feat, int spec) { return decode_pick_cl<kMamba2>(cl, feat, spec); }
}  // namespace rsq
