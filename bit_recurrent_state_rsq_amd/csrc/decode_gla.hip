// Decode-step kernel instances for the gla row of Table 1.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_gla(int cl, int feat, int spec) { return decode_pick_cl<kGLA>(cl, feat, spec); }
}  // namespace rsq
