// Decode-step kernel instances for the retnet row of Table 1.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_retnet(int cl, int feat, int spec) { return decode_pick_cl<kRetNet>(cl, feat, spec); }
}  // namespace rsq
