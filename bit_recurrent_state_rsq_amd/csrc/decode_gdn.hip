// Decode-step kernel instances for the gdn row of Table 1.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_gdn(int cl, int feat, int spec) { return decode_pick_cl<kGDN>(cl, feat, spec); }
DecodeFn decode_boost_twin(DecodeFn fn) { return decode_pick_boost<kGDN, 4>(fn); }
}  // namespace rsq
