// Decode-step kernel instances for the retnet row of Table 1.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_retnet(int cl, int feat, int spec) { return decode_pick_cl<kRetNet>(cl, feat, spec); }
DecodeFn decode_stream_retnet(int cl, int spec, int bits) { return decode_stream_pick<kRetNet>(cl, spec, bits); }
}  // namespace rsq
