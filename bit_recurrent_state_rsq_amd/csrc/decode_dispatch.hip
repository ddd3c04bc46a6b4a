// Decode kernel selection by model.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_kernel_for(int model, int cl, int feat, int spec) {
  switch (model) {
    case kRetNet: return decode_retnet(cl, feat, spec);
    case kMamba2: return decode_mamba2(cl, feat, spec);
    case kGLA: return decode_gla(cl, feat, spec);
    default: return decode_gdn(cl, feat, spec);
  }
}
}  // namespace rsq
