// Decode kernel selection by model.
#include "decode_impl.hpp"

namespace rsq {
DecodeFn decode_kernel_for(int model, int cl, int feat) {
  switch (model) {
    case kRetNet: return decode_retnet(cl, feat);
    case kMamba2: return decode_mamba2(cl, feat);
    case kGLA: return decode_gla(cl, feat);
    default: return decode_gdn(cl, feat);
  }
}
}  // namespace rsq
