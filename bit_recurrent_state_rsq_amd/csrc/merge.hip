// Low-Rank Bypass merge (placeholder until the merge kernel lands).
#include "rsq_kernels.hpp"

namespace rsq {
DecodeFn merge_kernel_for(int /*cl*/) { return nullptr; }
}  // namespace rsq
