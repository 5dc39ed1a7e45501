// Short-run kernels at head dim 256 (instantiations; see pa_verify_kernels.h).
#include "pa_verify_kernels.h"

namespace pa {
namespace verify_detail {

const void* verify_ptr_d256(int group, int rb, bool precise) {
  return precise ? by_group<true, 256>(group, rb) : by_group<false, 256>(group, rb);
}

}  // namespace verify_detail
}  // namespace pa
