// Short-run kernels at head dim 64 (instantiations; see pa_verify_kernels.h).
#include "pa_verify_kernels.h"

namespace pa {
namespace verify_detail {

const void* verify_ptr_d64(int group, int rb, bool precise) {
  return precise ? by_group<true, 64>(group, rb) : by_group<false, 64>(group, rb);
}

}  // namespace verify_detail
}  // namespace pa
