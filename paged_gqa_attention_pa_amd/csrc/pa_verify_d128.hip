// Short-run kernels at head dim 128 (instantiations; see pa_verify_kernels.h).
#include "pa_verify_kernels.h"

namespace pa {
namespace verify_detail {

const void* verify_ptr_d128(int group, int rb, bool precise) {
  return precise ? by_group<true, 128>(group, rb) : by_group<false, 128>(group, rb);
}

}  // namespace verify_detail
}  // namespace pa
