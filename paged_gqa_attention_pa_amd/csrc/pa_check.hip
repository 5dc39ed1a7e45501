// Device-side input checks (pa_check_inputs): the block tables, context
// lengths and query starts a compute call would read, checked against the
// problem's host bounds and the pool size.  The attention and append kernels
// trust these values (they only clamp, to stay inside the table and the
// workspace); this pass reports what is wrong instead.
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kCheckThreads = 256;

__global__ void check_clear_kernel(int32_t* flags) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0;
}

// Workgroup x = sequence x / chunks, block-table entries
// [256 * (x % chunks), +256) of its row.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckParams p) {
  const int s = blockIdx.x / p.chunks;
  const int c = blockIdx.x % p.chunks;
  const int L = p.context_lens[s];
  const int64_t nblk = L > 0 ? (((int64_t)L - 1) >> p.log2_page) + 1 : 0;
  const int64_t used = nblk < p.max_blocks ? nblk : p.max_blocks;
  int32_t bits = 0;
  const int64_t idx = (int64_t)c * kCheckThreads + threadIdx.x;
  if (idx < used) {
    const int32_t page = p.block_tables[(int64_t)s * p.max_blocks + idx];
    if (page < 0 || page >= p.num_pages) bits |= PA_CHECK_PAGE;
  }
  if (c == 0 && threadIdx.x == 0) {
    if (L < 0 || L > p.max_context_len) bits |= PA_CHECK_CONTEXT_BOUND;
    if (nblk > p.max_blocks) bits |= PA_CHECK_CONTEXT_BLOCKS;
    int qlen = 1;
    if (p.query_start_loc) {
      const int q0 = p.query_start_loc[s], q1 = p.query_start_loc[s + 1];
      if ((s == 0 && q0 != 0) || q1 < q0 || (s == p.num_seqs - 1 && q1 != p.total_tokens))
        bits |= PA_CHECK_QUERY_STARTS;
      qlen = q1 - q0;
    }
    if (qlen > p.max_query_len) bits |= PA_CHECK_QUERY_LEN;
    if (qlen > 0 && qlen > L) bits |= PA_CHECK_CONTEXT_SHORT;
  }
  if (bits) atomicOr(p.flags, bits);
}

}  // namespace

hipError_t launch_check(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(64), 0, stream, p.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.num_seqs == 0) return e;
  const int64_t grid = (int64_t)p.num_seqs * p.chunks;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(check_kernel, dim3((unsigned)grid), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
