// Debug aid: a device-side check of the lengths and block-table entries a
// decode-attention call would read. The attention kernels clamp both (a
// length to [0, max_ctx_len], a block id to [0, num_blocks)) so that no access
// leaves the cache tensors; a corrupt table is then read silently as the
// nearest valid block. This kernel reports such entries instead.
#include <hip/hip_runtime.h>

#include "ops_internal.h"

namespace dfa {

namespace {
constexpr int kCheckThreads = 1024;
}

// One workgroup scans every sequence: lane-parallel over the entries of each
// row, flags gathered in LDS and written once at the end (so the output needs
// no clearing beforehand and the result does not depend on timing).
__global__ __launch_bounds__(kCheckThreads) void check_table_kernel(TableCheckParams p) {
  __shared__ uint32_t bits, first;
  if (threadIdx.x == 0) {
    bits = 0;
    first = 0xFFFFFFFFu;
  }
  __syncthreads();
  for (int b = 0; b < p.batch; ++b) {
    const int len = p.ctx[b] + p.ctx_add;  // the same read the attention kernels make
    uint32_t mine = 0;
    if (len < 0 || len > p.max_ctx) mine |= kTableBadLen;
    const int lc = len < 0 ? 0 : (len > p.max_ctx ? p.max_ctx : len);
    const int nb = (lc + p.block_size - 1) / p.block_size;  // entries the kernels read for this sequence
    const int32_t* row = p.table + (size_t)b * p.max_blocks;
    for (int j = threadIdx.x; j < nb; j += kCheckThreads) {
      const int blk = row[j];
      if (blk < 0 || blk >= p.num_blocks) mine |= kTableBadBlock;
    }
    if (mine) {
      atomicOr(&bits, mine);
      atomicMin(&first, (uint32_t)b);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.flags[0] = bits;
    p.flags[1] = first;
  }
}

hipError_t launch_check_table(const TableCheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_table_kernel, dim3(1), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace dfa
