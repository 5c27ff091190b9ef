// Instantiates the decode kernels over 8-bit e4m3 pools with bf16 queries
// (every head_dim, block size, heads per workgroup, single/split) in a
// translation unit of its own.
#include "decode_kernel.hpp"

namespace pa {

hipError_t dispatch_e4m3_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt) {
  return dispatch_t<TBF16, TE4M3>(op, split, append, d, bs, gt);
}

hipError_t occupancy_e4m3_bf16(int* per_cu, int d, int bs, int gt) {
  return occupancy_t<TBF16, TE4M3>(per_cu, d, bs, gt);
}

}  // namespace pa
