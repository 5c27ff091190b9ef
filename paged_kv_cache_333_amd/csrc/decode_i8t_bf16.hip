// Instantiates the decode kernels over int8 pools with a scale per (token, KV
// head) and bf16 queries (every head_dim, block size, heads per workgroup,
// single/split) in a translation unit of its own.
#include "decode_kernel.hpp"

namespace pa {

hipError_t dispatch_i8t_bf16(const LaunchOp& op, bool split, bool append, int d, int bs, int gt) {
  return dispatch_t<TBF16, TI8T>(op, split, append, d, bs, gt);
}

hipError_t occupancy_i8t_bf16(int* per_cu, int d, int bs, int gt) {
  return occupancy_t<TBF16, TI8T>(per_cu, d, bs, gt);
}

}  // namespace pa
