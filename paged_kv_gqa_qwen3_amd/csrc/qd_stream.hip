// Batch-1 streaming step kernel: instantiation, LDS sizing and launch.
#include "qd_stream.h"

namespace qd {

size_t stream_lds_bytes(int head_dim, int group, int in_floats, int rt_max) {
  if (head_dim == 128 && group == 4) return stream_lds_bytes_t<128, 4>(in_floats, rt_max);
  if (head_dim == 64 && group == 2) return stream_lds_bytes_t<64, 2>(in_floats, rt_max);
  return 0;
}

static const void* stream_fn(int head_dim, int group) {
  if (head_dim == 128 && group == 4) return reinterpret_cast<const void*>(&stream_step_kernel<128, 4>);
  if (head_dim == 64 && group == 2) return reinterpret_cast<const void*>(&stream_step_kernel<64, 2>);
  return nullptr;
}

hipError_t stream_max_grid(int head_dim, int group, size_t lds, int num_cus, int* grid) {
  const void* fn = stream_fn(head_dim, group);
  if (fn == nullptr) return hipErrorInvalidValue;
  *grid = 0;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds);
  if (e != hipSuccess) return e;
  *grid = per_cu * num_cus;
  return hipSuccess;
}

hipError_t launch_stream(const StreamArgs& a, int head_dim, int group, int grid, size_t lds,
                         hipStream_t s) {
  const void* fn = stream_fn(head_dim, group);
  if (fn == nullptr) return hipErrorInvalidValue;
  void* args[] = {const_cast<StreamArgs*>(&a)};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(256), args, (unsigned)lds, s);
}

}  // namespace qd
