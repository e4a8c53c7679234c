// swa_debug.hip — test hooks that run the device index functions the kernels
// use (slot map of the rolling buffer, key-set predicate) over caller arrays,
// so that integer conventions can be compared bit-exactly with the oracle.
#include "swa_device.hpp"
#include "swa_launch.hpp"

namespace swa {
namespace {

__global__ void debug_slots_kernel(Shape sh, const int32_t* pos, int n, int32_t* slots) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) slots[t] = slot_of(pos[t], sh.W, sh.n_sink);
}

__global__ void debug_mask_kernel(Shape sh, int q_pos, const int32_t* k_pos, int n, uint8_t* mask) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) mask[t] = key_in_set(q_pos, k_pos[t], sh.W, sh.n_sink) ? 1 : 0;
}

}  // namespace

hipError_t launch_debug_slots(const Shape& sh, const int32_t* pos, int n, int32_t* slots,
                              hipStream_t st) {
  debug_slots_kernel<<<(n + 255) / 256, 256, 0, st>>>(sh, pos, n, slots);
  return hipGetLastError();
}

hipError_t launch_debug_mask(const Shape& sh, int q_pos, const int32_t* k_pos, int n,
                             uint8_t* mask, hipStream_t st) {
  debug_mask_kernel<<<(n + 255) / 256, 256, 0, st>>>(sh, q_pos, k_pos, n, mask);
  return hipGetLastError();
}

}  // namespace swa
