// swa_debug.hip — test hooks that run the device index functions of
// swa_device.hpp over caller arrays, so that the integer conventions can be
// compared bit-exactly with the oracle:
//  * slot_of is the slot map itself: the cache-write kernel, the decode
//    kernel's store of the new entry and the generic prefill kernel call it;
//  * key_in_set is the key set A(i) written as one predicate; only this hook
//    calls it.  The fast prefill kernel applies the same set as interval
//    bounds (a closed-form tile range and one interval test per key), the
//    fast decode kernel as the range of live slots, and the generic kernels
//    as loop bounds; the key-count tests (scale ~ 0, exp(lse) = |A(i)|)
//    check those end to end against the closed form.
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
  if (t < n) mask[t] = key_in_set(q_pos, k_pos[t], sh.W, sh.n_sink, sh.dil) ? 1 : 0;
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
