// Instantiations of the fused decode step for float32 caches (rkv_step.hpp).
#include "rkv_step.hpp"

namespace rkv {

hipError_t step_launch_f32(int D, int G, const step::Args& a, hipStream_t stream) {
  return D == 64 ? step::launch_d<float, 64>(G, a, stream) : step::launch_d<float, 128>(G, a, stream);
}

}  // namespace rkv
