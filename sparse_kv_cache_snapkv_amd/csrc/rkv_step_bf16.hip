// Instantiations of the fused decode step for bfloat16 caches (rkv_step.hpp).
#include "rkv_step.hpp"

namespace rkv {

hipError_t step_launch_bf16(int D, int G, const step::Args& a, hipStream_t stream) {
  return D == 64 ? step::launch_d<bf16_t, 64>(G, a, stream)
                 : step::launch_d<bf16_t, 128>(G, a, stream);
}

}  // namespace rkv
