// kern_nt_f32_64.hip - kernel builds of the updates for one operand type and tile
// edge (see plan.hpp).
#define NS_KERNEL_UNIT
#include "plan.hpp"

namespace nsr {

NS_NT_LAUNCHER(float, float, 64)

}  // namespace nsr
