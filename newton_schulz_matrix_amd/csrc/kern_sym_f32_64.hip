// kern_sym_f32_64.hip - kernel builds of the symmetric-result products for one operand type and tile
// edge (see plan.hpp).
#define NS_KERNEL_UNIT
#include "plan.hpp"

namespace nsr {

NS_SYM_LAUNCHERS(float, 64)

}  // namespace nsr
