// kern_nt_f16_128.hip - kernel builds of the updates for one operand type and tile
// edge (see plan.hpp).
#define NS_KERNEL_UNIT
#include "plan.hpp"

namespace nsr {

NS_NT_LAUNCHER(_Float16, _Float16, 128)
NS_NT_LAUNCHER(_Float16, __bf16, 128)

}  // namespace nsr
