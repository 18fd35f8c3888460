// fp32 instantiations of the attention kernels.
#include "dispatch.hpp"

ATL_DEFINE_TYPE_OPS(float, ops_f32)
