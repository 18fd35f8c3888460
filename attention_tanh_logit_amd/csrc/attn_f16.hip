// fp16 instantiations of the attention kernels (the generic kernels).
#include "dispatch.hpp"

ATL_DEFINE_TYPE_OPS(atl::f16, ops_f16)
