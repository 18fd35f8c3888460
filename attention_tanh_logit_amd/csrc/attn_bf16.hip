// bf16 instantiations of the attention kernels.
#include "dispatch.hpp"

ATL_DEFINE_TYPE_OPS(atl::bf16, ops_bf16)
