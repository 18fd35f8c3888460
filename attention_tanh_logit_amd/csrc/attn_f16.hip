// fp16: the bf16 kernels compiled a second time with fp16 as their 16-bit
// element type (fp16 MFMA and dot instructions; the forward keeps a running
// row maximum, since probabilities taken relative to the cap could leave
// fp16's exponent range).  Everything here lives in namespace atl_f16; the
// library reaches it through the untyped entry points at the end, whose
// argument structs have the same layout as the library's own.
#define ATL_FAST_F16 1
#define ATL_NS atl_f16
#include "dispatch.hpp"

ATL_DEFINE_TYPE_OPS(atl_f16::bf16, ops_f16)

namespace atl_f16_bridge {
using namespace atl_f16;
hipError_t fwd(int D, bool cap, bool bias, const void* p, const void* l) {
  return ops_f16().fwd(D, cap, bias, *static_cast<const FwdParams*>(p), *static_cast<const Launch*>(l));
}
hipError_t dq(int D, bool cap, bool bias, const void* p, const void* l) {
  return ops_f16().dq(D, cap, bias, *static_cast<const BwdParams*>(p), *static_cast<const Launch*>(l));
}
hipError_t dkdv(int D, bool cap, bool bias, const void* p, const void* l) {
  return ops_f16().dkdv(D, cap, bias, *static_cast<const BwdParams*>(p), *static_cast<const Launch*>(l));
}
hipError_t pre(int D, const void* out, const void* out_lo, const void* dout, const float* lse, float* delta,
               float* part, const float* sink, int sink_mode, int Hq, int rpb, const void* l) {
  return ops_f16().pre(D, out, out_lo, dout, lse, delta, part, sink, sink_mode, Hq, rpb, *static_cast<const Launch*>(l));
}
hipError_t dbias_fill(void* dbias, const void* m, int Hq, int rpb, const void* l) {
  return ops_f16().dbias_fill(dbias, *static_cast<const Mask*>(m), Hq, rpb, *static_cast<const Launch*>(l));
}
hipError_t dbias_reduce(const void* full, void* out, int Hq, int bcast, const void* part, int D, const void* l) {
  return ops_f16().dbias_reduce(full, out, Hq, bcast, static_cast<const Mask*>(part), D,
                                *static_cast<const Launch*>(l));
}
}  // namespace atl_f16_bridge
