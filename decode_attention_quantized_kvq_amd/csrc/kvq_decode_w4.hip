// Decode kernels of 4-bit values with per-token scales (uint4 / uint4 with
// fp16 scale and zero point, int4 / int4 and int8 / int4 with fp32 scales):
// instantiations of kvq_decode_kernel.h (the kernels are described in
// kvq_decode.hip).
#include "kvq_decode_kernel.h"

namespace kvq {

bool launch_decode_w4(const DecodeArgs& a, hipStream_t s, hipError_t* e) {
  const TensorKind k = a.kk, v = a.vk;
  if (k.code == CK_U4 && k.meta == MK_F16Z && v.code == CK_U4 && v.meta == MK_F16Z) {
    *e = launch_g<CK_U4, MK_F16Z, false, CK_U4, MK_F16Z>(a, s);
    return true;
  }
  if (k.code == CK_I4 && k.meta == MK_F32 && v.code == CK_I4 && v.meta == MK_F32) {
    *e = launch_g<CK_I4, MK_F32, false, CK_I4, MK_F32>(a, s);
    return true;
  }
  if (k.code == CK_I8 && k.meta == MK_F32 && v.code == CK_I4 && v.meta == MK_F32) {
    *e = launch_g<CK_I8, MK_F32, false, CK_I4, MK_F32>(a, s);
    return true;
  }
  return false;
}

}  // namespace kvq
