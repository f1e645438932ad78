// Decode kernels of per-channel int8 keys with 8-bit value scale codes, and
// uint8 / uint8 with fp16 scale and zero point: instantiations of
// kvq_decode_kernel.h (the kernels are described in kvq_decode.hip).
#include "kvq_decode_kernel.h"

namespace kvq {

bool launch_decode_mixed(const DecodeArgs& a, hipStream_t s, hipError_t* e) {
  const TensorKind k = a.kk, v = a.vk;
  if (k.code == CK_I8 && k.channel && v.code == CK_I4 && v.meta == MK_U8) {
    *e = launch_g<CK_I8, MK_NONE, true, CK_I4, MK_U8>(a, s);
    return true;
  }
  if (k.code == CK_U8 && k.meta == MK_F16Z && v.code == CK_U8 && v.meta == MK_F16Z) {
    *e = launch_g<CK_U8, MK_F16Z, false, CK_U8, MK_F16Z>(a, s);
    return true;
  }
  return false;
}

}  // namespace kvq
