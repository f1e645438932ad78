// Decode kernels of 2-bit codes (int2 with fp32 scales or 8-bit scale codes,
// uint2 with fp16 scale and zero point): instantiations of kvq_decode_kernel.h
// (the kernels are described in kvq_decode.hip).
#include "kvq_decode_kernel.h"

namespace kvq {

bool launch_decode_w2(const DecodeArgs& a, hipStream_t s, hipError_t* e) {
  const TensorKind k = a.kk, v = a.vk;
  if (k.code == CK_I2 && k.meta == MK_F32 && v.code == CK_I2 && v.meta == MK_F32) {
    *e = launch_g<CK_I2, MK_F32, false, CK_I2, MK_F32>(a, s);
    return true;
  }
  if (k.code == CK_I2 && k.meta == MK_U8 && v.code == CK_I2 && v.meta == MK_U8) {
    *e = launch_g<CK_I2, MK_U8, false, CK_I2, MK_U8>(a, s);
    return true;
  }
  if (k.code == CK_U2 && k.meta == MK_F16Z && v.code == CK_U2 && v.meta == MK_F16Z) {
    *e = launch_g<CK_U2, MK_F16Z, false, CK_U2, MK_F16Z>(a, s);
    return true;
  }
  return false;
}

}  // namespace kvq
