// Dequantize-into-temporary-storage path of libkvq (gfx950).
//
// One layer of a quantized cache written out as bf16 keys and values in
// position order, the alternative to dequantizing inside the attention
// kernel that [P1] "KV Cache Quantization Perturbs Attention Through Stored
// Keys and Values", section "Cache growth changes the serving trade", names
// (dequantization fused into the attention kernel or performed into
// temporary storage); [P2] "KV cache quantization reduces cache bytes with
// separate accuracy and kernel costs", section "Lower payload does not imply
// proportional latency reduction", lists what the conversion costs.  The
// decode kernels then read the bf16 copy as an unquantized cache.
//
// Each value is the exact product code x scale (or scale x (code - zero),
// code x u x S, code x channel scale) rounded once to bf16; bf16 window and
// open-group tokens are copied.  Positions of a middle tier are its int8
// codes times their fp32 scales.

#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_quantize.h"

namespace kvq {
namespace {

constexpr int D = 128;

// The exact product c * s (c an integer of at most 15 bits, s fp32) rounded
// once to bf16 (nearest, ties to even).  p = fl32(c s) and the exact rest
// e = c s - p (one fma) give the product rounded to odd in fp32 (24 >= 8 + 2
// bits, so rounding that to bf16 cannot round twice): step p toward zero if
// the rest points the other way, then set its last bit if inexact.
__device__ inline uint16_t bf16_of_product(float c, float s) {
  const float p = c * s;
  const float e = __builtin_fmaf(c, s, -p);
  uint32_t u = __float_as_uint(p);
  if (e != 0.0f) {
    if ((e < 0.0f) != (p < 0.0f)) u -= 1u;  // |c s| < |p|: the neighbour toward zero
    u |= 1u;                                // round to odd
  }
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline int bits_of(CodeKind c) {
  return (c == CK_I8 || c == CK_U8) ? 8 : (c == CK_I4 || c == CK_U4) ? 4 : 2;
}

__device__ inline bool signed_codes(CodeKind c) { return c == CK_I8 || c == CK_I4 || c == CK_I2; }

// The codes of the 8 features starting at f0 (a multiple of 8) of a token
// row, in one aligned load: feature f0 + e at bits [b e, b e + b).
__device__ inline uint64_t codes8(const uint8_t* row, int bits, int f0) {
  if (bits == 8) return *(const uint64_t*)(row + f0);
  if (bits == 4) return *(const uint32_t*)(row + f0 / 2);
  return *(const uint16_t*)(row + f0 / 4);
}

__device__ inline int code_of(uint64_t raw, int bits, bool sgn, int e) {
  const int m = (1 << bits) - 1;
  int c = (int)((raw >> (bits * e)) & (uint64_t)m);
  if (sgn && c > (m >> 1)) c -= m + 1;
  return c;
}

// Writes features [f0, f0 + 8) of position p (< the sequence's length) of
// (sequence, KV head) head, for K and for V.  Positions [0, na) hold the
// cache's format, [na, nq) the middle tier, the rest bf16.
__device__ inline void dequant_position(const DequantArgs& a, size_t head, int b, int h, int p,
                                        int na, int nq, int f0) {
  for (int w = 0; w < 2; ++w) {
    uint16_t* out = (w ? a.v_out : a.k_out) + (head * a.out_tokens + p) * D + f0;
    uint16_t o[8];
    if (p >= nq) {  // bf16 window / open token group: a copy
      const uint16_t* ring = w ? a.v_win : a.k_win;
      const uint16_t* src = ring + (head * a.ring + (p % a.ring)) * D + f0;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = src[e];
    } else if (p >= na) {  // middle tier: int8 codes, one fp32 scale
      const size_t ms = head * a.mid.slots + (p % a.mid.slots);
      const uint64_t raw = codes8((w ? a.mid.v : a.mid.k) + ms * D, 8, f0);
      const float s = (w ? a.mid.vs : a.mid.ks)[ms];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = bf16_of_product((float)code_of(raw, 8, true, e), s);
    } else {
      const TensorKind k = w ? a.vk : a.kk;
      const uint8_t* codes = w ? a.v_codes : a.k_codes;
      const uint8_t* row = qz::code_row(a, k, codes, b, h, p);
      // the metadata element of the token's group
      const uint8_t* me = k.channel ? nullptr
                                    : qz::meta_elem(a, k, w ? a.v_meta : a.k_meta, b, h, p);
      // value = cm * s with cm an integer: c, c - z, or c u (8-bit scale codes)
      float s = 1.0f, z = 0.0f, um = 1.0f;
      if (!k.channel) {
        if (k.meta == MK_F32) {
          s = ((const float*)me)[0];
        } else if (k.meta == MK_F32Z) {
          s = ((const float*)me)[0];
          z = ((const float*)me)[1];
        } else if (k.meta == MK_F16) {
          s = (float)((const _Float16*)me)[0];
        } else if (k.meta == MK_F16Z) {
          s = (float)((const _Float16*)me)[0];
          z = (float)((const _Float16*)me)[1];
        } else if (k.meta == MK_U8) {
          s = (w ? a.v_super : a.k_super)[head];
          um = (float)me[0];
        }
      }
      const int bits = bits_of(k.code);
      const bool sgn = signed_codes(k.code);
      const uint64_t raw = codes8(row, bits, f0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = (float)code_of(raw, bits, sgn, e);
        o[e] = k.channel ? bf16_of_product(c, a.k_chan[head * D + f0 + e])
                         : bf16_of_product((c - z) * um, s);
      }
    }
    uint4 v;
    v.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
    v.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
    v.z = (uint32_t)o[4] | ((uint32_t)o[5] << 16);
    v.w = (uint32_t)o[6] | ((uint32_t)o[7] << 16);
    *(uint4*)out = v;
  }
}

// Grid (ceil(out_tokens / TPW), H_kv, B), 256 threads: thread (t, f) writes
// features [8f, 8f + 8) of positions TPW blockIdx.x + 16 i + t (i = 0 ..
// TPW/16 - 1), for K and for V.  (Measured: 16 positions per workgroup ran
// faster than 128.)
constexpr int TPW = 16;

__global__ void __launch_bounds__(256) dequant_kernel(DequantArgs a) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x >> 4, f0 = (threadIdx.x & 15) * 8;
  int len = a.seq_lens[b];
  len = len > 0 ? len : 0;
  const int cap = (a.paged ? a.bt_stride * 16 : a.max_tokens) + a.window + a.mid.tokens;
  len = len < cap ? len : cap;
  const int lim = len < a.out_tokens ? len : a.out_tokens;
  const int m = len - a.window > 0 ? len - a.window : 0;
  const int nq = (m >> a.tgshift) << a.tgshift;  // quantized positions
  // of which the cache's format holds whole blocks of 32 older than the middle tier
  const int na = a.mid.tokens ? (nq - a.mid.tokens > 0 ? nq - a.mid.tokens : 0) / MID_BLOCK * MID_BLOCK
                              : nq;
  const size_t head = (size_t)b * a.hkv + h;
#pragma unroll 4
  for (int i = 0; i < TPW / 16; ++i) {
    const int p = blockIdx.x * TPW + 16 * i + t;
    if (p >= lim) break;
    dequant_position(a, head, b, h, p, na, nq, f0);
  }
}

}  // namespace

kvq_status launch_dequant(const DequantArgs& a, void* stream) {
  if (a.out_tokens <= 0) return KVQ_OK;
  const dim3 grid((unsigned)((a.out_tokens + TPW - 1) / TPW), a.hkv, a.batch);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, (hipStream_t)stream, a);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
