// Device-side quantizer of one token group (codes and metadata), shared by
// the append kernels and the decode step that appends its new token itself.
// Both compile it from this header, so the two write the same bits.
#pragma once

#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace qz {

constexpr int QD = 128;

__device__ inline float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float f) {
  // Round to nearest, ties to even (inputs are finite).
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float load_in(const void* p, size_t idx, int bf16) {
  return bf16 ? bf16_bits_to_f32(((const uint16_t*)p)[idx]) : ((const float*)p)[idx];
}

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_min(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline double wave_max(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

__device__ inline double wave_min(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmin(v, __shfl_xor(v, o));
  return v;
}

// fp64 -> fp32 storage: one rounding, ties to even; 0 becomes 2^-149.
__device__ inline float store_f32(double v) {
  float f = (float)v;
  if (f == 0.0f) f = __uint_as_float(1u);
  return f;
}

// fp64 -> fp16 with a single rounding (ties to even): round to odd into fp32
// first (24 >= 11 + 2 bits, so the second rounding cannot double-round), then
// let the hardware convert fp32 -> fp16 to nearest even.
__device__ inline uint16_t f64_to_f16_bits(double x) {
  float f = (float)x;
  if ((double)f != x) {
    uint32_t u = __float_as_uint(f);
    if (fabs((double)f) > fabs(x)) u -= 1u;  // the fp32 value toward zero
    u |= 1u;                                 // its odd neighbour: round to odd
    f = __uint_as_float(u);
  }
  const _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// fp64 (positive) -> fp16 storage of a scale: 0 becomes 2^-24, overflow 65504.
__device__ inline uint16_t store_f16(double v) {
  uint16_t h = f64_to_f16_bits(v);
  if ((h & 0x7FFFu) == 0) h = 0x0001u;
  if ((h & 0x7FFFu) >= 0x7C00u) h = 0x7BFFu;
  return h;
}

__device__ inline double f16_bits_to_f64(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}

__device__ inline int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Where position p of (sequence b, KV head h) lives, for a tensor of kind k
// (Args: any of the launch argument structs, which name the layout fields
// alike).  Contiguous: token slot s = (b H_kv + h) max_tokens + p, code row
// at codes + s row, metadata element s >> gs at meta.  Paged: unit u =
// block_table[b][p / 16] H_kv + h (the entry clamped into the pool), code row
// p mod 16 of the tensor's unit u; the metadata elements of both tensors in
// the key unit u, after its 16 rows (at offset k.moff).
template <typename Args>
__device__ inline size_t unit_of(const Args& a, int b, int h, int p) {
  const int phys = clampi(a.block_table[(size_t)b * a.bt_stride + (p >> 4)], 0, a.num_blocks - 1);
  return (size_t)phys * a.hkv + h;
}
template <typename Args, typename P>
__device__ inline P* code_row(const Args& a, const TensorKind& k, P* codes, int b, int h, int p) {
  if (a.paged) return codes + unit_of(a, b, h, p) * k.unit + (size_t)(p & 15) * k.row;
  return codes + (((size_t)b * a.hkv + h) * a.max_tokens + p) * k.row;
}
template <typename Args, typename P>
__device__ inline P* meta_elem(const Args& a, const TensorKind& k, P* meta, int b, int h, int p) {
  if (a.paged)
    return (P*)a.k_codes + unit_of(a, b, h, p) * a.kk.unit + k.moff +
           (size_t)((p & 15) >> a.tgshift) * k.mb;
  return meta + ((((size_t)b * a.hkv + h) * a.max_tokens + p) >> a.tgshift) * k.mb;
}

__device__ inline int rne_code(double x, double s) { return (int)rint(x / s); }

__device__ inline int code_bits(CodeKind c) {
  return (c == CK_I8 || c == CK_U8) ? 8 : (c == CK_I4 || c == CK_U4) ? 4 : 2;
}

// Largest code magnitude: 2^(b-1) - 1 (symmetric) or 2^b - 1 (zero point).
__device__ inline int qmax_sym(int bits) { return (1 << (bits - 1)) - 1; }
__device__ inline int qmax_zp(int bits) { return (1 << bits) - 1; }

// Quantizes the token group at positions p0 .. p0+g-1 of one (sequence,
// head): one scale (and zero point, or 8-bit scale code) over all its g*D
// values, then the codes of each token.  ld(p, x0, x1) loads elements 2*lane
// and 2*lane+1 of position p; row(p) is the address of its code row; meta is
// the address of the group's metadata element (unused for per-channel
// scales).  g = 1 is the per-token case.  Values are taken in fp64: inputs
// are exact in it, and so is a middle-tier value c * s.
template <typename Load, typename Row>
__device__ void quantize_group(const TensorKind k, Load ld, Row row, int p0, int g,
                               uint8_t* meta, const float* chan, float super, int lane) {
  const int bits = code_bits(k.code);
  const bool zp = k.meta == MK_F32Z || k.meta == MK_F16Z;
  // 1. group statistics
  double amax = 0.0, lo = 0.0, hi = 0.0;
  if (!k.channel) {
    double mx = 0.0, mn = 0.0, ab = 0.0;
    for (int j = 0; j < g; ++j) {
      double x0, x1;
      ld(p0 + j, x0, x1);
      ab = fmax(ab, fmax(fabs(x0), fabs(x1)));
      mx = fmax(mx, fmax(x0, x1));
      mn = fmin(mn, fmin(x0, x1));
    }
    amax = wave_max(ab);
    hi = wave_max(mx);  // zero point: the range includes 0 (mx, mn start at 0)
    lo = wave_min(mn);
  }
  // 2. the group's scale (fp64, rounded once to its storage type)
  double s = 1.0;  // scale the codes divide by
  int z = 0, qmax = 0, u = 0;
  bool nonzero = true;
  uint32_t sbits = 0;
  if (k.channel) {
    qmax = qmax_sym(bits);
  } else if (k.meta == MK_U8) {
    // 8-bit scale code relative to the frozen per-head super-scale
    qmax = qmax_sym(bits);
    nonzero = amax != 0.0;
    if (nonzero) {
      const double sigma = amax / qmax;
      u = clampi((int)rint(sigma / (double)super), 1, 255);
      s = (double)u * (double)super;  // exact
    }
  } else if (!zp) {
    qmax = qmax_sym(bits);
    nonzero = amax != 0.0;
    if (k.meta == MK_F32) {
      const float sf = nonzero ? store_f32(amax / qmax) : 1.0f;
      s = (double)sf;
      sbits = __float_as_uint(sf);
    } else {
      const uint16_t hb = nonzero ? store_f16(amax / qmax) : (uint16_t)0x3C00u;
      s = f16_bits_to_f64(hb);
      sbits = hb;
    }
  } else {
    qmax = qmax_zp(bits);
    nonzero = hi != lo;
    if (k.meta == MK_F32Z) {
      const float sf = nonzero ? store_f32((hi - lo) / qmax) : 1.0f;
      s = (double)sf;
      sbits = __float_as_uint(sf);
    } else {
      const uint16_t hb = nonzero ? store_f16((hi - lo) / qmax) : (uint16_t)0x3C00u;
      s = f16_bits_to_f64(hb);
      sbits = hb;
    }
    if (nonzero) z = clampi((int)rint(-lo / s), 0, qmax);
  }
  if (lane == 0 && !k.channel) {
    if (k.meta == MK_U8) {
      *meta = (uint8_t)u;
    } else if (k.meta == MK_F32) {
      *(uint32_t*)meta = sbits;
    } else if (k.meta == MK_F16) {
      *(uint16_t*)meta = (uint16_t)sbits;
    } else if (k.meta == MK_F32Z) {
      ((uint32_t*)meta)[0] = sbits;
      ((float*)meta)[1] = (float)z;
    } else {
      const _Float16 zh = (_Float16)(float)z;
      *(uint32_t*)meta = sbits | ((uint32_t)__builtin_bit_cast(uint16_t, zh) << 16);
    }
  }
  // 3. codes of each token of the group
  for (int j = 0; j < g; ++j) {
    double x0, x1;
    ld(p0 + j, x0, x1);
    int c0 = 0, c1 = 0;
    if (k.channel) {
      c0 = clampi(rne_code(x0, (double)chan[2 * lane]), -qmax, qmax);
      c1 = clampi(rne_code(x1, (double)chan[2 * lane + 1]), -qmax, qmax);
    } else if (nonzero && !zp) {
      c0 = clampi(rne_code(x0, s), -qmax, qmax);
      c1 = clampi(rne_code(x1, s), -qmax, qmax);
    } else if (nonzero) {
      c0 = clampi(rne_code(x0, s) + z, 0, qmax);
      c1 = clampi(rne_code(x1, s) + z, 0, qmax);
    }
    uint8_t* r = row(p0 + j);
    if (bits == 8) {
      const uint32_t v = ((uint32_t)(c0 & 0xFF)) | ((uint32_t)(c1 & 0xFF) << 8);
      ((uint16_t*)r)[lane] = (uint16_t)v;
    } else if (bits == 4) {
      const uint32_t v = ((uint32_t)(c0 & 0xF)) | ((uint32_t)(c1 & 0xF) << 4);
      r[lane] = (uint8_t)v;
    } else {
      // four 2-bit codes per byte: elements 4j .. 4j+3 come from lanes 2j, 2j+1
      const uint32_t v = ((uint32_t)(c0 & 3)) | ((uint32_t)(c1 & 3) << 2);
      const uint32_t odd = (uint32_t)__shfl_xor((int)v, 1);
      if ((lane & 1) == 0) r[lane >> 1] = (uint8_t)(v | (odd << 4));
    }
  }
}

}  // namespace qz
}  // namespace kvq
