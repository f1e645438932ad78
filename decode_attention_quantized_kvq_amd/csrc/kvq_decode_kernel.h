// Kernel templates of the split-T decode (gfx950), included by the
// translation units that instantiate them for their key/value format pairs
// (kvq_decode.hip, kvq_decode_w4.hip, kvq_decode_mixed.hip, kvq_decode_w2.hip);
// the pairs are spread over several files only so that they compile in
// parallel.  What the kernels compute and how is described in kvq_decode.hip.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "kvq_internal.h"
#include "kvq_quantize.h"

namespace kvq {
namespace {


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int WAVES = 4;
constexpr int TILE = 32;
// Tiles each wave keeps in flight, by code bytes per token (key + value):
// more than the memory needs only queues (the first data of a new work item
// then waits behind it), fewer leaves it idle.  Measured on one MI355X
// (non-temporal loads): 256 bytes (int8 / int8, paged 64 x 8 heads) 407 us
// with two against 419 with one; 192 bytes (per-channel int8 keys, int4
// values) 257 us with one against 262 with two; 128 bytes (uint4 / uint4)
// 51.1 us with two against 53.9 with one.
#ifndef KVQ_NB8
#define KVQ_NB8 2
#endif
#ifndef KVQ_NB6
#define KVQ_NB6 1
#endif
#ifndef KVQ_NB4
#define KVQ_NB4 2
#endif
#ifndef KVQ_NB2
#define KVQ_NB2 2
#endif
// Cache policy of the loads that stream the cache (codes and metadata): the
// buffer instructions' cache-policy operand, 2 = nt (non-temporal).  Each
// cache byte is read once per step, so it gains nothing from staying in the
// caches; on one MI355X, nt loads took the paged int8 workload from 423 to
// 407 us and the uint4 workload from 57.3 to 51.1 us, and a plain streaming
// read from 6.3 to 7.1 TB/s.
#ifndef KVQ_CPOL
#define KVQ_CPOL 2
#endif
// Minimum waves per SIMD the decode kernel is compiled for.
#ifndef KVQ_MINW
#define KVQ_MINW 1
#endif
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float NEG_INF = -__builtin_inff();

// fp16 constants (two per dword)
constexpr uint32_t MAGIC = 0x64006400u;      // 1024.0 | 1024.0 exponent pattern
constexpr uint32_t H_M1024 = 0xE400E400u;    // -1024
constexpr uint32_t H_M1032 = 0xE408E408u;    // -1032 (signed nibble: bias 8)
constexpr uint32_t H_M1152 = 0xE480E480u;    // -1152 (signed byte: bias 128)
constexpr uint32_t H_SIXTEENTH = 0x2C002C00u;  // 1/16
constexpr uint32_t H_M64 = 0xD400D400u;      // -64
constexpr uint32_t H_M72 = 0xD480D480u;      // -72
// 2-bit fields at bit 2r (r = 0..3) of each half, scaled by 4^-r back to units
constexpr uint32_t H_QUARTER = 0x34003400u;    // 1/4
constexpr uint32_t H_1_64 = 0x24002400u;       // 1/64
constexpr uint32_t H_M1026 = 0xE402E402u;      // -1026 (signed 2-bit: bias 2)
constexpr uint32_t H_M256 = 0xDC00DC00u;       // -256
constexpr uint32_t H_M258 = 0xDC08DC08u;       // -258
constexpr uint32_t H_M66 = 0xD420D420u;        // -66
constexpr uint32_t H_M16 = 0xCC00CC00u;        // -16
constexpr uint32_t H_M18 = 0xCC80CC80u;        // -18

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ inline uint32_t h2_add(uint32_t a, uint32_t c) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, a) + __builtin_bit_cast(half2v, c));
}

__device__ inline uint32_t h2_fma(uint32_t a, uint32_t m, uint32_t c) {
  const half2v r = __builtin_bit_cast(half2v, a) * __builtin_bit_cast(half2v, m) +
                   __builtin_bit_cast(half2v, c);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, u32x4{a, b, c, d});
}

__device__ inline bf16x8 as_b8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}

__device__ inline uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__device__ inline uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ inline float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int G>
__device__ inline float ror_g(float v) {
  // Value of the lane G columns away inside the 16-lane row (DPP row_ror).
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), 0x120 + G, 0xF, 0xF, false));
}

// Reductions over the four 16-lane rows (lanes c, c+16, c+32, c+48).  A
// self-swap with v_permlane32_swap gives each lane its partner 32 lanes away
// in one of the two results (the other keeps its own value), so combining
// both results reduces lane pairs; v_permlane16_swap does the same for rows
// (0,1) and (2,3).  VALU only, no LDS crossbar.
__device__ inline float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Smallest power of two >= x (x >= 0 finite); 0 stays 0.
// Max / sum over the 16 lanes of this lane's row (DPP rotations inside a row).
__device__ inline float row16_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false)));
  return v;
}
__device__ inline float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}

__device__ inline float pow2_ceil(float x) {
  uint32_t u = __float_as_uint(x);
  if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
  return __uint_as_float(u);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Phase stamps of an instrumented build (KVQ_PHASE_STAMPS; the 100 MHz
// real-time counter) written by each workgroup's first thread: 0 start,
// 1 work item known, 2 query ready, 3 the wave's tiles done, 4 partial
// stored, 5 arrival counted, 6 end (times 2, plus 1 if it combined),
// 7 hardware ids (XCC id << 32 | HW_ID).  Compiled out otherwise.
__device__ inline void phase_stamp(unsigned long long* stamps, int i, unsigned long long v) {
#ifdef KVQ_PHASE_STAMPS
  if (stamps != nullptr && threadIdx.x == 0 && blockIdx.x < 65536u) stamps[blockIdx.x * 8 + i] = v;
#endif
}
__device__ inline void phase_stamp(unsigned long long* stamps, int i) {
#ifdef KVQ_PHASE_STAMPS
  phase_stamp(stamps, i, __builtin_amdgcn_s_memrealtime());
#endif
}

// ---------------------------------------------------------------------------
// Code formats: byte layout per token row and conversion to fp16 MFMA operands
// ---------------------------------------------------------------------------
template <int CK>
struct Codes {
  static constexpr bool B8 = (CK == CK_I8 || CK == CK_U8);
  static constexpr bool B2 = (CK == CK_I2 || CK == CK_U2);
  static constexpr bool SIGNED = (CK == CK_I8 || CK == CK_I4 || CK == CK_I2);
  static constexpr int ROW = B8 ? D : B2 ? D / 4 : D / 2;
};

// Converts 4 int8 codes of one dword into two fp16 pairs (d0,d1), (d2,d3),
// exactly: the byte becomes the mantissa of 1024 + u, then the bias goes.
template <bool SIGNED>
__device__ inline void cvt_b8(uint32_t w, uint32_t& p01, uint32_t& p23) {
  if (SIGNED) w ^= 0x80808080u;
  p01 = h2_add(perm(0x64646464u, w, 0x04010400u), SIGNED ? H_M1152 : H_M1024);
  p23 = h2_add(perm(0x64646464u, w, 0x04030402u), SIGNED ? H_M1152 : H_M1024);
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time
// indices, needed by instructions that encode a byte or lane selector).
template <typename F, int... I>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}


// A constant held in a VGPR.  VOP3 instructions of gfx9 cannot encode a
// literal, so (w & mask) | magic with literal operands costs two
// instructions; with both in VGPRs it is one v_and_or_b32.
__device__ inline uint32_t in_vgpr(uint32_t x) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(x));
  return r;
}

struct NibbleMasks {
  uint32_t lo, hi, magic;  // 0x000F000F, 0x00F000F0, 0x64006400
  uint32_t c[4];           // 2-bit fields: 0x00030003 << 2r
  __device__ inline void init() {
    lo = in_vgpr(0x000F000Fu);
    hi = in_vgpr(0x00F000F0u);
    magic = in_vgpr(MAGIC);
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] = in_vgpr(0x00030003u << (2 * r));
  }
};

// Converts 8 int4 codes of one dword into four fp16 pairs, ordered
// (n0,n4), (n1,n5), (n2,n6), (n3,n7) where n_i is nibble i (bits 4i..4i+3).
template <bool SIGNED>
__device__ inline void cvt_b4(uint32_t w, uint32_t out[4], const NibbleMasks& nm) {
  if (SIGNED) w ^= 0x88888888u;
  const uint32_t w8 = w >> 8;
  out[0] = h2_add((w & nm.lo) | nm.magic, SIGNED ? H_M1032 : H_M1024);
  out[1] = h2_fma((w & nm.hi) | nm.magic, H_SIXTEENTH, SIGNED ? H_M72 : H_M64);
  out[2] = h2_add((w8 & nm.lo) | nm.magic, SIGNED ? H_M1032 : H_M1024);
  out[3] = h2_fma((w8 & nm.hi) | nm.magic, H_SIXTEENTH, SIGNED ? H_M72 : H_M64);
}

// Converts the 2-bit codes of two tokens (token A in the low half-word of x,
// token B in the high one, feature f at bits 2f) into eight fp16 pairs
// (feature f of A, feature f of B), f = 0..7.  Field r of a byte, or'ed into
// the exponent pattern of 1024, reads 1024 + c 4^r; scaling by 4^-r and
// removing the bias leaves c exactly.
template <bool SIGNED>
__device__ inline void cvt_b2(uint32_t x, uint32_t out[8], const NibbleMasks& nm) {
  if (SIGNED) x ^= 0xAAAAAAAAu;  // two's complement c -> c + 2
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t y = m ? x >> 8 : x;
    out[4 * m + 0] = h2_add((y & nm.c[0]) | nm.magic, SIGNED ? H_M1026 : H_M1024);
    out[4 * m + 1] = h2_fma((y & nm.c[1]) | nm.magic, H_QUARTER, SIGNED ? H_M258 : H_M256);
    out[4 * m + 2] = h2_fma((y & nm.c[2]) | nm.magic, H_SIXTEENTH, SIGNED ? H_M66 : H_M64);
    out[4 * m + 3] = h2_fma((y & nm.c[3]) | nm.magic, H_1_64, SIGNED ? H_M18 : H_M16);
  }
}

// Feature index held by the lanes of k-group g at k-slot e of the j-th score
// MFMA.  Every key format covers features [32g, 32g + 32).  8-bit keys are
// used as stored; 4-bit keys are widened to bytes, even nibbles (features
// 2e) in slots 0..3 and odd nibbles (features 2e - 7) in slots 4..7; 2-bit
// keys come from dword j / 2 (features 16 (j / 2) + i at bits 2i), shifted
// right by 4 (j % 2) and 4 (j % 2) + 2 bits and masked to one code per
// byte: slot e holds code 4 (e % 4) + 2 (j % 2) + e / 4 of that dword.
template <int KC>
__device__ inline int key_feature(int j, int g, int e) {
  if (Codes<KC>::B8) return 32 * g + 8 * j + e;
  if (Codes<KC>::B2) return 32 * g + 16 * (j >> 1) + 4 * (e & 3) + 2 * (j & 1) + (e >> 2);
  return 32 * g + 8 * j + (e < 4 ? 2 * e : 2 * e - 7);
}

// ---------------------------------------------------------------------------
// Per-token metadata
// ---------------------------------------------------------------------------
template <int MK>
struct Meta {
  static constexpr int BYTES = MK == MK_F32 ? 4 : MK == MK_F32Z ? 8 : MK == MK_F16 ? 2
                             : MK == MK_F16Z ? 4 : MK == MK_U8 ? 1 : 0;
  static constexpr bool ZP = (MK == MK_F32Z || MK == MK_F16Z);
  uint32_t r0, r1;  // raw bytes of one token's metadata (r1: fp32 zero point)

  // metadata of one token through a buffer resource, at byte offset off
  __device__ inline void load_buf(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    r1 = 0;  // defined for every kind: copies of the struct stay 32-bit fields
    if (MK == MK_F32 || MK == MK_F16Z) {
      r0 = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, KVQ_CPOL);
    } else if (MK == MK_F32Z) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, KVQ_CPOL);
      r0 = v.x;
      r1 = v.y;
    } else if (MK == MK_F16) {
      r0 = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, KVQ_CPOL);
    } else if (MK == MK_U8) {
      r0 = __builtin_amdgcn_raw_buffer_load_b8(rs, off, 0, KVQ_CPOL);
    }
  }
  // metadata of one token at p (one 1-8 byte load per lane)
  __device__ inline void load_glob(const uint8_t* p) {
    r1 = 0;
#if KVQ_CPOL == 2
#define KVQ_LDM(T, q) __builtin_nontemporal_load((const T*)(q))
#else
#define KVQ_LDM(T, q) (*(const T*)(q))
#endif
    if (MK == MK_F32 || MK == MK_F16Z) {
      r0 = KVQ_LDM(uint32_t, p);
    } else if (MK == MK_F32Z) {
      const u32x2 v = KVQ_LDM(u32x2, p);
      r0 = v.x;
      r1 = v.y;
    } else if (MK == MK_F16) {
      r0 = KVQ_LDM(uint16_t, p);
    } else if (MK == MK_U8) {
      r0 = KVQ_LDM(uint8_t, p);
    }
#undef KVQ_LDM
  }
  // the same fields of lane (lane ^ 16)
  __device__ inline Meta xor16() const {
    Meta m;
    m.r0 = BYTES ? (uint32_t)__shfl_xor((int)r0, 16) : 0u;
    m.r1 = MK == MK_F32Z ? (uint32_t)__shfl_xor((int)r1, 16) : 0u;
    return m;
  }
  __device__ inline float scale() const {
    if (MK == MK_F32 || MK == MK_F32Z) return __uint_as_float(r0);
    if (MK == MK_F16 || MK == MK_F16Z)
      return (float)__builtin_bit_cast(_Float16, (uint16_t)(r0 & 0xFFFFu));
    if (MK == MK_U8) return (float)(r0 & 0xFFu);
    return 1.0f;
  }
  __device__ inline float zero() const {
    if (MK == MK_F32Z) return __uint_as_float(r1);
    if (MK == MK_F16Z) return (float)__builtin_bit_cast(_Float16, (uint16_t)(r0 >> 16));
    return 0.0f;
  }
};

// ---------------------------------------------------------------------------
// Where the 16-token blocks of a (sequence, KV head) live
// ---------------------------------------------------------------------------
struct Addr {
  const uint8_t* k;
  const uint8_t* v;
  const uint8_t* km;
  const uint8_t* vm;
  int num_blocks, hkv, h;
  int ku, vu;            // paged: bytes of one (block, head) unit of K and V
  int gs;                // log2 of the token group size (metadata per group)
  size_t head_tok;       // contiguous: first token slot of this head
  int nblk;              // blocks holding tokens
  int rblk;              // ring (middle tier): blocks of the ring, block i in slot i mod rblk
  // paged: block-table entries of this wave's blocks.  A wave whose tiles
  // are every WAVES-th of its chunk (ilv) has blocks blk0 + 2 WAVES k + c
  // (c = 0, 1) for its k-th tile, entry e = 2k + c; a wave with a contiguous
  // range has blocks blk0 + e.  Entry e sits in lane e & 63 of ent[e >> 6].
  int blk0;
  int ent[2];
  bool ilv;
};

// Table entries a wave holds: 64 tiles, 2048 of a chunk's tokens.
constexpr int WAVE_BLOCKS = 128;

// Token slot index of block `blk` (clamped to the blocks holding tokens and,
// when paged, to the pool), or when paged its unit index phys H_kv + h;
// wave-uniform.  Paged lookups read the entries preloaded into the wave's
// registers (v_readlane), so the token loop issues no memory access for
// them.  RING: the middle tier's ring of rblk blocks.
template <bool PAGED, bool RING = false>
__device__ inline size_t block_slot(const Addr& ad, int blk) {
  blk = blk < ad.nblk ? blk : ad.nblk - 1;
  if constexpr (RING) {
    return ad.head_tok + (size_t)(blk % ad.rblk) * 16;
  } else if constexpr (PAGED) {
    // block blk0 + 2 WAVES k + c is entry 2k + c (other offsets are not
    // this wave's blocks; they only occur for blocks past the chunk, whose
    // loads read nothing)
    int i = blk - ad.blk0;
    static_assert(2 * WAVES == 8, "entry index: tile k of a wave starts 8 blocks after tile k - 1");
    if (ad.ilv) i = ((i >> 3) << 1) | (i & 1);
    i = i < 0 ? 0 : (i >= WAVE_BLOCKS ? WAVE_BLOCKS - 1 : i);
    int phys = i < 64 ? __builtin_amdgcn_readlane(ad.ent[0], i)
                      : __builtin_amdgcn_readlane(ad.ent[1], i - 64);
    phys = phys < 0 ? 0 : (phys >= ad.num_blocks ? ad.num_blocks - 1 : phys);
    return (size_t)phys * ad.hkv + ad.h;
  } else {
    return ad.head_tok + (size_t)blk * 16;
  }
}

// Descriptor word 3 of a raw (byte-addressed, unswizzled) buffer resource.
constexpr int RSRC_WORD3 = 0x00020000;

// Buffer resource over `bytes` bytes at p.  A resource of 0 bytes makes every
// load through it out of range: it returns zeros and reads no memory.  The
// arguments are wave-uniform; readfirstlane says so to the compiler, which
// would otherwise wrap each load in a loop over distinct descriptors.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const uint8_t* p, int bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint8_t* q = (const uint8_t*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc((void*)q, 0, __builtin_amdgcn_readfirstlane(bytes),
                                           RSRC_WORD3);
}

// Byte offsets of lane (t, g) = (lane & 15, lane >> 4) inside a 16-token
// block; fixed for the whole kernel, so every load is a wave-uniform base plus
// a 32-bit offset.  Keys: token row t, bytes [32g, 32g + 32) (8-bit) or
// [16g, 16g + 16) (4-bit), i.e. features [32g, 32g + 32) either way.  Values:
// token rows 4i + g (i = 0..3), features [8t, 8t + 8), so that one load
// instruction (fixed i) covers 4 consecutive rows, whole 128-byte lines even
// for 64-byte (4-bit) rows.  Metadata: the element of token t's group.
struct LaneOff {
  uint32_t k0, k1, v[4], km, vm;
  bool odd;  // g odd: this lane loads the metadata of the tile's second block
};

template <int KC, int KM, int VC, int VM>
__device__ inline LaneOff lane_offsets(int t, int g, int gs) {
  constexpr int KROW = Codes<KC>::ROW, VROW = Codes<VC>::ROW;
  LaneOff o;
  o.k0 = t * KROW + (Codes<KC>::B8 ? 32 * g : Codes<KC>::B2 ? 8 * g : 16 * g);
  o.k1 = o.k0 + 16;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o.v[i] = (4 * i + g) * VROW + (Codes<VC>::B8 ? 8 * t : Codes<VC>::B2 ? 2 * t : 4 * t);
  o.km = (t >> gs) * Meta<KM>::BYTES;  // token t's group
  o.vm = (t >> gs) * Meta<VM>::BYTES;
  o.odd = g & 1;
  return o;
}

// Raw registers of one 32-token tile.  Metadata: PT, one load per tensor
// and tile (lane (t, g) reads token t of block g & 1 through a per-lane
// address, and compute_tile takes the other block's from lane (t, g ^ 1));
// otherwise one buffer load per tensor and block (token t of each block).
// The first costs vector ALU work and the second scalar registers (a buffer
// descriptor per load): kernels that run out of scalar registers take PT.
template <int KC, int KM, int VC, int VM, bool PT = false>
struct TileRaw {
  static constexpr bool KB8 = Codes<KC>::B8;
  static constexpr bool VB8 = Codes<VC>::B8;
  u32x4 k[2][KB8 ? 2 : 1];   // per 16-token block (2-bit keys: .x, .y)
  u32x2 v8[VB8 ? 8 : 1];     // 8-bit values: 8 tokens x 8 bytes
  uint32_t v4[VB8 ? 1 : 8];  // 4-bit values: 8 tokens x 4 bytes; 2-bit: 2 bytes
  Meta<KM> km[PT ? 1 : 2];
  Meta<VM> vm[PT ? 1 : 2];
};

// Loads the 32-token tile at t0 of a wave whose range ends at tend.  Every
// load is issued whatever t0 is, so the wait counts the compiler derives stay
// exact; a 16-token block at or past tend is read through an empty resource
// (zeros, no memory traffic) and its tokens are masked by compute_tile.
template <bool PAGED, bool RING, int KC, int KM, int VC, int VM, bool PT>
__device__ inline void load_tile(TileRaw<KC, KM, VC, VM, PT>& t, const Addr& ad, int t0, int tend,
                                 const LaneOff& o) {
  constexpr int KROW = Codes<KC>::ROW, VROW = Codes<VC>::ROW;
  const uint8_t* kmb[2];
  const uint8_t* vmb[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const bool live = t0 + 16 * bb < tend;
    const size_t slot = block_slot<PAGED, RING>(ad, (t0 >> 4) + bb);
    // the block's code rows and metadata: paged, its units (the key unit's 16
    // code rows followed by the key and then the value metadata elements);
    // otherwise slot rows and metadata element slot >> gs (one per token group)
    const uint8_t* kb = PAGED ? ad.k + slot * ad.ku : ad.k + slot * KROW;
    const uint8_t* vb = PAGED ? ad.v + slot * ad.vu : ad.v + slot * VROW;
    kmb[bb] = PAGED ? kb + 16 * KROW : ad.km + (slot >> ad.gs) * Meta<KM>::BYTES;
    vmb[bb] = PAGED ? kmb[bb] + (16 >> ad.gs) * Meta<KM>::BYTES
                    : ad.vm + (slot >> ad.gs) * Meta<VM>::BYTES;
    const auto rk = rsrc(kb, live ? 16 * KROW : 0);
    if (Codes<KC>::B2) {
      const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(rk, o.k0, 0, KVQ_CPOL);
      t.k[bb][0] = u32x4{w.x, w.y, 0u, 0u};
    } else {
      t.k[bb][0] = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k0, 0, KVQ_CPOL);
    }
    if (Codes<KC>::B8) t.k[bb][1] = __builtin_amdgcn_raw_buffer_load_b128(rk, o.k1, 0, KVQ_CPOL);
    const auto rv = rsrc(vb, live ? 16 * VROW : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (Codes<VC>::B8)
        t.v8[4 * bb + i] = __builtin_amdgcn_raw_buffer_load_b64(rv, o.v[i], 0, KVQ_CPOL);
      else if (Codes<VC>::B2)
        t.v4[4 * bb + i] = __builtin_amdgcn_raw_buffer_load_b16(rv, o.v[i], 0, KVQ_CPOL);
      else
        t.v4[4 * bb + i] = __builtin_amdgcn_raw_buffer_load_b32(rv, o.v[i], 0, KVQ_CPOL);
    }
    if constexpr (!PT) {
      if (Meta<KM>::BYTES)
        t.km[bb].load_buf(rsrc(kmb[bb], live ? (16 >> ad.gs) * Meta<KM>::BYTES : 0), o.km);
      if (Meta<VM>::BYTES)
        t.vm[bb].load_buf(rsrc(vmb[bb], live ? (16 >> ad.gs) * Meta<VM>::BYTES : 0), o.vm);
    }
  }
  if constexpr (PT) {
    // one load per tensor covers both blocks (lane (t, g): block g & 1); a
    // block past tend reads a stored slot (block_slot clamps) whose values
    // compute_tile masks
    if (Meta<KM>::BYTES) t.km[0].load_glob((o.odd ? kmb[1] : kmb[0]) + o.km);
    if (Meta<VM>::BYTES) t.vm[0].load_glob((o.odd ? vmb[1] : vmb[0]) + o.vm);
  }
}

// Key operand of the J-th score MFMA for block bb: 8 int8 values, the codes
// themselves for signed 8-bit keys, offset to signed range for the others
// (u - 128 for unsigned bytes; nibble + 8 or the unsigned nibble, widened).
template <int J, int KC, int KM, int VC, int VM, bool PT>
__device__ inline long key_frag(const TileRaw<KC, KM, VC, VM, PT>& t, int bb) {
  uint32_t lo, hi;
  if constexpr (Codes<KC>::B8) {
    const u32x4 r = t.k[bb][J >> 1];
    lo = (J & 1) ? r.z : r.x;
    hi = (J & 1) ? r.w : r.y;
    if (KC == CK_U8) {
      lo ^= 0x80808080u;
      hi ^= 0x80808080u;
    }
  } else if constexpr (Codes<KC>::B2) {
    uint32_t w = t.k[bb][0][J >> 1];
    if (KC == CK_I2) w ^= 0xAAAAAAAAu;  // two's complement 2-bit c -> c + 2
    constexpr int SH = 4 * (J & 1);
    lo = (w >> SH) & 0x03030303u;
    hi = (w >> (SH + 2)) & 0x03030303u;
  } else {
    uint32_t w = t.k[bb][0][J];
    if (KC == CK_I4) w ^= 0x88888888u;  // two's complement nibble c -> c + 8
    lo = w & 0x0F0F0F0Fu;
    hi = (w >> 4) & 0x0F0F0F0Fu;
  }
  return (long)(((uint64_t)hi << 32) | lo);
}

// What the key operand adds to the code value (the dot is taken over
// code + KOFF, so KOFF * sum(Q) comes off the score).
template <int KC>
__device__ inline float key_offset() {
  return KC == CK_U8 ? -128.0f : KC == CK_I4 ? 8.0f : KC == CK_I2 ? 2.0f : 0.0f;
}

// Value operands of the 8 output MFMAs: lane (c, g) gives feature 8c + j of
// its 8 tokens, two tokens per fp16 pair.
template <int KC, int KM, int VC, int VM, bool PT>
__device__ inline void value_frags(const TileRaw<KC, KM, VC, VM, PT>& t, half8 out[8],
                                   const NibbleMasks& nm) {
  constexpr bool S = Codes<VC>::SIGNED;
  uint32_t pr[8][4];  // [j][token pair]
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    if (Codes<VC>::B8) {
      const u32x2 A = t.v8[2 * pp], B = t.v8[2 * pp + 1];
      // bytes (A f, B f, A f+1, B f+1) for f = 0, 2, 4, 6
      const uint32_t x[4] = {perm(B.x, A.x, 0x05010400u), perm(B.x, A.x, 0x07030602u),
                             perm(B.y, A.y, 0x05010400u), perm(B.y, A.y, 0x07030602u)};
#pragma unroll
      for (int q = 0; q < 4; ++q) cvt_b8<S>(x[q], pr[2 * q][pp], pr[2 * q + 1][pp]);
    } else if (Codes<VC>::B2) {
      // bytes (A0, A1, B0, B1): features 0..7 of tokens A and B
      uint32_t o[8];
      cvt_b2<S>(perm(t.v4[2 * pp + 1], t.v4[2 * pp], 0x05040100u), o, nm);
#pragma unroll
      for (int q = 0; q < 8; ++q) pr[q][pp] = o[q];
    } else {
      const uint32_t A = t.v4[2 * pp], B = t.v4[2 * pp + 1];
      uint32_t o[4];
      // bytes (A0, A1, B0, B1): cvt_b4 pairs nibble n of the low half-word
      // (token A) with nibble n of the high half-word (token B), i.e. feature
      // n of both tokens, for n = 0..3 in that order.
      cvt_b4<S>(perm(B, A, 0x05040100u), o, nm);
#pragma unroll
      for (int q = 0; q < 4; ++q) pr[q][pp] = o[q];
      cvt_b4<S>(perm(B, A, 0x07060302u), o, nm);  // bytes (A2, A3, B2, B3): features 4..7
#pragma unroll
      for (int q = 0; q < 4; ++q) pr[4 + q][pp] = o[q];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = as_h8(pr[j][0], pr[j][1], pr[j][2], pr[j][3]);
}

// ---------------------------------------------------------------------------
// Per-wave state of the online softmax.  The reference max m moves only when
// a score exceeds it by 2^8 (base 2), and the weight reference R only when a
// weight p s_V exceeds it by 2^6, so the accumulators are rescaled on few
// tiles and the fp16 weights p s_V / R stay below 64.
// ---------------------------------------------------------------------------
constexpr float M_SLACK = 8.0f;
constexpr float R_SLACK = 64.0f;

struct Softmax {
  float m;   // reference max (base-2 units), identical across the 4 row groups
  float l;   // this lane's share of the running sum of 2^(s - m)
  float R;   // power-of-two reference of the folded value scale
  float z;   // this lane's share of sum w * zero_point (zero-point values)
  f32x4 o[8];

  __device__ inline void init(float r0) {
    m = NEG_INF;
    l = 0.0f;
    R = r0;
    z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Moves the reference max if the tile max exceeds it by more than M_SLACK;
  // returns the rescale factor of the accumulators and the max to use.
  __device__ inline float update_max(float mt, float* mu) {
    float alpha = 1.0f;
    if (mt > m + M_SLACK) {
      alpha = exp2_fast(m - mt);  // 0 when m = -inf
      m = mt;
    }
    *mu = m == NEG_INF ? 0.0f : m;
    return alpha;
  }
};

// Per-wave state of the quantized-token path.  The scores come out of the
// matrix cores transposed (query rows x token columns), so lane (t, g) holds
// whole scores of the HPG query heads of row group g for token t of each
// block: HPG = 2 when G = 8, else 1 (row group g is query head g).  The
// lane also holds the output rows of those heads, so every per-head
// reference (m, R) is uniform over a row group and local to the lane.
template <int G>
struct RowState {
  static constexpr int HPG = G == 8 ? 2 : 1;
  float m[HPG];     // reference max per head (base-2 units), uniform over the row
  float l[HPG];     // this lane's share of the running sum of 2^(s - m)
  float z[HPG];     // this lane's share of sum w * zero_point (zero-point values)
  float R[HPG];     // power-of-two weight reference per head: w = p s_V / R
  float invR[HPG];  // 1 / R (exact)
  f32x4 o[8];       // O^T: rows 4g + i = (head, limb), columns = features 8t + J

  __device__ inline void init(float r0) {
#pragma unroll
    for (int u = 0; u < HPG; ++u) {
      m[u] = NEG_INF;
      l[u] = 0.0f;
      z[u] = 0.0f;
      R[u] = r0;
      invR[u] = 1.0f / r0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Query operand row r of the score MFMAs: the query head it holds and which
// fp16 half (limb 0 high, 1 low); rows holding no head are zero.
template <int G>
__device__ inline int row_head(int r) { return G == 8 ? r >> 1 : r >> 2; }
template <int G>
__device__ inline int row_limb(int r) { return G == 8 ? (r & 1) : (r & 3); }

// Processes one 32-token tile already in registers.
//   scores  S^T[16 rows x 16 tok] += Q'[16 rows x 32 d] K^T[32 d x 16 tok]
//   output  O^T[16 rows x 16 d]   += P^T[16 rows x 32 tok] V[32 tok x 16 d]
// Rows are (query head, fp16 limb) pairs.  The weights P^T go through LDS
// (pw, this wave's region) from the score layout to the operand layout.
// qs[u], sumq[u]: score scale and query sum of local head u.
template <int KC, int KM, bool KCH, int VC, int VM, int G, bool PT>
__device__ inline void compute_tile(const TileRaw<KC, KM, VC, VM, PT>& t, int t0, int tend,
                                    const long (*qa)[4], const float* qs, const float* sq,
                                    int lt, int g, uint32_t psel, const uint32_t* prd,
                                    uint32_t* pwr, const NibbleMasks& nm, RowState<G>& st) {
  constexpr int HPG = RowState<G>::HPG;
  // scores on the int8 matrix cores: rows (head, limb) of the query, exact
  // int32 dot products per limb
  i32x4 sa[HPG][2];
#pragma unroll
  for (int u = 0; u < HPG; ++u) sa[u][0] = sa[u][1] = i32x4{0, 0, 0, 0};
  static_for<4>([&](auto jc) {
    constexpr int J = decltype(jc)::value;
    const long k0 = key_frag<J>(t, 0), k1 = key_frag<J>(t, 1);
#pragma unroll
    for (int u = 0; u < HPG; ++u) {
      sa[u][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(qa[u][J], k0, sa[u][0], 0, 0, 0);
      sa[u][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(qa[u][J], k1, sa[u][1], 0, 0, 0);
    }
  });
  // metadata of token lt of blocks 0 and 1: one is this lane's, the other
  // lane (lt, g ^ 1)'s
  Meta<KM> kmb[2];
  Meta<VM> vmb[2];
  if constexpr (PT) {
    const bool odd = g & 1;
    const Meta<KM> ko = t.km[0].xor16();
    const Meta<VM> vo = t.vm[0].xor16();
    kmb[0] = odd ? ko : t.km[0];
    kmb[1] = odd ? t.km[0] : ko;
    vmb[0] = odd ? vo : t.vm[0];
    vmb[1] = odd ? t.vm[0] : vo;
  } else {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      kmb[bb] = t.km[bb];
      vmb[bb] = t.vm[bb];
    }
  }
  // scores before the query scale qs (> 0): sk[u][bb] for token t of block bb
  float sk[HPG][2], vs[2], vz[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const bool valid = t0 + 16 * bb + lt < tend;
#pragma unroll
    for (int u = 0; u < HPG; ++u) {
      const i32x4 c = sa[u][bb];  // limbs of weight 2^16, 2^8, 1
      const float raw = fmaf((float)c[0], 65536.0f, fmaf((float)c[1], 256.0f, (float)c[2]));
      float v;
      if (KCH) {
        v = raw;
      } else {
        const float off = key_offset<KC>() + (Meta<KM>::ZP ? kmb[bb].zero() : 0.0f);
        v = (off != 0.0f ? fmaf(-off, sq[u], raw) : raw) * kmb[bb].scale();
      }
      sk[u][bb] = valid ? v : NEG_INF;
    }
    vs[bb] = valid ? vmb[bb].scale() : 0.0f;
    vz[bb] = Meta<VM>::ZP && valid ? vmb[bb].zero() : 0.0f;
  }
  float f[HPG], p[HPG][2];
  bool moved = false;
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    f[u] = 1.0f;
    // The row maximum is needed only when it moves the reference max, which
    // is rare: test each lane's own scores first (qs > 0, so scaling keeps
    // the order) and reduce across the row only if some lane exceeds.
    if (__any(fmaxf(sk[u][0], sk[u][1]) * qs[u] > st.m[u] + M_SLACK)) {
      const float mt = row16_max(fmaxf(sk[u][0], sk[u][1])) * qs[u];
      if (mt > st.m[u] + M_SLACK) {  // move the reference max
        f[u] = exp2_fast(st.m[u] - mt);  // 0 when m = -inf
        st.m[u] = mt;
        moved = true;
      }
    }
    const float mu = st.m[u] == NEG_INF ? 0.0f : st.m[u];
    p[u][0] = exp2_fast(fmaf(sk[u][0], qs[u], -mu));
    p[u][1] = exp2_fast(fmaf(sk[u][1], qs[u], -mu));
    st.l[u] = st.l[u] * f[u] + (p[u][0] + p[u][1]);
  }
  // weights w = p s_V / R_u (8-bit scale codes: p u / 256, below p).  R_u
  // follows the head's largest p s_V lazily: it moves when some weight of the
  // tile exceeds R_SLACK, to that row's largest p s_V rounded up to a power
  // of two, so weights stay below 64.  Tracking the product, not s_V alone,
  // keeps the weights of the tokens that carry the output clear of fp16's
  // subnormal floor when a token with a far larger value scale but a
  // negligible attention weight shares the range.
  float w[HPG][2];
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    const float i0 = VM == MK_U8 ? 1.0f / 256.0f : st.invR[u];
    w[u][0] = p[u][0] * vs[0] * i0;
    w[u][1] = p[u][1] * vs[1] * i0;
  }
  if (VM != MK_U8) {
    bool up = false;
#pragma unroll
    for (int u = 0; u < HPG; ++u) up |= fmaxf(w[u][0], w[u][1]) > R_SLACK;
    if (__any(up)) {
#pragma unroll
      for (int u = 0; u < HPG; ++u) {
        const float pm = row16_max(fmaxf(p[u][0] * vs[0], p[u][1] * vs[1]));
        if (pm > st.R[u] * R_SLACK) {  // uniform over the row: its head's R moves
          const float Rn = pow2_ceil(pm);
          f[u] *= st.R[u] / Rn;
          st.R[u] = Rn;
          st.invR[u] = 1.0f / Rn;
          w[u][0] = p[u][0] * vs[0] * st.invR[u];
          w[u][1] = p[u][1] * vs[1] * st.invR[u];
          moved = true;
        }
      }
    }
  }
  if (__any(moved)) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[j][i] *= f[HPG == 2 ? (i >> 1) : 0];
#pragma unroll
    for (int u = 0; u < HPG; ++u) st.z[u] *= f[u];
  }
  // the weights as fp16 (high, low) pairs into LDS: pwr[u] is this lane's
  // (head, token) slot, 2 words: block 0, block 1
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    const float w0 = w[u][0], w1 = w[u][1];
    if (Meta<VM>::ZP) st.z[u] += w0 * vz[0] + w1 * vz[1];
    const half2v hi = __builtin_convertvector((float2v){w0, w1}, half2v);
    const half2v lo = __builtin_convertvector((float2v){w0 - (float)hi.x, w1 - (float)hi.y}, half2v);
    // word per block: high half in bits 0..15, low half in bits 16..31
    const uint32_t hb = __builtin_bit_cast(uint32_t, hi), lb = __builtin_bit_cast(uint32_t, lo);
    *(u32x2*)(pwr + 32 * u) = u32x2{perm(lb, hb, 0x05040100u), perm(lb, hb, 0x07060302u)};
  }
  // Other lanes of this wave read these words next; a wavefront's LDS
  // operations complete in issue order, so only the compiler needs fencing.
  __builtin_amdgcn_wave_barrier();
  // operand row r = (head, limb), k-group kg: tokens 4i + kg (i = 0..3) of
  // both blocks (k-slot e = 4 bb + i); they sit in slots 4kg .. 4kg+3 of the
  // exchange, 8 words, slot-major, block-minor
  const u32x4 A = *(const u32x4*)prd, B = *(const u32x4*)(prd + 4);
  const uint32_t M[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
  const uint32_t pa0 = perm(M[2], M[0], psel), pa1 = perm(M[6], M[4], psel);
  const uint32_t pa2 = perm(M[3], M[1], psel), pa3 = perm(M[7], M[5], psel);
  const half8 pf = as_h8(pa0, pa1, pa2, pa3);
  __builtin_amdgcn_wave_barrier();
  half8 vf[8];
  value_frags(t, vf, nm);
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf, vf[j], st.o[j], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Window tiles: bf16 keys and values, no metadata (bf16 MFMA)
// ---------------------------------------------------------------------------
struct WinRaw {
  u32x4 k[2][4];   // per block: token row c, features [32j + 8g, +8)
  u32x4 v[8];      // 8 tokens, features [8c, 8c + 8)
};

// Slot of bf16 token i (0 <= i < n, clamped) of a range: (r0 + i) mod ring in
// a ring, or r0 + i in a linear cache (ring = 0).
__device__ inline int ring_slot(int i, int nw, int r0, int ring) {
  i = i < nw ? i : nw - 1;
  const int s = r0 + i;
  return ring == 0 || s < ring ? s : s - ring;
}

// knew, vnew (or null): bf16 rows read in place of ring slot pslot (a
// decode step's new token, which another workgroup may still be writing
// there).
__device__ inline void load_win_tile(WinRaw& t, const uint16_t* kw, const uint16_t* vw, int t0,
                                     int nw, int r0, int ring, int c, int g,
                                     const uint16_t* knew = nullptr, const uint16_t* vnew = nullptr,
                                     int pslot = -1) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int sk = ring_slot(t0 + 16 * bb + c, nw, r0, ring);
    const uint16_t* kr = knew && sk == pslot ? knew : kw + (size_t)sk * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) t.k[bb][j] = __builtin_nontemporal_load((const u32x4*)(kr + 32 * j + 8 * g));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sv = ring_slot(t0 + 16 * bb + 4 * g + i, nw, r0, ring);
      const uint16_t* vr = vnew && sv == pslot ? vnew : vw + (size_t)sv * D;
      t.v[4 * bb + i] = __builtin_nontemporal_load((const u32x4*)(vr + 8 * c));
    }
  }
}

template <int G>
__device__ inline void compute_win_tile(const WinRaw& t, int t0, int tend, const bf16x8 qf[4],
                                        float qs, int g, int limb, Softmax& st) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 a = t.k[0][j], b = t.k[1][j];
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(a.x, a.y, a.z, a.w), qf[j], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(b.x, b.y, b.z, b.w), qf[j], s1, 0, 0, 0);
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int bb = e >> 2, i = e & 3;
    const float raw0 = bb ? s1[i] : s0[i];
    const float raw = raw0 + ror_g<G>(raw0);
    s[e] = (t0 + 16 * bb + 4 * g + i) < tend ? raw * qs : NEG_INF;
  }
  float mt = s[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mt = fmaxf(mt, s[e]);
  float mu;
  const float alpha = st.update_max(rows_max(mt), &mu);
  float p[8], lsum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2_fast(s[e] - mu);
    lsum += p[e];
  }
  st.l = st.l * alpha + lsum;
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
  }
  uint32_t pw[4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    uint16_t h[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float x = p[2 * pp + k];
      const uint16_t hi = bf16_rne(x);
      const uint16_t lo = bf16_rne(x - bf16_f32(hi));
      h[k] = limb ? lo : hi;
    }
    pw[pp] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
  }
  const bf16x8 pf = as_b8(pw[0], pw[1], pw[2], pw[3]);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t pr[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const u32x4 A = t.v[2 * pp], B = t.v[2 * pp + 1];
      const uint32_t a = A[j >> 1], b = B[j >> 1];
      pr[pp] = (j & 1) ? perm(b, a, 0x07060302u) : perm(b, a, 0x05040100u);
    }
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(pr[0], pr[1], pr[2], pr[3]), pf,
                                                      st.o[j], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Query setup: lane (c, g) holds query head (c mod G), as the high (limb 0)
// or low (limb 1) half, for the 32 features its key operand covers, read as
// runs of consecutive features with vector loads.
// ---------------------------------------------------------------------------
__device__ inline void unpack_bf16x8(const u32x4 r, float* out) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = __uint_as_float(r[k] << 16);
    out[2 * k + 1] = __uint_as_float(r[k] & 0xFFFF0000u);
  }
}

// Loads features run0 .. run0+nrun-1 (nrun 16 or 32) of one query row.
struct QRaw {
  u32x4 r[8];
};

template <bool BF16>
__device__ inline void load_q_run(QRaw& q, const void* base, size_t row, int start, int len,
                                  int slot) {
  // bf16: len/8 vectors of 8 values; f32: len/4 vectors of 4 values
  if constexpr (BF16) {
    const uint16_t* p = (const uint16_t*)base + row + start;
    for (int k = 0; k < len / 8; ++k) q.r[slot + k] = *(const u32x4*)(p + 8 * k);
  } else {
    const float* p = (const float*)base + row + start;
    for (int k = 0; k < len / 4; ++k) q.r[slot + k] = *(const u32x4*)(p + 4 * k);
  }
}

template <bool BF16>
__device__ inline void unpack_q(const QRaw& q, int nvals, float* out) {
  if constexpr (BF16) {
    for (int k = 0; k < nvals / 8; ++k) unpack_bf16x8(q.r[k], out + 8 * k);
  } else {
    for (int k = 0; k < nvals / 4; ++k)
      for (int i = 0; i < 4; ++i) out[4 * k + i] = __uint_as_float(q.r[k][i]);
  }
}

// Power-of-two scale that brings the head's largest |q| into [2^12, 2^13).
__device__ inline float q_norm_scale(float amax, float* inv) {
  if (!(amax > 0.0f)) {
    *inv = 1.0f;
    return 1.0f;
  }
  int ex;
  frexpf(amax, &ex);            // amax = m 2^ex, m in [0.5, 1)
  const int e = 13 - ex;
  *inv = ldexpf(1.0f, -e);
  return ldexpf(1.0f, e);
}

// Power-of-two scale 2^e that brings the head's largest |q| into
// [2^21, 2^22), so rint(q 2^e) splits into three int8 limbs; *inv = 2^-e.
__device__ inline float q_int_scale(float amax, float* inv) {
  if (!(amax > 0.0f)) {
    *inv = 1.0f;
    return 1.0f;
  }
  int ex;
  frexpf(amax, &ex);            // amax = m 2^ex, m in [0.5, 1)
  const int e = 22 - ex;
  *inv = ldexpf(1.0f, -e);
  return ldexpf(1.0f, e);
}

// ---------------------------------------------------------------------------
// Wave -> workgroup merge and partial write
// ---------------------------------------------------------------------------
template <int G>
struct Shared {
  float o[WAVES][G][D];
  float m[WAVES][G];
  float l[WAVES][G];
  // per wave: fp16 (high, low) weight pairs [head][token][block] of one tile
  uint32_t pw[WAVES][G == 8 ? 8 : 4][16][2];
};

template <int G>
__device__ inline void wave_finish(Softmax& st, float scale_out, int c, int g, int wave,
                                   Shared<G>& sh) {
  const float l = rows_sum(st.l);
  const float z = rows_sum(st.z);
  float ofs[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) ofs[j][i] = st.o[j][i] + ror_g<G>(st.o[j][i]);
  if (c < G) {
    const float k = l > 0.0f ? scale_out / l : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) sh.o[wave][c][32 * g + 8 * i + j] = (ofs[j][i] - z) * k;
    if (g == 0) {
      sh.m[wave][c] = l > 0.0f ? st.m : NEG_INF;
      sh.l[wave][c] = l;
    }
  }
}

// Wave epilogue of the quantized-token path: lane (t, g) writes features
// 8t + J of its row group's heads.
// scale_out[u]: what the accumulated weights of local head u are relative to
// (its R, or 256 S with 8-bit scale codes).
template <int G>
__device__ inline void row_finish(RowState<G>& st, const float* scale_out, int t, int g, int wave,
                                  Shared<G>& sh) {
  constexpr int HPG = RowState<G>::HPG;
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    const int head = G == 8 ? 2 * g + u : g;
    const float l = row16_sum(st.l[u]);
    const float z = row16_sum(st.z[u]);
    if (head < G) {
      const float k = l > 0.0f ? scale_out[u] / l : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sh.o[wave][head][8 * t + j] = (st.o[j][2 * u] + st.o[j][2 * u + 1] - z) * k;
      if (t == 0) {
        sh.m[wave][head] = l > 0.0f ? st.m[u] : NEG_INF;
        sh.l[wave][head] = l;
      }
    }
  }
}

__device__ inline void store_agent(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// The 4 waves' partials merged by log-sum-exp into partial row `split` of
// each of the G query heads, or, with split = DIRECT_OUT (the pair has this
// one partial), straight into the output: no arrival, no combine.
constexpr int DIRECT_OUT = -1;

template <int G>
__device__ inline void block_merge(const DecodeArgs& a, const Shared<G>& sh, int b, int h,
                                   int split) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64) {
    const int hh = idx / D, d = idx % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.m[w][hh]);
    float ws = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float e = sh.l[w][hh] > 0.0f ? sh.l[w][hh] * exp2_fast(sh.m[w][hh] - M) : 0.0f;
      ws += e;
      acc += e * sh.o[w][hh][d];
    }
    if (split == DIRECT_OUT) {
      a.out[((size_t)b * a.hq + (size_t)h * G + hh) * D + d] = ws > 0.0f ? acc / ws : 0.0f;
      continue;
    }
    const size_t row = ((size_t)b * a.hq + (size_t)h * G + hh) * a.nsp + split;
    // agent-scope stores write through this XCD's L2: the workgroup that
    // merges the splits may run on another XCD
    store_agent(a.part_o + row * D + d, ws > 0.0f ? acc / ws : 0.0f);
    if (d == 0) {
      store_agent(a.part_ml + 2 * row, M);
      store_agent(a.part_ml + 2 * row + 1, ws);
    }
  }
}

// Positions of a sequence: [0, nq) in the cache's format, [nq, nq + nm) in
// the middle tier, the last nw in bf16.
struct SeqInfo {
  int len, nw, nq, nm;
};

__device__ inline SeqInfo seq_info(const DecodeArgs& a, int b) {
  SeqInfo s;
  int len = a.seq_lens[b];
  len = len > 0 ? len : 0;
  const int cap = (a.paged ? a.bt_stride * 16 : a.max_tokens) + a.window + a.mid.tokens;
  len = len < cap ? len : cap;
  s.len = len;
  // quantized: whole token groups older than the window; the rest is bf16
  const int m = len - a.window > 0 ? len - a.window : 0;
  const int q = (m >> a.tgshift) << a.tgshift;
  // middle tier: the cache's format holds whole blocks of 32 positions at
  // least M older than the window
  const int r = q - a.mid.tokens;
  s.nq = a.mid.tokens ? (r > 0 ? r / MID_BLOCK * MID_BLOCK : 0) : q;
  s.nm = q - s.nq;
  s.nw = len - q;
  return s;
}

// ---------------------------------------------------------------------------
// Window split: the newest tokens, kept as bf16
// ---------------------------------------------------------------------------
// Attends the n bf16 tokens at slots ring_slot(i, n, r0, ring) of kw / vw
// with the G query heads of KV head h, and writes the partial row `row`
// (DIRECT_OUT: the output).
// PF: keep two tiles in flight per wave (long ranges of a bf16 cache).
template <int G, bool QB, bool PF>
__device__ void bf16_tokens(const DecodeArgs& a, int b, int h, const uint16_t* kw,
                            const uint16_t* vw, int r0, int ring, int nw, int row, Shared<G>& sh,
                            const uint16_t* knew = nullptr, const uint16_t* vnew = nullptr,
                            int pslot = -1) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (an SGPR): keeps each wave's token loop and its addressing scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int hh = c % G, limb = (c / G) & 1;
  const size_t qrow = ((size_t)b * a.hq + (size_t)h * G + hh) * D;
  // features 32j + 8g + e: four runs of 8
  QRaw qr;
  float qv[32];
  if constexpr (QB) {
#pragma unroll
    for (int j = 0; j < 4; ++j) qr.r[j] = *(const u32x4*)((const uint16_t*)a.q + qrow + 32 * j + 8 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) unpack_bf16x8(qr.r[j], qv + 8 * j);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qr.r[2 * j] = *(const u32x4*)((const float*)a.q + qrow + 32 * j + 8 * g);
      qr.r[2 * j + 1] = *(const u32x4*)((const float*)a.q + qrow + 32 * j + 8 * g + 4);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[4 * k + i] = __uint_as_float(qr.r[k][i]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(qv[k]));
  if (a.qbits == 8) {
    // integer query: the bf16 tokens are attended with Q s as well (s and
    // the quotient in fp64, Q s rounded once to fp32)
    const float hmax = rows_max(amax);
    const double s = hmax > 0.0f ? (double)hmax / 127.0 : 1.0;
    amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      qv[k] = (float)(fmin(fmax(rint((double)qv[k] / s), -127.0), 127.0) * s);
      amax = fmaxf(amax, fabsf(qv[k]));
    }
  }
  float inv;
  const float sc = q_norm_scale(rows_max(amax), &inv);
  const float qs = LOG2E * 0.08838834764831845f * inv;  // log2(e) / sqrt(128)
  bf16x8 qf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      uint16_t hv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x = qv[8 * j + 2 * pp + k] * sc;
        const uint16_t hi = bf16_rne(x);
        hv[k] = limb ? bf16_rne(x - bf16_f32(hi)) : hi;
      }
      w[pp] = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
    }
    qf[j] = as_b8(w[0], w[1], w[2], w[3]);
  }
  Softmax st;
  st.init(1.0f);
  const int per = (nw + WAVES * TILE - 1) / (WAVES * TILE) * TILE;
  const int w0 = wave * per, w1 = min(w0 + per, nw);
  if constexpr (PF) {
    // tile pairs, loads of tile i+2 issued after tile i's compute; the last
    // tile index is reused past the end, so every load stays in range (an L2
    // hit) and the loop has no exit in its middle
    const int ntile = w1 > w0 ? (w1 - w0 + TILE - 1) / TILE : 0;
    if (ntile > 0) {
      auto tl = [&](int i) { return w0 + min(i, ntile - 1) * TILE; };
      WinRaw t0r, t1r;
      load_win_tile(t0r, kw, vw, tl(0), nw, r0, ring, c, g);
      load_win_tile(t1r, kw, vw, tl(1), nw, r0, ring, c, g);
      int i = 0;
      for (; i + 1 < ntile; i += 2) {
        compute_win_tile<G>(t0r, tl(i), w1, qf, qs, g, limb, st);
        load_win_tile(t0r, kw, vw, tl(i + 2), nw, r0, ring, c, g);
        compute_win_tile<G>(t1r, tl(i + 1), w1, qf, qs, g, limb, st);
        load_win_tile(t1r, kw, vw, tl(i + 3), nw, r0, ring, c, g);
      }
      if (i < ntile) compute_win_tile<G>(t0r, tl(i), w1, qf, qs, g, limb, st);
    }
  } else {
    for (int t0 = w0; t0 < w1; t0 += TILE) {
      WinRaw t;
      load_win_tile(t, kw, vw, t0, nw, r0, ring, c, g, knew, vnew, pslot);
      compute_win_tile<G>(t, t0, w1, qf, qs, g, limb, st);
    }
  }
  wave_finish<G>(st, 1.0f, c, g, wave, sh);
  block_merge<G>(a, sh, b, h, row);
}

// The bf16 tokens of a quantized cache: the window and an open token group,
// positions [nq, nq + nw) in ring slots (nq + i) mod ring.
// In a decode step (a.k_new set, bf16 input) ring slot (seq_lens[b] - 1)
// mod ring, which receives the new token, is read from the input, whose bf16
// row is what the slot receives: the workgroup that writes the slot may
// still be reading the token it held.
template <int G, bool QB, bool STEP>
__device__ void window_split(const DecodeArgs& a, int b, int h, int q0, int nw, bool direct,
                             Shared<G>& sh) {
  const size_t head = ((size_t)b * a.hkv + h) * a.ring * D;
  const size_t in_row = ((size_t)b * a.hkv + h) * D;
  const bool step = STEP && a.k_new != nullptr;
  const int p = step ? a.seq_lens[b] - 1 : -1;
  bf16_tokens<G, QB, false>(a, b, h, a.k_win + head, a.v_win + head, q0 % a.ring, a.ring, nw,
                            direct ? DIRECT_OUT : a.n_split, sh,
                            step ? (const uint16_t*)a.k_new + in_row : nullptr,
                            step ? (const uint16_t*)a.v_new + in_row : nullptr,
                            p >= 0 ? p % a.ring : -1);
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine of the splits, by the last workgroup of each
// (sequence, KV head) to finish
// ---------------------------------------------------------------------------
// Splits of sequence b holding quantized tokens (at most the n_split
// launched; a longer sequence is an overflow of the plan).
struct Plan {
  int ns;
  bool overflow, win, mid;
  int total;  // workgroups that write a partial
};

__device__ inline Plan plan_of(const DecodeArgs& a, const SeqInfo& si) {
  Plan p;
  const int need = (si.nq + a.split_tokens - 1) / a.split_tokens;
  p.overflow = need > a.n_split;
  p.ns = p.overflow ? a.n_split : need;
  p.win = si.nw > 0;
  p.mid = si.nm > 0;
  p.total = p.ns + (p.win ? 1 : 0) + (p.mid ? 1 : 0);
  return p;
}

// Partial row slots of a (sequence, query head): the splits in 0 ..
// n_split - 1, the bf16 item in n_split (if the cache has a ring), the middle
// tier after it.
__device__ inline int mid_row(const DecodeArgs& a) { return a.n_split + (a.ring ? 1 : 0); }

// Slot of the j-th partial row that a pair's combine reads: its splits,
// then its bf16 item, then its middle tier (those it has).
__device__ inline int partial_slot(const DecodeArgs& a, const Plan& pl, int j) {
  if (j < pl.ns) return j;
  return (j == pl.ns && pl.win) ? a.n_split : mid_row(a);
}

__device__ inline float2 load_agent2(const float* p) {
  const uint64_t u = __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32))};
}

__device__ inline void write_combined(const DecodeArgs& a, int b, int h, int G, int hh, const Plan& pl,
                                      float ws, float2 acc, int lane) {
  float2 r;
  if (pl.overflow) {
    r.x = r.y = __builtin_nanf("");
  } else if (ws > 0.0f) {
    r.x = acc.x / ws;
    r.y = acc.y / ws;
  } else {
    r.x = r.y = 0.0f;
  }
  *(float2*)(a.out + ((size_t)b * a.hq + (size_t)h * G + hh) * D + 2 * lane) = r;
}

// Wave w merges query heads w, w + 4 (G = 8) of KV head h.  Up to 64
// partial rows: lane j reads row j's (m, l) while every lane reads its two
// output features of the first CB rows, all in flight together (one memory
// round trip); further rows follow CB at a time.
template <int G>
__device__ void combine_heads(const DecodeArgs& a, int b, int h, const Plan& pl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nr = pl.total;  // partial rows: splits, then the window, then the middle tier
  if (nr <= 64) {
    constexpr int HPW = G > WAVES ? G / WAVES : 1;
    constexpr int CB = 16;
    if (wave >= G) return;
    size_t row0[HPW];
    float2 ml[HPW], v[HPW][CB];
    auto prow = [&](int u, int j) { return row0[u] + partial_slot(a, pl, j); };
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      row0[u] = ((size_t)b * a.hq + (size_t)h * G + wave + u * WAVES) * a.nsp;
      ml[u] = load_agent2(a.part_ml + 2 * prow(u, min(lane, nr - 1)));
#pragma unroll
      for (int k = 0; k < CB; ++k) v[u][k] = load_agent2(a.part_o + prow(u, min(k, nr - 1)) * D + 2 * lane);
    }
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
      const bool mine = lane < nr;
      float M = mine ? ml[u].x : NEG_INF;
      for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      const float e = mine && ml[u].y > 0.0f ? ml[u].y * exp2_fast(ml[u].x - M) : 0.0f;
      float ws = e;
      for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
      float2 acc = {0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < CB; ++k) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), k));
        acc.x += w * v[u][k].x;  // e is 0 on lanes k >= nr
        acc.y += w * v[u][k].y;
      }
      for (int k0 = CB; k0 < nr; k0 += CB) {
        float2 x[CB];
#pragma unroll
        for (int k = 0; k < CB; ++k) x[k] = load_agent2(a.part_o + prow(u, min(k0 + k, nr - 1)) * D + 2 * lane);
#pragma unroll
        for (int k = 0; k < CB; ++k) {
          const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), k0 + k));
          acc.x += w * x[k].x;
          acc.y += w * x[k].y;
        }
      }
      write_combined(a, b, h, G, wave + u * WAVES, pl, ws, acc, lane);
    }
    return;
  }
  for (int hh = wave; hh < G; hh += WAVES) {
    const size_t row0 = ((size_t)b * a.hq + (size_t)h * G + hh) * a.nsp;
    auto prow = [&](int j) { return row0 + partial_slot(a, pl, j); };
    float M = NEG_INF;
    for (int j = lane; j < nr; j += 64) M = fmaxf(M, load_agent(a.part_ml + 2 * prow(j)));
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float ws = 0.0f;
    float2 acc = {0.0f, 0.0f};
    for (int j0 = 0; j0 < nr; j0 += 64) {
      const int j = j0 + lane;
      float e = 0.0f;
      if (j < nr) {
        const size_t rj = prow(j);
        const float m = load_agent(a.part_ml + 2 * rj), l = load_agent(a.part_ml + 2 * rj + 1);
        e = l > 0.0f ? l * exp2_fast(m - M) : 0.0f;
      }
      ws += e;
      const int cnt = min(64, nr - j0);
      for (int k0 = 0; k0 < cnt; k0 += 8) {
        float2 v[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {  // eight loads in flight
          const int k = min(k0 + kk, cnt - 1);
          const float* po = a.part_o + prow(j0 + k) * D + 2 * lane;
          v[kk] = float2{load_agent(po), load_agent(po + 1)};
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const float ek = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), min(k0 + kk, 63)));
          const float w = k0 + kk < cnt ? ek : 0.0f;
          acc.x += w * v[kk].x;
          acc.y += w * v[kk].y;
        }
      }
    }
    for (int o = 32; o > 0; o >>= 1) ws += __shfl_xor(ws, o);
    write_combined(a, b, h, G, hh, pl, ws, acc, lane);
  }
}

// After this workgroup's partial (or, in a decode step with a window, its
// two partials) is written: count it in the arrival counter of (b, h); the
// workgroup that brings the count to pl.total resets the counter and merges.  Each thread first waits for its own partial stores to
// complete (they write through to memory), so the counter cannot run ahead
// of the data it announces; no cache-wide fence is needed.
template <int G>
__device__ void arrive_and_combine(const DecodeArgs& a, int b, int h, const Plan& pl, int* flag,
                                   uint32_t partials = 1) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = a.counters + (size_t)b * a.hkv + h;
    const uint32_t prev = __hip_atomic_fetch_add(cnt, partials, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev + partials == (uint32_t)pl.total;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  phase_stamp(a.stamps, 5);
  if (*flag) combine_heads<G>(a, b, h, pl);
#ifdef KVQ_PHASE_STAMPS
  phase_stamp(a.stamps, 6, (__builtin_amdgcn_s_memrealtime() << 1) | (*flag ? 1u : 0u));
#endif
}

// ---------------------------------------------------------------------------
// Workgroup -> work item.  Items in dispatch order, largest first, so that
// with sequences of mixed length the last workgroups to start are the
// shortest ones and the compute units finish together:
//   1. every full chunk of split_tokens quantized tokens: sequence-major,
//      then KV-head-major, the chunk order of each (sequence, KV head) pair
//      rotated by the pair index (consecutive workgroups go to different
//      XCDs; this way the chunks that start together on one XCD lie at
//      different offsets of their pairs),
//   2. with a middle tier, one item per (sequence, KV head) for it (up to
//      M + 31 int8 tokens: about a full chunk's work or less),
//   3. the remainder chunk of each sequence, by size class from large to
//      small (NSIZE classes of split_tokens / NSIZE tokens),
//   4. one item per (sequence, KV head) for the bf16 window, if any,
//   5. workgroups past the last item return at once.
// Every wave derives the workgroup's item on its own from the sequence
// lengths (one length per lane, 64 sequences per pass), with wave scans and
// ballots: no workgroup barrier before the first tile loads.
// ---------------------------------------------------------------------------
constexpr int NSIZE = 32;

struct Item {
  int kind;  // 0 quantized chunk, 1 bf16 tokens, 2 nothing, 3 middle tier
  int b, h, split;
  SeqInfo si;
};

struct Chunks {
  int full, part, rem;  // full chunks, remainder chunk (0/1), its tokens
};

__device__ inline Chunks chunks_of(const DecodeArgs& a, const SeqInfo& si) {
  Chunks c;
  const int S = a.split_tokens;
  const int ns = min((si.nq + S - 1) / S, a.n_split);  // a longer sequence overflows the plan
  c.full = min(si.nq / S, ns);
  c.part = ns - c.full;
  c.rem = c.part ? si.nq - c.full * S : 0;
  return c;
}

__device__ inline int size_class(const DecodeArgs& a, int rem) {
  return NSIZE - 1 - min(NSIZE - 1, (int)(((long long)rem * NSIZE) / a.split_tokens));
}

// Inclusive scan over the 64 lanes: shifts within rows of 16, then the row
// totals carried across rows.
__device__ inline int wave_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

__device__ inline int lane_of(uint64_t m) { return __builtin_ctzll(m); }
__device__ inline int rdl(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

__device__ inline SeqInfo read_si(const SeqInfo& s, int l) {
  return SeqInfo{rdl(s.len, l), rdl(s.nw, l), rdl(s.nq, l), rdl(s.nm, l)};
}

// hist: this wave's NSIZE counters in LDS
__device__ Item map_item(const DecodeArgs& a, int item, int* hist, bool tier) {
  const int lane = threadIdx.x & 63;
  Item it{2, 0, 0, 0, {0, 0, 0, 0}};
  if (lane < NSIZE) hist[lane] = 0;
  __builtin_amdgcn_wave_barrier();
  // 1. full chunks
  int carry = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    SeqInfo si{0, 0, 0};
    Chunks c{0, 0, 0};
    if (b < a.batch) {
      si = seq_info(a, b);
      c = chunks_of(a, si);
    }
    const int inc = wave_scan(c.full);
    const long long lo = (long long)a.hkv * (carry + inc - c.full);
    const uint64_t m = __ballot(item >= lo && item < lo + (long long)a.hkv * c.full);
    if (m) {
      const int L = lane_of(m);
      const int n = rdl(c.full, L);
      const int j = item - (int)(__builtin_amdgcn_readlane((int)lo, L));
      it.kind = 0;
      it.b = b0 + L;
      it.h = j / n;
      it.split = (j % n + it.b * a.hkv + it.h) % n;
      it.si = read_si(si, L);
      return it;
    }
    if (c.part) atomicAdd(&hist[size_class(a, c.rem)], 1);
    carry += rdl(inc, 63);
  }
  __builtin_amdgcn_wave_barrier();
  long long r = item - (long long)a.hkv * carry;
  if (tier) {  // 2. middle tiers
    if (r < (long long)a.batch * a.hkv) {
      it.kind = 3;
      it.b = (int)(r / a.hkv);
      it.h = (int)(r % a.hkv);
      it.split = mid_row(a);
      it.si = seq_info(a, it.b);
      return it;
    }
    r -= (long long)a.batch * a.hkv;
  }
  // 3. remainder chunks: the rank-th one in (size class, sequence) order
  const int cnt = lane < NSIZE ? hist[lane] : 0;
  const int cinc = wave_scan(cnt);
  const int np = rdl(cinc, 63);
  if (r < (long long)a.hkv * np) {
    const int rank = (int)(r / a.hkv);
    const int cls = lane_of(__ballot(lane < NSIZE && cinc > rank));
    int k = rank - (rdl(cinc, cls) - rdl(cnt, cls));
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
      const int b = b0 + lane;
      SeqInfo si{0, 0, 0};
      Chunks c{0, 0, 0};
      if (b < a.batch) {
        si = seq_info(a, b);
        c = chunks_of(a, si);
      }
      const uint64_t m = __ballot(c.part && size_class(a, c.rem) == cls);
      const int here = __builtin_popcountll(m);
      if (k < here) {
        const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const int L = lane_of(__ballot(((m >> lane) & 1) && before == k));
        it.kind = 0;
        it.b = b0 + L;
        it.h = (int)(r % a.hkv);
        it.split = rdl(c.full, L);
        it.si = read_si(si, L);
        return it;
      }
      k -= here;
    }
    return it;  // not reached: the rank-th remainder chunk exists
  }
  r -= (long long)a.hkv * np;
  if (a.ring && r < (long long)a.batch * a.hkv) {  // 4. bf16 items (window, open group)
    it.kind = 1;
    it.b = (int)(r / a.hkv);
    it.h = (int)(r % a.hkv);
    it.split = a.n_split;
    it.si = seq_info(a, it.b);
  }
  return it;
}

// Attends quantized positions [tok0, tok1) of (sequence b, KV head h) with
// the G query heads of h and writes partial row `row` (DIRECT_OUT: the
// output).  The codes and
// metadata live at kc, vc, km, vm: token slot head_tok + position
// (contiguous), through the block table (PAGED), or in a ring of rblk
// 16-token blocks (RING, the middle tier); nend bounds the blocks read.
struct NoPre {
  __device__ void operator()() const {}
};

template <int KC, int KM, bool KCH, int VC, int VM, int G, bool PAGED, bool QB, bool RING,
          bool PT, typename Pre = NoPre>
__device__ void quant_range(const DecodeArgs& a, int b, int h, int tok0, int tok1, int nend,
                            int row, const uint8_t* kc, const uint8_t* vc, const uint8_t* km,
                            const uint8_t* vm, size_t head_tok, int rblk, Shared<G>& sh,
                            int hold_pos = -1, Pre pre = Pre()) {
  const int lane = threadIdx.x & 63;
  // wave-uniform (an SGPR): keeps each wave's token loop and its addressing scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lt = lane & 15, g = lane >> 4;
  constexpr int HPG = RowState<G>::HPG;

  // 1. query (and per-channel key scale) loads, issued first.  Score operand
  //    row lt holds limb qlimb (0..2) of query head qhead(u) in row tile u;
  //    the lane covers features [32g, 32g + 32) of it.
  const int hl = lt >> 2, qlimb = lt & 3;
  int qhead[HPG];
  QRaw qr[HPG], cr;
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    const int hd = G == 8 ? 2 * hl + u : hl;
    qhead[u] = hd < G ? hd : G - 1;
    const size_t qrow = ((size_t)b * a.hq + (size_t)h * G + qhead[u]) * D;
    load_q_run<QB>(qr[u], a.q, qrow, 32 * g, 32, 0);
  }
  const size_t crow = ((size_t)b * a.hkv + h) * D;
  if (KCH) load_q_run<false>(cr, a.k_chan, crow, 32 * g, 32, 0);
  // 8-bit key scale codes: their per-head super-scale joins the score scale
  const float ksup = KM == MK_U8 ? a.k_super[(size_t)b * a.hkv + h] : 1.0f;
  const bool qvalid = qlimb < 3 && (G == 8 || hl < G);

  // 2. the first two tiles of this wave's range, in flight while the query
  //    is prepared
  Addr ad;
  ad.k = kc;
  ad.v = vc;
  ad.km = km;
  ad.vm = vm;
  ad.num_blocks = a.num_blocks;
  ad.ku = a.kk.unit;
  ad.vu = a.vk.unit;
  ad.hkv = a.hkv;
  ad.h = h;
  ad.gs = a.tgshift;
  ad.nblk = (nend + 15) >> 4;
  ad.rblk = rblk;
  ad.blk0 = 0;
  ad.ent[0] = ad.ent[1] = 0;
  ad.head_tok = head_tok;
  const LaneOff lo = lane_offsets<KC, KM, VC, VM>(lt, g, a.tgshift);
  // Tiles of the chunk per wave.  ILV: dealt round-robin, wave w takes tiles
  // w, w + WAVES, w + 2 WAVES, ... (its k-th tile starts at w0 + k STRIDE),
  // so that the workgroup's waves read adjacent tiles at the same time, and
  // every wave masks against the chunk's end.  Otherwise each wave streams
  // a contiguous quarter of the chunk.  Measured on one MI355X: with 8-bit
  // keys round-robin is faster (gqa_int8 20.1 -> 19.2-19.6 us, asym_kv
  // 257.5 -> 252.6 us, paged_mixed unchanged); with narrower tokens it is
  // not (int4_asym 51.5 -> 52.7 us over six runs, the 2-bit and tiered
  // workloads unchanged).  A plain read of 268 MB in this launch shape
  // streamed 6.46 TB/s round-robin against 6.08 in quarters.
  constexpr int ROWB = Codes<KC>::ROW + Codes<VC>::ROW;
  constexpr bool ILV = ROWB >= 192;
  constexpr int STRIDE = ILV ? WAVES * TILE : TILE;
  int w0, w1, ntile;
  if constexpr (ILV) {
    w0 = __builtin_amdgcn_readfirstlane(tok0 + wave * TILE);
    w1 = tok1;
    const int nchunk = tok1 > tok0 ? (tok1 - tok0 + TILE - 1) / TILE : 0;
    ntile = __builtin_amdgcn_readfirstlane(nchunk > wave ? (nchunk - wave + WAVES - 1) / WAVES : 0);
  } else {
    const int per = (tok1 - tok0 + WAVES * TILE - 1) / (WAVES * TILE) * TILE;
    w0 = __builtin_amdgcn_readfirstlane(tok0 + wave * per);
    w1 = __builtin_amdgcn_readfirstlane(min(w0 + per, tok1));
    ntile = w1 > w0 ? (w1 - w0 + TILE - 1) / TILE : 0;
  }
  ad.ilv = ILV;
  if constexpr (PAGED) {  // this wave's block-table entries (64 tiles, 128 blocks)
    const int32_t* row = a.block_table + (size_t)b * a.bt_stride;
    const int lim = a.bt_stride - 1;
    ad.blk0 = w0 >> 4;
    if constexpr (ILV) {
      ad.ent[0] = row[min(ad.blk0 + 2 * WAVES * (lane >> 1) + (lane & 1), lim)];
      ad.ent[1] = row[min(ad.blk0 + 2 * WAVES * (32 + (lane >> 1)) + (lane & 1), lim)];
    } else {
      ad.ent[0] = row[min(ad.blk0 + lane, lim)];
      ad.ent[1] = row[min(ad.blk0 + 64 + lane, lim)];
    }
  }
  // The scheduling barriers keep each tile's loads together and in order
  // (first tile, second, ..., then the refills): the compiler derives its
  // wait counts from that order, and interleaved loads would make every wait
  // in the loop a wait for all of them.
  constexpr int NB = ROWB >= 256 ? KVQ_NB8 : ROWB >= 192 ? KVQ_NB6 : ROWB >= 128 ? KVQ_NB4 : KVQ_NB2;
  // pre (a decode step's move of the token leaving the window into the
  // cache, at hold_pos): run by the wave whose range holds that position
  // (wave 0 if none does), so that its own later load of the position reads
  // the stores.  Wave memory operations complete in issue order: a load
  // issued after the wave has waited for data that it requested after the
  // stores comes after them.  The refill of tile j follows the wait for
  // tile j - NB, so a position in tile 2 NB or later may be moved while the
  // first tiles are in flight; one in an earlier tile is moved first and
  // waited for.
  const bool mine = ILV ? (hold_pos - tok0) / TILE % WAVES == wave : hold_pos >= w0 && hold_pos < w1;
  const bool mover = hold_pos >= 0 && (hold_pos >= tok0 && hold_pos < tok1 ? mine : wave == 0);
  const bool move_first = mover && hold_pos < w0 + 2 * NB * STRIDE;
  if (move_first) {
    pre();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  TileRaw<KC, KM, VC, VM, PT> buf[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    load_tile<PAGED, RING>(buf[k], ad, w0 + k * STRIDE, w1, lo);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (mover && !move_first) pre();
  __builtin_amdgcn_sched_barrier(0);

  // 3. query operand: Q = rint(q 2^e) per head, |Q| < 2^22, as three int8
  //    limbs Q = l0 2^16 + l1 2^8 + l2 (each in [-128, 127])
  long qa[HPG][4];
  float qs_row[HPG], sq_row[HPG];
  float cv[32];
  if (KCH) unpack_q<false>(cr, 32, cv);
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    float qv[32];
    unpack_q<QB>(qr[u], 32, qv);
    if (KCH) {
#pragma unroll
      for (int n = 0; n < 32; ++n) qv[n] *= cv[n];  // per-channel key scale moved onto the query
    }
    float amax = 0.0f;
#pragma unroll
    for (int n = 0; n < 32; ++n) amax = fmaxf(amax, fabsf(qv[n]));
    const float hmax = rows_max(amax);  // max over the row's 4 lanes: the head's
    float inv, sc = 0.0f;
    // integer query: s = fl64(amax / 127), Q = clamp(rint(fl64(q / s))), the
    // cache quantizer's fp64 rule; the score scale takes s rounded to fp32
    const double s64 = hmax > 0.0f ? (double)hmax / 127.0 : 1.0;
    if (a.qbits == 8)
      inv = (float)s64;
    else
      sc = q_int_scale(hmax, &inv);
    float qsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint64_t pk = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = qv[key_feature<KC>(j, 0, e)];
        const float x = a.qbits == 8 ? (float)fmin(fmax(rint((double)y / s64), -127.0), 127.0)
                                     : rintf(y * sc);
        qsum += x;
        const int Q = (int)x;
        const int l2 = (int)(int8_t)(Q & 0xFF);
        const int Q1 = (Q - l2) >> 8;
        const int l1 = (int)(int8_t)(Q1 & 0xFF);
        const int l0 = (Q1 - l1) >> 8;
        const int lv = qlimb == 0 ? l0 : (qlimb == 1 ? l1 : l2);
        pk |= (uint64_t)(uint8_t)(qvalid ? lv : 0) << (8 * e);
      }
      qa[u][j] = (long)pk;
    }
    qs_row[u] = LOG2E * 0.08838834764831845f * inv * ksup;  // log2(e) / sqrt(128) / 2^e (or s)
    sq_row[u] = rows_sum(qsum);
  }
  // score scale and query sum of each head, from the lane of its limb-0 row
  // (row 4 hl, k-group 0) to the lanes that score that head (row group hl)
  float qs[HPG], sumq[HPG];
#pragma unroll
  for (int u = 0; u < HPG; ++u) {
    qs[u] = 0.0f;
    sumq[u] = 0.0f;
#pragma unroll
    for (int src = 0; src < 4; ++src) {
      const float a_qs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qs_row[u]), 4 * src));
      const float a_sq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sq_row[u]), 4 * src));
      const bool mine = src == g;  // row tile u's head of row group g sits in row 4g
      qs[u] = mine ? a_qs : qs[u];
      sumq[u] = mine ? a_sq : sumq[u];
    }
  }
  // output operand rows (P^T): head and fp16 limb of row lt
  const int ph = row_head<G>(lt), plimb = row_limb<G>(lt);
  const bool pvalid = ph < G && plimb < 2;
  const int phc = ph < G ? ph : G - 1;
  // weight exchange: this lane writes (head of row group g, token lt), reads
  // operand row lt's head, tokens 4i + g
  // token lt goes to exchange slot 4 (lt mod 4) + lt / 4
  uint32_t* pwr = &sh.pw[wave][G == 8 ? 2 * g : g][4 * (lt & 3) + (lt >> 2)][0];
  const uint32_t* prd = &sh.pw[wave][phc][4 * g][0];
  const uint32_t psel = !pvalid ? 0x0c0c0c0cu : (plimb == 0 ? 0x05040100u : 0x07060302u);

  phase_stamp(a.stamps, 2);
  // 4. stream the range: compute one buffer, refill it two tiles ahead
  NibbleMasks nm;
  nm.init();
  RowState<G> st;
  st.init(__uint_as_float(0x00800000u));  // 2^-126
  // Groups of NB tiles, then the remaining ones.  No exit in the middle of
  // the loop body: an edge from there back to the loop head would make the
  // compiler wait there as if only the first refill were in flight.
  int t = w0;
  for (int i = 0; i < ntile / NB; ++i) {
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      compute_tile<KC, KM, KCH, VC, VM, G>(buf[k], t + k * STRIDE, w1, qa, qs, sumq, lt, g, psel,
                                           prd, pwr, nm, st);
      __builtin_amdgcn_sched_barrier(0);
      load_tile<PAGED, RING>(buf[k], ad, t + (k + NB) * STRIDE, w1, lo);
      __builtin_amdgcn_sched_barrier(0);
    }
    t += NB * STRIDE;
  }
  const int rem = ntile - (ntile / NB) * NB;
#pragma unroll
  for (int k = 0; k < NB - 1; ++k)
    if (k < rem)
      compute_tile<KC, KM, KCH, VC, VM, G>(buf[k], t + k * STRIDE, w1, qa, qs, sumq, lt, g, psel,
                                           prd, pwr, nm, st);
  phase_stamp(a.stamps, 3);
  float scale_out[HPG];
#pragma unroll
  for (int u = 0; u < HPG; ++u)
    scale_out[u] = VM == MK_U8 ? 256.0f * a.v_super[(size_t)b * a.hkv + h] : st.R[u];
  row_finish<G>(st, scale_out, lt, g, wave, sh);
  block_merge<G>(a, sh, b, h, row);
  phase_stamp(a.stamps, 4);
}


// Decode step: quantizes the new token of (b, h), at position p, into the
// cache with the append kernels' own quantizer (wave 0 the key, wave 1 the
// value), and waits until the stores are done, so that this workgroup's
// tile loads, which cover p, read it.  Only runs for per-token scales
// without a window, a middle tier or token groups (checked on the host).
__device__ void step_append(const DecodeArgs& a, int b, int h, int p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (w < 2) {
    const TensorKind k = w == 0 ? a.kk : a.vk;
    const size_t head = (size_t)b * a.hkv + h;
    const void* src = w == 0 ? a.k_new : a.v_new;
    auto ld = [&](int, double& x0, double& x1) {
      x0 = qz::load_in(src, head * D + 2 * lane, a.in_bf16);
      x1 = qz::load_in(src, head * D + 2 * lane + 1, a.in_bf16);
    };
    uint8_t* codes = const_cast<uint8_t*>(w == 0 ? a.k_codes : a.v_codes);
    uint8_t* meta = const_cast<uint8_t*>(w == 0 ? a.k_meta : a.v_meta);
    auto row = [&](int pos) { return qz::code_row(a, k, codes, b, h, pos); };
    qz::quantize_group(k, ld, row, p, 1, qz::meta_elem(a, k, meta, b, h, p), nullptr, 1.0f, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
}

// Decode step with a bf16 window (token groups of 1, no middle tier, bf16
// input), run by one wave: as kvq_quantize_append with one new token, the
// token leaving the window (position p - W, from its ring slot) is quantized
// into the cache unless it lies past the capacity (evict: the sequence has
// quantized tokens), then the new token (position p) is written into the
// ring slot that frees (the ring holds W slots); the key, then the value.
// The stores are not waited for: the caller orders its later loads of
// position p - W behind them.
__device__ void step_window(const DecodeArgs& a, int b, int h, bool evict) {
  const int lane = threadIdx.x & 63;
  const int p = a.seq_lens[b] - 1;
  if (p < 0) return;
  const size_t head = (size_t)b * a.hkv + h;
  const int e = p - a.window;
  const int cap = a.paged ? a.bt_stride * 16 : a.max_tokens;
  for (int w = 0; w < 2; ++w) {
    uint16_t* ring = const_cast<uint16_t*>(w == 0 ? a.k_win : a.v_win);
    if (evict && e >= 0 && e < cap) {
      const TensorKind k = w == 0 ? a.kk : a.vk;
      const size_t row = (head * a.ring + (size_t)(e % a.ring)) * D;
      auto ld = [&](int, double& x0, double& x1) {
        x0 = qz::bf16_bits_to_f32(ring[row + 2 * lane]);
        x1 = qz::bf16_bits_to_f32(ring[row + 2 * lane + 1]);
      };
      uint8_t* codes = const_cast<uint8_t*>(w == 0 ? a.k_codes : a.v_codes);
      uint8_t* meta = const_cast<uint8_t*>(w == 0 ? a.k_meta : a.v_meta);
      auto crow = [&](int pos) { return qz::code_row(a, k, codes, b, h, pos); };
      qz::quantize_group(k, ld, crow, e, 1, qz::meta_elem(a, k, meta, b, h, e), nullptr, 1.0f,
                         lane);
    }
    // the ring slot of p is the one e held: its values were read above
    const uint16_t* src = (const uint16_t*)(w == 0 ? a.k_new : a.v_new);
    const size_t out_row = (head * a.ring + (size_t)(p % a.ring)) * D;
    for (int i = lane; i < D; i += 64) ring[out_row + i] = src[head * D + i];
  }
}

// Formats whose decode step the host fuses into the decode kernel: per-token
// fp32 / fp16 scales (with or without a zero point), no middle tier.
template <int KM, bool KCH, int VM, bool TIER>
constexpr bool step_format() {
  return !TIER && !KCH && (KM == MK_F32 || KM == MK_F32Z || KM == MK_F16 || KM == MK_F16Z) &&
         (VM == MK_F32 || VM == MK_F32Z || VM == MK_F16 || VM == MK_F16Z);
}

// STEPK: the decode step's kernel (a.k_new set), a separate instantiation so
// that the plain decode carries none of the step's code.
template <int KC, int KM, bool KCH, int VC, int VM, int G, bool PAGED, bool QB, bool TIER,
          bool STEPK>
__global__ void __launch_bounds__(256, KVQ_MINW) decode_split(DecodeArgs a) {
  constexpr bool STEP = STEPK && step_format<KM, KCH, VM, TIER>();
  __shared__ Shared<G> sh;
  // 1-D grid of work items, largest first (map_item).  Consecutive items,
  // which the hardware sends to different XCDs, are mostly the KV heads of
  // one chunk.
  __shared__ int last_flag;
  __shared__ int hist[WAVES][NSIZE];
  // workgroup p < batch * hkv also writes the (zero) output of pair p if
  // its sequence is empty
  phase_stamp(a.stamps, 0);
#ifdef KVQ_PHASE_STAMPS
  {
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    phase_stamp(a.stamps, 7, ((unsigned long long)xcc << 32) | hw);
  }
#endif
  const bool zduty = blockIdx.x < (unsigned)(a.batch * a.hkv);
  const int zlen = zduty ? a.seq_lens[blockIdx.x / a.hkv] : 1;
  const Item it = map_item(a, blockIdx.x, hist[threadIdx.x >> 6], TIER);
  phase_stamp(a.stamps, 1);
  if (zduty && zlen <= 0) {
    const int zb = blockIdx.x / a.hkv, zh = blockIdx.x % a.hkv;
    for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64)
      a.out[((size_t)zb * a.hq + (size_t)zh * G) * D + idx] = 0.0f;
  }
  if (it.kind == 2) return;
  const int b = it.b, h = it.h, split = it.split;
  const SeqInfo si = it.si;
  const Plan pl = plan_of(a, si);
  // a pair whose tokens one workgroup attends writes its output directly
  const bool direct = pl.total == 1 && !pl.overflow;
  if (it.kind == 1) {
    if (si.nw > 0) {
      // decode step with a window, a sequence with no quantized token: the
      // new token into the ring (nothing leaves the window); the window
      // itself reads it from the input
      if (STEP && a.k_new != nullptr && si.nq == 0) {
        if (threadIdx.x < 64) step_window(a, b, h, false);  // the window reads p from the input
      }
      window_split<G, QB, STEP>(a, b, h, si.nq + si.nm, si.nw, direct, sh);
      if (!direct) arrive_and_combine<G>(a, b, h, pl, &last_flag);
    }
    return;
  }
  const size_t pair = (size_t)b * a.hkv + h;
  if constexpr (TIER) {
    if (it.kind == 3) {  // the middle tier: int8 codes, fp32 scales, in its ring
      if (si.nm > 0) {
        quant_range<CK_I8, MK_F32, false, CK_I8, MK_F32, G, false, QB, true, true>(
            a, b, h, si.nq, si.nq + si.nm, si.nq + si.nm, direct ? DIRECT_OUT : split, a.mid.k,
            a.mid.v, (const uint8_t*)a.mid.ks, (const uint8_t*)a.mid.vs, pair * a.mid.slots,
            a.mid.slots >> 4, sh);
        if (!direct) arrive_and_combine<G>(a, b, h, pl, &last_flag);
      }
      return;
    }
  }
  const int tok0 = split * a.split_tokens;
  const int tok1 = min(tok0 + a.split_tokens, si.nq);
  // decode step with a window: the workgroup of the pair's last chunk, which
  // holds the position leaving the window, moves it into the cache and the
  // new token into the ring; quant_range orders the load of that position's
  // tile behind the stores
  if constexpr (STEP) {
    const bool evict = a.k_new != nullptr && a.ring && split == pl.ns - 1;
    if (a.k_new != nullptr) {
      if (!a.ring) {
        // the decode step's new token, at position seq_lens[b] - 1 of the
        // unclamped length: the split that holds it stores it first (the
        // last split if the sequence overflows the plan).  A position at or
        // past the capacity is not stored, as kvq_quantize_append skips it;
        // si.len is the length clamped to the capacity.
        const int p = a.seq_lens[b] - 1;
        if (p >= 0 && p < si.len && split == min(p / a.split_tokens, pl.ns - 1))
          step_append(a, b, h, p);
      }
    }
    // the wave whose range holds the position leaving the window moves the
    // tokens (quant_range decides when)
    auto move = [&]() { step_window(a, b, h, true); };
    quant_range<KC, KM, KCH, VC, VM, G, PAGED, QB, false, TIER>(
        a, b, h, tok0, tok1, si.nq, direct ? DIRECT_OUT : split, a.k_codes, a.v_codes, a.k_meta,
        a.v_meta, PAGED ? 0 : pair * a.max_tokens, 0, sh, evict ? si.nq - 1 : -1, move);
  } else {
    quant_range<KC, KM, KCH, VC, VM, G, PAGED, QB, false, TIER>(
        a, b, h, tok0, tok1, si.nq, direct ? DIRECT_OUT : split, a.k_codes, a.v_codes, a.k_meta,
        a.v_meta, PAGED ? 0 : pair * a.max_tokens, 0, sh);
  }
  if (!direct) arrive_and_combine<G>(a, b, h, pl, &last_flag);
}

// Decode over an unquantized (bf16) contiguous cache, e.g. the output of
// kvq_dequantize: the same work items (chunks, largest first) and the same
// combine as decode_split, the tokens attended by bf16_tokens.
template <int G, bool QB>
__global__ void __launch_bounds__(256) decode_bf16(DecodeArgs a) {
  __shared__ Shared<G> sh;
  __shared__ int last_flag;
  __shared__ int hist[WAVES][NSIZE];
  const bool zduty = blockIdx.x < (unsigned)(a.batch * a.hkv);
  const int zlen = zduty ? a.seq_lens[blockIdx.x / a.hkv] : 1;
  const Item it = map_item(a, blockIdx.x, hist[threadIdx.x >> 6], false);
  if (zduty && zlen <= 0) {
    const int zb = blockIdx.x / a.hkv, zh = blockIdx.x % a.hkv;
    for (int idx = threadIdx.x; idx < G * D; idx += WAVES * 64)
      a.out[((size_t)zb * a.hq + (size_t)zh * G) * D + idx] = 0.0f;
  }
  if (it.kind != 0) return;  // a bf16 cache has no window items
  const int b = it.b, h = it.h, split = it.split;
  const int tok0 = split * a.split_tokens;
  const int tok1 = min(tok0 + a.split_tokens, it.si.nq);
  const size_t head = ((size_t)b * a.hkv + h) * a.max_tokens * D;
  const Plan pl = plan_of(a, it.si);
  const bool direct = pl.total == 1 && !pl.overflow;
  bf16_tokens<G, QB, true>(a, b, h, (const uint16_t*)a.k_codes + head,
                           (const uint16_t*)a.v_codes + head, tok0, 0, tok1 - tok0,
                           direct ? DIRECT_OUT : split, sh);
  if (!direct) arrive_and_combine<G>(a, b, h, pl, &last_flag);
}

// Launches one decode_split variant.  With events, hipExtLaunchKernel stamps
// them with the start and end of the dispatch itself, so their difference
// is the kernel's own duration.
template <int KC, int KM, bool KCH, int VC, int VM, int G, bool PAGED, bool QB, bool TIER = false>
void launch_one(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  auto k = decode_split<KC, KM, KCH, VC, VM, G, PAGED, QB, TIER, false>;
  if constexpr (step_format<KM, KCH, VM, TIER>()) {
    if (a.k_new != nullptr) k = decode_split<KC, KM, KCH, VC, VM, G, PAGED, QB, TIER, true>;
  }
  if (a.ev_begin)
    hipExtLaunchKernelGGL(k, grid, dim3(256), 0, s, (hipEvent_t)a.ev_begin, (hipEvent_t)a.ev_end, 0,
                          a);
  else
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
}

// Pairs that run with a middle tier (contiguous, per token).
template <int KC, int KM, bool KCH, int VC, int VM>
constexpr bool tier_pair() {
  return !KCH && KC == VC && KM == VM &&
         ((KC == CK_I8 && KM == MK_F32) || (KC == CK_I4 && KM == MK_F32) ||
          (KC == CK_U4 && KM == MK_F16Z) || (KC == CK_U2 && KM == MK_F16Z));
}

template <int KC, int KM, bool KCH, int VC, int VM, int G>
void launch_split(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (tier_pair<KC, KM, KCH, VC, VM>()) {
    if (a.mid.tokens) {
      if (a.in_bf16)
        launch_one<KC, KM, KCH, VC, VM, G, false, true, true>(a, grid, s);
      else
        launch_one<KC, KM, KCH, VC, VM, G, false, false, true>(a, grid, s);
      return;
    }
  }
  if (a.paged) {
    if (a.in_bf16)
      launch_one<KC, KM, KCH, VC, VM, G, true, true>(a, grid, s);
    else
      launch_one<KC, KM, KCH, VC, VM, G, true, false>(a, grid, s);
  } else {
    if (a.in_bf16)
      launch_one<KC, KM, KCH, VC, VM, G, false, true>(a, grid, s);
    else
      launch_one<KC, KM, KCH, VC, VM, G, false, false>(a, grid, s);
  }
}

template <int KC, int KM, bool KCH, int VC, int VM>
hipError_t launch_g(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nsp * a.hkv * a.batch);
  if (a.nsp > 0) {
    switch (a.group) {
      case 1: launch_split<KC, KM, KCH, VC, VM, 1>(a, grid, s); break;
      case 2: launch_split<KC, KM, KCH, VC, VM, 2>(a, grid, s); break;
      case 4: launch_split<KC, KM, KCH, VC, VM, 4>(a, grid, s); break;
      case 8: launch_split<KC, KM, KCH, VC, VM, 8>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

// Launchers of the other translation units: each launches the pairs it
// instantiates and returns false (launching nothing) for any other pair.
bool launch_decode_w4(const DecodeArgs& a, hipStream_t s, hipError_t* e);
bool launch_decode_mixed(const DecodeArgs& a, hipStream_t s, hipError_t* e);
bool launch_decode_w2(const DecodeArgs& a, hipStream_t s, hipError_t* e);

}  // namespace kvq
