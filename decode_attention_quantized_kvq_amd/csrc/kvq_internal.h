// Internal declarations shared by the host code and the HIP kernels of libkvq.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// How the codes of one tensor are stored.
enum CodeKind : int {
  CK_I8 = 0,   // signed int8, two's complement
  CK_U8 = 1,   // unsigned int8 (zero-point formats)
  CK_I4 = 2,   // signed int4 nibbles, two per byte
  CK_U4 = 3,   // unsigned int4 nibbles (zero-point formats)
  CK_BF16 = 4, // unquantized bf16 values
  CK_I2 = 5,   // signed int2, four per byte (symmetric codes -1..1)
  CK_U2 = 6    // unsigned int2 (zero-point formats)
};

// What is stored per token beside the codes.
enum MetaKind : int {
  MK_NONE = 0,  // nothing per token (per-channel scales, or bf16 values)
  MK_F32 = 1,   // fp32 scale
  MK_F32Z = 2,  // fp32 scale, fp32 zero point
  MK_F16 = 3,   // fp16 scale
  MK_F16Z = 4,  // fp16 scale (low half), fp16 zero point (high half)
  MK_U8 = 5     // u8 scale code relative to a per-head fp32 super-scale
};

struct TensorKind {
  CodeKind code;
  MetaKind meta;
  bool channel;   // per-channel scales (keys only)
  bool grow;      // ... that follow the running absmax (stored codes re-quantized)
  bool hold;      // ... fixed when the sequence's first position leaves the window
  // where the codes and metadata live: row = code bytes of one token; mb =
  // bytes of one metadata element; paged caches only: unit = bytes of this
  // tensor's (block, KV head) unit, moff = byte offset of this tensor's
  // metadata elements in the key unit (the key unit holds 16 key code rows,
  // then the block's key and then value metadata elements in whole key rows;
  // a value unit holds its 16 code rows)
  int row, mb, unit, moff;
};

// Code bytes of one token row of one head (0 for unsupported widths).
inline int row_bytes(int bits, int d) { return d * bits / 8; }

int meta_bytes(const kvq_tensor_fmt& f);

// Bytes of one (block, KV head) key unit of a paged cache: 16 key code rows,
// then the block's key and value metadata (meta_block bytes) in whole key
// rows (P2, "Metadata and block layout remain part of physical memory use":
// the block carries its scales).
inline int key_unit_bytes(int row, int meta_block) {
  return 16 * row + (meta_block + row - 1) / row * row;
}

// Classifies a format; returns KVQ_OK, KVQ_ERR_INVALID_ARG or
// KVQ_ERR_UNSUPPORTED (for the kernels).  is_key: keys accept channel axis.
kvq_status classify(const kvq_tensor_fmt& f, bool is_key, TensorKind* out);

// Middle tier of a cache (int8 codes, one fp32 scale per token; positions
// [A, Q) with Q = max(len - window, 0), A = floor(max(Q - tokens, 0) / 32) 32),
// resolved to one layer; tokens == 0: none.
constexpr int MID_BLOCK = 32;
struct MidTier {
  uint8_t* k;       // [B][H_kv][slots][D] int8
  uint8_t* v;
  float* ks;        // [B][H_kv][slots] fp32
  float* vs;
  int tokens;       // M
  int slots;        // M + 32; position p sits in slot p % slots
};

// Everything a quantize-append launch needs, resolved to one layer.
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* new_lens;
  const int32_t* seq_lens;
  const int32_t* block_table;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint8_t* k_meta;
  uint8_t* v_meta;
  uint16_t* k_win;
  uint16_t* v_win;
  float* k_chan;
  float* v_super;
  float* k_super;
  int batch, hkv, n_new, max_tokens, window, paged, num_blocks, bt_stride;
  int in_bf16;
  int tgroup, tgshift;  // token group size g (1 = per token) and log2 g
  int ring;           // bf16 ring slots per (sequence, head): window (+ g if g > 1)
  MidTier mid;
  TensorKind kk, vk;
};

// Everything a decode launch needs, resolved to one layer.
struct DecodeArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_meta;
  const uint8_t* v_meta;
  const uint16_t* k_win;
  const uint16_t* v_win;
  const float* k_chan;
  const float* v_super;
  const float* k_super;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const void* q;
  float* out;
  float* part_o;   // [B][Hq][nsp][D]
  float* part_ml;  // [B][Hq][nsp][2]
  uint32_t* counters;  // [B][H_kv] arrival counters, zero between calls
  int batch, hq, hkv, group;
  int max_tokens, paged, num_blocks, bt_stride, window;
  int tgroup, tgshift;  // token group size g (1 = per token) and log2 g
  int ring;           // bf16 ring slots per (sequence, head): window (+ g if g > 1)
  int qbits;          // 0: exact query limbs; 8: the query quantized to int8 per head
  MidTier mid;
  int split_tokens;  // quantized tokens per workgroup (multiple of 128)
  int n_split;       // workgroups over the quantized tokens
  int nsp;           // n_split, + 1 if there is a window, + 1 with a middle tier
  int in_bf16;
  TensorKind kk, vk;
  void* ev_begin;    // hipEvent_t recorded before the split kernel, or null
  void* ev_end;      // hipEvent_t recorded after it, or null
  // decode step: one new token per sequence ([B][H_kv][D] in the input
  // dtype) that the kernel quantizes into the cache before attending; null
  // for a plain decode
  const void* k_new;
  const void* v_new;
  // phase stamps of an instrumented build (KVQ_PHASE_STAMPS): 8 words per
  // workgroup in the workspace's last PHASE_STAMP_BYTES; null otherwise
  unsigned long long* stamps;
};

// Instrumented builds (-DKVQ_PHASE_STAMPS) append this many bytes to the
// decode workspace: 8 stamps of 8 bytes for each of up to 65536 workgroups.
constexpr size_t PHASE_STAMP_BYTES = size_t(65536) * 64;

// Everything a dequantize launch needs, resolved to one layer.
struct DequantArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_meta;
  const uint8_t* v_meta;
  const uint16_t* k_win;
  const uint16_t* v_win;
  const float* k_chan;
  const float* v_super;
  const float* k_super;
  const int32_t* seq_lens;
  const int32_t* block_table;
  uint16_t* k_out;  // [B][H_kv][out_tokens][D] bf16
  uint16_t* v_out;
  int out_tokens;
  int batch, hkv, max_tokens, window, paged, num_blocks, bt_stride;
  int tgshift, ring;
  MidTier mid;
  TensorKind kk, vk;
};

// Scratch of kvq_decode_attn_noalloc: one array per device, held by the
// library until the process ends.  The first NOALLOC_COUNTER_BYTES hold
// the arrival counters (one uint32 per (sequence, KV head), at most 16384);
// the partials follow.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
constexpr size_t NOALLOC_COUNTER_BYTES = size_t(64) << 10;

// This device's scratch address (looked up once per device, when its
// arrival counters are also cleared by a kernel on `stream`).
kvq_status noalloc_scratch(void* stream, uint8_t** base);

kvq_status launch_append(const AppendArgs& a, void* stream);
kvq_status launch_dequant(const DequantArgs& a, void* stream);
kvq_status launch_decode(const DecodeArgs& a, void* stream);

}  // namespace kvq
