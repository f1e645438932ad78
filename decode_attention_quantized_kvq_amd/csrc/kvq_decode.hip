// Split-T decode attention over a quantized KV cache (gfx950).
//
// Computes, for each query head, s_i = q . k_hat_i / sqrt(D), a = softmax(s),
// o = sum_i a_i v_hat_i over every cached token ([P1] "KV Cache Quantization
// Perturbs Attention Through Stored Keys and Values", section "Key error acts
// before the softmax"; [P2] "KV cache quantization reduces cache bytes with
// separate accuracy and kernel costs", section "Keys and values need not have
// identical error sensitivity").  As in [P3] "KV Cache Quantization and
// Per-Token Scale Placement", section "The axis choice is a kernel decision",
// the dot product runs on the integer-valued codes, the per-token key scale
// multiplies each score once after it, and a per-channel key scale is moved
// onto the query.
//
// decode_split: one workgroup of 4 waves per work item (a chunk of one
// sequence's tokens for one KV head, that sequence's bf16 window, or its
// middle tier).  Each wave streams its share of the chunk's 32-token tiles
// (every fourth tile with 8-bit keys, so that the four waves read adjacent
// tiles at once; a contiguous quarter for narrower tokens) straight from HBM
// into registers with buffer loads (one or two tiles in flight) and runs both
// contractions on the matrix cores, transposed so that the query heads are
// the rows:
//   scores  S^T[16 rows x 16 tok] += Q'[16 rows x 32 d] K^T[32 d x 16 tok]
//           (int8: the query as an exact integer in three int8 limbs per
//           head against the integer codes, int32 sums)
//   output  O^T[16 rows x 16 d]   += P^T[16 rows x 32 tok] V[32 tok x 16 d]
//           (fp16: the weights p s_V / R as (high, low) halves against the
//           codes converted exactly to fp16)
// The G query heads that share the KV head occupy the rows, so every loaded
// tile is used by all G heads.  The per-token key scale multiplies each
// score after the integer dot product; the online softmax runs in base 2.
// The 4 waves merge through LDS and the workgroup writes one partial (max,
// sum, normalized output) per query head; the last workgroup of a
// (sequence, KV head) to finish, found with an arrival counter, merges the
// partials by log-sum-exp into the fp32 output.  A (sequence, KV head) that
// one workgroup covers writes its output directly.

// This file instantiates the int8 / int8 pair and the unquantized (bf16)
// decode, holds the scratch of the allocation-free entry point and
// dispatches every pair; the others are instantiated in kvq_decode_w4.hip,
// kvq_decode_mixed.hip and kvq_decode_w2.hip from kvq_decode_kernel.h.

#include <mutex>

#include "kvq_decode_kernel.h"

namespace kvq {
namespace {

template <int G>
void launch_bf16(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  const auto k = a.in_bf16 ? decode_bf16<G, true> : decode_bf16<G, false>;
  if (a.ev_begin)
    hipExtLaunchKernelGGL(k, grid, dim3(256), 0, s, (hipEvent_t)a.ev_begin, (hipEvent_t)a.ev_end, 0,
                          a);
  else
    hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
}

hipError_t launch_bf16_g(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.nsp * a.hkv * a.batch);
  switch (a.group) {
    case 1: launch_bf16<1>(a, grid, s); break;
    case 2: launch_bf16<2>(a, grid, s); break;
    case 4: launch_bf16<4>(a, grid, s); break;
    case 8: launch_bf16<8>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Clears n words (the arrival counters of the no-allocation scratch).
__global__ void __launch_bounds__(256) zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

// The scratch of kvq_decode_attn_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address, one per GPU,
// comes from hipGetSymbolAddress and is the only way host code refers to it.
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
uint8_t* scratch_at[MAX_DEVICES] = {};  // device address of each GPU's copy
}  // namespace

kvq_status noalloc_scratch(void* stream, uint8_t** base) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_at[dev]) {
    // first use on this device (the current one): its copy's address, then
    // its arrival counters cleared by a kernel (no memset node, so the call
    // can sit in a captured graph); every decode leaves them at zero again
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return KVQ_ERR_HIP;
    constexpr int words = (int)(NOALLOC_COUNTER_BYTES / 4);
    hipLaunchKernelGGL(zero_words, dim3(words / 256), dim3(256), 0, (hipStream_t)stream,
                       (uint32_t*)p, words);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
    scratch_at[dev] = (uint8_t*)p;
  }
  *base = scratch_at[dev];
  return KVQ_OK;
}

kvq_status launch_decode(const DecodeArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const TensorKind k = a.kk, v = a.vk;
  hipError_t e = hipErrorInvalidValue;
  if (k.code == CK_I8 && k.meta == MK_F32 && v.code == CK_I8 && v.meta == MK_F32)
    e = launch_g<CK_I8, MK_F32, false, CK_I8, MK_F32>(a, s);
  else if (k.code == CK_BF16 && v.code == CK_BF16)
    e = launch_bf16_g(a, s);
  else if (!launch_decode_w4(a, s, &e) && !launch_decode_mixed(a, s, &e) &&
           !launch_decode_w2(a, s, &e))
    return KVQ_ERR_UNSUPPORTED;
  return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace kvq
