// Quantize-append kernels of libkvq (gfx950).
//
// Each new key/value vector is quantized from itself at write time and its
// scale stored beside it ([P3] "KV Cache Quantization and Per-Token Scale
// Placement", section "Per-token scales and where they can live"), following
// q = clamp(round(x / s)), x_hat = q * s ([P2] "KV cache quantization reduces
// cache bytes with separate accuracy and kernel costs", section "Quantization
// needs a scale convention").  Rounding is rint() of the IEEE fp64 quotient
// (ties to even, the rule of the quantizer listing in [P3] section "The axis
// choice is a kernel decision"); scales are evaluated in fp64 and rounded once
// to their storage type, so codes and metadata are bit-exact against any
// implementation of the same rule.  The write side moves a few hundred bytes
// per token and head; these kernels favour exactness over speed.
//
// Launch order on the caller's stream:
//   1. append_stats: per-channel key scales and key / value super-scales of
//      sequences whose append starts at position 0 (their prefill), then
//      frozen; for growing channel scales, their update and the
//      re-quantization of the stored codes of the channels that grew; for
//      held channel scales, their one computation when the sequence's first
//      position leaves the window.
//   2. append_quantize: one workgroup per (token, head, sequence); wave 0
//      quantizes the key, wave 1 the value.  With a recent window it takes
//      the tokens leaving the window (from the ring or from the input).
//   3. append_window: writes the new tokens that stay in the bf16 window
//      ([P1] "KV Cache Quantization Perturbs Attention Through Stored Keys and
//      Values", section "Cache growth changes the serving trade").  Runs after
//      2 so that ring slots are read before they are overwritten.

#include <hip/hip_runtime.h>

#include "kvq_internal.h"
#include "kvq_quantize.h"

namespace kvq {
namespace {

using namespace qz;

constexpr int D = 128;

struct SeqRange {
  int len, start, newb;
};

__device__ inline SeqRange seq_range(const AppendArgs& a, int b) {
  SeqRange r;
  r.len = a.seq_lens[b] > 0 ? a.seq_lens[b] : 0;
  int nb = a.new_lens ? a.new_lens[b] : a.n_new;
  nb = clampi(nb, 0, a.n_new);
  if (nb > r.len) nb = r.len;
  r.newb = nb;
  r.start = r.len - nb;
  return r;
}

// Capacity of quantized positions per sequence.
__device__ inline int q_capacity(const AppendArgs& a) {
  return a.paged ? a.bt_stride * 16 : a.max_tokens;
}

__device__ inline int meta_size(MetaKind m) {
  switch (m) {
    case MK_F32: return 4;
    case MK_F32Z: return 8;
    case MK_F16: return 2;
    case MK_F16Z: return 4;
    case MK_U8: return 1;
    default: return 0;
  }
}

// Quantized positions of an n-token sequence: whole token groups older than
// the window.
__device__ inline int quantized_count(const AppendArgs& a, int n) {
  const int m = n - a.window > 0 ? n - a.window : 0;
  return (m >> a.tgshift) << a.tgshift;
}

// A later append of a sequence whose per-channel key scales follow the
// running absmax: a channel whose keys quantized by this append exceed
// qmax * s gets s' = RN32(max / qmax), and its stored codes are re-quantized,
// c' = clamp(rint(fl64(c s / s'))); then the new scales are stored.
__device__ void grow_channels(const AppendArgs& a, int b, int h, const SeqRange& r) {
  const int qlo = quantized_count(a, r.start);
  int qhi = quantized_count(a, r.len);
  qhi = qhi < q_capacity(a) ? qhi : q_capacity(a);
  if (qhi <= qlo) return;
  __shared__ float snew[D];
  const int tid = threadIdx.x;
  const size_t head = (size_t)b * a.hkv + h;
  const int qmax = qmax_sym(code_bits(a.kk.code));
  float* chan = a.k_chan + head * D;
  bool grow = false;
  if (tid < D) {
    float amax = 0.0f;
    for (int p = qlo; p < qhi; ++p) {
      const float x = p >= r.start
                          ? load_in(a.k_new, (head * a.n_new + (p - r.start)) * D + tid, a.in_bf16)
                          : bf16_bits_to_f32(a.k_win[(head * a.ring + (p % a.ring)) * D + tid]);
      amax = fmaxf(amax, fabsf(x));
    }
    const float s = chan[tid];
    grow = (double)amax > (double)qmax * (double)s;
    snew[tid] = grow ? store_f32((double)amax / qmax) : s;
  }
  if (!__syncthreads_or(grow)) return;
  // two code rows per pass, one byte per thread: coalesced over the channels
  const int d = tid & (D - 1);
  const float s0 = chan[d], s1 = snew[d];
  if (s1 != s0) {
    for (int t = tid >> 7; t < qlo; t += 2) {
      uint8_t* cp = code_row(a, a.kk, a.k_codes, b, h, t) + d;
      const int c = (int)(int8_t)*cp;
      *cp = (uint8_t)clampi((int)rint((double)c * (double)s0 / (double)s1), -qmax, qmax);
    }
  }
  __syncthreads();
  if (tid < D) chan[tid] = snew[tid];
}

// Held channel scales: the append that quantizes a sequence's first
// position fixes its per-channel key scales, RN32(max / qmax) over every
// token it holds: positions [0, start) from the bf16 ring (none of them is
// quantized yet, so all are there) and the new ones from the input.
__device__ void hold_channels(const AppendArgs& a, int b, int h, const SeqRange& r) {
  if (quantized_count(a, r.start) != 0 || quantized_count(a, r.len) == 0) return;
  const int tid = threadIdx.x;
  if (tid >= D) return;
  const size_t head = (size_t)b * a.hkv + h;
  float amax = 0.0f;
  for (int p = 0; p < r.len; ++p) {
    const float x = p >= r.start
                        ? load_in(a.k_new, (head * a.n_new + (p - r.start)) * D + tid, a.in_bf16)
                        : bf16_bits_to_f32(a.k_win[(head * a.ring + (p % a.ring)) * D + tid]);
    amax = fmaxf(amax, fabsf(x));
  }
  const int qmax = qmax_sym(code_bits(a.kk.code));
  a.k_chan[head * D + tid] = amax == 0.0f ? 1.0f : store_f32((double)amax / qmax);
}

__global__ void __launch_bounds__(256) append_stats(AppendArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const SeqRange r = seq_range(a, b);
  if (r.newb == 0) return;
  if (a.kk.hold) hold_channels(a, b, h, r);
  if (r.start != 0) {  // a later append: only growing channel scales change
    if (a.kk.grow) grow_channels(a, b, h, r);
    return;
  }
  const size_t in_base = ((size_t)b * a.hkv + h) * a.n_new;
  const int tid = threadIdx.x;
  if (a.kk.channel && !a.kk.hold && tid < D) {
    // Absmax of each feature over the prefill, one rounding to fp32.
    float amax = 0.0f;
    for (int i = 0; i < r.newb; ++i)
      amax = fmaxf(amax, fabsf(load_in(a.k_new, (in_base + i) * D + tid, a.in_bf16)));
    const int qmax = qmax_sym(code_bits(a.kk.code));
    a.k_chan[((size_t)b * a.hkv + h) * D + tid] =
        amax == 0.0f ? 1.0f : store_f32((double)amax / qmax);
  }
  for (int w = 0; w < 2; ++w) {
    const TensorKind k = w == 0 ? a.kk : a.vk;
    if (k.channel || k.meta != MK_U8) continue;
    // sigma_t = amax_t / qmax per token; S = RN32(max sigma / 255).
    __shared__ double wmax[4];
    const int wave = tid >> 6, lane = tid & 63;
    const int qmax = qmax_sym(code_bits(k.code));
    const void* src = w == 0 ? a.k_new : a.v_new;
    double smax = 0.0;
    for (int i = wave; i < r.newb; i += 4) {
      const size_t row = (in_base + i) * D;
      const float x0 = load_in(src, row + 2 * lane, a.in_bf16);
      const float x1 = load_in(src, row + 2 * lane + 1, a.in_bf16);
      const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      smax = fmax(smax, (double)amax / qmax);
    }
    if (lane == 0) wmax[wave] = smax;
    __syncthreads();
    if (tid == 0) {
      const double m = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
      float* super = w == 0 ? a.k_super : a.v_super;
      super[(size_t)b * a.hkv + h] = m == 0.0 ? 1.0f : store_f32(m / 255.0);
    }
    __syncthreads();
  }
}

// Positions of an n-token sequence held in the cache's format: with a middle
// tier of M positions, whole blocks of 32 at least M older than the window;
// otherwise every quantized position.
__device__ inline int main_count(const AppendArgs& a, int n) {
  const int q = quantized_count(a, n);
  if (!a.mid.tokens) return q;
  const int m = q - a.mid.tokens;
  return m > 0 ? m / MID_BLOCK * MID_BLOCK : 0;
}

// Loads elements 2 lane, 2 lane + 1 of position p of (b, h) for wave w
// (0 = key, 1 = value): a position of this append from the input, an older
// one from its bf16 copy in the ring.
struct InputLoader {
  const void* src;
  const uint16_t* ring;
  size_t head;
  int start, lane;
  __device__ void operator()(const AppendArgs& a, int p, double& x0, double& x1) const {
    if (p >= start) {
      const size_t row = (head * a.n_new + (p - start)) * D;
      x0 = load_in(src, row + 2 * lane, a.in_bf16);
      x1 = load_in(src, row + 2 * lane + 1, a.in_bf16);
    } else {
      const size_t row = (head * a.ring + (p % a.ring)) * D;
      x0 = bf16_bits_to_f32(ring[row + 2 * lane]);
      x1 = bf16_bits_to_f32(ring[row + 2 * lane + 1]);
    }
  }
};

__device__ inline InputLoader input_loader(const AppendArgs& a, int w, size_t head, int start,
                                           int lane) {
  return InputLoader{w == 0 ? a.k_new : a.v_new, w == 0 ? a.k_win : a.v_win, head, start, lane};
}

constexpr TensorKind MID_KIND{CK_I8, MK_F32, false, false, false, 128, 4, 0, 0};

__global__ void __launch_bounds__(128) append_quantize(AppendArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const SeqRange r = seq_range(a, b);
  // token groups completed by this append: positions [qlo, qhi); with a
  // middle tier, those of them that stay in it
  int qlo = quantized_count(a, r.start);
  const int qhi = quantized_count(a, r.len);
  if (a.mid.tokens) {
    const int na = main_count(a, r.len);
    qlo = qlo > na ? qlo : na;
  }
  const int g = a.tgroup;
  const int p0 = qlo + i * g;
  if (p0 >= qhi) return;
  if (!a.mid.tokens && p0 + g > q_capacity(a)) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const TensorKind k = w == 0 ? a.kk : a.vk;
  const size_t head = (size_t)b * a.hkv + h;
  const InputLoader in = input_loader(a, w, head, r.start, lane);
  auto ld = [&](int p, double& x0, double& x1) { in(a, p, x0, x1); };
  if (a.mid.tokens) {  // into the middle tier: int8, fp32 scale, ring slot p % slots
    auto mslot = [&](int p) { return head * a.mid.slots + (size_t)(p % a.mid.slots); };
    uint8_t* mc = w == 0 ? a.mid.k : a.mid.v;
    auto mrow = [&](int p) { return mc + mslot(p) * (size_t)D; };
    quantize_group(MID_KIND, ld, mrow, p0, 1, (uint8_t*)((w == 0 ? a.mid.ks : a.mid.vs) + mslot(p0)),
                   nullptr, 1.0f, lane);
    return;
  }
  uint8_t* codes = w == 0 ? a.k_codes : a.v_codes;
  auto row = [&](int p) { return code_row(a, k, codes, b, h, p); };
  if (k.code == CK_BF16) {  // unquantized (bits 16): the bf16 values themselves
    for (int j = 0; j < g; ++j) {
      double x0, x1;
      ld(p0 + j, x0, x1);
      const uint32_t v = (uint32_t)f32_to_bf16_bits((float)x0) |
                         ((uint32_t)f32_to_bf16_bits((float)x1) << 16);
      ((uint32_t*)row(p0 + j))[lane] = v;
    }
    return;
  }
  uint8_t* meta = w == 0 ? a.k_meta : a.v_meta;
  const float* chan = (w == 0 && k.channel) ? a.k_chan + head * D : nullptr;
  const float* sup = w == 0 ? a.k_super : a.v_super;
  const float super = k.meta == MK_U8 ? sup[head] : 1.0f;
  quantize_group(k, ld, row, p0, g, meta_elem(a, k, meta, b, h, p0), chan, super, lane);
}

// Middle tier: the positions an append moves into the cache's format,
// [main_count(start), main_count(len)), re-quantized from their exact
// middle-tier value c * s.  One that was in the middle tier before this
// append is read from its ring slot; one that passes through it within the
// append (a long append) is quantized to int8 here first, as
// append_quantize would have stored it.  Runs before append_quantize, which
// may reuse those ring slots.
__global__ void __launch_bounds__(128) append_demote(AppendArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const SeqRange r = seq_range(a, b);
  const int p = main_count(a, r.start) + i;
  if (p >= main_count(a, r.len) || p >= a.max_tokens) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t head = (size_t)b * a.hkv + h;
  double v0, v1;  // the middle-tier value c * s (exact in fp64)
  if (p < quantized_count(a, r.start)) {
    const size_t ms = head * a.mid.slots + (size_t)(p % a.mid.slots);
    const uint8_t* row = (w == 0 ? a.mid.k : a.mid.v) + ms * D;
    const double sc = (double)(w == 0 ? a.mid.ks : a.mid.vs)[ms];
    v0 = (double)(int8_t)row[2 * lane] * sc;
    v1 = (double)(int8_t)row[2 * lane + 1] * sc;
  } else {
    double x0, x1;
    input_loader(a, w, head, r.start, lane)(a, p, x0, x1);
    // int8, one fp32 scale: the middle tier's quantizer
    const double amax = wave_max(fmax(fabs(x0), fabs(x1)));
    if (amax == 0.0) {
      v0 = v1 = 0.0;
    } else {
      const double sc = (double)store_f32(amax / 127);
      v0 = (double)clampi(rne_code(x0, sc), -127, 127) * sc;
      v1 = (double)clampi(rne_code(x1, sc), -127, 127) * sc;
    }
  }
  auto ld = [&](int, double& x0, double& x1) {
    x0 = v0;
    x1 = v1;
  };
  const TensorKind k = w == 0 ? a.kk : a.vk;
  uint8_t* codes = w == 0 ? a.k_codes : a.v_codes;
  auto row = [&](int q) { return code_row(a, k, codes, b, h, q); };
  quantize_group(k, ld, row, p, 1, meta_elem(a, k, w == 0 ? a.k_meta : a.v_meta, b, h, p), nullptr,
                 1.0f, lane);
}

__global__ void __launch_bounds__(128) append_window(AppendArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const SeqRange r = seq_range(a, b);
  // the new positions that stay unquantized: [max(Q, start), len)
  const int q = quantized_count(a, r.len);
  const int first = q > r.start ? q : r.start;
  const int p = first + i;
  if (p >= r.len) return;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const void* src = w == 0 ? a.k_new : a.v_new;
  uint16_t* ring = w == 0 ? a.k_win : a.v_win;
  const size_t in_row = (((size_t)b * a.hkv + h) * a.n_new + (p - r.start)) * D;
  const size_t out_row = (((size_t)b * a.hkv + h) * a.ring + (p % a.ring)) * D;
  for (int e = lane; e < D; e += 64) {
    const uint16_t v = a.in_bf16 ? ((const uint16_t*)src)[in_row + e]
                                 : f32_to_bf16_bits(((const float*)src)[in_row + e]);
    ring[out_row + e] = v;
  }
}

}  // namespace

kvq_status launch_append(const AppendArgs& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const dim3 heads(a.hkv, a.batch);
  if (a.kk.channel || a.kk.meta == MK_U8 || a.vk.meta == MK_U8) {
    hipLaunchKernelGGL(append_stats, heads, dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  }
  if (a.mid.tokens) {
    // positions an append moves into the cache's format: at most n_new + 31
    hipLaunchKernelGGL(append_demote, dim3(a.n_new + MID_BLOCK, a.hkv, a.batch), dim3(128), 0, s,
                       a);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  }
  // Token groups an append completes: the quantized count Q(n) = g floor((n
  // - W)^+ / g) grows by at most floor(n_new / g) + 1 groups when a sequence
  // grows by n_new positions, and by at most n_new positions when g = 1, so
  // that many workgroups cover every sequence (one new token behind a
  // 128-token window launches one per head, not 130).
  const int ng = a.tgroup == 1 ? a.n_new : a.n_new / a.tgroup + 1;
  hipLaunchKernelGGL(append_quantize, dim3(ng, a.hkv, a.batch), dim3(128), 0, s, a);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  if (a.ring) {
    const int nw = a.n_new < a.ring ? a.n_new : a.ring;
    hipLaunchKernelGGL(append_window, dim3(nw, a.hkv, a.batch), dim3(128), 0, s, a);
    if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace kvq
