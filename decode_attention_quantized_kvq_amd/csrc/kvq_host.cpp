// libkvq host side: argument validation, byte accounting, split planning and
// the C entry points.  No device code here; launches live in the .hip files.
//
// Pages: [P1] "KV Cache Quantization Perturbs Attention Through Stored Keys
// and Values"; [P2] "KV cache quantization reduces cache bytes with separate
// accuracy and kernel costs"; [P3] "KV Cache Quantization and Per-Token Scale
// Placement".

#include <algorithm>
#include <cstdint>

#include "kvq.h"
#include "kvq_internal.h"

namespace kvq {

int meta_bytes(const kvq_tensor_fmt& f) {
  // P3 "Per-token scales and where they can live": a 4-byte scale per token,
  // or a scale plus a zero point; an 8-bit scale code under a super-scale.
  if (f.bits == 16 || f.axis != KVQ_AXIS_TOKEN) return 0;
  if (f.scale_fmt == KVQ_SCALE_U8_SUPER) return 1;
  const int w = f.scale_fmt == KVQ_SCALE_F32 ? 4 : 2;
  return f.zero_point ? 2 * w : w;
}

// Tokens per scale (1 = per token).
static int token_group(const kvq_config* c) { return c->group_tokens > 1 ? c->group_tokens : 1; }

// Code row, metadata element and (paged) unit bytes of the key and value
// tensors.
static void set_layout(const kvq_config* c, TensorKind* k, TensorKind* v) {
  k->row = row_bytes(c->key.bits, c->head_dim);
  v->row = row_bytes(c->value.bits, c->head_dim);
  k->mb = meta_bytes(c->key);
  v->mb = meta_bytes(c->value);
  k->unit = v->unit = k->moff = v->moff = 0;
  if (c->block_tokens) {
    const int per = 16 / token_group(c);
    k->unit = key_unit_bytes(k->row, per * (k->mb + v->mb));
    v->unit = 16 * v->row;
    k->moff = 16 * k->row;
    v->moff = k->moff + per * k->mb;
  }
}

// bf16 ring slots per (sequence, head): the window plus room for the
// positions of a token group not yet complete.
static int ring_slots(const kvq_config* c) {
  return c->window + (token_group(c) > 1 ? token_group(c) : 0);
}

// Quantized positions of an n-token sequence: whole groups older than the
// window.
static size_t quantized_count(const kvq_config* c, size_t n) {
  const size_t g = (size_t)token_group(c);
  return (n > (size_t)c->window ? n - c->window : 0) / g * g;
}

// Middle-tier slots per (sequence, head): M plus one block, since the tier
// holds M .. M + 31 positions once full.
static int mid_slots(const kvq_config* c) { return c->mid_tokens > 0 ? c->mid_tokens + MID_BLOCK : 0; }

// (cache format, middle tier, bf16) positions of an n-token sequence.
struct TierCounts {
  size_t main, mid, bf16;
};
static TierCounts tier_counts(const kvq_config* c, size_t n) {
  const size_t q = quantized_count(c, n);
  TierCounts t{q, 0, n - q};
  if (c->mid_tokens > 0) {
    const size_t m = (size_t)c->mid_tokens;
    t.main = (q > m ? q - m : 0) / MID_BLOCK * MID_BLOCK;
    t.mid = q - t.main;
  }
  return t;
}

static size_t side_bytes(const kvq_tensor_fmt& f, int d) {
  if (f.bits == 16) return 0;
  if (f.axis != KVQ_AXIS_TOKEN) return size_t(4) * d;
  if (f.scale_fmt == KVQ_SCALE_U8_SUPER) return 4;
  return 0;
}

kvq_status classify(const kvq_tensor_fmt& f, bool is_key, TensorKind* out) {
  TensorKind k{CK_I8, MK_NONE, false, false, false, 0, 0, 0, 0};
  if (f.scale_fmt != KVQ_SCALE_F32 && f.scale_fmt != KVQ_SCALE_F16 &&
      f.scale_fmt != KVQ_SCALE_U8_SUPER)
    return KVQ_ERR_INVALID_ARG;
  if (f.axis != KVQ_AXIS_TOKEN && f.axis != KVQ_AXIS_CHANNEL && f.axis != KVQ_AXIS_CHANNEL_GROW &&
      f.axis != KVQ_AXIS_CHANNEL_HOLD)
    return KVQ_ERR_INVALID_ARG;
  if (f.zero_point != 0 && f.zero_point != 1) return KVQ_ERR_INVALID_ARG;
  if (f.bits == 16) {
    if (f.axis != KVQ_AXIS_TOKEN || f.zero_point) return KVQ_ERR_INVALID_ARG;
    k.code = CK_BF16;
    k.meta = MK_NONE;
    if (out) *out = k;
    return KVQ_OK;  // unquantized: the kernels run it as a key/value pair, contiguous
  }
  if (f.bits != 8 && f.bits != 4 && f.bits != 2) return KVQ_ERR_INVALID_ARG;
  if (f.scale_fmt == KVQ_SCALE_U8_SUPER && f.zero_point) return KVQ_ERR_INVALID_ARG;
  if (f.axis != KVQ_AXIS_TOKEN && (f.zero_point || f.scale_fmt != KVQ_SCALE_F32))
    return KVQ_ERR_INVALID_ARG;
  if (f.bits == 8)
    k.code = f.zero_point ? CK_U8 : CK_I8;
  else if (f.bits == 4)
    k.code = f.zero_point ? CK_U4 : CK_I4;
  else
    k.code = f.zero_point ? CK_U2 : CK_I2;
  if (f.axis != KVQ_AXIS_TOKEN) {
    if (f.bits == 2) return KVQ_ERR_UNSUPPORTED;
    k.channel = true;
    k.grow = f.axis == KVQ_AXIS_CHANNEL_GROW;
    k.hold = f.axis == KVQ_AXIS_CHANNEL_HOLD;
    k.meta = MK_NONE;
    if (out) *out = k;
    return is_key ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
  }
  if (f.scale_fmt == KVQ_SCALE_U8_SUPER) {
    k.meta = MK_U8;
    if (out) *out = k;
    return KVQ_OK;
  }
  if (f.scale_fmt == KVQ_SCALE_F32)
    k.meta = f.zero_point ? MK_F32Z : MK_F32;
  else
    k.meta = f.zero_point ? MK_F16Z : MK_F16;
  if (out) *out = k;
  return KVQ_OK;
}

// Shape checks shared by accounting and compute.  kernels: also require what
// the kernels run (D = 128, G in {1,2,4,8}, capacity multiple of 16, ...).
static kvq_status check_config(const kvq_config* c, bool kernels) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->num_layers < 1 || c->batch < 1 || c->num_q_heads < 1 || c->num_kv_heads < 1 ||
      c->head_dim < 1 || c->max_tokens < 0 || c->window < 0 || c->block_tokens < 0 ||
      c->group_tokens < 0 || c->mid_tokens < 0 || c->mid_tokens % MID_BLOCK)
    return KVQ_ERR_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads) return KVQ_ERR_INVALID_ARG;
  if (c->in_dtype != KVQ_DT_F32 && c->in_dtype != KVQ_DT_BF16) return KVQ_ERR_INVALID_ARG;
  if (c->block_tokens && (c->num_blocks < 1 || c->max_blocks_per_seq < 1))
    return KVQ_ERR_INVALID_ARG;
  const int tg = token_group(c);
  if (tg != 1 && tg != 2 && tg != 4 && tg != 8 && tg != 16) return KVQ_ERR_INVALID_ARG;
  if (c->max_tokens % tg || (c->block_tokens && c->block_tokens % tg)) return KVQ_ERR_INVALID_ARG;
  TensorKind kk, vk;
  const kvq_status sk = classify(c->key, true, &kk);
  const kvq_status sv = classify(c->value, false, &vk);
  if (sk == KVQ_ERR_INVALID_ARG || sv == KVQ_ERR_INVALID_ARG) return KVQ_ERR_INVALID_ARG;
  if ((c->head_dim * c->key.bits) % 8 || (c->head_dim * c->value.bits) % 8)
    return KVQ_ERR_INVALID_ARG;
  if (!kernels) return KVQ_OK;
  if (sk != KVQ_OK || sv != KVQ_OK) return KVQ_ERR_UNSUPPORTED;
  const int g = c->num_q_heads / c->num_kv_heads;
  if (c->head_dim != 128) return KVQ_ERR_UNSUPPORTED;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_ERR_UNSUPPORTED;
  if (c->max_tokens % 16) return KVQ_ERR_UNSUPPORTED;
  if (c->block_tokens != 0 && c->block_tokens != 16) return KVQ_ERR_UNSUPPORTED;
  if (c->window % 16 || c->window > 256) return KVQ_ERR_UNSUPPORTED;
  if (token_group(c) > 1 && (kk.channel || kk.meta == MK_U8 || vk.meta == MK_U8))
    return KVQ_ERR_UNSUPPORTED;
  if (c->mid_tokens > 0) {
    // a middle tier runs with these per-token pairs, contiguous, per token
    if (c->block_tokens || tg != 1) return KVQ_ERR_UNSUPPORTED;
    const bool tier_ok =
        (kk.code == CK_I8 && kk.meta == MK_F32 && vk.code == CK_I8 && vk.meta == MK_F32) ||
        (kk.code == CK_I4 && kk.meta == MK_F32 && vk.code == CK_I4 && vk.meta == MK_F32) ||
        (kk.code == CK_U4 && kk.meta == MK_F16Z && vk.code == CK_U4 && vk.meta == MK_F16Z) ||
        (kk.code == CK_U2 && kk.meta == MK_F16Z && vk.code == CK_U2 && vk.meta == MK_F16Z);
    if (!tier_ok) return KVQ_ERR_UNSUPPORTED;
  }
  // The decode kernels are instantiated for these key/value pairs.
  const bool ok =
      (kk.code == CK_I8 && kk.meta == MK_F32 && vk.code == CK_I8 && vk.meta == MK_F32) ||
      (kk.code == CK_U4 && kk.meta == MK_F16Z && vk.code == CK_U4 && vk.meta == MK_F16Z) ||
      (kk.code == CK_I8 && kk.channel && vk.code == CK_I4 && vk.meta == MK_U8) ||
      (kk.code == CK_I4 && kk.meta == MK_F32 && vk.code == CK_I4 && vk.meta == MK_F32) ||
      (kk.code == CK_I8 && kk.meta == MK_F32 && vk.code == CK_I4 && vk.meta == MK_F32) ||
      (kk.code == CK_U8 && kk.meta == MK_F16Z && vk.code == CK_U8 && vk.meta == MK_F16Z) ||
      (kk.code == CK_I2 && kk.meta == MK_F32 && vk.code == CK_I2 && vk.meta == MK_F32) ||
      (kk.code == CK_I2 && kk.meta == MK_U8 && vk.code == CK_I2 && vk.meta == MK_U8) ||
      (kk.code == CK_U2 && kk.meta == MK_F16Z && vk.code == CK_U2 && vk.meta == MK_F16Z) ||
      (kk.code == CK_BF16 && vk.code == CK_BF16 && !c->block_tokens && !c->window && tg == 1);
  return ok ? KVQ_OK : KVQ_ERR_UNSUPPORTED;
}

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Quantized tokens per workgroup, aiming at one round of workgroups of four
// waves over the 256 compute units (a second round pays each workgroup's
// fixed start and merge again; on one MI355X it measured slower):
//  - codes of at most 4 bits on both sides, no middle tier: 768 workgroups.
//    Those kernels hold about 150 VGPRs per lane, three waves per SIMD, and
//    their VALU-heavy tiles need the third wave to hide load latency.
//  - otherwise 512.  Kernels with 8-bit per-token codes or the middle tier's
//    second tile loop hold about 200 VGPRs (two waves per SIMD); per-channel
//    8-bit keys over long caches measured faster with fewer, longer splits.
// A paged wave addresses at most 128 blocks, so paged splits stop at 8192.
static int choose_split(const kvq_config* c, int max_seq_len) {
  const long long nq = std::max(0, max_seq_len - c->window - c->mid_tokens);
  const long long pairs = (long long)c->batch * c->num_kv_heads;
  const bool narrow = c->key.bits <= 4 && c->value.bits <= 4 && c->mid_tokens == 0;
  const long long target = narrow ? 768 : 512;
  long long per = (nq * pairs + target - 1) / target;
  per = (long long)round_up((size_t)std::max<long long>(per, 1), 128);
  per = std::min<long long>(std::max<long long>(per, 256), c->block_tokens ? 8192 : 16384);
  // A short cache gets one workgroup per pair, which writes the output
  // directly: no arrival atomic and no combine, about 2 us less per launch
  // than two workgroups and a merge (measured: 512 tokens, 8.3 against 9.2 us).
  if (nq <= 512) per = std::max<long long>(per, (long long)round_up((size_t)std::max<long long>(nq, 1), 128));
  return (int)per;
}

struct Plan {
  int split_tokens, n_split, nsp;
  size_t o_bytes, ml_bytes, cnt_bytes, total;
};

static Plan make_plan(const kvq_config* c, int max_seq_len, int split_tokens) {
  Plan p{};
  p.split_tokens = split_tokens > 0 ? split_tokens : choose_split(c, max_seq_len);
  const int nq = std::max(0, max_seq_len - c->window);
  // at least one split: its workgroup writes the zeros of empty sequences
  p.n_split = std::max(1, (nq + p.split_tokens - 1) / p.split_tokens);
  // partial rows per query head: the splits, the bf16 item, the middle tier
  p.nsp = p.n_split + (ring_slots(c) > 0 ? 1 : 0) + (c->mid_tokens > 0 ? 1 : 0);
  const size_t rows = (size_t)c->batch * c->num_q_heads * p.nsp;
  p.o_bytes = round_up(rows * c->head_dim * sizeof(float), 256);
  p.ml_bytes = round_up(rows * 2 * sizeof(float), 256);
  p.cnt_bytes = round_up((size_t)c->batch * c->num_kv_heads * sizeof(uint32_t), 256);
  // the arrival counters come first, at an offset that does not depend on
  // the plan: a workspace that stays zero there serves calls with any
  // max_seq_len or split whose plan fits it
  p.total = p.cnt_bytes + p.ml_bytes + p.o_bytes;
#ifdef KVQ_PHASE_STAMPS
  p.total += PHASE_STAMP_BYTES;  // instrumented build: per-workgroup phase stamps
#endif
  return p;
}

struct LayerSizes {  // bytes of one layer of each buffer
  size_t k_codes, v_codes, k_meta, v_meta, k_win, v_win, k_chan, v_super, k_super;
  size_t mid_codes, mid_scale;  // each of K and V
};

static LayerSizes layer_sizes(const kvq_config* c) {
  LayerSizes s{};
  if (c->block_tokens) {
    // paged: one unit per (block, KV head), its metadata inside it
    const size_t units = (size_t)c->num_blocks * c->num_kv_heads;
    TensorKind k{}, v{};
    set_layout(c, &k, &v);
    s.k_codes = units * k.unit;
    s.v_codes = units * v.unit;
  } else {
    const size_t slots = (size_t)c->batch * c->num_kv_heads * c->max_tokens;
    s.k_codes = slots * row_bytes(c->key.bits, c->head_dim);
    s.v_codes = slots * row_bytes(c->value.bits, c->head_dim);
    s.k_meta = slots / token_group(c) * meta_bytes(c->key);
    s.v_meta = slots / token_group(c) * meta_bytes(c->value);
  }
  const size_t heads = (size_t)c->batch * c->num_kv_heads;
  s.k_win = s.v_win = heads * ring_slots(c) * c->head_dim * 2;
  s.k_chan = (c->key.bits != 16 && c->key.axis != KVQ_AXIS_TOKEN) ? heads * c->head_dim * 4 : 0;
  s.v_super = (c->value.bits != 16 && c->value.scale_fmt == KVQ_SCALE_U8_SUPER) ? heads * 4 : 0;
  s.k_super = (c->key.bits != 16 && c->key.axis == KVQ_AXIS_TOKEN &&
               c->key.scale_fmt == KVQ_SCALE_U8_SUPER) ? heads * 4 : 0;
  s.mid_codes = heads * mid_slots(c) * c->head_dim;
  s.mid_scale = heads * mid_slots(c) * 4;
  return s;
}

// The middle tier of one layer (tokens = 0 without one); false if a buffer
// it needs is missing.
static bool resolve_mid(const kvq_config* c, const kvq_cache* cache, int layer,
                        const LayerSizes& s, MidTier* m) {
  *m = MidTier{};
  if (c->mid_tokens <= 0) return true;
  if (!cache->k_mid || !cache->v_mid || !cache->k_mid_scale || !cache->v_mid_scale) return false;
  const size_t L = (size_t)layer;
  m->k = (uint8_t*)cache->k_mid + L * s.mid_codes;
  m->v = (uint8_t*)cache->v_mid + L * s.mid_codes;
  m->ks = (float*)((uint8_t*)cache->k_mid_scale + L * s.mid_scale);
  m->vs = (float*)((uint8_t*)cache->v_mid_scale + L * s.mid_scale);
  m->tokens = c->mid_tokens;
  m->slots = mid_slots(c);
  return true;
}

static bool resolve_layer(const kvq_config* c, const kvq_cache* cache, int layer,
                          const LayerSizes& s, uint8_t** kc, uint8_t** vc, uint8_t** km,
                          uint8_t** vm, uint16_t** kw, uint16_t** vw, float** kch, float** vsu,
                          float** ksu) {
  const size_t L = (size_t)layer;
  auto at = [&](void* base, size_t per) -> uint8_t* {
    return base ? (uint8_t*)base + L * per : nullptr;
  };
  *kc = at(cache->k_codes, s.k_codes);
  *vc = at(cache->v_codes, s.v_codes);
  *km = at(cache->k_meta, s.k_meta);
  *vm = at(cache->v_meta, s.v_meta);
  *kw = (uint16_t*)at(cache->k_win, s.k_win);
  *vw = (uint16_t*)at(cache->v_win, s.v_win);
  *kch = (float*)at(cache->k_chan_scale, s.k_chan);
  *vsu = (float*)at(cache->v_super, s.v_super);
  *ksu = (float*)at(cache->k_super, s.k_super);
  if (!*kc || !*vc) return false;
  if (s.k_meta && !*km) return false;
  if (s.v_meta && !*vm) return false;
  if (s.k_win && (!*kw || !*vw)) return false;
  if (s.k_chan && !*kch) return false;
  if (s.v_super && !*vsu) return false;
  if (s.k_super && !*ksu) return false;
  if (!cache->seq_lens) return false;
  if (c->block_tokens && !cache->block_table) return false;
  return true;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
  }
  return "KVQ_ERR_UNKNOWN";
}

kvq_status kvq_validate(const kvq_config* cfg) { return check_config(cfg, true); }

kvq_status kvq_get_buffer_sizes(const kvq_config* cfg, kvq_buffer_sizes* out) {
  const kvq_status st = check_config(cfg, false);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_INVALID_ARG;
  const LayerSizes s = layer_sizes(cfg);
  const size_t L = (size_t)cfg->num_layers;
  out->k_codes = L * s.k_codes;
  out->v_codes = L * s.v_codes;
  out->k_meta = L * s.k_meta;
  out->v_meta = L * s.v_meta;
  out->k_win = L * s.k_win;
  out->v_win = L * s.v_win;
  out->k_chan_scale = L * s.k_chan;
  out->v_super = L * s.v_super;
  out->k_super = L * s.k_super;
  out->k_mid = out->v_mid = L * s.mid_codes;
  out->k_mid_scale = out->v_mid_scale = L * s.mid_scale;
  return KVQ_OK;
}

size_t kvq_cache_bytes(const kvq_config* cfg, const int32_t* host_seq_lens, kvq_bytes* out) {
  if (check_config(cfg, false) != KVQ_OK) {
    if (out) *out = kvq_bytes{};
    return 0;
  }
  const size_t D = cfg->head_dim, H = cfg->num_kv_heads, L = cfg->num_layers;
  const size_t rk = row_bytes(cfg->key.bits, cfg->head_dim);
  const size_t rv = row_bytes(cfg->value.bits, cfg->head_dim);
  const size_t mk = meta_bytes(cfg->key), mv = meta_bytes(cfg->value);  // per group
  const size_t side = side_bytes(cfg->key, cfg->head_dim) + side_bytes(cfg->value, cfg->head_dim);
  const size_t g = (size_t)token_group(cfg), ring = (size_t)ring_slots(cfg);
  const size_t mslots = (size_t)mid_slots(cfg), mrow = 2 * D, mmeta = 2 * 4;  // int8 K, V + fp32 scales
  kvq_bytes b{};
  for (int i = 0; i < cfg->batch; ++i) {
    const size_t n = host_seq_lens ? (size_t)std::max(0, host_seq_lens[i]) : (size_t)cfg->max_tokens;
    const TierCounts t = tier_counts(cfg, n);
    const size_t nq = t.main, nw = t.bf16;
    // 2 L H_kv D T b with per-tensor b, per tier
    b.payload += L * H * (nq * (rk + rv) + t.mid * mrow);
    b.metadata += L * H * (nq / g * (mk + mv) + t.mid * mmeta + side);
    if (mslots) b.padding += L * H * (mslots > t.mid ? mslots - t.mid : 0) * (mrow + mmeta);
    b.window += L * H * nw * D * 2 * 2;
    size_t alloc_q;
    if (cfg->block_tokens)
      alloc_q = (nq + cfg->block_tokens - 1) / cfg->block_tokens * cfg->block_tokens;
    else
      alloc_q = std::max<size_t>((size_t)cfg->max_tokens, nq);
    b.padding += L * H * ((alloc_q - nq) * (rk + rv) + (alloc_q - nq) / g * (mk + mv));
    if (cfg->block_tokens) {
      // the key rows that hold a block's metadata, beyond the metadata itself
      TensorKind k{}, v{};
      set_layout(cfg, &k, &v);
      b.padding += L * H * alloc_q / 16 * (k.unit - 16 * rk - 16 / g * (mk + mv));
    }
    // the bf16 ring is a fixed buffer per (sequence, head) in both layouts
    if (ring) b.padding += L * H * (ring > nw ? ring - nw : 0) * D * 2 * 2;
  }
  b.total = b.payload + b.metadata + b.window + b.padding;
  // decode workspace at the library's split for the longest sequence (per
  // call, not part of the cache's total)
  if (check_config(cfg, true) == KVQ_OK) {
    int longest = 0;
    for (int i = 0; i < cfg->batch; ++i)
      longest = std::max(longest, host_seq_lens ? host_seq_lens[i] : cfg->max_tokens);
    b.workspace = make_plan(cfg, longest, 0).total;
  }
  if (out) *out = b;
  return b.total;
}

size_t kvq_decode_traffic_bytes(const kvq_config* cfg, const int32_t* host_seq_lens) {
  if (check_config(cfg, false) != KVQ_OK) return 0;
  kvq_config one = *cfg;
  one.num_layers = 1;
  kvq_bytes b{};
  kvq_cache_bytes(&one, host_seq_lens, &b);
  return b.payload + b.metadata + b.window;
}

static void set_groups(const kvq_config* c, int* g, int* gshift, int* ring) {
  *g = token_group(c);
  *gshift = *g == 16 ? 4 : *g == 8 ? 3 : *g == 4 ? 2 : *g == 2 ? 1 : 0;
  *ring = ring_slots(c);
}

kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache, int layer, void* k_out,
                          void* v_out, int out_tokens, void* stream) {
  const kvq_status st = check_config(cfg, true);
  if (st != KVQ_OK) return st;
  if (!cache || !k_out || !v_out || layer < 0 || layer >= cfg->num_layers || out_tokens < 0)
    return KVQ_ERR_INVALID_ARG;
  DequantArgs a{};
  classify(cfg->key, true, &a.kk);
  classify(cfg->value, false, &a.vk);
  set_layout(cfg, &a.kk, &a.vk);
  if (a.kk.code == CK_BF16 || a.vk.code == CK_BF16) return KVQ_ERR_UNSUPPORTED;
  const LayerSizes s = layer_sizes(cfg);
  uint8_t *kc, *vc, *km, *vm;
  uint16_t *kw, *vw;
  float *kch, *vsu, *ksu;
  if (!resolve_layer(cfg, cache, layer, s, &kc, &vc, &km, &vm, &kw, &vw, &kch, &vsu, &ksu))
    return KVQ_ERR_INVALID_ARG;
  a.k_codes = kc;
  a.v_codes = vc;
  a.k_meta = km;
  a.v_meta = vm;
  a.k_win = kw;
  a.v_win = vw;
  a.k_chan = kch;
  a.v_super = vsu;
  a.k_super = ksu;
  a.seq_lens = cache->seq_lens;
  a.block_table = cache->block_table;
  a.k_out = (uint16_t*)k_out;
  a.v_out = (uint16_t*)v_out;
  a.out_tokens = out_tokens;
  a.batch = cfg->batch;
  a.hkv = cfg->num_kv_heads;
  a.max_tokens = cfg->max_tokens;
  a.window = cfg->window;
  a.paged = cfg->block_tokens ? 1 : 0;
  a.num_blocks = cfg->num_blocks;
  a.bt_stride = cfg->max_blocks_per_seq;
  int g;
  set_groups(cfg, &g, &a.tgshift, &a.ring);
  if (!resolve_mid(cfg, cache, layer, s, &a.mid)) return KVQ_ERR_INVALID_ARG;
  return launch_dequant(a, stream);
}

static bool split_ok(int split) { return split >= 0 && split % 128 == 0 && split <= (1 << 20); }

size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int max_seq_len,
                                  const kvq_decode_opts* opts) {
  const int split = opts ? opts->split_tokens : 0;
  if (check_config(cfg, true) != KVQ_OK || max_seq_len < 0 || !split_ok(split)) return 0;
  if (cfg->block_tokens && split > 8192) return 0;
  return make_plan(cfg, max_seq_len, split).total;
}

// Validates an append and resolves its arguments to one layer; launches
// nothing.  KVQ_OK with *empty set when there is nothing to append.
static kvq_status prepare_append(const kvq_config* cfg, const kvq_cache* cache, int layer,
                                 const void* k_new, const void* v_new, int n_new,
                                 const int32_t* new_lens, AppendArgs* out, bool* empty) {
  *empty = false;
  kvq_status st = check_config(cfg, true);
  if (st != KVQ_OK) return st;
  if (!cache || layer < 0 || layer >= cfg->num_layers || n_new < 0) return KVQ_ERR_INVALID_ARG;
  if (n_new == 0) {
    *empty = true;
    return KVQ_OK;
  }
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  AppendArgs a{};
  const LayerSizes s = layer_sizes(cfg);
  if (!resolve_layer(cfg, cache, layer, s, &a.k_codes, &a.v_codes, &a.k_meta, &a.v_meta,
                     &a.k_win, &a.v_win, &a.k_chan, &a.v_super, &a.k_super))
    return KVQ_ERR_INVALID_ARG;
  classify(cfg->key, true, &a.kk);
  classify(cfg->value, false, &a.vk);
  set_layout(cfg, &a.kk, &a.vk);
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_lens = new_lens;
  a.seq_lens = cache->seq_lens;
  a.block_table = cache->block_table;
  a.batch = cfg->batch;
  a.hkv = cfg->num_kv_heads;
  a.n_new = n_new;
  a.max_tokens = cfg->max_tokens;
  a.window = cfg->window;
  set_groups(cfg, &a.tgroup, &a.tgshift, &a.ring);
  a.paged = cfg->block_tokens ? 1 : 0;
  a.num_blocks = cfg->num_blocks;
  a.bt_stride = cfg->max_blocks_per_seq;
  a.in_bf16 = cfg->in_dtype == KVQ_DT_BF16;
  if (!resolve_mid(cfg, cache, layer, s, &a.mid)) return KVQ_ERR_INVALID_ARG;
  *out = a;
  return KVQ_OK;
}

kvq_status kvq_quantize_append(const kvq_config* cfg, const kvq_cache* cache, int layer,
                               const void* k_new, const void* v_new, int n_new,
                               const int32_t* new_lens, void* stream) {
  AppendArgs a{};
  bool empty = false;
  const kvq_status st =
      prepare_append(cfg, cache, layer, k_new, v_new, n_new, new_lens, &a, &empty);
  if (st != KVQ_OK || empty) return st;
  return launch_append(a, stream);
}

// Validates a decode call (configuration, pointers, options, the split
// plan and the workspace) and resolves its arguments to one layer; launches
// nothing.  Shared by kvq_decode_attn_ex and kvq_decode_step, which runs it
// before its append so that a rejected step leaves the cache untouched.
static kvq_status prepare_decode(const kvq_config* cfg, const kvq_cache* cache, int layer,
                                 const void* q, float* out, void* workspace,
                                 size_t workspace_bytes, int max_seq_len,
                                 const kvq_decode_opts* opts, DecodeArgs* args,
                                 size_t counter_region = 0) {
  kvq_status st = check_config(cfg, true);
  if (st != KVQ_OK) return st;
  if (!cache || !q || !out || layer < 0 || layer >= cfg->num_layers || max_seq_len < 0)
    return KVQ_ERR_INVALID_ARG;
  const int split = opts ? opts->split_tokens : 0;
  if (!split_ok(split)) return KVQ_ERR_INVALID_ARG;
  if (opts && (!opts->split_begin_event != !opts->split_end_event)) return KVQ_ERR_INVALID_ARG;
  const int qbits = opts ? opts->query_bits : 0;
  if (qbits != 0 && qbits != 8) return KVQ_ERR_INVALID_ARG;
  // the per-channel key scale is folded onto the query in fp32; an int8 query
  // of the folded product is not a path the kernels run
  if (qbits == 8 && cfg->key.axis != KVQ_AXIS_TOKEN) return KVQ_ERR_UNSUPPORTED;
  // a paged wave addresses at most 128 blocks: splits of at most 4 x 2048 tokens
  if (cfg->block_tokens && split > 8192) return KVQ_ERR_INVALID_ARG;
  const Plan p = make_plan(cfg, max_seq_len, split);
  // one 1-D grid of nsp x H_kv x B workgroups of 256 threads
  if ((unsigned long long)p.nsp * cfg->num_kv_heads * cfg->batch >= (1ull << 24))
    return KVQ_ERR_UNSUPPORTED;
  // the arrival counters come first: the plan's own region, or a fixed one
  // (counter_region bytes) that the partials never overlap
  const size_t cnt = counter_region ? counter_region : p.cnt_bytes;
  if (p.cnt_bytes > cnt) return KVQ_ERR_WORKSPACE;
  const size_t need = cnt + p.ml_bytes + p.o_bytes;
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  if ((uintptr_t)workspace & 255) return KVQ_ERR_WORKSPACE;
  DecodeArgs a{};
  const LayerSizes s = layer_sizes(cfg);
  uint8_t *kc, *vc, *km, *vm;
  uint16_t *kw, *vw;
  float *kch, *vsu, *ksu;
  if (!resolve_layer(cfg, cache, layer, s, &kc, &vc, &km, &vm, &kw, &vw, &kch, &vsu, &ksu))
    return KVQ_ERR_INVALID_ARG;
  a.k_codes = kc;
  a.v_codes = vc;
  a.k_meta = km;
  a.v_meta = vm;
  a.k_win = kw;
  a.v_win = vw;
  a.k_chan = kch;
  a.v_super = vsu;
  a.k_super = ksu;
  a.block_table = cache->block_table;
  a.seq_lens = cache->seq_lens;
  a.q = q;
  a.out = out;
  a.counters = (uint32_t*)workspace;
  a.part_ml = (float*)((uint8_t*)workspace + cnt);
  a.part_o = (float*)((uint8_t*)workspace + cnt + p.ml_bytes);
  a.batch = cfg->batch;
  a.hq = cfg->num_q_heads;
  a.hkv = cfg->num_kv_heads;
  a.group = cfg->num_q_heads / cfg->num_kv_heads;
  a.max_tokens = cfg->max_tokens;
  a.paged = cfg->block_tokens ? 1 : 0;
  a.num_blocks = cfg->num_blocks;
  a.bt_stride = cfg->max_blocks_per_seq;
  a.window = cfg->window;
  set_groups(cfg, &a.tgroup, &a.tgshift, &a.ring);
  a.split_tokens = p.split_tokens;
  a.n_split = p.n_split;
  a.nsp = p.nsp;
  a.in_bf16 = cfg->in_dtype == KVQ_DT_BF16;
  classify(cfg->key, true, &a.kk);
  classify(cfg->value, false, &a.vk);
  set_layout(cfg, &a.kk, &a.vk);
  a.qbits = qbits;
  a.ev_begin = opts ? opts->split_begin_event : nullptr;
  a.ev_end = opts ? opts->split_end_event : nullptr;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.stamps = nullptr;
#ifdef KVQ_PHASE_STAMPS
  if (workspace_bytes >= need + PHASE_STAMP_BYTES)
    a.stamps = (unsigned long long*)((uint8_t*)workspace + workspace_bytes - PHASE_STAMP_BYTES);
#endif
  if (!resolve_mid(cfg, cache, layer, s, &a.mid)) return KVQ_ERR_INVALID_ARG;
  *args = a;
  return KVQ_OK;
}

kvq_status kvq_decode_attn_ex(const kvq_config* cfg, const kvq_cache* cache, int layer,
                              const void* q, float* out, void* workspace,
                              size_t workspace_bytes, int max_seq_len,
                              const kvq_decode_opts* opts, void* stream) {
  DecodeArgs a{};
  const kvq_status st = prepare_decode(cfg, cache, layer, q, out, workspace, workspace_bytes,
                                       max_seq_len, opts, &a);
  if (st != KVQ_OK) return st;
  return launch_decode(a, stream);
}

// The decode kernel quantizes the new token itself when the cache keeps
// per-token scales (fp32 or fp16, with or without a zero point) and has no
// middle tier or token groups.  With a bf16 window (and bf16 input), the
// workgroup of each pair's last chunk quantizes the token leaving the window
// and writes the new one into the ring, and the window's workgroup reads
// the new token from the input.  Otherwise the step is the append followed
// by the decode.
static bool step_fusable(const kvq_config* c) {
  auto ok = [](const kvq_tensor_fmt& f) {
    return f.bits != 16 && f.axis == KVQ_AXIS_TOKEN && f.scale_fmt != KVQ_SCALE_U8_SUPER;
  };
  return c->mid_tokens == 0 && token_group(c) == 1 && ok(c->key) && ok(c->value) &&
         (c->window == 0 || c->in_dtype == KVQ_DT_BF16);
}

kvq_status kvq_decode_step(const kvq_config* cfg, const kvq_cache* cache, int layer,
                           const void* k_new, const void* v_new, const void* q, float* out,
                           void* workspace, size_t workspace_bytes, int max_seq_len,
                           void* stream) {
  kvq_status st = check_config(cfg, true);
  if (st != KVQ_OK) return st;
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  // every check of both halves runs before anything is launched: a step the
  // library rejects leaves the cache as it was
  DecodeArgs d{};
  st = prepare_decode(cfg, cache, layer, q, out, workspace, workspace_bytes, max_seq_len,
                      nullptr, &d);
  if (st != KVQ_OK) return st;
  if (step_fusable(cfg)) {
    d.k_new = k_new;
    d.v_new = v_new;
    return launch_decode(d, stream);
  }
  AppendArgs ap{};
  bool empty = false;
  st = prepare_append(cfg, cache, layer, k_new, v_new, 1, nullptr, &ap, &empty);
  if (st != KVQ_OK) return st;
  st = launch_append(ap, stream);
  if (st != KVQ_OK) return st;
  return launch_decode(d, stream);
}

kvq_status kvq_decode_attn_noalloc(const kvq_config* cfg, const kvq_cache* cache, int layer,
                                   const void* q, float* out, int max_seq_len, void* stream) {
  // Every check runs first, against the scratch's size and layout at a
  // placeholder (aligned) address: a rejected call launches nothing and
  // does not touch the scratch.
  uint8_t* const placeholder = (uint8_t*)(uintptr_t)256;
  DecodeArgs a{};
  kvq_status st = prepare_decode(cfg, cache, layer, q, out, placeholder, NOALLOC_SCRATCH_BYTES,
                                 max_seq_len, nullptr, &a, NOALLOC_COUNTER_BYTES);
  if (st != KVQ_OK) return st;
  uint8_t* base = nullptr;
  st = noalloc_scratch(stream, &base);  // this device's copy of the scratch
  if (st != KVQ_OK) return st;
  a.counters = (uint32_t*)base;
  a.part_ml = (float*)(base + ((uint8_t*)a.part_ml - placeholder));
  a.part_o = (float*)(base + ((uint8_t*)a.part_o - placeholder));
  a.stamps = nullptr;  // no phase stamps from the scratch (instrumented builds)
  return launch_decode(a, stream);
}

kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_cache* cache, int layer,
                           const void* q, float* out, void* workspace, size_t workspace_bytes,
                           int max_seq_len, void* stream) {
  return kvq_decode_attn_ex(cfg, cache, layer, q, out, workspace, workspace_bytes, max_seq_len,
                            nullptr, stream);
}

}  // extern "C"
