/*
 * kvq.h - single-query decode attention over a low-bit KV cache (libkvq).
 *
 * C ABI of the library.  Plain pointers and sizes only.  Every compute call is
 * asynchronous on the caller's HIP stream; the library never allocates,
 * frees or synchronizes, and keeps no global state (calls are thread-safe as
 * long as calls that write the same buffers are ordered by their streams).
 *
 * Pages this follows (cited by title and section):
 *  [P1] "KV Cache Quantization Perturbs Attention Through Stored Keys and
 *       Values" (nalar.dev)
 *  [P2] "KV cache quantization reduces cache bytes with separate accuracy and
 *       kernel costs" (nalar.dev)
 *  [P3] "KV Cache Quantization and Per-Token Scale Placement" (mercemay.com)
 *
 * What the library computes:
 *  - kvq_quantize_append: each new key and value vector is quantized when it
 *    is written, q = clamp(round(x / s)) with reconstruction x_hat = q * s
 *    (P2, "Quantization needs a scale convention"), with a scale computed from
 *    the vector itself and stored beside it (P3, "Per-token scales and where
 *    they can live").  Variants: an integer zero point (P1, "Quantization
 *    granularity defines which values share a scale"); per-channel key scales
 *    fixed by the first append (P3, "Per-token scales and where they can
 *    live"); an 8-bit scale code relative to a per-head fp32 super-scale
 *    for keys or values, and 2-bit codes, the width at which the same
 *    section says 4-byte per-token scales cost 12 percent and schemes move
 *    to such 8-bit relative scales; the newest tokens kept in bf16 (P1, "Cache growth changes
 *    the serving trade"); 16-token blocks placed through a block table (P2,
 *    "Metadata and block layout remain part of physical memory use").
 *  - kvq_decode_attn: s_i = q . k_hat_i / sqrt(D), a = softmax(s),
 *    o = sum_i a_i v_hat_i over every cached token (P1, "Key error acts before
 *    the softmax"; P2, "Keys and values need not have identical error
 *    sensitivity"), with the per-token key scale applied once to each score
 *    after the dot product over the integer-valued codes and the per-channel
 *    key scale moved onto the query (P3, "The axis choice is a kernel
 *    decision").
 *  - kvq_cache_bytes: KV_bytes = 2 L H_kv D T b plus metadata, window and
 *    padding (P2, "Cache precision is separate from weight precision" and
 *    "Metadata and block layout remain part of physical memory use").
 *
 * Rounding contract of the write side (codes and metadata are bit-exact
 * against a reference that follows it):
 *  - codes are rint() (ties to even, as the quantizer listing of P3 "The axis
 *    choice is a kernel decision" rounds with Python's round()) of the IEEE
 *    fp64 quotient x / s_stored, then clamped to [-(2^(b-1)-1), 2^(b-1)-1]
 *    (symmetric) or [0, 2^b-1] (zero point; rint(x/s) + z, then clamp);
 *  - a scale is evaluated in fp64 and rounded once (ties to even) to its
 *    storage type, over the D values of a token (or the g D values of a
 *    token group): s = amax/qmax (symmetric), s = (hi-lo)/(2^b-1) with
 *    lo = min(min x, 0), hi = max(max x, 0) and z = clamp(rint(-lo/s))
 *    (zero point); an all-zero vector stores s = 1 (and z = 0) and codes 0;
 *    a scale that rounds to 0 stores the type's smallest positive value, an
 *    fp16 scale above 65504 stores 65504;
 *  - per-channel key scales: RN32(absmax over the first append / qmax) per
 *    feature (every token of it, also those that stay in the window), frozen
 *    (later tokens clamp) or growing (KVQ_AXIS_CHANNEL_GROW);
 *  - super-scaled keys or values: sigma_t = fl64(amax_t/qmax); per head
 *    S = RN32(max_t sigma_t / 255) over the first append, frozen;
 *    u_t = clamp(rint(fl64(sigma_t / S)), 1, 255) (0 for an all-zero vector);
 *    codes use the exact effective scale u_t * S.
 *
 * Device memory layout (all buffers caller-allocated; sizes from
 * kvq_buffer_sizes; "row" = D * bits / 8 code bytes of one token and head):
 *  contiguous (block_tokens == 0):
 *    codes  [L][B][H_kv][max_tokens][row]
 *    meta   [L][B][H_kv][max_tokens / g] of the meta element below
 *  paged (block_tokens == 16): per (block, KV head) a key unit and a value
 *    unit.  The key unit holds the 16 key code rows, then the block's 16 / g
 *    key meta elements and its 16 / g value meta elements, in whole key rows
 *    (UK = 16 + ceil(16 / g * (key + value meta bytes) / row_K) rows, the
 *    rest of the last row unused); the value unit holds the 16 value rows:
 *    k_codes [L][num_blocks][H_kv][UK][row_K]
 *    v_codes [L][num_blocks][H_kv][16][row_V]
 *    (no separate meta buffers: the k_meta / v_meta pointers are not read)
 *    quantized position p of sequence b lives in units
 *    (block_table[b][p / 16], h), row p % 16; its key meta element at byte
 *    16 row_K + ((p % 16) / g) * (key meta bytes) of the key unit, its value
 *    meta element at byte 16 row_K + (16 / g) * (key meta bytes) +
 *    ((p % 16) / g) * (value meta bytes).  A decode reads each block's scales
 *    with its key codes, one line for both tensors (scattered 64-byte scale
 *    runs cost about twice their bytes in time).
 *  ring   [L][B][H_kv][R][D] bf16 with R = window (+ g if g > 1); position
 *    p sits in slot p % R
 *  middle tier (mid_tokens = M > 0): codes [L][B][H_kv][M + 32][D] int8 and
 *    scales [L][B][H_kv][M + 32] fp32, for K and V each; position p sits in
 *    slot p % (M + 32)
 *  k_chan_scale [L][B][H_kv][D] fp32;  k_super, v_super [L][B][H_kv] fp32
 *  code bytes: bits 16 stores the bf16 values themselves (2 bytes each);
 *    int8 codes as two's complement bytes (unsigned bytes with a
 *    zero point); int4 codes packed two per byte, element 2j in the low nibble
 *    and 2j+1 in the high nibble (two's complement nibbles, or unsigned with a
 *    zero point); int2 codes packed four per byte, element 4j+i in bits
 *    [2i, 2i+2) of byte j (two's complement, symmetric codes in [-1, 1], or
 *    unsigned in [0, 3] with a zero point)
 *  meta element per token: f32 scale (4 B); f32 scale + f32 zero point
 *    (8 B); f16 scale (2 B); f16 scale + f16 zero point (4 B, scale in the
 *    low half); u8 scale code (1 B)
 *  Positions [0, Q) with Q = floor(max(len - window, 0) / g) * g are
 *  quantized; the newest len - Q (the window, plus the positions of a token
 *  group not yet complete) are kept as bf16 in the ring.  g = group_tokens
 *  (1 when 0).  Metadata element j of a (sequence, head) belongs to
 *  positions [j g, j g + g).
 *  With a middle tier of M positions, Q = max(len - window, 0) and
 *  A = floor(max(Q - M, 0) / 32) * 32: positions [0, A) hold the cache's
 *  format, [A, Q) the middle tier, [Q, len) the bf16 ring.  A token leaving
 *  the window is quantized into the middle tier (int8, symmetric, fp32 scale,
 *  by the rounding contract above); a token leaving the middle tier, 32
 *  positions at a time, is re-quantized to the cache's format from its exact
 *  middle-tier value c * s.  The cache's format is then per token, contiguous,
 *  without token groups or 8-bit scale codes; max_tokens bounds A.
 *
 * Error behaviour: every call validates its arguments on the host before
 * launching anything and returns a kvq_status; nothing is thrown across the
 * ABI.  Launch failures return KVQ_ERR_HIP; faults inside kernels surface at
 * the caller's next synchronization.  Device-resident values the host cannot
 * see are clamped, never trusted: a sequence length beyond the cache's
 * capacity is clamped to it, a block-table entry outside [0, num_blocks) is
 * clamped into it, and a sequence longer than the max_seq_len a decode call
 * was planned for gets NaN outputs.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent sizes */
  KVQ_ERR_UNSUPPORTED = 2, /* a valid format or shape the kernels do not run */
  KVQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KVQ_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} kvq_status;

/* Which values share a scale (P1, "Quantization granularity defines which
 * values share a scale"; P3, "Per-token scales and where they can live"). */
typedef enum {
  KVQ_AXIS_TOKEN = 0,  /* one scale per token per head */
  KVQ_AXIS_CHANNEL = 1, /* one scale per feature per head (keys only), from
                           a sequence's first append, then frozen */
  KVQ_AXIS_CHANNEL_GROW = 2, /* per feature per head (keys only), following the
                           running absmax: before tokens are quantized, a
                           channel whose new keys exceed qmax s gets
                           s' = RN32(max / qmax) and its stored codes become
                           clamp(rint(fl64(c s / s'))) (P3, "Per-token scales
                           and where they can live": the estimate has to be
                           updated as the sequence grows) */
  KVQ_AXIS_CHANNEL_HOLD = 3 /* per feature per head (keys only), the entries
                           held in floating point until the estimate is
                           stable (P3, "Per-token scales and where they can
                           live"): a sequence's keys stay in the bf16 window
                           until its first position leaves it; the scales
                           are then fixed once from every token it holds
                           (window and new), RN32(max / qmax), and frozen;
                           later tokens clamp.  Without a window: as
                           KVQ_AXIS_CHANNEL */
} kvq_axis;

/* Storage type of a per-token scale (and zero point). */
typedef enum {
  KVQ_SCALE_F32 = 0,
  KVQ_SCALE_F16 = 1,
  KVQ_SCALE_U8_SUPER = 2 /* u8 code times a per-head fp32 super-scale */
} kvq_scale_fmt;

typedef enum { KVQ_DT_F32 = 0, KVQ_DT_BF16 = 1 } kvq_dtype;

/* How one of K or V is stored (P1, "Quantization granularity defines which
 * values share a scale": bit width, grouping, scale precision and the key /
 * value treatment together define a format). */
typedef struct {
  int bits;                /* 8, 4 or 2; 16 = bf16 kept unquantized */
  kvq_axis axis;
  int zero_point;          /* 1: unsigned codes with an integer zero point */
  kvq_scale_fmt scale_fmt;
} kvq_tensor_fmt;

/* Shape and format of a cache (P2, "Cache precision is separate from weight
 * precision": layers, KV heads, head dimension, retained length, bytes per
 * element). */
typedef struct {
  int num_layers;
  int batch;
  int num_q_heads;
  int num_kv_heads;
  int head_dim;            /* D; the kernels run D = 128 */
  int max_tokens;          /* capacity per sequence, a multiple of 16 */
  kvq_tensor_fmt key;
  kvq_tensor_fmt value;
  int window;              /* newest tokens kept bf16 (0 = none, else a
                              multiple of 16, at most 256) */
  int block_tokens;        /* 0 = contiguous, 16 = paged */
  int num_blocks;          /* paged: blocks per layer in the pool */
  int max_blocks_per_seq;  /* paged: columns of block_table */
  kvq_dtype in_dtype;      /* dtype of k_new, v_new and q */
  int group_tokens;        /* 0 or 1: one scale per token; 2, 4, 8 or 16: one
                              scale (and zero point) per group of that many
                              consecutive positions of a sequence and head
                              (P3, "Per-token scales and where they can
                              live": several tokens under one scale) */
  int mid_tokens;          /* 0 = none; else a multiple of 32: a middle tier
                              of that many positions between the window and
                              the cache's format, stored as int8 with one fp32
                              scale per token, for keys and values (precision
                              by recency, P3 "Precision floors and mixed cache
                              formats"; layout and rules below) */
} kvq_config;

/* Device pointers of one cache (all layers).  Unused buffers may be NULL. */
typedef struct {
  void* k_codes;
  void* v_codes;
  void* k_meta;
  void* v_meta;
  void* k_win;             /* bf16 window ring of keys */
  void* v_win;
  void* k_chan_scale;      /* per-channel key scales */
  void* v_super;           /* per-head value super-scales */
  const int32_t* block_table; /* [batch][max_blocks_per_seq], paged only */
  const int32_t* seq_lens; /* [batch]: tokens of each sequence, counting the
                              tokens of the current append; the library only
                              reads it */
  void* k_super;           /* per-head key super-scales (keys with an 8-bit
                              scale code) */
  void* k_mid;             /* middle tier: int8 key codes, value codes, and */
  void* v_mid;             /* their fp32 scales (mid_tokens > 0 only) */
  void* k_mid_scale;
  void* v_mid_scale;
} kvq_cache;

/* Byte breakdown of a cache (P2, "Metadata and block layout remain part of
 * physical memory use"). */
typedef struct {
  size_t payload;   /* code bytes of the quantized tokens: L H_kv D T (bK+bV)/8 */
  size_t metadata;  /* per-token scales / zero points / scale codes and
                       per-head channel scales or super-scales */
  size_t window;    /* bf16 recent tokens of K and V */
  size_t padding;   /* allocated but unused slots (code and metadata slots
                       past a sequence's tokens, the unfilled tail of its last
                       16-token block, the unused end of the key rows that
                       hold a paged block's metadata, unused bf16 ring and
                       middle-tier slots) */
  size_t workspace; /* bytes of the decode workspace kvq_decode_attn needs
                       at the library's split for the longest of the
                       sequences (0 if the kernels do not run this
                       configuration); per call, not part of total */
  size_t total;     /* payload + metadata + window + padding */
} kvq_bytes;

/* Bytes to allocate for each buffer of kvq_cache (0 = not used). */
typedef struct {
  size_t k_codes, v_codes, k_meta, v_meta, k_win, v_win, k_chan_scale, v_super;
  size_t k_super;
  size_t k_mid, v_mid, k_mid_scale, v_mid_scale;
} kvq_buffer_sizes;

/* Human-readable name of a status.  Never NULL. */
const char* kvq_status_string(kvq_status s);

/* Checks that cfg describes a cache the kernels run: KVQ_OK,
 * KVQ_ERR_INVALID_ARG or KVQ_ERR_UNSUPPORTED.  The decode kernels run these
 * (key; value) pairs, per token unless marked:
 *   int8 f32 scale; int8 f32 scale          int8 f32; int4 f32
 *   int4 f32; int4 f32                      int8 per-channel; int4 u8 super
 *   uint4 f16 scale + zero; the same        uint8 f16 scale + zero; the same
 *   int2 f32; int2 f32                      int2 u8 super; int2 u8 super
 *   uint2 f16 scale + zero; the same        bf16 (bits 16); bf16, contiguous,
 *                                           no window, no token groups
 * An 8-bit scale code (u8 super) or per-channel keys exclude token groups.
 * A middle tier (mid_tokens > 0) runs with the pairs int8 f32 / int8 f32,
 * int4 f32 / int4 f32, uint4 f16 scale + zero (both) and uint2 f16 scale +
 * zero (both), contiguous, per token, without token groups. */
kvq_status kvq_validate(const kvq_config* cfg);

/* Fills *out with the byte size of each buffer of the layout above. */
kvq_status kvq_get_buffer_sizes(const kvq_config* cfg, kvq_buffer_sizes* out);

/* Byte accounting of P2 "Cache precision is separate from weight precision"
 * (payload 2 L H_kv D T b, generalised to separate key and value widths) plus
 * metadata (P3, "Per-token scales and where they can live"), window and
 * padding, and the decode workspace.  host_seq_lens: [batch] host array, or
 * NULL for max_tokens each.  Pure host arithmetic.  Returns the total (0 on an invalid configuration) and fills
 * *out when out is not NULL. */
size_t kvq_cache_bytes(const kvq_config* cfg, const int32_t* host_seq_lens, kvq_bytes* out);

/* Bytes one decode step reads from the cache of one layer: codes, per-token
 * metadata, window values and per-head side data, without padding. */
size_t kvq_decode_traffic_bytes(const kvq_config* cfg, const int32_t* host_seq_lens);


/* Quantizes and stores new tokens of one layer (P3, "Per-token scales and
 * where they can live": scale from the vector itself at write time).
 *  k_new, v_new: device [batch][num_kv_heads][n_new][head_dim] in in_dtype.
 *  new_lens:     device [batch] int32, tokens of sequence b taken from the
 *                first new_lens[b] rows (each <= n_new), or NULL for n_new.
 *  The tokens of sequence b take positions
 *  [seq_lens[b] - new_lens[b], seq_lens[b]): cache->seq_lens already counts
 *  them.  A sequence whose first position is 0 fixes its per-channel key
 *  scales and value super-scale from these tokens.
 *  stream: a hipStream_t (NULL = the null stream). */
kvq_status kvq_quantize_append(const kvq_config* cfg, const kvq_cache* cache, int layer,
                               const void* k_new, const void* v_new, int n_new,
                               const int32_t* new_lens, void* stream);

/* Dequantizes one layer into bf16 copies of its keys and values: the
 * dequantize-into-temporary-storage path of P1, "Cache growth changes the
 * serving trade" (its cost is what P2, "Lower payload does not imply
 * proportional latency reduction", weighs against the fused path).
 *  k_out, v_out: device [batch][num_kv_heads][out_tokens][head_dim] bf16,
 *    caller-owned.  Position p < min(seq_lens[b], out_tokens) of each
 *    sequence and head gets the exact reconstruction (code x scale, or
 *    scale x (code - zero point), code x u x S, code x channel scale) rounded
 *    once to bf16, or the stored bf16 value of a window / open-group token;
 *    other positions are left untouched.  The two buffers are then the codes
 *    of an unquantized cache (key and value bits 16, max_tokens = out_tokens,
 *    no window, contiguous) that kvq_decode_attn reads.
 *  A format with bits 16 has nothing to dequantize: KVQ_ERR_UNSUPPORTED.
 *  Launches one kernel on stream. */
kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache, int layer,
                          void* k_out, void* v_out, int out_tokens, void* stream);

/* Tuning and measurement knobs of kvq_decode_attn; zero / NULL fields take
 * the library's choice. */
typedef struct {
  int split_tokens;         /* quantized tokens per workgroup, a multiple of 128
                               (at most 8192 for a paged cache) */
  void* split_begin_event;  /* hipEvent_t stamped with the start of the decode
                               kernel's dispatch, or NULL */
  void* split_end_event;    /* hipEvent_t stamped with its end; both events or
                               neither (KVQ_ERR_INVALID_ARG otherwise) */
  int query_bits;           /* 0: the query is not quantized (its scale moves
                               onto integer limbs exactly); 8: the integer-query
                               path of P3, "Precision floors and mixed cache
                               formats": per query head s = fl64(amax / 127),
                               Q = clamp(rint(fl64(q / s))) in [-127, 127]
                               (the fp64 quotient of the cache's quantizer),
                               and every score uses Q s, with s rounded to
                               fp32 in the score scale (window tokens too).  8 is not
                               run with per-channel keys (KVQ_ERR_UNSUPPORTED);
                               other values are KVQ_ERR_INVALID_ARG. */
} kvq_decode_opts;

/* Single-query decode attention of one layer over every cached token (P2,
 * "Keys and values need not have identical error sensitivity").
 *  q:   device [batch][num_q_heads][head_dim] in in_dtype; query head h reads
 *       KV head h / (num_q_heads / num_kv_heads).
 *  out: device [batch][num_q_heads][head_dim] fp32.  A sequence with no
 *       tokens gets zeros.
 *  workspace: device scratch of at least
 *       kvq_decode_workspace_bytes(cfg, max_seq_len) bytes, 256-byte aligned,
 *       owned by the caller.  Its first bytes hold one uint32 arrival counter
 *       per (sequence, KV head), at the same place whatever the plan; they
 *       must be zero before the first call, and every call leaves them at
 *       zero again, so one workspace sized for the largest max_seq_len serves
 *       every later call whose kvq_decode_workspace_bytes is no larger (a
 *       growing or shrinking bound, another split).  The rest holds the
 *       split partials.  Calls that overlap in time must not share a
 *       workspace.
 *  max_seq_len: host upper bound of seq_lens (plans the split of the tokens
 *       over workgroups).  A sequence longer than max_seq_len gets NaN.  A
 *       plan of 2^24 or more workgroups (splits x H_kv x batch) returns
 *       KVQ_ERR_UNSUPPORTED.
 *  Launches one kernel on stream.  Each workgroup attends over one split of
 *  a sequence's tokens for the G query heads of one KV head; the last
 *  workgroup of each (sequence, KV head) to finish merges the splits by
 *  log-sum-exp.  Splitting the tokens over workgroups is this library's own
 *  design (the pages give no kernel), made because one decode step of a
 *  sequence must be spread over many compute units to stream the cache at
 *  the memory's rate (P3, "What the cache holds and how it is read": the
 *  read is memory-bound).  A
 *  (sequence, KV head) that one workgroup covers is written directly.  The
 *  library's split aims at one round of workgroups over the GPU; a cache of
 *  at most 512 quantized tokens per sequence gets a single split. */
kvq_status kvq_decode_attn(const kvq_config* cfg, const kvq_cache* cache, int layer,
                           const void* q, float* out, void* workspace, size_t workspace_bytes,
                           int max_seq_len, void* stream);

/* Workspace bytes kvq_decode_attn (opts == NULL) or kvq_decode_attn_ex
 * (same opts) needs for sequences of at most max_seq_len tokens; 0 on an
 * invalid configuration or option. */
size_t kvq_decode_workspace_bytes(const kvq_config* cfg, int max_seq_len,
                                  const kvq_decode_opts* opts);

/* One decode step of one layer: appends one new token to every sequence
 * (k_new, v_new: device [batch][num_kv_heads][1][head_dim] in in_dtype, as
 * kvq_quantize_append with n_new = 1 and new_lens = NULL; seq_lens must
 * already count the new token), then attends as kvq_decode_attn.  The
 * stored codes and metadata and the output are bit for bit those of the two
 * calls, also for a sequence whose length exceeds the cache's capacity (its
 * new token is not stored, as kvq_quantize_append skips it).  With per-token
 * fp32 or fp16 scales (with or without a zero point) and no middle tier or
 * token groups, one kernel does both.  Without a window, the workgroup whose
 * split holds a sequence's new token quantizes and stores it before reading
 * that split.  With a bf16 window (and in_dtype bf16), the workgroup of a
 * (sequence, KV head)'s last split quantizes the token leaving the window
 * from its ring slot and writes the new token into that slot before it
 * reads the tile that holds the quantized token; the window's workgroup
 * reads the new token from k_new, v_new (and, for a sequence with no
 * quantized token, writes it into the ring).  Otherwise it launches the
 * append kernels and then the decode kernel.  Every argument of both halves is checked before anything is
 * launched, so a call that returns an error has not changed the cache.
 * Errors as kvq_quantize_append and kvq_decode_attn; KVQ_ERR_INVALID_ARG if
 * k_new or v_new is NULL. */
kvq_status kvq_decode_step(const kvq_config* cfg, const kvq_cache* cache, int layer,
                           const void* k_new, const void* v_new, const void* q, float* out,
                           void* workspace, size_t workspace_bytes, int max_seq_len,
                           void* stream);

/* kvq_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  The split partials and arrival
 * counters live in a scratch array the library holds on each GPU it runs
 * on, 16 MiB per GPU, kept until the process ends; the call itself
 * allocates nothing.  Its first call on a device looks up that device's
 * copy and clears its counters with a kernel on `stream`.  Accepted calls:
 * batch x num_kv_heads <= 16384 and partial rows (batch x num_q_heads x
 * (splits + 1 per bf16 window and middle tier)) x (head_dim + 2) x 4 bytes
 * within the rest (about 16 MiB); a larger call returns KVQ_ERR_WORKSPACE
 * and launches nothing.  Calls on one GPU share its scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race, and must
 * be ordered by the caller.  Otherwise as kvq_decode_attn (same kernels,
 * same split plan, bit-identical outputs). */
kvq_status kvq_decode_attn_noalloc(const kvq_config* cfg, const kvq_cache* cache, int layer,
                                   const void* q, float* out, int max_seq_len, void* stream);

/* kvq_decode_attn with tuning knobs (opts may be NULL). */
kvq_status kvq_decode_attn_ex(const kvq_config* cfg, const kvq_cache* cache, int layer,
                              const void* q, float* out, void* workspace,
                              size_t workspace_bytes, int max_seq_len,
                              const kvq_decode_opts* opts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
