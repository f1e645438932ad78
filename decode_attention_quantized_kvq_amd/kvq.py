"""Python binding of libkvq (argument marshalling only).

Every computation runs in the HIP library; this module builds the C structs,
checks tensor shapes/dtypes/devices against the configuration and passes raw
device pointers and the current HIP stream.  PyTorch provides device memory
and streams.  When libkvq.so is missing every call raises: there is no
fallback path.

The names mirror the C ABI in include/kvq.h: ``quantize_append``,
``decode_attn``, ``cache_bytes``, ``decode_workspace_bytes`` ...
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # first: libkvq then binds to the HIP runtime torch loaded

# KVQ_LIB names another build of the library (for A/B comparisons of builds)
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                     "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARG, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP = range(5)
AXIS = {"token": 0, "channel": 1, "channel_grow": 2, "channel_hold": 3}
SCALE = {"f32": 0, "f16": 1, "u8_super": 2}
DTYPE = {"f32": 0, "bf16": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}

# Every symbol include/kvq.h declares.
EXPORTS = (
    "kvq_status_string", "kvq_validate", "kvq_get_buffer_sizes", "kvq_cache_bytes",
    "kvq_decode_traffic_bytes", "kvq_decode_workspace_bytes", "kvq_quantize_append",
    "kvq_decode_attn", "kvq_decode_attn_ex", "kvq_dequantize", "kvq_decode_step",
    "kvq_decode_attn_noalloc",
)


class TensorFmt(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int), ("axis", ctypes.c_int),
                ("zero_point", ctypes.c_int), ("scale_fmt", ctypes.c_int)]


class Config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int), ("batch", ctypes.c_int),
                ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("max_tokens", ctypes.c_int),
                ("key", TensorFmt), ("value", TensorFmt), ("window", ctypes.c_int),
                ("block_tokens", ctypes.c_int), ("num_blocks", ctypes.c_int),
                ("max_blocks_per_seq", ctypes.c_int), ("in_dtype", ctypes.c_int),
                ("group_tokens", ctypes.c_int), ("mid_tokens", ctypes.c_int)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_meta", ctypes.c_void_p), ("v_meta", ctypes.c_void_p),
                ("k_win", ctypes.c_void_p), ("v_win", ctypes.c_void_p),
                ("k_chan_scale", ctypes.c_void_p), ("v_super", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("k_super", ctypes.c_void_p), ("k_mid", ctypes.c_void_p),
                ("v_mid", ctypes.c_void_p), ("k_mid_scale", ctypes.c_void_p),
                ("v_mid_scale", ctypes.c_void_p)]


class Bytes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("payload", "metadata", "window", "padding",
                                                "workspace", "total")]


class BufferSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("k_codes", "v_codes", "k_meta", "v_meta",
                                                "k_win", "v_win", "k_chan_scale", "v_super",
                                                "k_super", "k_mid", "v_mid", "k_mid_scale",
                                                "v_mid_scale")]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("split_tokens", ctypes.c_int), ("split_begin_event", ctypes.c_void_p),
                ("split_end_event", ctypes.c_void_p), ("query_bits", ctypes.c_int)]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkvq; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decode_attention_quantized_kvq_amd.build`")
        L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        P, I, S, VP = ctypes.POINTER, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
        L.kvq_status_string.restype = ctypes.c_char_p
        L.kvq_status_string.argtypes = [I]
        L.kvq_validate.restype = I
        L.kvq_validate.argtypes = [P(Config)]
        L.kvq_get_buffer_sizes.restype = I
        L.kvq_get_buffer_sizes.argtypes = [P(Config), P(BufferSizes)]
        L.kvq_cache_bytes.restype = S
        L.kvq_cache_bytes.argtypes = [P(Config), VP, P(Bytes)]
        L.kvq_decode_traffic_bytes.restype = S
        L.kvq_decode_traffic_bytes.argtypes = [P(Config), VP]
        L.kvq_decode_workspace_bytes.restype = S
        L.kvq_decode_workspace_bytes.argtypes = [P(Config), I, P(DecodeOpts)]
        L.kvq_quantize_append.restype = I
        L.kvq_quantize_append.argtypes = [P(Config), P(CacheDesc), I, VP, VP, I, VP, VP]
        L.kvq_decode_attn.restype = I
        L.kvq_decode_attn.argtypes = [P(Config), P(CacheDesc), I, VP, VP, VP, S, I, VP]
        L.kvq_decode_attn_ex.restype = I
        L.kvq_decode_attn_ex.argtypes = [P(Config), P(CacheDesc), I, VP, VP, VP, S, I,
                                         P(DecodeOpts), VP]
        L.kvq_dequantize.restype = I
        L.kvq_dequantize.argtypes = [P(Config), P(CacheDesc), I, VP, VP, I, VP]
        L.kvq_decode_attn_noalloc.restype = I
        L.kvq_decode_attn_noalloc.argtypes = [P(Config), P(CacheDesc), I, VP, VP, I, VP]
        L.kvq_decode_step.restype = I
        L.kvq_decode_step.argtypes = [P(Config), P(CacheDesc), I, VP, VP, VP, VP, VP, S, I, VP]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvq_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != KVQ_OK:
        raise KvqError(status, what)


def tensor_fmt(spec: dict) -> TensorFmt:
    return TensorFmt(int(spec["bits"]), AXIS[spec.get("axis", "token")],
                     int(bool(spec.get("zero_point", False))), SCALE[spec.get("scale", "f32")])


def make_config(*, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                max_tokens: int, key: dict, value: dict, window: int = 0,
                block_tokens: int = 0, num_blocks: int = 0, max_blocks_per_seq: int = 0,
                in_dtype: str = "bf16", num_layers: int = 1, group_tokens: int = 1,
                mid_tokens: int = 0) -> Config:
    return Config(num_layers, batch, num_q_heads, num_kv_heads, head_dim, max_tokens,
                  tensor_fmt(key), tensor_fmt(value), window, block_tokens, num_blocks,
                  max_blocks_per_seq, DTYPE[in_dtype], group_tokens, mid_tokens)


def validate(cfg: Config) -> int:
    return lib().kvq_validate(ctypes.byref(cfg))


def buffer_sizes(cfg: Config) -> BufferSizes:
    out = BufferSizes()
    _check(lib().kvq_get_buffer_sizes(ctypes.byref(cfg), ctypes.byref(out)), "kvq_get_buffer_sizes")
    return out


def _host_lens(cfg: Config, lens: Optional[Sequence[int]]):
    if lens is None:
        return None, None
    arr = (ctypes.c_int32 * cfg.batch)(*[int(x) for x in lens])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def cache_bytes(cfg: Config, lens: Optional[Sequence[int]] = None) -> dict:
    """kvq_cache_bytes: payload / metadata / window / padding / workspace /
    total (total excludes the per-call decode workspace)."""
    keep, ptr = _host_lens(cfg, lens)
    out = Bytes()
    total = lib().kvq_cache_bytes(ctypes.byref(cfg), ptr, ctypes.byref(out))
    d = {n: int(getattr(out, n)) for n, _ in Bytes._fields_}
    assert d["total"] == total
    return d


def decode_traffic_bytes(cfg: Config, lens: Optional[Sequence[int]] = None) -> int:
    keep, ptr = _host_lens(cfg, lens)
    return int(lib().kvq_decode_traffic_bytes(ctypes.byref(cfg), ptr))


def decode_workspace_bytes(cfg: Config, max_seq_len: int, split_tokens: int = 0) -> int:
    """kvq_decode_workspace_bytes for the given split size (0 = library's choice)."""
    opts = DecodeOpts(int(split_tokens))
    return int(lib().kvq_decode_workspace_bytes(ctypes.byref(cfg), int(max_seq_len),
                                                ctypes.byref(opts)))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class KvqCache:
    """Device buffers of one cache (all layers), allocated with torch.

    ``seq_lens`` (int32, device) holds each sequence's token count; callers
    advance it by the tokens of an append before calling ``quantize_append``
    (the library only reads it).  ``block_table`` is set for paged caches.
    """

    def __init__(self, cfg: Config, device: torch.device | str = "cuda",
                 block_table: Optional[torch.Tensor] = None):
        self.cfg = cfg
        self.device = torch.device(device)
        sz = buffer_sizes(cfg)
        self.buffers = {}
        for name, _ in BufferSizes._fields_:
            n = int(getattr(sz, name))
            # 256-byte aligned by the caching allocator; zero-filled
            self.buffers[name] = torch.zeros(n, dtype=torch.uint8, device=self.device) if n else None
        self.seq_lens = torch.zeros(cfg.batch, dtype=torch.int32, device=self.device)
        if cfg.block_tokens:
            if block_table is None:
                raise ValueError("a paged cache needs a block table")
            bt = block_table.to(device=self.device, dtype=torch.int32).contiguous()
            if tuple(bt.shape) != (cfg.batch, cfg.max_blocks_per_seq):
                raise ValueError(f"block table shape {tuple(bt.shape)}")
            self.block_table = bt
        else:
            self.block_table = None

    def desc(self) -> CacheDesc:
        b = self.buffers
        return CacheDesc(_ptr(b["k_codes"]), _ptr(b["v_codes"]), _ptr(b["k_meta"]),
                         _ptr(b["v_meta"]), _ptr(b["k_win"]), _ptr(b["v_win"]),
                         _ptr(b["k_chan_scale"]), _ptr(b["v_super"]),
                         _ptr(self.block_table), _ptr(self.seq_lens), _ptr(b["k_super"]),
                         _ptr(b["k_mid"]), _ptr(b["v_mid"]), _ptr(b["k_mid_scale"]),
                         _ptr(b["v_mid_scale"]))


def _check_input(t: torch.Tensor, cfg: Config, shape, what: str):
    want = TORCH_DTYPE["bf16" if cfg.in_dtype == DTYPE["bf16"] else "f32"]
    if t.dtype != want or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected contiguous {want} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def quantize_append(cache: KvqCache, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                    new_lens: Optional[torch.Tensor] = None, stream=None) -> None:
    """kvq_quantize_append: k_new/v_new [B][H_kv][n_new][D]; seq_lens already
    counts the new tokens."""
    cfg = cache.cfg
    n_new = k_new.shape[2] if k_new.dim() == 4 else -1
    shape = (cfg.batch, cfg.num_kv_heads, n_new, cfg.head_dim)
    _check_input(k_new, cfg, shape, "k_new")
    _check_input(v_new, cfg, shape, "v_new")
    if new_lens is not None and (new_lens.dtype != torch.int32 or not new_lens.is_cuda
                                 or tuple(new_lens.shape) != (cfg.batch,)):
        raise ValueError("new_lens: expected int32 [batch] on the GPU")
    desc = cache.desc()
    _check(lib().kvq_quantize_append(ctypes.byref(cfg), ctypes.byref(desc), int(layer),
                                     _ptr(k_new), _ptr(v_new), int(n_new), _ptr(new_lens),
                                     _stream(stream)), "kvq_quantize_append")


def decode_attn(cache: KvqCache, layer: int, q: torch.Tensor, max_seq_len: int,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                split_tokens: int = 0, stream=None, split_events=None,
                query_bits: int = 0) -> torch.Tensor:
    """kvq_decode_attn: q [B][Hq][D] -> out [B][Hq][D] fp32.

    query_bits: 0 (the query is not quantized) or 8 (the integer-query path).

    workspace: scratch of decode_workspace_bytes() bytes, zero-filled before
    its first use (the library leaves it reusable); one is allocated per
    call when omitted.
    split_events: optional (begin, end) torch.cuda.Event pair stamped with
    the decode kernel's dispatch (already created, e.g. by one record() call)."""
    cfg = cache.cfg
    _check_input(q, cfg, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "q")
    if out is None:
        out = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32,
                          device=q.device)
    elif (out.dtype != torch.float32 or not out.is_contiguous()
          or tuple(out.shape) != (cfg.batch, cfg.num_q_heads, cfg.head_dim)):
        raise ValueError("out: expected contiguous fp32 [B][Hq][D]")
    if workspace is None:
        need = decode_workspace_bytes(cfg, max_seq_len, split_tokens)
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    opts = DecodeOpts(int(split_tokens))
    opts.query_bits = int(query_bits)
    if split_events is not None:
        opts.split_begin_event = split_events[0].cuda_event
        opts.split_end_event = split_events[1].cuda_event
    _check(lib().kvq_decode_attn_ex(ctypes.byref(cfg), ctypes.byref(desc), int(layer),
                                    _ptr(q), _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    int(max_seq_len), ctypes.byref(opts), _stream(stream)),
           "kvq_decode_attn")
    return out


def decode_attn_noalloc(cache: KvqCache, layer: int, q: torch.Tensor, max_seq_len: int,
                        out: torch.Tensor, stream=None) -> torch.Tensor:
    """kvq_decode_attn_noalloc: as decode_attn, with the library's own
    per-GPU scratch instead of a workspace; `out` is caller-allocated."""
    cfg = cache.cfg
    _check_input(q, cfg, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "q")
    if (out.dtype != torch.float32 or not out.is_contiguous() or not out.is_cuda
            or tuple(out.shape) != (cfg.batch, cfg.num_q_heads, cfg.head_dim)):
        raise ValueError("out: expected contiguous fp32 [B][Hq][D] on the GPU")
    desc = cache.desc()
    _check(lib().kvq_decode_attn_noalloc(ctypes.byref(cfg), ctypes.byref(desc), int(layer),
                                         _ptr(q), _ptr(out), int(max_seq_len), _stream(stream)),
           "kvq_decode_attn_noalloc")
    return out


def decode_step(cache: KvqCache, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                q: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvq_decode_step: appends k_new/v_new [B][H_kv][1][D] (seq_lens already
    counts them) and attends with q [B][Hq][D] -> out [B][Hq][D] fp32."""
    cfg = cache.cfg
    shape = (cfg.batch, cfg.num_kv_heads, 1, cfg.head_dim)
    _check_input(k_new, cfg, shape, "k_new")
    _check_input(v_new, cfg, shape, "v_new")
    _check_input(q, cfg, (cfg.batch, cfg.num_q_heads, cfg.head_dim), "q")
    if out is None:
        out = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32,
                          device=q.device)
    elif (out.dtype != torch.float32 or not out.is_contiguous()
          or tuple(out.shape) != (cfg.batch, cfg.num_q_heads, cfg.head_dim)):
        raise ValueError("out: expected contiguous fp32 [B][Hq][D]")
    if workspace is None:
        need = decode_workspace_bytes(cfg, max_seq_len)
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=q.device)
    desc = cache.desc()
    _check(lib().kvq_decode_step(ctypes.byref(cfg), ctypes.byref(desc), int(layer), _ptr(k_new),
                                 _ptr(v_new), _ptr(q), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), int(max_seq_len),
                                 _stream(stream)), "kvq_decode_step")
    return out


def bf16_cache_like(cache: KvqCache, out_tokens: int) -> "KvqCache":
    """An empty unquantized (bits 16) cache shaped like `cache`, with room for
    out_tokens positions (a multiple of 16)."""
    cfg = cache.cfg
    cfg16 = make_config(batch=cfg.batch, num_q_heads=cfg.num_q_heads,
                        num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                        max_tokens=int(out_tokens), key=dict(bits=16), value=dict(bits=16),
                        in_dtype="bf16" if cfg.in_dtype == DTYPE["bf16"] else "f32")
    return KvqCache(cfg16, cache.device)


def dequantize(cache: KvqCache, layer: int, out_tokens: int, out: Optional["KvqCache"] = None,
               stream=None) -> "KvqCache":
    """kvq_dequantize: the layer's keys and values as an unquantized bf16
    cache (key/value bits 16, max_tokens = out_tokens, contiguous, no
    window), with the same sequence lengths; into `out` (from
    bf16_cache_like) when given.  out_tokens: a multiple of 16 at least the
    longest sequence."""
    cfg = cache.cfg
    if out is None:
        out = bf16_cache_like(cache, out_tokens)
    out.seq_lens.copy_(cache.seq_lens)
    desc = cache.desc()
    _check(lib().kvq_dequantize(ctypes.byref(cfg), ctypes.byref(desc), int(layer),
                                _ptr(out.buffers["k_codes"]), _ptr(out.buffers["v_codes"]),
                                int(out_tokens), _stream(stream)), "kvq_dequantize")
    return out
