"""Python binding of libllama_layer.so, the gfx950 decoder-layer library.

Argument marshalling only: torch supplies device memory and the stream, every
step of the layer runs in the library's HIP kernels.  The names mirror the C
ABI in include/llama_layer.h.  Importing this module does not load the
library; the first call does, and raises if it is not built.
"""
from __future__ import annotations

import ctypes
import enum
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllama_layer.so")

_lib = None


class Status(enum.IntEnum):
    OK = 0
    INVALID_ARGUMENT = 1
    UNSUPPORTED = 2
    OUT_OF_MEMORY = 3
    HIP = 4


class Dtype(enum.IntEnum):
    BF16 = 0
    FP32 = 1


class Epilogue(enum.IntEnum):
    STORE = 0
    ADD = 1
    SILU_MUL = 2


class LlamaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (Status(status).name, msg))
        self.status = Status(status)


class Config(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("num_attention_heads", ctypes.c_int32),
        ("num_key_value_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("intermediate_size", ctypes.c_int32),
        ("max_position_embeddings", ctypes.c_int32),
        ("rms_norm_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_double),
        ("hidden_act", ctypes.c_char_p),
        ("rope_type", ctypes.c_char_p),
        ("rope_factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
        ("original_max_position_embeddings", ctypes.c_int32),
        ("attention_bias", ctypes.c_int32),
        ("mlp_bias", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("kv_block_size", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("num_experts_per_tok", ctypes.c_int32),
        ("moe_intermediate_size", ctypes.c_int32),
        ("norm_topk_prob", ctypes.c_int32),
        ("qk_norm", ctypes.c_int32),
    ]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "input_layernorm", "qkv_proj", "o_proj", "post_attention_layernorm", "gate_up_proj", "down_proj",
        "q_norm", "k_norm", "router", "experts_gate_up", "experts_down")]


class KvCache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("num_blocks", ctypes.c_int32)]


def lib() -> ctypes.CDLL:
    """Loads the library (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libllama_layer.so is not built: run `python -m llama_decoder_layer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    L.llama_layer_last_error.restype = ctypes.c_char_p
    L.llama_layer_last_error.argtypes = []
    L.llama_layer_config_validate.restype = st
    L.llama_layer_config_validate.argtypes = [ctypes.POINTER(Config)]
    L.llama_layer_create.restype = st
    L.llama_layer_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp, ctypes.POINTER(vp)]
    L.llama_layer_workspace_bytes.restype = ctypes.c_size_t
    L.llama_layer_workspace_bytes.argtypes = [vp, i32, i32, i32]
    L.llama_layer_forward.restype = st
    L.llama_layer_forward.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(KvCache), vp, i32, vp, vp, i32, i32,
                                      vp, vp, vp, vp]
    L.llama_layer_forward_noalloc.restype = st
    L.llama_layer_forward_noalloc.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(KvCache), vp, i32, vp, vp, i32, i32,
                                              vp, vp, vp]
    L.llama_layer_destroy.restype = None
    L.llama_layer_destroy.argtypes = [vp]
    L.llama_layer_workspace_tensor.restype = st
    L.llama_layer_workspace_tensor.argtypes = [vp, i32, i32, i32, ctypes.c_char_p,
                                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.llama_layer_rope_table.restype = st
    L.llama_layer_rope_table.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.llama_layer_set_timing.restype = st
    L.llama_layer_set_timing.argtypes = [vp, i32]
    L.llama_layer_timing_read.restype = i32
    L.llama_layer_timing_read.argtypes = [vp, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64), i32]
    L.llama_diag_stream_read.restype = st
    L.llama_diag_stream_read.argtypes = [vp, ctypes.c_size_t, i32, i32, i32, vp, vp]
    L.llama_diag_block_read.restype = st
    L.llama_diag_block_read.argtypes = [vp, ctypes.c_size_t, vp, i32, i32, i32, i32, vp, vp]
    L.llama_op_linear.restype = st
    L.llama_op_linear.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, vp]
    L.llama_op_reorder_gate_up.restype = st
    L.llama_op_reorder_gate_up.argtypes = [vp, i32, i32, vp, vp]
    L.llama_op_add_rmsnorm.restype = st
    L.llama_op_add_rmsnorm.argtypes = [i32, vp, vp, vp, ctypes.c_float, i32, i32, vp, vp, vp]
    L.llama_stack_create.restype = st
    L.llama_stack_create.argtypes = [ctypes.POINTER(Config), i32, ctypes.POINTER(Weights), vp, vp, ctypes.POINTER(vp)]
    L.llama_stack_workspace_bytes.restype = ctypes.c_size_t
    L.llama_stack_workspace_bytes.argtypes = [vp, i32, i32, i32]
    fwd = [vp, vp, vp, i32, ctypes.POINTER(KvCache), vp, i32, vp, vp, i32, i32, vp, vp, vp]
    L.llama_stack_forward.restype = st
    L.llama_stack_forward.argtypes = fwd
    L.llama_stack_destroy.restype = None
    L.llama_stack_destroy.argtypes = [vp]
    L.llama_stack_graph_create.restype = st
    L.llama_stack_graph_create.argtypes = fwd + [ctypes.POINTER(vp)]
    L.llama_graph_launch.restype = st
    L.llama_graph_launch.argtypes = [vp, vp]
    L.llama_graph_destroy.restype = None
    L.llama_graph_destroy.argtypes = [vp]
    _lib = L
    return L


EXPORTED = ["llama_layer_config_validate", "llama_layer_create", "llama_layer_workspace_bytes",
            "llama_layer_forward", "llama_layer_forward_noalloc", "llama_layer_destroy", "llama_layer_last_error",
            "llama_layer_workspace_tensor", "llama_layer_rope_table", "llama_layer_set_timing", "llama_layer_timing_read",
            "llama_op_linear", "llama_op_reorder_gate_up", "llama_op_add_rmsnorm",
            "llama_stack_create", "llama_stack_workspace_bytes", "llama_stack_forward", "llama_stack_destroy",
            "llama_stack_graph_create", "llama_graph_launch", "llama_graph_destroy", "llama_diag_stream_read",
            "llama_diag_block_read"]


_hip_rt = None


def _hip():
    """The HIP runtime torch already loaded (for plain copies of memory the
    library owns)."""
    global _hip_rt
    if _hip_rt is None:
        _hip_rt = ctypes.CDLL("libamdhip64.so")
        _hip_rt.hipMemcpy.restype = ctypes.c_int
        _hip_rt.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return _hip_rt


def _check(status: int) -> None:
    if status != 0:
        raise LlamaError(status, lib().llama_layer_last_error().decode())


def _dtype_of(t: torch.dtype) -> Dtype:
    if t == torch.bfloat16:
        return Dtype.BF16
    if t == torch.float32:
        return Dtype.FP32
    raise TypeError("unsupported dtype %s" % t)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _torch_stream(stream):
    """The torch stream object of `stream` (None: torch's current stream)."""
    if stream is None:
        return torch.cuda.current_stream()
    if hasattr(stream, "cuda_stream"):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _alloc_on(stream, make):
    """A tensor the library will use on `stream`: allocated while that stream
    is torch's current one, so torch's caching allocator ties the memory to it
    and never hands it out again while work queued there may still use it."""
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        t = make()
    t.record_stream(ts)
    return t


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, not %s" % (name, tuple(shape), tuple(t.shape)))


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s" % (name, dtype))
    return t


def make_config(cfg: dict, dtype: Dtype) -> Config:
    """config.json-style dict -> Config."""
    rs = cfg.get("rope_scaling") or {}
    rope_type = rs.get("rope_type", "default") if rs else "default"
    c = Config()
    c.hidden_size = cfg["hidden_size"]
    c.num_attention_heads = cfg["num_attention_heads"]
    c.num_key_value_heads = cfg["num_key_value_heads"]
    c.head_dim = cfg.get("head_dim", cfg["hidden_size"] // cfg["num_attention_heads"])
    c.intermediate_size = cfg["intermediate_size"]
    c.max_position_embeddings = cfg["max_position_embeddings"]
    c.rms_norm_eps = cfg["rms_norm_eps"]
    c.rope_theta = cfg["rope_theta"]
    c.hidden_act = cfg.get("hidden_act", "silu").encode()
    c.rope_type = rope_type.encode()
    c.rope_factor = float(rs.get("factor", 1.0))
    c.low_freq_factor = float(rs.get("low_freq_factor", 1.0))
    c.high_freq_factor = float(rs.get("high_freq_factor", 4.0))
    c.original_max_position_embeddings = int(rs.get("original_max_position_embeddings", 8192))
    c.attention_bias = int(bool(cfg.get("attention_bias", False)))
    c.mlp_bias = int(bool(cfg.get("mlp_bias", False)))
    c.dtype = int(dtype)
    c.kv_block_size = int(cfg.get("kv_block_size", 16))
    c.num_experts = int(cfg.get("num_experts", 0))
    c.num_experts_per_tok = int(cfg.get("num_experts_per_tok", 0))
    c.moe_intermediate_size = int(cfg.get("moe_intermediate_size", 0))
    c.norm_topk_prob = int(bool(cfg.get("norm_topk_prob", True)))
    c.qk_norm = int(bool(cfg.get("qk_norm", False)))
    return c


def make_weights(weights: dict, dtype) -> Weights:
    """Weights struct from a dict of device tensors (absent names stay NULL)."""
    w = Weights()
    for n, _ in Weights._fields_:
        if weights.get(n) is not None:
            setattr(w, n, _dev(weights[n], n, dtype).data_ptr())
    return w


def validate(cfg, dtype: Dtype = Dtype.BF16) -> Status:
    c = cfg if isinstance(cfg, Config) else make_config(cfg, dtype)
    return Status(lib().llama_layer_config_validate(ctypes.byref(c)))


class Layer:
    """One decoder layer on the current device (llama_layer_create)."""

    WEIGHT_NAMES = tuple(n for n, _ in Weights._fields_)
    # workspace tensors that are not in the layer dtype
    _WS_DTYPES = {"router_logits": torch.float32, "topk_ids": torch.int32, "topk_weights": torch.float32,
                  "moe_sorted": torch.int32}

    def __init__(self, cfg: dict, weights: dict, stream=None):
        self.cfg = dict(cfg)
        self.dtype = weights["qkv_proj"].dtype
        self._config = make_config(cfg, _dtype_of(self.dtype))
        w = make_weights(weights, self.dtype)
        h = ctypes.c_void_p()
        _check(lib().llama_layer_create(ctypes.byref(self._config), ctypes.byref(w), _stream(stream),
                                        ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().llama_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, num_tokens: int, num_seqs: int, max_seq_len: int) -> int:
        return int(lib().llama_layer_workspace_bytes(self._h, num_tokens, num_seqs, max_seq_len))

    def alloc_workspace(self, num_tokens: int, num_seqs: int, max_seq_len: int, device=None) -> torch.Tensor:
        n = self.workspace_bytes(num_tokens, num_seqs, max_seq_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")

    def forward(self, hidden, residual, positions, k_cache, v_cache, block_table, seq_lens, max_seq_len: int,
                hidden_out=None, residual_out=None, workspace=None, stream=None, query_start_loc=None):
        hidden_out, residual_out, kv, T, B = self._check(hidden, residual, positions, k_cache, v_cache, block_table,
                                                          seq_lens, hidden_out, residual_out, stream, query_start_loc)
        if workspace is None:
            workspace = _alloc_on(stream, lambda: self.alloc_workspace(T, B, max_seq_len, hidden.device))
        elif workspace.numel() < self.workspace_bytes(T, B, max_seq_len):
            raise ValueError("workspace too small")
        _check(lib().llama_layer_forward(
            self._h, _ptr(hidden), _ptr(residual), _ptr(positions), T, ctypes.byref(kv), _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), _ptr(query_start_loc), B, int(max_seq_len), _ptr(hidden_out),
            _ptr(residual_out), _ptr(workspace), _stream(stream)))
        return hidden_out, residual_out

    def forward_noalloc(self, hidden, residual, positions, k_cache, v_cache, block_table, seq_lens,
                        max_seq_len: int, hidden_out, residual_out, stream=None, query_start_loc=None):
        """llama_layer_forward_noalloc: the forward with the library's own
        scratch instead of a workspace; the caller supplies the outputs."""
        if hidden_out is None or residual_out is None:
            raise ValueError("the no-allocation forward writes into caller-supplied outputs")
        hidden_out, residual_out, kv, T, B = self._check(hidden, residual, positions, k_cache, v_cache, block_table,
                                                          seq_lens, hidden_out, residual_out, stream, query_start_loc)
        _check(lib().llama_layer_forward_noalloc(
            self._h, _ptr(hidden), _ptr(residual), _ptr(positions), T, ctypes.byref(kv), _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), _ptr(query_start_loc), B, int(max_seq_len), _ptr(hidden_out),
            _ptr(residual_out), _stream(stream)))
        return hidden_out, residual_out

    def _check(self, hidden, residual, positions, k_cache, v_cache, block_table, seq_lens, hidden_out, residual_out,
               stream, query_start_loc):
        """Argument checks shared by the forwards; allocates missing outputs
        on the call's stream.  Returns (hidden_out, residual_out, KvCache, T, B)."""
        _dev(hidden, "hidden", self.dtype)
        if hidden.dim() != 2 or hidden.shape[1] != self.cfg["hidden_size"]:
            raise ValueError("hidden must be [num_tokens, hidden_size]")
        T = hidden.shape[0]
        _dev(seq_lens, "seq_lens", torch.int32)
        if seq_lens.dim() != 1:
            raise ValueError("seq_lens must be [num_seqs]")
        B = seq_lens.shape[0]
        if residual is not None:
            _dev(residual, "residual", self.dtype)
            _shape(residual, "residual", hidden.shape)
        _dev(positions, "positions", torch.int32)
        _shape(positions, "positions", (T,))
        _dev(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
        _dev(k_cache, "k_cache", self.dtype)
        _dev(v_cache, "v_cache", self.dtype)
        nb, nkv, d = k_cache.shape[0], self.cfg["num_key_value_heads"], self.cfg.get(
            "head_dim", self.cfg["hidden_size"] // self.cfg["num_attention_heads"])
        _shape(k_cache, "k_cache", (nb, nkv, 16, d))
        _shape(v_cache, "v_cache", (nb, nkv, d, 16))
        if query_start_loc is not None:
            _dev(query_start_loc, "query_start_loc", torch.int32)
            if tuple(query_start_loc.shape) != (B + 1,):
                raise ValueError("query_start_loc must have num_seqs + 1 entries")
        if hidden_out is None:
            hidden_out = _alloc_on(stream, lambda: torch.empty_like(hidden))
        if residual_out is None:
            residual_out = _alloc_on(stream, lambda: torch.empty_like(hidden))
        for name, t in (("hidden_out", hidden_out), ("residual_out", residual_out)):
            _dev(t, name, self.dtype)
            _shape(t, name, hidden.shape)
        kv = KvCache(k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[0])
        return hidden_out, residual_out, kv, T, B

    def workspace_tensor(self, workspace: torch.Tensor, name: str, num_tokens: int, num_seqs: int,
                         max_seq_len: int) -> torch.Tensor:
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().llama_layer_workspace_tensor(self._h, num_tokens, num_seqs, max_seq_len, name.encode(),
                                                  ctypes.byref(off), ctypes.byref(nb)))
        raw = workspace[off.value: off.value + nb.value]
        return raw.view(self._WS_DTYPES.get(name, self.dtype)).view(num_tokens, -1)

    def rope_table(self):
        """A host copy of the layer's RoPE table, numpy float32
        [max_position_embeddings, head_dim/2, 2] of (cos, sin)
        (llama_layer_rope_table)."""
        import numpy as np
        p, n, pairs = ctypes.c_void_p(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().llama_layer_rope_table(self._h, ctypes.byref(p), ctypes.byref(n), ctypes.byref(pairs)))
        out = np.empty((n.value, pairs.value, 2), dtype=np.float32)
        torch.cuda.synchronize()
        rc = _hip().hipMemcpy(ctypes.c_void_p(out.ctypes.data), p, ctypes.c_size_t(out.nbytes), 2)  # device to host
        if rc != 0:
            raise RuntimeError("hipMemcpy of the RoPE table failed (%d)" % rc)
        return out

    def set_timing(self, enable: bool) -> None:
        _check(lib().llama_layer_set_timing(self._h, int(bool(enable))))

    def timing_read(self) -> dict:
        """{kernel name: (total ms, launches)} since the last read."""
        cap = 32
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_double * cap)()
        cnt = (ctypes.c_int64 * cap)()
        n = lib().llama_layer_timing_read(self._h, names, ms, cnt, cap)
        if n < 0:
            _check(Status.INVALID_ARGUMENT)
        return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n, cap))}


class Stack:
    """num_layers decoder layers plus the final RMSNorm (llama_stack_create):
    the model body from embedded hidden states to the normed output."""

    def __init__(self, cfg: dict, layer_weights: list, final_norm: torch.Tensor, stream=None):
        self.cfg = dict(cfg)
        self.num_layers = len(layer_weights)
        self.dtype = layer_weights[0]["qkv_proj"].dtype
        self._config = make_config(cfg, _dtype_of(self.dtype))
        ws = (Weights * self.num_layers)()
        for l, weights in enumerate(layer_weights):
            ws[l] = make_weights(weights, self.dtype)
        _dev(final_norm, "final_norm", self.dtype)
        h = ctypes.c_void_p()
        _check(lib().llama_stack_create(ctypes.byref(self._config), self.num_layers, ws, _ptr(final_norm),
                                        _stream(stream), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().llama_stack_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self, num_tokens: int, num_seqs: int, max_seq_len: int) -> int:
        return int(lib().llama_stack_workspace_bytes(self._h, num_tokens, num_seqs, max_seq_len))

    def alloc_workspace(self, num_tokens: int, num_seqs: int, max_seq_len: int, device=None) -> torch.Tensor:
        n = self.workspace_bytes(num_tokens, num_seqs, max_seq_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")

    def _args(self, hidden, positions, kv_caches, block_table, seq_lens, max_seq_len, out, workspace,
              query_start_loc):
        T, B = hidden.shape[0], seq_lens.shape[0]
        _dev(hidden, "hidden", self.dtype)
        if hidden.dim() != 2 or hidden.shape[1] != self.cfg["hidden_size"]:
            raise ValueError("hidden must be [num_tokens, hidden_size]")
        _dev(positions, "positions", torch.int32)
        _shape(positions, "positions", (T,))
        _dev(block_table, "block_table", torch.int32)
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
        _dev(seq_lens, "seq_lens", torch.int32)
        if len(kv_caches) != self.num_layers:
            raise ValueError("one (k, v) cache pair per layer")
        kvs = (KvCache * self.num_layers)()
        for l, (k, v) in enumerate(kv_caches):
            _dev(k, "k_cache", self.dtype)
            _dev(v, "v_cache", self.dtype)
            kvs[l] = KvCache(k.data_ptr(), v.data_ptr(), k.shape[0])
        if query_start_loc is not None:
            _dev(query_start_loc, "query_start_loc", torch.int32)
            if tuple(query_start_loc.shape) != (B + 1,):
                raise ValueError("query_start_loc must have num_seqs + 1 entries")
        _dev(out, "out", self.dtype)
        _shape(out, "out", hidden.shape)
        if workspace.numel() < self.workspace_bytes(T, B, max_seq_len):
            raise ValueError("workspace too small")
        self._kvs = kvs  # kept alive: a graph reads the array only at capture, a forward during the call
        return (self._h, _ptr(hidden), _ptr(positions), T, kvs, _ptr(block_table), block_table.shape[1],
                _ptr(seq_lens), _ptr(query_start_loc), B, int(max_seq_len), _ptr(out), _ptr(workspace))

    def forward(self, hidden, positions, kv_caches, block_table, seq_lens, max_seq_len: int, out=None,
                workspace=None, stream=None, query_start_loc=None):
        """kv_caches: list of (k_cache, v_cache), one per layer.  Returns out."""
        if out is None:
            out = _alloc_on(stream, lambda: torch.empty_like(hidden))
        if workspace is None:
            workspace = _alloc_on(stream, lambda: self.alloc_workspace(hidden.shape[0], seq_lens.shape[0],
                                                                         max_seq_len, hidden.device))
        a = self._args(hidden, positions, kv_caches, block_table, seq_lens, max_seq_len, out, workspace,
                       query_start_loc)
        _check(lib().llama_stack_forward(*a, _stream(stream)))
        return out

    def capture(self, hidden, positions, kv_caches, block_table, seq_lens, max_seq_len: int, out, workspace,
                stream, query_start_loc=None) -> "Graph":
        """A HIP graph of one forward with these buffers (llama_stack_graph_create)."""
        a = self._args(hidden, positions, kv_caches, block_table, seq_lens, max_seq_len, out, workspace,
                       query_start_loc)
        g = ctypes.c_void_p()
        _check(lib().llama_stack_graph_create(*a, _stream(stream), ctypes.byref(g)))
        return Graph(g, keep=(hidden, positions, kv_caches, block_table, seq_lens, out, workspace, query_start_loc))


class Graph:
    """A captured stack forward (llama_graph)."""

    def __init__(self, handle, keep):
        self._h = handle
        self._keep = keep  # the buffers the graph points at stay alive with it

    def launch(self, stream=None):
        _check(lib().llama_graph_launch(self._h, _stream(stream)))

    def close(self):
        if getattr(self, "_h", None):
            lib().llama_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stream_read(src: torch.Tensor, workgroups: int, threads: int, sink: torch.Tensor, nontemporal: bool = False,
                stream=None) -> None:
    """llama_diag_stream_read: reads all of src (device, contiguous) and
    nothing else, with or without the nontemporal load hint; sink holds
    workgroups * threads int32."""
    _dev(src, "src")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < workgroups * threads * 4:
        raise ValueError("sink too small")
    _check(lib().llama_diag_stream_read(_ptr(src), src.numel() * src.element_size(), workgroups, threads,
                                        int(bool(nontemporal)), _ptr(sink), _stream(stream)))


def block_read(src: torch.Tensor, block_ids: torch.Tensor, block_bytes: int, workgroups: int, sink: torch.Tensor,
               nontemporal: bool = False, stream=None, check_ids: bool = True) -> None:
    """llama_diag_block_read: reads the blocks block_ids (int32, device) of
    block_bytes each from src (device, contiguous); sink holds
    workgroups * block_bytes / 16 int32.  check_ids: verify on the host that
    every id is in range first (a device reduction and a synchronisation;
    a timing loop checks once and passes False)."""
    _dev(src, "src")
    _dev(block_ids, "block_ids", torch.int32)
    _dev(sink, "sink")
    nb = src.numel() * src.element_size() // block_bytes
    if check_ids and block_ids.numel() and (int(block_ids.min()) < 0 or int(block_ids.max()) >= nb):
        raise ValueError("block id out of range")
    if sink.numel() * sink.element_size() < workgroups * block_bytes // 16 * 4:
        raise ValueError("sink too small")
    _check(lib().llama_diag_block_read(_ptr(src), src.numel() * src.element_size(), _ptr(block_ids),
                                       block_ids.numel(), block_bytes, workgroups, int(bool(nontemporal)),
                                       _ptr(sink), _stream(stream)))


def linear(x: torch.Tensor, w: torch.Tensor, epilogue: Epilogue = Epilogue.STORE, out=None, stream=None):
    """llama_op_linear: out = x W^T (+ epilogue)."""
    _dev(x, "x")
    _dev(w, "w", x.dtype)
    M, K = x.shape
    N = w.shape[0] // 2 if epilogue == Epilogue.SILU_MUL else w.shape[0]
    if out is None:
        if epilogue == Epilogue.ADD:
            raise ValueError("ADD needs out (the addend)")
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype)
    _check(lib().llama_op_linear(int(_dtype_of(x.dtype)), _ptr(x), _ptr(w), M, N, K, int(epilogue), _ptr(out),
                                 _stream(stream)))
    return out


def reorder_gate_up(w: torch.Tensor, stream=None) -> torch.Tensor:
    _dev(w, "w", torch.bfloat16)
    out = torch.empty_like(w)
    _check(lib().llama_op_reorder_gate_up(_ptr(w), w.shape[0] // 2, w.shape[1], _ptr(out), _stream(stream)))
    return out


def add_rmsnorm(x: torch.Tensor, residual: Optional[torch.Tensor], w: torch.Tensor, eps: float,
                write_residual: bool = True, stream=None):
    """llama_op_add_rmsnorm -> (normed, residual_out or None)."""
    _dev(x, "x")
    normed = torch.empty_like(x)
    res_out = torch.empty_like(x) if (residual is not None or write_residual) else None
    _check(lib().llama_op_add_rmsnorm(int(_dtype_of(x.dtype)), _ptr(x), _ptr(residual), _ptr(w), eps, x.shape[0],
                                      x.shape[1], _ptr(normed), _ptr(res_out), _stream(stream)))
    return normed, res_out
