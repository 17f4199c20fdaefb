"""ctypes binding of ``librlt.so`` (declared in include/rlt.h).

Argument marshalling only: every step of the decoder runs in the library's HIP kernels. The
functions carry the C names; small handle classes own the torch device buffers that the C
handles borrow, so the memory stays alive as long as the handle. torch is used for device
memory and streams, nothing else. There is no fallback: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librlt.so")

RLT_F32, RLT_BF16 = 0, 1
STATUS_NAMES = {0: "RLT_OK", 1: "RLT_ERR_ARG", 2: "RLT_ERR_SHAPE", 3: "RLT_ERR_DTYPE",
                4: "RLT_ERR_CAPACITY", 5: "RLT_ERR_NOT_PROJECTED", 6: "RLT_ERR_HIP",
                7: "RLT_ERR_VERSION"}

WEIGHT_FIELDS = ("s_star", "w_gate", "b_gate", "gamma", "wq", "wk", "wv", "wo", "wcq", "wco",
                 "w1", "w3", "w2", "wmk", "wmv")
FP32_FIELDS = ("s_star", "b_gate", "gamma")


class rlt_config(ctypes.Structure):
    _fields_ = [("d", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
                ("n_layers", c_int32), ("ffn", c_int32), ("window", c_int32),
                ("n_groups", c_int32), ("dtype", c_int32), ("alpha", c_float), ("eps", c_float),
                ("version", c_uint64)]


class rlt_weights(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in WEIGHT_FIELDS]


KERNEL_NAMES = ("gate", "qkv", "self_attn", "self_out", "cross_q", "cross_attn", "cross_out",
                "ffn_up", "ffn_down", "memproj", "par_gemm", "par_self_attn", "par_cross_attn",
                "par_other", "bwd_proj", "bwd_self_attn", "bwd_cross_attn", "bwd_memory",
                "bwd_wgrad", "bwd_other")


class rlt_grads(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in WEIGHT_FIELDS]


class rlt_truncation(ctypes.Structure):
    _fields_ = [("segment", c_int64), ("detach", ctypes.c_uint32)]


DETACH_BITS = {"state": 1, "window": 2}  # RLT_DETACH_STATE, RLT_DETACH_WINDOW


class rlt_timing(ctypes.Structure):
    _fields_ = [("kernels", ctypes.c_uint32), ("token_stride", c_int32), ("clk", c_void_p),
                ("clk_bytes", c_size_t)]


class rlt_kernel_stats(ctypes.Structure):
    _fields_ = [("launches", c_int64), ("total_ms", ctypes.c_double), ("bytes", ctypes.c_double),
                ("flops", ctypes.c_double)]


HEAD_FIELDS = ("embed", "enc_gamma", "enc_gamma_out", "out_gamma", "w_out")
HEAD_FP32_FIELDS = ("enc_gamma", "enc_gamma_out", "out_gamma")


class rlt_head_weights(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in HEAD_FIELDS]


class rlt_sampling(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("top_k", c_int32), ("top_p", c_float)]


class RLTError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load librlt.so (``LIB_PATH`` unless `path` is given) and declare its signatures.
    Raises if it has not been built."""
    global _lib
    path = LIB_PATH if path is None else path
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m stateful_decoding_amd.build`")
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "rlt_last_error": (c_char_p, []),
        "rlt_config_check": (c_int32, [POINTER(rlt_config)]),
        "rlt_model_ws_bytes": (c_size_t, [POINTER(rlt_config)]),
        "rlt_model_create": (c_int32, [POINTER(rlt_config), POINTER(rlt_weights), P, c_size_t, P,
                                       POINTER(P)]),
        "rlt_model_destroy": (None, [P]),
        "rlt_state_bytes": (c_size_t, [POINTER(rlt_config), c_int32]),
        "rlt_state_create": (c_int32, [P, c_int32, P, c_size_t, P, POINTER(P)]),
        "rlt_state_reset": (c_int32, [P, P]),
        "rlt_state_position": (c_int64, [P]),
        "rlt_state_positions": (c_int32, [P, P, P]),
        "rlt_decoder_step_ragged": (c_int32, [P, P, P, P, P, P, P]),
        "rlt_state_destroy": (None, [P]),
        "rlt_memory_bytes": (c_size_t, [POINTER(rlt_config), c_int32, c_int64]),
        "rlt_memory_create": (c_int32, [P, c_int32, c_int64, P, c_size_t, POINTER(P)]),
        "rlt_memory_length": (c_int64, [P]),
        "rlt_memory_reset": (c_int32, [P]),
        "rlt_profile_begin": (c_int32, [P, ctypes.c_uint32, c_int32]),
        "rlt_profile_end": (c_int32, [P, POINTER(rlt_kernel_stats)]),
        "rlt_profile_clock": (c_int32, [P, P, c_size_t]),
        "rlt_memory_destroy": (None, [P]),
        "rlt_memproj": (c_int32, [P, P, P, c_int64, c_int64, P]),
        "rlt_decoder_step": (c_int32, [P, P, P, P, P, P]),
        "rlt_run_sequence": (c_int32, [P, P, P, P, c_int64, P, P]),
        "rlt_parallel_ws_bytes": (c_size_t, [POINTER(rlt_config), c_int32, c_int64]),
        "rlt_run_parallel": (c_int32, [P, P, P, P, c_int64, P, P, c_size_t, P]),
        "rlt_run_parallel_noalloc": (c_int32, [P, P, P, P, c_int64, P, P]),
        "rlt_scratch_bytes": (c_size_t, []),
        "rlt_state_export": (c_int32, [P, P, P, P, POINTER(c_int32), POINTER(c_int64),
                                       POINTER(c_uint64), P]),
        "rlt_state_import": (c_int32, [P, P, P, P, c_int64, c_uint64, P]),
        "rlt_state_import_ragged": (c_int32, [P, P, P, P, P, c_uint64, P]),
        "rlt_bptt_ws_bytes": (c_size_t, [POINTER(rlt_config), c_int32, c_int64]),
        "rlt_head_ws_bytes": (c_size_t, [POINTER(rlt_config), c_int32]),
        "rlt_head_create": (c_int32, [P, c_int32, POINTER(rlt_head_weights), P, c_size_t, P,
                                      POINTER(c_void_p)]),
        "rlt_head_destroy": (None, [P]),
        "rlt_encode_ws_bytes": (c_size_t, [POINTER(rlt_config), c_int32, c_int64]),
        "rlt_encode": (c_int32, [P, P, P, c_int32, c_int64, P, P, c_size_t, P]),
        "rlt_readout_ws_bytes": (c_size_t, [POINTER(rlt_config), c_int32, c_int32]),
        "rlt_readout": (c_int32, [P, P, P, c_int32, POINTER(rlt_sampling), P, P, P, P, P, P,
                                  c_size_t, P]),
        "rlt_bptt": (c_int32, [P, P, c_int32, c_int64, P, P, POINTER(rlt_grads), P, P, c_size_t,
                               POINTER(rlt_truncation), POINTER(rlt_timing), P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise RLTError(status, load_library().rlt_last_error().decode())


def make_config(cfg, version: int = 0) -> rlt_config:
    """rlt_config from any object with the fields d, n_heads, head_dim, n_layers, ffn,
    window, n_groups, alpha, eps and dtype ('fp32' | 'bf16')."""
    g = (lambda k: cfg[k]) if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    dt = g("dtype")
    return rlt_config(int(g("d")), int(g("n_heads")), int(g("head_dim")), int(g("n_layers")),
                      int(g("ffn")), int(g("window")), int(g("n_groups")),
                      RLT_BF16 if dt in ("bf16", RLT_BF16) else RLT_F32 if dt in ("fp32", RLT_F32) else int(dt),
                      float(g("alpha")), float(g("eps")), int(version))


def torch_dtype(c: rlt_config):
    return torch.bfloat16 if c.dtype == RLT_BF16 else torch.float32


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _device_buffer(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def upload_weights(params: dict, cfg: rlt_config, device="cuda") -> dict:
    """Host arrays (numpy or torch) -> contiguous device tensors in the layouts of
    rlt_weights: matrices in the config dtype, s*, b_g and the gains in float32."""
    out = {}
    dt = torch_dtype(cfg)
    for name in WEIGHT_FIELDS:
        x = params[name]
        x = torch.as_tensor(x) if not isinstance(x, torch.Tensor) else x
        out[name] = x.to(device=device, dtype=torch.float32 if name in FP32_FIELDS else dt).contiguous()
    return out


class Model:
    """Packed weights on the device (rlt_model_create)."""

    def __init__(self, cfg, weights: dict, version: int = 0, stream=None, device="cuda"):
        self.lib = load_library()
        self.cfg = cfg if isinstance(cfg, rlt_config) else make_config(cfg, version)
        _check(self.lib.rlt_config_check(byref(self.cfg)))
        self.dtype = torch_dtype(self.cfg)
        w = rlt_weights(*[_ptr(weights[n]) for n in WEIGHT_FIELDS])
        nbytes = self.lib.rlt_model_ws_bytes(byref(self.cfg))
        self.ws = _device_buffer(nbytes, device)
        h = c_void_p()
        _check(self.lib.rlt_model_create(byref(self.cfg), byref(w), self.ws.data_ptr(), nbytes,
                                         _stream(stream), byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None):
            self.lib.rlt_model_destroy(self.handle)
            self.handle = None


class State:
    """Decoder state of `batch` sequences (rlt_state_create): s, caches, working buffers."""

    def __init__(self, model: Model, batch: int, stream=None):
        self.lib, self.model, self.batch = model.lib, model, int(batch)
        nbytes = self.lib.rlt_state_bytes(byref(model.cfg), self.batch)
        if nbytes == 0:
            raise RLTError(2, f"invalid batch {batch}")
        self.buf = _device_buffer(nbytes, model.ws.device)
        h = c_void_p()
        _check(self.lib.rlt_state_create(model.handle, self.batch, self.buf.data_ptr(), nbytes,
                                         _stream(stream), byref(h)))
        self.handle = h

    @property
    def position(self) -> int:
        return self.lib.rlt_state_position(self.handle)

    def reset(self, stream=None):
        _check(self.lib.rlt_state_reset(self.handle, _stream(stream)))

    def positions(self, stream=None):
        """Per-sequence positions (waits for the stream), as a list of ints."""
        out = (c_int64 * self.batch)()
        _check(self.lib.rlt_state_positions(self.handle, out, _stream(stream)))
        return list(out)

    def profile_clock(self, slots: int | None):
        """Attach a device buffer of `slots` clock slot pairs (one per workgroup of each
        self-timed attention launch, i.e. H per sequence and launch): later sessions time the
        attention kernels by their own clock stamps instead of events. None detaches it."""
        if slots is None:
            _check(self.lib.rlt_profile_clock(self.handle, None, 0))
            self._clk = None
            return
        buf = clock_buffer(slots, self.buf.device)
        _check(self.lib.rlt_profile_clock(self.handle, buf.data_ptr(), buf.numel()))
        self._clk = buf  # kept alive while attached

    def profile_begin(self, kernels=KERNEL_NAMES, token_stride: int = 1):
        """Time launches of `kernels` in the steps of every token_stride-th token."""
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_NAMES.index(k)
        _check(self.lib.rlt_profile_begin(self.handle, mask, int(token_stride)))

    def profile_end(self) -> dict:
        """{kernel name: {launches, total_ms, bytes, flops}} for the timed kernels."""
        out = (rlt_kernel_stats * len(KERNEL_NAMES))()
        _check(self.lib.rlt_profile_end(self.handle, out))
        return {n: {"launches": o.launches, "total_ms": o.total_ms, "bytes": o.bytes,
                    "flops": o.flops} for n, o in zip(KERNEL_NAMES, out) if o.launches}

    def __del__(self):
        if getattr(self, "handle", None):
            self.lib.rlt_state_destroy(self.handle)
            self.handle = None


class Memory:
    """Encoder key/value memory of `batch` sequences for up to `capacity` tokens."""

    def __init__(self, model: Model, batch: int, capacity: int):
        self.lib, self.model, self.batch, self.capacity = model.lib, model, int(batch), int(capacity)
        nbytes = self.lib.rlt_memory_bytes(byref(model.cfg), self.batch, self.capacity)
        if nbytes == 0:
            raise RLTError(4, f"invalid batch {batch} or capacity {capacity}")
        self.buf = _device_buffer(nbytes, model.ws.device)
        h = c_void_p()
        _check(self.lib.rlt_memory_create(model.handle, self.batch, self.capacity,
                                          self.buf.data_ptr(), nbytes, byref(h)))
        self.handle = h

    @property
    def length(self) -> int:
        return self.lib.rlt_memory_length(self.handle)

    def reset(self):
        _check(self.lib.rlt_memory_reset(self.handle))

    def views(self):
        """(K, V) as tensors [G, B, H, capacity, hd] aliasing the memory buffer."""
        c = self.model.cfg
        n = c.n_groups * self.batch * c.n_heads * self.capacity * c.head_dim
        es = 2 if c.dtype == RLT_BF16 else 4
        half = (n * es + 255) // 256 * 256
        shape = (c.n_groups, self.batch, c.n_heads, self.capacity, c.head_dim)
        k = self.buf[: n * es].view(self.model.dtype).view(shape)
        v = self.buf[half: half + n * es].view(self.model.dtype).view(shape)
        return k, v

    def __del__(self):
        if getattr(self, "handle", None):
            self.lib.rlt_memory_destroy(self.handle)
            self.handle = None


def _need(t: torch.Tensor, shape, dtype, what):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA tensor")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)}")


def rlt_memproj(model: Model, mem: Memory, e: torch.Tensor, t0: int, stream=None):
    """Project e [B, n, d] into memory entries t0 .. t0+n-1."""
    B, n, d = e.shape
    _need(e, (mem.batch, n, model.cfg.d), model.dtype, "e")
    _check(model.lib.rlt_memproj(model.handle, mem.handle, e.data_ptr(), int(t0), int(n),
                                 _stream(stream)))


def rlt_decoder_step(model: Model, state: State, mem: Memory, e_t: torch.Tensor,
                     s_out: torch.Tensor | None = None, stream=None):
    """One recurrent step; e_t [B, d]; optional s_out [B, d] float32."""
    _need(e_t, (state.batch, model.cfg.d), model.dtype, "e_t")
    if s_out is not None:
        _need(s_out, (state.batch, model.cfg.d), torch.float32, "s_out")
    _check(model.lib.rlt_decoder_step(model.handle, state.handle, mem.handle, e_t.data_ptr(),
                                      _ptr(s_out), _stream(stream)))


def rlt_decoder_step_ragged(model: Model, state: State, mem: Memory, e_t: torch.Tensor,
                            active: torch.Tensor | None = None,
                            s_out: torch.Tensor | None = None, stream=None):
    """One step for the sequences with active[b] != 0 (device uint8 [B]; None = all), each at
    its own position; e_t [B, d]; optional s_out [B, d] float32."""
    _need(e_t, (state.batch, model.cfg.d), model.dtype, "e_t")
    if active is not None:
        _need(active, (state.batch,), torch.uint8, "active")
    if s_out is not None:
        _need(s_out, (state.batch, model.cfg.d), torch.float32, "s_out")
    _check(model.lib.rlt_decoder_step_ragged(model.handle, state.handle, mem.handle,
                                             e_t.data_ptr(), _ptr(active), _ptr(s_out),
                                             _stream(stream)))


def rlt_run_sequence(model: Model, state: State, mem: Memory, e: torch.Tensor,
                     s_traj: torch.Tensor | None = None, stream=None):
    """Memory projection of the missing tokens, then e.shape[1] steps; optional s_traj
    [B, n, d] float32."""
    n = e.shape[1]
    _need(e, (state.batch, n, model.cfg.d), model.dtype, "e")
    if s_traj is not None:
        _need(s_traj, (state.batch, n, model.cfg.d), torch.float32, "s_traj")
    _check(model.lib.rlt_run_sequence(model.handle, state.handle, mem.handle, e.data_ptr(), int(n),
                                      _ptr(s_traj), _stream(stream)))


def parallel_workspace(model: Model, batch: int, n: int) -> torch.Tensor:
    """Device workspace for rlt_run_parallel over n tokens of `batch` sequences."""
    nbytes = model.lib.rlt_parallel_ws_bytes(byref(model.cfg), int(batch), int(n))
    if nbytes == 0:
        raise RLTError(2, f"invalid batch {batch} or n {n} for the token-parallel pass")
    return _device_buffer(nbytes, model.ws.device)


def rlt_run_parallel(model: Model, state: State, mem: Memory, e: torch.Tensor,
                     s_traj: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                     stream=None):
    """Token-parallel pass over e [B, n, d] from a reset state (alpha = 0 models, bf16);
    optional s_traj [B, n, d] float32; `ws` from parallel_workspace (allocated if None)."""
    n = e.shape[1]
    _need(e, (state.batch, n, model.cfg.d), model.dtype, "e")
    if s_traj is not None:
        _need(s_traj, (state.batch, n, model.cfg.d), torch.float32, "s_traj")
    if ws is None:
        ws = parallel_workspace(model, state.batch, n)
    _check(model.lib.rlt_run_parallel(model.handle, state.handle, mem.handle, e.data_ptr(),
                                      int(n), _ptr(s_traj), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def rlt_run_parallel_noalloc(model: Model, state: State, mem: Memory, e: torch.Tensor,
                             s_traj: torch.Tensor | None = None, stream=None):
    """rlt_run_parallel with the library's own scratch array as workspace (nothing allocated;
    passes whose workspace exceeds rlt_scratch_bytes() raise RLT_ERR_CAPACITY)."""
    n = e.shape[1]
    _need(e, (state.batch, n, model.cfg.d), model.dtype, "e")
    if s_traj is not None:
        _need(s_traj, (state.batch, n, model.cfg.d), torch.float32, "s_traj")
    _check(model.lib.rlt_run_parallel_noalloc(model.handle, state.handle, mem.handle,
                                              e.data_ptr(), int(n), _ptr(s_traj),
                                              _stream(stream)))


def bptt_workspace(model: Model, batch: int, n: int) -> torch.Tensor:
    """Device workspace for rlt_bptt over n tokens of `batch` sequences."""
    nbytes = model.lib.rlt_bptt_ws_bytes(byref(model.cfg), int(batch), int(n))
    if nbytes == 0:
        raise RLTError(2, f"invalid batch {batch} or n {n} for the backward pass")
    return _device_buffer(nbytes, model.ws.device)


def grad_buffers(model: Model) -> dict:
    """Zero-initialised float32 device buffers shaped like the weights, one per rlt_grads
    field."""
    c = model.cfg
    d, F, L, G = c.d, c.ffn, c.n_layers, c.n_groups
    shapes = {"s_star": (d,), "w_gate": (2 * d, d), "b_gate": (d,), "gamma": (L, 3, d),
              "wq": (L, d, d), "wk": (L, d, d), "wv": (L, d, d), "wo": (L, d, d),
              "wcq": (L, d, d), "wco": (L, d, d), "w1": (L, d, F), "w3": (L, d, F),
              "w2": (L, F, d), "wmk": (G, d, d), "wmv": (G, d, d)}
    return {k: torch.zeros(shapes[k], dtype=torch.float32, device=model.ws.device)
            for k in WEIGHT_FIELDS}


def clock_buffer(slots: int, device="cuda") -> torch.Tensor:
    """Device buffer of `slots` clock slot pairs (16 bytes each): one per workgroup of each
    self-timed launch, i.e. H per sequence and launch for the attention kernels."""
    return torch.empty(int(slots) * 16, dtype=torch.uint8, device=device)


def rlt_bptt(model: Model, e: torch.Tensor, ds: torch.Tensor, grads: dict,
             de: torch.Tensor | None = None, s_traj: torch.Tensor | None = None,
             ws: torch.Tensor | None = None, stream=None, time_kernels=None,
             token_stride: int = 1, segment: int = 0, detach=(),
             clock: torch.Tensor | None = None):
    """Forward from s* over e [B, n, d] and backpropagation through time of the upstream
    gradients ds [B, n, d] float32 into `grads` (from grad_buffers; overwritten), de [B, n, d]
    float32 and s_traj [B, n, d] float32 (both optional); `ws` from bptt_workspace. With
    `time_kernels` (names from KERNEL_NAMES) the call waits for the stream and returns
    {name: {launches, total_ms, bytes, flops}} of those kernels' sampled launches.

    `clock` (a device buffer from clock_buffer) makes the backward attention kernels time
    themselves by their own clock stamps instead of events.

    segment = k > 0 truncates the backpropagation: at every start of a k-token segment the
    tensors named in `detach` ("state": the carried output s; "window": the self-attention
    keys/values of earlier tokens) pass no gradient back into the previous segment."""
    B, n = int(e.shape[0]), int(e.shape[1])
    d = model.cfg.d
    _need(e, (B, n, d), model.dtype, "e")
    _need(ds, (B, n, d), torch.float32, "ds")
    if de is not None:
        _need(de, (B, n, d), torch.float32, "de")
    if s_traj is not None:
        _need(s_traj, (B, n, d), torch.float32, "s_traj")
    for k in WEIGHT_FIELDS:
        if not isinstance(grads.get(k), torch.Tensor) or grads[k].dtype != torch.float32 \
                or not grads[k].is_contiguous() or not grads[k].is_cuda:
            raise ValueError(f"grads[{k!r}] must be a contiguous float32 CUDA tensor")
    if ws is None:
        ws = bptt_workspace(model, B, n)
    g = rlt_grads(*[grads[k].data_ptr() for k in WEIGHT_FIELDS])
    trunc = None
    if segment:
        bits = 0
        for k in detach:
            if k not in DETACH_BITS:
                raise ValueError(f"unknown detached tensor {k!r}")
            bits |= DETACH_BITS[k]
        trunc = rlt_truncation(int(segment), bits)
    timing = None
    stats = None
    if time_kernels:
        mask = 0
        for k in time_kernels:
            mask |= 1 << KERNEL_NAMES.index(k)
        timing = rlt_timing(mask, int(token_stride), _ptr(clock),
                            0 if clock is None else clock.numel() * clock.element_size())
        stats = (rlt_kernel_stats * len(KERNEL_NAMES))()
    _check(model.lib.rlt_bptt(model.handle, e.data_ptr(), B, n, ds.data_ptr(), _ptr(s_traj),
                              byref(g), _ptr(de), ws.data_ptr(), ws.numel() * ws.element_size(),
                              None if trunc is None else byref(trunc),
                              None if timing is None else byref(timing), stats, _stream(stream)))
    if stats is None:
        return None
    return {KERNEL_NAMES[i]: {"launches": stats[i].launches, "total_ms": stats[i].total_ms,
                              "bytes": stats[i].bytes, "flops": stats[i].flops}
            for i in range(len(KERNEL_NAMES)) if (timing.kernels >> i) & 1}


def rlt_state_export(state: State, stream=None):
    """Snapshot (s [B, d] f32, k, v [L, B, W-1, d] dtype, n_valid, position, version)."""
    c = state.model.cfg
    dev = state.buf.device
    s = torch.empty(state.batch, c.d, dtype=torch.float32, device=dev)
    keep = c.window - 1
    k = torch.empty(c.n_layers, state.batch, keep, c.d, dtype=state.model.dtype, device=dev)
    v = torch.empty_like(k)
    n_valid, pos, ver = c_int32(), c_int64(), c_uint64()
    _check(state.lib.rlt_state_export(state.handle, s.data_ptr(), _ptr(k) if keep else None,
                                      _ptr(v) if keep else None, byref(n_valid), byref(pos),
                                      byref(ver), _stream(stream)))
    return s, k, v, n_valid.value, pos.value, ver.value


def rlt_state_import(state: State, s: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     position: int, version: int, stream=None):
    c = state.model.cfg
    _need(s, (state.batch, c.d), torch.float32, "s")
    shape = (c.n_layers, state.batch, c.window - 1, c.d)
    _need(k, shape, state.model.dtype, "k")
    _need(v, shape, state.model.dtype, "v")
    if c.window == 1:  # nothing retained; pass any valid pointer
        k = v = s
    _check(state.lib.rlt_state_import(state.handle, s.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      int(position), int(version), _stream(stream)))


def rlt_state_import_ragged(state: State, s: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            positions, version: int, stream=None):
    """rlt_state_import for sequences at different positions (a list of B ints)."""
    c = state.model.cfg
    _need(s, (state.batch, c.d), torch.float32, "s")
    shape = (c.n_layers, state.batch, c.window - 1, c.d)
    _need(k, shape, state.model.dtype, "k")
    _need(v, shape, state.model.dtype, "v")
    if len(positions) != state.batch:
        raise ValueError(f"positions must have {state.batch} entries")
    if c.window == 1:
        k = v = s
    pos = (c_int64 * state.batch)(*[int(x) for x in positions])
    _check(state.lib.rlt_state_import_ragged(state.handle, s.data_ptr(), k.data_ptr(),
                                             v.data_ptr(), pos, int(version), _stream(stream)))


# ---- encoder and readout around the decoder ------------------------------------------------------

def upload_head_weights(params: dict, cfg: rlt_config, device="cuda") -> dict:
    """Host arrays -> contiguous device tensors in the layouts of rlt_head_weights (matrices and
    the embedding in the config dtype, gains in float32)."""
    out = {}
    dt = torch_dtype(cfg)
    for name in HEAD_FIELDS:
        x = params[name]
        x = torch.as_tensor(x) if not isinstance(x, torch.Tensor) else x
        out[name] = x.to(device=device,
                         dtype=torch.float32 if name in HEAD_FP32_FIELDS else dt).contiguous()
    return out


class Head:
    """Encoder and readout weights bound to a model (rlt_head_create)."""

    def __init__(self, model: Model, vocab: int, weights: dict, stream=None):
        self.lib, self.model, self.vocab = model.lib, model, int(vocab)
        nbytes = self.lib.rlt_head_ws_bytes(byref(model.cfg), self.vocab)
        if nbytes == 0:
            raise RLTError(2, f"invalid vocabulary size {vocab}")
        self.ws = _device_buffer(nbytes, model.ws.device)
        w = rlt_head_weights(*[_ptr(weights[n]) for n in HEAD_FIELDS])
        h = c_void_p()
        _check(self.lib.rlt_head_create(model.handle, self.vocab, byref(w), self.ws.data_ptr(),
                                        nbytes, _stream(stream), byref(h)))
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None):
            self.lib.rlt_head_destroy(self.handle)
            self.handle = None


def rlt_encode(head: Head, tokens: torch.Tensor, e: torch.Tensor | None = None,
               ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Token-parallel causal encoder over token ids [B, n] (int32, device) -> e [B, n, d]."""
    m = head.model
    B, n = tokens.shape
    if tokens.dtype != torch.int32 or not tokens.is_contiguous():
        raise ValueError("tokens must be a contiguous int32 tensor")
    if e is None:
        e = torch.empty(B, n, m.cfg.d, dtype=m.dtype, device=tokens.device)
    _need(e, (B, n, m.cfg.d), m.dtype, "e")
    if ws is None:
        nbytes = head.lib.rlt_encode_ws_bytes(byref(m.cfg), int(B), int(n))
        if nbytes == 0:
            raise RLTError(3 if m.cfg.dtype != RLT_BF16 else 2,
                           "the encoder needs a bf16 model and a valid batch and length")
        ws = _device_buffer(nbytes, tokens.device)
    _check(head.lib.rlt_encode(m.handle, head.handle, tokens.data_ptr(), int(B), int(n),
                               e.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                               _stream(stream)))
    return e


def readout_workspace(head: Head, batch: int) -> torch.Tensor:
    nbytes = head.lib.rlt_readout_ws_bytes(byref(head.model.cfg), head.vocab, int(batch))
    if nbytes == 0:
        raise RLTError(2, f"invalid batch {batch}")
    return _device_buffer(nbytes, head.ws.device)


def rlt_readout(head: Head, s: torch.Tensor, u: torch.Tensor, temperature: float = 1.0,
                top_k: int = 0, top_p: float = 1.0, logits: torch.Tensor | None = None,
                ws: torch.Tensor | None = None, stream=None):
    """Readout and sampling of s [B, d] (float32) with uniforms u [B] (float32): returns
    (tokens [B] int32, logp_behaviour [B], logp_model [B]) as device tensors; `logits`
    [B, V] float32 receives the logits when given."""
    m = head.model
    B = s.shape[0]
    _need(s, (B, m.cfg.d), torch.float32, "s")
    _need(u, (B,), torch.float32, "u")
    if logits is not None:
        _need(logits, (B, head.vocab), torch.float32, "logits")
    if ws is None:
        ws = readout_workspace(head, B)
    tok = torch.empty(B, dtype=torch.int32, device=s.device)
    lpb = torch.empty(B, dtype=torch.float32, device=s.device)
    lpm = torch.empty(B, dtype=torch.float32, device=s.device)
    sp = rlt_sampling(float(temperature), int(top_k), float(top_p))
    _check(head.lib.rlt_readout(m.handle, head.handle, s.data_ptr(), int(B), byref(sp),
                                u.data_ptr(), tok.data_ptr(), lpb.data_ptr(), lpm.data_ptr(),
                                _ptr(logits), ws.data_ptr(), ws.numel() * ws.element_size(),
                                _stream(stream)))
    return tok, lpb, lpm
