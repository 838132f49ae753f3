"""Python binding of the MLA gather-decode C ABI (include/mla_gather_decode.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, and their device pointers are handed to the HIP library, which
runs every part of the step.  There is no fallback: if the library is not
built, or the step fails, an exception is raised.

    from sparse_gather_mla_amd import MlaGatherDecode
    step = MlaGatherDecode(dims, max_tokens=T, device=0)
    out = step(inputs)              # inputs: dict keyed by the page's parameter names
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# MLA_GD_LIBRARY selects another build of the same library (same ABI).
LIB_PATH = os.environ.get("MLA_GD_LIBRARY") or os.path.join(_PKG, "libmla_gather_decode.so")

MLA_GD_FLAG_FUSED = 1
MLA_GD_FLAG_GRAPH = 2
MLA_GD_FLAG_DEBUG_CHECKS = 4
MLA_GD_FLAG_SINGLE_LAUNCH = 8
MLA_GD_CHECK_SLOT_RANGE, MLA_GD_CHECK_BLOCK_RANGE, MLA_GD_CHECK_TABLE_COLUMN, MLA_GD_CHECK_SLOT_SHARED = 1, 2, 4, 8
MLA_GD_CHECK_SEQ_RANGE = 16
MLA_GD_CHECK_WAIT_TIMEOUT = 32


class MlaGdError(RuntimeError):
    def __init__(self, code: int, what: str, hip_error: int = 0):
        self.code = code
        self.hip_error = hip_error
        super().__init__(f"{what}: {_strerror(code)} (code {code}, hipError {hip_error})")


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "q_lora_rank", "kv_lora_rank", "qk_nope_head_dim", "qk_rope_head_dim", "v_head_dim",
        "n_heads", "block_size", "max_blocks_per_seq", "n_blocks", "n_prior", "max_tokens")] + [
        ("softmax_scale", ctypes.c_float), ("norm_eps", ctypes.c_float), ("flags", ctypes.c_uint32)]


TENSOR_FIELDS = ("hidden_states", "input_norm_w", "wq_a", "q_norm_w", "wq_b", "wkv_a", "kv_norm_w",
                 "q_absorb_w", "out_absorb_w", "o_proj_w", "cos_table", "sin_table", "kv_cache",
                 "slot_mapping", "block_table", "positions", "gather_indices", "out", "gather_rows_out",
                 "token_seq")


class _Tensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TENSOR_FIELDS]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} (run sparse_gather_mla_amd/build.py)")
    lib = ctypes.CDLL(path)
    lib.mla_gather_decode_create.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
    lib.mla_gather_decode_create.restype = ctypes.c_int
    lib.mla_gather_decode_destroy.argtypes = [ctypes.c_void_p]
    lib.mla_gather_decode_destroy.restype = None
    lib.mla_gather_decode_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.mla_gather_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_gather_decode_workspace_init.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_gather_decode_workspace_init.restype = ctypes.c_int
    lib.mla_gather_decode_step.argtypes = [ctypes.c_void_p, ctypes.POINTER(_Tensors), ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mla_gather_decode_step.restype = ctypes.c_int
    lib.mla_gather_decode_strerror.argtypes = [ctypes.c_int]
    lib.mla_gather_decode_strerror.restype = ctypes.c_char_p
    lib.mla_gather_decode_last_hip_error.argtypes = [ctypes.c_void_p]
    lib.mla_gather_decode_last_hip_error.restype = ctypes.c_int
    lib.mla_gather_decode_step_profiled.argtypes = [ctypes.c_void_p, ctypes.POINTER(_Tensors), ctypes.c_int32,
                                                    ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    lib.mla_gather_decode_step_profiled.restype = ctypes.c_int
    lib.mla_gather_decode_debug_status.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32),
                                                   ctypes.c_void_p]
    lib.mla_gather_decode_debug_status.restype = ctypes.c_int
    lib.mla_gather_decode_kernel_count.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.mla_gather_decode_kernel_count.restype = ctypes.c_int
    lib.mla_gather_decode_kernel_name.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int]
    lib.mla_gather_decode_kernel_name.restype = ctypes.c_char_p
    lib.mla_gather_decode_step_noalloc.argtypes = [ctypes.c_void_p, ctypes.POINTER(_Tensors), ctypes.c_int32,
                                                   ctypes.c_void_p]
    lib.mla_gather_decode_step_noalloc.restype = ctypes.c_int
    lib.mla_gather_decode_abi_version.argtypes = []
    lib.mla_gather_decode_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _strerror(code: int) -> str:
    try:
        return load_library().mla_gather_decode_strerror(code).decode()
    except Exception:  # pragma: no cover
        return "?"


@dataclass
class Dims:
    """Step dimensions (the fields of mla_gd_dims)."""

    hidden: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    n_heads: int
    block_size: int
    max_blocks_per_seq: int
    n_blocks: int
    n_prior: int
    softmax_scale: float
    norm_eps: float = 1e-6

    @classmethod
    def from_shape(cls, sh) -> "Dims":
        """From any object with the page's dimension names (e.g. workload.MlaShape)."""
        return cls(hidden=sh.hidden, q_lora_rank=sh.q_lora_rank, kv_lora_rank=sh.kv_lora_rank,
                   qk_nope_head_dim=sh.qk_nope_head_dim, qk_rope_head_dim=sh.qk_rope_head_dim,
                   v_head_dim=sh.v_head_dim, n_heads=sh.n_heads, block_size=sh.block_size,
                   max_blocks_per_seq=sh.max_blocks_per_seq, n_blocks=sh.n_blocks, n_prior=sh.n_prior,
                   softmax_scale=sh.softmax_scale, norm_eps=sh.norm_eps)


class MlaGatherDecode:
    """One handle of the C library plus a workspace, for up to ``max_tokens`` tokens."""

    def __init__(self, dims: Dims, max_tokens: int, device: int = 0, fused: bool = False,
                 allocate_workspace: bool = True, graph: bool = False, debug_checks: bool = False,
                 single_launch: bool = False):
        """``fused``: the fused variant (kv rows, absorption and core in one launch).
        ``single_launch``: the whole step as one launch (few tokens, at most 16 heads).
        ``graph``: capture the step once into a HIP graph and replay it (default:
        kernels launched one by one).  ``debug_checks``: device-side checks of
        the index data (slot range and sharing, block-table column and block id
        ranges); see debug_status()."""
        import torch

        self.lib = load_library()
        self.dims = dims
        self.max_tokens = int(max_tokens)
        self.device = torch.device("cuda", device)
        self.fused = fused
        self.single_launch = single_launch
        self.graph = graph
        cd = _Dims(hidden=dims.hidden, q_lora_rank=dims.q_lora_rank, kv_lora_rank=dims.kv_lora_rank,
                   qk_nope_head_dim=dims.qk_nope_head_dim, qk_rope_head_dim=dims.qk_rope_head_dim,
                   v_head_dim=dims.v_head_dim, n_heads=dims.n_heads, block_size=dims.block_size,
                   max_blocks_per_seq=dims.max_blocks_per_seq, n_blocks=dims.n_blocks, n_prior=dims.n_prior,
                   max_tokens=self.max_tokens, softmax_scale=dims.softmax_scale, norm_eps=dims.norm_eps,
                   flags=(MLA_GD_FLAG_FUSED if fused else 0) | (MLA_GD_FLAG_GRAPH if graph else 0)
                   | (MLA_GD_FLAG_DEBUG_CHECKS if debug_checks else 0)
                   | (MLA_GD_FLAG_SINGLE_LAUNCH if single_launch else 0))
        h = ctypes.c_void_p()
        rc = self.lib.mla_gather_decode_create(ctypes.byref(cd), int(device), ctypes.byref(h))
        if rc != 0:
            raise MlaGdError(rc, "mla_gather_decode_create")
        self.handle = h
        self.workspace = None
        if allocate_workspace:
            self.workspace = self.new_workspace(self.max_tokens)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self.lib.mla_gather_decode_destroy(h)
            self.handle = None

    def workspace_size(self, n_tokens: int) -> int:
        return int(self.lib.mla_gather_decode_workspace_size(self.handle, int(n_tokens)))

    def new_workspace(self, n_tokens: int):
        """Allocate (torch) and zero (library) a workspace for steps of up to n_tokens."""
        import torch

        nbytes = self.workspace_size(n_tokens)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.mla_gather_decode_workspace_init(self.handle, ctypes.c_void_p(ws.data_ptr()),
                                                       ctypes.c_size_t(nbytes), ctypes.c_void_p(stream))
        if rc != 0:
            raise MlaGdError(rc, "mla_gather_decode_workspace_init", self.lib.mla_gather_decode_last_hip_error(self.handle))
        return ws

    def _check(self, name, t, dtype, shape):
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch tensor")
        if t.device != self.device:
            raise ValueError(f"{name}: on {t.device}, expected {self.device}")
        if t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        return t.data_ptr()

    def __call__(self, inp: Dict[str, object], **kw):
        return self.step(inp, **kw)

    def debug_status(self, workspace=None) -> int:
        """Error bits (MLA_GD_CHECK_*) the debug checks recorded since the last
        read, after the work enqueued on the current stream; clears them."""
        import torch

        ws = self.workspace if workspace is None else workspace
        bits = ctypes.c_uint32(0)
        stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = self.lib.mla_gather_decode_debug_status(self.handle, ctypes.c_void_p(ws.data_ptr()), ctypes.byref(bits),
                                                     ctypes.c_void_p(stream))
        if rc not in (0, 6):  # MLA_GD_OK, MLA_GD_E_DEVICE_CHECK
            raise MlaGdError(rc, "mla_gather_decode_debug_status", self.lib.mla_gather_decode_last_hip_error(self.handle))
        return int(bits.value)

    def kernel_names(self, n_tokens: int):
        """Names of the kernels a step of ``n_tokens`` tokens launches, in order."""
        n = self.lib.mla_gather_decode_kernel_count(self.handle, n_tokens)
        return [self.lib.mla_gather_decode_kernel_name(self.handle, n_tokens, i).decode() for i in range(n)]

    def step(self, inp: Dict[str, object], out=None, gather_rows_out=None, workspace=None, stream=None,
             events=None, noalloc=False):
        """Enqueue one step on ``stream`` (default: torch's current stream); returns ``out``.

        ``events``: optional list of len(kernel_names(T))+1 torch.cuda.Event(enable_timing=True)
        recorded around each kernel of the step on that stream.  ``noalloc``:
        the allocation-free entry point (mla_gather_decode_step_noalloc), whose
        workspace is the library's static device array (``workspace`` and
        ``events`` must be None; pass ``out``, or a new tensor is allocated here)."""
        import torch

        d = self.dims
        bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
        x = inp["hidden_states"]
        T = int(x.shape[0])
        if not 1 <= T <= self.max_tokens:
            raise ValueError(f"n_tokens {T} outside [1, {self.max_tokens}]")
        for k, v in (("n_heads", d.n_heads), ("qk_nope_head_dim", d.qk_nope_head_dim),
                     ("qk_rope_head_dim", d.qk_rope_head_dim), ("kv_lora_rank", d.kv_lora_rank)):
            if k in inp and int(inp[k]) != v:
                raise ValueError(f"{k}={inp[k]} does not match the handle ({v})")
        H, Q, r, dn, dr, dv, nh = (d.hidden, d.q_lora_rank, d.kv_lora_rank, d.qk_nope_head_dim,
                                   d.qk_rope_head_dim, d.v_head_dim, d.n_heads)
        kvr = r + dr
        if out is None:
            out = torch.empty((T, H), dtype=bf, device=self.device)
        spec = {
            "hidden_states": (inp["hidden_states"], bf, (T, H)),
            "input_norm_w": (inp["input_norm_w"], f32, (1, H)),
            "wq_a": (inp["wq_a"], bf, (H, Q)),
            "q_norm_w": (inp["q_norm_w"], f32, (1, Q)),
            "wq_b": (inp["wq_b"], bf, (Q, nh * (dn + dr))),
            "wkv_a": (inp["wkv_a"], bf, (H, kvr)),
            "kv_norm_w": (inp["kv_norm_w"], f32, (1, r)),
            "q_absorb_w": (inp["q_absorb_w"], bf, (nh, dn, r)),
            "out_absorb_w": (inp["out_absorb_w"], bf, (nh, dv, r)),
            "o_proj_w": (inp["o_proj_w"], bf, (nh * dv, H)),
            "cos_table": (inp["cos"], f32, (T, dr // 2)),
            "sin_table": (inp["sin"], f32, (T, dr // 2)),
            "kv_cache": (inp["kv_cache"], bf, (d.n_blocks, 1, d.block_size, kvr)),
            "slot_mapping": (inp["slot_mapping"], i32, (T,)),
            # with token_seq the table has one row per sequence of the step (at most T)
            "block_table": (inp["block_table"], i32,
                            ((int(inp["block_table"].shape[0]) if inp.get("token_seq") is not None else T),
                             d.max_blocks_per_seq)),
            "positions": (inp["positions"], i32, (T,)),
            "gather_indices": (inp["gather_indices"], i32, (T, d.n_prior)),
            "out": (out, bf, (T, H)),
        }
        tn = _Tensors()
        for name, (t, dt, shp) in spec.items():
            setattr(tn, name, self._check(name, t, dt, shp))
        if gather_rows_out is not None:
            tn.gather_rows_out = self._check("gather_rows_out", gather_rows_out, i32, (T, d.n_prior))
        if inp.get("token_seq") is not None:
            if not 1 <= int(inp["block_table"].shape[0]) <= T:
                raise ValueError("block_table with token_seq: one row per sequence, at most n_tokens rows")
            tn.token_seq = self._check("token_seq", inp["token_seq"], i32, (T,))
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        if noalloc:
            if workspace is not None or events is not None:
                raise ValueError("noalloc steps take neither a workspace nor events")
            rc = self.lib.mla_gather_decode_step_noalloc(self.handle, ctypes.byref(tn), T,
                                                         ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise MlaGdError(rc, "mla_gather_decode_step_noalloc",
                                 self.lib.mla_gather_decode_last_hip_error(self.handle))
            return out
        ws = workspace if workspace is not None else self.workspace
        if ws is None:
            raise ValueError("no workspace")
        ws_ptr = ctypes.c_void_p(ws.data_ptr())
        ws_bytes = ctypes.c_size_t(ws.numel() * ws.element_size())
        st = ctypes.c_void_p(stream.cuda_stream)
        if events is None:
            rc = self.lib.mla_gather_decode_step(self.handle, ctypes.byref(tn), T, ws_ptr, ws_bytes, st)
        else:
            for ev in events:
                if not ev.cuda_event:  # torch creates the HIP event on first record
                    ev.record(stream)
            arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
            rc = self.lib.mla_gather_decode_step_profiled(self.handle, ctypes.byref(tn), T, ws_ptr, ws_bytes, st,
                                                          arr, len(events))
        if rc != 0:
            raise MlaGdError(rc, "mla_gather_decode_step", self.lib.mla_gather_decode_last_hip_error(self.handle))
        return out
