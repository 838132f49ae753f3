"""Thin binding of the fused RMSNorm + router top-K (include/rmsnorm_router_topk.h).

Argument marshalling only: every step runs in the library's HIP kernels; without
the built library this raises."""
import ctypes

from . import load_library

RT_ACT_SIGMOID, RT_ACT_SOFTMAX = 0, 1
RT_DTYPE_BF16, RT_DTYPE_FP16 = 0, 1
_ACTS = {"sigmoid": RT_ACT_SIGMOID, "softmax": RT_ACT_SOFTMAX}
_ready = set()


def _lib():
    lib = load_library()
    if id(lib) not in _ready:
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.rmsnorm_router_topk_workspace_size.argtypes = [i32, i32, i32]
        lib.rmsnorm_router_topk_workspace_size.restype = ctypes.c_size_t
        lib.rmsnorm_router_topk.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, vp, vp, vp, vp,
                                            ctypes.c_size_t, vp]
        lib.rmsnorm_router_topk.restype = ctypes.c_int
        lib.rmsnorm_router_topk_typed.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float, i32, vp, vp,
                                                  vp, vp, ctypes.c_size_t, vp]
        lib.rmsnorm_router_topk_typed.restype = ctypes.c_int
        _ready.add(id(lib))
    return lib


def workspace_size(n_tokens: int, hidden: int, n_experts: int) -> int:
    return int(_lib().rmsnorm_router_topk_workspace_size(n_tokens, hidden, n_experts))


def rmsnorm_router_topk(hidden_states, gamma, router_weights, router_bias=None, eps: float = 1e-6, top_k: int = 1,
                        act: str = "sigmoid", workspace=None, stream=None, out=None):
    """Returns (normed [T, H], indices [T, K] int32, affinities [T, E] bf16).  The
    three inputs are all bf16 or all fp16; normed has their type."""
    import torch

    lib = _lib()
    T, H = hidden_states.shape
    E = router_weights.shape[1]
    dev = hidden_states.device
    dt_in = hidden_states.dtype
    if dt_in not in (torch.bfloat16, torch.float16):
        raise ValueError(f"hidden_states: dtype {dt_in}, expected bfloat16 or float16")
    for name, t, dt, shp in (("hidden_states", hidden_states, dt_in, (T, H)),
                             ("gamma", gamma, dt_in, (H,)),
                             ("router_weights", router_weights, dt_in, (H, E))):
        if t.dtype != dt or tuple(t.shape) != shp or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name}: expected contiguous {dt} {shp} on {dev}")
    if router_bias is not None and (router_bias.dtype != torch.float32 or tuple(router_bias.shape) != (E,)
                                    or not router_bias.is_contiguous() or router_bias.device != dev):
        raise ValueError(f"router_bias: expected contiguous float32 ({E},) on {dev}")
    if out is None:
        out = (torch.empty((T, H), dtype=dt_in, device=dev),
               torch.empty((T, top_k), dtype=torch.int32, device=dev),
               torch.empty((T, E), dtype=torch.bfloat16, device=dev))
    normed, idx, aff = out
    nbytes = workspace_size(T, H, E)
    if workspace is None:
        workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)  # the counter starts at zero
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    dtype = RT_DTYPE_FP16 if dt_in == torch.float16 else RT_DTYPE_BF16
    rc = lib.rmsnorm_router_topk_typed(dtype, hidden_states.data_ptr(), gamma.data_ptr(), router_weights.data_ptr(),
                                 router_bias.data_ptr() if router_bias is not None else None, T, H, E, top_k, eps,
                                 _ACTS[act], normed.data_ptr(), idx.data_ptr(), aff.data_ptr(), workspace.data_ptr(),
                                 workspace.numel(), s)
    if rc != 0:
        raise RuntimeError(f"rmsnorm_router_topk failed with code {rc}")
    return normed, idx, aff
