"""Python binding of the MI355X MoE FFN layer library (``libmoe.so``, C ABI in ``include/moe.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of ``libmoe.so``.
PyTorch supplies device memory (tensors) and the stream. There is no CPU fallback: importing works
without the library, but every call raises ``MoeLibraryMissing`` if ``libmoe.so`` was not built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_EWORKSPACE", "MOE_EHIP", "MOE_ESCRATCH",
    "MOE_NOALLOC_SCRATCH_BYTES", "moe_layer_forward_noalloc",
    "MOE_BF16", "MOE_F32", "MOE_ACT_GELU", "MOE_ACT_GELU_TANH", "MOE_ACT_SWIGLU",
    "MOE_TOKEN_CHOICE", "MOE_EXPERT_CHOICE", "MOE_DES_VOTE", "MOE_DES_SEQ",
    "MOE_F_INPUT_PROBS", "MOE_F_SYNC_DEBUG", "MOE_F_FORCE_TILED", "MOE_F_FORCE_STREAM", "MOE_F_ROUTE_MULTI",
    "MoeDesc", "MoeRouting", "MoeWeights", "MoeError", "MoeLibraryMissing",
    "lib", "lib_path", "EXPORTS",
    "moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
    "moe_layer_forward", "moe_strerror", "moe_profile_begin", "moe_profile_end", "moe_attnres_aggregate",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_BF16, MOE_F32 = 0, 1
MOE_ACT_GELU, MOE_ACT_GELU_TANH, MOE_ACT_SWIGLU = 0, 1, 2
MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE, MOE_DES_VOTE, MOE_DES_SEQ = 0, 1, 2, 3
MOE_F_INPUT_PROBS, MOE_F_SYNC_DEBUG, MOE_F_FORCE_TILED, MOE_F_FORCE_STREAM = 0x1, 0x4, 0x8, 0x10
MOE_F_ROUTE_MULTI = 0x20

# the layer's C ABI (include/moe.h) and the measurement hooks (include/moe_prof.h)
EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine",
           "moe_layer_forward", "moe_layer_forward_noalloc", "moe_strerror", "moe_attnres_aggregate")
PROF_EXPORTS = ("moe_profile_begin", "moe_profile_end", "moe_profile_entry")

_i32, _f32, _u32, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_uint32, ctypes.c_void_p


class MoeDesc(ctypes.Structure):
    _fields_ = [("S", _i32), ("d", _i32), ("d_ff", _i32),
                ("E_heavy", _i32), ("n_identity", _i32), ("n_zero", _i32), ("n_const", _i32),
                ("n_shared", _i32), ("dtype", _i32), ("act", _i32), ("mode", _i32),
                ("k", _i32), ("renorm", _i32), ("capacity_factor", _f32),
                ("vote_k", _i32), ("m_core", _i32), ("reuse_tau", _f32), ("flags", _u32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("topk_idx", "topk_w", "probs", "counts", "offsets", "row_token", "row_w",
                                   "token_rows", "token_off", "token_list", "core", "votes", "reuse",
                                   "n_rows", "capacity")]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_router", "w1", "w3", "w2", "s_w1", "s_w3", "s_w2", "const_vec")]


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {status} ({moe_strerror(status)})")


class MoeLibraryMissing(RuntimeError):
    pass


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises MoeLibraryMissing when libmoe.so has not been built."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise MoeLibraryMissing(f"{p} is missing: build it with `python -m mixture_experts_layer_gemm_amd.build`")
        L = ctypes.CDLL(p)
        P = ctypes.POINTER
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [P(MoeDesc)]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [P(MoeDesc), _vp, P(MoeRouting), _vp, ctypes.c_size_t, _vp]
        L.moe_dispatch.restype = ctypes.c_int
        L.moe_dispatch.argtypes = [P(MoeDesc), _vp, P(MoeRouting), _vp, _vp]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [P(MoeDesc), _vp, _vp, P(MoeRouting), P(MoeWeights), _vp, _vp, _vp,
                                     ctypes.c_size_t, _vp]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [P(MoeDesc), _vp, P(MoeRouting), _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [P(MoeDesc), _vp, P(MoeWeights), _vp, _vp, P(MoeRouting), _vp, _vp, _vp,
                                        _vp, ctypes.c_size_t, _vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [P(MoeDesc), _vp, P(MoeWeights), _vp, _vp, P(MoeRouting), _vp, _vp,
                                                _vp, _vp]
        L.moe_attnres_aggregate.restype = ctypes.c_int
        L.moe_attnres_aggregate.argtypes = [_i32, _i32, _i32, _i32, P(_vp), _vp, _f32, _vp, _vp]
        L.moe_strerror.restype = ctypes.c_char_p
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_profile_begin.restype = ctypes.c_int
        L.moe_profile_begin.argtypes = []
        L.moe_profile_end.restype = ctypes.c_int
        L.moe_profile_end.argtypes = []
        L.moe_profile_entry.restype = ctypes.c_int
        L.moe_profile_entry.argtypes = [ctypes.c_int, P(ctypes.c_char_p), P(ctypes.c_double), P(_i32)]
        _LIB = L
    return _LIB


def _ptr(t) -> int | None:
    """Device address of a tensor (or an int address), None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str, raise_on_error: bool) -> int:
    if status != MOE_OK and raise_on_error:
        raise MoeError(status, call)
    return status


def moe_strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def moe_workspace_bytes(desc: MoeDesc) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc)))


def moe_route(desc, logits, routing: MoeRouting, ws, ws_bytes=None, stream=None, raise_on_error=True) -> int:
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    st = lib().moe_route(ctypes.byref(desc), _ptr(logits), ctypes.byref(routing), _ptr(ws), nb, _stream(stream))
    return _check(st, "moe_route", raise_on_error)


def moe_attnres_aggregate(dtype: int, S: int, d: int, states, query, eps: float, out, stream=None,
                          raise_on_error=True) -> int:
    """Attention-residual aggregation: ``states`` is a sequence of n device tensors (or addresses)
    of [S, d]; their addresses go to the library as a host array."""
    ptrs = (_vp * max(1, len(states)))(*[_ptr(t) for t in states])
    st = lib().moe_attnres_aggregate(int(dtype), int(S), int(d), len(states), ptrs if len(states) else None,
                                     _ptr(query), float(eps), _ptr(out), _stream(stream))
    return _check(st, "moe_attnres_aggregate", raise_on_error)


def moe_dispatch(desc, x, routing: MoeRouting, x_perm, stream=None, raise_on_error=True) -> int:
    st = lib().moe_dispatch(ctypes.byref(desc), _ptr(x), ctypes.byref(routing), _ptr(x_perm), _stream(stream))
    return _check(st, "moe_dispatch", raise_on_error)


def moe_expert_ffn(desc, x, x_perm, routing: MoeRouting, weights: MoeWeights, y_perm, y_shared, ws, ws_bytes=None,
                   stream=None, raise_on_error=True) -> int:
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    st = lib().moe_expert_ffn(ctypes.byref(desc), _ptr(x), _ptr(x_perm), ctypes.byref(routing),
                              ctypes.byref(weights), _ptr(y_perm), _ptr(y_shared), _ptr(ws), nb, _stream(stream))
    return _check(st, "moe_expert_ffn", raise_on_error)


def moe_combine(desc, x, routing: MoeRouting, y_perm, y_shared, const_vec, cache, residual, y, stream=None,
                raise_on_error=True) -> int:
    st = lib().moe_combine(ctypes.byref(desc), _ptr(x), ctypes.byref(routing), _ptr(y_perm), _ptr(y_shared),
                           _ptr(const_vec), _ptr(cache), _ptr(residual), _ptr(y), _stream(stream))
    return _check(st, "moe_combine", raise_on_error)


def moe_layer_forward(desc, x, weights: MoeWeights, prev_logits, logits_out, routing, cache, residual, y, ws,
                      ws_bytes=None, stream=None, raise_on_error=True) -> int:
    nb = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    rp = ctypes.byref(routing) if routing is not None else None
    st = lib().moe_layer_forward(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(prev_logits),
                                 _ptr(logits_out), rp, _ptr(cache), _ptr(residual), _ptr(y), _ptr(ws), nb,
                                 _stream(stream))
    return _check(st, "moe_layer_forward", raise_on_error)


def moe_layer_forward_noalloc(desc, x, weights: MoeWeights, prev_logits, logits_out, routing, cache, residual, y,
                              stream=None, raise_on_error=True) -> int:
    """moe_layer_forward with the library's static scratch array in place of a workspace."""
    rp = ctypes.byref(routing) if routing is not None else None
    st = lib().moe_layer_forward_noalloc(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(prev_logits),
                                         _ptr(logits_out), rp, _ptr(cache), _ptr(residual), _ptr(y), _stream(stream))
    return _check(st, "moe_layer_forward_noalloc", raise_on_error)


def moe_profile_begin() -> None:
    _check(lib().moe_profile_begin(), "moe_profile_begin", True)


def moe_profile_end() -> dict:
    """Stop profiling; {kernel name: (total ms, launches)} of the launches since moe_profile_begin."""
    L = lib()
    n = L.moe_profile_end()
    if n < 0:
        raise MoeError(n, "moe_profile_end")
    out = {}
    for i in range(n):
        name, ms, cnt = ctypes.c_char_p(), ctypes.c_double(), _i32()
        _check(L.moe_profile_entry(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt)), "moe_profile_entry",
               True)
        out[name.value.decode()] = (ms.value, cnt.value)
    return out


# ------------------------------------------------------------------------------------------------
# Marshalling helpers: descriptors from a layer spec, and device buffers for the routing outputs.

_ACT = {"gelu": MOE_ACT_GELU, "gelu_tanh": MOE_ACT_GELU_TANH, "swiglu": MOE_ACT_SWIGLU}
_MODE = {"tc": MOE_TOKEN_CHOICE, "ec": MOE_EXPERT_CHOICE, "des": MOE_DES_VOTE, "des_seq": MOE_DES_SEQ}


def desc_from_spec(spec, flags: int = 0) -> MoeDesc:
    """MoeDesc for an object with the fields of ``synth.LayerSpec``."""
    return MoeDesc(S=spec.S, d=spec.d, d_ff=spec.f, E_heavy=spec.E_heavy, n_identity=spec.n_identity,
                   n_zero=spec.n_zero, n_const=spec.n_const, n_shared=spec.n_shared,
                   dtype=MOE_BF16 if spec.dtype == "bf16" else MOE_F32, act=_ACT[spec.act], mode=_MODE[spec.mode],
                   k=spec.k, renorm=1 if spec.renorm else 0, capacity_factor=spec.capacity_factor,
                   vote_k=spec.vote_k, m_core=spec.m_core, reuse_tau=spec.reuse_tau, flags=flags)


@dataclass
class RoutingBuffers:
    """Device tensors behind a MoeRouting (allocated with torch). ``slots`` is the slot count of
    topk_idx / topk_w / token_rows and ``rows`` the length of row_token / row_w / token_list: upper
    bounds on what a call writes. The expert-choice capacity is read back from ``capacity``."""

    slots: int
    rows: int
    tensors: dict
    struct: MoeRouting

    def __getitem__(self, name):
        return self.tensors[name]


def routing_bounds(desc: MoeDesc) -> tuple[int, int]:
    """(slots per token, rows) upper bounds for the routing arrays of a descriptor: k slots (DES-Vote
    fills min(k, m_core) of them as a dense [S, min(k, m_core)] array, which fits), and S * k rows
    (token choice, DES) or S * E_r rows (expert choice: each expert takes at most every token)."""
    E_r = desc.E_heavy + desc.n_identity + desc.n_zero + desc.n_const
    if desc.mode == MOE_EXPERT_CHOICE:
        return 1, desc.S * E_r
    return max(desc.k, 1), desc.S * max(desc.k, 1)


def alloc_routing(desc: MoeDesc, device="cuda", with_probs: bool = True) -> RoutingBuffers:
    import torch
    E_r = desc.E_heavy + desc.n_identity + desc.n_zero + desc.n_const
    kk, R = routing_bounds(desc)
    S = desc.S
    i32, f32 = torch.int32, torch.float32
    t = {}
    t["topk_idx"] = torch.full((S, kk), -7, dtype=i32, device=device)
    t["topk_w"] = torch.zeros((S, kk), dtype=f32, device=device)
    if with_probs:
        t["probs"] = torch.zeros((S, E_r), dtype=f32, device=device)
    t["counts"] = torch.zeros(E_r, dtype=i32, device=device)
    t["offsets"] = torch.zeros(E_r + 1, dtype=i32, device=device)
    t["row_token"] = torch.full((max(R, 1),), -7, dtype=i32, device=device)
    t["row_w"] = torch.zeros(max(R, 1), dtype=f32, device=device)
    t["token_rows"] = torch.full((S, kk), -7, dtype=i32, device=device)
    t["token_off"] = torch.zeros(S + 1, dtype=i32, device=device)
    t["token_list"] = torch.full((max(R, 1),), -7, dtype=i32, device=device)
    t["core"] = torch.full((E_r,), -7, dtype=i32, device=device)
    t["votes"] = torch.zeros(E_r, dtype=f32, device=device)
    t["reuse"] = torch.zeros(S, dtype=torch.uint8, device=device)
    t["n_rows"] = torch.zeros(1, dtype=i32, device=device)
    t["capacity"] = torch.zeros(1, dtype=i32, device=device)
    st = MoeRouting(**{n: (v.data_ptr() if v is not None else None) for n, v in t.items()})
    return RoutingBuffers(kk, R, t, st)


def workspace(desc: MoeDesc, device="cuda"):
    """A workspace tensor of moe_workspace_bytes(desc) bytes (torch allocations are 256-byte aligned)."""
    import torch
    n = moe_workspace_bytes(desc)
    if n == 0:
        raise MoeError(MOE_EINVAL, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def weights_struct(tensors: dict) -> MoeWeights:
    """MoeWeights from a dict of device tensors (missing keys -> NULL)."""
    return MoeWeights(**{n: _ptr(tensors.get(n)) for n, _ in MoeWeights._fields_})
