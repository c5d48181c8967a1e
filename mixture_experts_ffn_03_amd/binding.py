"""ctypes binding of libmoe_fp4.so (the C ABI in include/moe_fp4.h).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
torch is used for device memory (tensors) and for the current HIP stream. If the
library has not been built, loading raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_fp4.so")

MOE_OK = 0
FMT_NVFP4, FMT_MXFP4, FMT_FP8, FMT_BF16 = 0, 1, 2, 3
SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_SQRT_SOFTPLUS, SCORE_SOFTMAX_BIAS = 0, 1, 2, 3
SELECT_TOPK, SELECT_HASH = 0, 1
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
DEVERR_EXPERT_ID, DEVERR_TOKEN_ID, DEVERR_TABLE, DEVERR_Y_RANGE = 1, 2, 4, 8
MAX_EXPERTS, MAX_TOP_K = 1024, 32


class MoeFp4Weight(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("packed", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p),
                ("experts", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32)]


class MoeExpertWeights(ctypes.Structure):
    _fields_ = [("gate", MoeFp4Weight), ("up", MoeFp4Weight), ("down", MoeFp4Weight)]


class MoeConfig(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("score_mode", ctypes.c_int32),
                ("select_mode", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("has_shared", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("pre_norm", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("vocab", ctypes.c_int64),
                ("path", ctypes.c_int32), ("zero_experts", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t

EXPORTS = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_workspace_size": (ctypes.c_int, [ctypes.POINTER(MoeConfig), ctypes.POINTER(_SZ)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(MoeConfig)] + [_P] * 10 + [_P, _SZ, _P]),
    "moe_experts_forward": (ctypes.c_int, [ctypes.POINTER(MoeConfig), _P, _P, _P,
                                           ctypes.POINTER(MoeExpertWeights),
                                           ctypes.POINTER(MoeExpertWeights), _P, _P, _P, _SZ, _P]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(MoeConfig)] + [_P] * 7 +
                          [ctypes.POINTER(MoeExpertWeights), ctypes.POINTER(MoeExpertWeights)] +
                          [_P] * 5 + [_P, _SZ, _P]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(MoeConfig)] + [_P] * 7 +
                                  [ctypes.POINTER(MoeExpertWeights),
                                   ctypes.POINTER(MoeExpertWeights)] + [_P] * 5 + [_P]),
    "moe_debug_dequant_fp4": (ctypes.c_int, [ctypes.POINTER(MoeFp4Weight), ctypes.c_int32,
                                             ctypes.c_int32, _P, _P]),
    "moe_get_device_error": (ctypes.c_int, [_P, _SZ, ctypes.POINTER(ctypes.c_int32), _P]),
    "moe_set_stage_events": (ctypes.c_int, [_P, ctypes.c_int32]),
    "moe_probe_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "moe_probe_mfma_blocks": (ctypes.c_int, [ctypes.c_int32]),
    "moe_probe_mfma": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
}
PROBE_READ_BLOCKS = 2048

STAGE_COUNT = 7
STAGE_NAMES = ["begin", "routed", "dispatched", "gate_up", "down", "shared", "combined"]


def load_library(path: str = LIB_PATH):
    """Load the HIP library (once). Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with mixture_experts_ffn_03_amd/build.py "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(tokens, hidden, num_experts, top_k, inter, score_mode=SCORE_SOFTMAX,
                select_mode=SELECT_TOPK, renormalize=False, routed_scaling=1.0,
                has_shared=False, shared_inter=0, pre_norm=False, norm_eps=1e-6, vocab=0,
                path=PATH_AUTO, zero_experts=0) -> MoeConfig:
    return MoeConfig(tokens, hidden, num_experts, top_k, inter, score_mode, select_mode,
                     int(bool(renormalize)), float(routed_scaling), int(bool(has_shared)),
                     shared_inter, int(bool(pre_norm)), float(norm_eps), int(vocab), path,
                     int(zero_experts))


def fp4_weight(w) -> MoeFp4Weight:
    """Marshal an object with fmt, packed ([E,N,K/2] FP4, [E,N,K] FP8 or BF16), scales (or
    None for BF16), global_scale, n, k."""
    return MoeFp4Weight(w.fmt, _ptr(w.packed), _ptr(w.scales),
                        _ptr(w.global_scale) if w.global_scale is not None else None,
                        w.packed.shape[0], w.n, w.k)


def expert_weights(ws) -> MoeExpertWeights:
    """Marshal an object with gate, up, down projections (see fp4_weight)."""
    return MoeExpertWeights(fp4_weight(ws.gate), fp4_weight(ws.up), fp4_weight(ws.down))


def workspace_size(cfg: MoeConfig) -> int:
    n = _SZ(0)
    _check(load_library().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_size(cfg), dtype=torch.uint8, device=device)


def route(cfg, x, router_w, ids, w, workspace, logit_bias=None, correction_bias=None,
          token_ids=None, tid2eid=None, logits_in=None, logits_out=None, stream=None):
    _check(load_library().moe_route(
        ctypes.byref(cfg), _ptr(x), _ptr(router_w), _ptr(logit_bias), _ptr(correction_bias),
        _ptr(token_ids), _ptr(tid2eid), _ptr(logits_in), _ptr(logits_out), _ptr(ids), _ptr(w),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_route")


def experts_forward(cfg, x_experts, ids, w, routed: MoeExpertWeights,
                    shared: Optional[MoeExpertWeights], residual, out, workspace, stream=None):
    _check(load_library().moe_experts_forward(
        ctypes.byref(cfg), _ptr(x_experts), _ptr(ids), _ptr(w), ctypes.byref(routed),
        ctypes.byref(shared) if shared is not None else None, _ptr(residual), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(stream)), "moe_experts_forward")


def layer_forward(cfg, x, router_w, routed: MoeExpertWeights, out, workspace, *,
                  norm_gamma=None, logit_bias=None, correction_bias=None, token_ids=None,
                  tid2eid=None, shared: Optional[MoeExpertWeights] = None, residual=None,
                  dbg_logits=None, dbg_ids=None, dbg_w=None, stream=None):
    _check(load_library().moe_layer_forward(
        ctypes.byref(cfg), _ptr(x), _ptr(norm_gamma), _ptr(router_w), _ptr(logit_bias),
        _ptr(correction_bias), _ptr(token_ids), _ptr(tid2eid), ctypes.byref(routed),
        ctypes.byref(shared) if shared is not None else None, _ptr(residual), _ptr(out),
        _ptr(dbg_logits), _ptr(dbg_ids), _ptr(dbg_w), _ptr(workspace), workspace.numel(),
        _stream(stream)), "moe_layer_forward")


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def layer_forward_noalloc(cfg, x, router_w, routed: MoeExpertWeights, out, *,
                          norm_gamma=None, logit_bias=None, correction_bias=None,
                          token_ids=None, tid2eid=None, shared: Optional[MoeExpertWeights] = None,
                          residual=None, dbg_logits=None, dbg_ids=None, dbg_w=None, stream=None):
    """moe_layer_forward on the library's own fixed scratch array (no workspace argument)."""
    _check(load_library().moe_layer_forward_noalloc(
        ctypes.byref(cfg), _ptr(x), _ptr(norm_gamma), _ptr(router_w), _ptr(logit_bias),
        _ptr(correction_bias), _ptr(token_ids), _ptr(tid2eid), ctypes.byref(routed),
        ctypes.byref(shared) if shared is not None else None, _ptr(residual), _ptr(out),
        _ptr(dbg_logits), _ptr(dbg_ids), _ptr(dbg_w), _stream(stream)),
        "moe_layer_forward_noalloc")


def debug_dequant(weight: MoeFp4Weight, expert: int, path: int, out: torch.Tensor, stream=None):
    _check(load_library().moe_debug_dequant_fp4(ctypes.byref(weight), expert, path, _ptr(out),
                                                _stream(stream)), "moe_debug_dequant_fp4")


def get_device_error(workspace: torch.Tensor, stream=None) -> int:
    v = ctypes.c_int32(0)
    _check(load_library().moe_get_device_error(_ptr(workspace), workspace.numel(),
                                               ctypes.byref(v), _stream(stream)),
           "moe_get_device_error")
    return v.value


def set_stage_events(events_array, count: int):
    """Ask the next layer_forward on this thread to record the given HIP events
    (a ctypes array of hipEvent_t handles) at its stage boundaries."""
    _check(load_library().moe_set_stage_events(
        ctypes.cast(events_array, ctypes.c_void_p) if events_array is not None else None, count),
        "moe_set_stage_events")


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Enqueue the streaming-read probe over all of `src` (bytes a multiple of 16);
    `sink`: PROBE_READ_BLOCKS float32."""
    _check(load_library().moe_probe_stream_read(_ptr(src), src.numel() * src.element_size(),
                                                _ptr(sink), _stream(stream)),
           "moe_probe_stream_read")


def probe_mfma_blocks(blocks_per_cu: int) -> int:
    n = load_library().moe_probe_mfma_blocks(blocks_per_cu)
    if n < 0:
        raise MoeError(n, "moe_probe_mfma_blocks")
    return n


def probe_mfma(kind: int, iters: int, blocks_per_cu: int, sink: torch.Tensor,
               cycles: torch.Tensor, stream=None):
    """Enqueue the MFMA-rate probe (kind 0 bf16, 1 scaled FP4 x FP8, 2 MXFP4 decode + bf16);
    `sink` float32 and `cycles` int64, probe_mfma_blocks(blocks_per_cu) entries each."""
    _check(load_library().moe_probe_mfma(kind, iters, blocks_per_cu, _ptr(sink), _ptr(cycles),
                                         _stream(stream)), "moe_probe_mfma")
