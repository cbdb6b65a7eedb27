"""Python binding of the gfx950 MoE-FP4 C ABI (``include/moe_fp4.h``).

Argument marshalling only: every step of the layer runs in the HIP library
``libmoefp4.so``; torch provides device memory and the current stream.  If the
library is missing the import fails loudly -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch  # loads the HIP runtime first, so the library binds to the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoefp4.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, 1, 2, 3, 4
MOE_FP4_MX, MOE_FP4_NV, MOE_FP4_MXC = 0, 1, 2
MOE_FP4_SCALES_POW2, MOE_FP4_TILED, MOE_FP4_MX_EXACT = 1, 2, 4
MOE_ACT_BF16, MOE_ACT_NVFP4, MOE_ACT_MXFP8, MOE_ACT_NVFP4_PLANES = 0, 1, 2, 3
MOE_OUT_NVFP4, MOE_OUT_MXFP8, MOE_OUT_NVFP4_PLANES = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SWIGLU = 0, 1
MOE_ALGO_AUTO, MOE_ALGO_DECODE, MOE_ALGO_PREFILL = 0, 1, 2

EXPORTS = ("moe_status_string", "moe_last_error", "moe_version", "moe_route", "moe_permute_workspace_bytes",
           "moe_permute", "moe_route_permute", "moe_fp4_grouped_gemm", "moe_combine", "fp4_transcode_mx_to_nv", "moe_quantize_nvfp4",
           "moe_fp4_tile_weights", "moe_route_permute_noalloc", "moe_quantize_mxfp8", "moe_quantize_nvfp4_planes",
           "moe_route_gemv_workspace_bytes", "moe_route_gemv", "moe_reap_saliency_accumulate", "moe_fp4_compact_mx")


class RouteParams(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("routed_scaling_factor", ctypes.c_float),
                ("norm_topk_prob", ctypes.c_int32)]


class Fp4Weights(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("packed", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("flags", ctypes.c_int32)]


class Act(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("input_scale", ctypes.c_float), ("gather", ctypes.c_void_p), ("gather_div", ctypes.c_int32),
                ("rows_src", ctypes.c_int64)]


class Out(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("output_scale", ctypes.c_float), ("dequant", ctypes.c_void_p), ("format", ctypes.c_int32),
                ("row_sumsq", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python block_scaled_fp4_group_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [i32]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_route.restype = i32
    lib.moe_route.argtypes = [vp, vp, i64, ctypes.POINTER(RouteParams), vp, vp, vp]
    lib.moe_permute_workspace_bytes.restype = sz
    lib.moe_permute_workspace_bytes.argtypes = [i64, i32, i32]
    lib.moe_permute.restype = i32
    lib.moe_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.moe_route_permute.restype = i32
    lib.moe_route_permute.argtypes = [vp, vp, i64, ctypes.POINTER(RouteParams), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_fp4_grouped_gemm.restype = i32
    lib.moe_fp4_grouped_gemm.argtypes = [ctypes.POINTER(Act), ctypes.POINTER(Fp4Weights), ctypes.POINTER(Fp4Weights),
                                         i32, vp, i64, ctypes.POINTER(Out), i32, vp]
    lib.moe_combine.restype = i32
    lib.moe_combine.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, vp]
    lib.fp4_transcode_mx_to_nv.restype = i32
    lib.fp4_transcode_mx_to_nv.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp]
    lib.moe_quantize_nvfp4.restype = i32
    lib.moe_quantize_nvfp4.argtypes = [vp, i64, i32, f32, vp, vp, vp, vp]
    lib.moe_route_permute_noalloc.restype = i32
    lib.moe_route_permute_noalloc.argtypes = [vp, vp, i64, ctypes.POINTER(RouteParams), vp, vp, vp, vp, vp, vp]
    lib.moe_route_gemv_workspace_bytes.restype = sz
    lib.moe_route_gemv_workspace_bytes.argtypes = [i64, i32]
    lib.moe_route_gemv.restype = i32
    lib.moe_route_gemv.argtypes = [vp, vp, vp, i64, i32, ctypes.POINTER(RouteParams), vp, vp, vp, sz, vp]
    lib.moe_reap_saliency_accumulate.restype = i32
    lib.moe_reap_saliency_accumulate.argtypes = [vp, i64, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.moe_fp4_compact_mx.restype = i32
    lib.moe_fp4_compact_mx.argtypes = [vp, vp, i64, i32, i32, vp, vp, vp, vp]
    lib.moe_quantize_mxfp8.restype = i32
    lib.moe_quantize_mxfp8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.moe_quantize_nvfp4_planes.restype = i32
    lib.moe_quantize_nvfp4_planes.argtypes = [vp, i64, i32, f32, vp, vp, vp]
    lib.moe_fp4_tile_weights.restype = i32
    lib.moe_fp4_tile_weights.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    return lib


lib = _load()


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib.moe_last_error().decode() or lib.moe_status_string(status).decode()
        super().__init__(f"{what}: status {status} ({lib.moe_status_string(status).decode()}): {msg}")


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# --------------------------------------------------------------------- calls
def route(logits: torch.Tensor, bias: Optional[torch.Tensor], num_experts: int, n_group: int, topk_group: int,
          top_k: int, routed_scaling_factor: float, norm_topk_prob: bool = True, ids=None, weights=None, stream=None):
    _dev(logits, "logits")
    T = logits.shape[0]
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device) if ids is None else ids
    weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device) if weights is None else weights
    p = RouteParams(num_experts, n_group, topk_group, top_k, routed_scaling_factor, int(norm_topk_prob))
    _check(lib.moe_route(_ptr(logits), _ptr(bias), T, ctypes.byref(p), _ptr(ids), _ptr(weights), _stream(stream)),
           "moe_route")
    return ids, weights


def route_gemv_workspace_bytes(T: int, num_experts: int) -> int:
    return int(lib.moe_route_gemv_workspace_bytes(T, num_experts))


def route_gemv(x: torch.Tensor, gate_weight: torch.Tensor, bias: Optional[torch.Tensor], num_experts: int,
               n_group: int, topk_group: int, top_k: int, routed_scaling_factor: float, workspace: torch.Tensor,
               norm_topk_prob: bool = True, ids=None, weights=None, stream=None):
    """Router matmul (bf16 x, FP32 gate_weight [E, hidden], float64 sums), then
    the group top-k on its logits.  ``workspace``: uint8 of at least
    route_gemv_workspace_bytes(T, E); after the call its first T*E*8 bytes hold
    the float64 logits."""
    _dev(x, "x")
    _dev(gate_weight, "gate_weight")
    T, H = x.shape
    ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device) if ids is None else ids
    weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device) if weights is None else weights
    p = RouteParams(num_experts, n_group, topk_group, top_k, routed_scaling_factor, int(norm_topk_prob))
    _check(lib.moe_route_gemv(_ptr(x), _ptr(gate_weight), _ptr(bias), T, H, ctypes.byref(p), _ptr(ids), _ptr(weights),
                              _ptr(workspace), workspace.numel(), _stream(stream)), "moe_route_gemv")
    return ids, weights


def permute_workspace_bytes(T: int, top_k: int, num_experts: int) -> int:
    return int(lib.moe_permute_workspace_bytes(T, top_k, num_experts))


def permute(ids: torch.Tensor, num_experts: int, workspace: Optional[torch.Tensor] = None, offsets=None,
            sorted_slots=None, slot_rows=None, stream=None):
    _dev(ids, "ids")
    T, top_k = ids.shape
    dev = ids.device
    R = T * top_k
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_slots = torch.empty(R, dtype=torch.int32, device=dev) if sorted_slots is None else sorted_slots
    slot_rows = torch.empty(R, dtype=torch.int32, device=dev) if slot_rows is None else slot_rows
    if workspace is None:
        workspace = torch.empty(max(permute_workspace_bytes(T, top_k, num_experts), 16), dtype=torch.uint8, device=dev)
    _check(lib.moe_permute(_ptr(ids), T, top_k, num_experts, _ptr(offsets), _ptr(sorted_slots), _ptr(slot_rows),
                           _ptr(workspace), workspace.numel(), _stream(stream)), "moe_permute")
    return offsets, sorted_slots, slot_rows


def route_permute(logits: torch.Tensor, bias: Optional[torch.Tensor], num_experts: int, n_group: int,
                  topk_group: int, top_k: int, routed_scaling_factor: float, counter: torch.Tensor,
                  norm_topk_prob: bool = True, ids=None, weights=None, workspace: Optional[torch.Tensor] = None,
                  offsets=None, sorted_slots=None, slot_rows=None, stream=None):
    """route() then permute() of its ids, in one launch for up to 2048 slots.
    ``counter``: one int32 on the device, zero before the first call (each call
    leaves it zero); calls sharing it must not overlap."""
    _dev(logits, "logits")
    _dev(counter, "counter")
    if counter.dtype != torch.int32 or counter.numel() < 1:
        raise ValueError("counter must hold one int32")
    T = logits.shape[0]
    dev = logits.device
    R = T * top_k
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if ids is None else ids
    weights = torch.empty((T, top_k), dtype=torch.float32, device=dev) if weights is None else weights
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    sorted_slots = torch.empty(R, dtype=torch.int32, device=dev) if sorted_slots is None else sorted_slots
    slot_rows = torch.empty(R, dtype=torch.int32, device=dev) if slot_rows is None else slot_rows
    if workspace is None:
        workspace = torch.empty(max(permute_workspace_bytes(T, top_k, num_experts), 16), dtype=torch.uint8, device=dev)
    p = RouteParams(num_experts, n_group, topk_group, top_k, routed_scaling_factor, int(norm_topk_prob))
    _check(lib.moe_route_permute(_ptr(logits), _ptr(bias), T, ctypes.byref(p), _ptr(ids), _ptr(weights),
                                 _ptr(offsets), _ptr(sorted_slots), _ptr(slot_rows), _ptr(counter), _ptr(workspace),
                                 workspace.numel(), _stream(stream)), "moe_route_permute")
    return ids, weights, offsets, sorted_slots, slot_rows


def route_permute_noalloc(logits: torch.Tensor, bias: Optional[torch.Tensor], num_experts: int, n_group: int,
                          topk_group: int, top_k: int, routed_scaling_factor: float, ids: torch.Tensor,
                          weights: torch.Tensor, offsets: torch.Tensor, sorted_slots: torch.Tensor,
                          slot_rows: torch.Tensor, norm_topk_prob: bool = True, stream=None):
    """route_permute() into caller-provided outputs, with the library's static
    scratch instead of a counter and workspace (no device allocation)."""
    _dev(logits, "logits")
    T = logits.shape[0]
    p = RouteParams(num_experts, n_group, topk_group, top_k, routed_scaling_factor, int(norm_topk_prob))
    _check(lib.moe_route_permute_noalloc(_ptr(logits), _ptr(bias), T, ctypes.byref(p), _ptr(ids), _ptr(weights),
                                         _ptr(offsets), _ptr(sorted_slots), _ptr(slot_rows), _stream(stream)),
           "moe_route_permute_noalloc")
    return ids, weights, offsets, sorted_slots, slot_rows


@dataclasses.dataclass
class Weights:
    """One stacked expert matrix [E, n, k] in MXFP4, NVFP4 or compact MXFP4 (device tensors)."""
    packed: torch.Tensor                  # u8 [E, n, k/2]
    scale: torch.Tensor                   # u8 [E, n, k/32] (MX) | [E, n, k/16] (NV) | [E, n, k/64] (compact)
    global_scale: Optional[torch.Tensor] = None   # f32 [E] (NV global; compact base 2^b)
    scales_pow2: bool = False             # NV: every scale byte is 0 or a power of two (a transcode)
    tiled: bool = False                   # codes and scales in the tiled layout (see tile_weights)
    mx_exact: bool = False                # NV: an exact MXFP4 transcode (E8M0 per 32 exists)
    compact: bool = False                 # compact MXFP4 (see compact_mx): 4-bit exponent codes + base

    @property
    def format(self):
        if self.compact:
            return MOE_FP4_MXC
        return MOE_FP4_NV if self.global_scale is not None else MOE_FP4_MX

    def c(self) -> Fp4Weights:
        E, n, k2 = self.packed.shape
        return Fp4Weights(self.format, E, n, 2 * k2, self.packed.data_ptr(), self.scale.data_ptr(),
                          None if self.global_scale is None else self.global_scale.data_ptr(),
                          (MOE_FP4_SCALES_POW2 if self.scales_pow2 else 0) | (MOE_FP4_TILED if self.tiled else 0)
                          | (MOE_FP4_MX_EXACT if self.mx_exact else 0))


_ACT_MODES = {"bf16": MOE_ACT_BF16, "nvfp4": MOE_ACT_NVFP4, "mxfp8": MOE_ACT_MXFP8, "planes": MOE_ACT_NVFP4_PLANES}
_OUT_FORMATS = {"nvfp4": MOE_OUT_NVFP4, "mxfp8": MOE_OUT_MXFP8, "planes": MOE_OUT_NVFP4_PLANES}


def grouped_gemm(a: torch.Tensor, w0: Weights, w1: Optional[Weights], offsets: torch.Tensor, rows: int,
                 gather: Optional[torch.Tensor] = None, gather_div: int = 1, a_scales: Optional[torch.Tensor] = None,
                 input_scale: float = 1.0, out: Optional[torch.Tensor] = None, out_codes: Optional[torch.Tensor] = None,
                 out_scales: Optional[torch.Tensor] = None, output_scale: float = 1.0, want_bf16: bool = True,
                 out_dequant: Optional[torch.Tensor] = None, algo: int = MOE_ALGO_AUTO, a_mode: Optional[str] = None,
                 out_format: str = "nvfp4", row_sumsq: Optional[torch.Tensor] = None, stream=None):
    """A: bf16 [rows_src, k] (W4A16); NVFP4 codes u8 [rows_src, k/2] with ``a_scales`` (W4A4);
    ``a_mode="mxfp8"``: E4M3 codes [rows_src, k] + E8M0 [rows_src, k/32] (W4A8);
    ``a_mode="planes"``: NVFP4 planes [rows_src, 2k] + E8M0 [rows_src, k/16] (W4A4, block-scaled MFMA).
    ``out_codes``/``out_scales`` receive the output quantised in ``out_format`` ("nvfp4", "mxfp8",
    "planes"); ``out_dequant``: bf16 [rows, n] receiving an NVFP4 output's values."""
    _dev(a, "a")
    n = w0.packed.shape[1]
    dev = a.device
    if want_bf16 and out is None:
        out = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
    mode = _ACT_MODES[a_mode] if a_mode is not None else (MOE_ACT_NVFP4 if a_scales is not None else MOE_ACT_BF16)
    act = Act(mode, a.data_ptr(), None if a_scales is None else a_scales.data_ptr(), float(input_scale),
              None if gather is None else gather.data_ptr(), int(gather_div), a.shape[0])
    o = Out(None if out is None else out.data_ptr(), None if out_codes is None else out_codes.data_ptr(),
            None if out_scales is None else out_scales.data_ptr(), float(output_scale),
            None if out_dequant is None else out_dequant.data_ptr(), _OUT_FORMATS[out_format],
            None if row_sumsq is None else row_sumsq.data_ptr())
    cw0 = w0.c()
    cw1 = w1.c() if w1 is not None else None
    epi = MOE_EPI_SWIGLU if w1 is not None else MOE_EPI_NONE
    _check(lib.moe_fp4_grouped_gemm(ctypes.byref(act), ctypes.byref(cw0), None if cw1 is None else ctypes.byref(cw1),
                                    epi, _ptr(offsets), rows, ctypes.byref(o), algo, _stream(stream)),
           "moe_fp4_grouped_gemm")
    return out


def combine(expert_out: torch.Tensor, slot_rows: torch.Tensor, topk_weights: torch.Tensor,
            residual: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None, stream=None):
    T, top_k = topk_weights.shape
    h = expert_out.shape[1]
    y = torch.empty((T, h), dtype=torch.bfloat16, device=expert_out.device) if y is None else y
    _check(lib.moe_combine(_ptr(expert_out), _ptr(slot_rows), _ptr(topk_weights), _ptr(residual), T, top_k, h,
                           _ptr(y), _stream(stream)), "moe_combine")
    return y


def transcode_mx_to_nv(mx_scale: torch.Tensor, packed: torch.Tensor, nv=None, g=None, cnt=None, stream=None):
    """mx_scale u8 [M, n, k/32], packed u8 [M, n, k/2] -> (nv_scale, global f32 [M], counters i64 [4])
    (written into ``nv``, ``g``, ``cnt`` when given)."""
    M, n, kb = mx_scale.shape
    k = kb * 32
    dev = mx_scale.device
    nv = torch.empty((M, n, k // 16), dtype=torch.uint8, device=dev) if nv is None else nv
    g = torch.empty(M, dtype=torch.float32, device=dev) if g is None else g
    cnt = torch.empty(4, dtype=torch.int64, device=dev) if cnt is None else cnt
    _check(lib.fp4_transcode_mx_to_nv(_ptr(mx_scale), _ptr(packed), M, n, k, _ptr(nv), _ptr(g), _ptr(cnt),
                                      _stream(stream)), "fp4_transcode_mx_to_nv")
    return nv, g, cnt


def tile_weights(w: Weights, stream=None) -> Weights:
    """Copy of ``w`` in the tiled layout (same values; shapes unchanged, flag MOE_FP4_TILED)."""
    if w.tiled:
        return w
    E, n, k2 = w.packed.shape
    packed = torch.empty_like(w.packed)
    scale = torch.empty_like(w.scale)
    _check(lib.moe_fp4_tile_weights(w.format, E, n, 2 * k2, _ptr(w.packed), _ptr(w.scale), _ptr(packed), _ptr(scale),
                                    _stream(stream)), "moe_fp4_tile_weights")
    return Weights(packed, scale, w.global_scale, w.scales_pow2, tiled=True, mx_exact=w.mx_exact, compact=w.compact)


def compact_mx(mx_scale: torch.Tensor, packed: torch.Tensor, codes=None, base=None, cnt=None, stream=None):
    """mx_scale u8 [M, n, k/32], packed u8 [M, n, k/2] -> (exponent codes u8 [M, n, k/64],
    base f32 [M], counters i64 [4]: blocks, all-zero below the window, re-rounded, NaN)."""
    M, n, kb = mx_scale.shape
    k = kb * 32
    dev = mx_scale.device
    codes = torch.empty((M, n, k // 64), dtype=torch.uint8, device=dev) if codes is None else codes
    base = torch.empty(M, dtype=torch.float32, device=dev) if base is None else base
    cnt = torch.empty(4, dtype=torch.int64, device=dev) if cnt is None else cnt
    _check(lib.moe_fp4_compact_mx(_ptr(mx_scale), _ptr(packed), M, n, k, _ptr(codes), _ptr(base), _ptr(cnt),
                                  _stream(stream)), "moe_fp4_compact_mx")
    return codes, base, cnt


def compact_weights(w: Weights, stream=None):
    """Compact copy of row-major MXFP4 weights (codes shared) -> (Weights, counters i64 [4])."""
    if w.format != MOE_FP4_MX or w.tiled:
        raise ValueError("compact_weights takes row-major MXFP4 weights")
    codes, base, cnt = compact_mx(w.scale, w.packed, stream=stream)
    return Weights(w.packed, codes, base, compact=True), cnt


def quantize_nvfp4(x: torch.Tensor, input_scale: float = 1.0, codes=None, scales=None, dequant=None, stream=None):
    """-> (codes u8 [rows, k/2], scales u8 [rows, k/16]); ``dequant`` (bf16 [rows, k]) optionally
    receives the NVFP4 values themselves."""
    rows, k = x.shape
    codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device) if scales is None else scales
    _check(lib.moe_quantize_nvfp4(_ptr(x), rows, k, float(input_scale), _ptr(codes), _ptr(scales), _ptr(dequant),
                                  _stream(stream)), "moe_quantize_nvfp4")
    return codes, scales


def reap_saliency_accumulate(row_sumsq: torch.Tensor, offsets: torch.Tensor, sorted_slots: torch.Tensor,
                             topk_weights: torch.Tensor, sums: torch.Tensor, counts: torch.Tensor, rows: int,
                             stream=None):
    """sums (float64 [E]) += per-expert sum of g * ||o_row||; counts (int64 [E]) += rows per expert."""
    E = sums.numel()
    _check(lib.moe_reap_saliency_accumulate(_ptr(row_sumsq), rows, row_sumsq.shape[1], _ptr(offsets), E,
                                            _ptr(sorted_slots), _ptr(topk_weights), _ptr(sums), _ptr(counts),
                                            _stream(stream)), "moe_reap_saliency_accumulate")
    return sums, counts


def quantize_mxfp8(x: torch.Tensor, codes=None, scales=None, stream=None):
    """bf16 [rows, k] -> (E4M3 codes u8 [rows, k], E8M0 scales u8 [rows, k/32])."""
    rows, k = x.shape
    codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device) if codes is None else codes
    scales = torch.empty((rows, k // 32), dtype=torch.uint8, device=x.device) if scales is None else scales
    _check(lib.moe_quantize_mxfp8(_ptr(x), rows, k, _ptr(codes), _ptr(scales), _stream(stream)), "moe_quantize_mxfp8")
    return codes, scales


def quantize_nvfp4_planes(x: torch.Tensor, input_scale: float = 1.0, planes=None, scales=None, stream=None):
    """bf16 [rows, k] -> (E4M3 planes u8 [rows, 2k], E8M0 scales u8 [rows, k/16]): the NVFP4
    quantisation of x in the block-scaled MFMA's operand form."""
    rows, k = x.shape
    planes = torch.empty((rows, 2 * k), dtype=torch.uint8, device=x.device) if planes is None else planes
    scales = torch.empty((rows, k // 16), dtype=torch.uint8, device=x.device) if scales is None else scales
    _check(lib.moe_quantize_nvfp4_planes(_ptr(x), rows, k, float(input_scale), _ptr(planes), _ptr(scales),
                                         _stream(stream)), "moe_quantize_nvfp4_planes")
    return planes, scales


from .layer import MoELayer, LayerWeights  # noqa: E402  (composition of the calls above)
