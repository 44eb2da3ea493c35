"""Python binding of libnvfp4kv, the gfx950 NVFP4 paged KV-cache library.

Argument marshalling only: every step of the path runs in the HIP kernels of
libnvfp4kv.so (built in-tree by ``nvfp4_quantized_paged_amd.build``). torch
supplies device memory and the current HIP stream. There is no fallback: if
the library is missing or a call fails, an exception is raised.

torch is imported before the library is loaded: torch ships its own HIP
runtime (soname libamdhip64.so.7), and loading it first makes the library
bind to that same runtime, so torch's stream handles are valid here.

Function names and argument meanings follow include/nvfp4kv.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4kv.so")

OK, EINVAL, EUNSUPPORTED, EALIGN, EWORKSPACE, ELAUNCH = 0, -1, -2, -3, -4, -5
VARIANT_AUTO, VARIANT_VALU, VARIANT_MFMA, VARIANT_MFMA_LUT = 0, 1, 2, 3

c_i32, c_i64, c_f32, c_vp, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class Geom(ctypes.Structure):
    _fields_ = [("num_pages", c_i32), ("page_size", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32)]


class NVFP4CacheDesc(ctypes.Structure):
    _fields_ = [("data", c_vp), ("scale", c_vp), ("global_scale", c_f32)]


class FP8CacheDesc(ctypes.Structure):
    _fields_ = [("data", c_vp), ("scale", c_f32)]


P_GEOM, P_NV, P_F8 = ctypes.POINTER(Geom), ctypes.POINTER(NVFP4CacheDesc), ctypes.POINTER(FP8CacheDesc)

_SIGNATURES = {
    "nvfp4kv_abi_version": (ctypes.c_int, []),
    "nvfp4kv_last_error": (ctypes.c_char_p, []),
    "nvfp4_paged_decode_num_splits": (c_i32, [c_i32, c_i32, c_i32, c_i32]),
    "nvfp4_paged_decode_workspace_bytes": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "nvfp4_kv_quantize": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_i64, c_i32, c_vp, P_NV, P_NV, c_vp]),
    "fp8_kv_quantize": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_i64, c_i32, c_vp, P_F8, P_F8, c_vp]),
    "nvfp4_kv_dequant_workspace": (ctypes.c_int, [P_GEOM, P_NV, P_NV, c_vp, c_i32, c_vp, c_vp, c_i32,
                                                  c_vp, c_vp, c_vp]),
    "nvfp4_paged_decode_attn": (ctypes.c_int, [P_GEOM, c_vp, P_NV, P_NV, c_vp, c_i32, c_vp, c_i32, c_i32,
                                               c_f32, c_i32, c_vp, c_size, c_vp, c_vp]),
    "nvfp4_paged_decode_partial": (ctypes.c_int, [P_GEOM, c_vp, P_NV, P_NV, c_vp, c_i32, c_vp, c_i32, c_i32,
                                                  c_f32, c_i32, c_i32, c_vp, c_size, c_vp]),
    "nvfp4_paged_decode_attn_shared_prefix": (ctypes.c_int, [P_GEOM, c_vp, P_NV, P_NV, c_vp, c_i32, c_vp, c_i32,
                                                             c_i32, c_f32, c_i32, c_i32, c_i32, c_vp, c_size, c_vp,
                                                             c_vp]),
    "nvfp4_paged_decode_shared_prefix_workspace_bytes": (c_size, [P_GEOM, c_i32, c_i32, c_i32, c_i32, c_i32,
                                                                  c_i32]),
    "nvfp4_paged_decode_attn_noalloc": (ctypes.c_int, [P_GEOM, c_vp, P_NV, P_NV, c_vp, c_i32, c_vp, c_i32, c_i32,
                                                       c_f32, c_i32, c_vp, c_vp]),
    "nvfp4_paged_decode_noalloc_scratch_bytes": (c_size, []),
    "fp8_paged_decode_attn": (ctypes.c_int, [P_GEOM, c_vp, P_F8, P_F8, c_vp, c_i32, c_vp, c_i32, c_i32,
                                             c_f32, c_i32, c_vp, c_size, c_vp, c_vp]),
    "nvfp4_paged_decode_append_attn": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_vp, c_i64, P_NV, P_NV, c_vp, c_i32,
                                                      c_vp, c_i32, c_i32, c_f32, c_i32, c_vp, c_size, c_vp,
                                                      c_vp]),
    "fp8_paged_decode_append_attn": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_vp, c_i64, P_F8, P_F8, c_vp, c_i32,
                                                    c_vp, c_i32, c_i32, c_f32, c_i32, c_vp, c_size, c_vp,
                                                    c_vp]),
    "nvfp4_paged_decode_append_partial": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_vp, c_i64, P_NV, P_NV, c_vp, c_i32,
                                                         c_vp, c_i32, c_i32, c_f32, c_i32, c_vp, c_size, c_vp]),
    "fp8_paged_decode_append_partial": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_vp, c_i64, P_F8, P_F8, c_vp, c_i32,
                                                       c_vp, c_i32, c_i32, c_f32, c_i32, c_vp, c_size, c_vp]),
    "fp8_paged_decode_partial": (ctypes.c_int, [P_GEOM, c_vp, P_F8, P_F8, c_vp, c_i32, c_vp, c_i32, c_i32,
                                                c_f32, c_i32, c_i32, c_vp, c_size, c_vp]),
    "nvfp4kv_lse_merge": (ctypes.c_int, [c_vp, c_size, c_i32, c_i32, c_i32, c_i32, c_f32, c_vp, c_vp]),
    "nvfp4_kv_absmax": (ctypes.c_int, [c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "nvfp4_extend_attn": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i32,
                                         c_f32, c_vp, c_vp]),
    "nvfp4_extend_attn_fp8": (ctypes.c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                             c_i32, c_f32, c_f32, c_f32, c_vp, c_vp]),
    "nvfp4_kv_quantize_fp8": (ctypes.c_int, [P_GEOM, c_vp, c_vp, c_i64, c_i32, c_vp, c_f32, c_f32, P_NV, P_NV,
                                             c_vp, c_vp, c_vp, c_vp]),
    "nvfp4_kv_dequant_workspace_fp8": (ctypes.c_int, [P_GEOM, P_NV, P_NV, c_vp, c_i32, c_vp, c_vp, c_i32,
                                                      c_f32, c_f32, c_vp, c_vp, c_vp]),
    "nvfp4_global_scale_from_absmax": (c_f32, [c_f32]),
    "nvfp4kv_hbm_read_probe": (ctypes.c_int, [c_vp, c_i64, c_i32, c_i32, c_vp, c_vp]),
}

_lib_handle = None


class NVFP4KVError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m nvfp4_quantized_paged_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = handle
    return _lib_handle


def last_error() -> str:
    return lib().nvfp4kv_last_error().decode()


def abi_version() -> int:
    return lib().nvfp4kv_abi_version()


def _check(rc: int):
    if rc != OK:
        raise NVFP4KVError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_vp(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# Shape checks. The C ABI receives pointers and the sizes passed beside them;
# it cannot see how large each tensor is. A tensor smaller than those sizes
# imply (fewer V tokens than K tokens, a short slot mapping, a smaller V pool)
# would make a kernel read or write past it, so the binding compares every
# tensor with the sizes it passes. They only inspect shapes, so they work on
# tensors of any device.

def _shape(t: torch.Tensor, shape, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows_of(t: torch.Tensor, g: "Geom", name: str):
    """t must be [rows][Hkv][d] for the pool geometry g."""
    if t.dim() != 3 or tuple(t.shape[1:]) != (g.num_kv_heads, g.head_dim):
        raise ValueError(f"{name} must be [rows][{g.num_kv_heads}][{g.head_dim}], got {tuple(t.shape)}")


def _pool_geom(k_pool, v_pool) -> "Geom":
    gk, gv = k_pool.geom, v_pool.geom
    if (gk.num_pages, gk.page_size, gk.num_kv_heads, gk.head_dim) != \
            (gv.num_pages, gv.page_size, gv.num_kv_heads, gv.head_dim):
        raise ValueError("the K and V pools must have the same geometry")
    return gk


def _check_quantize_shapes(k, v, slot_mapping, k_pool, v_pool) -> "Geom":
    g = _pool_geom(k_pool, v_pool)
    T = k.shape[0] if k.dim() == 3 else -1
    _shape(k, (T, g.num_kv_heads, g.head_dim), "k")
    _shape(v, (T, g.num_kv_heads, g.head_dim), "v")
    _shape(slot_mapping, (T,), "slot_mapping")
    return g


def _check_workspace_shapes(k_pool, v_pool, block_tables, prefix_lens, ws_row_offsets, k_ws, v_ws) -> "Geom":
    g = _pool_geom(k_pool, v_pool)
    if block_tables.dim() != 2:
        raise ValueError(f"block_tables must be [batch][max_pages], got {tuple(block_tables.shape)}")
    B = block_tables.shape[0]
    _shape(prefix_lens, (B,), "prefix_lens")
    _shape(ws_row_offsets, (B + 1,), "ws_row_offsets")
    _rows_of(k_ws, g, "k_ws")
    _shape(v_ws, k_ws.shape, "v_ws")
    return g


def _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens, out=None) -> "Geom":
    g = _pool_geom(k_pool, v_pool)
    if q.dim() != 3 or q.shape[2] != g.head_dim:
        raise ValueError(f"q must be [batch][num_q_heads][{g.head_dim}], got {tuple(q.shape)}")
    B = q.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_pages], got {tuple(block_tables.shape)}")
    _shape(seq_lens, (B,), "seq_lens")
    if out is not None:
        _shape(out, q.shape, "out")
    return g


def _check_extend_shapes(q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, out=None):
    B = prefix_lens.shape[0] if prefix_lens.dim() == 1 else -1
    _shape(prefix_lens, (B,), "prefix_lens")
    _shape(q_row_offsets, (B + 1,), "q_row_offsets")
    _shape(ws_row_offsets, (B + 1,), "ws_row_offsets")
    if q.dim() != 3 or k_ws.dim() != 3 or q.shape[2] != k_ws.shape[2]:
        raise ValueError(f"q [rows][Hq][d] and k_ws [rows][Hkv][d] must share d, got {tuple(q.shape)} and "
                         f"{tuple(k_ws.shape)}")
    _shape(v_ws, k_ws.shape, "v_ws")
    if out is not None:
        _shape(out, q.shape, "out")


# ---------------------------------------------------------------------------
# pools
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class NVFP4Pool:
    """One paged NVFP4 pool (K or V): data [pages][Hkv][P][d/2], scale [pages][Hkv][P][d/16]."""

    data: torch.Tensor
    scale: torch.Tensor
    global_scale: float = 1.0

    @staticmethod
    def empty(num_pages, num_kv_heads, page_size, head_dim, device="cuda", global_scale=1.0):
        return NVFP4Pool(
            torch.empty((num_pages, num_kv_heads, page_size, head_dim // 2), dtype=torch.uint8, device=device),
            torch.empty((num_pages, num_kv_heads, page_size, head_dim // 16), dtype=torch.uint8, device=device),
            global_scale)

    @property
    def geom(self) -> Geom:
        n, h, p, half = self.data.shape
        return Geom(n, p, h, 2 * half)

    def desc(self) -> NVFP4CacheDesc:
        _need(self.data, torch.uint8, "pool data")
        _need(self.scale, torch.uint8, "pool scale")
        _shape(self.scale, tuple(self.data.shape[:3]) + (self.data.shape[3] // 8,), "pool scale")
        return NVFP4CacheDesc(self.data.data_ptr(), self.scale.data_ptr(), self.global_scale)


@dataclasses.dataclass
class FP8Pool:
    """One paged FP8-E4M3 pool: data [pages][Hkv][P][d] uint8, per-tensor scale."""

    data: torch.Tensor
    scale: float = 1.0

    @staticmethod
    def empty(num_pages, num_kv_heads, page_size, head_dim, device="cuda", scale=1.0):
        return FP8Pool(torch.empty((num_pages, num_kv_heads, page_size, head_dim), dtype=torch.uint8,
                                   device=device), scale)

    @property
    def geom(self) -> Geom:
        n, h, p, d = self.data.shape
        return Geom(n, p, h, d)

    def desc(self) -> FP8CacheDesc:
        _need(self.data, torch.uint8, "pool data")
        return FP8CacheDesc(self.data.data_ptr(), self.scale)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def _quantize(fn, k, v, slot_mapping, k_pool, v_pool, stream):
    _need(slot_mapping, torch.int64, "slot_mapping")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError(f"{name} must be a bf16 device tensor")
        if t.dim() != 3:
            raise ValueError(f"{name} must be [T][Hkv][d]")
        if t.shape[0] > 0 and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{name} must be [T][Hkv][d] with dense heads")
    g = _check_quantize_shapes(k, v, slot_mapping, k_pool, v_pool)
    if k.shape[0] == 0:
        stride = g.num_kv_heads * g.head_dim
    else:
        if k.stride(0) != v.stride(0):
            raise ValueError("k and v must share a token stride")
        stride = k.stride(0)
    _check(fn(ctypes.byref(g), k.data_ptr(), v.data_ptr(), stride, k.shape[0],
              slot_mapping.data_ptr(), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
              _stream(stream)))


def nvfp4_kv_quantize(k, v, slot_mapping, k_pool: NVFP4Pool, v_pool: NVFP4Pool, stream=None):
    """Quantize-on-write of k, v [T][Hkv][d] (bf16) into the pools at slot_mapping [T] (int64)."""
    _quantize(lib().nvfp4_kv_quantize, k, v, slot_mapping, k_pool, v_pool, stream)


def fp8_kv_quantize(k, v, slot_mapping, k_pool: FP8Pool, v_pool: FP8Pool, stream=None):
    _quantize(lib().fp8_kv_quantize, k, v, slot_mapping, k_pool, v_pool, stream)


PROBE_NONTEMPORAL, PROBE_RANGE = 1, 2


def hbm_read_probe(buf, blocks, flags=PROBE_NONTEMPORAL, sink=None, stream=None):
    """Stream-read every byte of buf (a 16-byte aligned device tensor whose size is a multiple of 16)
    with the library's read-bandwidth kernel (a measurement utility); flags: PROBE_NONTEMPORAL,
    PROBE_RANGE (one contiguous range per workgroup)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check(lib().nvfp4kv_hbm_read_probe(buf.data_ptr(), nbytes, int(blocks), int(flags), sink.data_ptr(),
                                        _stream(stream)))
    return sink


def nvfp4_kv_absmax(x, amax, stream=None):
    """Fold max |x| of x [T][Hkv][d] (bf16, dense heads) into amax (float32 device tensor of
    one element, caller-initialised, >= 0)."""
    _need(amax, torch.float32, "amax")
    if amax.numel() != 1:
        raise ValueError("amax must hold one float")
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 3:
        raise TypeError("x must be a bf16 device tensor [T][Hkv][d]")
    if x.shape[0] > 0 and (x.stride(2) != 1 or x.stride(1) != x.shape[2]):
        raise ValueError("x must be [T][Hkv][d] with dense heads")
    stride = x.stride(0) if x.shape[0] > 0 else x.shape[1] * x.shape[2]
    _check(lib().nvfp4_kv_absmax(x.data_ptr(), stride, x.shape[0], x.shape[1], x.shape[2], amax.data_ptr(),
                                 _stream(stream)))


def nvfp4_extend_attn(q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, sm_scale, max_chunk=None,
                      out=None, stream=None):
    """Extend attention of chunk queries q [rows][Hq][d] (bf16) over workspaces k_ws, v_ws ([rows][Hkv][d] bf16):
    sequence b's queries are rows q_row_offsets[b].. (int64 [B+1]); its keys are workspace rows
    ws_row_offsets[b] + j, j < prefix_lens[b] + chunk_b, attended causally. Returns out."""
    _need(q, torch.bfloat16, "q")
    _need(k_ws, torch.bfloat16, "k_ws")
    _need(v_ws, torch.bfloat16, "v_ws")
    _need(q_row_offsets, torch.int64, "q_row_offsets")
    _need(ws_row_offsets, torch.int64, "ws_row_offsets")
    _need(prefix_lens, torch.int32, "prefix_lens")
    _check_extend_shapes(q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, out)
    if max_chunk is None:
        max_chunk = int((q_row_offsets[1:] - q_row_offsets[:-1]).max().item()) if prefix_lens.numel() else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out")
    _check(lib().nvfp4_extend_attn(q.data_ptr(), q_row_offsets.data_ptr(), k_ws.data_ptr(), v_ws.data_ptr(),
                                   ws_row_offsets.data_ptr(), prefix_lens.data_ptr(), prefix_lens.shape[0],
                                   q.shape[1], k_ws.shape[1], q.shape[2], int(max_chunk), float(sm_scale),
                                   out.data_ptr(), _stream(stream)))
    return out


def nvfp4_extend_attn_fp8(q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, sm_scale, k_scale=1.0,
                          v_scale=1.0, max_chunk=None, out=None, stream=None):
    """nvfp4_extend_attn over the FP8-E4M3 workspaces k_ws, v_ws ([rows][Hkv][d] uint8 bytes) with per-tensor
    scales: key t is e4m3(k_ws[t]) * k_scale, value t is e4m3(v_ws[t]) * v_scale. Returns out (bf16)."""
    _need(q, torch.bfloat16, "q")
    _need(k_ws, torch.uint8, "k_ws")
    _need(v_ws, torch.uint8, "v_ws")
    _need(q_row_offsets, torch.int64, "q_row_offsets")
    _need(ws_row_offsets, torch.int64, "ws_row_offsets")
    _need(prefix_lens, torch.int32, "prefix_lens")
    _check_extend_shapes(q, q_row_offsets, k_ws, v_ws, ws_row_offsets, prefix_lens, out)
    if max_chunk is None:
        max_chunk = int((q_row_offsets[1:] - q_row_offsets[:-1]).max().item()) if prefix_lens.numel() else 0
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out")
    _check(lib().nvfp4_extend_attn_fp8(q.data_ptr(), q_row_offsets.data_ptr(), k_ws.data_ptr(), v_ws.data_ptr(),
                                       ws_row_offsets.data_ptr(), prefix_lens.data_ptr(), prefix_lens.shape[0],
                                       q.shape[1], k_ws.shape[1], q.shape[2], int(max_chunk), float(sm_scale),
                                       float(k_scale), float(v_scale), out.data_ptr(), _stream(stream)))
    return out


def nvfp4_global_scale_from_absmax(amax: float) -> float:
    """amax / (448 * 6) in FP32 (1.0 for amax 0, negative or non-finite)."""
    return float(lib().nvfp4_global_scale_from_absmax(float(amax)))


def nvfp4_kv_quantize_fp8(k, v, slot_mapping, k_pool: NVFP4Pool, v_pool: NVFP4Pool, k_src_scale=1.0,
                          v_src_scale=1.0, ws_rows=None, k_ws=None, v_ws=None, stream=None):
    """Quantize-on-write from FP8-E4M3 k, v [T][Hkv][d] (uint8 bytes) into the NVFP4 pools; with ws_rows
    ([T] int64) the source bytes are also copied to those rows of k_ws, v_ws ([rows][Hkv][d] uint8)."""
    _need(slot_mapping, torch.int64, "slot_mapping")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 3:
            raise TypeError(f"{name} must be a uint8 (FP8-E4M3) device tensor [T][Hkv][d]")
        if t.shape[0] > 0 and (t.stride(2) != 1 or t.stride(1) != t.shape[2]):
            raise ValueError(f"{name} must be [T][Hkv][d] with dense heads")
    g = _check_quantize_shapes(k, v, slot_mapping, k_pool, v_pool)
    if k.shape[0] > 0 and k.stride(0) != v.stride(0):
        raise ValueError("k and v must share a token stride")
    stride = k.stride(0) if k.shape[0] > 0 else g.num_kv_heads * g.head_dim
    if ws_rows is not None:
        _need(ws_rows, torch.int64, "ws_rows")
        _need(k_ws, torch.uint8, "k_ws")
        _need(v_ws, torch.uint8, "v_ws")
        _shape(ws_rows, (k.shape[0],), "ws_rows")
        _rows_of(k_ws, g, "k_ws")
        _shape(v_ws, k_ws.shape, "v_ws")
    _check(lib().nvfp4_kv_quantize_fp8(
        ctypes.byref(g), k.data_ptr(), v.data_ptr(), stride, k.shape[0], slot_mapping.data_ptr(),
        float(k_src_scale), float(v_src_scale), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
        _ptr(ws_rows), _ptr(k_ws), _ptr(v_ws), _stream(stream)))


def nvfp4_kv_dequant_workspace_fp8(k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, prefix_lens,
                                   ws_row_offsets, k_ws, v_ws, k_ws_scale=1.0, v_ws_scale=1.0, stream=None):
    """As nvfp4_kv_dequant_workspace, into FP8-E4M3 workspaces ([rows][Hkv][d] uint8)."""
    _need(block_tables, torch.int32, "block_tables")
    _need(prefix_lens, torch.int32, "prefix_lens")
    _need(ws_row_offsets, torch.int64, "ws_row_offsets")
    _need(k_ws, torch.uint8, "k_ws")
    _need(v_ws, torch.uint8, "v_ws")
    g = _check_workspace_shapes(k_pool, v_pool, block_tables, prefix_lens, ws_row_offsets, k_ws, v_ws)
    _check(lib().nvfp4_kv_dequant_workspace_fp8(
        ctypes.byref(g), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()), block_tables.data_ptr(),
        block_tables.shape[1], prefix_lens.data_ptr(), ws_row_offsets.data_ptr(), prefix_lens.shape[0],
        float(k_ws_scale), float(v_ws_scale), k_ws.data_ptr(), v_ws.data_ptr(), _stream(stream)))


def nvfp4_kv_dequant_workspace(k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, prefix_lens,
                               ws_row_offsets, k_ws, v_ws, stream=None):
    """Dequantize prefixes [0, prefix_lens[b]) into rows ws_row_offsets[b].. of k_ws, v_ws ([rows][Hkv][d] bf16)."""
    _need(block_tables, torch.int32, "block_tables")
    _need(prefix_lens, torch.int32, "prefix_lens")
    _need(ws_row_offsets, torch.int64, "ws_row_offsets")
    _need(k_ws, torch.bfloat16, "k_ws")
    _need(v_ws, torch.bfloat16, "v_ws")
    g = _check_workspace_shapes(k_pool, v_pool, block_tables, prefix_lens, ws_row_offsets, k_ws, v_ws)
    _check(lib().nvfp4_kv_dequant_workspace(
        ctypes.byref(g), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()), block_tables.data_ptr(),
        block_tables.shape[1], prefix_lens.data_ptr(), ws_row_offsets.data_ptr(), prefix_lens.shape[0],
        k_ws.data_ptr(), v_ws.data_ptr(), _stream(stream)))


def nvfp4_paged_decode_num_splits(batch, num_kv_heads, max_pages_per_seq, page_size) -> int:
    return lib().nvfp4_paged_decode_num_splits(batch, num_kv_heads, max_pages_per_seq, page_size)


def nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits) -> int:
    return lib().nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits)


def decode_workspace(batch, num_q_heads, head_dim, num_splits, device="cuda") -> torch.Tensor:
    n = nvfp4_paged_decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _decode_args(q, block_tables, seq_lens):
    _need(q, torch.bfloat16, "q")
    _need(block_tables, torch.int32, "block_tables")
    _need(seq_lens, torch.int32, "seq_lens")
    if q.dim() != 3:
        raise ValueError(f"q must be [batch][num_q_heads][head_dim], got {tuple(q.shape)}")
    B, Hq, d = q.shape
    return B, Hq, d


def _resolve_splits(num_splits, B, pool_geom, max_pages):
    if num_splits == 0:
        return nvfp4_paged_decode_num_splits(B, pool_geom.num_kv_heads, max_pages, pool_geom.page_size)
    return num_splits


def _decode(fn_name, pool_cls_desc, q, k_pool, v_pool, block_tables, seq_lens, sm_scale, num_splits,
            workspace, out, stream):
    B, Hq, d = _decode_args(q, block_tables, seq_lens)
    g = _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens, out)
    splits = _resolve_splits(num_splits, B, g, block_tables.shape[1])
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, splits, q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out")
    _check(getattr(lib(), fn_name)(
        ctypes.byref(g), q.data_ptr(), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
        block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), B, Hq, float(sm_scale),
        splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(), out.data_ptr(),
        _stream(stream)))
    return out


def _partial(fn_name, q, k_pool, v_pool, block_tables, seq_lens, sm_scale, num_splits, variant, workspace,
             stream):
    B, Hq, d = _decode_args(q, block_tables, seq_lens)
    g = _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens)
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, num_splits, q.device)
    _check(getattr(lib(), fn_name)(
        ctypes.byref(g), q.data_ptr(), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
        block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), B, Hq, float(sm_scale),
        num_splits, variant, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return workspace


def nvfp4_paged_decode_attn(q, k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, seq_lens, sm_scale,
                            num_splits=0, workspace=None, out=None, stream=None):
    """Decode attention of q [B][Hq][d] (bf16) over the NVFP4 pools; returns out [B][Hq][d] bf16."""
    return _decode("nvfp4_paged_decode_attn", None, q, k_pool, v_pool, block_tables, seq_lens, sm_scale,
                   num_splits, workspace, out, stream)


def nvfp4_paged_decode_shared_prefix_workspace_bytes(k_pool: NVFP4Pool, max_pages_per_seq, batch, num_q_heads,
                                                     shared_len, prefix_splits=0, num_splits=0) -> int:
    g = k_pool.geom
    return int(lib().nvfp4_paged_decode_shared_prefix_workspace_bytes(ctypes.byref(g), max_pages_per_seq, batch,
                                                                      num_q_heads, shared_len, prefix_splits,
                                                                      num_splits))


def nvfp4_paged_decode_attn_shared_prefix(q, k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, seq_lens, sm_scale,
                                          shared_len, prefix_splits=0, num_splits=0, workspace=None, out=None,
                                          stream=None):
    """nvfp4_paged_decode_attn for a batch whose first shared_len tokens sit on the same pages in
    every block-table row; the prefix is unpacked once per 16 query columns. Returns out [B][Hq][d]."""
    B, Hq, d = _decode_args(q, block_tables, seq_lens)
    g = _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens, out)
    if workspace is None:
        n = nvfp4_paged_decode_shared_prefix_workspace_bytes(k_pool, block_tables.shape[1], B, Hq, shared_len,
                                                             prefix_splits, num_splits)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out")
    _check(lib().nvfp4_paged_decode_attn_shared_prefix(
        ctypes.byref(g), q.data_ptr(), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
        block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), B, Hq, float(sm_scale),
        int(shared_len), int(prefix_splits), int(num_splits), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), out.data_ptr(), _stream(stream)))
    return out


def nvfp4_paged_decode_attn_noalloc(q, k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, seq_lens, sm_scale,
                                    out, num_splits=0, stream=None):
    """nvfp4_paged_decode_attn with the partials in the library's static scratch
    array: no workspace, and no allocation by the binding either (out is
    required)."""
    B, Hq, d = _decode_args(q, block_tables, seq_lens)
    g = _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens, out)
    _need(out, torch.bfloat16, "out")
    _check(lib().nvfp4_paged_decode_attn_noalloc(
        ctypes.byref(g), q.data_ptr(), ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()),
        block_tables.data_ptr(), block_tables.shape[1], seq_lens.data_ptr(), B, Hq, float(sm_scale),
        int(num_splits), out.data_ptr(), _stream(stream)))
    return out


def nvfp4_paged_decode_noalloc_scratch_bytes() -> int:
    return int(lib().nvfp4_paged_decode_noalloc_scratch_bytes())


def fp8_paged_decode_attn(q, k_pool: FP8Pool, v_pool: FP8Pool, block_tables, seq_lens, sm_scale,
                          num_splits=0, workspace=None, out=None, stream=None):
    return _decode("fp8_paged_decode_attn", None, q, k_pool, v_pool, block_tables, seq_lens, sm_scale,
                   num_splits, workspace, out, stream)


def _append_decode(fn_name, q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, sm_scale, num_splits,
                   workspace, out, stream, merge=True):
    B, Hq, d = _decode_args(q, block_tables, seq_lens)
    g = _check_decode_shapes(q, k_pool, v_pool, block_tables, seq_lens, out if merge else None)
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, torch.bfloat16, name)
        if t.dim() != 3 or tuple(t.shape[1:]) != (g.num_kv_heads, d) or t.shape[0] != B:
            raise ValueError(f"{name} must be [batch][num_kv_heads][head_dim] = [{B}][{g.num_kv_heads}][{d}], "
                             f"got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError(f"{name}: the heads of a row must be contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must have the same row stride")
    splits = _resolve_splits(num_splits, B, g, block_tables.shape[1]) if merge else num_splits
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, splits, q.device)
    args = [ctypes.byref(g), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), int(k_new.stride(0)),
            ctypes.byref(k_pool.desc()), ctypes.byref(v_pool.desc()), block_tables.data_ptr(),
            block_tables.shape[1], seq_lens.data_ptr(), B, Hq, float(sm_scale), splits, workspace.data_ptr(),
            workspace.numel() * workspace.element_size()]
    if not merge:
        _check(getattr(lib(), fn_name)(*args, _stream(stream)))
        return workspace
    if out is None:
        out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out")
    _check(getattr(lib(), fn_name)(*args, out.data_ptr(), _stream(stream)))
    return out


def nvfp4_paged_decode_append_attn(q, k_new, v_new, k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables, seq_lens,
                                   sm_scale, num_splits=0, workspace=None, out=None, stream=None):
    """One decode step with each sequence's new token (k_new, v_new: [B][Hkv][d] bf16, at position
    seq_lens[b] - 1) quantized into its pool slot by the decode kernel itself; the same pool bytes
    and output as nvfp4_kv_quantize into those slots followed by nvfp4_paged_decode_attn."""
    return _append_decode("nvfp4_paged_decode_append_attn", q, k_new, v_new, k_pool, v_pool, block_tables,
                          seq_lens, sm_scale, num_splits, workspace, out, stream)


def fp8_paged_decode_append_attn(q, k_new, v_new, k_pool: FP8Pool, v_pool: FP8Pool, block_tables, seq_lens,
                                 sm_scale, num_splits=0, workspace=None, out=None, stream=None):
    return _append_decode("fp8_paged_decode_append_attn", q, k_new, v_new, k_pool, v_pool, block_tables,
                          seq_lens, sm_scale, num_splits, workspace, out, stream)


def nvfp4_paged_decode_append_partial(q, k_new, v_new, k_pool: NVFP4Pool, v_pool: NVFP4Pool, block_tables,
                                      seq_lens, sm_scale, num_splits, workspace=None, stream=None):
    """nvfp4_paged_decode_append_attn without the merge: appends the new tokens and returns the
    workspace holding the partials (as nvfp4_paged_decode_partial lays them out)."""
    return _append_decode("nvfp4_paged_decode_append_partial", q, k_new, v_new, k_pool, v_pool, block_tables,
                          seq_lens, sm_scale, num_splits, workspace, None, stream, merge=False)


def fp8_paged_decode_append_partial(q, k_new, v_new, k_pool: FP8Pool, v_pool: FP8Pool, block_tables, seq_lens,
                                    sm_scale, num_splits, workspace=None, stream=None):
    return _append_decode("fp8_paged_decode_append_partial", q, k_new, v_new, k_pool, v_pool, block_tables,
                          seq_lens, sm_scale, num_splits, workspace, None, stream, merge=False)


def nvfp4_paged_decode_partial(q, k_pool, v_pool, block_tables, seq_lens, sm_scale, num_splits,
                               variant=VARIANT_AUTO, workspace=None, stream=None):
    return _partial("nvfp4_paged_decode_partial", q, k_pool, v_pool, block_tables, seq_lens, sm_scale,
                    num_splits, variant, workspace, stream)


def fp8_paged_decode_partial(q, k_pool, v_pool, block_tables, seq_lens, sm_scale, num_splits,
                             variant=VARIANT_AUTO, workspace=None, stream=None):
    return _partial("fp8_paged_decode_partial", q, k_pool, v_pool, block_tables, seq_lens, sm_scale,
                    num_splits, variant, workspace, stream)


def nvfp4kv_lse_merge(workspace, batch, num_q_heads, head_dim, num_splits, out_scale, out, stream=None):
    _need(out, torch.bfloat16, "out")
    _shape(out, (batch, num_q_heads, head_dim), "out")
    _check(lib().nvfp4kv_lse_merge(workspace.data_ptr(), workspace.numel() * workspace.element_size(), batch,
                                   num_q_heads, head_dim, num_splits, float(out_scale), out.data_ptr(),
                                   _stream(stream)))
    return out


def split_partials(workspace: torch.Tensor, batch, num_q_heads, head_dim, num_splits):
    """Views (u [B][Hq][S][d] f16, ml [B][Hq][S][2] fp32) of a decode workspace's partials:
    u is each split's o / l, (m, l) its base-2 maximum logit and softmax denominator."""
    raw = workspace.view(torch.uint8)
    n = batch * num_q_heads * num_splits * head_dim
    u = raw[:2 * n].view(torch.float16).view(batch, num_q_heads, num_splits, head_dim)
    ml = raw[2 * n:2 * n + 8 * batch * num_q_heads * num_splits].view(torch.float32)
    return u, ml.view(batch, num_q_heads, num_splits, 2)
