"""Python binding of the MI355X OUT_PROD library (libretro_out_prod.so).

    dst[t][k] = sum_n W[n][k] * G[t][n]

the backward of mul_mat(W, x) with respect to x through a resident
block-quantized (Q8_0, Q4_0, Q4_1, Q5_0, Q5_1, MXFP4, Q2_K..Q6_K), F16, BF16 or F32 weight W (llama.cpp PR
#3 "cuda: out_prod accepts a quantized src0", commit message and section
"What"). This module marshals torch tensors into the C ABI of
include/retro_out_prod.h and nothing else: every step runs in the HIP
library. There is no CPU path; if the library is not built, importing this
package raises.
"""

from __future__ import annotations

import ctypes
import functools
import os

# torch ships its own HIP runtime under the same soname (libamdhip64.so.7) as
# the system ROCm one this library links against. Whichever is loaded first
# serves the whole process, and torch only works on its own, so torch must be
# loaded before the library: then the library's kernels, torch's memory and
# torch's streams all belong to one runtime.
import torch  # noqa: F401

from . import _build

F32, F16, Q4_0, Q4_1, Q5_0, Q5_1, Q8_0 = 0, 1, 2, 3, 6, 7, 8
Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, BF16, MXFP4, NVFP4 = 10, 11, 12, 13, 14, 30, 39, 40
TYPES = {"f32": F32, "f16": F16, "bf16": BF16, "q8_0": Q8_0, "q4_0": Q4_0, "q4_1": Q4_1, "q5_0": Q5_0,
         "q5_1": Q5_1, "mxfp4": MXFP4, "nvfp4": NVFP4, "q2_k": Q2_K, "q3_k": Q3_K, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}

OK = 0
E_TYPE, E_SHAPE, E_NULL, E_ALIGN, E_ALIAS, E_HIP, E_VARIANT, E_WORKSPACE = -1, -2, -3, -4, -5, -6, -7, -8

VARIANT_AUTO = 0
VARIANT_SKINNY = 1
VARIANT_TILE_128x128 = 2
VARIANT_TILE_128x256 = 3
VARIANT_TILE_64x128 = 4
VARIANT_TILE_64x64 = 5
VARIANT_TILE_64x256 = 6
VARIANT_WS_128x256 = 7
VARIANT_WS_64x256 = 8
VARIANT_WS_128x128 = 9
VARIANT_WS_64x128 = 10
VARIANT_WS_32x256 = 11
VARIANT_WS_32x128 = 12
VARIANT_WS2_64x128 = 13
VARIANT_SIMPLE = 15
VARIANT_SPLIT_128x256 = 16
VARIANT_SPLIT_128x128 = 17
VARIANT_WS_256x256 = 18
VARIANT_WS_256x128 = 19
VARIANT_SKINNY_8 = 20
VARIANT_SKINNY_16 = 21
VARIANT_SKINNY_SPLIT = 22
VARIANT_NAMES = {
    VARIANT_SKINNY: "skinny", VARIANT_TILE_128x128: "tile_128x128", VARIANT_TILE_128x256: "tile_128x256",
    VARIANT_TILE_64x128: "tile_64x128", VARIANT_TILE_64x64: "tile_64x64", VARIANT_TILE_64x256: "tile_64x256",
    VARIANT_WS_128x256: "ws_128x256", VARIANT_WS_64x256: "ws_64x256", VARIANT_WS_128x128: "ws_128x128",
    VARIANT_WS_64x128: "ws_64x128", VARIANT_WS_32x256: "ws_32x256", VARIANT_WS_32x128: "ws_32x128",
    VARIANT_WS2_64x128: "ws2_64x128", VARIANT_SIMPLE: "simple", VARIANT_SPLIT_128x256: "split_128x256",
    VARIANT_SPLIT_128x128: "split_128x128", VARIANT_WS_256x256: "ws_256x256",
    VARIANT_WS_256x128: "ws_256x128", VARIANT_SKINNY_8: "skinny_8", VARIANT_SKINNY_16: "skinny_16",
    VARIANT_SKINNY_SPLIT: "skinny_split",
}

LIB_PATH = _build.LIB_PATH

# The exported symbols, as declared in include/retro_out_prod.h and
# include/retro_probe.h.
EXPORTS = ("retro_out_prod", "retro_out_prod_variant", "retro_out_prod_strided", "retro_out_prod_strided_variant",
           "retro_dequantize", "retro_out_prod_supported", "retro_out_prod_choice", "retro_out_prod_variant_applies",
           "retro_out_prod_strided_variant_applies", "retro_out_prod_batched", "retro_out_prod_batched_variant",
           "retro_out_prod_views", "retro_out_prod_views_variant", "retro_out_prod_views_variant_applies",
           "retro_out_prod_views_choice", "retro_out_prod_plan", "retro_out_prod_views_plan",
           "retro_out_prod_column_split", "retro_out_prod_ws", "retro_out_prod_workspace_size",
           "retro_out_prod_noalloc",
           "retro_mul_mat", "retro_mul_mat_variant", "retro_mul_mat_choice", "retro_mul_mat_variant_applies",
           "retro_mul_mat_plan", "retro_mul_mat_row_split",
           "retro_row_bytes", "retro_strerror",
           "retro_probe_sink_floats", "retro_probe_mfma", "retro_probe_mfma_valu", "retro_probe_copy")

PROBE_MFMA_F32 = 0
PROBE_MFMA_BF16 = 1


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() or "
            "python -m quantized_weight_backward_amd._build")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    lib.retro_out_prod.restype = i32
    lib.retro_out_prod.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_out_prod_variant.restype = i32
    lib.retro_out_prod_variant.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_out_prod_strided.restype = i32
    lib.retro_out_prod_strided.argtypes = [i32, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.retro_out_prod_strided_variant.restype = i32
    lib.retro_out_prod_strided_variant.argtypes = [i32, i32, vp, i64, vp, i64, vp, i64, i64, i64, i64, vp]
    lib.retro_out_prod_batched.restype = i32
    lib.retro_out_prod_batched.argtypes = [i32, vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64, i64,
                                           i64, i64, i64, i64, i64, i64, i64, vp]
    lib.retro_out_prod_batched_variant.restype = i32
    lib.retro_out_prod_batched_variant.argtypes = [i32, i32, vp, i64, i64, i64, vp, i64, i64, i64, vp, i64, i64,
                                                   i64, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.retro_out_prod_views.restype = i32
    lib.retro_out_prod_views.argtypes = [i32, vp, i64, i64, i64, vp, i64, i64, i64, i64, vp, i64, i64, i64,
                                         i64, i64, i64, i64, i64, i64, i64, vp]
    lib.retro_out_prod_views_variant.restype = i32
    lib.retro_out_prod_views_variant.argtypes = [i32, i32, vp, i64, i64, i64, vp, i64, i64, i64, i64, vp, i64, i64,
                                                 i64, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.retro_out_prod_views_variant_applies.restype = i32
    lib.retro_out_prod_views_variant_applies.argtypes = [i32, i32, i64, i64, i64, i64, i64, i64, i64]
    lib.retro_out_prod_views_choice.restype = i32
    lib.retro_out_prod_views_choice.argtypes = [i32, i64, i64, i64, i64, i64, i64, i64, i64, i64]
    lib.retro_mul_mat.restype = i32
    lib.retro_mul_mat.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_mul_mat_variant.restype = i32
    lib.retro_mul_mat_variant.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_mul_mat_choice.restype = i32
    lib.retro_mul_mat_choice.argtypes = [i32, i64, i64, i64]
    lib.retro_mul_mat_plan.restype = i32
    lib.retro_mul_mat_plan.argtypes = [i32, i64, i64, i64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(i64),
                                       ctypes.POINTER(ctypes.c_int32)]
    lib.retro_mul_mat_row_split.restype = i32
    lib.retro_mul_mat_row_split.argtypes = [i32, i64, i32, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_mul_mat_variant_applies.restype = i32
    lib.retro_mul_mat_variant_applies.argtypes = [i32, i32, i64, i64, i64]
    lib.retro_out_prod_strided_variant_applies.restype = i32
    lib.retro_out_prod_strided_variant_applies.argtypes = [i32, i32, i64, i64, i64, i64, i64, i64]
    lib.retro_dequantize.restype = i32
    lib.retro_dequantize.argtypes = [i32, vp, vp, i64, i64, vp]
    lib.retro_out_prod_supported.restype = i32
    lib.retro_out_prod_supported.argtypes = [i32, i64, i64, i64]
    lib.retro_out_prod_choice.restype = i32
    lib.retro_out_prod_choice.argtypes = [i32, i64, i64, i64]
    lib.retro_out_prod_plan.restype = i32
    lib.retro_out_prod_plan.argtypes = [i32, i64, i64, i64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(i64),
                                        ctypes.POINTER(ctypes.c_int32)]
    lib.retro_out_prod_views_plan.restype = i32
    lib.retro_out_prod_views_plan.argtypes = [i32, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                              ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(i64),
                                              ctypes.POINTER(ctypes.c_int32)]
    lib.retro_out_prod_column_split.restype = i32
    lib.retro_out_prod_column_split.argtypes = [i32, i64, i32, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_out_prod_ws.restype = i32
    lib.retro_out_prod_ws.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.retro_out_prod_noalloc.restype = i32
    lib.retro_out_prod_noalloc.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, vp]
    lib.retro_out_prod_workspace_size.restype = i64
    lib.retro_out_prod_workspace_size.argtypes = [i32, i32, i64, i64, i64]
    lib.retro_out_prod_variant_applies.restype = i32
    lib.retro_out_prod_variant_applies.argtypes = [i32, i32, i64, i64, i64]
    lib.retro_row_bytes.restype = i64
    lib.retro_row_bytes.argtypes = [i32, i64]
    lib.retro_probe_sink_floats.restype = i64
    lib.retro_probe_sink_floats.argtypes = []
    lib.retro_probe_mfma.restype = i32
    lib.retro_probe_mfma.argtypes = [i32, vp, i64, ctypes.POINTER(ctypes.c_double), vp]
    lib.retro_probe_mfma_valu.restype = i32
    lib.retro_probe_mfma_valu.argtypes = [i64, i64, vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), vp]
    lib.retro_probe_copy.restype = i32
    lib.retro_probe_copy.argtypes = [vp, vp, i64, vp]
    lib.retro_strerror.restype = ctypes.c_char_p
    lib.retro_strerror.argtypes = [i32]
    return lib


lib = _load()


class RetroError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"{strerror(code)} (code {code})")
        self.code = code


def strerror(code: int) -> str:
    return lib.retro_strerror(int(code)).decode()


@functools.lru_cache(maxsize=256)
def row_bytes(wtype: int, K: int) -> int:
    return int(lib.retro_row_bytes(int(wtype), int(K)))


def supported(wtype: int, K: int, N: int, T: int) -> bool:
    return lib.retro_out_prod_supported(int(wtype), int(K), int(N), int(T)) == 1


def choice(wtype: int, K: int, N: int, T: int) -> int:
    return int(lib.retro_out_prod_choice(int(wtype), int(K), int(N), int(T)))


def plan(wtype: int, K: int, N: int, T: int) -> tuple[int, int, int]:
    """The launches out_prod makes: (variant0, k_split, variant1), variant0
    over dst columns [0, k_split) and variant1 (0 when k_split == K: one
    launch) over the rest."""
    v0, v1, ks = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    n = lib.retro_out_prod_plan(int(wtype), int(K), int(N), int(T), ctypes.byref(v0), ctypes.byref(ks),
                                ctypes.byref(v1))
    _check(OK if n > 0 else n)
    return int(v0.value), int(ks.value), int(v1.value)


def views_plan(wtype: int, K: int, N: int, T: int, ldw: int, sgt: int, sgn: int, ldd: int, ne2: int = 1,
               ne3: int = 1) -> tuple[int, int, int]:
    """The launches out_prod_batched makes for ne2 x ne3 matrices with these
    strides, as plan()."""
    v0, v1, ks = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    n = lib.retro_out_prod_views_plan(int(wtype), int(K), int(N), int(T), int(ldw), int(sgt), int(sgn), int(ldd),
                                      int(ne2), int(ne3), ctypes.byref(v0), ctypes.byref(ks), ctypes.byref(v1))
    _check(OK if n > 0 else n)
    return int(v0.value), int(ks.value), int(v1.value)


def plan_names(wtype: int, K: int, N: int, T: int) -> str:
    """The plan as text: 'ws_64x128', or 'ws_128x256[0:4096]+ws2_64x128[4096:5120]'."""
    v0, ks, v1 = plan(wtype, K, N, T)
    if ks >= K:
        return VARIANT_NAMES[v0]
    return f"{VARIANT_NAMES[v0]}[0:{ks}]+{VARIANT_NAMES[v1]}[{ks}:{K}]"


def variant_applies(variant: int, wtype: int, K: int, N: int, T: int) -> bool:
    return lib.retro_out_prod_variant_applies(int(variant), int(wtype), int(K), int(N), int(T)) == 1


def _check(code: int) -> None:
    if code != OK:
        raise RetroError(code)


# The current stream's handle without building a torch Stream object per call
# (torch's raw accessor, when this torch has it).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_current_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream_handle(stream) -> int:
    if stream is not None:
        return int(stream.cuda_stream)
    if _raw_stream is not None and _current_device is not None:
        return int(_raw_stream(_current_device()))
    return int(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _device_tensor(t, name, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _row_stride(t, name) -> int:
    """Elements between rows of a 2-D view whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D view with contiguous rows")
    return int(t.stride(0)) if t.shape[0] > 1 else int(t.shape[1])


def out_prod(wtype: int, W, G, K: int, out=None, variant: int = VARIANT_AUTO, stream=None):
    """dst = out_prod(W, G): W packed bytes (N rows), G float32 T x N, dst float32 T x K.

    W is a contiguous device tensor of N * row_bytes(wtype, K) bytes, or a
    2-D uint8 view of N rows whose first row_bytes bytes hold a W row; out is
    a 2-D float32 view whose rows are contiguous (its row stride may exceed
    K); G is a 2-D float32 view whose rows are contiguous, or whose columns
    are (G stored t-fastest, such as the transpose of a contiguous N x T
    tensor). Runs asynchronously on `stream` (default: torch's current
    stream).
    """
    _device_tensor(W, "W", contiguous=False)
    _device_tensor(G, "G", contiguous=False)
    if G.dtype != torch.float32 or G.dim() != 2:
        raise ValueError("G must be a 2-D float32 tensor (T x N)")
    T, N = G.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if W.is_contiguous():
        if W.numel() * W.element_size() != N * rb:
            raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
        ldw = rb
    else:
        if W.dtype != torch.uint8 or W.shape[0] != N or W.shape[1] < rb:
            raise ValueError(f"a strided W must be a uint8 view of N rows of at least {rb} bytes")
        ldw = _row_stride(W, "W")
    sgt, sgn = _g_strides2(G)
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=G.device)
    else:
        _device_tensor(out, "out", contiguous=False)
        if out.dtype != torch.float32 or tuple(out.shape) != (T, K):
            raise ValueError("out must be float32 T x K")
    ldd = _row_stride(out, "out")
    if (ldw, sgt, sgn, ldd) == (rb, N, 1, K):
        _check(lib.retro_out_prod_variant(int(variant), int(wtype), _ptr(W), _ptr(G), _ptr(out), int(K), int(N),
                                          int(T), _stream_handle(stream)))
    elif sgn == 1:
        _check(lib.retro_out_prod_strided_variant(int(variant), int(wtype), _ptr(W), ldw, _ptr(G), sgt, _ptr(out),
                                                  ldd, int(K), int(N), int(T), _stream_handle(stream)))
    else:
        _check(lib.retro_out_prod_views_variant(int(variant), int(wtype), _ptr(W), ldw, 0, 0, _ptr(G), sgt, sgn, 0,
                                                0, _ptr(out), ldd, 0, 0, int(K), int(N), int(T), 1, 1, 1, 1,
                                                _stream_handle(stream)))
    return out



def workspace_size(wtype: int, K: int, N: int, T: int, variant: int = VARIANT_AUTO) -> int:
    """Bytes of workspace out_prod_ws uses for this shape (0: none; negative: an error code)."""
    return int(lib.retro_out_prod_workspace_size(int(variant), int(wtype), int(K), int(N), int(T)))


def new_workspace(device=None):
    """A zeroed workspace for out_prod_ws, large enough for any shape."""
    nbytes = workspace_size(Q4_K, 4096, 4096, 48, VARIANT_SKINNY_SPLIT)
    return torch.zeros(nbytes, dtype=torch.uint8, device=device if device is not None else "cuda")


def out_prod_ws(wtype: int, W, G, K: int, workspace, out=None, variant: int = VARIANT_AUTO, stream=None):
    """out_prod with a workspace (contiguous W, G and out): for T <= 16 and
    few 64-column slabs of dst, the split over all CUs. The workspace is a
    device tensor from new_workspace (or None); calls sharing one must be
    ordered on a stream."""
    _device_tensor(W, "W")
    _device_tensor(G, "G")
    if G.dtype != torch.float32 or G.dim() != 2:
        raise ValueError("G must be a contiguous 2-D float32 tensor (T x N)")
    T, N = G.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if W.numel() * W.element_size() != N * rb:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=G.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (T, K):
            raise ValueError("out must be a contiguous float32 T x K tensor")
    if workspace is not None:
        _device_tensor(workspace, "workspace")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.retro_out_prod_ws(int(variant), int(wtype), _ptr(W), _ptr(G), _ptr(out), int(K), int(N), int(T),
                                 _ptr(workspace), int(nbytes), _stream_handle(stream)))
    return out


def out_prod_noalloc(wtype: int, W, G, K: int, out=None, variant: int = VARIANT_AUTO, stream=None):
    """out_prod_ws with the library's static per-GPU workspace: the library
    call allocates nothing (pass out, or this wrapper allocates dst). Calls
    on one GPU must be ordered."""
    _device_tensor(W, "W")
    _device_tensor(G, "G")
    if G.dtype != torch.float32 or G.dim() != 2:
        raise ValueError("G must be a contiguous 2-D float32 tensor (T x N)")
    T, N = G.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if W.numel() * W.element_size() != N * rb:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=G.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (T, K):
            raise ValueError("out must be a contiguous float32 T x K tensor")
    _check(lib.retro_out_prod_noalloc(int(variant), int(wtype), _ptr(W), _ptr(G), _ptr(out), int(K), int(N), int(T),
                                      _stream_handle(stream)))
    return out


def out_prod_column_split(wtype: int, W, G, K: int, variant0: int, k_split: int, variant1: int, out=None,
                          stream=None):
    """out_prod as two launches: variant0 over dst columns [0, k_split),
    variant1 over [k_split, K) (contiguous W, G and out)."""
    _device_tensor(W, "W")
    _device_tensor(G, "G")
    if G.dtype != torch.float32 or G.dim() != 2:
        raise ValueError("G must be a contiguous 2-D float32 tensor (T x N)")
    T, N = G.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if W.numel() * W.element_size() != N * rb:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((T, K), dtype=torch.float32, device=G.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (T, K):
            raise ValueError("out must be a contiguous float32 T x K tensor")
    _check(lib.retro_out_prod_column_split(int(variant0), int(k_split), int(variant1), int(wtype), _ptr(W), _ptr(G),
                                           _ptr(out), int(K), int(N), int(T), _stream_handle(stream)))
    return out

def _as4(t):
    while t.dim() < 4:
        t = t.unsqueeze(0)
    return t


def _matrix_strides(t, rows, name):
    """(row stride, stride of dim 1, stride of dim 0) in elements of a 4-D
    view with contiguous rows; strides of size-1 dimensions read as 0 and
    a single row's stride as its length."""
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name} must have contiguous rows")
    ld = int(t.stride(2)) if t.shape[2] > 1 else rows
    return ld, (int(t.stride(1)) if t.shape[1] > 1 else 0), (int(t.stride(0)) if t.shape[0] > 1 else 0)


def _g_strides2(G):
    """_g_strides of one T x N matrix, read from the 2-D view itself."""
    T, N = G.shape
    st, sn = G.stride()
    if N <= 1 or sn == 1:
        return (st if T > 1 else max(N, 1)), 1
    if T <= 1 or st == 1:
        return 1, sn
    raise ValueError("G must have contiguous rows or contiguous columns")


def _g_strides(G4):
    """(sgt, sgn): element strides of the T x N matrices of a 4-D G view
    whose rows or columns are contiguous. The stride of a dimension of size
    1 is never used and is reported so that the layout rule holds."""
    T, N = int(G4.shape[2]), int(G4.shape[3])
    st, sn = int(G4.stride(2)), int(G4.stride(3))
    if N <= 1 or sn == 1:
        return (st if T > 1 else max(N, 1)), 1
    if T <= 1 or st == 1:
        return 1, sn
    raise ValueError("G must have contiguous rows or contiguous columns")


def out_prod_batched(wtype: int, W, G, K: int, out=None, variant: int = VARIANT_AUTO, stream=None):
    """Batched out_prod over two outer dimensions with W broadcast (see
    retro_out_prod_batched): W uint8 [ne03, ne02, N, >= row_bytes],
    G float32 [ne3, ne2, T, N], out float32 [ne3, ne2, T, K] (leading
    dimensions may be left out; ne03 divides ne3 and ne02 divides ne2).
    Rows of W and out are contiguous; G's rows or its columns are (see
    out_prod); rows and matrices may be any distance apart."""
    _device_tensor(W, "W", contiguous=False)
    _device_tensor(G, "G", contiguous=False)
    if G.dtype != torch.float32 or not 2 <= G.dim() <= 4 or W.dtype != torch.uint8 or not 2 <= W.dim() <= 4:
        raise ValueError("W must be a 2-4-D uint8 tensor and G a 2-4-D float32 tensor")
    W4, G4 = _as4(W), _as4(G)
    ne03, ne02, N, wcols = W4.shape
    ne3, ne2, T, n_g = G4.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if n_g != N or wcols < rb:
        raise ValueError(f"W must hold N = {n_g} rows of at least {rb} bytes per matrix")
    if out is None:
        out = torch.empty(tuple(G.shape[:-2]) + (T, K), dtype=torch.float32, device=G.device)
    else:
        _device_tensor(out, "out", contiguous=False)
        if out.dtype != torch.float32 or tuple(out.shape) != tuple(G.shape[:-2]) + (T, K):
            raise ValueError("out must be float32 with G's leading dimensions and T x K matrices")
    D4 = _as4(out)
    ldw, sw2, sw3 = _matrix_strides(W4, rb, "W")
    sgt, sgn = _g_strides(G4)
    sg2 = int(G4.stride(1)) if G4.shape[1] > 1 else 0
    sg3 = int(G4.stride(0)) if G4.shape[0] > 1 else 0
    ldd, sd2, sd3 = _matrix_strides(D4, K, "out")
    _check(lib.retro_out_prod_views_variant(int(variant), int(wtype), _ptr(W), ldw, sw2, sw3, _ptr(G), sgt, sgn, sg2,
                                            sg3, _ptr(out), ldd, sd2, sd3, int(K), int(N), int(T), int(ne02),
                                            int(ne03), int(ne2), int(ne3), _stream_handle(stream)))
    return out


def variant_applies_strided(variant: int, wtype: int, K: int, N: int, T: int, ldw: int, ldg: int, ldd: int) -> bool:
    return lib.retro_out_prod_strided_variant_applies(int(variant), int(wtype), int(K), int(N), int(T), int(ldw),
                                                      int(ldg), int(ldd)) == 1


def variant_applies_views(variant: int, wtype: int, K: int, N: int, T: int, ldw: int, sgt: int, sgn: int,
                          ldd: int) -> bool:
    return lib.retro_out_prod_views_variant_applies(int(variant), int(wtype), int(K), int(N), int(T), int(ldw),
                                                    int(sgt), int(sgn), int(ldd)) == 1


def choice_views(wtype: int, K: int, N: int, T: int, ldw: int, sgt: int, sgn: int, ldd: int, ne2: int = 1,
                 ne3: int = 1) -> int:
    return int(lib.retro_out_prod_views_choice(int(wtype), int(K), int(N), int(T), int(ldw), int(sgt), int(sgn),
                                               int(ldd), int(ne2), int(ne3)))


def mul_mat(wtype: int, W, X, N: int | None = None, out=None, variant: int = VARIANT_AUTO, stream=None):
    """Y = mul_mat(W, X), the forward Y[t][n] = sum_k W[n][k] X[t][k]: X a
    contiguous float32 T x K device tensor, W contiguous packed bytes of N
    rows (N taken from W's size unless given), Y float32 T x N."""
    _device_tensor(W, "W")
    _device_tensor(X, "X")
    if X.dtype != torch.float32 or X.dim() != 2:
        raise ValueError("X must be a contiguous 2-D float32 tensor (T x K)")
    T, K = X.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    nbytes = W.numel() * W.element_size()
    if N is None:
        if rb == 0:
            raise ValueError("N must be given when K = 0")
        N = nbytes // rb
    if nbytes != N * rb:
        raise ValueError(f"W holds {nbytes} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=X.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (T, N):
            raise ValueError("out must be contiguous float32 T x N")
    _check(lib.retro_mul_mat_variant(int(variant), int(wtype), _ptr(W), _ptr(X), _ptr(out), int(K), int(N), int(T),
                                     _stream_handle(stream)))
    return out


def mul_mat_choice(wtype: int, K: int, N: int, T: int) -> int:
    return int(lib.retro_mul_mat_choice(int(wtype), int(K), int(N), int(T)))


def mul_mat_plan(wtype: int, K: int, N: int, T: int) -> tuple[int, int, int]:
    """The launches mul_mat makes: (variant0, n_split, variant1), variant0
    over W rows [0, n_split) and variant1 (0 when n_split == N: one launch)
    over the rest."""
    v0, v1, ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    n = lib.retro_mul_mat_plan(int(wtype), int(K), int(N), int(T), ctypes.byref(v0), ctypes.byref(ns),
                               ctypes.byref(v1))
    _check(OK if n > 0 else n)
    return int(v0.value), int(ns.value), int(v1.value)


def mul_mat_plan_names(wtype: int, K: int, N: int, T: int) -> str:
    v0, ns, v1 = mul_mat_plan(wtype, K, N, T)
    if ns >= N:
        return VARIANT_NAMES[v0]
    return f"{VARIANT_NAMES[v0]}[0:{ns}]+{VARIANT_NAMES[v1]}[{ns}:{N}]"


def mul_mat_row_split(wtype: int, W, X, N: int, variant0: int, n_split: int, variant1: int, out=None, stream=None):
    """mul_mat as two launches: variant0 over W rows [0, n_split), variant1
    over the rest (contiguous W, X and out)."""
    _device_tensor(W, "W")
    _device_tensor(X, "X")
    if X.dtype != torch.float32 or X.dim() != 2:
        raise ValueError("X must be a contiguous 2-D float32 tensor (T x K)")
    T, K = X.shape
    rb = row_bytes(wtype, K)
    if rb < 0:
        _check(E_SHAPE if wtype in TYPES.values() else E_TYPE)
    if W.numel() * W.element_size() != N * rb:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=X.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (T, N):
            raise ValueError("out must be contiguous float32 T x N")
    _check(lib.retro_mul_mat_row_split(int(variant0), int(n_split), int(variant1), int(wtype), _ptr(W), _ptr(X),
                                       _ptr(out), int(K), int(N), int(T), _stream_handle(stream)))
    return out


def mul_mat_variant_applies(variant: int, wtype: int, K: int, N: int, T: int) -> bool:
    return lib.retro_mul_mat_variant_applies(int(variant), int(wtype), int(K), int(N), int(T)) == 1


def probe_sink(device=None):
    """A float32 device buffer of the size the matrix-core probe writes."""
    return torch.empty(int(lib.retro_probe_sink_floats()), dtype=torch.float32, device=device or "cuda")


def probe_mfma(kind: int, sink, iterations: int, stream=None) -> float:
    """Enqueue the matrix-core probe (PROBE_MFMA_F32 or PROBE_MFMA_BF16);
    returns the FLOPs of the launch."""
    _device_tensor(sink, "sink")
    if sink.dtype != torch.float32 or sink.numel() < int(lib.retro_probe_sink_floats()):
        raise ValueError("sink must be a float32 buffer of retro_probe_sink_floats() elements")
    flops = ctypes.c_double(0.0)
    _check(lib.retro_probe_mfma(int(kind), _ptr(sink), int(iterations), ctypes.byref(flops), _stream_handle(stream)))
    return flops.value


def probe_mfma_valu(sink, mfma_iterations: int, valu_iterations: int, stream=None):
    """Enqueue the matrix-core-beside-vector-ALU probe; returns (MFMA FLOPs,
    wave-level FMA instructions) of the launch."""
    _device_tensor(sink, "sink")
    if sink.dtype != torch.float32 or sink.numel() < int(lib.retro_probe_sink_floats()):
        raise ValueError("sink must be a float32 buffer of retro_probe_sink_floats() elements")
    flops = ctypes.c_double(0.0)
    instrs = ctypes.c_int64(0)
    _check(lib.retro_probe_mfma_valu(int(mfma_iterations), int(valu_iterations), _ptr(sink), ctypes.byref(flops),
                                     ctypes.byref(instrs), _stream_handle(stream)))
    return flops.value, instrs.value


def probe_copy(src, dst, stream=None) -> None:
    """Enqueue the copy probe: dst = src, two contiguous device tensors of the
    same number of bytes (a multiple of 16)."""
    _device_tensor(src, "src")
    _device_tensor(dst, "dst")
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must hold the same number of bytes")
    _check(lib.retro_probe_copy(_ptr(src), _ptr(dst), n, _stream_handle(stream)))


def dequantize(wtype: int, W, K: int, N: int, out=None, stream=None):
    """Decoded float32 N x K copy of W (a test hook; out_prod never makes one)."""
    _device_tensor(W, "W")
    rb = row_bytes(wtype, K)
    if rb >= 0 and W.numel() * W.element_size() != N * rb:
        raise ValueError(f"W holds {W.numel() * W.element_size()} bytes, expected N*row_bytes = {N * rb}")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    else:
        _device_tensor(out, "out")
        if out.dtype != torch.float32 or tuple(out.shape) != (N, K):
            raise ValueError("out must be float32 N x K")
    _check(lib.retro_dequantize(int(wtype), _ptr(W), _ptr(out), int(K), int(N), _stream_handle(stream)))
    return out
