"""Python binding of libdvssq.so, the DV-SSQ quantized linear layer for MI355X.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI of include/dvssq.h.  PyTorch supplies device memory
(tensor.data_ptr()) and streams; nothing here computes the layer, and there is
no CPU fallback: if the library is missing, importing this module fails.

Names follow the C ABI: pack_info, fwht, linear_decode, linear_prefill,
status_str.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdvssq.so")

DVSSQ_OK = 0
DVSSQ_EINVAL = -1
DVSSQ_EUNSUPPORTED = -2
DVSSQ_EHIP = -3
DVSSQ_X_ROTATED = 1
DVSSQ_TEST_NO_PUBLISH = 0x80000000
DVSSQ_WS_STATUS_BYTES = 256
DVSSQ_STATUS_WAIT_TIMEOUT = 1
DECODE_MAX_M = 32

EXPORTS = ("dvssq_pack_info", "dvssq_fwht", "dvssq_linear_decode", "dvssq_linear_prefill",
           "dvssq_materialize", "dvssq_mlp_ws_bytes", "dvssq_mlp_ws_offsets", "dvssq_mlp_decode",
           "dvssq_mlp_prefill", "dvssq_stream_read", "dvssq_linear_decode_noalloc", "dvssq_quantize_ws_bytes",
           "dvssq_quantize", "dvssq_kvbss_attention_ws_bytes", "dvssq_kvbss_attention", "dvssq_status_str")


class Layout(C.Structure):
    """Mirror of struct dvssq_layout."""
    _fields_ = [(n, C.c_int32) for n in ("N", "K", "r", "block", "group", "n_seg", "n_int8",
                                         "n_int4", "M_max", "reserved")] + \
               [(n, C.c_int64) for n in ("off_idx", "off_q4", "off_s4", "off_q8", "off_s8",
                                         "off_U", "off_V", "blob_bytes", "algo_bytes", "ws_bytes")]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


class AttnShape(C.Structure):
    """Mirror of struct dvssq_attn_shape."""
    _fields_ = [(n, C.c_int32) for n in ("B", "Mq", "Nk", "Hq", "Hkv", "D", "window")] + \
               [("scale", C.c_float), ("haze", C.c_float)]


class DvssqError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_str(code)} ({code})")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run bit_linear_amd/build.py (hipcc, gfx950)")

# One HIP runtime per process: PyTorch loads the HIP runtime it ships by path.
# Importing it first lets libdvssq.so bind to that same runtime (same soname)
# instead of loading a second copy from the ROCm install, which would then
# compete with PyTorch's for the device.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = C.CDLL(LIB_PATH)
_P = C.c_void_p
_lib.dvssq_pack_info.restype = C.c_int
_lib.dvssq_pack_info.argtypes = [C.c_int32] * 6 + [C.POINTER(Layout)]
_lib.dvssq_fwht.restype = C.c_int
_lib.dvssq_fwht.argtypes = [_P, _P, C.c_int32, C.c_int32, C.c_int32, _P]
for _n in ("dvssq_linear_decode", "dvssq_linear_prefill"):
    getattr(_lib, _n).restype = C.c_int
    getattr(_lib, _n).argtypes = [C.POINTER(Layout), _P, _P, _P, C.c_int32, _P, C.c_uint32, _P]
_lib.dvssq_linear_decode_noalloc.restype = C.c_int
_lib.dvssq_linear_decode_noalloc.argtypes = [C.POINTER(Layout), _P, _P, _P, C.c_int32, C.c_uint32, _P]
_lib.dvssq_materialize.restype = C.c_int
_lib.dvssq_materialize.argtypes = [C.POINTER(Layout), _P, _P, _P]
_lib.dvssq_mlp_ws_bytes.restype = C.c_int
_lib.dvssq_mlp_ws_bytes.argtypes = [C.POINTER(Layout), C.POINTER(Layout), C.POINTER(C.c_int64)]
_lib.dvssq_mlp_ws_offsets.restype = C.c_int
_lib.dvssq_mlp_ws_offsets.argtypes = [C.POINTER(Layout), C.POINTER(Layout), C.POINTER(C.c_int64),
                                      C.POINTER(C.c_int64)]
for _n in ("dvssq_mlp_decode", "dvssq_mlp_prefill"):
    getattr(_lib, _n).restype = C.c_int
    getattr(_lib, _n).argtypes = [C.POINTER(Layout), _P, C.POINTER(Layout), _P, _P, _P, C.c_int32, _P, C.c_uint32, _P]
_lib.dvssq_quantize_ws_bytes.restype = C.c_int64
_lib.dvssq_quantize_ws_bytes.argtypes = [C.POINTER(Layout), C.c_int32]
_lib.dvssq_quantize.restype = C.c_int
_lib.dvssq_quantize.argtypes = [C.POINTER(Layout), _P, _P, C.c_int32, C.c_int32, _P, _P, _P]
_lib.dvssq_kvbss_attention.restype = C.c_int
_lib.dvssq_kvbss_attention.argtypes = [C.POINTER(AttnShape), _P, _P, _P, _P, _P, _P]
_lib.dvssq_kvbss_attention_ws_bytes.restype = C.c_int
_lib.dvssq_kvbss_attention_ws_bytes.argtypes = [C.POINTER(AttnShape), C.POINTER(C.c_int64)]
_lib.dvssq_stream_read.restype = C.c_int
_lib.dvssq_stream_read.argtypes = [_P, C.c_int64, _P, _P]
_lib.dvssq_status_str.restype = C.c_char_p
_lib.dvssq_status_str.argtypes = [C.c_int]


def lib():
    return _lib


def status_str(code: int) -> str:
    return _lib.dvssq_status_str(int(code)).decode()


def _ptr(t) -> int | None:
    """Device (or host) address of a tensor, or an int address, or None."""
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


def _check(rc: int, where: str) -> None:
    if rc != DVSSQ_OK:
        raise DvssqError(rc, where)


def pack_info(N: int, K: int, r: int, block: int, n_seg: int = 1, M_max: int = 32) -> Layout:
    out = Layout()
    _check(_lib.dvssq_pack_info(N, K, r, block, n_seg, M_max, C.byref(out)), "dvssq_pack_info")
    return out


def fwht(x, xrot, M: int, K: int, block: int, stream=None) -> None:
    _check(_lib.dvssq_fwht(_ptr(x), _ptr(xrot), M, K, block, _stream(stream)), "dvssq_fwht")


def linear_decode(layout: Layout, blob, x, y, M: int, ws, flags: int = 0, stream=None) -> None:
    _check(_lib.dvssq_linear_decode(C.byref(layout), _ptr(blob), _ptr(x), _ptr(y), M, _ptr(ws),
                                    flags, _stream(stream)), "dvssq_linear_decode")


def linear_prefill(layout: Layout, blob, x, y, M: int, ws, flags: int = 0, stream=None) -> None:
    _check(_lib.dvssq_linear_prefill(C.byref(layout), _ptr(blob), _ptr(x), _ptr(y), M, _ptr(ws),
                                     flags, _stream(stream)), "dvssq_linear_prefill")


def linear_decode_noalloc(layout: Layout, blob, x, y, M: int, flags: int = 0, stream=None) -> None:
    _check(_lib.dvssq_linear_decode_noalloc(C.byref(layout), _ptr(blob), _ptr(x), _ptr(y), M, flags,
                                            _stream(stream)), "dvssq_linear_decode_noalloc")


def materialize(layout: Layout, blob, w, stream=None) -> None:
    _check(_lib.dvssq_materialize(C.byref(layout), _ptr(blob), _ptr(w), _stream(stream)), "dvssq_materialize")


def quantize_ws_bytes(layout: Layout, l: int) -> int:
    n = int(_lib.dvssq_quantize_ws_bytes(C.byref(layout), l))
    if n < 0:
        raise DvssqError(DVSSQ_EINVAL, "dvssq_quantize_ws_bytes")
    return n


def quantize(layout: Layout, W, omega, l: int, power_iters: int, blob, ws, stream=None) -> None:
    _check(_lib.dvssq_quantize(C.byref(layout), _ptr(W), _ptr(omega), l, power_iters, _ptr(blob), _ptr(ws),
                               _stream(stream)), "dvssq_quantize")


def kvbss_attention_ws_bytes(shape: AttnShape) -> int:
    n = C.c_int64(0)
    _check(_lib.dvssq_kvbss_attention_ws_bytes(C.byref(shape), C.byref(n)), "dvssq_kvbss_attention_ws_bytes")
    return int(n.value)


def kvbss_attention(shape: AttnShape, q, k, v, o, ws=None, stream=None) -> None:
    _check(_lib.dvssq_kvbss_attention(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(ws), _stream(stream)),
           "dvssq_kvbss_attention")


def mlp_ws_bytes(gu: Layout, down: Layout) -> int:
    out = C.c_int64(0)
    _check(_lib.dvssq_mlp_ws_bytes(C.byref(gu), C.byref(down), C.byref(out)), "dvssq_mlp_ws_bytes")
    return int(out.value)


def mlp_ws_offsets(gu: Layout, down: Layout) -> tuple[int, int]:
    """(off_ygu, off_h): byte offsets of the block's intermediates in its workspace."""
    a, b = C.c_int64(0), C.c_int64(0)
    _check(_lib.dvssq_mlp_ws_offsets(C.byref(gu), C.byref(down), C.byref(a), C.byref(b)), "dvssq_mlp_ws_offsets")
    return int(a.value), int(b.value)


def mlp_decode(gu: Layout, gu_blob, down: Layout, down_blob, x, y, M: int, ws, flags: int = 0,
               stream=None) -> None:
    _check(_lib.dvssq_mlp_decode(C.byref(gu), _ptr(gu_blob), C.byref(down), _ptr(down_blob), _ptr(x), _ptr(y), M,
                                 _ptr(ws), flags, _stream(stream)), "dvssq_mlp_decode")


def mlp_prefill(gu: Layout, gu_blob, down: Layout, down_blob, x, y, M: int, ws, flags: int = 0,
                stream=None) -> None:
    _check(_lib.dvssq_mlp_prefill(C.byref(gu), _ptr(gu_blob), C.byref(down), _ptr(down_blob), _ptr(x), _ptr(y), M,
                                  _ptr(ws), flags, _stream(stream)), "dvssq_mlp_prefill")


def stream_read(buf, nbytes: int, sink, stream=None) -> None:
    """Measurement aid: a plain streaming read of nbytes of buf (no computation)."""
    _check(_lib.dvssq_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "dvssq_stream_read")


def pack_blob(layout: Layout, parts: dict) -> np.ndarray:
    """Place given sub-arrays (idx, q4, s4, q8, s8, U, V) at the layout's offsets."""
    blob = np.zeros(layout.blob_bytes, dtype=np.uint8)
    for name in ("idx", "q4", "s4", "q8", "s8", "U", "V"):
        raw = np.ascontiguousarray(parts[name]).view(np.uint8).reshape(-1)
        off = getattr(layout, "off_" + name)
        blob[off:off + raw.size] = raw
    return blob


# ------------------------------------------------------------------ torch helpers

def device_buffer(nbytes: int, device="cuda"):
    """uint8 device tensor of nbytes (the caching allocator returns >= 512-byte alignment)."""
    import torch
    t = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


class Linear:
    """One packed DV-SSQ layer resident on a GPU, with its workspace.

    forward(x) picks the decode path for M <= 32 and the prefill path above it.
    """

    def __init__(self, blob: np.ndarray, N: int, K: int, r: int, block: int, n_seg: int = 1,
                 M_max: int = 32, device="cuda"):
        import torch
        self.layout = pack_info(N, K, r, block, n_seg, M_max)
        if blob.size != self.layout.blob_bytes:
            raise ValueError(f"blob has {blob.size} bytes, layout needs {self.layout.blob_bytes}")
        self.blob = torch.from_numpy(np.ascontiguousarray(blob)).to(device)
        self.ws = device_buffer(self.layout.ws_bytes, device)
        self.device = device

    def forward(self, x, y=None, flags: int = 0, stream=None, path: str | None = None):
        import torch
        M = x.shape[0]
        if y is None:
            y = torch.empty((M, self.layout.N), dtype=torch.bfloat16, device=x.device)
        if path is None:
            path = "decode" if M <= DECODE_MAX_M else "prefill"
        fn = linear_decode if path == "decode" else linear_prefill
        fn(self.layout, self.blob, x, y, M, self.ws, flags, stream)
        return y


class MLP:
    """Gated MLP block (fused gate+up layer, then down) resident on a GPU:
    dvssq_mlp_decode for M <= 32, dvssq_mlp_prefill above (or as `path` says)."""

    def __init__(self, gu: Linear, down: Linear):
        self.gu, self.down = gu, down
        self.ws = device_buffer(mlp_ws_bytes(gu.layout, down.layout), gu.device)

    def forward(self, x, y=None, flags: int = 0, stream=None, path: str | None = None):
        import torch
        M = x.shape[0]
        if y is None:
            y = torch.empty((M, self.down.layout.N), dtype=torch.bfloat16, device=x.device)
        if path is None:
            path = "decode" if M <= DECODE_MAX_M else "prefill"
        fn = mlp_decode if path == "decode" else mlp_prefill
        fn(self.gu.layout, self.gu.blob, self.down.layout, self.down.blob, x, y, M, self.ws, flags, stream)
        return y
