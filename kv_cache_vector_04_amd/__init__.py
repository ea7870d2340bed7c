"""Python binding of the gfx950 TurboQuant KV-cache codec library (libtq.so).

Argument marshalling only: every step of encode, attention and search runs
in the HIP kernels behind the C ABI declared in include/tq.h.  PyTorch
provides device memory and the current stream; nothing here computes.

The library must be built (``python -m kv_cache_vector_04_amd.build``):
without it the first call into the binding raises ImportError (there is no
fallback path).  The import itself does not load it, so that tests which
import this module fail, rather than skip, when it is missing.
"""

import ctypes
import functools
import inspect
import os

import numpy as np
import torch  # loaded first so libtq.so binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED = 0, -1, -2
TQ_ERR_NOT_CONVERGED, TQ_ERR_HIP, TQ_ERR_WORKSPACE, TQ_ERR_TOO_LARGE = -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 16 << 20
TQ_MSE, TQ_PROD = 0, 1
TQ_F16, TQ_F32 = 0, 1

EXPORTS = ("tq_status_string", "tq_build_codebook", "tq_codec_init", "tq_encode_kv_workspace",
           "tq_encode_kv", "tq_decode_kv", "tq_encode_split", "tq_decode_split", "tq_attend_split",
           "tq_outlier_order",
           "tq_build_vq_codebook", "tq_vq_codec_init", "tq_vq_search_build", "tq_encode_vq",
           "tq_decode_vq",
           "tq_attend_decode_workspace", "tq_attend_decode", "tq_attend_decode_noalloc",
           "tq_inner_product_workspace", "tq_inner_product")


class TQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))
        self.status = status


class TQCodec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("mode", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("code_bits", ctypes.c_int32), ("m", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("centroids", ctypes.c_float * 16), ("thresholds", ctypes.c_float * 16),
                ("flip", ctypes.c_uint32 * 48), ("S", ctypes.c_void_p)]


class TQSplitCodec(ctypes.Structure):
    _fields_ = [("hi", TQCodec), ("lo", TQCodec)]


class TQVqCodec(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("n_codes", ctypes.c_int32), ("block_bits", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("codewords", ctypes.c_float * (2 * 256)),
                ("flip", ctypes.c_uint32 * 48), ("search", ctypes.c_void_p)]


class TQPacked(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("qjl", ctypes.c_void_p),
                ("norm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p)]


class TQRope(ctypes.Structure):
    _fields_ = [("base", ctypes.c_float), ("pos0", ctypes.c_int32), ("seq_len", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded libtq.so (raises ImportError if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtq.so is not built: run `python -m kv_cache_vector_04_amd.build` "
                          "(or __graft_entry__.build()) first; there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.tq_status_string.restype = ctypes.c_char_p
    L.tq_status_string.argtypes = [I]
    L.tq_build_codebook.restype = I
    L.tq_build_codebook.argtypes = [I, I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    L.tq_codec_init.restype = I
    L.tq_codec_init.argtypes = [ctypes.POINTER(TQCodec), I, I, I, ctypes.POINTER(ctypes.c_uint32), P]
    L.tq_encode_kv_workspace.restype = SZ
    L.tq_encode_kv_workspace.argtypes = [ctypes.POINTER(TQCodec), ctypes.POINTER(TQCodec), I64]
    L.tq_encode_kv.restype = I
    L.tq_encode_kv.argtypes = [ctypes.POINTER(TQCodec), ctypes.POINTER(TQCodec), P, P, I, I64,
                               ctypes.POINTER(TQRope), ctypes.POINTER(TQPacked),
                               ctypes.POINTER(TQPacked), P, SZ, P]
    L.tq_build_vq_codebook.restype = I
    L.tq_build_vq_codebook.argtypes = [I, I, ctypes.POINTER(ctypes.c_double)]
    L.tq_vq_codec_init.restype = I
    L.tq_vq_codec_init.argtypes = [ctypes.POINTER(TQVqCodec), I, I, ctypes.POINTER(ctypes.c_uint32)]
    L.tq_vq_search_build.restype = I
    L.tq_vq_search_build.argtypes = [ctypes.POINTER(TQVqCodec), P, SZ]
    L.tq_encode_vq.restype = I
    L.tq_encode_vq.argtypes = [ctypes.POINTER(TQVqCodec), P, I, I64, P, P, P]
    L.tq_decode_vq.restype = I
    L.tq_decode_vq.argtypes = [ctypes.POINTER(TQVqCodec), P, P, I64, P, I, P]
    L.tq_decode_kv.restype = I
    L.tq_decode_kv.argtypes = [ctypes.POINTER(TQCodec), ctypes.POINTER(TQPacked), I64, P, I, P]
    L.tq_outlier_order.restype = I
    L.tq_outlier_order.argtypes = [P, I64, I, I, P]
    L.tq_attend_split.restype = I
    L.tq_attend_split.argtypes = [ctypes.POINTER(TQSplitCodec), ctypes.POINTER(TQSplitCodec), P, I, I,
                                  I, I, I, ctypes.POINTER(TQPacked), ctypes.POINTER(TQPacked), I64,
                                  F, P, P, P, SZ, P]
    L.tq_encode_split.restype = I
    L.tq_encode_split.argtypes = [ctypes.POINTER(TQSplitCodec), ctypes.POINTER(TQSplitCodec), P, P, I,
                                  I64, ctypes.POINTER(TQPacked), ctypes.POINTER(TQPacked), P]
    L.tq_decode_split.restype = I
    L.tq_decode_split.argtypes = [ctypes.POINTER(TQSplitCodec), ctypes.POINTER(TQPacked), I64, P, I, P]
    L.tq_attend_decode_workspace.restype = SZ
    L.tq_attend_decode_workspace.argtypes = [I, I, I, I, I64, I]
    L.tq_attend_decode.restype = I
    L.tq_attend_decode.argtypes = [ctypes.POINTER(TQCodec), ctypes.POINTER(TQCodec), P, I, I, I, I, I,
                                   ctypes.POINTER(TQRope), ctypes.POINTER(TQPacked),
                                   ctypes.POINTER(TQPacked), I64, F, P, P, P, SZ, P]
    L.tq_attend_decode_noalloc.restype = I
    L.tq_attend_decode_noalloc.argtypes = [ctypes.POINTER(TQCodec), ctypes.POINTER(TQCodec), P, I, I, I,
                                           I, I, ctypes.POINTER(TQRope), ctypes.POINTER(TQPacked),
                                           ctypes.POINTER(TQPacked), I64, F, P, P, P]
    L.tq_inner_product_workspace.restype = SZ
    L.tq_inner_product_workspace.argtypes = [I64, I64, I, I]
    L.tq_inner_product.restype = I
    L.tq_inner_product.argtypes = [ctypes.POINTER(TQCodec), P, I, I64, ctypes.POINTER(TQPacked), I64,
                                   P, I, P, P, P, SZ, P]
    _lib = L
    return L


def status_string(status):
    return lib().tq_status_string(int(status)).decode()


def _check(status, what):
    if status != TQ_OK:
        raise TQError(status, what)


def build_codebook(d, bits):
    """Host Lloyd-Max table of the library: (centroids, thresholds) fp64."""
    n = 1 << bits
    c = (ctypes.c_double * n)()
    t = (ctypes.c_double * max(n - 1, 1))()
    _check(lib().tq_build_codebook(int(d), int(bits), c, t), "tq_build_codebook")
    return np.array(c[:], dtype=np.float64), np.array(t[:n - 1], dtype=np.float64)


def flip_words(flip):
    """bool sign-flip vector (True = -1) -> uint32 words, bit i%32 of word i/32."""
    flip = np.asarray(flip, dtype=bool)
    d = flip.shape[0]
    bits = np.zeros(((d + 31) // 32) * 32, dtype=np.uint8)
    bits[:d] = flip
    return np.packbits(bits.reshape(-1, 32), axis=1, bitorder="little").view(np.uint32).ravel()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _on_stream(fn):
    """A call given an explicit stream allocates its outputs and temporaries
    on that stream, so the caching allocator keeps them until the stream's
    work is done (a temporary freed on another stream could be reused while
    the kernels still read it).  `stream` is keyword-only in every wrapped
    call, so it cannot arrive positionally and bypass this."""
    if inspect.signature(fn).parameters["stream"].kind is not inspect.Parameter.KEYWORD_ONLY:
        raise TypeError("%s: stream must be keyword-only" % fn.__name__)

    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float16:
        return TQ_F16
    if t.dtype == torch.float32:
        return TQ_F32
    raise TypeError("vectors must be float16 or float32, got %s" % t.dtype)


def _device_tensor(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _out_tensor(t, name, shape, dtype):
    """A caller-given output buffer: CUDA, contiguous, of exactly `shape`
    and `dtype` (the kernels write that many elements through its pointer)."""
    _device_tensor(t, name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be a %s tensor of shape %s, got %s %s"
                         % (name, dtype, tuple(shape), t.dtype, tuple(t.shape)))
    return t


def _workspace(t, need, device):
    """The caller's workspace (CUDA uint8, at least `need` bytes), or a new
    one.  The kernels write every byte they read back, so it is not cleared."""
    if t is None:
        return torch.empty((max(need, 16),), dtype=torch.uint8, device=device)
    _device_tensor(t, "workspace")
    if t.numel() * t.element_size() < need:
        raise ValueError("workspace holds %d bytes, the call needs %d"
                         % (t.numel() * t.element_size(), need))
    return t


def _check_packed(pk, codec, n, name):
    """pk must be a Packed laid out for `codec` and hold at least n rows:
    the C ABI's tq_packed carries no row count, so this is the only place an
    undersized or mismatched buffer can be caught before a kernel runs."""
    if not isinstance(pk, Packed):
        raise ValueError("%s must be a Packed" % name)
    if pk.n < n:
        raise ValueError("%s holds %d rows, the call reads or writes %d" % (name, pk.n, n))
    row = codec.d * codec.code_bits // 8
    if pk.idx.dim() != 2 or pk.idx.shape[1] != row or pk.idx.dtype != torch.uint8:
        raise ValueError("%s.idx rows are not %d bytes (codec d=%d, %d-bit codes)"
                         % (name, row, codec.d, codec.code_bits))
    if (pk.qjl is None) != (codec.mode != TQ_PROD):
        raise ValueError("%s planes do not match the codec's mode" % name)
    planes = [("idx", pk.idx), ("norm", pk.norm)]
    if codec.mode == TQ_PROD:
        if pk.qjl.dim() != 2 or pk.qjl.shape[1] != codec.m // 8:
            raise ValueError("%s.qjl rows are not %d bytes" % (name, codec.m // 8))
        planes += [("qjl", pk.qjl), ("rnorm", pk.rnorm)]
    for what, t in planes:
        _device_tensor(t, "%s.%s" % (name, what))
        if t.shape[0] < pk.n:
            raise ValueError("%s.%s holds fewer than %d rows" % (name, what, pk.n))


def _check_split_packed(pk, codec, n, name):
    if not isinstance(pk, SplitPacked):
        raise ValueError("%s must be a SplitPacked" % name)
    _check_packed(pk.hi, codec.hi, n, name + ".hi")
    _check_packed(pk.lo, codec.lo, n, name + ".lo")


def _check_heads(hq, hkv, ctx):
    if hkv <= 0 or hq <= 0 or hq % hkv:
        raise ValueError("hq = %d must be a positive multiple of hkv = %d" % (hq, hkv))
    if ctx <= 0:
        raise ValueError("ctx must be positive")


class Codec:
    """One codec instance: dimension, mode, total bits, sign flip D and (prod)
    the QJL matrix S, held on the device."""

    def __init__(self, d, mode, bits, flip, S=None, device="cuda"):
        self.d, self.mode, self.bits = int(d), int(mode), int(bits)
        self.flip = np.asarray(flip, dtype=bool)
        self.S = None
        if mode == TQ_PROD:
            S = torch.as_tensor(S, dtype=torch.float32)
            self.S = S.to(device).contiguous() if S.device.type != "cuda" else S.contiguous()
        self.struct = TQCodec()
        words = flip_words(self.flip)
        wbuf = (ctypes.c_uint32 * len(words))(*[int(w) for w in words])
        _check(lib().tq_codec_init(ctypes.byref(self.struct), self.d, self.mode, self.bits, wbuf,
                                   _ptr(self.S)), "tq_codec_init")

    @property
    def code_bits(self):
        return self.struct.code_bits

    @property
    def m(self):
        return self.struct.m

    def centroids(self):
        return np.array(self.struct.centroids[:1 << self.code_bits], dtype=np.float32)

    def thresholds(self):
        return np.array(self.struct.thresholds[:(1 << self.code_bits) - 1], dtype=np.float32)


class Packed:
    """Packed planes of n vectors (device tensors)."""

    def __init__(self, codec, n, device="cuda"):
        self.n = int(n)
        row = codec.d * codec.code_bits // 8
        self.idx = torch.empty((self.n, row), dtype=torch.uint8, device=device)
        self.norm = torch.empty((self.n,), dtype=torch.float32, device=device)
        if codec.mode == TQ_PROD:
            self.qjl = torch.empty((self.n, codec.m // 8), dtype=torch.uint8, device=device)
            self.rnorm = torch.empty((self.n,), dtype=torch.float32, device=device)
        else:
            self.qjl = None
            self.rnorm = None
        self.struct = TQPacked(_ptr(self.idx).value, _ptr(self.qjl).value, _ptr(self.norm).value,
                               _ptr(self.rnorm).value)


def encode_workspace_bytes(kcodec, vcodec, n):
    return int(lib().tq_encode_kv_workspace(ctypes.byref(kcodec.struct) if kcodec else None,
                                            ctypes.byref(vcodec.struct) if vcodec else None,
                                            int(n)))


@_on_stream
def encode_kv(kcodec, vcodec, k, v, rope=None, kout=None, vout=None, workspace=None, *,
              stream=None):
    """Encode rows of k with kcodec and rows of v with vcodec (either side may
    be None).  k / v: device tensors [..., d], fp16 or fp32.  rope: None or
    (base, seq_len), applied to k.  workspace: None (allocated here when the
    codecs need one) or a device uint8 tensor.  Returns (kout, vout) Packed."""
    n = None
    dt = None
    for c, x in ((kcodec, k), (vcodec, v)):
        if c is None:
            continue
        _device_tensor(x, "input")
        if x.shape[-1] != c.d:
            raise ValueError("last dimension must be d=%d" % c.d)
        rows = x.numel() // c.d
        n = rows if n is None else n
        if rows != n:
            raise ValueError("k and v must hold the same number of rows")
        d2 = _dtype_code(x)
        dt = d2 if dt is None else dt
        if d2 != dt:
            raise ValueError("k and v must share a dtype")
    if n is None:
        raise ValueError("encode_kv needs at least one codec")
    dev = (k if kcodec is not None else v).device
    if kcodec is not None:
        if kout is None:
            kout = Packed(kcodec, n, dev)
        _check_packed(kout, kcodec, n, "kout")
    if vcodec is not None:
        if vout is None:
            vout = Packed(vcodec, n, dev)
        _check_packed(vout, vcodec, n, "vout")
    r = None
    if rope is not None:
        r = TQRope(float(rope[0]), 0, int(rope[1]))
    need = encode_workspace_bytes(kcodec, vcodec, n)
    if workspace is not None or need > 0:
        workspace = _workspace(workspace, need, dev)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().tq_encode_kv(ctypes.byref(kcodec.struct) if kcodec else None,
                            ctypes.byref(vcodec.struct) if vcodec else None,
                            _ptr(k) if kcodec else None, _ptr(v) if vcodec else None, dt, n,
                            ctypes.byref(r) if r is not None else None,
                            ctypes.byref(kout.struct) if kcodec else None,
                            ctypes.byref(vout.struct) if vcodec else None, _ptr(workspace),
                            wbytes, _stream(stream))
    _check(st, "tq_encode_kv")
    return kout, vout


def build_vq_codebook(d, n_codes):
    """The library's FibQuant k = 2 codebook: (n_codes, 2) fp64."""
    cw = (ctypes.c_double * (2 * n_codes))()
    _check(lib().tq_build_vq_codebook(int(d), int(n_codes), cw), "tq_build_vq_codebook")
    return np.array(cw[:], dtype=np.float64).reshape(n_codes, 2)


VQ_SEARCH_BYTES = 16 + 2 * (64 * 64 + 8) + 24576


class VQCodec:
    """FibQuant k = 2 codec: N codewords on the unit disk for 2-coordinate
    blocks, log2(N) / 2 bits per coordinate.  With `search` the encoder's
    cell table is built on the host and kept on `device` (the encoder then
    tests each block against its cell's candidates only).  By default the
    table is used from N = 64 up, where it is faster than testing all N
    codewords (both give the same codes)."""

    def __init__(self, d, n_codes, flip, search=None, device="cuda"):
        if search is None:
            search = int(n_codes) >= 64
        self.d, self.n_codes = int(d), int(n_codes)
        self.block_bits = int(round(np.log2(n_codes)))
        self.struct = TQVqCodec()
        words = flip_words(flip)
        w = (ctypes.c_uint32 * 48)(*[int(x) for x in words])
        _check(lib().tq_vq_codec_init(ctypes.byref(self.struct), self.d, self.n_codes, w),
               "tq_vq_codec_init")
        self.search_table = None
        self.search_dev = None
        if search:
            self.search_table = np.zeros(VQ_SEARCH_BYTES, dtype=np.uint8)
            _check(lib().tq_vq_search_build(ctypes.byref(self.struct),
                                            self.search_table.ctypes.data_as(ctypes.c_void_p),
                                            VQ_SEARCH_BYTES), "tq_vq_search_build")
            self.search_dev = torch.from_numpy(self.search_table).to(device)
            self.struct.search = _ptr(self.search_dev).value

    @property
    def row_bytes(self):
        return self.d // 2 * self.block_bits // 8


@_on_stream
def encode_vq(codec, x, idx=None, norm=None, *, stream=None):
    """x: device [n, d] fp16/fp32 -> (idx [n, row_bytes] uint8, norm [n] fp32)."""
    _device_tensor(x, "x")
    if x.shape[-1] != codec.d:
        raise ValueError("last dimension must be d=%d" % codec.d)
    n = x.numel() // codec.d
    if idx is None:
        idx = torch.empty((n, codec.row_bytes), dtype=torch.uint8, device=x.device)
    if norm is None:
        norm = torch.empty((n,), dtype=torch.float32, device=x.device)
    _out_tensor(idx, "idx", (n, codec.row_bytes), torch.uint8)
    _out_tensor(norm, "norm", (n,), torch.float32)
    st = lib().tq_encode_vq(ctypes.byref(codec.struct), _ptr(x), _dtype_code(x), n, _ptr(idx),
                            _ptr(norm), _stream(stream))
    _check(st, "tq_encode_vq")
    return idx, norm


@_on_stream
def decode_vq(codec, idx, norm, n, dtype=None, out=None, *, stream=None):
    """Block codes back to vectors: out [n, d] (float16 unless dtype / out say float32)."""
    _device_tensor(idx, "idx")
    _device_tensor(norm, "norm")
    if idx.dim() != 2 or idx.shape[0] < n or idx.shape[1] != codec.row_bytes or norm.numel() < n \
            or idx.dtype != torch.uint8 or norm.dtype != torch.float32:
        raise ValueError("idx must hold n x %d uint8 and norm n float32" % codec.row_bytes)
    if out is None:
        out = torch.empty((n, codec.d), dtype=dtype if dtype is not None else torch.float16,
                          device=idx.device)
    _device_tensor(out, "out")
    if out.numel() != n * codec.d:
        raise ValueError("out must hold n x d elements")
    st = lib().tq_decode_vq(ctypes.byref(codec.struct), _ptr(idx), _ptr(norm), int(n), _ptr(out),
                            _dtype_code(out), _stream(stream))
    _check(st, "tq_decode_vq")
    return out


@_on_stream
def decode_kv(codec, pk, n, dtype=None, out=None, *, stream=None):
    """Packed rows back to vectors: returns out [n, d] (float16 unless dtype
    or out says float32)."""
    _check_packed(pk, codec, n, "pk")
    if out is None:
        dt = dtype if dtype is not None else torch.float16
        out = torch.empty((n, codec.d), dtype=dt, device=pk.idx.device)
    _device_tensor(out, "out")
    if out.numel() != n * codec.d:
        raise ValueError("out must hold n x d elements")
    st = lib().tq_decode_kv(ctypes.byref(codec.struct), ctypes.byref(pk.struct), int(n), _ptr(out),
                            _dtype_code(out), _stream(stream))
    _check(st, "tq_decode_kv")
    return out


class SplitCodec:
    """Outlier-channel split: channels [0, 64) of each 128-channel row through
    `hi` (a Codec of d = 64, more bits), channels [64, 128) through `lo`."""

    def __init__(self, hi, lo):
        if hi.d != 64 or lo.d != 64 or hi.mode != lo.mode:
            raise ValueError("a split codec pairs two d = 64 codecs of one mode")
        self.hi, self.lo = hi, lo
        self.d, self.mode = 128, hi.mode
        self.struct = TQSplitCodec(hi.struct, lo.struct)

    @property
    def bits_per_channel(self):
        return (self.hi.bits + self.lo.bits) / 2.0


def outlier_order(calib, d_hi):
    """The library's outlier-first channel order for calibration rows
    (host array n x d): int32 array of d channels."""
    x = np.ascontiguousarray(np.asarray(calib, dtype=np.float32))
    n, d = x.shape
    order = np.empty(d, dtype=np.int32)
    _check(lib().tq_outlier_order(x.ctypes.data_as(ctypes.c_void_p), n, d, int(d_hi),
                                  order.ctypes.data_as(ctypes.c_void_p)), "tq_outlier_order")
    return order


class SplitPacked:
    """The two halves' packed planes of n rows."""

    def __init__(self, codec, n, device="cuda"):
        self.n = int(n)
        self.hi = Packed(codec.hi, n, device)
        self.lo = Packed(codec.lo, n, device)
        self.structs = (TQPacked * 2)(self.hi.struct, self.lo.struct)


@_on_stream
def encode_split(kcodec, vcodec, k, v, kout=None, vout=None, *, stream=None):
    """Encode [..., 128] rows of k with the split codec kcodec and of v with
    vcodec (either may be None).  Returns (kout, vout) SplitPacked."""
    n = dt = None
    for c, x in ((kcodec, k), (vcodec, v)):
        if c is None:
            continue
        _device_tensor(x, "input")
        if x.shape[-1] != 128:
            raise ValueError("split rows hold 128 channels")
        rows = x.numel() // 128
        n = rows if n is None else n
        if rows != n:
            raise ValueError("k and v must hold the same number of rows")
        d2 = _dtype_code(x)
        dt = d2 if dt is None else dt
        if d2 != dt:
            raise ValueError("k and v must share a dtype")
    if n is None:
        raise ValueError("encode_split needs at least one codec")
    dev = (k if kcodec is not None else v).device
    if kcodec is not None:
        if kout is None:
            kout = SplitPacked(kcodec, n, dev)
        _check_split_packed(kout, kcodec, n, "kout")
    if vcodec is not None:
        if vout is None:
            vout = SplitPacked(vcodec, n, dev)
        _check_split_packed(vout, vcodec, n, "vout")
    st = lib().tq_encode_split(ctypes.byref(kcodec.struct) if kcodec else None,
                               ctypes.byref(vcodec.struct) if vcodec else None,
                               _ptr(k) if kcodec else None, _ptr(v) if vcodec else None, dt, n,
                               kout.structs if kcodec else None, vout.structs if vcodec else None,
                               _stream(stream))
    _check(st, "tq_encode_split")
    return kout, vout


@_on_stream
def decode_split(codec, pk, n, dtype=None, out=None, *, stream=None):
    """Both halves back to [n, 128] rows (float16 unless dtype / out say float32)."""
    _check_split_packed(pk, codec, n, "pk")
    if out is None:
        dt = dtype if dtype is not None else torch.float16
        out = torch.empty((n, 128), dtype=dt, device=pk.hi.idx.device)
    _device_tensor(out, "out")
    if out.numel() != n * 128:
        raise ValueError("out must hold n x 128 elements")
    st = lib().tq_decode_split(ctypes.byref(codec.struct), pk.structs, int(n), _ptr(out),
                               _dtype_code(out), _stream(stream))
    _check(st, "tq_decode_split")
    return out


@_on_stream
def attend_split(kcodec, vcodec, q, kpk, vpk, ctx, hkv, scale=0.0, out=None, scores_out=None,
                 workspace=None, *, stream=None):
    """Attention of q [batch, hq, n_q, 128] over split codes (SplitPacked with
    rows [batch][hkv][ctx]); returns out [batch, hq, n_q, 128] fp32."""
    _device_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [batch, hq, n_q, 128]")
    batch, hq, n_q, d = q.shape
    if d != 128:
        raise ValueError("split attention takes 128 channels")
    _check_heads(hq, hkv, ctx)
    _check_split_packed(kpk, kcodec, batch * hkv * ctx, "kpk")
    _check_split_packed(vpk, vcodec, batch * hkv * ctx, "vpk")
    if out is None:
        out = torch.empty((batch, hq, n_q, d), dtype=torch.float32, device=q.device)
    _out_tensor(out, "out", (batch, hq, n_q, d), torch.float32)
    if scores_out is not None:
        _out_tensor(scores_out, "scores_out", (batch, hq, n_q, ctx), torch.float32)
    workspace = _workspace(workspace, attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d), q.device)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib().tq_attend_split(ctypes.byref(kcodec.struct), ctypes.byref(vcodec.struct), _ptr(q),
                               _dtype_code(q), batch, n_q, hq, hkv, kpk.structs, vpk.structs,
                               int(ctx), float(scale), _ptr(out), _ptr(scores_out), _ptr(workspace),
                               wbytes, _stream(stream))
    _check(st, "tq_attend_split")
    return out


def attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d):
    return int(lib().tq_attend_decode_workspace(batch, n_q, hq, hkv, ctx, d))


@_on_stream
def attend_decode(kcodec, vcodec, q, kpk, vpk, ctx, hkv, scale=0.0, rope=None, out=None,
                  want_scores=False, workspace=None, *, stream=None):
    """Attention from codes.  q: device [batch, hq, n_q, d] fp16/fp32; kpk,
    vpk: Packed rows [batch][hkv][ctx].  rope: None or (base, pos0).
    Returns out [batch, hq, n_q, d] fp32 (and scores [batch, hq, n_q, ctx])."""
    _device_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [batch, hq, n_q, d]")
    batch, hq, n_q, d = q.shape
    if d != kcodec.d or d != vcodec.d:
        raise ValueError("q rows hold %d elements, the codecs d = %d / %d" % (d, kcodec.d, vcodec.d))
    _check_heads(hq, hkv, ctx)
    _check_packed(kpk, kcodec, batch * hkv * ctx, "kpk")
    _check_packed(vpk, vcodec, batch * hkv * ctx, "vpk")
    if out is None:
        out = torch.empty((batch, hq, n_q, d), dtype=torch.float32, device=q.device)
    _out_tensor(out, "out", (batch, hq, n_q, d), torch.float32)
    scores = None
    if want_scores:
        scores = torch.empty((batch, hq, n_q, ctx), dtype=torch.float32, device=q.device)
    workspace = _workspace(workspace, attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d), q.device)
    r = TQRope(float(rope[0]), int(rope[1]), 0) if rope is not None else None
    st = lib().tq_attend_decode(ctypes.byref(kcodec.struct), ctypes.byref(vcodec.struct), _ptr(q),
                                _dtype_code(q), batch, n_q, hq, hkv,
                                ctypes.byref(r) if r is not None else None,
                                ctypes.byref(kpk.struct), ctypes.byref(vpk.struct), int(ctx),
                                float(scale), _ptr(out), _ptr(scores), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tq_attend_decode")
    return (out, scores) if want_scores else out


@_on_stream
def attend_decode_noalloc(kcodec, vcodec, q, kpk, vpk, ctx, hkv, out, scale=0.0, rope=None,
                          scores_out=None, *, stream=None):
    """attend_decode through the library's allocation-free entry point: no
    workspace (the kernels use the library's fixed per-GPU scratch), and the
    caller passes the output (and optional scores) buffers, so this call
    allocates nothing either.  Calls that overlap in time on one GPU race."""
    _device_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [batch, hq, n_q, d]")
    batch, hq, n_q, d = q.shape
    if d != kcodec.d or d != vcodec.d:
        raise ValueError("q rows hold %d elements, the codecs d = %d / %d" % (d, kcodec.d, vcodec.d))
    _check_heads(hq, hkv, ctx)
    _check_packed(kpk, kcodec, batch * hkv * ctx, "kpk")
    _check_packed(vpk, vcodec, batch * hkv * ctx, "vpk")
    _out_tensor(out, "out", (batch, hq, n_q, d), torch.float32)
    if scores_out is not None:
        _out_tensor(scores_out, "scores_out", (batch, hq, n_q, ctx), torch.float32)
    r = TQRope(float(rope[0]), int(rope[1]), 0) if rope is not None else None
    st = lib().tq_attend_decode_noalloc(ctypes.byref(kcodec.struct), ctypes.byref(vcodec.struct),
                                        _ptr(q), _dtype_code(q), batch, n_q, hq, hkv,
                                        ctypes.byref(r) if r is not None else None,
                                        ctypes.byref(kpk.struct), ctypes.byref(vpk.struct),
                                        int(ctx), float(scale), _ptr(out), _ptr(scores_out),
                                        _stream(stream))
    _check(st, "tq_attend_decode_noalloc")
    return out


def inner_product_workspace_bytes(n_q, n, d, top_k):
    return int(lib().tq_inner_product_workspace(n_q, n, d, top_k))


@_on_stream
def inner_product(codec, q, pk, n, top_k=0, want_matrix=True, workspace=None, out_ids=None,
                  out_vals=None, *, stream=None):
    """Estimated inner products of q [n_q, d] against n packed rows.  Returns
    the [n_q, n] matrix (if want_matrix) and, for top_k > 0, (ids, scores)
    (written into out_ids / out_vals when given)."""
    _device_tensor(q, "q")
    if q.dim() != 2 or q.shape[1] != codec.d:
        raise ValueError("q must be [n_q, %d]" % codec.d)
    n_q, d = q.shape
    _check_packed(pk, codec, n, "pk")
    out = torch.empty((n_q, n), dtype=torch.float32, device=q.device) if want_matrix else None
    ids = vals = None
    if top_k:
        ids = out_ids if out_ids is not None else \
            torch.empty((n_q, top_k), dtype=torch.int64, device=q.device)
        vals = out_vals if out_vals is not None else \
            torch.empty((n_q, top_k), dtype=torch.float32, device=q.device)
        _device_tensor(ids, "out_ids")
        _device_tensor(vals, "out_vals")
        if ids.shape != (n_q, top_k) or vals.shape != (n_q, top_k) or ids.dtype != torch.int64 \
                or vals.dtype != torch.float32:
            raise ValueError("out_ids / out_vals must be [n_q, top_k] int64 / float32")
    workspace = _workspace(workspace, inner_product_workspace_bytes(n_q, n, d, top_k), q.device)
    st = lib().tq_inner_product(ctypes.byref(codec.struct), _ptr(q), _dtype_code(q), n_q,
                                ctypes.byref(pk.struct), int(n), _ptr(out), int(top_k), _ptr(ids),
                                _ptr(vals), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "tq_inner_product")
    if top_k:
        return out, ids, vals
    return out
