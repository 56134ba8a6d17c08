"""Python binding of ``libtq`` (the MI355X online KV-cache vector quantizer).

Argument marshalling only: every step of the method runs in the HIP kernels
behind the C ABI of ``include/tq.h``.  PyTorch provides device memory and the
current stream.  The library is loaded from ``lib/libtq.so`` inside this
package (built by ``build.build_library()`` / ``__graft_entry__.build()``);
importing this module raises if it is missing - there is no fallback.

Method: page "TurboQuant 설명: 무엇인지와 LLM 메모리 6배 절약 구현 방법"
(sections "1단계: 무작위 회전 + PolarQuant 압축", "2단계: QJL 잔차 보정",
"TurboQuant 구현 방법").
"""

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_NO_CONVERGENCE = -3
TQ_ERR_HIP = -4
MODE_MSE = 0
MODE_PROD = 1
MODE_POLAR = 2
TQ_F32 = 0
TQ_BF16 = 1
KIND_PI = 0
KIND_S = 1
KIND_M = 2

EXPORTED = ["tq_make_codebook", "tq_make_polar_codebook", "tq_make_rotation", "tq_quantize_kv",
            "tq_attn_logits_workspace_size", "tq_attn_logits", "tq_append_attn_logits", "tq_attn_logits_paged",
            "tq_append_attn_logits_paged", "tq_prepare_queries", "tq_attn_logits_prepared",
            "tq_attn_output_workspace_size", "tq_attn_output", "tq_attn_output_noalloc", "tq_dequantize",
            "tq_probe_sink_words", "tq_probe", "tq_status_string"]
PROBE_READ, PROBE_WRITE, PROBE_MFMA_F16, PROBE_MFMA_I8 = 0, 1, 2, 3
NOALLOC_SCRATCH_BYTES = 4 << 20


class TQError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))


class Params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("pi", ctypes.c_void_p), ("qjl", ctypes.c_void_p),
                ("qjl_rot", ctypes.c_void_p), ("centroids", ctypes.c_void_p),
                ("boundaries", ctypes.c_void_p)]


class Packed(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("norm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p)]


class Pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("page_tokens", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("n_pages", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtq.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.tq_make_codebook.argtypes = [i32, i32, vp, vp, vp]
    lib.tq_make_polar_codebook.argtypes = [i32, vp, vp]
    lib.tq_make_rotation.argtypes = [i32, ctypes.c_uint64, i32, vp]
    lib.tq_quantize_kv.argtypes = [ctypes.POINTER(Params), vp, i32, i64, i64, ctypes.POINTER(Packed),
                                   i64, vp]
    sz, psz = ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
    lib.tq_attn_logits_workspace_size.argtypes = [ctypes.POINTER(Params), i32, i32, i32, i64, i32, psz]
    lib.tq_attn_logits.argtypes = [ctypes.POINTER(Params), vp, i32, i32, i32, i32,
                                   ctypes.POINTER(Packed), i64, i64, f32, vp, i32, vp, vp, sz, vp]
    lib.tq_append_attn_logits.argtypes = [ctypes.POINTER(Params), vp, i32, vp, i32, i32, i32, i32,
                                          ctypes.POINTER(Packed), i64, i64, f32, vp, vp, sz, vp]
    lib.tq_attn_logits_paged.argtypes = [ctypes.POINTER(Params), vp, i32, i32, i32, i32, ctypes.POINTER(Packed),
                                         ctypes.POINTER(Pages), i64, f32, vp, vp, sz, vp]
    lib.tq_append_attn_logits_paged.argtypes = [ctypes.POINTER(Params), vp, i32, vp, i32, i32, i32, i32,
                                                ctypes.POINTER(Packed), ctypes.POINTER(Pages), i64, f32, vp, vp, sz,
                                                vp]
    lib.tq_prepare_queries.argtypes = [ctypes.POINTER(Params), vp, i32, i32, i32, i32, vp, sz, vp]
    lib.tq_attn_logits_prepared.argtypes = [ctypes.POINTER(Params), i32, i32, i32, ctypes.POINTER(Packed), i64,
                                            ctypes.POINTER(Pages), i64, f32, vp, vp, sz, vp]
    lib.tq_attn_output_workspace_size.argtypes = [ctypes.POINTER(Params), i32, i32, i32, i64, psz]
    lib.tq_attn_output.argtypes = [ctypes.POINTER(Params), vp, i32, i32, i32, ctypes.POINTER(Packed),
                                   i64, i64, vp, i32, vp, sz, vp]
    lib.tq_attn_output_noalloc.argtypes = [ctypes.POINTER(Params), vp, i32, i32, i32, ctypes.POINTER(Packed),
                                           i64, i64, vp, i32, vp]
    lib.tq_dequantize.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Packed), i64, vp, i32, vp]
    lib.tq_probe_sink_words.argtypes = [ctypes.POINTER(i64)]
    lib.tq_probe.argtypes = [i32, vp, i64, i32, vp, i64, vp]
    lib.tq_status_string.argtypes = [i32]
    lib.tq_status_string.restype = ctypes.c_char_p
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = i32
    return lib


LIB = _load()


def status_string(status):
    return LIB.tq_status_string(int(status)).decode()


def _check(status, what):
    if status != TQ_OK:
        raise TQError(status, what)


def lloyd_bits(bits, mode):
    return bits if mode == MODE_MSE else bits - 1


def make_polar_codebook(d):
    """Angle codebooks of levels 2..log2(d) of the polar format: (centroids [L-1, 4], boundaries [L-1, 3])."""
    nl = int(round(math.log2(d))) - 1
    c = np.zeros(4 * nl)
    t = np.zeros(3 * nl)
    _check(LIB.tq_make_polar_codebook(d, c.ctypes.data, t.ctypes.data), "tq_make_polar_codebook")
    return c.reshape(nl, 4), t.reshape(nl, 3)


# ------------------------------------------------------------------ host math
def make_codebook(d, lloyd_bits_):
    """(centroids, boundaries, mse_per_coord) from the library (fp64, host)."""
    k = 1 << lloyd_bits_
    c = np.zeros(k)
    t = np.zeros(k - 1)
    mse = np.zeros(1)
    _check(LIB.tq_make_codebook(d, lloyd_bits_, c.ctypes.data, t.ctypes.data, mse.ctypes.data),
           "tq_make_codebook")
    return c, t, float(mse[0])


def make_rotation(d, seed, kind):
    """d x d fp64 matrix: KIND_PI, KIND_S or KIND_M (host)."""
    out = np.zeros((d, d))
    _check(LIB.tq_make_rotation(d, seed, kind, out.ctypes.data), "tq_make_rotation")
    return out


# ------------------------------------------------------------------ device side
def _torch():
    import torch
    return torch


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError("tensor dtype must be float32 or bfloat16, got %s" % t.dtype)


class PackedKV:
    """Device SoA buffers of ``capacity`` packed vectors."""

    def __init__(self, d, bits, mode, capacity, device="cuda"):
        torch = _torch()
        self.d, self.bits, self.mode, self.capacity = d, bits, mode, capacity
        # b bits per coordinate: b' Lloyd-Max planes (+ the QJL sign plane)
        self.codes = torch.empty((capacity, bits * d // 8), dtype=torch.uint8, device=device)
        self.norm = torch.empty((capacity,), dtype=torch.int16, device=device)
        self.rnorm = torch.empty((capacity,), dtype=torch.int16, device=device) \
            if mode == MODE_PROD else None

    @classmethod
    def from_tensors(cls, d, bits, mode, codes, norm, rnorm=None):
        obj = cls.__new__(cls)
        obj.d, obj.bits, obj.mode, obj.capacity = d, bits, mode, codes.shape[0]
        obj.codes, obj.norm, obj.rnorm = codes, norm, rnorm
        return obj

    def struct(self):
        return Packed(self.codes.data_ptr(), self.norm.data_ptr(),
                      self.rnorm.data_ptr() if self.rnorm is not None else None)

    def bytes_per_vector(self):
        return self.bits * self.d // 8 + (4 if self.mode == MODE_PROD else 2)


class PreparedQueries:
    """Query tables written by Quantizer.prepare_queries (device workspace)
    and the shape they were prepared for."""

    def __init__(self, workspace, batch, n_q_heads, n_kv_heads):
        self.workspace, self.batch, self.n_q_heads, self.n_kv_heads = workspace, batch, n_q_heads, n_kv_heads


class Quantizer:
    """Tables of one (d, bits, mode, seed) quantizer on a device.

    The host library builds the Lloyd-Max codebook and the seeded Pi, S and
    M = S Pi^T in fp64; fp32 copies live in device memory.
    """

    def __init__(self, d, bits, mode, seed=0, device="cuda"):
        torch = _torch()
        self.d, self.bits, self.mode, self.seed = d, bits, mode, seed
        self.device = torch.device(device)
        if mode == MODE_POLAR:
            if bits != 3:
                raise ValueError("the polar format has 3 bits per coordinate")
            c2, t2 = make_polar_codebook(d)
            c, t, self.mse_per_coord = c2.reshape(-1), t2.reshape(-1), None
        else:
            lb = lloyd_bits(bits, mode)
            c, t, self.mse_per_coord = make_codebook(d, lb)
        self.centroids64, self.boundaries64 = c, t
        self.pi64 = make_rotation(d, seed, KIND_PI)
        f = dict(dtype=torch.float32, device=self.device)
        self.pi = torch.tensor(self.pi64, **f)
        self.centroids = torch.tensor(c, **f)
        self.boundaries = torch.tensor(t, **f)
        if mode == MODE_PROD:
            self.s64 = make_rotation(d, seed, KIND_S)
            self.m64 = make_rotation(d, seed, KIND_M)
            self.s = torch.tensor(self.s64, **f)
            self.m = torch.tensor(self.m64, **f)
        else:
            self.s64 = self.m64 = self.s = self.m = None
        self._params = Params(d, bits, mode, 0, self.pi.data_ptr(),
                              self.s.data_ptr() if self.s is not None else None,
                              self.m.data_ptr() if self.m is not None else None,
                              self.centroids.data_ptr(), self.boundaries.data_ptr())
        self._ws = {}       # stream handle -> uint8 device tensor (workspace of the calls on it)

    def logits_workspace_size(self, batch, n_q_heads, n_kv_heads, seq_len, topk=0):
        """Bytes of device scratch tq_attn_logits needs for this shape."""
        n = ctypes.c_size_t(0)
        _check(LIB.tq_attn_logits_workspace_size(ctypes.byref(self._params), batch, n_q_heads, n_kv_heads,
                                                 seq_len, topk, ctypes.byref(n)), "tq_attn_logits_workspace_size")
        return n.value

    def attn_output_workspace_size(self, batch, n_q_heads, n_kv_heads, seq_len):
        """Bytes of device scratch tq_attn_output needs for this shape."""
        n = ctypes.c_size_t(0)
        _check(LIB.tq_attn_output_workspace_size(ctypes.byref(self._params), batch, n_q_heads, n_kv_heads,
                                                 seq_len, ctypes.byref(n)), "tq_attn_output_workspace_size")
        return n.value

    def _workspace(self, nbytes, workspace):
        """(pointer, bytes) of a workspace of at least nbytes: the caller's
        tensor, or a device buffer kept per stream (calls queued on one stream
        run in order, so they can share it)."""
        if workspace is not None:
            if workspace.numel() * workspace.element_size() < nbytes:
                raise ValueError("workspace holds %d bytes, the call needs %d"
                                 % (workspace.numel() * workspace.element_size(), nbytes))
            return ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
        if nbytes == 0:
            return None, 0
        torch = _torch()
        key = torch.cuda.current_stream(self.device).cuda_stream
        buf = self._ws.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws[key] = buf
        return ctypes.c_void_p(buf.data_ptr()), buf.numel()

    def new_cache(self, capacity):
        return PackedKV(self.d, self.bits, self.mode, capacity, self.device)

    def quantize(self, x, out=None, out_offset=0):
        """Quantise rows of x [n, d] (fp32 or bf16, CUDA) into ``out``."""
        n = x.shape[0]
        if x.dim() != 2 or x.shape[1] != self.d:
            raise ValueError("x must be [n, %d]" % self.d)
        if out is None:
            out = self.new_cache(n)
        st = LIB.tq_quantize_kv(ctypes.byref(self._params), ctypes.c_void_p(x.data_ptr()),
                                _dtype_code(x), n, x.stride(0), ctypes.byref(out.struct()),
                                out_offset, _stream_ptr(self.device))
        _check(st, "tq_quantize_kv")
        return out

    def attn_logits(self, q, cache, n_kv_heads, seq_len, scale, row_tokens=None, out=None, workspace=None):
        """Dense logits [batch, n_q_heads, seq_len] (fp32)."""
        torch = _torch()
        bsz, hq, _ = q.shape
        row_tokens = seq_len if row_tokens is None else row_tokens
        if out is None:
            out = torch.empty((bsz, hq, seq_len), dtype=torch.float32, device=self.device)
        ws, wsb = self._workspace(self.logits_workspace_size(bsz, hq, n_kv_heads, seq_len), workspace)
        st = LIB.tq_attn_logits(ctypes.byref(self._params), ctypes.c_void_p(q.data_ptr()),
                                _dtype_code(q), bsz, hq, n_kv_heads, ctypes.byref(cache.struct()),
                                row_tokens, seq_len, float(scale), ctypes.c_void_p(out.data_ptr()),
                                0, None, ws, wsb, _stream_ptr(self.device))
        _check(st, "tq_attn_logits")
        return out

    def append_attn_logits(self, x_new, q, cache, n_kv_heads, pos, scale, row_tokens=None, out=None,
                           workspace=None):
        """Quantise x_new [batch, n_kv_heads, d] into token ``pos`` of every stream of
        ``cache`` and return the logits [batch, n_q_heads, pos + 1] (fp32)."""
        torch = _torch()
        bsz, hq, _ = q.shape
        if row_tokens is None:            # the cache split evenly over the streams
            row_tokens = cache.capacity // max(bsz * n_kv_heads, 1)
        if out is None:
            out = torch.empty((bsz, hq, pos + 1), dtype=torch.float32, device=self.device)
        need = self.logits_workspace_size(bsz, hq, n_kv_heads, pos + 1) if 0 <= pos < row_tokens else 0
        ws, wsb = self._workspace(need, workspace)
        st = LIB.tq_append_attn_logits(ctypes.byref(self._params), ctypes.c_void_p(x_new.data_ptr()),
                                       _dtype_code(x_new), ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                       bsz, hq, n_kv_heads, ctypes.byref(cache.struct()), row_tokens, pos,
                                       float(scale), ctypes.c_void_p(out.data_ptr()), ws, wsb,
                                       _stream_ptr(self.device))
        _check(st, "tq_append_attn_logits")
        return out

    def _pages(self, block_table, page_tokens, n_pages):
        return Pages(block_table.data_ptr(), page_tokens, block_table.shape[1], n_pages)

    def attn_logits_paged(self, q, pool, block_table, page_tokens, n_kv_heads, seq_len, scale, out=None,
                          workspace=None):
        """Dense logits [batch, n_q_heads, seq_len] over a paged pool; block_table
        is an int32 device tensor [batch, max_pages]; the pool holds
        pool.capacity // (n_kv_heads * page_tokens) pages."""
        torch = _torch()
        bsz, hq, _ = q.shape
        if out is None:
            out = torch.empty((bsz, hq, seq_len), dtype=torch.float32, device=self.device)
        pg = self._pages(block_table, page_tokens, pool.capacity // (n_kv_heads * page_tokens))
        ws, wsb = self._workspace(self.logits_workspace_size(bsz, hq, n_kv_heads, seq_len), workspace)
        st = LIB.tq_attn_logits_paged(ctypes.byref(self._params), ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                      bsz, hq, n_kv_heads, ctypes.byref(pool.struct()), ctypes.byref(pg), seq_len,
                                      float(scale), ctypes.c_void_p(out.data_ptr()), ws, wsb,
                                      _stream_ptr(self.device))
        _check(st, "tq_attn_logits_paged")
        return out

    def append_attn_logits_paged(self, x_new, q, pool, block_table, page_tokens, n_kv_heads, pos, scale, out=None,
                                 workspace=None):
        """Quantise x_new [batch, n_kv_heads, d] into token ``pos`` of every
        sequence of a paged pool and return the logits [batch, n_q_heads, pos + 1]."""
        torch = _torch()
        bsz, hq, _ = q.shape
        if out is None:
            out = torch.empty((bsz, hq, pos + 1), dtype=torch.float32, device=self.device)
        pg = self._pages(block_table, page_tokens, pool.capacity // (n_kv_heads * page_tokens))
        ws, wsb = self._workspace(self.logits_workspace_size(bsz, hq, n_kv_heads, pos + 1) if pos >= 0 else 0,
                                  workspace)
        st = LIB.tq_append_attn_logits_paged(ctypes.byref(self._params), ctypes.c_void_p(x_new.data_ptr()),
                                             _dtype_code(x_new), ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                             bsz, hq, n_kv_heads, ctypes.byref(pool.struct()), ctypes.byref(pg), pos,
                                             float(scale), ctypes.c_void_p(out.data_ptr()), ws, wsb,
                                             _stream_ptr(self.device))
        _check(st, "tq_append_attn_logits_paged")
        return out

    def prepare_queries(self, q, n_kv_heads, workspace=None):
        """Run the query preparation of the dense logit call once; returns a
        PreparedQueries that attn_logits_prepared reads.  ``workspace`` (a
        uint8 device tensor) receives the tables; by default a new one."""
        torch = _torch()
        bsz, hq, _ = q.shape
        need = self.logits_workspace_size(bsz, hq, n_kv_heads, 1)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=self.device)
        ws, wsb = self._workspace(need, workspace)
        st = LIB.tq_prepare_queries(ctypes.byref(self._params), ctypes.c_void_p(q.data_ptr()), _dtype_code(q),
                                    bsz, hq, n_kv_heads, ws, wsb, _stream_ptr(self.device))
        _check(st, "tq_prepare_queries")
        return PreparedQueries(workspace, bsz, hq, n_kv_heads)

    def attn_logits_prepared(self, prepared, cache, seq_len, scale, row_tokens=None, out=None, block_table=None,
                             page_tokens=None):
        """Dense logits [batch, n_q_heads, seq_len] of prepared queries over a
        contiguous cache, or over a paged pool when block_table is given."""
        torch = _torch()
        bsz, hq, hkv = prepared.batch, prepared.n_q_heads, prepared.n_kv_heads
        if out is None:
            out = torch.empty((bsz, hq, seq_len), dtype=torch.float32, device=self.device)
        pg = None
        if block_table is not None:
            pg = ctypes.byref(self._pages(block_table, page_tokens, cache.capacity // (hkv * page_tokens)))
            row_tokens = 0
        elif row_tokens is None:
            row_tokens = seq_len
        ws = prepared.workspace
        st = LIB.tq_attn_logits_prepared(ctypes.byref(self._params), bsz, hq, hkv, ctypes.byref(cache.struct()),
                                         row_tokens, pg, seq_len, float(scale), ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                         _stream_ptr(self.device))
        _check(st, "tq_attn_logits_prepared")
        return out

    def search(self, q, cache, n_kv_heads, seq_len, topk, scale=1.0, row_tokens=None, workspace=None):
        """Top-k (scores, indices), each [batch, n_q_heads, topk]."""
        torch = _torch()
        bsz, hq, _ = q.shape
        row_tokens = seq_len if row_tokens is None else row_tokens
        vals = torch.empty((bsz, hq, topk), dtype=torch.float32, device=self.device)
        idx = torch.empty((bsz, hq, topk), dtype=torch.int32, device=self.device)
        ws, wsb = self._workspace(self.logits_workspace_size(bsz, hq, n_kv_heads, seq_len, topk), workspace)
        st = LIB.tq_attn_logits(ctypes.byref(self._params), ctypes.c_void_p(q.data_ptr()),
                                _dtype_code(q), bsz, hq, n_kv_heads, ctypes.byref(cache.struct()),
                                row_tokens, seq_len, float(scale), ctypes.c_void_p(vals.data_ptr()),
                                topk, ctypes.c_void_p(idx.data_ptr()), ws, wsb, _stream_ptr(self.device))
        _check(st, "tq_attn_logits(topk)")
        return vals, idx

    def attn_output(self, logits, cache, n_kv_heads, seq_len, row_tokens=None, out_dtype=None, out=None,
                    workspace=None):
        """Decode attention output [batch, n_q_heads, d]: softmax(logits) . values."""
        torch = _torch()
        bsz, hq, _ = logits.shape
        row_tokens = seq_len if row_tokens is None else row_tokens
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((bsz, hq, self.d), dtype=out_dtype, device=self.device)
        ws, wsb = self._workspace(self.attn_output_workspace_size(bsz, hq, n_kv_heads, seq_len), workspace)
        st = LIB.tq_attn_output(ctypes.byref(self._params), ctypes.c_void_p(logits.data_ptr()), bsz, hq,
                                n_kv_heads, ctypes.byref(cache.struct()), row_tokens, seq_len,
                                ctypes.c_void_p(out.data_ptr()), _dtype_code(out), ws, wsb,
                                _stream_ptr(self.device))
        _check(st, "tq_attn_output")
        return out

    def attn_output_noalloc(self, logits, cache, n_kv_heads, seq_len, out, row_tokens=None):
        """attn_output into ``out`` with no workspace: the library's fixed
        device array holds the partials (see tq_attn_output_noalloc)."""
        bsz, hq, _ = logits.shape
        row_tokens = seq_len if row_tokens is None else row_tokens
        st = LIB.tq_attn_output_noalloc(ctypes.byref(self._params), ctypes.c_void_p(logits.data_ptr()), bsz, hq,
                                        n_kv_heads, ctypes.byref(cache.struct()), row_tokens, seq_len,
                                        ctypes.c_void_p(out.data_ptr()), _dtype_code(out), _stream_ptr(self.device))
        _check(st, "tq_attn_output_noalloc")
        return out

    def dequantize(self, cache, n_vec, out_dtype=None, out=None):
        """Reconstructed vectors [n_vec, d] (fp32 or bf16)."""
        torch = _torch()
        out_dtype = torch.float32 if out_dtype is None else out_dtype
        if out is None:
            out = torch.empty((n_vec, self.d), dtype=out_dtype, device=self.device)
        st = LIB.tq_dequantize(ctypes.byref(self._params), ctypes.byref(cache.struct()), n_vec,
                               ctypes.c_void_p(out.data_ptr()), _dtype_code(out),
                               _stream_ptr(self.device))
        _check(st, "tq_dequantize")
        return out


def probe(kind, buf=None, iters=0, device="cuda"):
    """One launch of a ceiling probe (tq_probe) on the current stream: a
    read or write stream over the uint8 device tensor ``buf``, or an MFMA loop
    of ``iters`` steps.  Returns the work of the launch: bytes, or flops."""
    torch = _torch()
    n = ctypes.c_int64(0)
    _check(LIB.tq_probe_sink_words(ctypes.byref(n)), "tq_probe_sink_words")
    key = (str(device), n.value)
    sink = _PROBE_SINKS.get(key)
    if sink is None:
        sink = torch.zeros(n.value, dtype=torch.int32, device=device)
        _PROBE_SINKS[key] = sink
    nbytes = buf.numel() * buf.element_size() if buf is not None else 0
    _check(LIB.tq_probe(kind, ctypes.c_void_p(buf.data_ptr()) if buf is not None else None, nbytes, iters,
                        ctypes.c_void_p(sink.data_ptr()), n.value, _stream_ptr(torch.device(device))), "tq_probe")
    if kind in (PROBE_READ, PROBE_WRITE):
        return nbytes
    return n.value * iters * 4 * 32768


_PROBE_SINKS = {}


def default_scale(d):
    return 1.0 / math.sqrt(d)
