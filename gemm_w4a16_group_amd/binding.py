"""Python binding of ``libw4a16.so``: argument marshalling only.

Every function takes torch tensors on the current HIP device, checks dtype,
shape, device and contiguity, and forwards raw pointers and the current
stream to the C ABI declared in ``include/w4a16.h``.  All arithmetic runs in
the library's HIP kernels; there is no fallback path.  If the shared library
is missing, loading fails with an error naming the build command.
"""

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "w4a16.h")

GROUP = 128
KERNEL_SKINNY = 1
KERNEL_TILED = 2
KERNEL_NARROW = 3
LAYOUT_KN = 0      # x [K, N], c [M, N]
LAYOUT_TOKEN = 1   # x [N, K], c [N, M]

_lib = None
_lock = threading.Lock()


class W4A16Error(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status, message):
        super().__init__("w4a16 status %d: %s" % (status, message))
        self.status = status


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("ncol", ctypes.c_int32), ("rb", ctypes.c_int32),
                ("wm", ctypes.c_int32), ("wk", ctypes.c_int32), ("bm", ctypes.c_int32),
                ("bn", ctypes.c_int32), ("splitk", ctypes.c_int32), ("pf", ctypes.c_int32),
                ("xpf", ctypes.c_int32)]

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}

    @classmethod
    def make(cls, **kw):
        p = cls()
        for k, v in kw.items():
            setattr(p, k, int(v))
        return p


class Linear(ctypes.Structure):
    _fields_ = [("q_packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("z_packed", ctypes.c_void_p)]


class DecoderLayer(ctypes.Structure):
    _fields_ = [("qkv", Linear), ("o", Linear), ("gate_up", Linear), ("down", Linear),
                ("attn_norm", ctypes.c_void_p), ("mlp_norm", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


def load_library(path=None):
    """Load (once) and return the ctypes handle of libw4a16.so.

    With no path, the in-tree library is loaded on first use and kept as
    the handle every function of this module calls.  With a path, the
    library there is loaded and returned, and the module's handle is left
    as it was (functions here keep calling the in-tree library)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise ImportError("%s is not built; run `python -m gemm_w4a16_group_amd.build`" % p)
        lib = ctypes.CDLL(p)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        lib.w4a16_status_string.restype = ctypes.c_char_p
        lib.w4a16_status_string.argtypes = [ctypes.c_int]
        lib.w4a16_last_error.restype = ctypes.c_char_p
        lib.w4a16_last_error.argtypes = []
        lib.w4a16_version.restype = ctypes.c_int
        lib.w4a16_version.argtypes = []
        lib.w4a16_pack.restype = ctypes.c_int
        lib.w4a16_pack.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
        lib.w4a16_gemv.restype = ctypes.c_int
        lib.w4a16_gemv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, vp]
        lib.w4a16_plan_default.restype = ctypes.c_int
        lib.w4a16_plan_default.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        lib.w4a16_workspace_size_plan.restype = sz
        lib.w4a16_workspace_size_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        lib.w4a16_gemm_workspace_size.restype = sz
        lib.w4a16_gemm_workspace_size.argtypes = [i64, i64, i64, i32]
        lib.w4a16_quantize.restype = ctypes.c_int
        lib.w4a16_quantize.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
        lib.w4a16_kernel_name.restype = ctypes.c_int
        lib.w4a16_kernel_name.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan), ctypes.c_char_p,
                                          ctypes.c_size_t]
        lib.w4a16_gemm.restype = ctypes.c_int
        lib.w4a16_gemm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
        lib.w4a16_gemm_plan.restype = ctypes.c_int
        lib.w4a16_gemm_plan.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32,
                                        ctypes.POINTER(Plan), vp, sz, vp]
        lib.w4a16_gemm_ex.restype = ctypes.c_int
        lib.w4a16_gemm_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32,
                                      ctypes.POINTER(Plan), vp, sz, vp]
        lib.w4a16_plan_default_ex.restype = ctypes.c_int
        lib.w4a16_plan_default_ex.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(Plan)]
        lib.w4a16_workspace_size_ex.restype = sz
        lib.w4a16_workspace_size_ex.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(Plan)]
        f32 = ctypes.c_float
        lib.w4a16_add_rmsnorm.restype = ctypes.c_int
        lib.w4a16_add_rmsnorm.argtypes = [vp, vp, vp, f32, vp, vp, i64, i64, vp]
        lib.w4a16_gemm_add_rmsnorm.restype = ctypes.c_int
        lib.w4a16_gemm_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, vp, i64, i64, i64, i32,
                                               ctypes.POINTER(Plan), vp, sz, vp]
        lib.w4a16_gemm_add_rmsnorm_workspace_size.restype = sz
        lib.w4a16_gemm_add_rmsnorm_workspace_size.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        lib.w4a16_decode_attention.restype = ctypes.c_int
        lib.w4a16_decode_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, f32, vp, sz, vp]
        lib.w4a16_decode_attention_workspace_size.restype = sz
        lib.w4a16_decode_attention_workspace_size.argtypes = [i64, i64, i64, i64, i64]
        lib.w4a16_decode_attention_plan.restype = ctypes.c_int
        lib.w4a16_decode_attention_plan.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, f32, i32, i32,
                                                    vp, sz, vp]
        lib.w4a16_decode_attention_workspace_size_plan.restype = sz
        lib.w4a16_decode_attention_workspace_size_plan.argtypes = [i64, i64, i64, i64, i64, i32, i32]
        lib.w4a16_tune.restype = ctypes.c_int
        lib.w4a16_tune.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, sz, vp, sz, i32,
                                   ctypes.POINTER(Plan), ctypes.POINTER(ctypes.c_float),
                                   ctypes.POINTER(ctypes.c_int32), vp]
        lib.w4a16_silu_mul.restype = ctypes.c_int
        lib.w4a16_silu_mul.argtypes = [vp, vp, i64, i64, vp]
        lib.w4a16_decode_layer.restype = ctypes.c_int
        lib.w4a16_decode_layer.argtypes = [ctypes.POINTER(DecoderLayer), i64, i64, i64, i64, i64, i64, vp, f32, f32,
                                           vp, vp, vp, sz, vp]
        lib.w4a16_decode_layer_workspace_size.restype = sz
        lib.w4a16_decode_layer_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64]
        lib.w4a16_gemm_silu.restype = ctypes.c_int
        lib.w4a16_gemm_silu.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.POINTER(Plan), vp, sz, vp]
        lib.w4a16_stream_read_sink_words.restype = i64
        lib.w4a16_stream_read_sink_words.argtypes = [i64, i32, i32]
        lib.w4a16_stream_read.restype = ctypes.c_int
        lib.w4a16_stream_read.argtypes = [vp, i64, vp, i32, i32, vp]
        lib.w4a16_gemm_noalloc_max_bytes.restype = sz
        lib.w4a16_gemm_noalloc_max_bytes.argtypes = []
        lib.w4a16_gemm_noalloc.restype = ctypes.c_int
        lib.w4a16_gemm_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
        if path is None:
            _lib = lib
        return lib


def lib():
    return load_library()


def header_functions():
    """Names of the functions declared in include/w4a16.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def _check(status):
    if status != 0:
        msg = lib().w4a16_last_error().decode(errors="replace")
        raise W4A16Error(status, msg)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def pack(q=None, z=None):
    """Pack uint8 codes on the GPU: q [M, K] -> uint32 [M, K/8] (as int32),
    z [M, K/128] -> uint32 [M, ceil(G/8)] (as int32).  Returns (qpk, zpk)."""
    if q is None and z is None:
        raise ValueError("nothing to pack")
    ref = q if q is not None else z
    M = ref.shape[0]
    if q is not None:
        _need(q, "q", torch.uint8)
        K = q.shape[1]
    else:
        _need(z, "z", torch.uint8)
        K = z.shape[1] * GROUP
    G = K // GROUP
    if z is not None:
        _need(z, "z", torch.uint8, (M, G))
    qpk = torch.empty((M, K // 8), dtype=torch.int32, device=ref.device) if q is not None else None
    zpk = torch.empty((M, (G + 7) // 8), dtype=torch.int32, device=ref.device) if z is not None else None
    _check(lib().w4a16_pack(_p(q), _p(z), M, K, GROUP, _p(qpk), _p(zpk), _stream()))
    return qpk, zpk


def quantize(w):
    """Round-to-nearest group quantization on the GPU: fp16 w [M, K] ->
    (q_packed int32 [M, K/8], scales fp16 [M, K/128], z_packed int32
    [M, ceil(G/8)]), ready for gemm()."""
    _need(w, "w", torch.float16)
    M, K = w.shape
    G = K // GROUP
    qpk = torch.empty((M, K // 8), dtype=torch.int32, device=w.device)
    s = torch.empty((M, G), dtype=torch.float16, device=w.device)
    zpk = torch.empty((M, (G + 7) // 8), dtype=torch.int32, device=w.device)
    _check(lib().w4a16_quantize(_p(w), M, K, GROUP, _p(qpk), _p(s), _p(zpk), _stream()))
    return qpk, s, zpk


def _dims(qpk, s, zpk, x, layout=LAYOUT_KN):
    _need(qpk, "q_packed", torch.int32)
    M, KW = qpk.shape
    K = KW * 8
    G = K // GROUP
    _need(s, "scales", torch.float16, (M, G))
    _need(zpk, "z_packed", torch.int32, (M, (G + 7) // 8))
    if x.dim() == 1:
        _need(x, "x", torch.float16, (K,))
        N = 1
    elif layout == LAYOUT_TOKEN:
        _need(x, "x", torch.float16)
        if x.dim() != 2 or x.shape[1] != K:
            raise ValueError("x must be [N, K=%d], got %s" % (K, tuple(x.shape)))
        N = x.shape[0]
    else:
        _need(x, "x", torch.float16)
        if x.dim() != 2 or x.shape[0] != K:
            raise ValueError("x must be [K=%d, N], got %s" % (K, tuple(x.shape)))
        N = x.shape[1]
    return M, N, K


def plan_default(M, N, K, layout=LAYOUT_KN):
    p = Plan()
    if layout == LAYOUT_KN:
        _check(lib().w4a16_plan_default(M, N, K, GROUP, ctypes.byref(p)))
    else:
        _check(lib().w4a16_plan_default_ex(M, N, K, GROUP, layout, ctypes.byref(p)))
    return p


def kernel_name(M, N, K, plan=None):
    """Name of the main kernel a plan (None: the default) launches."""
    buf = ctypes.create_string_buffer(128)
    _check(lib().w4a16_kernel_name(M, N, K, GROUP, None if plan is None else ctypes.byref(plan), buf, 128))
    return buf.value.decode()


def workspace_size(M, N, K, plan=None, layout=LAYOUT_KN):
    if layout != LAYOUT_KN:
        return int(lib().w4a16_workspace_size_ex(M, N, K, GROUP, layout,
                                                 None if plan is None else ctypes.byref(plan)))
    if plan is None:
        return int(lib().w4a16_gemm_workspace_size(M, N, K, GROUP))
    return int(lib().w4a16_workspace_size_plan(M, N, K, GROUP, ctypes.byref(plan)))


class Workspace:
    """A zero-filled device buffer for split reductions (kept zeroed by the
    kernels between calls).  One per stream."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=self.device or "cuda")
        return self.buf


_default_ws = {}


def _workspace_for(device):
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _default_ws.get(key)
    if ws is None:
        ws = _default_ws[key] = Workspace(device)
    return ws


def gemv(qpk, s, zpk, x, out=None):
    """c[M] = Wdeq . x[K] (N = 1, no workspace)."""
    M, N, K = _dims(qpk, s, zpk, x)
    if N != 1:
        raise ValueError("gemv wants one activation column")
    if out is None:
        out = torch.empty((M,), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", torch.float16)
        if out.numel() != M:
            raise ValueError("out must hold M=%d values" % M)
    _check(lib().w4a16_gemv(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, K, GROUP, _stream()))
    return out


def gemm(qpk, s, zpk, x, out=None, plan=None, workspace=None, layout=LAYOUT_KN):
    """c[M, N] = Wdeq[M, K] . x[K, N] with the library's dispatch (or a plan).
    With layout=LAYOUT_TOKEN, x is [N, K] and the result [N, M]
    (c = x . Wdeq^T, one row per token)."""
    if layout not in (LAYOUT_KN, LAYOUT_TOKEN):
        raise ValueError("unknown layout %r" % (layout,))
    M, N, K = _dims(qpk, s, zpk, x, layout)
    shape = (N, M) if layout == LAYOUT_TOKEN else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", torch.float16)
        if out.numel() != M * N:
            raise ValueError("out must hold M*N=%d values" % (M * N))
    need = workspace_size(M, N, K, plan, layout)
    if plan is not None and need == 0:
        # invalid plans report size 0; let the library say why
        need = 0
    ws = None
    if need:
        if workspace is None:
            ws = _workspace_for(x.device).get(need)
        else:
            ws = workspace.get(need) if isinstance(workspace, Workspace) else workspace
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if layout != LAYOUT_KN:
        _check(lib().w4a16_gemm_ex(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, N, K, GROUP, layout,
                                   None if plan is None else ctypes.byref(plan), _p(ws), ws_bytes, _stream()))
    elif plan is None:
        _check(lib().w4a16_gemm(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, N, K, GROUP,
                                _p(ws), ws_bytes, _stream()))
    else:
        _check(lib().w4a16_gemm_plan(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, N, K, GROUP,
                                     ctypes.byref(plan), _p(ws), ws_bytes, _stream()))
    return out


def add_rmsnorm(x, residual, gamma, eps=1e-6, h=None, y=None):
    """h = fp16(x + residual), y = RMSNorm(h) * gamma, token-major [N, K].
    Pass h=residual to update the residual stream in place.  Returns (y, h)."""
    _need(x, "x", torch.float16)
    if x.dim() != 2:
        raise ValueError("x must be [N, K]")
    N, K = x.shape
    _need(residual, "residual", torch.float16, (N, K))
    _need(gamma, "gamma", torch.float16, (K,))
    if h is None:
        h = torch.empty_like(x)
    else:
        _need(h, "h", torch.float16, (N, K))
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", torch.float16, (N, K))
    _check(lib().w4a16_add_rmsnorm(_p(x), _p(residual), _p(gamma), float(eps), _p(h), _p(y), N, K, _stream()))
    return y, h


def gemm_add_rmsnorm(qpk, s, zpk, x, residual, gamma, eps=1e-6, h=None, out=None, plan=None, workspace=None):
    """Token-major fused prologue + product: h = fp16(x + residual) and
    out[N, M] = RMSNorm(h) * gamma . Wdeq^T.  Returns (out, h)."""
    M, N, K = _dims(qpk, s, zpk, x, LAYOUT_TOKEN)
    if x.dim() != 2:
        raise ValueError("x must be [N, K]")
    _need(residual, "residual", torch.float16, (N, K))
    _need(gamma, "gamma", torch.float16, (K,))
    if h is None:
        h = torch.empty_like(x)
    else:
        _need(h, "h", torch.float16, (N, K))
    if out is None:
        out = torch.empty((N, M), dtype=torch.float16, device=x.device)
    else:
        _need(out, "out", torch.float16)
        if out.numel() != M * N:
            raise ValueError("out must hold M*N=%d values" % (M * N))
    need = int(lib().w4a16_gemm_add_rmsnorm_workspace_size(M, N, K, GROUP,
                                                           None if plan is None else ctypes.byref(plan)))
    if workspace is None:
        ws = _workspace_for(x.device).get(max(need, 1))
    else:
        ws = workspace.get(max(need, 1)) if isinstance(workspace, Workspace) else workspace
    ws_bytes = ws.numel() * ws.element_size()
    _check(lib().w4a16_gemm_add_rmsnorm(_p(qpk), _p(s), _p(zpk), _p(x), _p(residual), _p(gamma), float(eps),
                                        _p(h), _p(out), M, N, K, GROUP,
                                        None if plan is None else ctypes.byref(plan), _p(ws), ws_bytes,
                                        _stream()))
    return out, h


def decode_attention(qkv, k_cache, v_cache, pos, max_len=None, rope_base=10000.0, scale=None, out=None,
                     workspace=None, shape=None):
    """One decode step of multi-head attention with rotary encoding:
    qkv fp16 [B, 3 H D] (q | k | v of each sequence's new token), caches fp16
    [B, H, S, D] (updated at each sequence's position), pos int32 [B] on the
    device, max_len a bound on pos + 1 (default S); shape (keys per wave,
    waves) or None for the default.  Returns out [B, H D]."""
    _need(k_cache, "k_cache", torch.float16)
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, H, S, D]")
    Bn, H, S, D = k_cache.shape
    _need(v_cache, "v_cache", torch.float16, (Bn, H, S, D))
    _need(qkv, "qkv", torch.float16, (Bn, 3 * H * D))
    _need(pos, "pos", torch.int32, (Bn,))
    if max_len is None:
        max_len = S
    if scale is None:
        scale = 1.0 / float(D) ** 0.5
    if out is None:
        out = torch.empty((Bn, H * D), dtype=torch.float16, device=qkv.device)
    else:
        _need(out, "out", torch.float16, (Bn, H * D))
    kpw, waves = (0, 0) if shape is None else shape
    need = int(lib().w4a16_decode_attention_workspace_size_plan(Bn, H, D, S, max_len, kpw, waves))
    ws = None
    if need:
        if workspace is None:
            ws = _workspace_for(qkv.device).get(need)
        else:
            ws = workspace.get(need) if isinstance(workspace, Workspace) else workspace
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().w4a16_decode_attention_plan(_p(qkv), _p(k_cache), _p(v_cache), _p(pos), _p(out), Bn, H, D, S,
                                             max_len, float(rope_base), float(scale), kpw, waves, _p(ws), ws_bytes,
                                             _stream()))
    return out


def tune(qpk, s, zpk, x, layout=LAYOUT_KN, iters=20, flush=None, workspace_bytes=None):
    """Time the candidate plans of this call's shape on the device (the
    library's tuner) and return (plan, microseconds per call, plans timed).
    flush: an optional device tensor overwritten before every timed call
    (cold-cache timing).  The workspace is the stream's default one, grown
    to the largest candidate's need (or to workspace_bytes)."""
    M, N, K = _dims(qpk, s, zpk, x, layout)
    out = torch.empty((N, M) if layout == LAYOUT_TOKEN else (M, N), dtype=torch.float16, device=x.device)
    if workspace_bytes is None:
        workspace_bytes = (64 << 10) + 8 * M * N * 4 + 2 * K * N + 4096
    ws = _workspace_for(x.device).get(workspace_bytes)
    best = Plan()
    us = ctypes.c_float()
    n = ctypes.c_int32()
    fb = 0 if flush is None else flush.numel() * flush.element_size()
    _check(lib().w4a16_tune(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, N, K, GROUP, layout, _p(ws),
                            ws.numel() * ws.element_size(), _p(flush), fb, int(iters), ctypes.byref(best),
                            ctypes.byref(us), ctypes.byref(n), _stream()))
    return best, float(us.value), int(n.value)


def silu_mul(gu, out=None):
    """act[N, I] = silu(gu[:, :I]) * gu[:, I:] (fp16, token-major)."""
    _need(gu, "gu", torch.float16)
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be [N, 2 I]")
    N, I = gu.shape[0], gu.shape[1] // 2
    if out is None:
        out = torch.empty((N, I), dtype=torch.float16, device=gu.device)
    else:
        _need(out, "out", torch.float16, (N, I))
    _check(lib().w4a16_silu_mul(_p(gu), _p(out), N, I, _stream()))
    return out


def decode_layer_workspace_size(B, H, D, I, S, max_len):
    return int(lib().w4a16_decode_layer_workspace_size(B, H, D, I, S, max_len))


def _linear(w):
    qpk, s, zpk = w
    _need(qpk, "q_packed", torch.int32)
    _need(s, "scales", torch.float16)
    _need(zpk, "z_packed", torch.int32)
    return Linear(_p(qpk), _p(s), _p(zpk))


def decode_layer(layer, pos, residual, x, workspace, max_len=None, eps=1e-6, rope_base=10000.0):
    """One decode step of one decoder layer (w4a16_decode_layer).  layer: a
    dict with "qkv", "o", "gate_up", "down" (each (q_packed, scales,
    z_packed)), "attn_norm", "mlp_norm", "k_cache", "v_cache".  residual and
    x (fp16 [B, H D]) are updated in place; workspace is a zero-initialised
    uint8 device tensor of at least decode_layer_workspace_size() bytes."""
    kc = layer["k_cache"]
    _need(kc, "k_cache", torch.float16)
    Bn, H, S, D = kc.shape
    _need(layer["v_cache"], "v_cache", torch.float16, (Bn, H, S, D))
    gu_rows = layer["gate_up"][0].shape[0]
    I = gu_rows // 2
    _need(layer["attn_norm"], "attn_norm", torch.float16, (H * D,))
    _need(layer["mlp_norm"], "mlp_norm", torch.float16, (H * D,))
    _need(residual, "residual", torch.float16, (Bn, H * D))
    _need(x, "x", torch.float16, (Bn, H * D))
    _need(pos, "pos", torch.int32, (Bn,))
    _need(workspace, "workspace", torch.uint8)
    st = DecoderLayer(_linear(layer["qkv"]), _linear(layer["o"]), _linear(layer["gate_up"]), _linear(layer["down"]),
                      _p(layer["attn_norm"]), _p(layer["mlp_norm"]), _p(kc), _p(layer["v_cache"]))
    _check(lib().w4a16_decode_layer(ctypes.byref(st), Bn, H, D, I, S, S if max_len is None else max_len, _p(pos),
                                    float(eps), float(rope_base), _p(residual), _p(x), _p(workspace),
                                    workspace.numel(), _stream()))


def gemm_silu(qpk, s, zpk, gu, out=None, plan=None, workspace=None):
    """Down projection with the gated activation as its prologue:
    out[N, M] = (silu(gu[:, :K]) * gu[:, K:]) . Wdeq^T (token-major)."""
    _need(qpk, "q_packed", torch.int32)
    M, K = qpk.shape[0], qpk.shape[1] * 8
    _need(gu, "gu", torch.float16)
    if gu.dim() != 2 or gu.shape[1] != 2 * K:
        raise ValueError("gu must be [N, 2K=%d], got %s" % (2 * K, tuple(gu.shape)))
    N = gu.shape[0]
    G = K // GROUP
    _need(s, "scales", torch.float16, (M, G))
    _need(zpk, "z_packed", torch.int32, (M, (G + 7) // 8))
    if out is None:
        out = torch.empty((N, M), dtype=torch.float16, device=gu.device)
    else:
        _need(out, "out", torch.float16)
        if out.numel() != M * N:
            raise ValueError("out must hold M*N=%d values" % (M * N))
    need = workspace_size(M, N, K, plan, LAYOUT_TOKEN)
    ws = None
    if need:
        ws = _workspace_for(gu.device).get(need) if workspace is None else (
            workspace.get(need) if isinstance(workspace, Workspace) else workspace)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().w4a16_gemm_silu(_p(qpk), _p(s), _p(zpk), _p(gu), _p(out), M, N, K, GROUP,
                                 None if plan is None else ctypes.byref(plan), _p(ws), ws_bytes, _stream()))
    return out


def stream_read(buf, sink=None, waves=8, loads=4):
    """One launch of the streaming-read probe over the bytes of ``buf`` (a
    contiguous device tensor), ``loads`` KB per wave; returns the sink (one
    word per wave)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    words = int(lib().w4a16_stream_read_sink_words(nbytes, waves, loads))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=buf.device)
    _check(lib().w4a16_stream_read(_p(buf), nbytes, _p(sink), int(waves), int(loads), _stream()))
    return sink


def gemm_noalloc(qpk, s, zpk, x, out):
    """w4a16_gemm_noalloc: the default-plan product with the library's own
    device scratch instead of a workspace.  ``out`` [M, N] is required (the
    call allocates nothing)."""
    M, N, K = _dims(qpk, s, zpk, x)
    _need(out, "out", torch.float16)
    if out.numel() != M * N:
        raise ValueError("out must hold M*N=%d values" % (M * N))
    _check(lib().w4a16_gemm_noalloc(_p(qpk), _p(s), _p(zpk), _p(x), _p(out), M, N, K, GROUP, _stream()))
    return out
