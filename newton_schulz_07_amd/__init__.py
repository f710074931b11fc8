"""MI355X (gfx950) Newton–Schulz orthogonalization: Python binding of libns_hip.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  If the library is not
built, every call raises; there is no other implementation to fall back to.

The functions carry the C ABI's names (include/ns_hip.h) and take torch
tensors in place of pointers; `orthogonalize` is the convenience form.
"""

import ctypes
import os

DEFAULT_COEFFS = (3.4445, -4.7750, 2.0315)
DEFAULT_STEPS = 5

NS_DTYPE_F32 = 0
NS_DTYPE_BF16 = 1

NS_KIND_SUMSQ, NS_KIND_SCALE, NS_KIND_GRAM, NS_KIND_POLY, NS_KIND_UPDATE = range(5)
KIND_NAMES = {NS_KIND_SUMSQ: "sumsq", NS_KIND_SCALE: "scale", NS_KIND_GRAM: "gram",
              NS_KIND_POLY: "poly", NS_KIND_UPDATE: "update"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libns_hip.so")

# exported symbols and their C signatures (include/ns_hip.h)
_i64, _int, _flt, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_pvp, _pi64 = ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_int64)
NS_MAX_GROUPS = 4096
SIGNATURES = {
    "ns_orthogonalize": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _flt, _flt, _flt, _vp]),
    "ns_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "ns_orthogonalize_noalloc": (_int, [_vp, _vp, _i64, _i64, _i64, _int, _int, _flt, _flt, _flt, _vp]),
    "ns_orthogonalize_grouped": (_int, [_int, _pvp, _pvp, _pi64, _pi64, _pi64, _int, _int, _flt, _flt, _flt, _vp]),
    "ns_workspace_bytes_grouped": (_sz, [_int, _pi64, _pi64, _pi64, _int]),
    "ns_release_workspace": (_int, []),
    "ns_workspace_allocations": (_i64, []),
    "ns_status_string": (ctypes.c_char_p, [_int]),
    "ns_last_error": (ctypes.c_char_p, []),
    "ns_query_last_config": (_int, [ctypes.c_char_p, _sz]),
    "ns_timing_enable": (_int, [_int]),
    "ns_timing_sample": (_int, [_int, _int]),
    "ns_timing_reset": (_int, []),
    "ns_timing_query": (_int, [_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    "ns_set_workspace_poison": (_int, [_int]),
    "ns_peak_mfma": (_int, [_int, _i64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), _vp]),
    "ns_stage_normalize": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]),
    "ns_stage_gram": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]),
    "ns_stage_poly": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _flt, _flt, _flt, _vp]),
    "ns_stage_update": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _int, _vp]),
}

_lib = None


class NSError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def lib():
    """Load libns_hip.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python -m newton_schulz_07_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != 0:
        L = lib()
        raise NSError(status, f"{L.ns_status_string(status).decode()}: {L.ns_last_error().decode()}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return NS_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return NS_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.float32 or torch.bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_gpu_tensor(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _brc(x):
    if x.dim() < 2:
        raise ValueError("need a matrix or a stack of matrices")
    rows, cols = x.shape[-2], x.shape[-1]
    batch = x.numel() // (rows * cols) if rows * cols else 0
    return batch, rows, cols


def ns_orthogonalize(x, out=None, ns_steps=DEFAULT_STEPS, a=DEFAULT_COEFFS[0], b=DEFAULT_COEFFS[1],
                     c=DEFAULT_COEFFS[2]):
    """Newton–Schulz of every [rows, cols] slice of x (leading dims = batch)."""
    import torch
    _need_gpu_tensor(x, "x")
    if out is None:
        out = torch.empty_like(x)
    _need_gpu_tensor(out, "out")
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    batch, rows, cols = _brc(x)
    with torch.cuda.device(x.device):
        _check(lib().ns_orthogonalize(_ptr(x), _ptr(out), batch, rows, cols, _dtype_code(x),
                                      int(ns_steps), float(a), float(b), float(c), _stream(x)))
    return out


NS_NOALLOC_SCRATCH_BYTES = 256 << 20


def ns_orthogonalize_noalloc(x, out, ns_steps=DEFAULT_STEPS, a=DEFAULT_COEFFS[0], b=DEFAULT_COEFFS[1],
                             c=DEFAULT_COEFFS[2]):
    """ns_orthogonalize on the library's fixed device scratch: no device
    allocation by the library (out must be given; the binding allocates
    nothing either).  Shapes needing more than NS_NOALLOC_SCRATCH_BYTES of
    workspace raise NSError (NS_ERR_SCRATCH)."""
    _need_gpu_tensor(x, "x")
    _need_gpu_tensor(out, "out")
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype")
    batch, rows, cols = _brc(x)
    import torch
    with torch.cuda.device(x.device):
        _check(lib().ns_orthogonalize_noalloc(_ptr(x), _ptr(out), batch, rows, cols, _dtype_code(x),
                                              int(ns_steps), float(a), float(b), float(c), _stream(x)))
    return out


def orthogonalize(x, steps=DEFAULT_STEPS, coeffs=DEFAULT_COEFFS, out=None):
    """Convenience form: orthogonalize(x, steps, (a, b, c))."""
    a, b, c = coeffs
    return ns_orthogonalize(x, out=out, ns_steps=steps, a=a, b=b, c=c)


def _arrays(shapes):
    n = len(shapes)
    return ((ctypes.c_int64 * n)(*[s[0] for s in shapes]), (ctypes.c_int64 * n)(*[s[1] for s in shapes]),
            (ctypes.c_int64 * n)(*[s[2] for s in shapes]))


def ns_orthogonalize_grouped(xs, outs=None, ns_steps=DEFAULT_STEPS, a=DEFAULT_COEFFS[0], b=DEFAULT_COEFFS[1],
                             c=DEFAULT_COEFFS[2]):
    """Newton–Schulz of every slice of several stacks of different shapes in one
    call (shared launches); xs is a list of tensors of one dtype on one device.
    Returns the list of outputs."""
    import torch
    xs = list(xs)
    if not xs:
        return []
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    outs = list(outs)
    if len(outs) != len(xs):
        raise ValueError("outs must have one tensor per input")
    dev, dt = xs[0].device, xs[0].dtype
    for i, (x, o) in enumerate(zip(xs, outs)):
        _need_gpu_tensor(x, f"xs[{i}]")
        _need_gpu_tensor(o, f"outs[{i}]")
        if x.device != dev or o.device != dev or x.dtype != dt or o.dtype != dt:
            raise ValueError("every tensor must share the first input's device and dtype")
        if o.shape != x.shape:
            raise ValueError(f"outs[{i}] must match xs[{i}] in shape")
    n = len(xs)
    bt, rt, ct = _arrays([_brc(x) for x in xs])
    pin = (ctypes.c_void_p * n)(*[x.data_ptr() for x in xs])
    pout = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    with torch.cuda.device(dev):
        _check(lib().ns_orthogonalize_grouped(n, pin, pout, bt, rt, ct, _dtype_code(xs[0]), int(ns_steps),
                                              float(a), float(b), float(c), _stream(xs[0])))
    return outs


def orthogonalize_grouped(xs, steps=DEFAULT_STEPS, coeffs=DEFAULT_COEFFS, outs=None):
    """Convenience form: orthogonalize_grouped([x0, x1, ...], steps, (a, b, c))."""
    a, b, c = coeffs
    return ns_orthogonalize_grouped(xs, outs=outs, ns_steps=steps, a=a, b=b, c=c)


def ns_workspace_bytes_grouped(shapes, dtype_code):
    """Workspace bytes of a grouped call over stacks of the given (batch, rows, cols)."""
    bt, rt, ct = _arrays(shapes)
    return int(lib().ns_workspace_bytes_grouped(len(shapes), bt, rt, ct, dtype_code))


def ns_workspace_bytes(batch, rows, cols, dtype_code):
    return int(lib().ns_workspace_bytes(batch, rows, cols, dtype_code))


def ns_release_workspace():
    _check(lib().ns_release_workspace())


def ns_workspace_allocations():
    """Workspace allocations the library has made since it was loaded."""
    return int(lib().ns_workspace_allocations())


def ns_query_last_config():
    buf = ctypes.create_string_buffer(1024)
    lib().ns_query_last_config(buf, len(buf))
    return buf.value.decode()


def ns_timing_enable(mask):
    _check(lib().ns_timing_enable(int(mask)))


def ns_timing_sample(every=1, offset=0):
    """Time only launch i of each kind with i % every == offset."""
    _check(lib().ns_timing_sample(int(every), int(offset)))


def ns_timing_reset():
    _check(lib().ns_timing_reset())


def ns_timing_query(kind):
    """(total_ms, launches) of the kernel kind since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().ns_timing_query(int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def ns_set_workspace_poison(on):
    """Fill every later call's workspace with NaN bytes first (diagnostic)."""
    _check(lib().ns_set_workspace_poison(1 if on else 0))


def ns_peak_mfma(dtype="bf16", iters=1 << 20, stream=None):
    """(TFLOP/s, MHz): the dense MFMA rate of a register-only loop on the
    current device and the average shader clock during it."""
    import torch
    code = {"bf16": NS_DTYPE_BF16, "fp32": NS_DTYPE_F32}[dtype]
    st = stream if stream is not None else torch.cuda.current_stream()
    tf = ctypes.c_double()
    mhz = ctypes.c_double()
    _check(lib().ns_peak_mfma(code, int(iters), ctypes.byref(tf), ctypes.byref(mhz), ctypes.c_void_p(st.cuda_stream)))
    return tf.value, mhz.value


# ------------------------------------------------------------------ stages

def ns_stage_normalize(x, x0=None, norms=None):
    """X0 = x / (||x||_F + 1e-7) per slice."""
    import torch
    _need_gpu_tensor(x, "x")
    x0 = torch.empty_like(x) if x0 is None else x0
    batch, rows, cols = _brc(x)
    with torch.cuda.device(x.device):
        _check(lib().ns_stage_normalize(_ptr(x), _ptr(x0), _ptr(norms), batch, rows, cols,
                                        _dtype_code(x), _stream(x)))
    return x0


def ns_stage_gram(x):
    """Returns (a_off [batch, m, m] in x's dtype, a_diag fp32 [batch, m])."""
    import torch
    _need_gpu_tensor(x, "x")
    batch, rows, cols = _brc(x)
    m = min(rows, cols)
    a_off = torch.empty((batch, m, m), dtype=x.dtype, device=x.device)
    a_diag = torch.empty((batch, m), dtype=torch.float32, device=x.device)
    with torch.cuda.device(x.device):
        _check(lib().ns_stage_gram(_ptr(x), _ptr(a_off), _ptr(a_diag), batch, rows, cols,
                                   _dtype_code(x), _stream(x)))
    return a_off, a_diag


def ns_stage_poly(a_off, a_diag, a=DEFAULT_COEFFS[0], b=DEFAULT_COEFFS[1], c=DEFAULT_COEFFS[2]):
    """Returns (c_off, c_diag) of C = aI + bA + cAA for A = a_off + diag(a_diag)."""
    import torch
    _need_gpu_tensor(a_off, "a_off")
    _need_gpu_tensor(a_diag, "a_diag")
    batch, m, m2 = _brc(a_off)
    if m != m2 or a_diag.dtype != torch.float32 or a_diag.numel() != batch * m:
        raise ValueError("a_off must be [batch, m, m] and a_diag fp32 [batch, m]")
    c_off = torch.empty_like(a_off)
    c_diag = torch.empty_like(a_diag)
    with torch.cuda.device(a_off.device):
        _check(lib().ns_stage_poly(_ptr(a_off), _ptr(a_diag), _ptr(c_off), _ptr(c_diag), batch, m,
                                   _dtype_code(a_off), float(a), float(b), float(c), _stream(a_off)))
    return c_off, c_diag


def ns_stage_update(x, c_off, c_diag):
    """x_out = C x (rows <= cols) or x C (rows > cols), C = c_off + diag(c_diag)."""
    import torch
    _need_gpu_tensor(x, "x")
    _need_gpu_tensor(c_off, "c_off")
    _need_gpu_tensor(c_diag, "c_diag")
    batch, rows, cols = _brc(x)
    m = min(rows, cols)
    if c_off.numel() != batch * m * m or c_diag.numel() != batch * m or c_diag.dtype != torch.float32:
        raise ValueError("c_off must be [batch, m, m] and c_diag fp32 [batch, m], m = min(rows, cols)")
    x_out = torch.empty_like(x)
    with torch.cuda.device(x.device):
        _check(lib().ns_stage_update(_ptr(x), _ptr(c_off), _ptr(c_diag), _ptr(x_out), batch, rows, cols,
                                     _dtype_code(x), _stream(x)))
    return x_out
