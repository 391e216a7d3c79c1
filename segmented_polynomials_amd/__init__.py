"""Python binding of ``libsegpoly.so`` (argument marshalling only).

The functions keep the names of the C ABI in ``include/segpoly.h``:
``tp_create`` / ``tp_conv_fwd`` / ``tp_conv_bwd`` / ``symcon_create`` / ``symcon_fwd`` /
``symcon_bwd`` / ``linear_create`` / ``linear_fwd`` / ``linear_bwd`` / ``fctp_create`` /
``fctp_fwd`` / ``fctp_bwd`` / ``sh_fwd`` / ``sh_bwd``.  Every
step of the computation runs in the library's HIP kernels; PyTorch only
supplies device memory and the current stream.  There is no CPU fallback:
importing this package fails loudly if the library has not been built.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SEGPOLY_LIB selects another build of the same library (the sanitizer
# build of build_sanitize.py); by default the one built next to this file
LIB_PATH = os.environ.get("SEGPOLY_LIB") or os.path.join(_HERE, "libsegpoly.so")

OK = 0
E_INVALID, E_PARSE, E_UNSUPPORTED, E_UNSORTED, E_HIP, E_OOM, E_RANGE = -1, -2, -3, -4, -5, -6, -7
MUL_IR, IR_MUL = 0, 1
F32, F64 = 0, 1
I32, I64 = 0, 1
SHARED_WEIGHTS, VALIDATE, FORCE_GENERIC, REDUCE_MEAN, MERGE_PATHS = 1, 2, 4, 8, 16
(Q_DIM_IN1, Q_DIM_IN2, Q_DIM_OUT, Q_WEIGHT_NUMEL, Q_NUM_PATHS, Q_CG_NNZ, Q_SPECIALIZED, Q_MUL,
 Q_DIM_IN, Q_NUM_COUPLINGS, Q_NUM_TERMS, Q_NUM_ELEMENTS, Q_NUM_MONOMIALS) = range(13)

_LAYOUTS = {"mul_ir": MUL_IR, "ir_mul": IR_MUL}
_DTYPES = {"f32": F32, "f64": F64}

# every symbol include/segpoly.h declares
EXPORTS = ("tp_create", "tp_query", "tp_irreps_out", "tp_path_info", "tp_path_cg", "tp_kernel_name",
           "tp_conv_fwd", "tp_conv_fwd_vec", "tp_rowptr_build", "tp_conv_fwd_rowptr", "tp_src_rowptr_build", "tp_conv_bwd_workspace", "tp_conv_bwd", "tp_conv_bwd_rowptr", "tp_destroy", "symcon_create", "symcon_query", "symcon_coupling_info",
           "symcon_coupling_dense", "symcon_fwd", "symcon_bwd_workspace", "symcon_bwd", "symcon_bwd_noalloc", "symcon_destroy", "linear_create", "linear_query", "linear_fwd",
           "linear_bwd_workspace", "linear_bwd", "linear_destroy", "fctp_create", "fctp_query", "fctp_path_info",
           "fctp_fwd", "fctp_bwd_workspace", "fctp_bwd", "fctp_fwd_per_sample", "fctp_bwd_per_sample", "fctp_conv_fwd", "fctp_conv_bwd_workspace", "fctp_conv_bwd", "fctp_destroy", "edge_scalars_fwd", "edge_scalars_bwd", "sh_fwd", "sh_bwd", "segpoly_real_cg",
           "segpoly_last_error", "segpoly_version")


class SegpolyError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"segpoly error {code}: {msg}")
        self.code = code


def _hip_runtime_of_torch():
    """Load PyTorch's HIP runtime first.  The library's dependency
    libamdhip64.so.7 then resolves (by soname) to that same copy, so device
    pointers and streams from PyTorch are valid in the library: one HIP
    runtime per process."""
    import torch  # noqa: F401
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    if os.path.exists(path):
        ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)


def hip_runtimes_loaded():
    """Distinct libamdhip64 files mapped into this process."""
    with open("/proc/self/maps") as f:
        return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python segmented_polynomials_amd/build.py`")
    _hip_runtime_of_torch()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, c_int, c_uint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint
    p64 = ctypes.POINTER(ctypes.c_int64)
    pd = ctypes.POINTER(ctypes.c_double)
    sig = {
        "tp_create": [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, c_int, c_int, c_uint, ctypes.POINTER(vp)],
        "tp_query": [vp, c_int, p64],
        "tp_irreps_out": [vp, ctypes.c_char_p, ctypes.c_size_t],
        "tp_path_info": [vp, c_int, p64],
        "tp_path_cg": [vp, c_int, pd],
        "tp_kernel_name": [vp, ctypes.c_char_p, ctypes.c_size_t],
        "tp_conv_fwd": [vp, vp, i64, vp, vp, vp, vp, c_int, i64, i64, vp, vp],
        "tp_conv_fwd_vec": [vp, vp, i64, vp, c_int, vp, vp, vp, c_int, i64, i64, vp, vp],
        "tp_rowptr_build": [vp, c_int, i64, i64, vp, vp],
        "tp_conv_fwd_rowptr": [vp, vp, i64, vp, vp, vp, vp, c_int, i64, i64, vp, vp],
        "tp_conv_bwd_workspace": [vp, i64, c_int, ctypes.POINTER(ctypes.c_size_t)],
        "tp_conv_bwd": [vp, vp, i64, vp, vp, vp, vp, vp, c_int, i64, i64, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "tp_src_rowptr_build": [vp, vp, c_int, i64, i64, vp, vp],
        "tp_conv_bwd_rowptr": [vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, c_int, i64, i64, vp, vp, vp, vp, vp,
                               ctypes.c_size_t, vp],
        "tp_destroy": [vp],
        "symcon_create": [ctypes.c_char_p, ctypes.c_char_p, c_int, c_int, c_int, c_int, c_uint, ctypes.POINTER(vp)],
        "symcon_query": [vp, c_int, p64],
        "symcon_coupling_info": [vp, c_int, p64],
        "symcon_coupling_dense": [vp, c_int, pd],
        "symcon_fwd": [vp, vp, vp, c_int, vp, i64, vp, vp],
        "symcon_bwd_workspace": [vp, i64, ctypes.POINTER(ctypes.c_size_t)],
        "symcon_bwd": [vp, vp, vp, vp, c_int, vp, vp, i64, vp, vp, vp, ctypes.c_size_t, vp],
        "symcon_bwd_noalloc": [vp, vp, vp, vp, c_int, vp, vp, i64, vp, vp, vp],
        "symcon_destroy": [vp],
        "linear_create": [ctypes.c_char_p, ctypes.c_char_p, c_int, c_int, c_uint, ctypes.POINTER(vp)],
        "linear_query": [vp, c_int, p64],
        "linear_fwd": [vp, vp, vp, vp, c_int, c_int, i64, vp, vp],
        "linear_bwd_workspace": [vp, i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
        "linear_bwd": [vp, vp, vp, vp, vp, c_int, c_int, i64, vp, vp, vp, ctypes.c_size_t, vp],
        "linear_destroy": [vp],
        "fctp_create": [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, c_int, c_int, c_uint, ctypes.POINTER(vp)],
        "fctp_query": [vp, c_int, p64],
        "fctp_path_info": [vp, c_int, p64],
        "fctp_fwd": [vp, vp, vp, vp, i64, vp, vp],
        "fctp_bwd_workspace": [vp, i64, ctypes.POINTER(ctypes.c_size_t)],
        "fctp_bwd": [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "fctp_fwd_per_sample": [vp, vp, vp, vp, i64, vp, vp],
        "fctp_bwd_per_sample": [vp, vp, vp, vp, vp, i64, vp, vp, vp, vp],
        "fctp_conv_fwd": [vp, vp, i64, vp, vp, i64, vp, vp, c_int, i64, i64, vp, vp],
        "fctp_conv_bwd_workspace": [vp, i64, i64, ctypes.POINTER(ctypes.c_size_t)],
        "fctp_conv_bwd": [vp, vp, i64, vp, vp, i64, vp, vp, vp, c_int, i64, i64, vp, vp, vp, vp, vp,
                          ctypes.c_size_t, vp],
        "fctp_destroy": [vp],
        "edge_scalars_fwd": [c_int, vp, i64, vp, i64, vp, i64, vp, vp, c_int, i64, i64, i64, vp, vp],
        "edge_scalars_bwd": [c_int, vp, i64, i64, i64, vp, vp, vp, c_int, i64, i64, i64, vp, vp, vp, vp],
        "sh_fwd": [c_int, c_int, c_int, vp, i64, vp, vp],
        "sh_bwd": [c_int, c_int, c_int, vp, vp, i64, vp, vp],
        "segpoly_real_cg": [c_int, c_int, c_int, pd],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = c_int
    lib.segpoly_last_error.restype = ctypes.c_char_p
    lib.segpoly_last_error.argtypes = []
    lib.segpoly_version.restype = ctypes.c_char_p
    lib.segpoly_version.argtypes = []
    return lib


lib = _load()


def _check(rc):
    if rc != OK:
        raise SegpolyError(rc, lib.segpoly_last_error().decode())


def version():
    return lib.segpoly_version().decode()


def real_cg(l1, l2, l3):
    """The real coupling tensor of l1 x l2 -> l3 used by the paths, [2l1+1, 2l2+1, 2l3+1]."""
    out = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1))
    _check(lib.segpoly_real_cg(l1, l2, l3, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return out.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)


def _str(fn, h, cap=1 << 16):
    buf = ctypes.create_string_buffer(cap)
    _check(fn(h, buf, cap))
    return buf.value.decode()


def _flags(shared_weights=False, validate=False, force_generic=False, reduce_mean=False, merge=False):
    return (SHARED_WEIGHTS if shared_weights else 0) | (VALIDATE if validate else 0) | \
        (FORCE_GENERIC if force_generic else 0) | (REDUCE_MEAN if reduce_mean else 0) | \
        (MERGE_PATHS if merge else 0)


def _stream_ptr(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------- TP

class TPHandle:
    """Owns one ``tp_handle``; sizes are read back from the library."""

    def __init__(self, raw, layout, dtype, shared_weights):
        self._h = raw
        self.layout = layout
        self.dtype = dtype
        self.shared_weights = shared_weights

    def _q(self, key):
        v = ctypes.c_int64()
        _check(lib.tp_query(self._h, key, ctypes.byref(v)))
        return v.value

    dim_in1 = property(lambda s: s._q(Q_DIM_IN1))
    dim_in2 = property(lambda s: s._q(Q_DIM_IN2))
    dim_out = property(lambda s: s._q(Q_DIM_OUT))
    weight_numel = property(lambda s: s._q(Q_WEIGHT_NUMEL))
    num_paths = property(lambda s: s._q(Q_NUM_PATHS))
    cg_nnz = property(lambda s: s._q(Q_CG_NNZ))
    specialized = property(lambda s: bool(s._q(Q_SPECIALIZED)))
    mul = property(lambda s: s._q(Q_MUL))
    irreps_out = property(lambda s: _str(lib.tp_irreps_out, s._h))
    kernel_name = property(lambda s: _str(lib.tp_kernel_name, s._h))

    def path_info(self, p):
        v = (ctypes.c_int64 * 10)()
        _check(lib.tp_path_info(self._h, p, v))
        keys = ("in1_block", "in2_block", "l1", "l2", "lo", "parity", "mul", "out_offset",
                "weight_offset", "nnz")
        return dict(zip(keys, list(v)))

    def path_cg(self, p):
        i = self.path_info(p)
        shape = (2 * i["l1"] + 1, 2 * i["l2"] + 1, 2 * i["lo"] + 1)
        out = np.zeros(int(np.prod(shape)))
        _check(lib.tp_path_cg(self._h, p, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
        return out.reshape(shape)

    def __del__(self):
        if getattr(self, "_h", None) and lib is not None:
            lib.tp_destroy(self._h)
            self._h = None


def tp_create(irreps_in1, irreps_in2, irreps_out, layout="mul_ir", dtype="f32", shared_weights=False,
              validate=False, force_generic=False, reduce="sum", merge=False):
    """Channelwise product / convolution handle; ``merge`` sums the paths of
    one output type into one block."""
    if reduce not in ("sum", "mean"):
        raise ValueError("reduce is 'sum' or 'mean'")
    raw = ctypes.c_void_p()
    _check(lib.tp_create(irreps_in1.encode(), irreps_in2.encode(), irreps_out.encode(), _LAYOUTS[layout],
                         _DTYPES[dtype], _flags(shared_weights, validate, force_generic, reduce == "mean", merge),
                         ctypes.byref(raw)))
    return TPHandle(raw, layout, dtype, shared_weights)


def _index_dtype(t):
    import torch
    if t.dtype == torch.int32:
        return I32
    if t.dtype == torch.int64:
        return I64
    raise TypeError("indices must be int32 or int64")


def _torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f64": torch.float64}[dt]


def tp_conv_fwd(h, x, sh, w, src=None, dst=None, n_nodes=None, out=None):
    """Gather x[src], couple with sh and w through every path, sum-scatter
    to dst.  Device tensors, contiguous, of the handle's dtype; src/dst int32
    or int64 (dst sorted) or both None (batch mode).  Returns ``out``
    [n_nodes, dim_out] (allocated if not given)."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("sh", sh), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n_src, n_edges = x.shape[0], sh.shape[0]
    if x.shape[1] != h.dim_in1 or sh.shape[1] != h.dim_in2 or w.shape[-1] != h.weight_numel:
        raise ValueError("operand widths do not match the descriptor")
    if w.shape[0] != (1 if h.shared_weights else n_edges):
        raise ValueError("weights must have one row per edge (or one row when shared)")
    if (src is None) != (dst is None):
        raise ValueError("give both src and dst or neither")
    idx = I32
    if src is not None:
        if src.shape != (n_edges,) or dst.shape != (n_edges,) or src.dtype != dst.dtype:
            raise ValueError("src and dst must be [n_edges] of one integer dtype")
        if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
            raise ValueError("src and dst must be contiguous device tensors")
        idx = _index_dtype(src)
    if n_nodes is None:
        if src is not None:
            raise ValueError("n_nodes is required with indices")
        n_nodes = n_edges
    if out is None:
        out = torch.empty((n_nodes, h.dim_out), dtype=t, device=x.device)
    elif out.shape != (n_nodes, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.tp_conv_fwd(h._h, _ptr(x), n_src, _ptr(sh), _ptr(w), _ptr(src), _ptr(dst), idx, n_edges,
                           n_nodes, _ptr(out), _stream_ptr(x.device)))
    return out


def tp_rowptr_build(dst, n_nodes, out=None):
    """Row pointers [n_nodes + 1] of a destination-sorted edge list:
    out[n] = first e with dst[e] >= n (same integer dtype as dst)."""
    import torch
    if dst.dim() != 1 or not dst.is_cuda or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous 1-d device tensor")
    idx = _index_dtype(dst)
    if out is None:
        out = torch.empty(n_nodes + 1, dtype=dst.dtype, device=dst.device)
    elif out.shape != (n_nodes + 1,) or out.dtype != dst.dtype or not out.is_contiguous():
        raise ValueError("out must be [n_nodes + 1] of the dtype of dst")
    _check(lib.tp_rowptr_build(_ptr(dst), idx, dst.shape[0], n_nodes, _ptr(out), _stream_ptr(dst.device)))
    return out


def tp_src_rowptr_build(src, src_perm, n_src, out=None):
    """Row pointers [n_src + 1] of the sources in src_perm order:
    out[s] = first i with src[src_perm[i]] >= s (same integer dtype)."""
    import torch
    for name, a in (("src", src), ("src_perm", src_perm)):
        if a.dim() != 1 or not a.is_cuda or not a.is_contiguous() or a.shape != src.shape or a.dtype != src.dtype:
            raise ValueError(f"{name} must be a contiguous 1-d device tensor like src")
    idx = _index_dtype(src)
    if out is None:
        out = torch.empty(n_src + 1, dtype=src.dtype, device=src.device)
    elif out.shape != (n_src + 1,) or out.dtype != src.dtype or not out.is_contiguous():
        raise ValueError("out must be [n_src + 1] of the dtype of src")
    _check(lib.tp_src_rowptr_build(_ptr(src), _ptr(src_perm), idx, src.shape[0], n_src, _ptr(out),
                                   _stream_ptr(src.device)))
    return out


def tp_conv_fwd_rowptr(h, x, sh, w, src, row_ptr, out=None):
    """``tp_conv_fwd`` with the destination ranges given as row pointers
    (``tp_rowptr_build``): n_nodes = len(row_ptr) - 1."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("sh", sh), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n_src, n_edges = x.shape[0], sh.shape[0]
    if x.shape[1] != h.dim_in1 or sh.shape[1] != h.dim_in2 or w.shape[-1] != h.weight_numel:
        raise ValueError("operand widths do not match the descriptor")
    if w.shape[0] != (1 if h.shared_weights else n_edges):
        raise ValueError("weights must have one row per edge (or one row when shared)")
    if src.shape != (n_edges,) or row_ptr.dim() != 1 or src.dtype != row_ptr.dtype:
        raise ValueError("src must be [n_edges] and row_ptr 1-d, of one integer dtype")
    if not (src.is_cuda and row_ptr.is_cuda and src.is_contiguous() and row_ptr.is_contiguous()):
        raise ValueError("src and row_ptr must be contiguous device tensors")
    n_nodes = row_ptr.shape[0] - 1
    if out is None:
        out = torch.empty((n_nodes, h.dim_out), dtype=t, device=x.device)
    elif out.shape != (n_nodes, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.tp_conv_fwd_rowptr(h._h, _ptr(x), n_src, _ptr(sh), _ptr(w), _ptr(src), _ptr(row_ptr),
                                  _index_dtype(src), n_edges, n_nodes, _ptr(out), _stream_ptr(x.device)))
    return out


def tp_conv_fwd_vec(h, x, vec, w, src=None, dst=None, n_nodes=None, normalize=True, out=None):
    """tp_conv_fwd with the harmonics computed in the kernel from the edge
    vectors vec [n_edges, 3] (input 2 must be 0e + 1o + 2e + ...)."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("vec", vec), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n_src, n_edges = x.shape[0], vec.shape[0]
    if x.shape[1] != h.dim_in1 or vec.shape[1] != 3 or w.shape[-1] != h.weight_numel:
        raise ValueError("operand widths do not match the descriptor")
    if w.shape[0] != (1 if h.shared_weights else n_edges):
        raise ValueError("weights must have one row per edge (or one row when shared)")
    idx = I32
    if src is not None:
        if src.shape != (n_edges,) or dst.shape != (n_edges,) or src.dtype != dst.dtype:
            raise ValueError("src and dst must be [n_edges] of one integer dtype")
        idx = _index_dtype(src)
    if n_nodes is None:
        if src is not None:
            raise ValueError("n_nodes is required with indices")
        n_nodes = n_edges
    if out is None:
        out = torch.empty((n_nodes, h.dim_out), dtype=t, device=x.device)
    _check(lib.tp_conv_fwd_vec(h._h, _ptr(x), n_src, _ptr(vec), 1 if normalize else 0, _ptr(w), _ptr(src),
                               _ptr(dst), idx, n_edges, n_nodes, _ptr(out), _stream_ptr(x.device)))
    return out


def tp_conv_bwd_workspace(h, n_edges, batch=False):
    """Bytes of device workspace ``tp_conv_bwd`` needs for ``n_edges`` edges
    (indexed mode, or batch mode with ``batch``)."""
    v = ctypes.c_size_t()
    _check(lib.tp_conv_bwd_workspace(h._h, n_edges, 1 if batch else 0, ctypes.byref(v)))
    return v.value


def tp_conv_bwd(h, x, sh, w, grad_out, src=None, dst=None, src_perm=None, n_nodes=None, workspace=None,
                grad_x=None, grad_sh=None, grad_w=None):
    """Gradients (grad_x, grad_sh, grad_w) of ``tp_conv_fwd`` for the output
    gradient ``grad_out`` [n_nodes, dim_out].  ``src_perm`` lists the edge ids
    ordered by src (a stable argsort of src), part of the graph like the
    sorted dst.  The workspace and the gradients are allocated if not given."""
    return _tp_conv_bwd(h, x, sh, w, grad_out, src, dst, src_perm, n_nodes, workspace, grad_x, grad_sh, grad_w)


def tp_conv_bwd_rowptr(h, x, sh, w, grad_out, src, dst, src_perm, row_ptr, src_row_ptr, workspace=None,
                       grad_x=None, grad_sh=None, grad_w=None):
    """``tp_conv_bwd`` with the destination ranges as row pointers
    (``tp_rowptr_build``) and the source ranges as row pointers over
    src_perm order (``tp_src_rowptr_build``): n_nodes = len(row_ptr) - 1."""
    for name, a, n in (("row_ptr", row_ptr, None), ("src_row_ptr", src_row_ptr, x.shape[0] + 1)):
        if a.dim() != 1 or not a.is_cuda or not a.is_contiguous() or a.dtype != src.dtype:
            raise ValueError(f"{name} must be a contiguous 1-d device tensor of the dtype of src")
        if n is not None and a.shape[0] != n:
            raise ValueError("src_row_ptr must be [n_src + 1]")
    return _tp_conv_bwd(h, x, sh, w, grad_out, src, dst, src_perm, row_ptr.shape[0] - 1, workspace, grad_x,
                        grad_sh, grad_w, row_ptr=row_ptr, src_row_ptr=src_row_ptr)


def _tp_conv_bwd(h, x, sh, w, grad_out, src, dst, src_perm, n_nodes, workspace, grad_x, grad_sh, grad_w,
                 row_ptr=None, src_row_ptr=None):
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("sh", sh), ("w", w), ("grad_out", grad_out)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n_src, n_edges = x.shape[0], sh.shape[0]
    w_rows = 1 if h.shared_weights else n_edges
    if x.shape[1] != h.dim_in1 or sh.shape[1] != h.dim_in2 or w.shape != (w_rows, h.weight_numel):
        raise ValueError("operand widths do not match the descriptor (weights: one row per edge, or one when shared)")
    if not (src is None) == (dst is None) == (src_perm is None):
        raise ValueError("give src, dst and src_perm, or none of them")
    idx = I32
    if src is not None:
        for name, a in (("src", src), ("dst", dst), ("src_perm", src_perm)):
            if a.shape != (n_edges,) or a.dtype != src.dtype or not a.is_cuda or not a.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [n_edges] device tensor of the index dtype")
        idx = _index_dtype(src)
    if n_nodes is None:
        if src is not None:
            raise ValueError("n_nodes is required with indices")
        n_nodes = n_edges
    if grad_out.shape != (n_nodes, h.dim_out):
        raise ValueError("grad_out must be [n_nodes, dim_out]")
    gx = torch.empty_like(x) if grad_x is None else grad_x
    gsh = torch.empty_like(sh) if grad_sh is None else grad_sh
    gw = torch.empty_like(w) if grad_w is None else grad_w
    for name, a, ref in (("grad_x", gx, x), ("grad_sh", gsh, sh), ("grad_w", gw, w)):
        if a.shape != ref.shape or a.dtype != t or not a.is_contiguous():
            raise ValueError(f"{name} has the wrong shape or dtype")
    need = tp_conv_bwd_workspace(h, n_edges, batch=src is None and n_edges > 0)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if row_ptr is None:
        _check(lib.tp_conv_bwd(h._h, _ptr(x), n_src, _ptr(sh), _ptr(w), _ptr(src), _ptr(dst), _ptr(src_perm), idx,
                               n_edges, n_nodes, _ptr(grad_out), _ptr(gx), _ptr(gsh), _ptr(gw), _ptr(workspace),
                               wbytes, _stream_ptr(x.device)))
    else:
        _check(lib.tp_conv_bwd_rowptr(h._h, _ptr(x), n_src, _ptr(sh), _ptr(w), _ptr(src), _ptr(dst), _ptr(src_perm),
                                      _ptr(row_ptr), _ptr(src_row_ptr), idx, n_edges, n_nodes, _ptr(grad_out),
                                      _ptr(gx), _ptr(gsh), _ptr(gw), _ptr(workspace), wbytes,
                                      _stream_ptr(x.device)))
    return gx, gsh, gw


# ---------------------------------------------------------------- symcon

class SymconHandle:
    def __init__(self, raw, layout, dtype):
        self._h = raw
        self.layout = layout
        self.dtype = dtype

    def _q(self, key):
        v = ctypes.c_int64()
        _check(lib.symcon_query(self._h, key, ctypes.byref(v)))
        return v.value

    dim_in = property(lambda s: s._q(Q_DIM_IN))
    dim_out = property(lambda s: s._q(Q_DIM_OUT))
    weight_numel = property(lambda s: s._q(Q_WEIGHT_NUMEL))
    num_couplings = property(lambda s: s._q(Q_NUM_COUPLINGS))
    num_terms = property(lambda s: s._q(Q_NUM_TERMS))
    specialized = property(lambda s: bool(s._q(Q_SPECIALIZED)))
    mul = property(lambda s: s._q(Q_MUL))
    num_elements = property(lambda s: s._q(Q_NUM_ELEMENTS))
    num_monomial_products = property(lambda s: s._q(Q_NUM_MONOMIALS))

    def coupling_info(self, c):
        v = (ctypes.c_int64 * 4)()
        _check(lib.symcon_coupling_info(self._h, c, v))
        return dict(zip(("degree", "out_block", "k", "l"), list(v)))

    def coupling_dense(self, c, n_components):
        i = self.coupling_info(c)
        shape = (n_components,) * i["degree"] + (2 * i["l"] + 1,)
        out = np.zeros(int(np.prod(shape)))
        _check(lib.symcon_coupling_dense(self._h, c, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
        return out.reshape(shape)

    def __del__(self):
        if getattr(self, "_h", None) and lib is not None:
            lib.symcon_destroy(self._h)
            self._h = None


def symcon_create(irreps_in, irreps_out, max_degree=3, num_elements=1, layout="ir_mul", dtype="f32",
                  validate=False, force_generic=False):
    raw = ctypes.c_void_p()
    _check(lib.symcon_create(irreps_in.encode(), irreps_out.encode(), max_degree, num_elements,
                             _LAYOUTS[layout], _DTYPES[dtype], _flags(False, validate, force_generic),
                             ctypes.byref(raw)))
    return SymconHandle(raw, layout, dtype)


def symcon_fwd(h, x, species, w, out=None):
    """Symmetric contraction of x [n_atoms, dim_in] with the weights of each
    atom's element (species int32/int64 [n_atoms]); returns [n_atoms, dim_out]."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n = x.shape[0]
    if x.shape[1] != h.dim_in or w.shape != (h.num_elements, h.weight_numel):
        raise ValueError("operand shapes do not match the descriptor")
    if species.shape != (n,) or not species.is_cuda or not species.is_contiguous():
        raise ValueError("species must be a contiguous [n_atoms] device tensor")
    idx = _index_dtype(species)
    if out is None:
        out = torch.empty((n, h.dim_out), dtype=t, device=x.device)
    elif out.shape != (n, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.symcon_fwd(h._h, _ptr(x), _ptr(species), idx, _ptr(w), n, _ptr(out), _stream_ptr(x.device)))
    return out


def symcon_bwd_workspace(h, n_atoms):
    """Bytes of device workspace ``symcon_bwd`` needs for ``n_atoms`` atoms."""
    v = ctypes.c_size_t()
    _check(lib.symcon_bwd_workspace(h._h, n_atoms, ctypes.byref(v)))
    return v.value


def symcon_bwd(h, x, species, w, grad_out, species_perm, workspace=None, grad_x=None, grad_w=None):
    """Gradients (grad_x, grad_w) of ``symcon_fwd`` for ``grad_out``
    [n_atoms, dim_out].  ``species_perm`` lists the atom ids ordered by
    element (a stable argsort of species).  The workspace and the gradients
    are allocated if not given."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("w", w), ("grad_out", grad_out)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n = x.shape[0]
    if x.shape[1] != h.dim_in or grad_out.shape != (n, h.dim_out) or w.shape != (h.num_elements, h.weight_numel):
        raise ValueError("operand shapes do not match the descriptor")
    for name, a in (("species", species), ("species_perm", species_perm)):
        if a.shape != (n,) or a.dtype != species.dtype or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n_atoms] device tensor of one integer dtype")
    gx = torch.empty_like(x) if grad_x is None else grad_x
    gw = torch.empty_like(w) if grad_w is None else grad_w
    if gx.shape != x.shape or gw.shape != w.shape or gx.dtype != t or gw.dtype != t:
        raise ValueError("gradient buffers have the wrong shape or dtype")
    if workspace is None:
        workspace = torch.empty(symcon_bwd_workspace(h, n), dtype=torch.uint8, device=x.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib.symcon_bwd(h._h, _ptr(x), _ptr(species), _ptr(species_perm), _index_dtype(species), _ptr(w),
                          _ptr(grad_out), n, _ptr(gx), _ptr(gw), _ptr(workspace), wbytes, _stream_ptr(x.device)))
    return gx, gw


NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024   # SEGPOLY_NOALLOC_SCRATCH_BYTES


def symcon_bwd_noalloc(h, x, species, w, grad_out, species_perm, grad_x=None, grad_w=None):
    """``symcon_bwd`` through the allocation-free entry point (its workspace
    is the library's fixed device scratch).  The gradients are allocated
    here if not given (the C call itself allocates nothing)."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("w", w), ("grad_out", grad_out)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n = x.shape[0]
    if x.shape[1] != h.dim_in or grad_out.shape != (n, h.dim_out) or w.shape != (h.num_elements, h.weight_numel):
        raise ValueError("operand shapes do not match the descriptor")
    for name, a in (("species", species), ("species_perm", species_perm)):
        if a.shape != (n,) or a.dtype != species.dtype or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n_atoms] device tensor of one integer dtype")
    gx = torch.empty_like(x) if grad_x is None else grad_x
    gw = torch.empty_like(w) if grad_w is None else grad_w
    if gx.shape != x.shape or gw.shape != w.shape or gx.dtype != t or gw.dtype != t:
        raise ValueError("gradient buffers have the wrong shape or dtype")
    _check(lib.symcon_bwd_noalloc(h._h, _ptr(x), _ptr(species), _ptr(species_perm), _index_dtype(species), _ptr(w),
                                  _ptr(grad_out), n, _ptr(gx), _ptr(gw), _stream_ptr(x.device)))
    return gx, gw


# ---------------------------------------------------------------- linear

class LinearHandle:
    def __init__(self, raw, layout, dtype):
        self._h = raw
        self.layout = layout
        self.dtype = dtype

    def _q(self, key):
        v = ctypes.c_int64()
        _check(lib.linear_query(self._h, key, ctypes.byref(v)))
        return v.value

    dim_in = property(lambda s: s._q(Q_DIM_IN))
    dim_out = property(lambda s: s._q(Q_DIM_OUT))
    weight_numel = property(lambda s: s._q(Q_WEIGHT_NUMEL))
    num_segments = property(lambda s: s._q(Q_NUM_PATHS))

    def __del__(self):
        if getattr(self, "_h", None) and lib is not None:
            lib.linear_destroy(self._h)
            self._h = None


def linear_create(irreps_in, irreps_out, layout="ir_mul", dtype="f32", validate=False):
    raw = ctypes.c_void_p()
    _check(lib.linear_create(irreps_in.encode(), irreps_out.encode(), _LAYOUTS[layout], _DTYPES[dtype],
                             VALIDATE if validate else 0, ctypes.byref(raw)))
    return LinearHandle(raw, layout, dtype)


def _lin_common(h, x, w, classes, num_classes):
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {t} device tensor")
    n = x.shape[0]
    if x.shape[1] != h.dim_in or w.shape[-1] != h.weight_numel:
        raise ValueError("operand widths do not match the descriptor")
    idx, nc = I32, 1
    if classes is not None:
        if classes.shape != (n,) or not classes.is_cuda or not classes.is_contiguous():
            raise ValueError("classes must be a contiguous [n] device tensor")
        idx = _index_dtype(classes)
        nc = w.shape[0] if num_classes is None else num_classes
        if w.shape[0] != nc:
            raise ValueError("class-indexed weights are [num_classes, weight_numel]")
    elif w.shape[0] != 1:
        raise ValueError("shared weights are one row [1, weight_numel]")
    return t, n, idx, nc


def linear_fwd(h, x, w, classes=None, num_classes=None, out=None):
    """Equivariant linear map of x [n, dim_in] with shared weights [1,
    weight_numel] or class-indexed weights [num_classes, weight_numel]
    (``classes`` [n] int32/int64)."""
    import torch
    t, n, idx, nc = _lin_common(h, x, w, classes, num_classes)
    if out is None:
        out = torch.empty((n, h.dim_out), dtype=t, device=x.device)
    elif out.shape != (n, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.linear_fwd(h._h, _ptr(x), _ptr(w), _ptr(classes), idx, nc, n, _ptr(out), _stream_ptr(x.device)))
    return out


def linear_bwd_workspace(h, n, num_classes=0):
    v = ctypes.c_size_t()
    _check(lib.linear_bwd_workspace(h._h, n, num_classes, ctypes.byref(v)))
    return v.value


def linear_bwd(h, x, w, grad_out, classes=None, num_classes=None, need_dw=True, workspace=None):
    """Gradients (grad_x, grad_w or None) of ``linear_fwd`` for ``grad_out``
    [n, dim_out]; grad_w is shaped like w (one row per class with
    ``classes``)."""
    import torch
    t, n, idx, nc = _lin_common(h, x, w, classes, num_classes)
    if grad_out.shape != (n, h.dim_out) or grad_out.dtype != t or not grad_out.is_contiguous():
        raise ValueError("grad_out has the wrong shape or dtype")
    gx = torch.empty_like(x)
    gw = torch.empty_like(w) if need_dw else None
    if need_dw and workspace is None:
        workspace = torch.empty(max(1, linear_bwd_workspace(h, n, nc if classes is not None else 0)),
                                dtype=torch.uint8, device=x.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.linear_bwd(h._h, _ptr(x), _ptr(w), _ptr(grad_out), _ptr(classes), idx, nc, n, _ptr(gx), _ptr(gw),
                          _ptr(workspace), wbytes, _stream_ptr(x.device)))
    return gx, gw


# ---------------------------------------------------------------- fully connected product

class FctpHandle:
    def __init__(self, raw, layout, dtype):
        self._h = raw
        self.layout = layout
        self.dtype = dtype

    def _q(self, key):
        v = ctypes.c_int64()
        _check(lib.fctp_query(self._h, key, ctypes.byref(v)))
        return v.value

    dim_in1 = property(lambda s: s._q(Q_DIM_IN1))
    dim_in2 = property(lambda s: s._q(Q_DIM_IN2))
    dim_out = property(lambda s: s._q(Q_DIM_OUT))
    weight_numel = property(lambda s: s._q(Q_WEIGHT_NUMEL))
    num_paths = property(lambda s: s._q(Q_NUM_PATHS))

    def path_info(self, p):
        """(i, j, o, weight offset) of path p."""
        info = (ctypes.c_int64 * 4)()
        _check(lib.fctp_path_info(self._h, p, info))
        return tuple(info)

    def __del__(self):
        if getattr(self, "_h", None) and lib is not None:
            lib.fctp_destroy(self._h)
            self._h = None


def fctp_create(irreps_in1, irreps_in2, irreps_out, layout="mul_ir", dtype="f32", validate=False, reduce="sum"):
    """Fully connected (uvw) tensor product (batch form with shared weights;
    convolution form with per-edge or shared weights, ``reduce`` "sum" or
    "mean")."""
    if reduce not in ("sum", "mean"):
        raise ValueError("reduce is 'sum' or 'mean'")
    raw = ctypes.c_void_p()
    flags = (VALIDATE if validate else 0) | (REDUCE_MEAN if reduce == "mean" else 0)
    _check(lib.fctp_create(irreps_in1.encode(), irreps_in2.encode(), irreps_out.encode(), _LAYOUTS[layout],
                           _DTYPES[dtype], flags, ctypes.byref(raw)))
    return FctpHandle(raw, layout, dtype)


def _fc_check(h, per_sample=None, **tensors):
    """Checks the operands; returns (dtype, n, per_sample).  Weights are one
    shared row [1, weight_numel] or one row per sample [n, weight_numel]
    (n > 1); ``per_sample`` True or False insists on one of the two."""
    t = _torch_dtype(h.dtype)
    n = None
    widths = {"x1": h.dim_in1, "x2": h.dim_in2, "grad_out": h.dim_out}
    w = None
    for name, a in tensors.items():
        if a is None:
            continue
        if a.dtype != t or not a.is_cuda or not a.is_contiguous() or a.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-d {t} device tensor")
        if name == "w":
            w = a
            continue
        if a.shape[1] != widths[name]:
            raise ValueError(f"{name} width does not match the descriptor")
        if n is not None and a.shape[0] != n:
            raise ValueError("operands have different sample counts")
        n = a.shape[0]
    per = bool(per_sample)
    if w is not None:
        if w.shape[1] != h.weight_numel:
            raise ValueError("weight width does not match the descriptor")
        if per_sample is None:
            per = w.shape[0] != 1
        if per and n is not None and w.shape[0] != n:
            raise ValueError("per-sample weights need one row per sample [n, weight_numel]")
        if not per and w.shape[0] != 1:
            raise ValueError("shared weights are one row [1, weight_numel]")
    return t, n, per


def fctp_fwd(h, x1, x2, w, out=None):
    """out [n, dim_out] for x1 [n, dim_in1], x2 [n, dim_in2] and w: one
    shared row [1, weight_numel] (matrix-core kernels), or one row per sample
    [n, weight_numel] with n > 1 (the per-sample kernel)."""
    import torch
    t, n, per = _fc_check(h, x1=x1, x2=x2, w=w)
    if out is None:
        out = torch.empty((n, h.dim_out), dtype=t, device=x1.device)
    elif out.shape != (n, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    fn = lib.fctp_fwd_per_sample if per else lib.fctp_fwd
    _check(fn(h._h, _ptr(x1), _ptr(x2), _ptr(w), n, _ptr(out), _stream_ptr(x1.device)))
    return out


def fctp_fwd_per_sample(h, x1, x2, w, out=None):
    """out [n, dim_out] for x1 [n, dim_in1], x2 [n, dim_in2] and one weight
    row per sample, w [n, weight_numel] (any n, 1 included)."""
    import torch
    t, n, _ = _fc_check(h, per_sample=True, x1=x1, x2=x2, w=w)
    if out is None:
        out = torch.empty((n, h.dim_out), dtype=t, device=x1.device)
    elif out.shape != (n, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.fctp_fwd_per_sample(h._h, _ptr(x1), _ptr(x2), _ptr(w), n, _ptr(out), _stream_ptr(x1.device)))
    return out


def fctp_bwd_per_sample(h, x1, x2, w, grad_out, need=(True, True, True)):
    """(grad_x1, grad_x2, grad_w) of ``fctp_fwd_per_sample``, grad_w
    [n, weight_numel]; each None where ``need`` is False."""
    import torch
    _, n, _ = _fc_check(h, per_sample=True, x1=x1, x2=x2, w=w, grad_out=grad_out)
    g1 = torch.empty_like(x1) if need[0] else None
    g2 = torch.empty_like(x2) if need[1] else None
    gw = torch.empty_like(w) if need[2] else None
    _check(lib.fctp_bwd_per_sample(h._h, _ptr(x1), _ptr(x2), _ptr(w), _ptr(grad_out), n, _ptr(g1), _ptr(g2),
                                   _ptr(gw), _stream_ptr(x1.device)))
    return g1, g2, gw


def fctp_bwd_workspace(h, n):
    v = ctypes.c_size_t()
    _check(lib.fctp_bwd_workspace(h._h, n, ctypes.byref(v)))
    return v.value


def fctp_bwd(h, x1, x2, w, grad_out, need=(True, True, True), workspace=None):
    """(grad_x1, grad_x2, grad_w), each None where ``need`` is False; with
    per-sample weights [n, weight_numel] (n > 1) grad_w has one row per
    sample and the per-sample kernel runs (no workspace)."""
    import torch
    _, n, per = _fc_check(h, x1=x1, x2=x2, w=w, grad_out=grad_out)
    if per:
        return fctp_bwd_per_sample(h, x1, x2, w, grad_out, need)
    g1 = torch.empty_like(x1) if need[0] else None
    g2 = torch.empty_like(x2) if need[1] else None
    gw = torch.empty_like(w) if need[2] else None
    if any(need) and workspace is None:
        workspace = torch.empty(max(1, fctp_bwd_workspace(h, n)), dtype=torch.uint8, device=x1.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.fctp_bwd(h._h, _ptr(x1), _ptr(x2), _ptr(w), _ptr(grad_out), n, _ptr(g1), _ptr(g2), _ptr(gw),
                        _ptr(workspace), wbytes, _stream_ptr(x1.device)))
    return g1, g2, gw


def fctp_conv_fwd(h, x, sh, w, src, dst, n_nodes, out=None):
    """Convolution form: out [n_nodes, dim_out] = sum (or mean) over the
    edges into each node of the product of x[src[e]] and sh[e] with weight
    row w[e] (w [n_edges, weight_numel]) or the shared row (w [1, ...])."""
    import torch
    t = _torch_dtype(h.dtype)
    for name, a in (("x", x), ("sh", sh), ("w", w)):
        if a.dtype != t or not a.is_cuda or not a.is_contiguous() or a.dim() != 2:
            raise ValueError(f"{name} must be a contiguous 2-d {t} device tensor")
    n_edges = sh.shape[0]
    if x.shape[1] != h.dim_in1 or sh.shape[1] != h.dim_in2 or w.shape[1] != h.weight_numel:
        raise ValueError("operand widths do not match the descriptor")
    if w.shape[0] not in (1, n_edges):
        raise ValueError("weights are [n_edges, weight_numel] or [1, weight_numel]")
    for name, a in (("src", src), ("dst", dst)):
        if a.shape != (n_edges,) or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n_edges] device tensor")
    if src.dtype != dst.dtype:
        raise ValueError("src and dst must have the same dtype")
    if out is None:
        out = torch.empty((n_nodes, h.dim_out), dtype=t, device=x.device)
    elif out.shape != (n_nodes, h.dim_out) or out.dtype != t or not out.is_contiguous():
        raise ValueError("out has the wrong shape or dtype")
    _check(lib.fctp_conv_fwd(h._h, _ptr(x), x.shape[0], _ptr(sh), _ptr(w), w.shape[0], _ptr(src), _ptr(dst),
                             _index_dtype(src), n_edges, n_nodes, _ptr(out), _stream_ptr(x.device)))
    return out


def fctp_conv_bwd_workspace(h, n_edges, w_rows=None):
    v = ctypes.c_size_t()
    _check(lib.fctp_conv_bwd_workspace(h._h, n_edges, n_edges if w_rows is None else w_rows, ctypes.byref(v)))
    return v.value


def fctp_conv_bwd(h, x, sh, w, grad_out, src, dst, src_perm, n_nodes=None, workspace=None):
    """(grad_x, grad_sh, grad_w) of ``fctp_conv_fwd`` with one weight row per
    edge or one shared row (grad_w shaped like w); ``src_perm`` orders the
    edges by source (stable argsort of src)."""
    import torch
    n_edges = sh.shape[0]
    n_nodes = grad_out.shape[0] if n_nodes is None else n_nodes
    if w.shape[0] not in (1, n_edges):
        raise ValueError("weights: one row per edge, or one shared row")
    for name, a in (("src", src), ("dst", dst), ("src_perm", src_perm)):
        if a.shape != (n_edges,) or a.dtype != src.dtype or not a.is_cuda or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n_edges] device tensor of src's dtype")
    if grad_out.shape != (n_nodes, h.dim_out) or not grad_out.is_contiguous():
        raise ValueError("grad_out has the wrong shape")
    gx, gs, gw = torch.empty_like(x), torch.empty_like(sh), torch.empty_like(w)
    if workspace is None:
        workspace = torch.empty(max(1, fctp_conv_bwd_workspace(h, n_edges, w.shape[0])), dtype=torch.uint8,
                                device=x.device)
    wbytes = workspace.numel() * workspace.element_size()
    _check(lib.fctp_conv_bwd(h._h, _ptr(x), x.shape[0], _ptr(sh), _ptr(w), w.shape[0], _ptr(src), _ptr(dst),
                             _ptr(src_perm), _index_dtype(src), n_edges, n_nodes, _ptr(grad_out), _ptr(gx), _ptr(gs),
                             _ptr(gw), _ptr(workspace), wbytes, _stream_ptr(x.device)))
    return gx, gs, gw


# ---------------------------------------------------------------- edge embedding assembly

def _dt_of(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float64:
        return F64
    raise ValueError("float32 or float64 tensors only")


def edge_scalars_fwd(edge_emb, src, dst, src_scalars=None, dst_scalars=None, out=None):
    """[edge_emb[e], src_scalars[src[e]], dst_scalars[dst[e]]] per edge (the
    convolution layer's edge MLP input)."""
    import torch
    n_edges, d_emb = edge_emb.shape
    d_src = 0 if src_scalars is None else src_scalars.shape[1]
    d_dst = 0 if dst_scalars is None else dst_scalars.shape[1]
    n_src = 0 if src_scalars is None else src_scalars.shape[0]
    n_dst = 0 if dst_scalars is None else dst_scalars.shape[0]
    for a in (edge_emb, src_scalars, dst_scalars):
        if a is not None and (a.dtype != edge_emb.dtype or not a.is_cuda or not a.is_contiguous()):
            raise ValueError("operands must be contiguous device tensors of one dtype")
    if out is None:
        out = torch.empty((n_edges, d_emb + d_src + d_dst), dtype=edge_emb.dtype, device=edge_emb.device)
    _check(lib.edge_scalars_fwd(_dt_of(edge_emb), _ptr(edge_emb), d_emb, _ptr(src_scalars), d_src, _ptr(dst_scalars),
                                d_dst, _ptr(src), _ptr(dst), _index_dtype(src), n_edges, n_src, n_dst, _ptr(out),
                                _stream_ptr(edge_emb.device)))
    return out


def edge_scalars_bwd(grad_out, d_emb, d_src, d_dst, src, dst, src_perm, n_src, n_dst):
    """(grad_emb, grad_src or None, grad_dst or None) of ``edge_scalars_fwd``."""
    import torch
    n_edges = grad_out.shape[0]
    kw = dict(dtype=grad_out.dtype, device=grad_out.device)
    ge = torch.empty((n_edges, d_emb), **kw)
    gs = torch.empty((n_src, d_src), **kw) if d_src else None
    gd = torch.empty((n_dst, d_dst), **kw) if d_dst else None
    _check(lib.edge_scalars_bwd(_dt_of(grad_out), _ptr(grad_out), d_emb, d_src, d_dst, _ptr(src), _ptr(dst),
                                _ptr(src_perm), _index_dtype(src), n_edges, n_src, n_dst, _ptr(ge), _ptr(gs), _ptr(gd),
                                _stream_ptr(grad_out.device)))
    return ge, gs, gd


# ---------------------------------------------------------------- spherical harmonics

def _sh_dtype(vec):
    import torch
    if vec.dtype == torch.float32:
        return F32
    if vec.dtype == torch.float64:
        return F64
    raise TypeError("vectors must be float32 or float64")


def sh_fwd(vec, lmax, normalize=True, out=None):
    """Real spherical harmonics of degrees 0..lmax of vec [n, 3] (device):
    [n, (lmax + 1)^2]."""
    import torch
    if vec.dim() != 2 or vec.shape[1] != 3 or not vec.is_cuda or not vec.is_contiguous():
        raise ValueError("vec must be a contiguous [n, 3] device tensor")
    n = vec.shape[0]
    if out is None:
        out = torch.empty((n, (lmax + 1) ** 2), dtype=vec.dtype, device=vec.device)
    _check(lib.sh_fwd(lmax, 1 if normalize else 0, _sh_dtype(vec), _ptr(vec), n, _ptr(out), _stream_ptr(vec.device)))
    return out


def sh_bwd(vec, grad_sh, lmax, normalize=True):
    """dL/dvec [n, 3] for grad_sh = dL/dY [n, (lmax + 1)^2]."""
    import torch
    n = vec.shape[0]
    if grad_sh.shape != (n, (lmax + 1) ** 2) or grad_sh.dtype != vec.dtype or not grad_sh.is_contiguous():
        raise ValueError("grad_sh must be [n, (lmax + 1)^2] of the vectors' dtype")
    out = torch.empty_like(vec)
    _check(lib.sh_bwd(lmax, 1 if normalize else 0, _sh_dtype(vec), _ptr(vec), _ptr(grad_sh), n, _ptr(out),
                      _stream_ptr(vec.device)))
    return out
