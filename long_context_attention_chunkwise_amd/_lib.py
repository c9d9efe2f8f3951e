"""ctypes binding of liblightning.so (declared in include/la.h).

Argument marshalling only: shapes, dtypes and device checks, output
allocation with torch, and the current torch stream.  Every step of the
computation runs in the library's HIP kernels; if the library is missing or
fails to load, every call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblightning.so")

LA_F32, LA_BF16 = 0, 1
LA_OK = 0
STATUS_NAMES = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_UNSUPPORTED", 4: "LA_ERR_ALIGN",
                5: "LA_ERR_ALIAS", 6: "LA_ERR_WORKSPACE", 7: "LA_ERR_HIP", 8: "LA_ERR_TOO_LARGE"}
EXPORTS = ("la_forward", "la_forward_ex", "la_forward_states", "la_forward_outputs", "la_forward_workspace_bytes",
           "la_forward_variant", "la_forward_variant_workspace_bytes", "la_backward", "la_backward_workspace_bytes",
           "la_decode_step", "la_status_str", "la_forward_noalloc", "la_forward_state",
           "la_forward_state_workspace_bytes", "la_backward_state", "la_backward_state_workspace_bytes")
LA_NOALLOC_SCRATCH_BYTES = 64 << 20
LA_FMAP_IDENTITY, LA_FMAP_RELU = 0, 1

_lib = None


class LAError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


def load_library(path=LIB_PATH):
    """Load liblightning.so and declare its C signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run long_context_attention_chunkwise_amd/build.py")
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    i32 = ctypes.c_int
    lib.la_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp]
    lib.la_forward.restype = i32
    lib.la_forward_ex.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp, sz, vp]
    lib.la_forward_ex.restype = i32
    lib.la_forward_states.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, vp, vp, sz, vp]
    lib.la_forward_states.restype = i32
    lib.la_forward_outputs.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp, sz,
                                       vp]
    lib.la_forward_outputs.restype = i32
    lib.la_forward_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, i32]
    lib.la_forward_workspace_bytes.restype = sz
    f32 = ctypes.c_float
    lib.la_forward_variant.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, i32, i32, i32,
                                       f32, vp, vp, vp, vp, vp, sz, vp]
    lib.la_forward_variant.restype = i32
    lib.la_forward_variant_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, i32, i32, i32]
    lib.la_forward_variant_workspace_bytes.restype = sz
    lib.la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp, vp,
                                vp, vp, sz, vp]
    lib.la_backward.restype = i32
    lib.la_backward_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, i32]
    lib.la_backward_workspace_bytes.restype = sz
    lib.la_forward_state.argtypes = [vp, vp, i64, i64, i64, i64, i64, i32, vp, vp, vp, sz, vp]
    lib.la_forward_state.restype = i32
    lib.la_forward_state_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i32]
    lib.la_forward_state_workspace_bytes.restype = sz
    lib.la_backward_state.argtypes = [vp, vp, i64, i64, i64, i64, i64, i64, i32, vp, vp, vp, sz, vp]
    lib.la_backward_state.restype = i32
    lib.la_backward_state_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i32]
    lib.la_backward_state_workspace_bytes.restype = sz
    lib.la_forward_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp]
    lib.la_forward_noalloc.restype = i32
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp]
    lib.la_decode_step.restype = i32
    lib.la_status_str.argtypes = [i32]
    lib.la_status_str.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_str(status):
    return load_library().la_status_str(int(status)).decode()


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t == torch.float32:
        return LA_F32
    if t == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, ndim, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(workspace, nbytes, device):
    """The scratch buffer for one call: None when the call needs none, a new
    buffer when none is given or the given one is smaller than `nbytes`, else
    the caller's buffer, which must be a contiguous tensor on `device`."""
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        _check_tensor("workspace", workspace, workspace.dim() if isinstance(workspace, torch.Tensor) else 1, device)
        if workspace.numel() * workspace.element_size() >= nbytes:
            return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def workspace_bytes(B, Hq, Hkv, N, d, dv, block=64, dtype=None):
    """Bytes of scratch la_forward_ex needs on the current device."""
    torch = _torch()
    code = _dtype_code(dtype if dtype is not None else torch.bfloat16)
    return int(load_library().la_forward_workspace_bytes(B, Hq, Hkv, N, d, dv, block, code))


def forward(q, k, v, block=64, out_dtype=None, s_in=None, return_state=False, out=None, s_out=None,
            workspace=None):
    """Causal chunkwise linear attention forward pass (la_forward_ex).

    q [B,Hq,N,d], k [B,Hkv,N,d], v [B,Hkv,N,dv] on one GPU, float32 or
    bfloat16 (all the same).  Returns o [B,Hq,N,dv] (out_dtype, default the
    input dtype) and, with return_state, the float32 final state
    [B,Hkv,d,dv].  s_in is an optional float32 initial state.
    """
    torch = _torch()
    lib = load_library()
    _check_tensor("q", q, 4, None)
    dev = q.device
    _check_tensor("k", k, 4, dev)
    _check_tensor("v", v, 4, dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, dv):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    in_code = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dtype)
    if s_in is not None:
        _check_tensor("s_in", s_in, 4, dev)
        if s_in.dtype != torch.float32 or tuple(s_in.shape) != (B, Hkv, d, dv):
            raise ValueError("s_in must be float32 [B, Hkv, d, dv]")
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, Hq, N, dv), dtype=out_dtype, device=dev)
        else:
            _check_tensor("out", out, 4, dev)
            if out.dtype != out_dtype or tuple(out.shape) != (B, Hq, N, dv):
                raise ValueError("out has the wrong dtype or shape")
        if return_state and s_out is None:
            s_out = torch.empty((B, Hkv, d, dv), dtype=torch.float32, device=dev)
        if s_out is not None:
            _check_tensor("s_out", s_out, 4, dev)
            if s_out.dtype != torch.float32 or tuple(s_out.shape) != (B, Hkv, d, dv):
                raise ValueError("s_out must be float32 [B, Hkv, d, dv]")
        ws_bytes = int(lib.la_forward_workspace_bytes(B, Hq, Hkv, N, d, dv, block, in_code))
        workspace = _workspace(workspace, ws_bytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, dv, block, in_code,
                               out_code, _ptr(s_in), _ptr(s_out), _ptr(workspace),
                               ws_bytes, ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_forward_ex")
    if return_state:
        return out, s_out
    return out


def forward_state(k, v, s_in=None, out=None, workspace=None):
    """la_forward_state: the final state s_in + sum_t k_t^T v_t per (batch,
    KV head) without outputs.  k [B,Hkv,N,d], v [B,Hkv,N,dv] (float32 or
    bfloat16, the same); s_in optional float32 [B,Hkv,d,dv]; returns the
    float32 state [B,Hkv,d,dv] (`out`, which may be s_in, when given)."""
    torch = _torch()
    lib = load_library()
    _check_tensor("k", k, 4, None)
    dev = k.device
    _check_tensor("v", v, 4, dev)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share one dtype")
    B, Hkv, N, d = k.shape
    dv = v.shape[3]
    if tuple(v.shape[:3]) != (B, Hkv, N):
        raise ValueError(f"shape mismatch: k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("s_in", s_in), ("out", out)):
        if t is not None:
            _check_tensor(name, t, 4, dev)
            if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, d, dv):
                raise ValueError(f"{name} must be float32 [B, Hkv, d, dv]")
    code = _dtype_code(k.dtype)
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, Hkv, d, dv), dtype=torch.float32, device=dev)
        ws_bytes = int(lib.la_forward_state_workspace_bytes(B, Hkv, N, d, dv, code))
        workspace = _workspace(workspace, ws_bytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_forward_state(_ptr(k), _ptr(v), B, Hkv, N, d, dv, code, _ptr(s_in), _ptr(out),
                                  _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_forward_state")
    return out


def backward_state(q, grad_o, Hkv, grad_s_out=None, out=None, workspace=None):
    """la_backward_state: grad_s_in = grad_s_out + sum over each KV head's
    query heads and all tokens of q_t^T grad_o_t, without dq, dk, dv.  q
    [B,Hq,N,d], grad_o [B,Hq,N,dv] (float32 or bfloat16, the same); Hkv KV
    heads; returns float32 [B,Hkv,d,dv] (`out`, which may be grad_s_out)."""
    torch = _torch()
    lib = load_library()
    _check_tensor("q", q, 4, None)
    dev = q.device
    _check_tensor("grad_o", grad_o, 4, dev)
    if q.dtype != grad_o.dtype:
        raise TypeError("q and grad_o must share one dtype")
    B, Hq, N, d = q.shape
    dv = grad_o.shape[3]
    if tuple(grad_o.shape[:3]) != (B, Hq, N):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, grad_o {tuple(grad_o.shape)}")
    for name, t in (("grad_s_out", grad_s_out), ("out", out)):
        if t is not None:
            _check_tensor(name, t, 4, dev)
            if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, d, dv):
                raise ValueError(f"{name} must be float32 [B, Hkv, d, dv]")
    code = _dtype_code(q.dtype)
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, Hkv, d, dv), dtype=torch.float32, device=dev)
        ws_bytes = int(lib.la_backward_state_workspace_bytes(B, Hq, Hkv, N, d, dv, code))
        workspace = _workspace(workspace, ws_bytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_backward_state(_ptr(q), _ptr(grad_o), B, Hq, Hkv, N, d, dv, code, _ptr(grad_s_out),
                                   _ptr(out), _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_backward_state")
    return out


def forward_noalloc(q, k, v, out, block=64, s_in=None, s_out=None):
    """la_forward_noalloc: the forward pass of `forward` writing into the
    caller's `out` (and `s_out`, optional), with the library's fixed device
    scratch as workspace; nothing is allocated, here or in the library.
    The output dtype is out.dtype.  Raises LAError(LA_ERR_TOO_LARGE) when the
    problem needs more than LA_NOALLOC_SCRATCH_BYTES of workspace."""
    torch = _torch()
    lib = load_library()
    _check_tensor("q", q, 4, None)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("out", out)):
        _check_tensor(name, t, 4, dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, dv) or tuple(out.shape) != (B, Hq, N, dv):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}, "
                         f"out {tuple(out.shape)}")
    for name, t in (("s_in", s_in), ("s_out", s_out)):
        if t is not None:
            _check_tensor(name, t, 4, dev)
            if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, d, dv):
                raise ValueError(f"{name} must be float32 [B, Hkv, d, dv]")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, dv, block,
                                    _dtype_code(q.dtype), _dtype_code(out.dtype), _ptr(s_in), _ptr(s_out),
                                    ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_forward_noalloc")
    return out


def forward_variant(q, k, v, causal=True, feature_map="identity", normalize=False, eps=0.0, block=64,
                    out_dtype=None, s_in=None, z_in=None, return_state=False, out=None, s_out=None, z_out=None,
                    workspace=None):
    """Forward variants (la_forward_variant): feature map "identity" or "relu"
    (phi = ReLU on q and k), causal or non-causal, optionally normalised by
    phi(q_t) . z_t + eps.  bf16 or float32 q, k, v; the matrix-core kernels
    serve bf16 at d = dv = 128 (blocks that are multiples of 64), the float32
    FMA kernels every other shape the float32 forward takes (any Hq/Hkv).
    Returns o and, with return_state, (S_out, z_out) (z_out None unless
    normalize)."""
    torch = _torch()
    lib = load_library()
    _check_tensor("q", q, 4, None)
    dev = q.device
    _check_tensor("k", k, 4, dev)
    _check_tensor("v", v, 4, dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    if tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, dv):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    fmaps = {"identity": LA_FMAP_IDENTITY, "relu": LA_FMAP_RELU}
    if feature_map not in fmaps:
        raise ValueError(f"feature_map must be one of {sorted(fmaps)}")
    in_code = _dtype_code(q.dtype)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    out_code = _dtype_code(out_dtype)
    for name, t, shape in (("s_in", s_in, (B, Hkv, d, dv)), ("z_in", z_in, (B, Hkv, d))):
        if t is not None:
            _check_tensor(name, t, len(shape), dev)
            if t.dtype != torch.float32 or tuple(t.shape) != shape:
                raise ValueError(f"{name} must be float32 {list(shape)}")
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, Hq, N, dv), dtype=out_dtype, device=dev)
        _check_tensor("out", out, 4, dev)
        if out.dtype != out_dtype or tuple(out.shape) != (B, Hq, N, dv):
            raise ValueError("out has the wrong dtype or shape")
        if return_state:
            if s_out is None:
                s_out = torch.empty((B, Hkv, d, dv), dtype=torch.float32, device=dev)
            if normalize and z_out is None:
                z_out = torch.empty((B, Hkv, d), dtype=torch.float32, device=dev)
        for name, t, shape in (("s_out", s_out, (B, Hkv, d, dv)), ("z_out", z_out, (B, Hkv, d))):
            if t is not None:
                _check_tensor(name, t, len(shape), dev)
                if t.dtype != torch.float32 or tuple(t.shape) != shape:
                    raise ValueError(f"{name} must be float32 {list(shape)}")
        ws_bytes = int(lib.la_forward_variant_workspace_bytes(B, Hq, Hkv, N, d, dv, block, in_code, int(causal),
                                                              int(normalize)))
        workspace = _workspace(workspace, ws_bytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_forward_variant(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, N, d, dv, block, in_code,
                                    out_code, int(causal), fmaps[feature_map], int(normalize), float(eps),
                                    _ptr(s_in), _ptr(s_out), _ptr(z_in), _ptr(z_out),
                                    _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_forward_variant")
    if return_state:
        return out, s_out, z_out
    return out


def backward_workspace_bytes(B, Hq, Hkv, N, d, dv, block=64, dtype=None):
    """Bytes of scratch la_backward needs on the current device."""
    torch = _torch()
    code = _dtype_code(dtype if dtype is not None else torch.bfloat16)
    return int(load_library().la_backward_workspace_bytes(B, Hq, Hkv, N, d, dv, block, code))


def backward(q, k, v, grad_o, block=64, grad_dtype=None, s_in=None, grad_s_out=None, return_state_grad=False,
             out=None, grad_s_in=None, workspace=None):
    """Gradients of the forward pass (la_backward).

    q, k, v and grad_o = dL/do (bfloat16 or float32, shaped like the
    forward's inputs and output).  Returns (dq, dk, dv) in grad_dtype (default
    the input dtype; float32 inputs take float32 gradients) and,
    with return_state_grad (or a grad_s_in buffer), the float32 gradient on
    the initial state as a fourth item.  s_in is the forward's initial state;
    grad_s_out an optional float32 gradient on its final state.  `out` may
    supply the (dq, dk, dv) buffers.
    """
    torch = _torch()
    lib = load_library()
    _check_tensor("q", q, 4, None)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("grad_o", grad_o)):
        _check_tensor(name, t, 4, dev)
    if not (q.dtype == k.dtype == v.dtype == grad_o.dtype):
        raise TypeError("q, k, v, grad_o must share one dtype")
    B, Hq, N, d = q.shape
    Hkv, dv = k.shape[1], v.shape[3]
    if (tuple(k.shape) != (B, Hkv, N, d) or tuple(v.shape) != (B, Hkv, N, dv)
            or tuple(grad_o.shape) != (B, Hq, N, dv)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}, "
                         f"grad_o {tuple(grad_o.shape)}")
    in_code = _dtype_code(q.dtype)
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    g_code = _dtype_code(grad_dtype)
    for name, t in (("s_in", s_in), ("grad_s_out", grad_s_out)):
        if t is not None:
            _check_tensor(name, t, 4, dev)
            if t.dtype != torch.float32 or tuple(t.shape) != (B, Hkv, d, dv):
                raise ValueError(f"{name} must be float32 [B, Hkv, d, dv]")
    with torch.cuda.device(dev):
        if out is None:
            out = (torch.empty((B, Hq, N, d), dtype=grad_dtype, device=dev),
                   torch.empty((B, Hkv, N, d), dtype=grad_dtype, device=dev),
                   torch.empty((B, Hkv, N, dv), dtype=grad_dtype, device=dev))
        for name, t, shape in zip(("dq", "dk", "dv"), out, ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, dv))):
            _check_tensor(name, t, 4, dev)
            if t.dtype != grad_dtype or tuple(t.shape) != shape:
                raise ValueError(f"{name} has the wrong dtype or shape")
        if return_state_grad and grad_s_in is None:
            grad_s_in = torch.empty((B, Hkv, d, dv), dtype=torch.float32, device=dev)
        if grad_s_in is not None:
            _check_tensor("grad_s_in", grad_s_in, 4, dev)
            if grad_s_in.dtype != torch.float32 or tuple(grad_s_in.shape) != (B, Hkv, d, dv):
                raise ValueError("grad_s_in must be float32 [B, Hkv, d, dv]")
        ws_bytes = int(lib.la_backward_workspace_bytes(B, Hq, Hkv, N, d, dv, block, in_code))
        workspace = _workspace(workspace, ws_bytes, dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(grad_o), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                             B, Hq, Hkv, N, d, dv, block, in_code, g_code, _ptr(s_in), _ptr(grad_s_out),
                             _ptr(grad_s_in), _ptr(workspace), ws_bytes,
                             ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_backward")
    if grad_s_in is not None:
        return out[0], out[1], out[2], grad_s_in
    return tuple(out)


def decode_step(S, q, k, v, out_dtype=None, out=None):
    """One decode token (la_decode_step): S += k^T v in place, o = q S.

    S [B,Hkv,d,dv] float32; q [B,Hq,d], k [B,Hkv,d], v [B,Hkv,dv] bfloat16 or
    float32.  Returns o [B,Hq,dv] (out_dtype, default float32).
    """
    torch = _torch()
    lib = load_library()
    _check_tensor("S", S, 4, None)
    dev = S.device
    _check_tensor("q", q, 3, dev)
    _check_tensor("k", k, 3, dev)
    _check_tensor("v", v, 3, dev)
    if S.dtype != torch.float32:
        raise TypeError("S must be float32")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hkv, d, dv = S.shape
    Hq = q.shape[1]
    if tuple(q.shape) != (B, Hq, d) or tuple(k.shape) != (B, Hkv, d) or tuple(v.shape) != (B, Hkv, dv):
        raise ValueError("decode shapes do not match the state")
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((B, Hq, dv), dtype=out_dtype, device=dev)
        _check_tensor("out", out, 3, dev)
        if out.dtype != out_dtype or tuple(out.shape) != (B, Hq, dv):
            raise ValueError("out has the wrong dtype or shape")
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.la_decode_step(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, d, dv,
                                _dtype_code(q.dtype), _dtype_code(out_dtype), ctypes.c_void_p(stream))
    if st != LA_OK:
        raise LAError(st, "la_decode_step")
    return out
