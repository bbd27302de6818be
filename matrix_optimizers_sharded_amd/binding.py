"""ctypes binding over libmatopt.so (C ABI in include/matopt.h).

Argument marshalling only: tensors are passed as raw device pointers with torch's
current stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: a missing library or a failed call raises MatoptError.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))

MO_F32, MO_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 256 << 20   # MO_NOALLOC_SCRATCH_BYTES in include/matopt.h
ERRORS = {-1: "MO_ERR_INVALID", -2: "MO_ERR_UNSUPPORTED", -3: "MO_ERR_WORKSPACE", -4: "MO_ERR_HIP"}


class MatoptError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class MoMatrix(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("grad", ctypes.c_void_p),
                ("momentum", ctypes.c_void_p), ("x", ctypes.c_void_p), ("out", ctypes.c_void_p)]


class MoNsParams(ctypes.Structure):
    _fields_ = [("a", ctypes.c_float), ("b", ctypes.c_float), ("c", ctypes.c_float),
                ("iters", ctypes.c_int32), ("eps", ctypes.c_float)]


class MoKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("busy_ms", ctypes.c_double)]


_lib = None


def library_path():
    return os.environ.get("MATOPT_LIB", os.path.join(PKG, "lib", "libmatopt.so"))


def load_library():
    """Load libmatopt.so (raises MatoptError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise MatoptError(-4, f"{path} not found; build it with python -m matrix_optimizers_sharded_amd.build")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.muon_workspace_bytes.argtypes = [ctypes.POINTER(MoMatrix), I32, I32]
    lib.muon_workspace_bytes.restype = SZ
    lib.muon_step_batched.argtypes = [ctypes.POINTER(MoMatrix), I32, I32, I32, I32, F,
                                      ctypes.POINTER(MoNsParams), P, SZ, P]
    lib.muon_step_batched.restype = I32
    lib.ns_orthogonalize.argtypes = [ctypes.POINTER(MoMatrix), I32, I32, I32, I32,
                                     ctypes.POINTER(MoNsParams), P, SZ, P]
    lib.ns_orthogonalize.restype = I32
    lib.sign_pack.argtypes = [P, I32, I64, P, P]
    lib.sign_pack.restype = I32
    lib.sign_pack_batched.argtypes = [P, I32, I32, I64, I64, P, P]
    lib.sign_pack_batched.restype = I32
    lib.sign_vote.argtypes = [P, I32, I64, P, P, P]
    lib.sign_vote.restype = I32
    lib.muon_step_batched_noalloc.argtypes = [ctypes.POINTER(MoMatrix), I32, I32, I32, I32, F,
                                              ctypes.POINTER(MoNsParams), P]
    lib.muon_step_batched_noalloc.restype = I32
    lib.muon_step_apply.argtypes = [ctypes.POINTER(MoMatrix), I32, I32, I32, I32, F,
                                    ctypes.POINTER(MoNsParams), F, P, SZ, P]
    lib.muon_step_apply.restype = I32
    lib.sign_unpack.argtypes = [P, I64, I32, P, P]
    lib.sign_unpack.restype = I32
    lib.sign_apply.argtypes = [P, I64, I32, P, F, P]
    lib.sign_apply.restype = I32
    D = ctypes.c_double
    lib.mo_plan_owners.argtypes = [P, P, I32, I32, I32, D, P, P, P]
    lib.mo_plan_owners.restype = I32
    lib.mo_last_error.argtypes = []
    lib.mo_last_error.restype = ctypes.c_char_p
    lib.mo_version.argtypes = []
    lib.mo_version.restype = I32
    lib.mo_profile_begin.argtypes = []
    lib.mo_profile_begin.restype = I32
    lib.mo_profile_end.argtypes = [ctypes.POINTER(MoKernelTime), I32]
    lib.mo_profile_end.restype = I32
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        msg = _lib.mo_last_error().decode(errors="replace")
        raise MatoptError(rc, msg)
    return rc


def version():
    return load_library().mo_version()


def _dtype_code(dt):
    import torch
    if dt == torch.float32:
        return MO_F32
    if dt == torch.bfloat16:
        return MO_BF16
    raise MatoptError(-2, f"unsupported dtype {dt}")


def _stream_ptr(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _one_device(*groups):
    """The device that every tensor in the given lists (or single tensors) is on;
    raises if they differ, since the kernels would then get another GPU's pointers."""
    devs = set()
    for g in groups:
        for t in (g if isinstance(g, (list, tuple)) else [g]):
            if t is not None:
                devs.add(t.device)
    if len(devs) != 1:
        raise MatoptError(-1, f"all tensors must be on one CUDA device, got {sorted(map(str, devs))}")
    return devs.pop()


def _on(dev):
    """Run the enclosed launch with dev current, so the library launches on it."""
    import torch
    return torch.cuda.device(dev)


def _mats(shapes, grads=None, moms=None, xs=None, outs=None):
    arr = (MoMatrix * max(len(shapes), 1))()
    for i, (r, c) in enumerate(shapes):
        arr[i].rows, arr[i].cols = int(r), int(c)
        if grads is not None:
            arr[i].grad = grads[i].data_ptr()
        if moms is not None:
            arr[i].momentum = moms[i].data_ptr()
        if xs is not None:
            arr[i].x = xs[i].data_ptr()
        if outs is not None:
            arr[i].out = outs[i].data_ptr()
    return arr


def workspace_bytes(shapes, compute):
    """Workspace bytes for a list of (rows, cols) with compute dtype torch.float32 or
    torch.bfloat16."""
    lib = load_library()
    n = lib.muon_workspace_bytes(_mats(shapes), len(shapes), _dtype_code(compute))
    if n == 0 and len(shapes) > 0:
        raise MatoptError(-1, lib.mo_last_error().decode())
    return n


class Workspace:
    """Device scratch for the batched calls, grown on demand (torch allocation)."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        import torch
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


def _validate(ts, shapes, name, dtypes=None):
    for t, (r, c) in zip(ts, shapes):
        if not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (r, c):
            raise MatoptError(-1, f"{name}: expected a contiguous CUDA tensor of shape {(r, c)}")
        if dtypes is not None and t.dtype not in dtypes:
            raise MatoptError(-2, f"{name}: unsupported dtype {t.dtype}")


def _ns_params(a, b, c, iters, eps):
    return MoNsParams(float(a), float(b), float(c), int(iters), float(eps))


def muon_step_batched(grads, moms, outs, beta, a, b, c, iters, eps=1e-7, compute=None,
                      workspace=None):
    """In place: moms[i] <- beta*moms[i] + grads[i]; outs[i] <- NS_k(moms[i] / (||.||+eps)).

    grads: list of fp32 or bf16 tensors (one dtype); moms: fp32; outs: fp32 or bf16
    (one dtype); compute: torch.float32 or torch.bfloat16 (bf16 operands, fp32
    accumulation).  workspace: a Workspace (one is made per call if None)."""
    import torch
    lib = load_library()
    if compute is None:
        compute = torch.bfloat16
    shapes = [tuple(g.shape) for g in grads]
    if not (len(grads) == len(moms) == len(outs)):
        raise MatoptError(-1, "grads, moms and outs must have the same length")
    if not shapes:
        return
    _validate(grads, shapes, "grads", (torch.float32, torch.bfloat16))
    _validate(moms, shapes, "moms", (torch.float32,))
    _validate(outs, shapes, "outs", (torch.float32, torch.bfloat16))
    gdt, odt = grads[0].dtype, outs[0].dtype
    if any(g.dtype != gdt for g in grads) or any(o.dtype != odt for o in outs):
        raise MatoptError(-2, "all grads (and all outs) must share one dtype")
    dev = _one_device(grads, moms, outs)
    mats = _mats(shapes, grads=grads, moms=moms, outs=outs)
    nbytes = lib.muon_workspace_bytes(mats, len(shapes), _dtype_code(compute))
    ws = (workspace or Workspace(dev)).get(nbytes)
    _one_device(grads, ws)
    ns = _ns_params(a, b, c, iters, eps)
    with _on(dev):
        _check(lib.muon_step_batched(mats, len(shapes), _dtype_code(gdt), _dtype_code(compute),
                                     _dtype_code(odt), float(beta), ctypes.byref(ns), ws.data_ptr(),
                                     ws.numel(), _stream_ptr(grads[0])))


def muon_step_batched_noalloc(grads, moms, outs, beta, a, b, c, iters, eps=1e-7, compute=None):
    """muon_step_batched without a workspace: the library's own fixed device scratch
    (MO_NOALLOC_SCRATCH_BYTES per GPU) is used and nothing is allocated, here or in
    the library.  Lists needing more scratch raise MatoptError (MO_ERR_WORKSPACE)."""
    import torch
    lib = load_library()
    if compute is None:
        compute = torch.bfloat16
    shapes = [tuple(g.shape) for g in grads]
    if not (len(grads) == len(moms) == len(outs)):
        raise MatoptError(-1, "grads, moms and outs must have the same length")
    if not shapes:
        return
    _validate(grads, shapes, "grads", (torch.float32, torch.bfloat16))
    _validate(moms, shapes, "moms", (torch.float32,))
    _validate(outs, shapes, "outs", (torch.float32, torch.bfloat16))
    gdt, odt = grads[0].dtype, outs[0].dtype
    if any(g.dtype != gdt for g in grads) or any(o.dtype != odt for o in outs):
        raise MatoptError(-2, "all grads (and all outs) must share one dtype")
    dev = _one_device(grads, moms, outs)
    mats = _mats(shapes, grads=grads, moms=moms, outs=outs)
    ns = _ns_params(a, b, c, iters, eps)
    with _on(dev):
        _check(lib.muon_step_batched_noalloc(mats, len(shapes), _dtype_code(gdt), _dtype_code(compute),
                                             _dtype_code(odt), float(beta), ctypes.byref(ns),
                                             _stream_ptr(grads[0])))


def muon_step_apply(grads, moms, weights, beta, a, b, c, iters, lr, eps=1e-7, compute=None,
                    workspace=None):
    """In place: moms[i] <- beta*moms[i] + grads[i]; weights[i] <- weights[i] - lr * U_i
    with U_i = NS_k(moms[i] / (||.||+eps)), never materialised.  weights: fp32 or
    bf16 (one dtype), shaped like the grads."""
    import torch
    lib = load_library()
    if compute is None:
        compute = torch.bfloat16
    shapes = [tuple(g.shape) for g in grads]
    if not (len(grads) == len(moms) == len(weights)):
        raise MatoptError(-1, "grads, moms and weights must have the same length")
    if not shapes:
        return
    _validate(grads, shapes, "grads", (torch.float32, torch.bfloat16))
    _validate(moms, shapes, "moms", (torch.float32,))
    _validate(weights, shapes, "weights", (torch.float32, torch.bfloat16))
    gdt, wdt = grads[0].dtype, weights[0].dtype
    if any(g.dtype != gdt for g in grads) or any(w.dtype != wdt for w in weights):
        raise MatoptError(-2, "all grads (and all weights) must share one dtype")
    dev = _one_device(grads, moms, weights)
    mats = _mats(shapes, grads=grads, moms=moms, outs=weights)
    nbytes = lib.muon_workspace_bytes(mats, len(shapes), _dtype_code(compute))
    ws = (workspace or Workspace(dev)).get(nbytes)
    _one_device(grads, ws)
    ns = _ns_params(a, b, c, iters, eps)
    with _on(dev):
        _check(lib.muon_step_apply(mats, len(shapes), _dtype_code(gdt), _dtype_code(compute), _dtype_code(wdt),
                                   float(beta), ctypes.byref(ns), float(lr), ws.data_ptr(), ws.numel(),
                                   _stream_ptr(grads[0])))


def ns_orthogonalize(xs, outs, a, b, c, iters, eps=1e-7, compute=None, workspace=None):
    """outs[i] <- NS_k(xs[i] / (||xs[i]||_F + eps)); xs[i] may be outs[i] when the
    dtypes match."""
    import torch
    lib = load_library()
    if compute is None:
        compute = torch.bfloat16
    shapes = [tuple(x.shape) for x in xs]
    if len(xs) != len(outs):
        raise MatoptError(-1, "xs and outs must have the same length")
    if not shapes:
        return
    _validate(xs, shapes, "xs", (torch.float32, torch.bfloat16))
    _validate(outs, shapes, "outs", (torch.float32, torch.bfloat16))
    idt, odt = xs[0].dtype, outs[0].dtype
    if any(x.dtype != idt for x in xs) or any(o.dtype != odt for o in outs):
        raise MatoptError(-2, "all xs (and all outs) must share one dtype")
    dev = _one_device(xs, outs)
    mats = _mats(shapes, xs=xs, outs=outs)
    nbytes = lib.muon_workspace_bytes(mats, len(shapes), _dtype_code(compute))
    ws = (workspace or Workspace(dev)).get(nbytes)
    _one_device(xs, ws)
    ns = _ns_params(a, b, c, iters, eps)
    with _on(dev):
        _check(lib.ns_orthogonalize(mats, len(shapes), _dtype_code(idt), _dtype_code(compute), _dtype_code(odt),
                                    ctypes.byref(ns), ws.data_ptr(), ws.numel(), _stream_ptr(xs[0])))


def sign_pack(u, packed=None):
    """1-bit signs of u (flat order) -> int32 tensor of ceil(numel/32) words (bit
    patterns of the uint32 words)."""
    import torch
    lib = load_library()
    if not u.is_cuda or not u.is_contiguous():
        raise MatoptError(-1, "u must be a contiguous CUDA tensor")
    numel = u.numel()
    nwords = (numel + 31) // 32
    if packed is None:
        packed = torch.empty(nwords, dtype=torch.int32, device=u.device)
    if packed.numel() < nwords or packed.dtype != torch.int32 or not packed.is_contiguous():
        raise MatoptError(-1, "packed must be a contiguous int32 tensor of ceil(numel/32) words")
    with _on(_one_device(u, packed)):
        _check(lib.sign_pack(u.data_ptr(), _dtype_code(u.dtype), numel, packed.data_ptr(), _stream_ptr(u)))
    return packed


def sign_pack_batched(u, packed=None):
    """1-bit signs of each row of u (M x numel, unit column stride; rows may be
    padded) -> int32 tensor [M][ceil(numel/32)], the stack sign_vote takes."""
    import torch
    lib = load_library()
    if not u.is_cuda or u.dim() != 2 or u.stride(1) != 1 or (u.shape[0] > 1 and u.stride(0) < u.shape[1]):
        raise MatoptError(-1, "u must be a CUDA tensor [M][numel] with contiguous rows")
    M, numel = u.shape
    nwords = (numel + 31) // 32
    if packed is None:
        packed = torch.empty((M, nwords), dtype=torch.int32, device=u.device)
    if packed.dtype != torch.int32 or not packed.is_contiguous() or tuple(packed.shape) != (M, nwords):
        raise MatoptError(-1, "packed must be a contiguous int32 tensor [M][ceil(numel/32)]")
    with _on(_one_device(u, packed)):
        _check(lib.sign_pack_batched(u.data_ptr(), _dtype_code(u.dtype), M, numel, u.stride(0), packed.data_ptr(),
                                     _stream_ptr(u)))
    return packed


def sign_vote(packed, numel, out_packed=None, with_sums=False):
    """Majority vote over packed[M][nwords] (int32 tensor).  Returns (out_packed,
    sums or None)."""
    import torch
    lib = load_library()
    if packed.dim() != 2 or packed.dtype != torch.int32 or not packed.is_contiguous() or not packed.is_cuda:
        raise MatoptError(-1, "packed must be a contiguous CUDA int32 tensor [M][nwords]")
    M, nwords = packed.shape
    if nwords != (numel + 31) // 32:
        raise MatoptError(-1, "packed width must be ceil(numel/32)")
    if out_packed is None:
        out_packed = torch.empty(nwords, dtype=torch.int32, device=packed.device)
    if out_packed.dtype != torch.int32 or not out_packed.is_contiguous() or out_packed.numel() < nwords:
        raise MatoptError(-1, "out_packed must be a contiguous int32 tensor of ceil(numel/32) words")
    sums = torch.empty(numel, dtype=torch.int8, device=packed.device) if with_sums else None
    with _on(_one_device(packed, out_packed)):
        _check(lib.sign_vote(packed.data_ptr(), M, numel, out_packed.data_ptr(),
                             sums.data_ptr() if sums is not None else None, _stream_ptr(packed)))
    return out_packed, sums


def _check_packed(packed, numel):
    import torch
    if packed.dtype != torch.int32 or not packed.is_contiguous() or not packed.is_cuda:
        raise MatoptError(-1, "packed must be a contiguous CUDA int32 tensor")
    if packed.numel() < (numel + 31) // 32:
        raise MatoptError(-1, "packed must hold ceil(numel/32) words")


def sign_unpack(packed, numel, out=None, dtype=None):
    """+1 / -1 per bit of packed (int32 words), as a flat tensor of numel values of
    dtype (torch.bfloat16 by default) or into out."""
    import torch
    lib = load_library()
    _check_packed(packed, numel)
    if out is None:
        out = torch.empty(numel, dtype=dtype or torch.bfloat16, device=packed.device)
    if not out.is_cuda or not out.is_contiguous() or out.numel() != numel:
        raise MatoptError(-1, "out must be a contiguous CUDA tensor of numel values")
    with _on(_one_device(packed, out)):
        _check(lib.sign_unpack(packed.data_ptr(), numel, _dtype_code(out.dtype), out.data_ptr(),
                               _stream_ptr(packed)))
    return out


def sign_apply(packed, weight, lr):
    """In place: weight <- weight - lr * S, S = +1 / -1 per bit of packed."""
    lib = load_library()
    numel = weight.numel()
    _check_packed(packed, numel)
    if not weight.is_cuda or not weight.is_contiguous():
        raise MatoptError(-1, "weight must be a contiguous CUDA tensor")
    with _on(_one_device(packed, weight)):
        _check(lib.sign_apply(packed.data_ptr(), numel, _dtype_code(weight.dtype), weight.data_ptr(), float(lr),
                              _stream_ptr(weight)))
    return weight


def plan_owners(shapes, ranks, iters, bytes_per_element=4.0):
    """Owner rank per matrix for a list of (rows, cols), plus per-rank work (NS flops)
    and bytes.  Host-only computation in the library; needs no GPU."""
    lib = load_library()
    n = len(shapes)
    I64s = ctypes.c_int64 * max(n, 1)
    rows = I64s(*[int(r) for r, _ in shapes])
    cols = I64s(*[int(c) for _, c in shapes])
    owner = (ctypes.c_int32 * max(n, 1))()
    work = (ctypes.c_double * max(int(ranks), 1))()
    nbytes = (ctypes.c_double * max(int(ranks), 1))()
    _check(lib.mo_plan_owners(rows, cols, n, int(ranks), int(iters), float(bytes_per_element), owner, work, nbytes))
    return [owner[i] for i in range(n)], [work[r] for r in range(ranks)], [nbytes[r] for r in range(ranks)]


def profile_begin():
    _check(load_library().mo_profile_begin())


def profile_end():
    """Per-kernel-kind {name: (launches, total_ms, busy_ms)} since profile_begin():
    busy_ms is the union of the launches' intervals (less than total_ms when launches
    of a kind overlap, as the two halves of a split product do)."""
    lib = load_library()
    buf = (MoKernelTime * 32)()
    n = lib.mo_profile_end(buf, 32)
    if n < 0:
        _check(n)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms, buf[i].busy_ms) for i in range(min(n, 32))}
