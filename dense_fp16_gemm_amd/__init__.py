"""MI355X (gfx950) dense fp16 NT GEMM: C = A @ B.T with fp32 accumulation.

Thin ctypes binding over the C ABI of ``libgemm_f16.so`` (declared in
``include/gemm_f16_nt.h``).  Every arithmetic step runs in the library's HIP
kernels; this module only marshals arguments.  PyTorch is used for device
memory and streams in :func:`gemm_nt`, nothing else.  There is no fallback:
if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

OK, INVALID_ARG, UNSUPPORTED, LAUNCH_FAILED, SCRATCH_LIMIT = 0, 1, 2, 3, 4

_lock = threading.Lock()
_lib = None


class GemmError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Plan(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("config_id", "block_m", "block_n", "block_k", "waves", "stages",
                 "swizzle", "tiles_m", "tiles_n", "grid")] + \
               [("tiles", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("xcds", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("b_layout", ctypes.c_int32), ("a_layout", ctypes.c_int32)]

    @property
    def layout(self) -> str:
        """'nt', 'nn', 'tn' or 'tt': how A and B are stored."""
        return ("t" if self.a_layout else "n") + ("n" if self.b_layout else "t")

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class TuneEntry(ctypes.Structure):
    """One autotuning candidate: a configuration and an effective split count."""
    _fields_ = [("config_id", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("status", ctypes.c_int32), ("ms", ctypes.c_float)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


# the library's layout codes: 2 * (A stored [K, M]) + (B stored [K, N])
LAYOUT_CODES = {"nt": 0, "nn": 1, "tt": 2, "tn": 3}


def library_path() -> str:
    return LIB_PATH


def load():
    """Load libgemm_f16.so (built in-tree); raise if it is not there."""
    global _lib
    lib = _lib
    if lib is not None:   # loaded: no lock on the per-call path
        return lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                "g.build()'` (hipcc, gfx950). There is no fallback path.")
        lib = ctypes.CDLL(LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        lib.gemm_f16_nt.argtypes = [i64, i64, i64, p, p, p, p]
        lib.gemm_f16_nt.restype = ctypes.c_int
        lib.gemm_f16_nt_with_config.argtypes = [i64, i64, i64, p, p, p, p, i32, i32, i32, i32]
        lib.gemm_f16_nt_with_config.restype = ctypes.c_int
        lib.gemm_f16_nt_status_string.argtypes = [ctypes.c_int]
        lib.gemm_f16_nt_status_string.restype = ctypes.c_char_p
        lib.gemm_f16_nt_validate.argtypes = [i64, i64, i64, p, p, p]
        lib.gemm_f16_nt_validate.restype = ctypes.c_int
        lib.gemm_f16_nt_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        lib.gemm_f16_nt_plan.restype = ctypes.c_int
        for lay in ("nt", "nn", "tn", "tt"):
            f = getattr(lib, f"gemm_f16_{lay}_splitk_plan")
            f.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(Plan), ctypes.POINTER(i32),
                          ctypes.POINTER(i64)]
            f.restype = ctypes.c_int
            f = getattr(lib, f"gemm_f16_{lay}_splitk")
            f.argtypes = [i64, i64, i64, p, p, p, i32, p, i64, p]
            f.restype = ctypes.c_int
            f = getattr(lib, f"gemm_f16_{lay}_splitk_with_config")
            f.argtypes = [i64, i64, i64, p, p, p, i32, p, i64, p, i32]
            f.restype = ctypes.c_int
        for lay in ("nn", "tn", "tt"):
            f = getattr(lib, f"gemm_f16_{lay}")
            f.argtypes = [i64, i64, i64, p, p, p, p]
            f.restype = ctypes.c_int
            f = getattr(lib, f"gemm_f16_{lay}_with_config")
            f.argtypes = [i64, i64, i64, p, p, p, p, i32, i32, i32, i32]
            f.restype = ctypes.c_int
            f = getattr(lib, f"gemm_f16_{lay}_plan")
            f.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
            f.restype = ctypes.c_int
        lib.gemm_f16_nt_num_configs.argtypes = []
        lib.gemm_f16_nt_num_configs.restype = ctypes.c_int
        lib.gemm_f16_nt_config_info.argtypes = [i32, ctypes.POINTER(Plan)]
        lib.gemm_f16_nt_config_info.restype = ctypes.c_int
        lib.gemm_f16_nt_tile_of_slot.argtypes = [ctypes.POINTER(Plan), i64,
                                                 ctypes.POINTER(i32), ctypes.POINTER(i32)]
        lib.gemm_f16_nt_tile_of_slot.restype = ctypes.c_int
        te = ctypes.POINTER(TuneEntry)
        lib.gemm_f16_autotune_candidates.argtypes = [i32, i64, i64, i64, i32, i32, i64, te, i32,
                                                     ctypes.POINTER(i32), ctypes.POINTER(i64)]
        lib.gemm_f16_autotune_candidates.restype = ctypes.c_int
        lib.gemm_f16_autotune.argtypes = [i32, i64, i64, i64, p, p, p, p, i64, i32, p, te, te,
                                          i32, ctypes.POINTER(i32)]
        lib.gemm_f16_autotune.restype = ctypes.c_int
        lib.gemm_f16_nt_splitk_noalloc.argtypes = [i64, i64, i64, p, p, p, i32, p]
        lib.gemm_f16_nt_splitk_noalloc.restype = ctypes.c_int
        lib.gemm_f16_splitk_workspace_bytes.argtypes = [i64, i64, i32, ctypes.POINTER(i64)]
        lib.gemm_f16_splitk_workspace_bytes.restype = ctypes.c_int
        lib.gemm_f16_device_cus.argtypes = [ctypes.POINTER(i32)]
        lib.gemm_f16_device_cus.restype = ctypes.c_int
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().gemm_f16_nt_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise GemmError(status, where)


# ---- C ABI, same names -----------------------------------------------------
def gemm_f16_nt(M: int, N: int, K: int, A: int, B: int, C: int, stream: int = 0) -> None:
    """C = A * B^T for device pointers A [M,K], B [N,K], C [M,N] (fp16)."""
    _check(load().gemm_f16_nt(M, N, K, A, B, C, stream), "gemm_f16_nt")


def gemm_f16_nt_with_config(M: int, N: int, K: int, A: int, B: int, C: int, stream: int,
                            config_id: int, swizzle: int = 0, grid: int = 0,
                            epilogue: int = -1) -> None:
    _check(load().gemm_f16_nt_with_config(M, N, K, A, B, C, stream, config_id, swizzle, grid,
                                          epilogue),
           "gemm_f16_nt_with_config")


def gemm_f16_nt_validate(M: int, N: int, K: int, A: int, B: int, C: int) -> int:
    return load().gemm_f16_nt_validate(M, N, K, A, B, C)


def gemm_f16_nt_plan(M: int, N: int, K: int, num_cus: int) -> Plan:
    plan = Plan()
    _check(load().gemm_f16_nt_plan(M, N, K, num_cus, ctypes.byref(plan)), "gemm_f16_nt_plan")
    return plan


def _layout_fns(lay: str):
    def call(M: int, N: int, K: int, A: int, B: int, C: int, stream: int = 0) -> None:
        _check(getattr(load(), f"gemm_f16_{lay}")(M, N, K, A, B, C, stream), f"gemm_f16_{lay}")

    def with_config(M: int, N: int, K: int, A: int, B: int, C: int, stream: int,
                    config_id: int, swizzle: int = 0, grid: int = 0, epilogue: int = -1) -> None:
        _check(getattr(load(), f"gemm_f16_{lay}_with_config")(M, N, K, A, B, C, stream, config_id,
                                                              swizzle, grid, epilogue),
               f"gemm_f16_{lay}_with_config")

    def plan(M: int, N: int, K: int, num_cus: int) -> Plan:
        out = Plan()
        _check(getattr(load(), f"gemm_f16_{lay}_plan")(M, N, K, num_cus, ctypes.byref(out)),
               f"gemm_f16_{lay}_plan")
        return out

    return call, with_config, plan


# C = op(A) op(B) for the other layouts: nn (A [M,K], B [K,N]), tn (A [K,M],
# B [K,N]), tt (A [K,M], B [N,K]); device pointers, fp16
gemm_f16_nn, gemm_f16_nn_with_config, gemm_f16_nn_plan = _layout_fns("nn")
gemm_f16_tn, gemm_f16_tn_with_config, gemm_f16_tn_plan = _layout_fns("tn")
gemm_f16_tt, gemm_f16_tt_with_config, gemm_f16_tt_plan = _layout_fns("tt")


def _splitk_fns(lay: str):
    def plan(M: int, N: int, K: int, num_cus: int, splits: int = 0) -> tuple[Plan, int, int]:
        """(plan, effective splits, workspace bytes) for the split-K entry point."""
        out, eff, wsb = Plan(), ctypes.c_int32(), ctypes.c_int64()
        _check(getattr(load(), f"gemm_f16_{lay}_splitk_plan")(M, N, K, num_cus, splits,
                                                              ctypes.byref(out), ctypes.byref(eff),
                                                              ctypes.byref(wsb)),
               f"gemm_f16_{lay}_splitk_plan")
        return out, eff.value, wsb.value

    def call(M: int, N: int, K: int, A: int, B: int, C: int, splits: int, workspace: int,
             workspace_bytes: int, stream: int = 0) -> None:
        _check(getattr(load(), f"gemm_f16_{lay}_splitk")(M, N, K, A, B, C, splits, workspace,
                                                         workspace_bytes, stream),
               f"gemm_f16_{lay}_splitk")

    def with_config(M: int, N: int, K: int, A: int, B: int, C: int, splits: int, workspace: int,
                    workspace_bytes: int, stream: int, config_id: int) -> None:
        _check(getattr(load(), f"gemm_f16_{lay}_splitk_with_config")(
            M, N, K, A, B, C, splits, workspace, workspace_bytes, stream, config_id),
            f"gemm_f16_{lay}_splitk_with_config")

    return plan, call, with_config


gemm_f16_nt_splitk_plan, gemm_f16_nt_splitk, gemm_f16_nt_splitk_with_config = _splitk_fns("nt")
gemm_f16_nn_splitk_plan, gemm_f16_nn_splitk, gemm_f16_nn_splitk_with_config = _splitk_fns("nn")
gemm_f16_tn_splitk_plan, gemm_f16_tn_splitk, gemm_f16_tn_splitk_with_config = _splitk_fns("tn")
gemm_f16_tt_splitk_plan, gemm_f16_tt_splitk, gemm_f16_tt_splitk_with_config = _splitk_fns("tt")


def gemm_f16_nt_splitk_noalloc(M: int, N: int, K: int, A: int, B: int, C: int, splits: int,
                               stream: int = 0) -> None:
    """gemm_f16_nt_splitk with the partials in the library's fixed scratch
    array: no workspace argument, no allocation (calls that overlap on one
    GPU race)."""
    _check(load().gemm_f16_nt_splitk_noalloc(M, N, K, A, B, C, splits, stream),
           "gemm_f16_nt_splitk_noalloc")


def gemm_f16_device_cus() -> int:
    """The current device's compute-unit count, from the library's cache."""
    out = ctypes.c_int32()
    _check(load().gemm_f16_device_cus(ctypes.byref(out)), "gemm_f16_device_cus")
    return out.value


def gemm_f16_splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    """Workspace bytes any configuration needs for at most `splits` ranges."""
    out = ctypes.c_int64()
    _check(load().gemm_f16_splitk_workspace_bytes(M, N, splits, ctypes.byref(out)),
           "gemm_f16_splitk_workspace_bytes")
    return out.value


def gemm_f16_nt_num_configs() -> int:
    return load().gemm_f16_nt_num_configs()


def gemm_f16_nt_config_info(config_id: int) -> Plan:
    info = Plan()
    _check(load().gemm_f16_nt_config_info(config_id, ctypes.byref(info)),
           "gemm_f16_nt_config_info")
    return info


def gemm_f16_nt_tile_of_slot(plan: Plan, slot: int) -> tuple[int, int]:
    tm, tn = ctypes.c_int32(), ctypes.c_int32()
    _check(load().gemm_f16_nt_tile_of_slot(ctypes.byref(plan), slot, ctypes.byref(tm),
                                           ctypes.byref(tn)), "gemm_f16_nt_tile_of_slot")
    return tm.value, tn.value


def gemm_f16_autotune_candidates(layout: int, M: int, N: int, K: int, num_cus: int,
                                 aligned: bool = True,
                                 workspace_bytes: int = 0) -> tuple[list[TuneEntry], int]:
    """(candidates gemm_f16_autotune would time, workspace bytes the largest split needs)."""
    lib, n, need = load(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib.gemm_f16_autotune_candidates(layout, M, N, K, num_cus, int(aligned),
                                            workspace_bytes, None, 0, ctypes.byref(n),
                                            ctypes.byref(need)), "gemm_f16_autotune_candidates")
    buf = (TuneEntry * max(n.value, 1))()
    _check(lib.gemm_f16_autotune_candidates(layout, M, N, K, num_cus, int(aligned),
                                            workspace_bytes, buf, n.value, ctypes.byref(n),
                                            ctypes.byref(need)), "gemm_f16_autotune_candidates")
    return list(buf[:n.value]), need.value


def gemm_f16_autotune(layout: int, M: int, N: int, K: int, A: int, B: int, C: int,
                      workspace: int, workspace_bytes: int, iters: int,
                      stream: int = 0, max_entries: int = 1024) -> tuple[TuneEntry, list[TuneEntry]]:
    """(fastest candidate, every timed candidate) from gemm_f16_autotune."""
    best, n = TuneEntry(), ctypes.c_int32()
    buf = (TuneEntry * max_entries)()
    _check(load().gemm_f16_autotune(layout, M, N, K, A, B, C, workspace, workspace_bytes, iters,
                                    stream, ctypes.byref(best), buf, max_entries,
                                    ctypes.byref(n)), "gemm_f16_autotune")
    return best, list(buf[:min(n.value, max_entries)])


# ---- torch convenience -------------------------------------------------------
class _NoDeviceSwitch:
    def __enter__(self):
        return None

    def __exit__(self, *exc):
        return False


_NO_SWITCH = _NoDeviceSwitch()


def _on_device(t):
    """Make t's device current for the call (the library launches on the
    current device); a no-op context when it already is, since switching
    costs more than a small GEMM's launch."""
    import torch

    idx = t.get_device()
    return _NO_SWITCH if idx == torch.cuda.current_device() else torch.cuda.device(idx)


def _stream_handle(t, stream) -> int:
    """The raw HIP stream of `stream`, or of t's device's current stream.
    torch's raw-stream query skips building a Stream object (the public
    torch.cuda.current_stream takes about 2 us); the public call is the
    fallback where the query is absent."""
    import torch

    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _operands(a, b, layout: str, out):
    """Check fp16 operands stored as `layout` says; return (M, N, K, out)."""
    import torch

    if layout not in LAYOUT_CODES:
        raise ValueError(f"unknown layout {layout!r}")
    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be torch.float16")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be matrices")
    m, k = (a.shape[1], a.shape[0]) if layout[0] == "t" else (a.shape[0], a.shape[1])
    kb, n = (b.shape[0], b.shape[1]) if layout[1] == "n" else (b.shape[1], b.shape[0])
    if k != kb:
        raise ValueError(f"shape mismatch for {layout}: a{tuple(a.shape)} b{tuple(b.shape)}")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (row-major)")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=a.device)
    elif (out.dtype != torch.float16 or tuple(out.shape) != (m, n) or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError("out must be a contiguous float16 [M, N] tensor on a's device")
    return m, n, k, out



def gemm_nt(a, b, out=None, config: int | None = None, swizzle: int = 0, grid: int = 0,
            stream=None, epilogue: int = -1):
    """C = a @ b.T for fp16 CUDA(HIP) tensors a [M,K] and b [N,K].

    Checks dtype, contiguity, device and shapes, then calls the C ABI on the
    current stream (or `stream`).  Returns the fp16 [M,N] output tensor.
    """
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be torch.float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"shape mismatch: a{tuple(a.shape)} b{tuple(b.shape)}")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (row-major)")
    m, k = a.shape
    n = b.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=a.device)
    elif (out.dtype != torch.float16 or tuple(out.shape) != (m, n) or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError("out must be a contiguous float16 [M, N] tensor on a's device")
    with _on_device(a):
        s = _stream_handle(a, stream)
        if config is None and swizzle <= 0 and grid <= 0 and epilogue < 0:
            gemm_f16_nt(m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(), s)
        else:
            gemm_f16_nt_with_config(m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(),
                                    s, -1 if config is None else config, swizzle,
                                    grid, epilogue)
    return out


def gemm_splitk(a, b, layout: str = "nt", splits: int = 0, out=None, workspace=None,
                config: int | None = None, stream=None):
    """C = op(a) @ op(b) with K split (gemm_f16_<layout>_splitk); operands as for
    gemm().  splits <= 0: the library's choice.  The fp32 workspace is
    allocated with torch unless `workspace` (a device tensor of at least the
    planned bytes) is given."""
    import torch

    m, n, k, out = _operands(a, b, layout, out)
    with _on_device(a):
        cus = gemm_f16_device_cus()
    _, _, need = globals()[f"gemm_f16_{layout}_splitk_plan"](m, n, k, cus, splits)
    if config is not None and splits > 1:
        # a forced configuration may split into more ranges than the planner's
        need = max(need, gemm_f16_splitk_workspace_bytes(m, n, splits))
    own = workspace is None
    if own:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    elif not workspace.is_cuda or workspace.device != a.device:
        raise ValueError("workspace must be a tensor on a's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(a):
        globals()[f"gemm_f16_{layout}_splitk_with_config"](
            m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(), splits, workspace.data_ptr(),
            ws_bytes, _stream_handle(a, stream), -1 if config is None else config)
    if own and stream is not None:
        # the allocator gave the workspace to the current stream; it is used
        # on `stream`, so it must not be reused before that work is done
        workspace.record_stream(stream)
    return out


def gemm_nt_splitk(a, b, splits: int = 0, out=None, workspace=None, config: int | None = None,
                   stream=None):
    """C = a @ b.T with K split (gemm_f16_nt_splitk) for fp16 tensors a [M,K], b [N,K]."""
    return gemm_splitk(a, b, "nt", splits=splits, out=out, workspace=workspace, config=config,
                       stream=stream)


def gemm(a, b, layout: str = "nt", out=None, config: int | None = None, swizzle: int = 0,
         grid: int = 0, stream=None, epilogue: int = -1):
    """C = op(a) @ op(b) for fp16 tensors, by operand layout:
    'nt': a [M,K], b [N,K] (C = a @ b.T);   'nn': a [M,K], b [K,N] (C = a @ b);
    'tn': a [K,M], b [K,N] (C = a.T @ b);   'tt': a [K,M], b [N,K] (C = a.T @ b.T).
    Same checks as gemm_nt."""
    if layout == "nt":
        return gemm_nt(a, b, out=out, config=config, swizzle=swizzle, grid=grid, stream=stream,
                       epilogue=epilogue)
    m, n, k, out = _operands(a, b, layout, out)
    fn = globals()[f"gemm_f16_{layout}_with_config"]
    with _on_device(a):
        fn(m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(), _stream_handle(a, stream),
           -1 if config is None else config, swizzle, grid, epilogue)
    return out


def gemm_nn(a, b, **kw):
    """C = a @ b for a [M,K], b [K,N] (gemm_f16_nn)."""
    return gemm(a, b, "nn", **kw)


class Tuned:
    """Result of autotune(): the fastest (config, splits), its time, every
    timed candidate, and the output tensor (which holds the fastest's C)."""

    def __init__(self, layout: str, best: TuneEntry, entries: list[TuneEntry], out):
        self.layout = layout
        self.config = best.config_id
        self.splits = best.splits
        self.ms = best.ms
        self.entries = [e.as_dict() for e in entries]
        self.out = out

    def __call__(self, a, b, out=None, workspace=None, stream=None):
        """Run the tuned choice (gemm_f16_<layout>_splitk_with_config)."""
        return gemm_splitk(a, b, self.layout, splits=self.splits, out=out, workspace=workspace,
                           config=None if self.config < 0 else self.config, stream=stream)

    def __repr__(self) -> str:
        return (f"Tuned(layout={self.layout!r}, config={self.config}, splits={self.splits}, "
                f"ms={self.ms:.4f}, candidates={len(self.entries)})")


def autotune(a, b, layout: str = "nt", iters: int = 10, out=None, workspace=None, stream=None):
    """Time every configuration of `layout` (and its split counts where the
    grid is under-filled) on these operands with gemm_f16_autotune; blocks
    until done.  The workspace the split candidates need (at most about 1 GiB)
    is allocated with torch unless `workspace` is given; candidates that do
    not fit it are not tried."""
    import torch

    m, n, k, out = _operands(a, b, layout, out)
    code = LAYOUT_CODES[layout]
    with _on_device(a):
        cus = gemm_f16_device_cus()
    aligned = a.data_ptr() % 16 == 0 and b.data_ptr() % 16 == 0
    _, need = gemm_f16_autotune_candidates(code, m, n, k, cus, aligned, 0)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    elif not workspace.is_cuda or workspace.device != a.device:
        raise ValueError("workspace must be a tensor on a's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with _on_device(a):
        best, entries = gemm_f16_autotune(code, m, n, k, a.data_ptr(), b.data_ptr(),
                                          out.data_ptr(), workspace.data_ptr(), ws_bytes, iters,
                                          _stream_handle(a, stream))
    return Tuned(layout, best, entries, out)


def matmul_layout(a, b):
    """How matmul() runs a @ b: (layout, A as stored, B as stored).

    Each operand must be row-major or the transposed view of a row-major
    matrix: a [M,K] row-major is A stored [M,K] ('n'); a.t() of a row-major
    [K,M] is A stored [K,M] ('t'); b [K,N] row-major is B stored [K,N] ('n');
    b.t() of a row-major [N,K] is B stored [N,K] ('t').  Pure function of the
    shapes and strides."""
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be matrices")

    def stored(x):
        if x.is_contiguous():
            return "n", x
        if x.t().is_contiguous():
            return "t", x.t()
        raise ValueError("each operand must be row-major or a transposed view of a "
                         f"row-major matrix (strides {tuple(x.stride())})")

    la, xa = stored(a)
    lb, xb = stored(b)
    return la + lb, xa, xb


# split counts the split planner chose, per (layout, M, N, K, device)
_split_choice: dict = {}


def matmul_splits(lay: str, m: int, n: int, k: int, a) -> int:
    """The split count matmul() runs (layout, M, N, K) with on a's device:
    the split planner's choice for 16-byte aligned operands (1: no split).
    Cached per shape, so a repeated call costs a dictionary lookup."""
    key = (lay, m, n, k, a.get_device())
    got = _split_choice.get(key)
    if got is None:
        with _on_device(a):
            cus = gemm_f16_device_cus()
        _, got, _ = globals()[f"gemm_f16_{lay}_splitk_plan"](m, n, k, cus, 0)
        if len(_split_choice) >= 1024:
            _split_choice.clear()
        _split_choice[key] = got
    return got


def matmul(a, b, out=None, stream=None):
    """C = a @ b for fp16 GPU matrices a [M,K] and b [K,N], each row-major or
    a transposed view of a row-major matrix (see matmul_layout): the storage
    picks gemm_f16_nn, gemm_f16_nt, gemm_f16_tn or gemm_f16_tt, with no copy.

    Where the split planner splits K (few output tiles, a long K), the call
    runs gemm_f16_<layout>_splitk with its fp32 workspace taken from torch's
    allocator: much faster there, and the result differs from the unsplit
    one only in the fp32 rounding of each sum (none for integer sums that
    fp32 holds exactly).  Use gemm() for the unsplit path."""
    lay, xa, xb = matmul_layout(a, b)
    if a.shape[1] != b.shape[0]:
        raise ValueError(f"shape mismatch: a{tuple(a.shape)} b{tuple(b.shape)}")
    m, k, n = a.shape[0], a.shape[1], b.shape[1]
    if m > 0 and n > 0 and k > 0 and a.is_cuda and matmul_splits(lay, m, n, k, a) > 1:
        return gemm_splitk(xa, xb, lay, out=out, stream=stream)
    return gemm(xa, xb, lay, out=out, stream=stream)
