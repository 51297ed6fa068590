"""ctypes binding of libragged_attn (include/ragged_attn.h).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and the call goes to the C ABI.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  If the built library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libragged_attn.so"

STATUS = {0: "RA_OK", 1: "RA_E_NULL", 2: "RA_E_SHAPE", 3: "RA_E_UNSUPPORTED",
          4: "RA_E_METADATA", 5: "RA_E_WORKSPACE", 6: "RA_E_HIP"}
VARIANTS = {"auto": 0, "generic": 1, "specialised": 2, "unfused": 3}


class RaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.name = STATUS.get(status, str(status))


class RaShape(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("causal", ctypes.c_int32)]


def lib_path() -> str:
    return os.environ.get("RA_LIB", os.path.join(_HERE, _LIB_NAME))


_lib = None


def load_library():
    """Load libragged_attn.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"libragged_attn is not built ({path} missing); run "
                           "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    shp = ctypes.POINTER(RaShape)
    lib.ra_workspace_bytes.restype = sz
    lib.ra_workspace_bytes.argtypes = [shp, P, P]
    fwd_args = [shp, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.ra_forward.restype = i32
    lib.ra_forward.argtypes = fwd_args
    lib.ra_forward_variant.restype = i32
    lib.ra_forward_variant.argtypes = fwd_args + [i32]
    lib.ra_forward_profiled.restype = i32
    lib.ra_forward_profiled.argtypes = fwd_args + [i32, P, i32]
    lib.ra_forward_noalloc.restype = i32
    lib.ra_forward_noalloc.argtypes = [shp, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.ra_validate_metadata.restype = i32
    lib.ra_validate_metadata.argtypes = [shp, P, P, P, P]
    lib.ra_status_str.restype = ctypes.c_char_p
    lib.ra_status_str.argtypes = [i32]
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_last_error.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().ra_last_error().decode()


def _check(status: int):
    if status != 0:
        raise RaError(status, last_error())


def make_shape(*, num_reqs, total_tokens, num_q_heads, num_kv_heads, head_dim, page_size,
               num_pages, max_pages_per_req, scale=0.0, causal=True) -> RaShape:
    return RaShape(int(num_reqs), int(total_tokens), int(num_q_heads), int(num_kv_heads),
                   int(head_dim), int(page_size), int(num_pages), int(max_pages_per_req),
                   float(scale or 0.0), int(bool(causal)))


def _host_i32(t: torch.Tensor) -> torch.Tensor:
    return t.detach().to("cpu", torch.int32).contiguous()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def shape_of(q, k_cache, page_table, context_lens, *, scale=None, causal=True) -> RaShape:
    T, Hq, D = q.shape
    P, S, Hkv, _ = k_cache.shape
    R = int(context_lens.shape[0])
    maxp = int(page_table.shape[1]) if page_table.dim() == 2 else 0
    return make_shape(num_reqs=R, total_tokens=T, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                      page_size=S, num_pages=P, max_pages_per_req=maxp, scale=scale or 0.0,
                      causal=causal)


def workspace_bytes(shape: RaShape, cu_q_lens_host: torch.Tensor | None,
                    context_lens_host: torch.Tensor | None) -> int:
    """Workspace for a batch; with both host copies None, the bound for any
    batch of the shape's R requests and T tokens (planning on the device)."""
    lib = load_library()
    if cu_q_lens_host is None and context_lens_host is None:
        return int(lib.ra_workspace_bytes(ctypes.byref(shape), None, None))
    cu, ctx = _host_i32(cu_q_lens_host), _host_i32(context_lens_host)
    return int(lib.ra_workspace_bytes(ctypes.byref(shape), _ptr(cu), _ptr(ctx)))


def validate_metadata(shape: RaShape, page_table, cu_q_lens, context_lens, slot_mapping):
    """Full CPU-side metadata check; raises RaError on the first violation."""
    lib = load_library()
    pt, cu, ctx, sm = (_host_i32(x) for x in (page_table, cu_q_lens, context_lens, slot_mapping))
    _check(lib.ra_validate_metadata(ctypes.byref(shape), _ptr(pt), _ptr(cu), _ptr(ctx), _ptr(sm)))


def forward(q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
            slot_mapping, *, causal=True, scale=None, out=None, cu_q_lens_host=None,
            context_lens_host=None, workspace=None, variant="auto", stream=None,
            plan_on_device=False):
    """Fused KV-cache update + ragged paged attention on the current stream.

    All tensors live on the GPU except the optional host copies of cu_q_lens
    and context_lens (taken from the device tensors when not given, which
    synchronises).  plan_on_device=True passes no host copies: the library
    plans from the bounds R = len(context_lens) and T = len(q) on the device,
    so nothing is synchronised and a captured graph stays valid when the
    lengths change.  k_cache / v_cache are updated in place; returns `out`.
    """
    lib = load_library()
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    for name, t in (("page_table", page_table), ("cu_q_lens", cu_q_lens),
                    ("context_lens", context_lens), ("slot_mapping", slot_mapping)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    shape = shape_of(q, k_cache, page_table, context_lens, scale=scale, causal=causal)
    if plan_on_device:
        cu_h = ctx_h = None
    else:
        cu_h = _host_i32(cu_q_lens if cu_q_lens_host is None else cu_q_lens_host)
        ctx_h = _host_i32(context_lens if context_lens_host is None else context_lens_host)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = lib.ra_workspace_bytes(ctypes.byref(shape), _ptr(cu_h), _ptr(ctx_h))
        workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = lib.ra_forward_variant(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), _ptr(cu_q_lens), _ptr(context_lens), _ptr(slot_mapping), _ptr(cu_h),
        _ptr(ctx_h), _ptr(out), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
        ctypes.c_void_p(stream), VARIANTS[variant])
    _check(status)
    return out


def forward_noalloc(q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
                    slot_mapping, *, causal=True, scale=None, out=None, cu_q_lens_host=None,
                    context_lens_host=None, stream=None, plan_on_device=False):
    """forward() through ra_forward_noalloc: no workspace (the library's static
    scratch array serves), no allocation inside the call.  `out` is allocated
    here when not given (that is the caller's memory, not the call's)."""
    lib = load_library()
    shape = shape_of(q, k_cache, page_table, context_lens, scale=scale, causal=causal)
    if plan_on_device:
        cu_h = ctx_h = None
    else:
        cu_h = _host_i32(cu_q_lens if cu_q_lens_host is None else cu_q_lens_host)
        ctx_h = _host_i32(context_lens if context_lens_host is None else context_lens_host)
    if out is None:
        out = torch.empty_like(q)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    status = lib.ra_forward_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), _ptr(cu_q_lens), _ptr(context_lens), _ptr(slot_mapping), _ptr(cu_h),
        _ptr(ctx_h), _ptr(out), ctypes.c_void_p(stream))
    _check(status)
    return out


# --------------------------------------------------------------------------
# Per-stage timing (plumbing for the bench: hipEvents through libamdhip64).
# --------------------------------------------------------------------------
STAGES = ("plan", "prefill", "decode", "merge")


class StageTimer:
    """Eight hipEvents for ra_forward_profiled: a start and a stop event per
    stage, given to the stage's kernel launch, so that each pair brackets
    that kernel's execution alone (a stage that launches nothing reads ~0)."""

    N_EVENTS = 2 * len(STAGES)

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = (ctypes.c_void_p * self.N_EVENTS)()
        for k in range(self.N_EVENTS):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[k] = ev

    def stage_ms(self) -> dict:
        """Milliseconds of each stage's kernel in the last profiled call (waits for it)."""
        for k in range(self.N_EVENTS):
            if self.hip.hipEventSynchronize(self.events[k]) != 0:
                raise RuntimeError("hipEventSynchronize failed")
        out = {}
        for k, name in enumerate(STAGES):
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * k], self.events[2 * k + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out[name] = float(ms.value)
        return out

    def close(self):
        for k in range(self.N_EVENTS):
            if self.events[k]:
                self.hip.hipEventDestroy(self.events[k])
                self.events[k] = None


class Prepared:
    """A call with every argument marshalled once, for repeated launches.

    Holds the shape, host copies, workspace and raw pointers, so that each
    launch is one C call on the given stream.
    """

    def __init__(self, q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
                 slot_mapping, *, causal=True, scale=None, out=None, variant="auto",
                 cu_q_lens_host=None, context_lens_host=None):
        self.lib = load_library()
        self.shape = shape_of(q, k_cache, page_table, context_lens, scale=scale, causal=causal)
        self.cu_h = _host_i32(cu_q_lens if cu_q_lens_host is None else cu_q_lens_host)
        self.ctx_h = _host_i32(context_lens if context_lens_host is None else context_lens_host)
        self.out = torch.empty_like(q) if out is None else out
        nbytes = self.lib.ra_workspace_bytes(ctypes.byref(self.shape), _ptr(self.cu_h), _ptr(self.ctx_h))
        self.workspace = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=q.device)
        self.variant = VARIANTS[variant]
        self.keep = (q, k_new, v_new, k_cache, v_cache, page_table, cu_q_lens, context_lens,
                     slot_mapping)
        self.args = [ctypes.byref(self.shape), *[_ptr(t) for t in self.keep], _ptr(self.cu_h),
                     _ptr(self.ctx_h), _ptr(self.out), _ptr(self.workspace),
                     ctypes.c_size_t(self.workspace.numel())]

    def __call__(self, stream, timer: StageTimer | None = None):
        if timer is None:
            st = self.lib.ra_forward_variant(*self.args, ctypes.c_void_p(stream), self.variant)
        else:
            st = self.lib.ra_forward_profiled(*self.args, ctypes.c_void_p(stream), self.variant,
                                              timer.events, StageTimer.N_EVENTS)
        _check(st)
        return self.out
