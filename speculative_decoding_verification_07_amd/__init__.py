"""MI355X (gfx950) batched verify step of speculative decoding.

Thin ctypes binding over the C ABI declared in include/spec_verify.h,
include/spec_ngram.h (prompt-lookup drafting) and include/spec_adapt.h
(adaptive draft length).  Every
step of the verify runs in the HIP kernels of libspecverify.so; this module
only checks tensor shapes, allocates outputs with torch, and passes raw device
pointers and the current HIP stream.  There is no CPU fallback: importing the
binding when the library has not been built raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SAMPLE, GREEDY, POINT = 0, 1, 2
F32, BF16 = 0, 1
OK, ERR_NULL, ERR_SHAPE, ERR_ARG, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP = 0, -1, -2, -3, -4, -5, -100
GAMMA_MAX_LIMIT = 63

EXPORTS = (
    "spec_verify", "spec_verify_noalloc", "spec_verify_probe", "spec_verify_filtered", "spec_verify_filtered_probe",
    "spec_filter_thresholds", "spec_verify_workspace_bytes",
    "spec_verify_workspace_reset", "spec_verify_plan", "spec_verify_tune",
    "spec_verify_diagnostics", "spec_verify_strerror", "spec_verify_version",
    "spec_probe_read", "spec_probe_read_blocks", "spec_probe_copy",
    "spec_ngram_draft", "spec_ngram_workspace_bytes", "spec_gamma_control",
    "spec_ngram_draft_adaptive",
)
NGRAM_MAX_N, NGRAM_MAX_GAMMA, NGRAM_MAX_STRIDE = 64, 256, 1 << 25

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


def load():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    # SPEC_VERIFY_LIB: another build of this library's sources to load
    # instead (the host-sanitizer build of tests/run_sanitized.py)
    path = os.environ.get("SPEC_VERIFY_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (__graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    verify_args = [P, P, P, P, P, P, i32, i32, i32, i32, f32, i32, P, P, P, P, sz, P]
    lib.spec_verify.argtypes = verify_args
    lib.spec_verify.restype = i32
    lib.spec_verify_noalloc.argtypes = verify_args[:15] + [P]
    lib.spec_verify_noalloc.restype = i32
    lib.spec_verify_probe.argtypes = verify_args + [P, P, P, P, P, P, P]
    lib.spec_verify_probe.restype = i32
    filtered_args = verify_args[:12] + [i32, f32] + verify_args[12:]
    lib.spec_verify_filtered.argtypes = filtered_args
    lib.spec_verify_filtered.restype = i32
    lib.spec_verify_filtered_probe.argtypes = filtered_args + [P, P, P, P, P, P, P]
    lib.spec_verify_filtered_probe.restype = i32
    lib.spec_filter_thresholds.argtypes = [P, P, P, i32, i32, i32, i32, f32, i32, i32, f32, P, P]
    lib.spec_filter_thresholds.restype = i32
    lib.spec_verify_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.spec_verify_workspace_bytes.restype = sz
    lib.spec_verify_workspace_reset.argtypes = [P, sz, P]
    lib.spec_verify_workspace_reset.restype = i32
    lib.spec_verify_plan.argtypes = [i32, i32, i32, i32, i32, P]
    lib.spec_verify_plan.restype = i32
    lib.spec_verify_tune.argtypes = [i32, i32, i32]
    lib.spec_verify_tune.restype = i32
    lib.spec_verify_diagnostics.argtypes = [P, P, P]
    lib.spec_verify_diagnostics.restype = i32
    lib.spec_verify_strerror.argtypes = [i32]
    lib.spec_verify_strerror.restype = ctypes.c_char_p
    lib.spec_verify_version.argtypes = []
    lib.spec_verify_version.restype = i32
    lib.spec_probe_read.argtypes = [P, sz, P, P]
    lib.spec_probe_read.restype = i32
    lib.spec_probe_read_blocks.argtypes = [sz]
    lib.spec_probe_read_blocks.restype = i32
    lib.spec_probe_copy.argtypes = [P, P, sz, P]
    lib.spec_probe_copy.restype = i32
    lib.spec_ngram_workspace_bytes.argtypes = [i32]
    lib.spec_ngram_workspace_bytes.restype = sz
    lib.spec_ngram_draft.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.spec_ngram_draft.restype = i32
    d = ctypes.c_double
    lib.spec_gamma_control.argtypes = [P, P, P, P, P, i32, i32, d, d, d, d, i32, P, P, P]
    lib.spec_gamma_control.restype = i32
    lib.spec_ngram_draft_adaptive.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, d, d, d, d,
                                              i32, P, P, P, P, P, P, P, sz, P]
    lib.spec_ngram_draft_adaptive.restype = i32
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().spec_verify_strerror(int(status)).decode()


def _check(status: int, what: str):
    if status != OK:
        raise SpecVerifyError(status, what)


def workspace_bytes(B: int, gamma_max: int, V: int, dtype: int, mode: int) -> int:
    return int(load().spec_verify_workspace_bytes(B, gamma_max, V, dtype, mode))


def plan(B: int, gamma_max: int, V: int, dtype: int, mode: int) -> dict:
    out = (ctypes.c_int64 * 8)()
    _check(load().spec_verify_plan(B, gamma_max, V, dtype, mode, out), "spec_verify_plan")
    keys = ("workgroups", "slices", "slice_len", "vectors", "vocab_rows", "threads",
            "workspace_bytes", "target_workgroups")
    return dict(zip(keys, (int(v) for v in out)))


TUNE_ONE_PASS = 1  # SPEC_TUNE_ONE_PASS


def tune(vectors: int = 0, target_workgroups: int = 0, one_pass: bool = False):
    """Process-wide launch tuning (see spec_verify_tune); no arguments
    restores the defaults.  one_pass: stream every row in one pass instead
    of reading the rows position by position (every mode)."""
    _check(load().spec_verify_tune(vectors, target_workgroups, TUNE_ONE_PASS if one_pass else 0),
           "spec_verify_tune")


# ---------------------------------------------------------------- torch helpers
def _torch():
    import torch
    return torch


def _stream_handle(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on(stream):
    """Allocation context of the stream a call runs on.  Temporaries (a
    workspace, outputs, probes) are allocated on that stream, so torch's
    caching allocator hands their blocks to nothing else until the work
    queued there with them has run."""
    import contextlib
    return contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("logits must be torch.float32 or torch.bfloat16")


class Workspace:
    """Device workspace: a torch byte tensor zero-filled once by the
    library's fill kernel; every completed call leaves it zero again."""

    def __init__(self, nbytes: int, device="cuda", stream=None):
        torch = _torch()
        self.nbytes = int(nbytes)
        self.tensor = torch.empty(max(self.nbytes, 256) + 256, dtype=torch.uint8, device=device)
        base = self.tensor.data_ptr()
        self.offset = (-base) % 256
        self.ptr = base + self.offset
        _check(load().spec_verify_workspace_reset(ctypes.c_void_p(self.ptr), self.nbytes,
                                                  _stream_handle(stream)), "workspace reset")

    def diagnostics(self, stream=None) -> int:
        flags = ctypes.c_uint32(0)
        _check(load().spec_verify_diagnostics(ctypes.c_void_p(self.ptr), ctypes.byref(flags),
                                              _stream_handle(stream)), "diagnostics")
        return int(flags.value)


def _shape_check(target, draft, tokens, uniforms, gamma, kv_len, mode):
    if target.dim() != 3:
        raise ValueError("target_logits must be [B, gamma_max+1, V]")
    B, G1, V = target.shape
    G = G1 - 1
    for name, t in (("target_logits", target), ("draft_logits", draft), ("draft_tokens", tokens),
                    ("uniforms", uniforms), ("gamma_per_row", gamma), ("kv_len_in", kv_len)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    torch = _torch()
    for name, t, want in (("draft_tokens", tokens, torch.int32), ("uniforms", uniforms, torch.float32),
                          ("gamma_per_row", gamma, torch.int32), ("kv_len_in", kv_len, torch.int32)):
        if t is not None and t.dtype != want:
            raise TypeError(f"{name} must be {want}")
    if draft is not None and (tuple(draft.shape) != (B, G, V) or draft.dtype != target.dtype):
        raise ValueError("draft_logits must be [B, gamma_max, V] with the target's dtype")
    if tokens is not None and tuple(tokens.shape) != (B, G):
        raise ValueError("draft_tokens must be int32 [B, gamma_max]")
    if uniforms is not None and tuple(uniforms.shape) != (B, G + 1):
        raise ValueError("uniforms must be float32 [B, gamma_max+1]")
    if tuple(gamma.shape) != (B,):
        raise ValueError("gamma_per_row must be int32 [B]")
    if kv_len is not None and tuple(kv_len.shape) != (B,):
        raise ValueError("kv_len_in must be int32 [B]")
    return B, G, V


def _filtering(top_k, top_p) -> bool:
    return top_k != 0 or top_p != 1.0


def verify(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row, kv_len_in=None,
           *, temperature: float = 1.0, mode: int = SAMPLE, workspace: Workspace | None = None,
           out=None, stream=None, probe: bool = False, top_k: int = 0, top_p: float = 1.0,
           check: bool = False):
    """Run spec_verify (spec_verify_filtered when top_k or top_p filter) on
    torch device tensors.

    Returns (tokens [B, G+1] int32, n_accepted [B] int32, new_len [B] int32),
    plus a dict of probe tensors (px, qx, z, m, s, flo, fhi) when probe=True.  `out`
    may pass preallocated (tokens, n_accepted, new_len).  The call is
    asynchronous on `stream` (default: torch's current stream).  Temporaries
    are allocated on that stream.  check=True waits for the call and reads
    the workspace's diagnostic word, raising WaitGaveUp if a workgroup gave
    up waiting (which a correct launch never does)."""
    torch = _torch()
    lib = load()
    B, G, V = _shape_check(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row,
                           kv_len_in, mode)
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    need = workspace_bytes(B, G, V, dt, mode)
    with _on(stream):
        if workspace is None:
            workspace = Workspace(need, device=dev, stream=stream)
        if out is None:
            out = (torch.empty((B, G + 1), dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev),
                   torch.empty(B, dtype=torch.int32, device=dev))
    tok, nacc, nlen = out
    filt = _filtering(top_k, top_p)
    head = [_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms),
            _ptr(gamma_per_row), _ptr(kv_len_in), B, G, V, dt, float(temperature), int(mode)]
    tail = [_ptr(tok), _ptr(nacc), _ptr(nlen), ctypes.c_void_p(workspace.ptr),
            workspace.nbytes, _stream_handle(stream)]
    args = head + ([int(top_k), float(top_p)] if filt else []) + tail
    if not probe:
        if filt:
            _check(lib.spec_verify_filtered(*args), "spec_verify_filtered")
        else:
            _check(lib.spec_verify(*args), "spec_verify")
        if check:
            _check_diagnostics(workspace, stream)
        return tok, nacc, nlen
    nan = float("nan")
    with _on(stream):
        pr = {
            "px": torch.full((B, G), nan, dtype=torch.float32, device=dev),
            "qx": torch.full((B, G), nan, dtype=torch.float32, device=dev),
            "z": torch.full((B,), nan, dtype=torch.float32, device=dev),
            "m": torch.full((B, 2 * G + 1), nan, dtype=torch.float32, device=dev),
            "s": torch.full((B, 2 * G + 1), nan, dtype=torch.float32, device=dev),
            "flo": torch.full((B,), nan, dtype=torch.float32, device=dev),
            "fhi": torch.full((B,), nan, dtype=torch.float32, device=dev),
        }
    fn = lib.spec_verify_filtered_probe if filt else lib.spec_verify_probe
    _check(fn(*args, _ptr(pr["px"]), _ptr(pr["qx"]), _ptr(pr["z"]), _ptr(pr["m"]),
              _ptr(pr["s"]), _ptr(pr["flo"]), _ptr(pr["fhi"])), "spec_verify_probe")
    if check:
        _check_diagnostics(workspace, stream)
    return tok, nacc, nlen, pr


NOALLOC_WORKSPACE_BYTES = 8 << 20


def verify_noalloc(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row,
                   kv_len_in=None, *, temperature: float = 1.0, mode: int = SAMPLE, out,
                   stream=None):
    """spec_verify_noalloc: the verify step with the library's own static
    workspace (no allocation in the call; `out` = preallocated (tokens,
    n_accepted, new_len) is required).  Calls that may overlap on one device
    race for that workspace."""
    B, G, V = _shape_check(target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row,
                           kv_len_in, mode)
    tok, nacc, nlen = out
    _check(load().spec_verify_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms),
        _ptr(gamma_per_row), _ptr(kv_len_in), B, G, V, _dtype_code(target_logits),
        float(temperature), int(mode), _ptr(tok), _ptr(nacc), _ptr(nlen),
        _stream_handle(stream)), "spec_verify_noalloc")
    return tok, nacc, nlen


class WaitGaveUp(RuntimeError):
    """A workgroup of the call gave up waiting for the rest of its batch row
    (diagnostic bit 0): the rows it served hold the sentinel, and the
    workspace must be zero-filled again before its next use."""


def _check_diagnostics(workspace, stream):
    flags = workspace.diagnostics(stream)
    if flags & 1:
        raise WaitGaveUp(f"a verify workgroup gave up waiting (diagnostics 0x{flags:x})")


def filter_thresholds(target_logits, draft_logits, gamma_per_row, *, temperature: float = 1.0,
                      mode: int = SAMPLE, top_k: int = 0, top_p: float = 1.0, out=None,
                      stream=None):
    """spec_filter_thresholds: fp32 [B, 2G+1] device tensor of per-row
    thresholds (-inf where nothing is cut)."""
    torch = _torch()
    B, G, V = _shape_check(target_logits, draft_logits, None, None, gamma_per_row, None, mode)
    if out is None:
        with _on(stream):
            out = torch.empty((B, 2 * G + 1), dtype=torch.float32, device=target_logits.device)
    _check(load().spec_filter_thresholds(_ptr(target_logits), _ptr(draft_logits),
                                         _ptr(gamma_per_row), B, G, V,
                                         _dtype_code(target_logits), float(temperature),
                                         int(mode), int(top_k), float(top_p), _ptr(out),
                                         _stream_handle(stream)), "spec_filter_thresholds")
    return out


class Prepared:
    """One spec_verify call with its arguments checked and marshalled once.

    Calling the object re-issues the same call (same tensors, workspace,
    outputs and stream); for tight loops where per-call Python work would
    otherwise delay the launches."""

    def __init__(self, target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row,
                 kv_len_in=None, *, temperature: float = 1.0, mode: int = SAMPLE,
                 workspace: Workspace, out, stream=None, top_k: int = 0, top_p: float = 1.0):
        B, G, V = _shape_check(target_logits, draft_logits, draft_tokens, uniforms,
                               gamma_per_row, kv_len_in, mode)
        dt = _dtype_code(target_logits)
        if workspace.nbytes < workspace_bytes(B, G, V, dt, mode):
            raise ValueError("workspace too small")
        self._keep = (target_logits, draft_logits, draft_tokens, uniforms, gamma_per_row,
                      kv_len_in, workspace, out)
        tok, nacc, nlen = out
        filt = _filtering(top_k, top_p)
        self._fn = load().spec_verify_filtered if filt else load().spec_verify
        self._args = ((_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens),
                       _ptr(uniforms), _ptr(gamma_per_row), _ptr(kv_len_in), B, G, V, dt,
                       ctypes.c_float(temperature), int(mode))
                      + ((int(top_k), ctypes.c_float(top_p)) if filt else ())
                      + (_ptr(tok), _ptr(nacc), _ptr(nlen), ctypes.c_void_p(workspace.ptr),
                         workspace.nbytes, _stream_handle(stream)))

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != OK:
            raise SpecVerifyError(rc, "spec_verify")


def ngram_workspace_bytes(B: int) -> int:
    return int(load().spec_ngram_workspace_bytes(B))


def ngram_draft(context, ctx_len, *, n_min: int = 1, n_max: int = 4, gamma: int = 4,
                workspace: Workspace | None = None, out=None, stream=None):
    """spec_ngram_draft (prompt-lookup drafting) on torch device tensors:
    context int32 [B, stride], ctx_len int32 [B].

    Returns (draft [B, gamma], length [B], n [B], pos [B]), all int32; draft
    and length are ready to pass to verify(mode=POINT) as draft_tokens and
    gamma_per_row.  `out` may pass preallocated tensors in that order.  The
    call is asynchronous on `stream` (default: torch's current stream)."""
    torch = _torch()
    if context.dim() != 2 or tuple(ctx_len.shape) != (context.shape[0],):
        raise ValueError("context must be int32 [B, stride] and ctx_len int32 [B]")
    for name, t in (("context", context), ("ctx_len", ctx_len)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be torch.int32")
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, stride = context.shape
    dev = context.device
    with _on(stream):
        if workspace is None:
            workspace = Workspace(ngram_workspace_bytes(B), device=dev, stream=stream)
        if out is None:
            out = (torch.empty((B, gamma), dtype=torch.int32, device=dev),
                   *(torch.empty(B, dtype=torch.int32, device=dev) for _ in range(3)))
    draft, length, n, pos = out
    _check(load().spec_ngram_draft(_ptr(context), _ptr(ctx_len), B, stride, int(n_min),
                                   int(n_max), int(gamma), _ptr(draft), _ptr(length), _ptr(n),
                                   _ptr(pos), ctypes.c_void_p(workspace.ptr), workspace.nbytes,
                                   _stream_handle(stream)), "spec_ngram_draft")
    return draft, length, n, pos


class GammaControl:
    """spec_gamma_control with its parameters fixed: the running-acceptance
    state of B request slots (float64 [B, 2] on the device, zero-filled) and
    one call per round.  Zero a slot's row of `state` when it takes a new
    request."""

    def __init__(self, B: int, *, gamma_max: int = 4, decay: float = 0.9,
                 prior_alpha: float = 0.6, prior_weight: float = 2.0, draft_cost: float = 0.05,
                 batch_off: int = 0, device="cuda"):
        torch = _torch()
        self.B = int(B)
        self.params = (int(gamma_max), float(decay), float(prior_alpha), float(prior_weight),
                       float(draft_cost), int(batch_off))
        self.state = torch.zeros((self.B, 2), dtype=torch.float64, device=device)

    def __call__(self, n_accepted=None, gamma_used=None, *, active=None, gamma_limit=None,
                 out=None, alpha=None, stream=None):
        """Returns out_gamma (int32 [B]); `alpha`, if given, receives the
        running acceptance (float64 [B])."""
        torch = _torch()
        for name, t in (("n_accepted", n_accepted), ("gamma_used", gamma_used),
                        ("active", active), ("gamma_limit", gamma_limit)):
            if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (self.B,)
                                  or not t.is_contiguous() or not t.is_cuda):
                raise ValueError(f"{name} must be a contiguous int32 [B] device tensor")
        if alpha is not None and (alpha.dtype != torch.float64 or tuple(alpha.shape) != (self.B,)):
            raise ValueError("alpha must be float64 [B]")
        if out is None:
            with _on(stream):
                out = torch.empty(self.B, dtype=torch.int32, device=self.state.device)
        g, decay, pa, pw, c, off = self.params
        _check(load().spec_gamma_control(_ptr(n_accepted), _ptr(gamma_used), _ptr(active),
                                         _ptr(gamma_limit), _ptr(self.state), self.B, g, decay,
                                         pa, pw, c, off, _ptr(out), _ptr(alpha),
                                         _stream_handle(stream)), "spec_gamma_control")
        return out


def ngram_draft_adaptive(context, ctx_len, control: GammaControl, n_accepted=None,
                         gamma_used=None, *, active=None, n_min: int = 1, n_max: int = 4,
                         workspace: Workspace | None = None, out=None, alpha=None, stream=None):
    """spec_ngram_draft_adaptive: prompt-lookup drafting with the draft-length
    rule in the same launch.  The draft length cap is the controller's
    gamma_max; `control` holds the rule's parameters and state.

    Returns (draft [B, gamma], length [B], n [B], pos [B], gamma [B]), all
    int32: `gamma` is this round's gamma_per_row for verify(mode=POINT), and
    the next round passes that verify's n_accepted with this `gamma` back."""
    torch = _torch()
    B, stride = context.shape
    if control.B != B:
        raise ValueError("the controller's batch differs from the context's")
    for name, t in (("context", context), ("ctx_len", ctx_len), ("n_accepted", n_accepted),
                    ("gamma_used", gamma_used), ("active", active)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    G, decay, pa, pw, c, off = control.params
    dev = context.device
    with _on(stream):
        if workspace is None:
            workspace = Workspace(ngram_workspace_bytes(B), device=dev, stream=stream)
        if out is None:
            out = (torch.empty((B, G), dtype=torch.int32, device=dev),
                   *(torch.empty(B, dtype=torch.int32, device=dev) for _ in range(4)))
    draft, length, n, pos, gam = out
    _check(load().spec_ngram_draft_adaptive(
        _ptr(context), _ptr(ctx_len), B, stride, int(n_min), int(n_max), G, _ptr(n_accepted),
        _ptr(gamma_used), _ptr(active), _ptr(control.state), decay, pa, pw, c, off, _ptr(draft),
        _ptr(length), _ptr(n), _ptr(pos), _ptr(gam), _ptr(alpha), ctypes.c_void_p(workspace.ptr),
        workspace.nbytes, _stream_handle(stream)), "spec_ngram_draft_adaptive")
    return draft, length, n, pos, gam


def probe_read(src, out=None, stream=None):
    """Streaming read of a device tensor (bandwidth probe)."""
    torch = _torch()
    nbytes = src.numel() * src.element_size()
    nb = int(load().spec_probe_read_blocks(nbytes))
    if out is None:
        with _on(stream):
            out = torch.empty(nb, dtype=torch.float32, device=src.device)
    _check(load().spec_probe_read(_ptr(src), nbytes, _ptr(out), _stream_handle(stream)),
           "spec_probe_read")
    return out


def probe_copy(src, dst, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("destination too small")
    _check(load().spec_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream_handle(stream)),
           "spec_probe_copy")
