"""ctypes binding of the C ABI in include/specverify.h.

Argument marshalling only: every step of the verification runs in the HIP
kernels of libspecverify.so.  The functions keep the C names
(``specverify_create``, ``specverify_run``, ``specverify_destroy``);
``SpecVerify`` wraps them for torch tensors, which serve as device memory,
and the current torch stream.  If the library is missing the import of this
module succeeds but every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIB selects another build of the library (same ABI)
LIB_PATH = os.environ.get("SPECVERIFY_LIB", os.path.join(PKG, "libspecverify.so"))

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_OUT_OF_MEMORY, ERR_DEVICE, ERR_TOO_LARGE = range(6)
F32, BF16 = 0, 1
STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "OUT_OF_MEMORY", 4: "DEVICE",
                5: "TOO_LARGE"}
CHUNK = {"bf16": 2048, "f32": 1024}   # logits per V-chunk (4 KB of a row: one wave's item)
MAX_CHUNKS = {"bf16": 128, "f32": 256}
EXPORTED = ("specverify_create", "specverify_run", "specverify_destroy",
            "specverify_set_timing", "specverify_timing_totals",
            "specverify_chunks_per_row", "specverify_workspace_bytes", "specverify_commit",
            "specverify_probe_read", "specverify_run_static", "specverify_run_tree")


class Config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_gamma", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("device", ctypes.c_int32), ("spin_limit", ctypes.c_int32)]


class Inputs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("cu_draft", ctypes.c_void_p), ("num_draft_rows", ctypes.c_int32),
                ("target_logits", ctypes.c_void_p), ("target_stride", ctypes.c_int64),
                ("draft_logits", ctypes.c_void_p), ("draft_stride", ctypes.c_int64),
                ("draft_tokens", ctypes.c_void_p), ("uniforms", ctypes.c_void_p),
                ("temperatures", ctypes.c_void_p)]


class Outputs(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("p_draft", ctypes.c_void_p), ("q_draft", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("resid_mass", ctypes.c_void_p)]


class TreeInputs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("cu_nodes", ctypes.c_void_p), ("num_nodes", ctypes.c_int32),
                ("parents", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("target_logits", ctypes.c_void_p), ("target_stride", ctypes.c_int64),
                ("uniforms", ctypes.c_void_p), ("temperatures", ctypes.c_void_p)]


class TreeOutputs(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("out_nodes", ctypes.c_void_p), ("p_cand", ctypes.c_void_p)]


class CommitArgs(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("cu_draft", ctypes.c_void_p), ("num_draft_rows", ctypes.c_int32),
                ("accepted_len", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("seq_tokens", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("capacity", ctypes.c_int32), ("seq_lens", ctypes.c_void_p),
                ("appended", ctypes.c_void_p), ("next_token", ctypes.c_void_p)]


class SpecVerifyError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where} failed: SPECVERIFY_ERR_{STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(the verifier has no fallback path)")
    # torch ships its own HIP runtime with the same soname (libamdhip64.so.7).
    # Importing torch first makes the library bind to that runtime, so that the
    # process holds one HIP runtime whose device pointers and streams both sides
    # share; without torch the library binds to the system ROCm runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.specverify_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_void_p)]
    lib.specverify_create.restype = ctypes.c_int
    lib.specverify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(Inputs), ctypes.POINTER(Outputs),
                                   ctypes.c_void_p]
    lib.specverify_run.restype = ctypes.c_int
    lib.specverify_run_static.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Inputs), ctypes.POINTER(Outputs),
                                          ctypes.c_void_p]
    lib.specverify_run_static.restype = ctypes.c_int
    lib.specverify_run_tree.argtypes = [ctypes.c_void_p, ctypes.POINTER(TreeInputs), ctypes.POINTER(TreeOutputs),
                                        ctypes.c_void_p]
    lib.specverify_run_tree.restype = ctypes.c_int
    lib.specverify_destroy.argtypes = [ctypes.c_void_p]
    lib.specverify_destroy.restype = ctypes.c_int
    lib.specverify_chunks_per_row.argtypes = [ctypes.c_void_p]
    lib.specverify_chunks_per_row.restype = ctypes.c_int32
    lib.specverify_workspace_bytes.argtypes = [ctypes.c_void_p]
    lib.specverify_workspace_bytes.restype = ctypes.c_int64
    lib.specverify_set_timing.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.specverify_set_timing.restype = ctypes.c_int
    lib.specverify_timing_totals.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_float),
                                             ctypes.POINTER(ctypes.c_float)]
    lib.specverify_timing_totals.restype = ctypes.c_int
    lib.specverify_commit.argtypes = [ctypes.c_void_p, ctypes.POINTER(CommitArgs), ctypes.c_void_p]
    lib.specverify_commit.restype = ctypes.c_int
    lib.specverify_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.specverify_probe_read.restype = ctypes.c_int
    _lib = lib
    return lib


def specverify_create(cfg: Config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    st = load_library().specverify_create(ctypes.byref(cfg), ctypes.byref(h))
    if st != OK:
        raise SpecVerifyError("specverify_create", st)
    return h


def specverify_run(h: ctypes.c_void_p, inputs: Inputs, outputs: Outputs, stream: int) -> None:
    st = load_library().specverify_run(h, ctypes.byref(inputs), ctypes.byref(outputs),
                                       ctypes.c_void_p(stream))
    if st != OK:
        raise SpecVerifyError("specverify_run", st)


def specverify_run_static(cfg: Config, inputs: Inputs, outputs: Outputs, stream: int) -> None:
    st = load_library().specverify_run_static(ctypes.byref(cfg), ctypes.byref(inputs), ctypes.byref(outputs),
                                              ctypes.c_void_p(stream))
    if st != OK:
        raise SpecVerifyError("specverify_run_static", st)


def specverify_run_tree(h: ctypes.c_void_p, inputs: TreeInputs, outputs: TreeOutputs, stream: int) -> None:
    st = load_library().specverify_run_tree(h, ctypes.byref(inputs), ctypes.byref(outputs), ctypes.c_void_p(stream))
    if st != OK:
        raise SpecVerifyError("specverify_run_tree", st)


def specverify_commit(h: ctypes.c_void_p, args: CommitArgs, stream: int) -> None:
    st = load_library().specverify_commit(h, ctypes.byref(args), ctypes.c_void_p(stream))
    if st != OK:
        raise SpecVerifyError("specverify_commit", st)


def specverify_probe_read(a, b, sink, stream: int) -> None:
    """The streaming-read probe over two device tensors (see the header)."""
    st = load_library().specverify_probe_read(
        ctypes.c_void_p(a.data_ptr()), a.numel() * a.element_size(),
        ctypes.c_void_p(b.data_ptr() if b is not None else 0), 0 if b is None else b.numel() * b.element_size(),
        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream))
    if st != OK:
        raise SpecVerifyError("specverify_probe_read", st)


def specverify_destroy(h: ctypes.c_void_p) -> None:
    st = load_library().specverify_destroy(h)
    if st != OK:
        raise SpecVerifyError("specverify_destroy", st)


_DEVICES = {}


def _cuda_device(i: int):
    """torch.device("cuda", i), built once per ordinal."""
    d = _DEVICES.get(i)
    if d is None:
        import torch
        d = _DEVICES[i] = torch.device("cuda", i)
    return d


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_vec(name, t, dtype, device, n, required=True):
    """A 1-D run of at least n elements of `dtype` on `device`, unit stride."""
    if t is None:
        if required and n > 0:
            raise ValueError(f"{name} is required")
        return
    # the common case in one expression (dtypes are singletons); the checks
    # below only name what failed
    if t.dtype is dtype and t.device == device and t.is_contiguous() and t.numel() >= n:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the run needs {n}")


def check_run_args(*, vocab, logits_dtype, device, target, draft, draft_tokens, uniforms, temperatures,
                   accepted_len, out_tokens, gamma=None, cu_draft=None, num_draft_rows=None,
                   diagnostics=()):
    """Check the tensors of one run against the C ABI's layout before any of
    their pointers is passed on (the library reads raw memory: a wrong dtype
    would be misread, a short tensor read past its end).  Returns
    (B, R_d, R_t).  Raises TypeError or ValueError.

    ``device`` is the handle's torch device; ``diagnostics`` holds the
    optional float32 outputs (p_draft, q_draft, beta, resid_mass), None
    entries skipped."""
    import torch
    if temperatures is None or temperatures.dim() != 1:
        raise ValueError("temperatures must be a 1-D tensor of B float32 values")
    B = int(temperatures.shape[0])
    if cu_draft is None:
        if gamma is None or int(gamma) < 0:
            raise ValueError("a uniform run needs gamma >= 0 (or cu_draft for a ragged one)")
        R_d = B * int(gamma)
    else:
        if num_draft_rows is None:
            raise ValueError("a ragged run needs num_draft_rows (the host copy of cu_draft[B])")
        R_d = int(num_draft_rows)
        if R_d < 0:
            raise ValueError("num_draft_rows must be >= 0")
        _check_vec("cu_draft", cu_draft, torch.int32, device, B + 1)
    R_t = R_d + B
    for name, t, rows in (("target", target, R_t), ("draft", draft, R_d)):
        if t is None or (name == "draft" and t.numel() == 0):
            if name == "target" and R_t > 0:
                raise ValueError("target logits are required")
            continue
        sh, st = t.shape, t.stride()
        if (t.dtype is logits_dtype and t.device == device and len(sh) == 2 and st[1] == 1 and sh[1] >= vocab
                and st[0] >= vocab and sh[0] >= rows):
            continue   # the common case; the checks below name what failed
        if t.dtype != logits_dtype:
            raise TypeError(f"{name} logits must be {logits_dtype}, got {t.dtype}")
        if t.device != device:
            raise ValueError(f"{name} logits must be on {device}, got {t.device}")
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} logits must be a 2-D tensor with unit column stride")
        if t.shape[1] < vocab or t.stride(0) < vocab:
            raise ValueError(f"{name} logits rows must hold the vocabulary ({vocab}), got shape "
                             f"{tuple(t.shape)} stride {t.stride(0)}")
        if t.shape[0] < rows:
            raise ValueError(f"{name} logits have {t.shape[0]} rows, the run needs {rows}")
    _check_vec("draft_tokens", draft_tokens, torch.int32, device, R_d)
    _check_vec("uniforms", uniforms, torch.float32, device, R_t)
    _check_vec("temperatures", temperatures, torch.float32, device, B)
    _check_vec("accepted_len", accepted_len, torch.int32, device, B)
    _check_vec("out_tokens", out_tokens, torch.int32, device, R_t)
    for name, t in diagnostics:
        _check_vec(name, t, torch.float32, device, R_d, required=False)
    return B, R_d, R_t


def check_tree_args(*, vocab, logits_dtype, device, target, cu_nodes, num_nodes, parents, tokens, uniforms,
                    temperatures, accepted_len, out_tokens, out_nodes=None, p_cand=None):
    """The tensors of one tree run (see specverify_run_tree): checked as
    check_run_args does.  Returns (B, N, R_t)."""
    import torch
    if temperatures is None or temperatures.dim() != 1:
        raise ValueError("temperatures must be a 1-D tensor of B float32 values")
    B = int(temperatures.shape[0])
    N = int(num_nodes)
    if N < 0:
        raise ValueError("num_nodes must be >= 0")
    R_t = N + B
    _check_vec("cu_nodes", cu_nodes, torch.int32, device, B + 1)
    if target is None:
        if R_t > 0:
            raise ValueError("target logits are required")
    else:
        if target.dtype != logits_dtype:
            raise TypeError(f"target logits must be {logits_dtype}, got {target.dtype}")
        if target.device != device:
            raise ValueError(f"target logits must be on {device}, got {target.device}")
        if target.dim() != 2 or target.stride(1) != 1:
            raise ValueError("target logits must be a 2-D tensor with unit column stride")
        if target.shape[1] < vocab or target.stride(0) < vocab:
            raise ValueError(f"target logits rows must hold the vocabulary ({vocab})")
        if target.shape[0] < R_t:
            raise ValueError(f"target logits have {target.shape[0]} rows, the run needs {R_t}")
    _check_vec("parents", parents, torch.int32, device, N)
    _check_vec("tokens", tokens, torch.int32, device, N)
    _check_vec("uniforms", uniforms, torch.float32, device, R_t)
    _check_vec("temperatures", temperatures, torch.float32, device, B)
    _check_vec("accepted_len", accepted_len, torch.int32, device, B)
    _check_vec("out_tokens", out_tokens, torch.int32, device, R_t)
    _check_vec("out_nodes", out_nodes, torch.int32, device, R_t, required=False)
    _check_vec("p_cand", p_cand, torch.float32, device, N, required=False)
    return B, N, R_t


def check_commit_args(*, device, accepted_len, out_tokens, seq_tokens, seq_lens, gamma=None, cu_draft=None,
                      num_draft_rows=None, appended=None, next_token=None):
    """Check the tensors of one commit (see ``check_run_args``).  Returns
    (B, R_t)."""
    import torch
    if accepted_len is None or accepted_len.dim() != 1:
        raise ValueError("accepted_len must be a 1-D int32 tensor of B values")
    B = int(accepted_len.shape[0])
    if cu_draft is None:
        if gamma is None or int(gamma) < 0:
            raise ValueError("a uniform commit needs gamma >= 0 (or cu_draft)")
        R_d = B * int(gamma)
    else:
        if num_draft_rows is None or int(num_draft_rows) < 0:
            raise ValueError("a ragged commit needs num_draft_rows >= 0")
        R_d = int(num_draft_rows)
        _check_vec("cu_draft", cu_draft, torch.int32, device, B + 1)
    R_t = R_d + B
    _check_vec("accepted_len", accepted_len, torch.int32, device, B)
    _check_vec("out_tokens", out_tokens, torch.int32, device, R_t)
    _check_vec("seq_lens", seq_lens, torch.int32, device, B)
    _check_vec("appended", appended, torch.int32, device, B, required=False)
    _check_vec("next_token", next_token, torch.int32, device, B, required=False)
    if seq_tokens is None or seq_tokens.dim() != 2 or seq_tokens.stride(1) != 1:
        raise ValueError("seq_tokens must be a 2-D tensor with unit column stride")
    if seq_tokens.dtype != torch.int32:
        raise TypeError(f"seq_tokens must be torch.int32, got {seq_tokens.dtype}")
    if seq_tokens.device != device:
        raise ValueError(f"seq_tokens must be on {device}, got {seq_tokens.device}")
    if seq_tokens.shape[0] < B:
        raise ValueError(f"seq_tokens has {seq_tokens.shape[0]} rows, the commit needs {B}")
    return B, R_t


def _marshal_run(cfg, target, draft, draft_tokens, uniforms, temperatures, accepted_len, out_tokens, gamma,
                 cu_draft, num_draft_rows, p_draft, q_draft, beta, resid_mass, stream):
    """Check the tensors of a run against cfg (.dtype, .vocab, .device) and
    fill the C structs; returns (Inputs, Outputs, stream handle)."""
    import torch
    want = torch.float32 if cfg.dtype == F32 else torch.bfloat16
    batch, R_d, _ = check_run_args(
        vocab=cfg.vocab, logits_dtype=want, device=_cuda_device(cfg.device), target=target,
        draft=draft, draft_tokens=draft_tokens, uniforms=uniforms, temperatures=temperatures,
        accepted_len=accepted_len, out_tokens=out_tokens, gamma=gamma, cu_draft=cu_draft,
        num_draft_rows=num_draft_rows,
        diagnostics=(("p_draft", p_draft), ("q_draft", q_draft), ("beta", beta), ("resid_mass", resid_mass)))
    # draft None with drafted tokens: token-only drafts (q_i = delta_{x_i})
    has_draft = draft is not None and draft.numel() > 0
    has_tokens = draft_tokens is not None and draft_tokens.numel() > 0
    # positional construction: one call instead of a ctypes assignment per field
    inp = Inputs(batch, 0 if cu_draft is not None else int(gamma), _ptr(cu_draft), R_d,
                 _ptr(target), int(target.stride(0)),
                 draft.data_ptr() if has_draft else None,
                 int(draft.stride(0)) if has_draft else int(cfg.vocab),
                 draft_tokens.data_ptr() if has_tokens else None,
                 _ptr(uniforms), _ptr(temperatures))
    out = Outputs(_ptr(accepted_len), _ptr(out_tokens), _ptr(p_draft), _ptr(q_draft),
                  _ptr(beta), _ptr(resid_mass))
    s = stream if stream is not None else torch.cuda.current_stream(cfg.device).cuda_stream
    return inp, out, int(s)


class SpecVerify:
    """A handle bound to one device, vocabulary and logits dtype.

    ``run`` takes torch tensors that already live on the device (target
    [R_t, V], draft [R_d, V], float32 or bfloat16) and launches on the
    current torch stream; it returns without synchronising.
    """

    def __init__(self, max_batch: int, max_gamma: int, vocab: int, dtype: str = "bf16",
                 device: int = 0, spin_limit: int = 0):
        self.dtype = {"f32": F32, "bf16": BF16}[dtype]
        self.vocab = vocab
        self.device = device
        self.cfg = Config(max_batch, max_gamma, vocab, self.dtype, device, spin_limit)
        self.handle = specverify_create(self.cfg)
        lib = load_library()
        self.chunks = int(lib.specverify_chunks_per_row(self.handle))
        self.workspace_bytes = int(lib.specverify_workspace_bytes(self.handle))

    def set_timing(self, enable: bool) -> None:
        st = load_library().specverify_set_timing(self.handle, 1 if enable else 0)
        if st != OK:
            raise SpecVerifyError("specverify_set_timing", st)

    def timing_totals(self):
        """(runs, stream_ms, finish_ms): the runs recorded since timing was
        enabled (or last read) and the summed kernel durations; waits for them."""
        n, a, f = ctypes.c_int32(), ctypes.c_float(), ctypes.c_float()
        st = load_library().specverify_timing_totals(self.handle, ctypes.byref(n), ctypes.byref(a),
                                                     ctypes.byref(f))
        if st != OK:
            raise SpecVerifyError("specverify_timing_totals", st)
        return n.value, a.value, f.value

    def close(self) -> None:
        if getattr(self, "handle", None):
            specverify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def run(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len, out_tokens, *,
            gamma: Optional[int] = None, cu_draft=None, num_draft_rows: Optional[int] = None,
            p_draft=None, q_draft=None, beta=None, resid_mass=None, stream=None) -> None:
        inp, out, s = _marshal_run(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len,
                                   out_tokens, gamma, cu_draft, num_draft_rows, p_draft, q_draft, beta,
                                   resid_mass, stream)
        specverify_run(self.handle, inp, out, s)

    def prepare(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len, out_tokens, *,
                gamma: Optional[int] = None, cu_draft=None, num_draft_rows: Optional[int] = None,
                p_draft=None, q_draft=None, beta=None, resid_mass=None) -> "PreparedRun":
        """The same arguments as ``run``, checked once: the returned
        ``PreparedRun`` launches on these tensors each time it is called,
        without checking them again (a serving loop that keeps its input and
        output buffers).  It holds references to the tensors; their storage,
        shape and dtype must not change while it is in use."""
        inp, out, _ = _marshal_run(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len,
                                   out_tokens, gamma, cu_draft, num_draft_rows, p_draft, q_draft, beta,
                                   resid_mass, 0)
        keep = (target, draft, draft_tokens, uniforms, temperatures, accepted_len, out_tokens, cu_draft, p_draft,
                q_draft, beta, resid_mass)
        return PreparedRun(self, inp, out, keep)

    def run_tree(self, target, cu_nodes, num_nodes: int, parents, tokens, uniforms, temperatures, accepted_len,
                 out_tokens, *, out_nodes=None, p_cand=None, stream=None) -> None:
        """Verification over draft trees (specverify_run_tree), on the current
        torch stream; returns without synchronising."""
        import torch
        want = torch.float32 if self.dtype == F32 else torch.bfloat16
        B, N, _ = check_tree_args(
            vocab=self.vocab, logits_dtype=want, device=torch.device("cuda", self.device), target=target,
            cu_nodes=cu_nodes, num_nodes=num_nodes, parents=parents, tokens=tokens, uniforms=uniforms,
            temperatures=temperatures, accepted_len=accepted_len, out_tokens=out_tokens, out_nodes=out_nodes,
            p_cand=p_cand)
        inp = TreeInputs(B, _ptr(cu_nodes), N, _ptr(parents) if N > 0 else None, _ptr(tokens) if N > 0 else None,
                         _ptr(target), int(target.stride(0)), _ptr(uniforms), _ptr(temperatures))
        out = TreeOutputs(_ptr(accepted_len), _ptr(out_tokens), _ptr(out_nodes), _ptr(p_cand))
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        specverify_run_tree(self.handle, inp, out, int(s))

    def commit(self, accepted_len, out_tokens, seq_tokens, seq_lens, *, gamma: Optional[int] = None,
               cu_draft=None, num_draft_rows: Optional[int] = None, appended=None, next_token=None,
               stream=None) -> None:
        """Append each sequence's emitted tokens of a run to its row of
        ``seq_tokens`` [B, capacity] (int32, device) at ``seq_lens`` [B]; see
        specverify_commit in include/specverify.h."""
        import torch
        B, R_t = check_commit_args(device=torch.device("cuda", self.device), accepted_len=accepted_len,
                                   out_tokens=out_tokens, seq_tokens=seq_tokens, seq_lens=seq_lens, gamma=gamma,
                                   cu_draft=cu_draft, num_draft_rows=num_draft_rows, appended=appended,
                                   next_token=next_token)
        a = CommitArgs()
        a.batch = B
        if cu_draft is None:
            a.gamma = int(gamma)
            a.cu_draft = None
            a.num_draft_rows = R_t - B
        else:
            a.gamma = 0
            a.cu_draft = _ptr(cu_draft)
            a.num_draft_rows = R_t - B
        a.accepted_len = _ptr(accepted_len)
        a.out_tokens = _ptr(out_tokens)
        a.seq_tokens = _ptr(seq_tokens)
        a.seq_stride = int(seq_tokens.stride(0))
        a.capacity = int(seq_tokens.shape[1])
        a.seq_lens = _ptr(seq_lens)
        a.appended = _ptr(appended)
        a.next_token = _ptr(next_token)
        s = stream if stream is not None else torch.cuda.current_stream(self.device).cuda_stream
        specverify_commit(self.handle, a, int(s))


class PreparedRun:
    """A run of one handle on fixed tensors (see ``SpecVerify.prepare``).
    ``prepared()`` launches on the current torch stream of the handle's
    device, ``prepared(stream)`` on a given HIP stream handle; like ``run``
    it returns without synchronising."""

    def __init__(self, sv: "SpecVerify", inp: Inputs, out: Outputs, keep):
        self._sv = sv            # keeps the handle open
        self._keep = keep        # keeps the tensors alive
        self._inp, self._out = inp, out
        self._fn = load_library().specverify_run
        self._args = (ctypes.byref(inp), ctypes.byref(out))
        self._device = sv.device

    def __call__(self, stream: Optional[int] = None) -> None:
        if not self._sv.handle:
            raise RuntimeError("the handle of this prepared run is closed")
        if stream is None:
            import torch
            stream = torch.cuda.current_stream(self._device).cuda_stream
        st = self._fn(self._sv.handle, self._args[0], self._args[1], ctypes.c_void_p(stream))
        if st != OK:
            raise SpecVerifyError("specverify_run", st)


class SpecVerifyStatic:
    """Runs without a handle or any device allocation (specverify_run_static):
    the same ``run`` as SpecVerify, on the library's per-device static
    scratch.  Calls on one device must be ordered (one stream)."""

    def __init__(self, max_batch: int, max_gamma: int, vocab: int, dtype: str = "bf16",
                 device: int = 0, spin_limit: int = 0):
        self.dtype = {"f32": F32, "bf16": BF16}[dtype]
        self.vocab = vocab
        self.device = device
        self.cfg = Config(max_batch, max_gamma, vocab, self.dtype, device, spin_limit)

    def run(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len, out_tokens, *,
            gamma: Optional[int] = None, cu_draft=None, num_draft_rows: Optional[int] = None,
            p_draft=None, q_draft=None, beta=None, resid_mass=None, stream=None) -> None:
        inp, out, s = _marshal_run(self, target, draft, draft_tokens, uniforms, temperatures, accepted_len,
                                   out_tokens, gamma, cu_draft, num_draft_rows, p_draft, q_draft, beta,
                                   resid_mass, stream)
        specverify_run_static(self.cfg, inp, out, s)

    def close(self) -> None:
        pass
