"""ctypes binding of libstca (include/stca.h), same call names, argument marshalling only.

Every step of the STCA forward runs in the HIP library; this module only lays inputs out in
device memory (through PyTorch tensors), fills the C structs and checks status codes.  If the
library has not been built it raises at import time: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

# STCA_LIB may name another build of the same library (for instance libstca_debug.so, whose kernels
# check their ragged indices); the default is the ordinary build next to this file.
LIB_PATH = os.environ.get("STCA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstca.so")
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstca_debug.so")
MAX_M = 8

F32, BF16 = 0, 1
(PHASE_PACK, PHASE_ENCODE, PHASE_QUERY, PHASE_UPROJ, PHASE_ATTEND, PHASE_COMBINE, PHASE_PROJECT,
 PHASE_BWD_RECOMPUTE, PHASE_BWD_ATTEND, PHASE_BWD_ENCODE, PHASE_BWD_TARGET) = range(11)
PHASE_NAMES = ["pack", "encode", "query", "uproj", "attend", "combine", "project",
               "bwd_recompute", "bwd_attend", "bwd_encode", "bwd_target"]
N_PHASES = 11

EXPORTS = [
    "stca_encode_workspace_size", "stca_attend_workspace_size", "stca_forward_workspace_size",
    "stca_predict_workspace_size", "stca_encode", "stca_attend", "stca_forward", "stca_predict",
    "stca_sl_beta", "stca_sl_plan", "stca_sl_pack", "stca_litm_plan", "stca_litm_merge",
    "stca_backward_workspace_size", "stca_backward_workspace_size_keep", "stca_backward", "stca_backward_profiled",
    "stca_forward_graph_create", "stca_graph_launch", "stca_graph_destroy", "stca_profiler_create", "stca_profiler_destroy",
    "stca_profiler_reset", "stca_profiler_read", "stca_forward_profiled", "stca_status_string",
    "stca_last_error", "stca_version", "stca_validate_batch", "stca_attend_noalloc", "stca_debug_flags",
    "stca_debug_selftest",
]


class Dims(ctypes.Structure):
    _fields_ = [("d", c_int32), ("h", c_int32), ("M", c_int32), ("r", c_int32), ("dtype", c_int32),
                ("ln_eps", c_float), ("query_ln", c_int32), ("attn_chunk", c_int32), ("encode_layers", c_int32)]


class Ffn(ctypes.Structure):
    _fields_ = [("Wu", c_void_p), ("Wv", c_void_p), ("Wo", c_void_p), ("gamma", c_void_p), ("beta", c_void_p)]


class WeightsC(ctypes.Structure):
    _fields_ = [("hist", Ffn * MAX_M), ("query", Ffn * MAX_M), ("WQ", c_void_p * MAX_M),
                ("WK", c_void_p * MAX_M), ("WV", c_void_p * MAX_M), ("WO", c_void_p * MAX_M),
                ("WC", c_void_p * MAX_M)]


class BatchC(ctypes.Structure):
    _fields_ = [("n_users", c_int32), ("hist_off", c_void_p), ("tgt_off", c_void_p), ("total_L", c_int64),
                ("total_T", c_int64), ("max_L", c_int64), ("max_T", c_int64)]


class FfnGrad(ctypes.Structure):
    _fields_ = [("dWu", c_void_p), ("dWv", c_void_p), ("dWo", c_void_p), ("dgamma", c_void_p), ("dbeta", c_void_p)]


class GradsC(ctypes.Structure):
    _fields_ = [("dX", c_void_p), ("dxt", c_void_p), ("hist", FfnGrad * MAX_M), ("query", FfnGrad * MAX_M),
                ("dWQ", c_void_p * MAX_M), ("dWK", c_void_p * MAX_M), ("dWV", c_void_p * MAX_M),
                ("dWO", c_void_p * MAX_M), ("dWC", c_void_p * MAX_M)]


class ProfileReport(ctypes.Structure):
    _fields_ = [("ms", c_double * N_PHASES), ("launches", c_int64 * N_PHASES)]


class SlParams(ctypes.Structure):
    _fields_ = [("L_min", c_int32), ("L_max", c_int32), ("L_avg", c_int32), ("L_infer", c_int32)]


class StcaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status}): {last_error()}")


def _load(path: str | None = None) -> ctypes.CDLL:
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"libstca.so not built at {path}; run `python -m target_cross_attention_amd.build`")
    # PyTorch ships its own HIP runtime (same soname, libamdhip64.so.7).  Loading it first makes
    # the dynamic loader bind libstca to that one copy, so device memory and streams created by
    # torch are valid in libstca's calls; loading libstca first would bring in a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "stca_encode_workspace_size": [P, c_int64, POINTER(c_size_t)],
        "stca_attend_workspace_size": [P, P, POINTER(c_size_t)],
        "stca_forward_workspace_size": [P, P, POINTER(c_size_t)],
        "stca_predict_workspace_size": [P, c_int64, POINTER(c_size_t)],
        "stca_encode": [P, P, c_int64, P, P, P, c_size_t, P],
        "stca_attend": [P, P, c_int32, P, P, P, P, P, c_size_t, P],
        "stca_forward": [P, P, P, P, P, P, P, c_size_t, P],
        "stca_forward_profiled": [P, P, P, P, P, P, P, c_size_t, P, P],
        "stca_predict": [P, P, P, c_int64, P, P, P, P, c_size_t, P],
        "stca_sl_beta": [P, ctypes.c_double, POINTER(ctypes.c_double)],
        "stca_sl_plan": [P, c_int32, P, P, P, P, P],
        "stca_sl_pack": [P, c_int32, P, P, c_int64, c_int64, P, P, P],
        "stca_litm_plan": [c_int32, P, P, c_int32, P, P, P, POINTER(c_int64)],
        "stca_litm_merge": [P, c_int64, c_int64, P, P, P, P, P],
        "stca_backward_workspace_size": [P, P, POINTER(c_size_t)],
        "stca_backward_workspace_size_keep": [P, P, POINTER(c_size_t)],
        "stca_backward": [P, P, P, P, P, P, P, P, c_size_t, P],
        "stca_backward_profiled": [P, P, P, P, P, P, P, P, c_size_t, P, P],
        "stca_forward_graph_create": [P, P, P, P, P, P, P, c_size_t, POINTER(c_void_p)],
        "stca_graph_launch": [P, P],
        "stca_graph_destroy": [P],
        "stca_profiler_create": [POINTER(c_void_p)],
        "stca_profiler_destroy": [P],
        "stca_profiler_reset": [P],
        "stca_profiler_read": [P, P],
        "stca_validate_batch": [P, P, P],
        "stca_attend_noalloc": [P, P, c_int32, P, P, P, P, P],
        "stca_debug_flags": [POINTER(ctypes.c_uint32), POINTER(c_int32), c_int32],
        "stca_debug_selftest": [P],
        "stca_status_string": [c_int],
        "stca_last_error": [],
        "stca_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_char_p if name in ("stca_status_string", "stca_last_error", "stca_version") else c_int
    return lib


LIB = _load()


def load_library(path: str) -> ctypes.CDLL:
    """Another build of the same library (a variant built with `build.py --define ... --out path`),
    with the same signatures.  The module's calls go to `LIB`; a caller that compares builds in one
    process assigns the handle to `LIB` around its calls."""
    return _load(path)


def status_string(status: int) -> str:
    return LIB.stca_status_string(status).decode()


def last_error() -> str:
    return LIB.stca_last_error().decode()


def version() -> str:
    return LIB.stca_version().decode()


def _check(status: int, where: str):
    if status != 0:
        raise StcaError(status, where)


def _ref(s):
    return ctypes.byref(s)


# ----------------------------------------------------------------------------------------------
# plain structs
# ----------------------------------------------------------------------------------------------
def make_dims(d: int, h: int, M: int, r: int, dtype: str = "bf16", ln_eps: float = 1e-5,
              query_ln: bool = False, attn_chunk: int = 0, encode_layers: int = 0) -> Dims:
    return Dims(d, h, M, r, BF16 if dtype == "bf16" else F32, ln_eps, int(bool(query_ln)), attn_chunk,
                encode_layers)


def dims_for(cfg, **kw) -> Dims:
    """Dims of a ``stca_inputs.Config``."""
    return make_dims(cfg.d, cfg.h, cfg.M, cfg.r, cfg.dtype, **kw)


def batch_struct(n_users: int, hist_off, tgt_off, total_L: int, total_T: int, max_L: int, max_T: int) -> BatchC:
    return BatchC(n_users, _ptr(hist_off), _ptr(tgt_off), total_L, total_T, max_L, max_T)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on(stream):
    """Context in which tensors the binding allocates for a call (outputs, workspaces) belong to the
    call's stream: torch's caching allocator ties a block to the stream current at allocation and
    reuses it on that stream once freed, so a workspace dropped after an asynchronous call on a
    non-current stream is never handed to other work before that call has finished."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


# ----------------------------------------------------------------------------------------------
# device-resident inputs
# ----------------------------------------------------------------------------------------------
def to_device(a: np.ndarray, dtype: str, device):
    """Host array -> device tensor in the storage type: uint16 bf16 patterns or float32."""
    import torch
    if dtype == "bf16":
        if a.dtype == np.uint16:  # already bf16 bit patterns
            return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)
        # torch's float32 -> bfloat16 conversion rounds to nearest even
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class DeviceWeights:
    """``stca_inputs.Weights`` uploaded in the storage type, plus the filled ``stca_weights`` struct."""

    def __init__(self, W, dtype: str, device="cuda"):
        import torch
        self.keep = []
        self.c = WeightsC()
        M = len(W.Wu)
        cache = {}

        def up(a, store=dtype):
            if a is None:
                return None
            key = (id(a), store)
            if key not in cache:
                t = to_device(a, store, device) if store != "f32ln" else \
                    torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
                cache[key] = t
                self.keep.append(t)
            return cache[key].data_ptr()

        for i in range(M):
            self.c.hist[i] = Ffn(up(W.Wu[i]), up(W.Wv[i]), up(W.Wo[i]), up(W.gamma[i], "f32ln"),
                                 up(W.beta[i], "f32ln"))
            self.c.query[i] = Ffn(up(W.qWu[i]), up(W.qWv[i]), up(W.qWo[i]), up(W.qgamma[i], "f32ln"),
                                  up(W.qbeta[i], "f32ln"))
            self.c.WQ[i] = up(W.WQ[i])
            self.c.WK[i] = up(W.WK[i])
            self.c.WV[i] = up(W.WV[i])
            self.c.WO[i] = up(W.WO[i])
            self.c.WC[i] = up(W.WC[i]) if W.WC[i] is not None else None


class DevicePredict:
    """``stca_inputs.PredictWeights`` uploaded in the storage type: ``WZ`` and the ``stca_ffn``
    struct of the prediction FFN (no LayerNorm parameters)."""

    def __init__(self, P, dtype: str, device="cuda"):
        self.WZ = to_device(P.WZ, dtype, device)
        self.Wu = to_device(P.Wu, dtype, device)
        self.Wv = to_device(P.Wv, dtype, device)
        self.Wo = to_device(P.Wo, dtype, device)
        self.ffn = Ffn(self.Wu.data_ptr(), self.Wv.data_ptr(), self.Wo.data_ptr(), None, None)


class DeviceBatch:
    """A ``stca_inputs.Inputs`` batch uploaded to the device, plus the ``stca_batch`` struct."""

    def __init__(self, inp, device="cuda"):
        import torch
        self.inp = inp
        dt = inp.cfg.dtype
        self.X = to_device(inp.X, dt, device) if inp.X.size else torch.empty(0, device=device)
        self.xt = to_device(inp.xt, dt, device) if inp.xt.size else torch.empty(0, device=device)
        self.hist_off = torch.from_numpy(inp.hist_off.astype(np.int64)).to(device)
        self.tgt_off = torch.from_numpy(inp.tgt_off.astype(np.int64)).to(device)
        self.total_L = int(inp.hist_off[-1])
        self.total_T = int(inp.tgt_off[-1])
        self.max_L = int(inp.L.max()) if len(inp.L) else 0
        self.max_T = int(inp.m.max()) if len(inp.m) else 0
        self.c = batch_struct(inp.n_users, self.hist_off, self.tgt_off, self.total_L, self.total_T,
                              self.max_L, self.max_T)


# ----------------------------------------------------------------------------------------------
# calls
# ----------------------------------------------------------------------------------------------
def encode_workspace_size(dims: Dims, n_rows: int) -> int:
    n = c_size_t(0)
    _check(LIB.stca_encode_workspace_size(_ref(dims), n_rows, ctypes.byref(n)), "stca_encode_workspace_size")
    return n.value


def attend_workspace_size(dims: Dims, batch: BatchC) -> int:
    n = c_size_t(0)
    _check(LIB.stca_attend_workspace_size(_ref(dims), _ref(batch), ctypes.byref(n)), "stca_attend_workspace_size")
    return n.value


def forward_workspace_size(dims: Dims, batch: BatchC) -> int:
    n = c_size_t(0)
    _check(LIB.stca_forward_workspace_size(_ref(dims), _ref(batch), ctypes.byref(n)),
           "stca_forward_workspace_size")
    return n.value


def predict_workspace_size(dims: Dims, n_targets: int) -> int:
    n = c_size_t(0)
    _check(LIB.stca_predict_workspace_size(_ref(dims), n_targets, ctypes.byref(n)), "stca_predict_workspace_size")
    return n.value


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def stca_encode(dims: Dims, ffn: Ffn, X, Xt=None, ws=None, stream=None):
    """eq. (2) for every row of X (device tensor, storage dtype).  Returns Xt."""
    import torch
    n = X.shape[0]
    with _on(stream):
        if Xt is None:
            Xt = torch.empty_like(X)
        if ws is None:
            ws = workspace(encode_workspace_size(dims, n), X.device)
    _check(LIB.stca_encode(_ref(dims), _ref(ffn), n, _ptr(X), _ptr(Xt), _ptr(ws), ws.numel(), _stream(stream)),
           "stca_encode")
    return Xt


def stca_attend(dims: Dims, w: DeviceWeights, layer: int, batch: DeviceBatch, Xt, q, o=None, ws=None, stream=None):
    """eqs. (13), (6) for one layer.  q: total_T x d float32 (device).  Returns o (total_T x d)."""
    import torch
    with _on(stream):
        if o is None:
            o = torch.empty((batch.total_T, dims.d), dtype=torch.float32, device=q.device)
        if ws is None:
            ws = workspace(attend_workspace_size(dims, batch.c), q.device)
    _check(LIB.stca_attend(_ref(dims), _ref(w.c), layer, _ref(batch.c), _ptr(Xt), _ptr(q), _ptr(o), _ptr(ws),
                           ws.numel(), _stream(stream)), "stca_attend")
    return o


def stca_attend_noalloc(dims: Dims, w: DeviceWeights, layer: int, batch: DeviceBatch, Xt, q, o, stream=None):
    """stca_attend in the library's fixed scratch array (no workspace, no allocation); o is the
    caller's (total_T x d float32, device).  Returns o."""
    _check(LIB.stca_attend_noalloc(_ref(dims), _ref(w.c), layer, _ref(batch.c), _ptr(Xt), _ptr(q), _ptr(o),
                                   _stream(stream)), "stca_attend_noalloc")
    return o


def stca_forward(dims: Dims, w: DeviceWeights, batch: DeviceBatch, Z=None, ws=None, stream=None, profiler=None):
    """eqs. (2)-(8) for the whole batch.  Returns Z (total_T x M x d float32)."""
    import torch
    with _on(stream):
        if Z is None:
            Z = torch.empty((batch.total_T, dims.M, dims.d), dtype=torch.float32, device=batch.X.device)
        if ws is None:
            ws = workspace(forward_workspace_size(dims, batch.c), batch.X.device)
    if profiler is None:
        st = LIB.stca_forward(_ref(dims), _ref(w.c), _ref(batch.c), _ptr(batch.X), _ptr(batch.xt), _ptr(Z),
                              _ptr(ws), ws.numel(), _stream(stream))
    else:
        st = LIB.stca_forward_profiled(_ref(dims), _ref(w.c), _ref(batch.c), _ptr(batch.X), _ptr(batch.xt),
                                       _ptr(Z), _ptr(ws), ws.numel(), _stream(stream), profiler.handle)
    _check(st, "stca_forward")
    return Z


def stca_predict(dims: Dims, pw: DevicePredict, Z, xt, z=None, ws=None, stream=None):
    """eq. (9): the prediction token of every target from Z (T x M x d fp32) and x_t (T x d,
    storage type).  Returns z (T x d float32)."""
    import torch
    T = int(Z.shape[0])
    with _on(stream):
        if z is None:
            z = torch.empty((T, dims.d), dtype=torch.float32, device=Z.device)
        if ws is None:
            ws = workspace(predict_workspace_size(dims, T), Z.device)
    st = LIB.stca_predict(_ref(dims), _ptr(pw.WZ), _ref(pw.ffn), T, _ptr(Z), _ptr(xt), _ptr(z), _ptr(ws),
                          ws.numel(), _stream(stream))
    _check(st, "stca_predict")
    return z


def validate_batch(batch: DeviceBatch, stream=None) -> int:
    """stca_validate_batch: the STCA_BATCH_* bits the batch's offsets break (0 = consistent).
    Waits for the stream to reach the check."""
    import torch
    with _on(stream):
        res = torch.full((4,), -1, dtype=torch.int32, device=batch.hist_off.device)
    _check(LIB.stca_validate_batch(_ref(batch.c), _ptr(res), _stream(stream)), "stca_validate_batch")
    (stream or torch.cuda.current_stream()).synchronize()
    return int(res[0].item())


def debug_flags(clear: bool = True) -> tuple[int, bool]:
    """(bits recorded by the kernels' index checks since the last clear, whether this build checks);
    see stca_debug_flags."""
    f = ctypes.c_uint32(0)
    en = c_int32(0)
    _check(LIB.stca_debug_flags(ctypes.byref(f), ctypes.byref(en), int(clear)), "stca_debug_flags")
    return int(f.value), bool(en.value)


def debug_selftest(stream=None):
    _check(LIB.stca_debug_selftest(_stream(stream)), "stca_debug_selftest")


def sl_beta(params: SlParams, alpha: float) -> float:
    """eq. (17): the Beta shape that puts the mean training length at L_avg."""
    b = ctypes.c_double(0.0)
    _check(LIB.stca_sl_beta(_ref(params), alpha, ctypes.byref(b)), "stca_sl_beta")
    return b.value


def sl_plan(params: SlParams, full_len, s, order):
    """Host-side stochastic-length plan: (lengths, hist_off) as int64 numpy arrays."""
    full_len = np.ascontiguousarray(full_len, np.int64)
    s = np.ascontiguousarray(s, np.float64)
    order = np.ascontiguousarray(order, np.int32)
    n = len(full_len)
    L = np.zeros(n, np.int64)
    off = np.zeros(n + 1, np.int64)
    vp = lambda a: a.ctypes.data_as(c_void_p) if a.size else None  # noqa: E731
    _check(LIB.stca_sl_plan(_ref(params), n, vp(full_len), vp(s), vp(order), vp(L), off.ctypes.data_as(c_void_p)),
           "stca_sl_plan")
    return L, off


def sl_pack(dims: Dims, full_off, hist_off, total: int, max_len: int, X_full, X_packed=None, stream=None):
    """Device gather of every user's temporal suffix (full_off/hist_off: device int64 tensors)."""
    import torch
    n_users = int(hist_off.numel()) - 1
    with _on(stream):
        if X_packed is None:
            X_packed = torch.empty((total, dims.d), dtype=X_full.dtype, device=X_full.device)
    _check(LIB.stca_sl_pack(_ref(dims), n_users, _ptr(full_off), _ptr(hist_off), total, max_len, _ptr(X_full),
                            _ptr(X_packed), _stream(stream)), "stca_sl_pack")
    return X_packed


def litm_plan(hist_off, item_id, T: int):
    """Host-side LITM grouping: (merged_off, group_off, members) as int64 numpy arrays."""
    hist_off = np.ascontiguousarray(hist_off, np.int64)
    item_id = np.ascontiguousarray(item_id, np.int64)
    n = len(hist_off) - 1
    total = int(hist_off[-1])
    merged_off = np.zeros(n + 1, np.int64)
    group_off = np.zeros(total + 1, np.int64)
    members = np.zeros(max(total, 1), np.int64)
    ng = c_int64(0)
    vp = lambda a: a.ctypes.data_as(c_void_p) if a.size else None  # noqa: E731
    _check(LIB.stca_litm_plan(n, hist_off.ctypes.data_as(c_void_p), vp(item_id), int(T),
                              merged_off.ctypes.data_as(c_void_p), group_off.ctypes.data_as(c_void_p),
                              members.ctypes.data_as(c_void_p), ctypes.byref(ng)), "stca_litm_plan")
    return merged_off, group_off[:ng.value + 1].copy(), members[:total].copy()


def litm_merge(dims: Dims, group_off, members, X, X_merged=None, stream=None):
    """Device merge of a plan's groups (group_off, members: device int64 tensors)."""
    import torch
    n_groups = int(group_off.numel()) - 1
    with _on(stream):
        if X_merged is None:
            X_merged = torch.empty((n_groups, dims.d), dtype=X.dtype, device=X.device)
    _check(LIB.stca_litm_merge(_ref(dims), int(X.shape[0]), n_groups, _ptr(group_off), _ptr(members), _ptr(X),
                               _ptr(X_merged), _stream(stream)), "stca_litm_merge")
    return X_merged


GRAD_SLOTS = ["Wu", "Wv", "Wo", "gamma", "beta", "qWu", "qWv", "qWo", "qgamma", "qbeta",
              "WQ", "WK", "WV", "WO", "WC"]


class DeviceGrads:
    """fp32 device tensors for every gradient of stca_backward, plus the filled ``stca_grads``
    struct.  ``slot(name)`` lists the per-layer tensors of a slot named as in ``oracle.grad.Grads``
    (None where the library writes nothing)."""

    def __init__(self, dims: Dims, total_L: int, total_T: int, device="cuda", with_dX=True, with_dxt=True):
        import torch
        d, M, rd = dims.d, dims.M, dims.r * dims.d
        z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=device)  # noqa: E731
        self.dX = z(max(total_L, 1), d) if with_dX else None
        self.dxt = z(max(total_T, 1), d) if with_dxt else None
        self.t = {k: [None] * M for k in GRAD_SLOTS}
        self.c = GradsC()
        self.c.dX, self.c.dxt = _ptr(self.dX), _ptr(self.dxt)
        for i in range(M):
            for pre, fg in (("", self.c.hist[i]), ("q", self.c.query[i])):
                self.t[pre + "Wu"][i], self.t[pre + "Wv"][i], self.t[pre + "Wo"][i] = z(d, rd), z(d, rd), z(rd, d)
                fg.dWu, fg.dWv, fg.dWo = (_ptr(self.t[pre + k][i]) for k in ("Wu", "Wv", "Wo"))
                if pre == "" or i == 0 or dims.query_ln:
                    self.t[pre + "gamma"][i], self.t[pre + "beta"][i] = z(d), z(d)
                    fg.dgamma, fg.dbeta = _ptr(self.t[pre + "gamma"][i]), _ptr(self.t[pre + "beta"][i])
            for k in ("WQ", "WK", "WV", "WO"):
                self.t[k][i] = z(d, d)
                getattr(self.c, "d" + k)[i] = _ptr(self.t[k][i])
            if i >= 1:
                self.t["WC"][i] = z((i + 1) * d, d)
                self.c.dWC[i] = _ptr(self.t["WC"][i])

    def slot(self, name: str):
        return self.t[name]


def backward_workspace_size(dims: Dims, batch: BatchC, keep: bool = False) -> int:
    """Workspace bytes of stca_backward; with ``keep`` the larger size that keeps the encode's
    intermediates from the forward recompute."""
    n = c_size_t(0)
    fn = LIB.stca_backward_workspace_size_keep if keep else LIB.stca_backward_workspace_size
    _check(fn(_ref(dims), _ref(batch), ctypes.byref(n)), "stca_backward_workspace_size")
    return n.value


def stca_backward(dims: Dims, w: DeviceWeights, batch: DeviceBatch, dZ, grads: DeviceGrads | None = None, ws=None,
                  stream=None, profiler=None, keep: bool = False):
    """Gradients of sum(dZ * Z) for the forward of ``batch`` (dZ: total_T x M x d float32, device).
    Returns the DeviceGrads holding them."""
    with _on(stream):
        if grads is None:
            grads = DeviceGrads(dims, batch.total_L, batch.total_T, batch.X.device)
        if ws is None:
            ws = workspace(backward_workspace_size(dims, batch.c, keep), batch.X.device)
    args = (_ref(dims), _ref(w.c), _ref(batch.c), _ptr(batch.X), _ptr(batch.xt), _ptr(dZ), _ref(grads.c), _ptr(ws),
            ws.numel(), _stream(stream))
    if profiler is None:
        _check(LIB.stca_backward(*args), "stca_backward")
    else:
        _check(LIB.stca_backward_profiled(*args, profiler.handle), "stca_backward")
    return grads


class ForwardGraph:
    """A recorded stca_forward (stca_forward_graph_create) over fixed buffers: ``launch()`` replays
    it on a stream.  Keeps the batch, weights, output and workspace tensors alive."""

    def __init__(self, dims: Dims, w: DeviceWeights, batch: DeviceBatch, Z=None, ws=None):
        import torch
        if Z is None:
            Z = torch.empty((batch.total_T, dims.M, dims.d), dtype=torch.float32, device=batch.X.device)
        if ws is None:
            ws = workspace(forward_workspace_size(dims, batch.c), batch.X.device)
        self.keep = (dims, w, batch)
        self.Z, self.ws = Z, ws
        h = c_void_p()
        _check(LIB.stca_forward_graph_create(_ref(dims), _ref(w.c), _ref(batch.c), _ptr(batch.X), _ptr(batch.xt),
                                             _ptr(Z), _ptr(ws), ws.numel(), ctypes.byref(h)),
               "stca_forward_graph_create")
        self.handle = h

    def launch(self, stream=None):
        _check(LIB.stca_graph_launch(self.handle, _stream(stream)), "stca_graph_launch")
        return self.Z

    def close(self):
        if self.handle:
            LIB.stca_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Profiler:
    """Per-phase HIP-event timing of stca_forward_profiled calls."""

    def __init__(self):
        h = c_void_p()
        _check(LIB.stca_profiler_create(ctypes.byref(h)), "stca_profiler_create")
        self.handle = h

    def reset(self):
        _check(LIB.stca_profiler_reset(self.handle), "stca_profiler_reset")

    def read(self) -> dict:
        rep = ProfileReport()
        _check(LIB.stca_profiler_read(self.handle, _ref(rep)), "stca_profiler_read")
        return {PHASE_NAMES[i]: (rep.ms[i], rep.launches[i]) for i in range(N_PHASES)}

    def close(self):
        if self.handle:
            LIB.stca_profiler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
