"""Python binding of libssd, the gfx950 batched lossless verify-and-resample
library (C ABI in include/ssd.h, which cites the method's sources).

Argument marshalling only: tensors are checked for device, dtype and layout,
their pointers and torch's current HIP stream are passed to the C entry
points, and every step of the path runs in the library's kernels.  PyTorch
supplies device memory and streams.  The library is loaded from this
package's directory; importing fails loudly if it has not been built
(`python -m lossless_verify_sample_amd.build`).
"""
import ctypes
import os

import torch  # provides the process's HIP runtime, which libssd then shares

__all__ = [
    "SSDError", "Cache", "softmax_t", "topf", "saguaro_sample", "verify", "verify_early", "verify_tree", "round_step",
    "cache_keys", "cache_lookup",
    "fanout", "fanout_greedy", "backoff", "workspace_bytes", "stats_fields", "timer_enable", "timer_read", "LIB_PATH",
    "use_library", "phase_read", "read_probe",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssd.so")

F32, BF16, F16 = 0, 1, 2
OP_SOFTMAX_T, OP_TOPF, OP_SAMPLE, OP_VERIFY, OP_VERIFY_TREE = 0, 1, 2, 3, 4
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}

_vp, _i32, _i64, _u64, _f32, _f64, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                           ctypes.c_float, ctypes.c_double, ctypes.c_size_t)


class SSDError(RuntimeError):
    pass


class _CacheStruct(ctypes.Structure):
    _fields_ = [("fanout", _vp), ("keys", _vp), ("payload", _vp), ("out_hit", _vp), ("out_slot", _vp),
                ("out_tokens", _vp), ("miss_fill", ctypes.c_int32)]


class _SampleArgs(ctypes.Structure):  # ssd_sample_args
    _fields_ = [("draft_logits", _vp), ("dt", ctypes.c_int), ("B", _i32), ("K", _i32), ("V", _i64), ("ld", _i64),
                ("temperature", _vp), ("F", _i32), ("C", _f32), ("F_out", _i32), ("seed", _u64),
                ("out_tokens", _vp), ("out_q", _vp), ("out_stats", _vp), ("out_topf_idx", _vp),
                ("out_topf_val", _vp), ("cache", _vp), ("workspace", _vp), ("ws_bytes", _sz)]


class _VerifyArgs(ctypes.Structure):  # ssd_verify_args
    _fields_ = [("target_logits", _vp), ("draft_logits", _vp), ("dt", ctypes.c_int), ("B", _i32), ("K", _i32),
                ("V", _i64), ("ld", _i64), ("temperature", _vp), ("F", _i32), ("C", _f32), ("seed", _u64),
                ("draft_tokens", _vp), ("draft_q", _vp), ("draft_stats", _vp), ("draft_topf_idx", _vp),
                ("ld_topf", _i32), ("out_accept_len", _vp), ("out_bonus", _vp), ("out_p", _vp),
                ("out_target_stats", _vp), ("cache", _vp), ("workspace", _vp), ("ws_bytes", _sz)]


class _TreeArgs(ctypes.Structure):  # ssd_tree_args
    _fields_ = [("target_logits", _vp), ("draft_logits", _vp), ("dt", ctypes.c_int), ("B", _i32), ("N", _i32),
                ("V", _i64), ("ld", _i64), ("parent", _vp), ("temperature", _vp), ("F", _i32), ("C", _f32),
                ("seed", _u64), ("tokens", _vp), ("draft_q", _vp), ("draft_stats", _vp), ("draft_topf_idx", _vp),
                ("ld_topf", _i32), ("out_accept_len", _vp), ("out_last", _vp), ("out_bonus", _vp),
                ("workspace", _vp), ("ws_bytes", _sz)]


class _BackoffCost(ctypes.Structure):
    _fields_ = [("t_round", ctypes.c_double), ("t_slow", ctypes.c_double), ("t_fast", ctypes.c_double),
                ("e_acc", ctypes.c_double), ("e_fast", ctypes.c_double)]


class Cache:
    """Speculation-cache descriptor (ssd_cache): the per-depth fan-out (host
    ints, e.g. from fanout()), the depth-major keys [B, Bgt] that sampling
    writes, and for verification the payload [B, Bgt, K] and the lookup
    outputs hit [B], slot [B], tokens [B, K] (allocated when not given).
    miss_fill: a miss gets random fallback tokens instead of -1."""

    def __init__(self, fanout, B, K, device, payload=None, keys=None, hit=None, slot=None, tokens=None,
                 miss_fill=False):
        self.fanout = [int(f) for f in fanout]
        if len(self.fanout) != K + 1:
            raise SSDError("fanout must have K+1 entries")
        self.Bgt = sum(self.fanout)
        self.B, self.K = B, K
        self._fan = (ctypes.c_int32 * (K + 1))(*self.fanout)
        i32 = dict(dtype=torch.int32, device=device)
        self.keys = keys if keys is not None else torch.empty((B, self.Bgt), **i32)
        self.payload = payload
        self.hit = hit if hit is not None else torch.empty(B, **i32)
        self.slot = slot if slot is not None else torch.empty(B, **i32)
        self.tokens = tokens if tokens is not None else torch.empty((B, K), **i32)
        off = [0]
        for f in self.fanout:
            off.append(off[-1] + f)
        self.depth_off = torch.tensor(off, **i32)
        self.miss_fill = bool(miss_fill)

    def _struct(self, dev, verify):
        _need(self.keys, torch.int32, "cache keys", dev)
        if tuple(self.keys.shape) != (self.B, self.Bgt):
            raise SSDError("cache keys must be [B, Bgt]")
        st = _CacheStruct(ctypes.cast(self._fan, _vp), _p(self.keys))
        if verify:
            if self.K > 0 and self.Bgt > 0:
                _need(self.payload, torch.int32, "cache payload", dev)
                if tuple(self.payload.shape) != (self.B, self.Bgt, self.K):
                    raise SSDError("cache payload must be [B, Bgt, K]")
                st.payload = _p(self.payload)
            for t, n, shp in ((self.hit, "hit", (self.B,)), (self.slot, "slot", (self.B,)),
                              (self.tokens, "tokens", (self.B, self.K))):
                _shaped(t, torch.int32, shp, "cache " + n, dev)
            st.out_hit, st.out_slot, st.out_tokens = _p(self.hit), _p(self.slot), _p(self.tokens)
            st.miss_fill = 1 if self.miss_fill else 0
        return st


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m lossless_verify_sample_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "ssd_softmax_t": [_vp, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp],
        "ssd_topf": [_vp, _i32, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _sz, _vp],
        "ssd_saguaro_sample": [_vp, _i32, _i32, _i32, _i64, _i64, _vp, _i32, _f32, _i32, _u64, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _sz, _vp],
        "ssd_verify": [_vp, _vp, _i32, _i32, _i32, _i64, _i64, _vp, _i32, _f32, _u64, _vp, _vp, _vp, _vp, _i32,
                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
        "ssd_cache_lookup": [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _u64, _vp],
        "ssd_backoff": [_vp, _i32, _vp, _vp, _vp],
        "ssd_round": [_vp, _vp, _vp],
        "ssd_round_noalloc": [_vp, _vp, _vp],
        "ssd_round_early": [_vp, _vp, _i32, _vp],
        "ssd_verify_early": [_vp, _i32, _vp],
        "ssd_verify_tree": [_vp, _vp],
        "ssd_fanout_greedy": [_vp, _vp, _i32, _i32, _i32, _vp],
        "ssd_cache_keys": [_vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp],
        "ssd_fanout": [_i32, _i32, _f64, _i64, _vp],
        "ssd_read_probe": [_vp, _sz, _i32, _vp, _sz, _vp],
        "ssd_phase_read": [_i32, _vp, _i64],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ssd_timer_enable.argtypes = [_i32]
    lib.ssd_timer_enable.restype = ctypes.c_int
    lib.ssd_timer_read.argtypes = [ctypes.c_int, ctypes.POINTER(_i32), ctypes.POINTER(_f64)]
    lib.ssd_timer_read.restype = ctypes.c_int
    lib.ssd_workspace_bytes.argtypes = [ctypes.c_int, _i64, _i32, _i64]
    lib.ssd_workspace_bytes.restype = _sz
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    return lib


def use_library(path):
    """Load libssd from `path` instead of the package's libssd.so (e.g. the
    instrumented libssd_phases.so); only before the library is first used."""
    global LIB_PATH
    if _Lazy.lib is not None:
        raise SSDError("the library is already loaded")
    LIB_PATH = path


class _Lazy:
    """The loaded library, on first use (a missing build raises ImportError)."""
    lib = None

    def __getattr__(self, name):
        if _Lazy.lib is None:
            _Lazy.lib = _load()
        return getattr(_Lazy.lib, name)


_lib = _Lazy()


def library():
    """The ctypes handle of libssd.so (loads it)."""
    _lib.ssd_status_string
    return _Lazy.lib


def _check(st, name):
    if st != 0:
        raise SSDError(f"{name}: {_lib.ssd_status_string(st).decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, dtype, name, dev=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SSDError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise SSDError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise SSDError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise SSDError(f"{name} must be contiguous")


def _shaped(t, dtype, shape, name, dev):
    """A device tensor of `dtype`, contiguous, of exactly `shape` (the
    kernels index it by B, K and the list widths with no bounds of their
    own)."""
    _need(t, dtype, name, dev)
    if tuple(t.shape) != tuple(shape):
        raise SSDError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stats_shaped(t, n, name, dev):
    """ssd_row_stats [n] as a contiguous float64 tensor of 2 n elements."""
    _need(t, torch.float64, name, dev)
    if t.numel() != 2 * n:
        raise SSDError(f"{name} must hold {n} row statistics ({2 * n} float64), got {t.numel()}")


def _rows_ld(x, nd):
    """Row stride of logits with the vocabulary contiguous and rows evenly spaced."""
    if not x.is_cuda or x.dtype not in _DT:
        raise SSDError("logits must be a device tensor of float32, bfloat16 or float16")
    if x.dim() != nd or x.stride(-1) != 1:
        raise SSDError(f"logits must be {nd}-D with a contiguous last dimension")
    ld = x.stride(-2)
    if nd == 3 and x.stride(0) != x.shape[1] * ld:
        raise SSDError("logits rows must be evenly spaced")
    return ld


def read_probe(buf, variant=0, out=None):
    """Streaming-read probe (ssd_read_probe): one read of the device tensor
    `buf` in launch layout `variant`; returns the scratch output tensor."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise SSDError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(nbytes // 16 // 512 + 1024, dtype=torch.int32, device=buf.device)
    _check(_lib.ssd_read_probe(_p(buf), nbytes, int(variant), _p(out), out.numel(), _stream(buf.device)),
           "ssd_read_probe")
    return out


def phase_read(kind, items):
    """Phase stamps of the instrumented build (ssd_phase_read): int64 numpy
    array [items, 8] of 100 MHz ticks."""
    import numpy as np
    out = np.zeros(items * 8, dtype=np.uint64)
    _check(_lib.ssd_phase_read(int(kind), out.ctypes.data_as(_vp), items * 8), "ssd_phase_read")
    return out.astype(np.int64).reshape(items, 8)


def timer_enable(max_launches):
    """Bracket up to max_launches streaming-pass launches per op with HIP
    events on their stream (0 disables)."""
    _check(_lib.ssd_timer_enable(int(max_launches)), "ssd_timer_enable")


def timer_read(op):
    """(launches timed, their total duration in ms) for `op` since enabling."""
    n, t = _i32(0), _f64(0.0)
    _check(_lib.ssd_timer_read(op, ctypes.byref(n), ctypes.byref(t)), "ssd_timer_read")
    return n.value, t.value


def workspace_bytes(op, n, K, V):
    return int(_lib.ssd_workspace_bytes(op, n, K, V))


_WS = {}


def _workspace(op, n, K, V, dev):
    """Workspace cached per (op, shape, device, current stream) and reused
    (its contents do not matter): calls of one op on one stream are ordered
    by that stream, and calls on different streams get different buffers."""
    key = (op, n, K, V, dev, torch.cuda.current_stream(dev).cuda_stream)
    w = _WS.get(key)
    if w is None:
        nb = workspace_bytes(op, n, K, V)
        if nb == 0:
            raise SSDError("invalid sizes for the workspace")
        w = torch.zeros(nb + 256, dtype=torch.uint8, device=dev)
        off = (-w.data_ptr()) % 256
        w = w[off:off + nb]
        _WS[key] = w
    return w


def _stats_tensor(n, dev):
    return torch.empty((n, 2), dtype=torch.float64, device=dev)  # ssd_row_stats, 16 bytes


def stats_fields(st):
    """(lse float64, max float32, argmax int32) views of an ssd_row_stats tensor."""
    flat = st.reshape(-1, 2)
    return flat[:, 0], flat.view(torch.float32)[:, 2], flat.view(torch.int32)[:, 3]


def softmax_t(logits, temperature, probs=False):
    """Row statistics of softmax(z / T) for logits [R, V]; optional dense probs."""
    ld = _rows_ld(logits, 2)
    R, V = logits.shape
    dev = logits.device
    _need(temperature, torch.float32, "temperature", dev)
    if temperature.numel() != R:
        raise SSDError("temperature must have one entry per row")
    st = _stats_tensor(R, dev)
    pr = torch.empty((R, V), dtype=torch.float32, device=dev) if probs else None
    ws = _workspace(OP_SOFTMAX_T, R, 0, V, dev)
    _check(_lib.ssd_softmax_t(_p(logits), _DT[logits.dtype], R, V, ld, _p(temperature), _p(st), _p(pr),
                              _p(ws), ws.numel(), _stream(dev)), "ssd_softmax_t")
    return st, pr


def topf(logits, F):
    """Top-F raw logits per row of [R, V]: (idx int32 [R, F], val float32 [R, F])."""
    ld = _rows_ld(logits, 2)
    R, V = logits.shape
    dev = logits.device
    idx = torch.empty((R, F), dtype=torch.int32, device=dev)
    val = torch.empty((R, F), dtype=torch.float32, device=dev)
    ws = _workspace(OP_TOPF, R, 0, V, dev)
    _check(_lib.ssd_topf(_p(logits), _DT[logits.dtype], R, V, ld, F, _p(idx), _p(val), _p(ws), ws.numel(),
                         _stream(dev)), "ssd_topf")
    return idx, val


def saguaro_sample(draft, temperature, F, C, seed, F_out=None, out=None, cache=None, _defer=None, _ws=True):
    """Draft sampling with sigma_{F,C} over draft logits [B, K+1, V].

    Returns dict(tokens [B,K] int32, q [B,K] f32, stats [B*(K+1), 2] (see
    stats_fields), topf_idx [B,K+1,F_out] int32, topf_val [B,K+1,F_out] f32).
    `out` may pass a dict of preallocated outputs with those keys.  With a
    Cache, row j also writes its top-F_j tokens into cache.keys."""
    ld = _rows_ld(draft, 3)
    B, K1, V = draft.shape
    K = K1 - 1
    dev = draft.device
    F_out = F if F_out is None else F_out
    _need(temperature, torch.float32, "temperature", dev)
    if temperature.numel() != B:
        raise SSDError("temperature must have one entry per sequence")
    if out is None:
        out = dict(tokens=torch.empty((B, K), dtype=torch.int32, device=dev),
                   q=torch.empty((B, K), dtype=torch.float32, device=dev),
                   stats=_stats_tensor(B * K1, dev),
                   topf_idx=torch.empty((B, K1, F_out), dtype=torch.int32, device=dev),
                   topf_val=torch.empty((B, K1, F_out), dtype=torch.float32, device=dev))
    _shaped(out["tokens"], torch.int32, (B, K), "tokens", dev)
    _shaped(out["q"], torch.float32, (B, K), "q", dev)
    _stats_shaped(out["stats"], B * K1, "stats", dev)
    if F_out > 0:
        _shaped(out["topf_idx"], torch.int32, (B, K1, F_out), "topf_idx", dev)
        if out.get("topf_val") is not None:
            _shaped(out["topf_val"], torch.float32, (B, K1, F_out), "topf_val", dev)
    if cache is not None and (cache.B, cache.K) != (B, K):
        raise SSDError("the cache was made for another batch size or K")
    ws = _workspace(OP_SAMPLE, B, K, V, dev) if _ws else None
    cs = cache._struct(dev, False) if cache is not None else None
    args = (_p(draft), _DT[draft.dtype], B, K, V, ld, _p(temperature), F, float(C), F_out, int(seed) & (2 ** 64 - 1),
            _p(out["tokens"]), _p(out["q"]), _p(out["stats"]), _p(out["topf_idx"]), _p(out["topf_val"]),
            ctypes.cast(ctypes.pointer(cs), _vp) if cs is not None else None, _p(ws), ws.numel() if _ws else 0)
    if _defer is not None:
        _defer.extend([cs])
        return out, args
    _check(_lib.ssd_saguaro_sample(*args, _stream(dev)), "ssd_saguaro_sample")
    return out


def verify(target, draft, temperature, F, C, seed, tokens, draft_q, draft_stats, draft_topf_idx, want_stats=False,
           out=None, cache=None, _defer=None, _ws=True):
    """Acceptance test, accepted length and bonus for target/draft [B, K+1, V].

    Returns dict(accept_len [B] int32, bonus [B] int32, p [B,K] f32, stats
    [B*(K+1), 2] or None).  With a Cache, (k*, bonus) is also looked up and
    cache.hit / cache.slot / cache.tokens are written."""
    ld = _rows_ld(target, 3)
    if draft.shape != target.shape or draft.dtype != target.dtype or _rows_ld(draft, 3) != ld:
        raise SSDError("target and draft logits must share shape, dtype and row stride")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    _need(temperature, torch.float32, "temperature", dev)
    if temperature.numel() != B:
        raise SSDError("temperature must have one entry per sequence")
    _shaped(tokens, torch.int32, (B, K), "tokens", dev)
    _shaped(draft_q, torch.float32, (B, K), "draft_q", dev)
    _stats_shaped(draft_stats, B * K1, "draft_stats", dev)
    ldf = 0
    if F > 0:
        _need(draft_topf_idx, torch.int32, "draft_topf_idx", dev)
        if draft_topf_idx.dim() != 3 or tuple(draft_topf_idx.shape[:2]) != (B, K1) or draft_topf_idx.shape[2] < F:
            raise SSDError(f"draft_topf_idx must be [B, K+1, >= F] = [{B}, {K1}, >= {F}], "
                           f"got {tuple(draft_topf_idx.shape)}")
        ldf = draft_topf_idx.shape[-1]
    if out is None:
        out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                   bonus=torch.empty(B, dtype=torch.int32, device=dev),
                   p=torch.empty((B, K), dtype=torch.float32, device=dev),
                   stats=_stats_tensor(B * K1, dev) if want_stats else None)
    _shaped(out["accept_len"], torch.int32, (B,), "accept_len", dev)
    _shaped(out["bonus"], torch.int32, (B,), "bonus", dev)
    _shaped(out["p"], torch.float32, (B, K), "p", dev)
    if out.get("stats") is not None:
        _stats_shaped(out["stats"], B * K1, "stats", dev)
    if cache is not None and (cache.B, cache.K) != (B, K):
        raise SSDError("the cache was made for another batch size or K")
    ws = _workspace(OP_VERIFY, B, K, V, dev) if _ws else None
    cs = cache._struct(dev, True) if cache is not None else None
    args = (_p(target), _p(draft), _DT[target.dtype], B, K, V, ld, _p(temperature), F, float(C),
            int(seed) & (2 ** 64 - 1), _p(tokens), _p(draft_q), _p(draft_stats),
            _p(draft_topf_idx) if F > 0 else None, ldf, _p(out["accept_len"]), _p(out["bonus"]),
            _p(out["p"]), _p(out.get("stats")), ctypes.cast(ctypes.pointer(cs), _vp) if cs is not None else None,
            _p(ws), ws.numel() if _ws else 0)
    if _defer is not None:
        _defer.extend([cs])
        return out, args
    _check(_lib.ssd_verify(*args, _stream(dev)), "ssd_verify")
    return out


def verify_early(target, draft, temperature, F, C, seed, tokens, draft_q, draft_stats, draft_topf_idx, J=None,
                 out=None, cache=None):
    """Verification with early exit (ssd_verify_early): the results of
    verify() on the same arguments, streaming target positions J .. K only
    for sequences without a clear rejection below J (default J = min(2, K+1)).
    out["p"][b, j] is NaN past the accepted length; no row statistics."""
    B, K1, V = target.shape
    J = min(2, K1) if J is None else int(J)
    keep = []
    if out is not None and out.get("stats") is not None:
        raise SSDError("verify_early writes no row statistics")
    o, a = verify(target, draft, temperature, F, C, seed, tokens, draft_q, draft_stats, draft_topf_idx,
                  out=out, cache=cache, _defer=keep)
    va = _VerifyArgs(*a)
    _check(_lib.ssd_verify_early(ctypes.byref(va), J, _stream(target.device)), "ssd_verify_early")
    return o


def verify_tree(target, draft, temperature, F, C, seed, parent, tokens, draft_q, draft_stats, draft_topf_idx,
                out=None):
    """Token-tree verification (ssd_verify_tree) of target/draft rows [B, N+1, V]
    (row n = node n, node 0 the root), parent: host list of N+1 ints
    (parent[0] = -1, parent[m] < m); tokens / draft_q [B, N+1] (node m's
    token and sigma_{parent[m]} of it; column 0 unused); draft_stats of the
    N+1 draft rows, draft_topf_idx [B, N+1, >= F].  Returns dict(accept_len,
    last, bonus), int32 [B] each."""
    ld = _rows_ld(target, 3)
    if draft.shape != target.shape or draft.dtype != target.dtype or _rows_ld(draft, 3) != ld:
        raise SSDError("target and draft logits must share shape, dtype and row stride")
    B, N1, V = target.shape
    dev = target.device
    if len(parent) != N1:
        raise SSDError("parent must have one entry per node (N+1)")
    _need(temperature, torch.float32, "temperature", dev)
    if temperature.numel() != B:
        raise SSDError("temperature must have one entry per sequence")
    _shaped(tokens, torch.int32, (B, N1), "tokens", dev)
    _shaped(draft_q, torch.float32, (B, N1), "draft_q", dev)
    _stats_shaped(draft_stats, B * N1, "draft_stats", dev)
    ldf = 0
    if F > 0:
        _need(draft_topf_idx, torch.int32, "draft_topf_idx", dev)
        if draft_topf_idx.dim() != 3 or tuple(draft_topf_idx.shape[:2]) != (B, N1) or draft_topf_idx.shape[2] < F:
            raise SSDError(f"draft_topf_idx must be [B, N+1, >= F] = [{B}, {N1}, >= {F}]")
        ldf = draft_topf_idx.shape[-1]
    if out is None:
        out = {k: torch.empty(B, dtype=torch.int32, device=dev) for k in ("accept_len", "last", "bonus")}
    for k in ("accept_len", "last", "bonus"):
        _shaped(out[k], torch.int32, (B,), k, dev)
    par = (ctypes.c_int32 * N1)(*[int(x) for x in parent])
    ws = _workspace(OP_VERIFY_TREE, B, N1 - 1, V, dev)
    a = _TreeArgs(_p(target), _p(draft), _DT[target.dtype], B, N1 - 1, V, ld, ctypes.cast(par, _vp), _p(temperature),
                  F, float(C), int(seed) & (2 ** 64 - 1), _p(tokens), _p(draft_q), _p(draft_stats),
                  _p(draft_topf_idx) if F > 0 else None, ldf, _p(out["accept_len"]), _p(out["last"]),
                  _p(out["bonus"]), _p(ws), ws.numel())
    _check(_lib.ssd_verify_tree(ctypes.byref(a), _stream(dev)), "ssd_verify_tree")
    return out


def round_step(verify_args=None, sample_args=None, noalloc=False, early_J=None):
    """One pipeline step (ssd_round): verification of round i and draft
    sampling of round i + 1, each given as a dict of the keyword arguments of
    verify() / saguaro_sample() (with their positional ones under the same
    names).  Results are those of verify(...) then saguaro_sample(...); the
    sampling's outputs must not be the verification's inputs.  With
    noalloc=True the step runs through ssd_round_noalloc on the library's own
    scratch (no workspace is passed; outputs the caller does not give are
    still allocated here).  With early_J the verification exits early
    (ssd_round_early, as verify_early: p is NaN past the accepted length).
    Returns (verify outputs or None, sample outputs or None)."""
    if early_J is not None and noalloc:
        raise SSDError("round_step: early exit runs on a caller workspace only")
    keep = []
    vo = so = None
    vs = ss = None
    if verify_args is not None:
        vo, a = verify(**verify_args, _defer=keep, _ws=not noalloc)
        vs = _VerifyArgs(*a)
    if sample_args is not None:
        so, a = saguaro_sample(**sample_args, _defer=keep, _ws=not noalloc)
        ss = _SampleArgs(*a)
    if vs is None and ss is None:
        raise SSDError("round_step needs a verification or a sampling")
    dev = (verify_args["target"] if verify_args is not None else sample_args["draft"]).device
    va = ctypes.byref(vs) if vs is not None else None
    sa = ctypes.byref(ss) if ss is not None else None
    if early_J is not None:
        _check(_lib.ssd_round_early(va, sa, int(early_J), _stream(dev)), "ssd_round_early")
        return vo, so
    fn, name = (_lib.ssd_round_noalloc, "ssd_round_noalloc") if noalloc else (_lib.ssd_round, "ssd_round")
    _check(fn(va, sa, _stream(dev)), name)
    return vo, so


def cache_keys(topf_idx, depth_off, Bgt):
    """keys [B, Bgt] int32 from per-row top-F lists [B, K+1, ldf] and depth offsets [K+2]."""
    _need(topf_idx, torch.int32, "topf_idx")
    dev = topf_idx.device
    _need(depth_off, torch.int32, "depth_off", dev)
    if topf_idx.dim() != 3:
        raise SSDError("topf_idx must be [B, K+1, ldf]")
    B, K1, ldf = topf_idx.shape
    if depth_off.numel() != K1 + 1:
        raise SSDError("depth_off must have K+2 entries")
    keys = torch.empty((B, Bgt), dtype=torch.int32, device=dev)
    _check(_lib.ssd_cache_keys(_p(topf_idx), ldf, _p(depth_off), B, K1 - 1, Bgt, _p(keys), _stream(dev)),
           "ssd_cache_keys")
    return keys


def cache_lookup(keys, depth_off, payload, accept_len, bonus, miss_fill=False, V=0, seed=0):
    """(hit [B], slot [B], tokens [B, K]) int32 for the realised (accepted length, bonus).
    A miss gets -1 tokens, or with miss_fill K random tokens in [0, V) keyed by seed."""
    _need(keys, torch.int32, "keys")
    dev = keys.device
    for t, n in ((depth_off, "depth_off"), (payload, "payload"), (accept_len, "accept_len"), (bonus, "bonus")):
        _need(t, torch.int32, n, dev)
    if keys.dim() != 2 or payload.dim() != 3:
        raise SSDError("keys must be [B, Bgt] and payload [B, Bgt, K]")
    B, Bgt = keys.shape
    K = payload.shape[2]
    if payload.shape[:2] != (B, Bgt) or depth_off.numel() != K + 2:
        raise SSDError("payload must be [B, Bgt, K] and depth_off [K+2]")
    if accept_len.numel() != B or bonus.numel() != B:
        raise SSDError("accept_len and bonus must have one entry per sequence")
    hit = torch.empty(B, dtype=torch.int32, device=dev)
    slot = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty((B, K), dtype=torch.int32, device=dev)
    _check(_lib.ssd_cache_lookup(_p(keys), _p(depth_off), _p(payload), B, K, Bgt, _p(accept_len), _p(bonus),
                                 _p(hit), _p(slot), _p(toks), 1 if miss_fill else 0, int(V),
                                 int(seed) & (2 ** 64 - 1), _stream(dev)), "ssd_cache_lookup")
    return hit, slot, toks


def fanout_greedy(a, h, Bgt):
    """Fan-out F_0..F_K from measured depth probabilities a [K+1] and hit
    curves h [K+1][Fmax+1] (host computation in libssd)."""
    K1 = len(a)
    Fmax = len(h[0]) - 1
    if any(len(row) != Fmax + 1 for row in h) or len(h) != K1:
        raise SSDError("h must be [K+1][Fmax+1]")
    av = (ctypes.c_double * K1)(*[float(x) for x in a])
    hv = (ctypes.c_double * (K1 * (Fmax + 1)))(*[float(x) for row in h for x in row])
    out = (ctypes.c_int32 * K1)()
    _check(_lib.ssd_fanout_greedy(av, hv, K1 - 1, Fmax, int(Bgt), out), "ssd_fanout_greedy")
    return list(out)


def backoff(p_hit, t_round, t_slow, t_fast, e_acc, e_fast):
    """(use_fast, gain): whether misses should get the fast backup (random
    tokens) rather than the accurate one, and its throughput ratio (host
    computation in libssd)."""
    p = [float(x) for x in p_hit]
    arr = (ctypes.c_double * len(p))(*p)
    c = _BackoffCost(float(t_round), float(t_slow), float(t_fast), float(e_acc), float(e_fast))
    use = ctypes.c_int32(0)
    gain = ctypes.c_double(0.0)
    _check(_lib.ssd_backoff(arr, len(p), ctypes.byref(c), ctypes.byref(use), ctypes.byref(gain)), "ssd_backoff")
    return bool(use.value), gain.value


def fanout(Bgt, K, ratio, V):
    """Per-depth fan-out F_0..F_K under budget Bgt (host computation in libssd)."""
    arr = (ctypes.c_int32 * (K + 1))()
    _check(_lib.ssd_fanout(Bgt, K, float(ratio), V, arr), "ssd_fanout")
    return list(arr)
