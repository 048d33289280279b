"""The C-ABI library: it loads, exports every entry point include/ssd.h
declares, rejects invalid arguments on the host before any launch, and its
host-only fan-out matches the oracle bit for bit.  No GPU needed."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def L():
    import lossless_verify_sample_amd as ssd
    if not os.path.exists(ssd.LIB_PATH):
        from lossless_verify_sample_amd import build
        build.build(verbose=False)
    ssd.library()  # loads libssd after the HIP runtime that torch brings
    return ctypes.CDLL(ssd.LIB_PATH)  # own function objects: argtypes set here stay here


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert {"ssd_softmax_t", "ssd_topf", "ssd_saguaro_sample", "ssd_verify", "ssd_cache_lookup",
            "ssd_cache_keys", "ssd_fanout", "ssd_workspace_bytes", "ssd_status_string"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    L.ssd_status_string.restype = ctypes.c_char_p
    assert L.ssd_status_string(0) == b"SSD_OK"
    assert L.ssd_status_string(1) == b"SSD_ERR_INVALID_ARG"
    assert L.ssd_status_string(3) == b"SSD_ERR_WORKSPACE"


def test_workspace_sizes(L):
    import lossless_verify_sample_amd as ssd
    a = ssd.workspace_bytes(ssd.OP_SAMPLE, 64, 7, 151936)
    b = ssd.workspace_bytes(ssd.OP_VERIFY, 64, 7, 151936)
    part = 64 * 8 * 75 * 8              # one (max, sum) float pair per 2048-token block and row
    assert a >= part and b >= part + 64 * 75 * 4
    assert ssd.workspace_bytes(ssd.OP_SAMPLE, 0, 7, 100) == 0
    assert ssd.workspace_bytes(ssd.OP_SOFTMAX_T, 4, 0, (1 << 20) + 1) == 0


def test_fanout_matches_oracle_bit_exact(L):
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    rng = np.random.default_rng(0)
    cases = [(64, 5, 0.6, 128256), (10, 3, 1.0, 100), (6, 2, 0.5, 2), (7, 0, 0.5, 100), (64, 7, 0.6, 151936)]
    for _ in range(300):
        K = int(rng.integers(0, 12))
        V = int(rng.integers(1, 40))
        Bgt = int(rng.integers(0, (K + 1) * V + 1))
        ratio = float(rng.choice([0.5, 0.6, 0.9, 1.0, 1.3, rng.random() * 2 + 1e-3]))
        cases.append((Bgt, K, ratio, V))
    for Bgt, K, ratio, V in cases:
        assert ssd.fanout(Bgt, K, ratio, V) == O.fanout(Bgt, K, ratio, V), (Bgt, K, ratio, V)


def test_fanout_rejects_bad_arguments(L):
    import lossless_verify_sample_amd as ssd
    for args in ((-1, 3, 0.5, 10), (10, -1, 0.5, 10), (10, 3, 0.0, 10), (10, 3, float("nan"), 10),
                 (100, 3, 0.5, 10), (10, 33, 0.5, 10)):
        with pytest.raises(ssd.SSDError):
            ssd.fanout(*args)


def test_entry_points_reject_invalid_arguments_on_host(L):
    """Each call returns SSD_ERR_INVALID_ARG (1) or SSD_ERR_WORKSPACE (3) before
    touching the GPU; fake non-null pointers are never dereferenced."""
    P = ctypes.c_void_p(16)
    N = None
    s = L.ssd_softmax_t
    s.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert s(N, 1, 4, 100, 100, P, P, N, P, 1 << 20, N) == 1          # null logits
    assert s(P, 7, 4, 100, 100, P, P, N, P, 1 << 20, N) == 1          # bad dtype
    assert s(P, 1, 4, 100, 99, P, P, N, P, 1 << 20, N) == 1           # ld < V
    assert s(P, 1, 4, (1 << 20) + 1, 1 << 21, P, P, N, P, 1 << 30, N) == 1  # V too large
    assert s(P, 1, 4, 100, 100, P, P, N, N, 1 << 20, N) == 3          # no workspace
    assert s(P, 1, 4, 100, 100, P, P, N, ctypes.c_void_p(256), 8, N) == 3  # too small
    assert s(P, 1, 4, 100, 100, P, P, N, ctypes.c_void_p(24), 1 << 20, N) == 3  # misaligned
    t = L.ssd_topf
    t.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert t(P, 1, 4, 100, 100, 0, P, N, P, 1 << 20, N) == 1          # F = 0
    assert t(P, 1, 4, 100, 100, 65, P, N, P, 1 << 20, N) == 1         # F > 64
    assert t(P, 1, 4, 10, 10, 11, P, N, P, 1 << 20, N) == 1           # F > V
    smp = L.ssd_saguaro_sample
    smp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                    ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_uint64,
                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    ok = dict(B=2, K=3, V=100, ld=100, F=2, C=0.5, Fo=2, cache=None)

    def call(**kw):
        a = dict(ok, **kw)
        return smp(P, 1, a["B"], a["K"], a["V"], a["ld"], P, a["F"], a["C"], a["Fo"], 0, P, P, P, P, P,
                   a["cache"], P, 1 << 24, N)

    assert call(C=0.0) == 1 and call(C=1.5) == 1 and call(C=float("nan")) == 1
    assert call(B=0) == 1 and call(K=-1) == 1 and call(K=33) == 1
    assert call(Fo=1) == 1            # F_out < F
    assert call(F=65, Fo=65) == 1
    import lossless_verify_sample_amd as ssd

    def cache(fan, keys=P):
        arr = (ctypes.c_int32 * len(fan))(*fan)
        st = ssd._CacheStruct(ctypes.cast(arr, ctypes.c_void_p), keys, P, P, P, P)
        st._keep = arr
        return st
    assert call(cache=ctypes.byref(cache([1, 2, 65, 1]))) == 1    # F_k > SSD_MAX_F
    assert call(cache=ctypes.byref(cache([1, -1, 2, 1]))) == 1    # negative F_k
    assert call(V=10, ld=10, cache=ctypes.byref(cache([11, 1, 1, 1]))) == 1  # F_k > V
    assert call(cache=ctypes.byref(cache([1, 2, 3, 1], keys=None))) == 1     # no keys
    v = L.ssd_verify
    v.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 1, P, P, P, N, N, P, 1 << 24, N) == 1  # ld_topf < F
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, N, P, 2, P, P, P, N, N, P, 1 << 24, N) == 1  # no stats
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, N, P, P, 2, P, P, P, N, N, P, 1 << 24, N) == 1  # no q
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, N, N, P, 16, N) == 3       # small ws
    c = cache([1, 2, 3, 1])
    c.payload = None
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, N, ctypes.byref(c), P, 1 << 24,
             N) == 1  # cache without payload
    c = cache([1, 2, 3, 1])
    c.out_tokens = None
    assert v(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, N, ctypes.byref(c), P, 1 << 24,
             N) == 1  # cache without token outputs
    te = L.ssd_timer_enable
    te.argtypes = [ctypes.c_int32]
    assert te(-1) == 1 and te((1 << 20) + 1) == 1
    tr = L.ssd_timer_read
    tr.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert tr(9, P, P) == 1 and tr(2, N, P) == 1
    lk = L.ssd_cache_lookup
    lk.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5
                   + [ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p])
    assert lk(P, N, P, 4, 3, 8, P, P, P, P, P, 0, 0, 0, N) == 1   # no depth offsets
    assert lk(P, P, P, 0, 3, 8, P, P, P, P, P, 0, 0, 0, N) == 1   # B = 0
    assert lk(P, P, P, 4, 3, 8, P, P, P, P, P, 2, 100, 0, N) == 1  # miss_fill not 0/1
    assert lk(P, P, P, 4, 3, 8, P, P, P, P, P, 1, 0, 0, N) == 1    # fill without a vocabulary


def test_backoff_matches_oracle(L):
    """The host back-off rule against the oracle's, on random hit rates,
    batch sizes and costs: the same decision, the same gain to 1e-12."""
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    rng = np.random.default_rng(11)
    for _ in range(300):
        B = int(rng.integers(1, 600))
        p = rng.uniform(0.3, 1.0, B) if rng.random() < 0.7 else np.full(B, rng.uniform(0.5, 1.0))
        c = dict(t_round=rng.uniform(0.5, 2.0), t_slow=rng.uniform(0.0, 3.0), t_fast=rng.uniform(0.0, 0.2),
                 e_acc=rng.uniform(1.0, 5.0), e_fast=rng.uniform(0.5, 1.5))
        got = ssd.backoff(p, **c)
        want = O.backoff(p, **c)
        assert got[0] == want[0] and abs(got[1] - want[1]) <= 1e-12 * want[1], (B, c)


def test_backoff_rejects_bad_arguments(L):
    import lossless_verify_sample_amd as ssd
    ok = dict(t_round=1.0, t_slow=1.0, t_fast=0.0, e_acc=2.0, e_fast=1.0)
    for p, kw in (([], {}), ([1.5], {}), ([-0.1], {}), ([float("nan")], {}), ([0.5], {"t_round": 0.0}),
                  ([0.5], {"t_slow": -1.0}), ([0.5], {"e_acc": 0.0}), ([0.5], {"e_fast": float("inf")})):
        with pytest.raises(ssd.SSDError):
            ssd.backoff(p, **dict(ok, **kw))


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of ssd_cache, ssd_sample_args, ssd_verify_args and
    ssd_backoff_cost have the C sizes and field offsets (compiled with gcc)."""
    import shutil
    import subprocess
    import lossless_verify_sample_amd as ssd
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("no C compiler")
    mirrors = {"ssd_cache": ssd._CacheStruct, "ssd_sample_args": ssd._SampleArgs,
               "ssd_verify_args": ssd._VerifyArgs, "ssd_backoff_cost": ssd._BackoffCost}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssd.h"', "int main(void) {"]
    for cname, py in mirrors.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        name, field, val = line.split()
        got[(name, field)] = int(val)
    for cname, py in mirrors.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_round_rejects_bad_arguments(L):
    import lossless_verify_sample_amd as ssd
    P = ctypes.c_void_p(1 << 20)
    r = L.ssd_round
    r.argtypes = [ctypes.c_void_p] * 3
    assert r(None, None, None) == 1  # neither call
    ws = ctypes.c_void_p(1 << 24)
    v = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, None, None, ws, 1 << 24)
    s = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 0.5, 2, 0, P, P, P, P, P, None, ws, 1 << 24)
    assert r(ctypes.byref(v), ctypes.byref(s), None) == 3  # one workspace for both
    bad = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 1.5, 2, 0, P, P, P, P, P, None, ws, 1 << 24)
    assert r(None, ctypes.byref(bad), None) == 1  # C > 1
    ws2 = ctypes.c_void_p(1 << 25)
    Q = ctypes.c_void_p(1 << 26)
    s2 = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 0.5, 2, 0, Q, Q, Q, Q, Q, None, ws2, 1 << 24)
    v2 = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, Q, P, P, P, 2, P, P, P, None, None, ws, 1 << 24)
    assert r(ctypes.byref(v2), ctypes.byref(s2), None) == 1  # sampling writes the tokens being verified


def test_fanout_greedy_matches_oracle(L):
    """The host allocation from measured statistics against the oracle's on
    random (also non-concave) curves: identical vectors."""
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    rng = np.random.default_rng(21)
    for _ in range(200):
        K1, Fmax = int(rng.integers(1, 9)), int(rng.integers(1, 40))
        a = rng.dirichlet(np.ones(K1))
        inc = rng.uniform(0, 1, (K1, Fmax))
        if rng.random() < 0.5:
            inc = np.sort(inc, axis=1)[:, ::-1]
        h = np.concatenate([np.zeros((K1, 1)), np.cumsum(inc, axis=1)], axis=1) / Fmax
        Bgt = int(rng.integers(0, K1 * Fmax + 1))
        assert ssd.fanout_greedy(a, h.tolist(), Bgt) == O.fanout_from_stats(a, h.tolist(), Bgt)
    with pytest.raises(ssd.SSDError):
        ssd.fanout_greedy([0.5, 0.5], [[0, 1], [0, 1]], 3)   # budget above (K+1) Fmax
    with pytest.raises(ssd.SSDError):
        ssd.fanout_greedy([0.5, -0.1], [[0, 1], [0, 1]], 1)  # negative probability


def test_verify_early_rejects_bad_arguments(L):
    """ssd_verify_early checks everything ssd_verify checks, plus J in
    [1, K+1] and no row statistics, before any launch."""
    import lossless_verify_sample_amd as ssd
    P = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    f = L.ssd_verify_early
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, 1, None) == 1
    # B = 2, K = 3, V = 100; out_target_stats NULL
    v = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, None, None, ws, 1 << 24)
    for J in (0, -1, 5):
        assert f(ctypes.byref(v), J, None) == 1, J
    with_stats = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, P, None, ws, 1 << 24)
    assert f(ctypes.byref(with_stats), 2, None) == 1
    small_ws = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, None, None, ws, 64)
    assert f(ctypes.byref(small_ws), 2, None) == 3
    bad_c = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 1.5, 0, P, P, P, P, 2, P, P, P, None, None, ws, 1 << 24)
    assert f(ctypes.byref(bad_c), 2, None) == 1


def test_round_noalloc_rejects_before_any_launch(L):
    """ssd_round_noalloc refuses a request larger than its static scratch
    (SSD_ERR_SCRATCH_LIMIT = 5) and bad arguments (SSD_ERR_INVALID_ARG),
    all before touching the GPU; fake non-null pointers are never
    dereferenced.  The workspace fields are ignored."""
    import lossless_verify_sample_amd as ssd
    P = ctypes.c_void_p(1 << 20)
    Q = ctypes.c_void_p(1 << 26)
    r = L.ssd_round_noalloc
    r.argtypes = [ctypes.c_void_p] * 3
    assert r(None, None, None) == 1
    # B = 130, K = 7, V = 2^20: 1040 rows of 512 blocks need 8.3 MiB of partials
    big = ssd._VerifyArgs(P, P, 1, 130, 7, 1 << 20, 1 << 20, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, None, None,
                          None, 0)
    assert r(ctypes.byref(big), None, None) == 5
    bigs = ssd._SampleArgs(P, 1, 130, 7, 1 << 20, 1 << 20, P, 2, 0.5, 2, 0, Q, Q, Q, Q, Q, None, None, 0)
    assert r(None, ctypes.byref(bigs), None) == 5
    bad = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 1.5, 2, 0, Q, Q, Q, Q, Q, None, None, 0)
    assert r(None, ctypes.byref(bad), None) == 1  # C > 1
    v2 = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, Q, P, P, P, 2, P, P, P, None, None, None, 0)
    s2 = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 0.5, 2, 0, Q, Q, Q, Q, Q, None, None, 0)
    assert r(ctypes.byref(v2), ctypes.byref(s2), None) == 1  # sampling writes the tokens being verified
    L.ssd_status_string.restype = ctypes.c_char_p
    assert L.ssd_status_string(5) == b"SSD_ERR_SCRATCH_LIMIT"


def test_verify_tree_rejects_bad_arguments(L):
    """ssd_verify_tree checks the topology, sizes, F, C and the workspace
    before any launch (fake non-null pointers are never dereferenced)."""
    import lossless_verify_sample_amd as ssd
    P = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_void_p(1 << 24)
    f = L.ssd_verify_tree
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, None) == 1

    def args(parent, N=None, F=2, C=0.5, wsb=1 << 24, tokens=P):
        par = (ctypes.c_int32 * len(parent))(*parent)
        a = ssd._TreeArgs(P, P, 1, 2, len(parent) - 1 if N is None else N, 100, 100, ctypes.cast(par, ctypes.c_void_p),
                          P, F, C, 0, tokens, P, P, P, 2, P, P, P, ws, wsb)
        a._keep = par
        return a
    ok = [-1, 0, 0, 1]
    for bad in ([0, 0, 0, 1], [-1, 1, 0, 1], [-1, 0, 3, 1], [-1, -1, 0, 1]):
        assert f(ctypes.byref(args(bad)), None) == 1, bad
    assert f(ctypes.byref(args(ok, C=1.5)), None) == 1
    assert f(ctypes.byref(args(ok, F=65)), None) == 1
    assert f(ctypes.byref(args(ok, tokens=None)), None) == 1
    assert f(ctypes.byref(args([-1] + [0] * 64)), None) == 1  # 65 nodes
    assert f(ctypes.byref(args(ok, wsb=64)), None) == 3
    assert ssd.workspace_bytes(ssd.OP_VERIFY_TREE, 2, 3, 100) > 0
    assert ssd.workspace_bytes(ssd.OP_VERIFY_TREE, 2, 64, 100) == 0


def test_phase_read_is_off_in_the_ordinary_build(L):
    """ssd_phase_read only serves the instrumented build; the ordinary
    library checks its arguments and then reports SSD_ERR_UNSUPPORTED."""
    f = L.ssd_phase_read
    f.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64]
    buf = (ctypes.c_uint64 * 8)()
    assert f(3, buf, 8) == 1
    assert f(0, None, 8) == 1
    assert f(0, buf, -1) == 1
    assert f(0, buf, 8192 * 8 + 1) == 1
    assert f(0, buf, 8) == 2


def test_round_early_rejects_bad_arguments(L):
    """ssd_round_early: no call, J outside [1, K+1] and target statistics are
    refused before any launch (fake pointers are never dereferenced)."""
    import lossless_verify_sample_amd as ssd
    P = ctypes.c_void_p(1 << 20)
    f = L.ssd_round_early
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, None, 2, None) == 1
    ws, ws2 = ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 25)
    Q = ctypes.c_void_p(1 << 26)
    v = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, None, None, ws, 1 << 24)
    s = ssd._SampleArgs(P, 1, 2, 3, 100, 100, P, 2, 0.5, 2, 0, Q, Q, Q, Q, Q, None, ws2, 1 << 24)
    assert f(ctypes.byref(v), ctypes.byref(s), 0, None) == 1  # J < 1
    assert f(ctypes.byref(v), ctypes.byref(s), 5, None) == 1  # J > K + 1
    vs = ssd._VerifyArgs(P, P, 1, 2, 3, 100, 100, P, 2, 0.5, 0, P, P, P, P, 2, P, P, P, P, None, ws, 1 << 24)
    assert f(ctypes.byref(vs), ctypes.byref(s), 2, None) == 1  # target statistics
