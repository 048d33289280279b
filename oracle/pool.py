"""Run the oracle over shards of sequences in worker processes.

Test infrastructure only (tests/, the smoke check, the benchmark's CPU
baseline).  Workers are spawned fresh interpreters that import numpy and
this package only; the inputs reach them as memory-mapped .npy files.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

from . import ssd as O

_G = {}


def default_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init(paths):
    _G.clear()
    for k, p in paths.items():
        _G[k] = np.load(p, mmap_mode="r")


def _task(a):
    paths, b0, b1, dtype, T, F, C, seed, F_out, blk, do_draft, do_verify = a
    if paths is not None:
        _init(paths)
    out = {}
    zd = O.decode(np.asarray(_G["draft"][b0:b1]), dtype)
    if do_draft:
        out["draft"] = O.draft_sample(zd, T[b0:b1], F, C, seed, F_out, blk, b0=b0)
    if do_verify:
        zt = O.decode(np.asarray(_G["target"][b0:b1]), dtype)
        toks = np.asarray(_G["tokens"][b0:b1]) if "tokens" in _G else out["draft"]["tokens"]
        out["verify"] = O.verify(zt, zd, T[b0:b1], F, C, seed, toks, blk, b0=b0)
    return b0, out


def _merge(parts, key):
    ds = [p[key] for _, p in sorted(parts, key=lambda t: t[0])]
    return {k: np.concatenate([d[k] for d in ds], axis=0) for k in ds[0]}


class Pool:
    """Worker processes kept across several run() calls (pass as `pool=`),
    so a long parity test spawns them once."""

    def __init__(self, workers=None):
        self.workers = workers or default_workers()
        self.ex = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"))

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.ex.shutdown(wait=True, cancel_futures=True)


def _tmpdir():
    # memory-backed when available: the inputs are written once per call
    base = "/dev/shm" if os.path.isdir("/dev/shm") and os.access("/dev/shm", os.W_OK) else None
    return tempfile.mkdtemp(prefix="ssd_oracle_", dir=base)


def run(draft_raw, dtype, T, F, C, seed, F_out=None, target_raw=None, tokens=None, draft=True,
        verify=True, workers=None, blk=O.BLK, shard=None, pool=None):
    """Oracle draft sampling and/or verification of a batch.

    draft_raw / target_raw: [B, K+1, V] raw stored logits (uint16 bit
    patterns for bf16/fp16, float32 for f32).  tokens: optional [B, K] drafted
    tokens to verify (default: the oracle's own draft).  pool: a Pool whose
    workers run the shards (else workers are spawned for this call).  Returns
    dict(draft=..., verify=...) with the oracle's per-batch outputs.
    """
    B = draft_raw.shape[0]
    workers = pool.workers if pool is not None else (workers or default_workers())
    shard = shard or max(1, -(-B // (workers * 2)))
    T = np.asarray(T, dtype=np.float64)
    tmp = _tmpdir()
    try:
        paths = {"draft": os.path.join(tmp, "draft.npy")}
        np.save(paths["draft"], np.ascontiguousarray(draft_raw))
        if target_raw is not None:
            paths["target"] = os.path.join(tmp, "target.npy")
            np.save(paths["target"], np.ascontiguousarray(target_raw))
        if tokens is not None:
            paths["tokens"] = os.path.join(tmp, "tokens.npy")
            np.save(paths["tokens"], np.ascontiguousarray(tokens))
        tasks = [(None, b0, min(B, b0 + shard), dtype, T, F, C, seed, F_out, blk, draft, verify)
                 for b0 in range(0, B, shard)]
        if pool is not None:
            parts = list(pool.ex.map(_task, [(paths,) + t[1:] for t in tasks]))
        elif workers == 1 or len(tasks) == 1:
            _init(paths)
            parts = [_task(t) for t in tasks]
            _G.clear()
        else:
            # a worker that dies raises BrokenProcessPool instead of being respawned
            with cf.ProcessPoolExecutor(min(workers, len(tasks)), mp_context=mp.get_context("spawn"),
                                        initializer=_init, initargs=(paths,)) as ex:
                parts = list(ex.map(_task, tasks))
        out = {}
        if draft:
            out["draft"] = _merge(parts, "draft")
        if verify:
            out["verify"] = _merge(parts, "verify")
        return out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
