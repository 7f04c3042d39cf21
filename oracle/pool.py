"""Process pool that runs the fp64 oracle over independent work units.

TEST INFRASTRUCTURE ONLY.  Only tests/ and bench.py's cpu_baseline leg use this module;
the GPU product path never does.  It adds no arithmetic of its own: every unit calls
``attention_rows`` or ``attention_decode`` from ``oracle.attention`` unchanged.

Work units are independent: one (batch, head) of a prefill workload, or one (sequence,
KV head) of a decode workload.  Each worker process runs numpy with one BLAS thread, and
as many workers run as this process may use cores (at most 16).

Two kinds of job:

* ``check_prefill_heads``: whole-output parity of a prefill workload.  A worker
  regenerates its head's Q, K, V from the seeded per-head streams of ``attn_inputs`` (no
  tensor is shipped to it), takes the GPU's output rows of that head, and compares them
  with the oracle over row blocks of 1,024 queries.  Under causal masking a block of rows
  [i0, i1) is evaluated against keys [0, i1 + Nk - Nq) only: every later key is masked
  for all of its rows (weight exactly 0), so the result is the definition itself.
* ``time_prefill`` / ``time_decode``: the oracle as it stands, over inputs placed in
  shared memory beforehand, timed as wall-clock time of the whole pool.

Call ``start()`` before the calling process initialises the GPU.  The workers are forked
from a server process started there, which never touches the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import shared_memory

import numpy as np

_CTX = None
_LIMITS = None          # worker-side threadpoolctl handle (kept alive)
_ATTACHED = {}          # worker-side shared-memory attachments by name


def start() -> None:
    """Start the fork server the workers come from (idempotent)."""
    global _CTX
    if _CTX is None:
        _CTX = mp.get_context("forkserver")
        _CTX.set_forkserver_preload([])
        from multiprocessing import forkserver
        forkserver.ensure_running()


def n_workers() -> int:
    """Cores this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init_worker() -> None:
    global _LIMITS
    try:
        from threadpoolctl import threadpool_limits
        _LIMITS = threadpool_limits(1)
    except Exception:  # pragma: no cover - threadpoolctl is installed here
        _LIMITS = None


def executor(workers: int | None = None) -> ProcessPoolExecutor:
    start()
    return ProcessPoolExecutor(max_workers=workers or n_workers(), mp_context=_CTX,
                               initializer=_init_worker)


# ---------------------------------------------------------------------------------- parity
def _prefill_head_errors(cfg_name: str, b: int, h: int, o_bits: np.ndarray,
                         lse: np.ndarray, row_block: int = 1024) -> dict:
    """Errors of one head's GPU output (bf16 bits [Nq, d], fp32 LSE [Nq]) against the
    oracle."""
    import attn_inputs as ai
    from oracle.attention import attention_rows

    cfg = ai.CONFIGS[cfg_name]
    kvh = h // (cfg.Hq // cfg.Hkv)
    Q = ai.bits_to_f64(ai.prefill_head(cfg, ai.T_Q, b, h), cfg.f16)
    K = ai.bits_to_f64(ai.prefill_head(cfg, ai.T_K, b, kvh), cfg.f16)
    V = ai.bits_to_f64(ai.prefill_head(cfg, ai.T_V, b, kvh), cfg.f16)
    go = ai.bits_to_f64(o_bits, cfg.f16)
    gl = lse.astype(np.float64)
    off = cfg.Nk - cfg.Nq
    worst = (0.0, -1, -1)
    sum_abs, lse_max, n = 0.0, 0.0, 0
    finite = bool(np.isfinite(go).all())
    for i0 in range(0, cfg.Nq, row_block):
        i1 = min(cfg.Nq, i0 + row_block)
        rows = np.arange(i0, i1)
        if cfg.causal:
            nk = i1 + off
            ro, rl = attention_rows(Q[i0:i1], K[:nk], V[:nk], cfg.scale, True, rows, i1)
        else:
            ro, rl = attention_rows(Q[i0:i1], K, V, cfg.scale, False, rows, cfg.Nq)
        err = np.abs(go[i0:i1] - ro)
        r, c = np.unravel_index(int(np.argmax(err)), err.shape)
        if err[r, c] > worst[0]:
            worst = (float(err[r, c]), int(i0 + r), int(c))
        sum_abs += float(err.sum())
        n += err.size
        lse_max = max(lse_max, float(np.abs(gl[i0:i1] - rl).max()))
    return {"b": b, "h": h, "n": n, "sum_abs": sum_abs, "max_abs": worst[0],
            "max_at": worst[1:], "lse_max_abs": lse_max, "finite": finite}


def check_prefill_heads(cfg_name: str, o_bits: np.ndarray, lse: np.ndarray,
                        heads=None, progress=None) -> dict:
    """Whole-output comparison of a prefill workload's GPU result (O as bf16/fp16 bits
    [B, Hq, Nq, d], LSE fp32 [B, Hq, Nq]) with the oracle, over the listed (b, h) heads
    (default: every head).  Returns the totals and the per-head results."""
    import attn_inputs as ai
    cfg = ai.CONFIGS[cfg_name]
    if heads is None:
        heads = [(b, h) for b in range(cfg.B) for h in range(cfg.Hq)]
    per = []
    with executor() as ex:
        futs = [ex.submit(_prefill_head_errors, cfg_name, b, h,
                          np.ascontiguousarray(o_bits[b, h]), np.ascontiguousarray(lse[b, h]))
                for b, h in heads]
        for i, f in enumerate(futs):
            per.append(f.result())
            if progress and ((i + 1) % 8 == 0 or i + 1 == len(futs)):
                progress(f"{cfg_name}: {i + 1}/{len(futs)} heads compared")
    n = sum(r["n"] for r in per)
    worst = max(per, key=lambda r: r["max_abs"])
    return {"n": n, "max_abs": worst["max_abs"],
            "max_at": (worst["b"], worst["h"], *worst["max_at"]),
            "mean_abs": sum(r["sum_abs"] for r in per) / n,
            "lse_max_abs": max(r["lse_max_abs"] for r in per),
            "finite": all(r["finite"] for r in per), "heads": per}


# ---------------------------------------------------------------------------- CPU baseline
class SharedArrays:
    """Copies numpy arrays into named shared-memory blocks for the workers; a context
    manager that unlinks them on exit."""

    def __init__(self, **arrays):
        self.desc, self._shm = {}, []
        for key, a in arrays.items():
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            np.ndarray(a.shape, a.dtype, buffer=shm.buf)[...] = a
            self._shm.append(shm)
            self.desc[key] = (shm.name, a.shape, a.dtype.str)

    def __enter__(self):
        return self.desc

    def __exit__(self, *exc):
        for shm in self._shm:
            shm.close()
            shm.unlink()


def _view(desc):
    name, shape, dt = desc
    shm = _ATTACHED.get(name)
    if shm is None:
        # (workers share the creating process's resource tracker, which unlinks the
        # block once, when the creator does)
        shm = shared_memory.SharedMemory(name=name)
        _ATTACHED[name] = shm
    return np.ndarray(shape, np.dtype(dt), buffer=shm.buf)


def _noop(_):
    return os.getpid()


def _warm(ex, workers):
    # start every worker (and attach nothing) before the timed region
    list(ex.map(_noop, range(4 * workers)))


def _prefill_unit(desc, b, h, kvh, i0, i1, scale, causal, Nq):
    import attn_inputs as ai
    from oracle.attention import attention_rows
    q = _view(desc["q"])
    k = _view(desc["k"])
    v = _view(desc["v"])
    up = ai.bf16_bits_to_f64
    rows = np.arange(i0, i1)
    attention_rows(up(q[b, h, i0:i1]), up(k[b, kvh]), up(v[b, kvh]), scale, causal, rows, Nq)
    return 0


def time_prefill(q, k, v, scale: float, causal: bool, units, row_block: int = 1024) -> dict:
    """Wall-clock time of the oracle (attention_rows over blocks of row_block queries, all
    keys, the three passes as written) on the given (b, h) heads of bf16-bit tensors
    q [B, Hq, Nq, d], k, v [B, Hkv, Nk, d].  Inputs are upcast to fp64 inside each unit."""
    B, Hq, Nq, d = q.shape
    G = Hq // k.shape[1]
    workers = n_workers()
    tasks = [(b, h, h // G, i0, min(Nq, i0 + row_block)) for b, h in units
             for i0 in range(0, Nq, row_block)]
    with SharedArrays(q=q, k=k, v=v) as desc, executor(workers) as ex:
        _warm(ex, workers)
        t0 = time.perf_counter()
        list(ex.map(_prefill_unit, *zip(*[(desc, *t, scale, causal, Nq) for t in tasks])))
        wall = time.perf_counter() - t0
    return {"seconds": wall, "workers": workers, "units": len(tasks)}


def _decode_unit(desc, b, kvh, n, G, scale):
    import attn_inputs as ai
    from oracle.attention import attention_decode
    q = _view(desc["q"])
    kp = _view(desc["k"])
    vp = _view(desc["v"])
    table = _view(desc["table"])
    up = ai.bf16_bits_to_f64
    # this sequence's pages, as a pool of its own with one KV head, and its table remapped
    npg = (n + 15) // 16
    pages = table[b, :npg]
    kk = up(kp[pages, kvh:kvh + 1])
    vv = up(vp[pages, kvh:kvh + 1])
    attention_decode(up(q[b:b + 1, kvh * G:(kvh + 1) * G]), kk, vv,
                     np.array([n], np.int32), scale,
                     np.arange(npg, dtype=np.int32)[None], 16)
    return 0


def time_decode(q, kpool, vpool, table, lens, scale: float, units) -> dict:
    """Wall-clock time of the oracle's paged decode on the given (b, kvh) units of a bf16
    paged cache (pool [P, Hkv, 16, d], table [B, max_blocks])."""
    G = q.shape[1] // kpool.shape[1]
    workers = n_workers()
    with SharedArrays(q=q, k=kpool, v=vpool, table=table) as desc, executor(workers) as ex:
        _warm(ex, workers)
        t0 = time.perf_counter()
        list(ex.map(_decode_unit, *zip(*[(desc, b, kvh, int(lens[b]), G, scale)
                                          for b, kvh in units])))
        wall = time.perf_counter() - t0
    return {"seconds": wall, "workers": workers, "units": len(units)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


__all__ = ["start", "n_workers", "executor", "check_prefill_heads", "SharedArrays",
           "time_prefill", "time_decode", "cpu_model"]
