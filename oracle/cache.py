"""On-disk cache of oracle results (test infrastructure only, like the rest
of oracle/).

A long float64 reference (full-size sampled rows, the whole-call attention)
can be stored and reused across runs, so an interrupted or repeated test run
resumes instead of recomputing.  The key follows the exact-bytes idea of the
pages' projection cache ([P3] "突破视频生成大模型的工程瓶颈", the exact-key
cache of the time projection): a SHA-256 over the oracle function's name,
the bytes of the oracle's own source files (any change to its arithmetic
gives new keys), and every argument exactly: an array by dtype, shape and
raw bytes, anything else by its repr.  Nothing approximate enters the key,
so a hit returns what the oracle would compute for exactly these inputs.

The cache is off unless H3_ORACLE_CACHE names a directory.  Entries are
.npz files written atomically (temporary file, then rename) and loaded with
allow_pickle=False; an entry that cannot be read is recomputed and
rewritten.  Results may be one array or a tuple / list of arrays."""
from __future__ import annotations

import hashlib
import os
import tempfile
from typing import Any, Callable, Optional

import numpy as np

_SRC_DIR = os.path.dirname(os.path.abspath(__file__))


def _source_digest() -> bytes:
    h = hashlib.sha256()
    for name in sorted(os.listdir(_SRC_DIR)):
        if name.endswith(".py") and name != "cache.py":
            with open(os.path.join(_SRC_DIR, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.digest()


def _feed(h, x: Any) -> None:
    if isinstance(x, np.ndarray):
        a = np.ascontiguousarray(x)
        h.update(b"A" + a.dtype.str.encode() + repr(a.shape).encode())
        h.update(a.tobytes())
    elif isinstance(x, (list, tuple)) and any(isinstance(e, np.ndarray) for e in x):
        h.update(b"L" + str(len(x)).encode())
        for e in x:
            _feed(h, e)
    else:
        h.update(b"R" + repr(x).encode())


def key(fn: Callable, args: tuple, kwargs: dict, source: Optional[bytes] = None) -> str:
    """The cache key of fn(*args, **kwargs)."""
    h = hashlib.sha256()
    h.update((fn.__module__ + "." + fn.__qualname__).encode())
    h.update(source if source is not None else _source_digest())
    for a in args:
        _feed(h, a)
    for k in sorted(kwargs):
        h.update(b"K" + k.encode())
        _feed(h, kwargs[k])
    return h.hexdigest()


def _save(path: str, result: Any) -> None:
    if isinstance(result, np.ndarray):
        parts, kind = [result], "array"
    elif isinstance(result, (tuple, list)) and all(isinstance(e, np.ndarray) for e in result):
        parts, kind = list(result), type(result).__name__
    else:
        return                                   # not cacheable: keep the result, store nothing
    fd, tmp = tempfile.mkstemp(dir=os.path.dirname(path), suffix=".tmp")
    os.close(fd)
    with open(tmp, "wb") as f:
        np.savez(f, __kind__=np.array(kind), **{"r%d" % i: p for i, p in enumerate(parts)})
    os.replace(tmp, path)


def _load(path: str) -> Any:
    with np.load(path, allow_pickle=False) as z:
        kind = str(z["__kind__"])
        parts = [z["r%d" % i] for i in range(len(z.files) - 1)]
    if kind == "array":
        return parts[0]
    return tuple(parts) if kind == "tuple" else parts


def cached(fn: Callable, *args, **kwargs):
    """fn(*args, **kwargs), from the cache directory when an entry exists."""
    d = os.environ.get("H3_ORACLE_CACHE")
    if not d:
        return fn(*args, **kwargs)
    os.makedirs(d, exist_ok=True)
    path = os.path.join(d, key(fn, args, kwargs) + ".npz")
    if os.path.exists(path):
        try:
            return _load(path)
        except Exception:                        # unreadable entry: recompute and rewrite
            pass
    result = fn(*args, **kwargs)
    _save(path, result)
    return result
