"""The oracle result cache (oracle/cache.py): a hit returns exactly what the
oracle computes; any change to an input's bytes, dtype or shape, to a
keyword argument, or to the oracle's source gives a new key; unreadable
entries are recomputed; with no cache directory nothing is stored."""
import os

import numpy as np
import pytest

import oracle
from oracle import cache


def _inputs(seed=0, rows=(37, 21), H=2, D=16):
    rng = np.random.default_rng(seed)
    n = sum(rows)
    q, k, v = (rng.standard_normal((n, H, D)) for _ in range(3))
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    return q, k, v, cu


def test_hit_returns_the_oracle_result_without_recomputing(tmp_path, monkeypatch):
    monkeypatch.setenv("H3_ORACLE_CACHE", str(tmp_path))
    calls = []

    def counted(*a, **kw):
        calls.append(1)
        return oracle.attention(*a, **kw)
    counted.__qualname__ = "counted_attention"

    q, k, v, cu = _inputs()
    first = cache.cached(counted, q, k, v, cu)
    second = cache.cached(counted, q, k, v, cu)
    assert len(calls) == 1 and len(os.listdir(tmp_path)) == 1
    assert np.array_equal(first, second) and first.dtype == second.dtype
    assert np.array_equal(first, oracle.attention(q, k, v, cu))


def test_tuple_and_list_results_round_trip(tmp_path, monkeypatch):
    monkeypatch.setenv("H3_ORACLE_CACHE", str(tmp_path))
    q, k, v, cu = _inputs(1)
    sel = np.array([[[0, -1], [1, 0]]] * 2, np.int32)       # [H][blocks][topk]
    got = cache.cached(oracle.vsa_attention_blocks, q, k, v, cu, sel, [0, 1])
    again = cache.cached(oracle.vsa_attention_blocks, q, k, v, cu, sel, [0, 1])
    assert isinstance(again, list) and len(again) == len(got) == 2
    assert all(np.array_equal(a, b) for a, b in zip(got, again))
    pk = cache.cached(oracle.pack, np.array([0, 0, 1, 1, 1], np.int32), 2)
    pk2 = cache.cached(oracle.pack, np.array([0, 0, 1, 1, 1], np.int32), 2)
    assert isinstance(pk2, tuple) and all(np.array_equal(a, b) for a, b in zip(pk, pk2))


def test_key_tracks_bytes_dtype_shape_kwargs_and_source():
    q, k, v, cu = _inputs()
    base = cache.key(oracle.attention, (q, k, v, cu), {})
    q2 = q.copy()
    q2.flat[5] = np.nextafter(q2.flat[5], np.inf)              # one ulp in one element
    assert cache.key(oracle.attention, (q2, k, v, cu), {}) != base
    assert cache.key(oracle.attention, (q.astype(np.float32), k, v, cu), {}) != base
    assert cache.key(oracle.attention, (q.reshape(q.shape[0], -1, 8), k, v, cu), {}) != base
    assert cache.key(oracle.attention, (q, k, v, cu), {"softmax_scale": 0.3}) != base
    assert cache.key(oracle.attention, (q, k, v, cu), {}, source=b"edited oracle") != base
    assert cache.key(oracle.attention, (q, k, v, cu), {}) == base             # deterministic


def test_unreadable_entry_is_recomputed(tmp_path, monkeypatch):
    monkeypatch.setenv("H3_ORACLE_CACHE", str(tmp_path))
    q, k, v, cu = _inputs(2)
    cache.cached(oracle.attention, q, k, v, cu)
    (entry,) = list(tmp_path.iterdir())
    entry.write_bytes(entry.read_bytes()[:40])                 # truncated
    again = cache.cached(oracle.attention, q, k, v, cu)
    assert np.array_equal(again, oracle.attention(q, k, v, cu))
    assert np.array_equal(cache.cached(oracle.attention, q, k, v, cu), again)   # rewritten entry reads back


def test_off_without_a_directory(monkeypatch):
    monkeypatch.delenv("H3_ORACLE_CACHE", raising=False)
    q, k, v, cu = _inputs(3)
    assert np.array_equal(cache.cached(oracle.attention, q, k, v, cu), oracle.attention(q, k, v, cu))
