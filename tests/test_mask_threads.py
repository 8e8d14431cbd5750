"""A mask shared across host threads: concurrent first requests for the same
cached schedules (plain, split, transposed) must build them once and hand
every thread the same result as a single-threaded call (ctypes releases the
GIL around each library call, so the threads really run concurrently)."""

import threading

import numpy as np

import attention_jvp_causal_attn_amd as aj

SHAPES = [(256, 32), (64, 32)]
SPLITS = [2, 3, 8]


def _snapshot(mask):
    out = []
    for bm, bn in SHAPES:
        s = aj.attn_jvp_mask_schedule(mask, bm, bn)
        out.append({k: np.asarray(v).copy() for k, v in s.items()})
        for S in SPLITS:
            u = aj.attn_jvp_mask_split_schedule(mask, bm, bn, S)
            out.append({k: np.asarray(v).copy() for k, v in u.items()})
    t = aj.attn_jvp_mask_transpose(mask)
    out.append({k: np.asarray(v).copy() for k, v in
                zip(("gq", "rp", "kb", "ke"), aj.attn_jvp_mask_export(t))})
    return out


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert x.keys() == y.keys()
        for k in x:
            assert np.array_equal(x[k], y[k]), k


def test_concurrent_first_use_of_a_shared_mask():
    ref = _snapshot(aj.attn_jvp_mask_tf(21, 1560, 3))
    mask = aj.attn_jvp_mask_tf(21, 1560, 3)          # fresh: nothing cached yet
    n = 8
    start = threading.Barrier(n)
    results, errors = [None] * n, []

    def work(i):
        try:
            start.wait()
            results[i] = _snapshot(mask)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for r in results:
        _same(r, ref)
