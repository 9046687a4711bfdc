"""Host calls from several threads at once (no GPU).

The library's shared host state (the registry of live rings and graphs) is
guarded by one mutex; everything else lives in a ring, and the last error
message is per thread.  Eight threads each create, fill, query, reset and
destroy metadata-only rings of their own, interleaved with calls that fail
argument checks, and compare every report with the oracle's deque ring:
no report and no error message may leak between threads.  ctypes releases
the interpreter lock around each call, so the calls really overlap; the
sanitizer tests run this file against the ThreadSanitizer build too.
"""

import random
import threading

import autoregressive_video_world_amd as wm
from oracle.ring import DequeRing

N_THREADS = 8
ROUNDS = 6


def oracle_append(dq, n):
    written, evicted = [], []
    for _ in range(n):
        f, s, ev = dq.commit()
        written.append((f, s, f))
        evicted.extend(ev)
    return {"written": written, "evicted": evicted}


def worker(tid, start, errors):
    rng = random.Random(1234 + tid)
    L = wm.lib()
    try:
        start.wait()
        for rnd in range(ROUNDS):
            sink, window = rng.randint(0, 2), rng.randint(1, 5)
            chunk = rng.randint(1, 3)
            r = wm.KVRing(1, 4, 2, 64, rng.randint(2, 6), rng.randint(2, 6), sink, window, chunk,
                          meta_only=True)
            dq = DequeRing(sink, window)
            for step in range(40):
                n = rng.randint(1, chunk)
                assert r.append_evict(None, None, n) == [oracle_append(dq, n)], (tid, rnd, step)
                if step % 7 == 3:
                    # a failing call: its message is this thread's, whatever the others do
                    assert L.wm_kvring_reset(None, 0, 0) == 1
                    assert b"NULL" in L.wm_last_error(), (tid, L.wm_last_error())
                    bad_b = 5 + tid
                    assert L.wm_kvring_reset(r._h, bad_b, 0) != 0
                    assert str(bad_b).encode() in L.wm_last_error(), (tid, L.wm_last_error())
                if step % 11 == 5:
                    assert r.view(0)["retained"] == [(f, s, f) for f, s in dq.retained()]
            r.reset(0, t0=100 * tid)
            assert r.view(0) == {"retained": [], "n_committed": 0, "t0": 100 * tid}
            r.close()
    except BaseException as e:  # reported by the main thread
        errors.append((tid, repr(e)))


def test_concurrent_host_calls_on_separate_rings():
    start = threading.Barrier(N_THREADS)
    errors = []
    threads = [threading.Thread(target=worker, args=(t, start, errors)) for t in range(N_THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors


def test_destroyed_handle_is_refused_from_another_thread():
    """A handle destroyed in one thread is no longer live in any other."""
    r = wm.KVRing(1, 2, 2, 64, 2, 2, 1, 2, 1, meta_only=True)
    h = r._h
    t = threading.Thread(target=r.close)
    t.start()
    t.join()
    L = wm.lib()
    assert L.wm_kvring_reset(h, 0, 0) == 3   # WM_E_STATE
    assert b"not live" in L.wm_last_error()
