"""ctypes binding of libwm.so: argument marshalling only.

Every step of the hot path runs inside the HIP library; this module turns
PyTorch tensors into device pointers, the current HIP stream into a handle,
and C status codes into exceptions.  If the library is missing the import of
any entry point fails loudly -- there is no fallback implementation.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# WM_LIB names another build of the same library (e.g. a host-sanitized one).
LIB_PATH = os.environ.get("WM_LIB") or os.path.join(_HERE, "libwm.so")

WM_MAX_CHUNK = 16
WM_MAX_RING = 256
EVICT_SLIDE = 0   # FIFO eviction of the oldest window frame
EVICT_RESET = 1   # appends that would evict fail; the caller starts a new window

STATUS = {0: "WM_OK", 1: "WM_E_ARG", 2: "WM_E_SHAPE", 3: "WM_E_STATE", 4: "WM_E_CAPACITY",
          5: "WM_E_HIP", 6: "WM_E_UNSUPPORTED"}

# Every symbol include/wm.h declares.
EXPORTS = ["wm_kvring_pool_bytes", "wm_kvring_create", "wm_kvring_destroy", "wm_kvring_reset",
           "wm_kvring_view", "wm_rope3d", "wm_rope3d_pair", "wm_chunk_attn", "wm_chunk_attn_layer",
           "wm_chunk_attn_workspace_bytes", "wm_chunk_attn_noalloc",
           "wm_kvring_append_evict", "wm_rollout_step", "wm_rollout_graph_create",
           "wm_rollout_graph_launch", "wm_rollout_graph_destroy", "wm_last_error"]


class WMError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status
        self.name = STATUS.get(status, str(status))


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("frame_h", ctypes.c_int32), ("frame_w", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("max_chunk", ctypes.c_int32), ("rope_theta", ctypes.c_double),
                ("rope_dims", ctypes.c_int32 * 3), ("n_layers", ctypes.c_int32),
                ("n_views", ctypes.c_int32), ("evict_policy", ctypes.c_int32)]


class AppendReport(ctypes.Structure):
    _fields_ = [("n_written", ctypes.c_int32), ("n_evicted", ctypes.c_int32),
                ("frame", ctypes.c_int64 * WM_MAX_CHUNK), ("slot", ctypes.c_int32 * WM_MAX_CHUNK),
                ("t", ctypes.c_int64 * WM_MAX_CHUNK), ("evicted", ctypes.c_int64 * WM_MAX_CHUNK)]


class RingView(ctypes.Structure):
    _fields_ = [("n_retained", ctypes.c_int32), ("frame", ctypes.c_int64 * WM_MAX_RING),
                ("slot", ctypes.c_int32 * WM_MAX_RING), ("t", ctypes.c_int64 * WM_MAX_RING),
                ("n_committed", ctypes.c_int64), ("t0", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded library (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwm.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        L.wm_kvring_pool_bytes.argtypes = [P(Desc)]
        L.wm_kvring_pool_bytes.restype = sz
        L.wm_kvring_create.argtypes = [P(Desc), vp, sz, P(vp)]
        L.wm_kvring_destroy.argtypes = [vp]
        L.wm_kvring_reset.argtypes = [vp, i32, i64]
        L.wm_kvring_view.argtypes = [vp, i32, P(RingView)]
        L.wm_rope3d.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp]
        L.wm_rope3d_pair.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, vp, vp, vp]
        L.wm_chunk_attn.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_float, vp, vp, sz, vp]
        L.wm_chunk_attn_layer.argtypes = [vp, i32, vp, vp, vp, i32, vp, ctypes.c_float, vp, vp, sz, vp]
        L.wm_chunk_attn_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, ctypes.c_float, vp, vp]
        L.wm_chunk_attn_workspace_bytes.argtypes = [vp, i32]
        L.wm_chunk_attn_workspace_bytes.restype = sz
        L.wm_kvring_append_evict.argtypes = [vp, vp, vp, i32, vp, vp, vp]
        L.wm_rollout_step.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.wm_rollout_graph_create.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, P(vp)]
        L.wm_rollout_graph_launch.argtypes = [vp, vp, P(i32), vp]
        L.wm_rollout_graph_destroy.argtypes = [vp]
        L.wm_last_error.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name not in ("wm_kvring_pool_bytes", "wm_chunk_attn_workspace_bytes", "wm_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise WMError(status, lib().wm_last_error().decode())


def _ptr(t, what, dtype=torch.bfloat16, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (what, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (what, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _active(active, batch):
    if active is None:
        return None, None
    arr = (ctypes.c_uint8 * batch)(*[1 if a else 0 for a in active])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def _report_dict(r):
    n, ne = r.n_written, r.n_evicted
    return {"written": list(zip(r.frame[:n], r.slot[:n], r.t[:n])), "evicted": r.evicted[:ne]}


class KVRing:
    """A bounded KV ring for ``batch`` independent rollouts and ``n_layers``
    attention layers that share its frames, slots and positions."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, frame_h, frame_w, n_sink, window,
                 max_chunk, rope_theta=10000.0, rope_dims=(0, 0, 0), device="cuda",
                 meta_only=False, pool=None, n_layers=1, n_views=1, evict_policy=EVICT_SLIDE):
        self.desc = Desc(batch, n_q_heads, n_kv_heads, head_dim, frame_h, frame_w, n_sink, window,
                         max_chunk, rope_theta, (ctypes.c_int32 * 3)(*rope_dims), n_layers, n_views,
                         evict_policy)
        self.n_layers = max(1, n_layers)
        self.n_views = max(1, n_views)
        self.batch, self.hq, self.hkv, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.fh, self.fw, self.ft = frame_h, frame_w, self.n_views * frame_h * frame_w
        self.n_sink, self.window, self.max_chunk = n_sink, window, max_chunk
        self.slots = n_sink + window
        # report buffer reused by every append (no per-call ctypes allocation)
        self._reps = (AppendReport * batch)()
        self._reps_ptr = ctypes.c_void_p(ctypes.addressof(self._reps))
        self.pool_bytes = lib().wm_kvring_pool_bytes(ctypes.byref(self.desc))
        if self.pool_bytes == 0:
            raise WMError(2, "invalid ring descriptor")
        self._h = ctypes.c_void_p()
        if meta_only:
            self.pool = None
            _check(lib().wm_kvring_create(ctypes.byref(self.desc), None, 0, ctypes.byref(self._h)))
        else:
            if pool is None:
                pool = torch.empty(self.pool_bytes, dtype=torch.uint8, device=device)
            self.pool = pool
            _check(lib().wm_kvring_create(ctypes.byref(self.desc), ctypes.c_void_p(pool.data_ptr()),
                                          pool.numel(), ctypes.byref(self._h)))

    # -- pool views (tests and debugging) -----------------------------------
    def _half(self, which, layer):
        n = self.batch * self.slots * self.hkv * self.ft * self.d
        half = (n * 2 + 255) // 256 * 256
        base = layer * 2 * half + which * half
        raw = self.pool[base: base + n * 2]
        return raw.view(torch.bfloat16).view(self.batch, self.slots, self.hkv, self.ft, self.d)

    def pool_k(self, layer=0):
        return self._half(0, layer)

    def pool_v(self, layer=0):
        return self._half(1, layer)

    # -- C calls ---------------------------------------------------------------
    def close(self):
        if self._h:
            _check(lib().wm_kvring_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, b, t0=0):
        _check(lib().wm_kvring_reset(self._h, b, t0))

    def view(self, b):
        v = RingView()
        _check(lib().wm_kvring_view(self._h, b, ctypes.byref(v)))
        n = v.n_retained
        return {"retained": [(v.frame[i], v.slot[i], v.t[i]) for i in range(n)],
                "n_committed": v.n_committed, "t0": v.t0}

    def tokens(self, n_frames, heads):
        return self.batch * n_frames * self.ft * heads * self.d

    def _t_first(self, t_first):
        if t_first is None:
            return None, None
        arr = (ctypes.c_int64 * self.batch)(*t_first)
        return arr, ctypes.cast(arr, ctypes.c_void_p)

    def rope3d(self, x, n_frames, y=None, t_first=None, active=None, stream=None):
        heads = x.shape[-2]
        if y is None:
            y = torch.empty_like(x)
        n = self.tokens(n_frames, heads)
        tf_arr, tf = self._t_first(t_first)
        act_arr, act = _active(active, self.batch)
        _check(lib().wm_rope3d(self._h, _ptr(x, "x", numel=n), _ptr(y, "y", numel=n), heads, n_frames,
                               tf, act, _stream(stream)))
        return y

    def rope3d_pair(self, x, x2, n_frames, y=None, y2=None, t_first=None, active=None, stream=None):
        """rope3d of x and x2 (same frames, e.g. Q and K) in one launch."""
        h1, h2 = x.shape[-2], x2.shape[-2]
        y = torch.empty_like(x) if y is None else y
        y2 = torch.empty_like(x2) if y2 is None else y2
        n1, n2 = self.tokens(n_frames, h1), self.tokens(n_frames, h2)
        tf_arr, tf = self._t_first(t_first)
        act_arr, act = _active(active, self.batch)
        _check(lib().wm_rope3d_pair(self._h, _ptr(x, "x", numel=n1), _ptr(y, "y", numel=n1), h1,
                                    _ptr(x2, "x2", numel=n2), _ptr(y2, "y2", numel=n2), h2, n_frames,
                                    tf, act, _stream(stream)))
        return y, y2

    def workspace_bytes(self, n_frames):
        return lib().wm_chunk_attn_workspace_bytes(self._h, n_frames)

    def chunk_attn(self, q_rot, k_rot, v, n_frames, out=None, active=None, scale=0.0,
                   workspace=None, stream=None, layer=0):
        if out is None:
            out = torch.empty_like(q_rot)
        nq_el = self.tokens(n_frames, self.hq)
        nk_el = self.tokens(n_frames, self.hkv)
        act_arr, act = _active(active, self.batch)
        ws = _ptr(workspace, "workspace", dtype=torch.uint8)
        ws_bytes = 0 if workspace is None else workspace.numel()
        _check(lib().wm_chunk_attn_layer(self._h, layer, _ptr(q_rot, "q_rot", numel=nq_el),
                                         _ptr(k_rot, "k_rot", numel=nk_el), _ptr(v, "v", numel=nk_el),
                                         n_frames, act, float(scale), _ptr(out, "out", numel=nq_el),
                                         ws, ws_bytes, _stream(stream)))
        return out

    def chunk_attn_noalloc(self, q_rot, k_rot, v, n_frames, out=None, active=None, scale=0.0,
                           stream=None):
        """chunk_attn without a caller workspace: split partials go to the
        library's static per-GPU scratch (calls that overlap on a GPU race)."""
        if out is None:
            out = torch.empty_like(q_rot)
        nq_el = self.tokens(n_frames, self.hq)
        nk_el = self.tokens(n_frames, self.hkv)
        act_arr, act = _active(active, self.batch)
        _check(lib().wm_chunk_attn_noalloc(self._h, _ptr(q_rot, "q_rot", numel=nq_el),
                                           _ptr(k_rot, "k_rot", numel=nk_el), _ptr(v, "v", numel=nk_el),
                                           n_frames, act, float(scale), _ptr(out, "out", numel=nq_el),
                                           _stream(stream)))
        return out

    def append_evict(self, k_raw, v, n_frames, active=None, stream=None):
        """k_raw, v: [B, n_frames*Ft, Hkv, d] per layer, stacked layer-major
        ([L, B, ...]) for a multi-layer ring."""
        nk_el = self.tokens(n_frames, self.hkv) * self.n_layers
        act_arr, act = _active(active, self.batch)
        if self.pool is None:                      # metadata-only ring: no device data
            kp = vp = None
        else:
            kp, vp = _ptr(k_raw, "k_raw", numel=nk_el), _ptr(v, "v", numel=nk_el)
        _check(lib().wm_kvring_append_evict(self._h, kp, vp, n_frames, act, self._reps_ptr,
                                            None if self.pool is None else _stream(stream)))
        return [_report_dict(r) for r in self._reps]

    def _step_args(self, qs, ks, vs, n_frames, outs, active, q_rot_scratch, k_rot_scratch, workspace):
        D = len(qs)
        nq_el = self.tokens(n_frames, self.hq)
        nk_el = self.tokens(n_frames, self.hkv)
        if outs is None:
            outs = [torch.empty_like(q) for q in qs]
        if q_rot_scratch is None:
            q_rot_scratch = torch.empty_like(qs[0])
        if k_rot_scratch is None:
            k_rot_scratch = torch.empty_like(ks[0])
        arr = lambda ts, what, n: (ctypes.c_void_p * D)(*[_ptr(t, what, numel=n) for t in ts])
        qa, ka, va = arr(qs, "q", nq_el), arr(ks, "k", nk_el), arr(vs, "v", nk_el)
        oa = arr(outs, "out", nq_el)
        act_arr, act = _active(active, self.batch)
        ws = _ptr(workspace, "workspace", dtype=torch.uint8)
        ws_bytes = 0 if workspace is None else workspace.numel()
        keep = (qa, ka, va, oa, act_arr, q_rot_scratch, k_rot_scratch, workspace, qs, ks, vs, outs)
        args = (D, qa, ka, va, n_frames, act, _ptr(q_rot_scratch, "q_rot_scratch", numel=nq_el),
                _ptr(k_rot_scratch, "k_rot_scratch", numel=nk_el), oa, ws, ws_bytes)
        return outs, args, keep

    def rollout_step(self, qs, ks, vs, n_frames, outs=None, active=None, q_rot_scratch=None,
                     k_rot_scratch=None, workspace=None, stream=None, finalize_stream=None):
        """n_denoise x (RoPE, attention), then the append; with finalize_stream
        the append runs there, overlapping the next step's RoPE."""
        outs, args, keep = self._step_args(qs, ks, vs, n_frames, outs, active, q_rot_scratch,
                                           k_rot_scratch, workspace)
        fs = None if finalize_stream is None else _stream(finalize_stream)
        _check(lib().wm_rollout_step(self._h, *args, self._reps_ptr, _stream(stream), fs))
        if finalize_stream is not None:
            # the append reads the last step's K and V there after this call
            # returns: the caching allocator must not hand their memory out
            # before that stream has passed it
            ks[-1].record_stream(finalize_stream)
            vs[-1].record_stream(finalize_stream)
        return outs, [_report_dict(r) for r in self._reps]

    def rollout_graph(self, qs, ks, vs, n_frames, outs=None, active=None, q_rot_scratch=None,
                      k_rot_scratch=None, workspace=None):
        """A HIP graph of one rollout step over these (fixed) buffers."""
        return RolloutGraph(self, qs, ks, vs, n_frames, outs, active, q_rot_scratch, k_rot_scratch,
                            workspace)


class RolloutGraph:
    """One rollout step as a HIP graph; launch() refreshes positions and slots
    from the ring's bookkeeping and runs it (rebuilding it first when the
    launch shapes have changed: see ``rebuilt``)."""

    def __init__(self, ring, qs, ks, vs, n_frames, outs, active, q_rot_scratch, k_rot_scratch,
                 workspace):
        self.ring = ring
        self.outs, args, self._keep = ring._step_args(qs, ks, vs, n_frames, outs, active, q_rot_scratch,
                                                      k_rot_scratch, workspace)
        self._h = ctypes.c_void_p()
        _check(lib().wm_rollout_graph_create(ring._h, *args, ctypes.byref(self._h)))
        self._rebuilt = ctypes.c_int32(0)
        self.rebuilt = None

    def launch(self, stream=None):
        _check(lib().wm_rollout_graph_launch(self._h, self.ring._reps_ptr, ctypes.byref(self._rebuilt),
                                             _stream(stream)))
        self.rebuilt = bool(self._rebuilt.value)
        return self.outs, [_report_dict(r) for r in self.ring._reps]

    def close(self):
        if self._h:
            _check(lib().wm_rollout_graph_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
