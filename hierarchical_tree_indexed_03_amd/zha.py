"""ctypes binding of libzha.so (include/zha.h): argument marshalling only.

Every function keeps the C name and argument order; tensors may be passed where the C
call takes a device pointer (their ``data_ptr()`` is used) and ``stream`` defaults to the
current torch stream.  Errors raise ``ZhaError`` with the library's message.  There is no
fallback: if libzha.so is missing the import of this module raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ZHA_LIB_PATH") or os.path.join(_HERE, "libzha.so")

ZHA_F32, ZHA_BF16, ZHA_MXFP4 = 0, 1, 2
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "capacity exceeded",
          4: "workspace too small", 5: "call out of order", 6: "HIP runtime error"}
GMAX = 8


class ZhaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class zha_config(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("block", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("num_ref", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("keep_sink", ctypes.c_int32),
                ("plane_dtype", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m hierarchical_tree_indexed_03_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "zha_workspace_bytes": (SZ, [ctypes.POINTER(zha_config)]),
        "zha_level1_key_form": (I32, [ctypes.POINTER(zha_config)]),
        "zha_route_keys": (I32, [ctypes.POINTER(zha_config)]),
        "zha_set_route_mode": (I32, [P, I32]),
        "zha_route_mode": (I32, [P]),
        "zha_create": (I32, [ctypes.POINTER(zha_config), P, SZ, ctypes.POINTER(P)]),
        "zha_tree_build": (I32, [P, P, P, I64, P, P]),
        "zha_tree_append": (I32, [P, P, P, P]),
        "zha_tree_append_n": (I32, [P, P, P, I64, P]),
        "zha_decode": (I32, [P, P, P, P, P]),
        "zha_decode_dense": (I32, [P, P, P, P]),
        "zha_decode_dense_static": (I32, [ctypes.POINTER(zha_config), P, P, I64, P, P, P]),
        "zha_prefill": (I32, [P, P, P, P, P, I64, P, P]),
        "zha_prefill_workspace_bytes": (SZ, [ctypes.POINTER(zha_config), I32]),
        "zha_prefill_batched": (I32, [P, P, P, P, P, I64, I32, P, SZ, P]),
        "zha_debug_prefill_trace": (I32, [P, I32, P, P, P, P]),
        "zha_debug_level": (I32, [P, I32, P, P, P]),
        "zha_debug_router_planes": (I32, [P, I32, P, P, P]),
        "zha_debug_trace": (I32, [P, I32, I64, P, P, P, P, P, P]),
        "zha_debug_route_level": (I32, [P, I32, P, P, P, P, I64, I32, P]),
        "zha_profile_start": (I32, [P, ctypes.c_char_p]),
        "zha_profile_stop": (I32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
        "zha_set_top_p_levels": (I32, [P, ctypes.POINTER(ctypes.c_float)]),
        "zha_fit_workspace_bytes": (SZ, [ctypes.POINTER(zha_config), I64, I64]),
        "zha_fit_step": (I32, [P, P, P, I64, P, P, I64, ctypes.c_float, P, P, P, SZ, P]),
        "zha_debug_check": (I32, [P, ctypes.POINTER(ctypes.c_uint32), P]),
        "zha_debug_checks_compiled": (I32, []),
        "zha_num_tokens": (I64, [P]),
        "zha_destroy": (I32, [P]),
        "zha_status_string": (ctypes.c_char_p, [I32]),
        "zha_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()
EXPORTED = ("zha_workspace_bytes", "zha_level1_key_form", "zha_route_keys", "zha_set_route_mode", "zha_route_mode",
            "zha_create", "zha_tree_build", "zha_tree_append",
            "zha_tree_append_n", "zha_decode", "zha_prefill", "zha_prefill_workspace_bytes", "zha_prefill_batched",
            "zha_debug_prefill_trace",
            "zha_decode_dense", "zha_decode_dense_static", "zha_debug_level", "zha_debug_router_planes", "zha_debug_trace", "zha_debug_route_level",
            "zha_profile_start", "zha_profile_stop", "zha_set_top_p_levels", "zha_fit_workspace_bytes", "zha_fit_step",
            "zha_debug_check", "zha_debug_checks_compiled",
            "zha_num_tokens", "zha_destroy", "zha_status_string", "zha_last_error")


def _p(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int):
    if status != 0:
        raise ZhaError(status, (_lib.zha_last_error() or b"").decode())


def _dtype(x) -> int:
    if isinstance(x, int):
        return x
    if x in ("bf16", torch.bfloat16):
        return ZHA_BF16
    return ZHA_MXFP4 if x in ("fp4", "mxfp4") else ZHA_F32


def make_config(head_dim, num_kv_heads, num_q_heads, block, levels, num_ref, capacity, dtype, top_p,
                keep_sink=True, planes="f32") -> zha_config:
    return zha_config(head_dim, num_kv_heads, num_q_heads, block, levels, num_ref, capacity, _dtype(dtype),
                      float(top_p), int(bool(keep_sink)), _dtype(planes))


def zha_level1_key_form(cfg: zha_config) -> int:
    return int(_lib.zha_level1_key_form(ctypes.byref(cfg)))


def zha_route_keys(cfg: zha_config) -> int:
    return int(_lib.zha_route_keys(ctypes.byref(cfg)))


def zha_set_route_mode(t, mode: int):
    _check(_lib.zha_set_route_mode(t, int(mode)))


def zha_route_mode(t) -> int:
    return int(_lib.zha_route_mode(t))


def zha_workspace_bytes(cfg: zha_config) -> int:
    return int(_lib.zha_workspace_bytes(ctypes.byref(cfg)))


def zha_create(cfg: zha_config, workspace, workspace_bytes: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(_lib.zha_create(ctypes.byref(cfg), _p(workspace), workspace_bytes, ctypes.byref(h)))
    return h


def zha_tree_build(t, k_cache, v_cache, n_tokens: int, ref_queries, stream=None):
    _check(_lib.zha_tree_build(t, _p(k_cache), _p(v_cache), int(n_tokens), _p(ref_queries), _s(stream)))


def zha_tree_append(t, k_new, v_new, stream=None):
    _check(_lib.zha_tree_append(t, _p(k_new), _p(v_new), _s(stream)))


def zha_tree_append_n(t, k_new, v_new, m: int, stream=None):
    _check(_lib.zha_tree_append_n(t, _p(k_new), _p(v_new), int(m), _s(stream)))


def zha_decode(t, q, out, stats=None, stream=None):
    _check(_lib.zha_decode(t, _p(q), _p(out), _p(stats), _s(stream)))


def zha_prefill(t, k_new, v_new, q, out, m: int, stats=None, stream=None):
    _check(_lib.zha_prefill(t, _p(k_new), _p(v_new), _p(q), _p(out), int(m), _p(stats), _s(stream)))


def zha_prefill_workspace_bytes(cfg: zha_config, batch: int) -> int:
    return _lib.zha_prefill_workspace_bytes(ctypes.byref(cfg), batch)


def zha_prefill_batched(t, k_new, v_new, q, out, m: int, batch: int, workspace, workspace_bytes: int, stream=None):
    _check(_lib.zha_prefill_batched(t, _p(k_new), _p(v_new), _p(q), _p(out), m, batch, _p(workspace),
                                    workspace_bytes, _s(stream)))


def zha_debug_prefill_trace(t, level: int, scores, kept, own=None, stream=None):
    _check(_lib.zha_debug_prefill_trace(t, level, _p(scores), _p(kept), _p(own), _s(stream)))


def zha_decode_dense(t, q, out, stream=None):
    _check(_lib.zha_decode_dense(t, _p(q), _p(out), _s(stream)))


def zha_decode_dense_static(cfg: zha_config, k_cache, v_cache, n_tokens: int, q, out, stream=None):
    _check(_lib.zha_decode_dense_static(ctypes.byref(cfg), _p(k_cache), _p(v_cache), int(n_tokens), _p(q), _p(out),
                                        _s(stream)))


def zha_debug_level(t, level: int, s_out, c_out, stream=None):
    _check(_lib.zha_debug_level(t, int(level), _p(s_out), _p(c_out), _s(stream)))


def zha_debug_router_planes(t, level: int, s_out, scale_out=None, stream=None):
    _check(_lib.zha_debug_router_planes(t, int(level), _p(s_out), _p(scale_out), _s(stream)))


def zha_debug_trace(t, level: int, cap: int, nodes, masks, scores, keep, counts, stream=None):
    _check(_lib.zha_debug_trace(t, int(level), int(cap), _p(nodes), _p(masks), _p(scores), _p(keep),
                                _p(counts), _s(stream)))


def zha_debug_route_level(t, level: int, q, nodes, masks, counts, cap: int, path: int = 0, stream=None):
    _check(_lib.zha_debug_route_level(t, int(level), _p(q), _p(nodes), _p(masks), _p(counts), int(cap),
                                      int(path), _s(stream)))


def zha_profile_start(t, key_prefix: str):
    _check(_lib.zha_profile_start(t, key_prefix.encode()))


def zha_profile_stop(t) -> tuple[float, int]:
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(_lib.zha_profile_stop(t, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def zha_set_top_p_levels(t, p_levels=None):
    """p_levels: p of levels 1..L in order, or None to restore the config's top_p."""
    if p_levels is None:
        _check(_lib.zha_set_top_p_levels(t, None))
        return
    arr = (ctypes.c_float * len(p_levels))(*[float(x) for x in p_levels])
    _check(_lib.zha_set_top_p_levels(t, arr))


def zha_fit_workspace_bytes(cfg: zha_config, n_tokens: int, nq: int) -> int:
    return _lib.zha_fit_workspace_bytes(ctypes.byref(cfg), n_tokens, nq)


def zha_fit_step(t, k_cache, v_cache, n_tokens: int, ref_queries, q, nq: int, lr: float, loss, grad, fit_ws,
                 fit_ws_bytes: int, stream=None):
    _check(_lib.zha_fit_step(t, _p(k_cache), _p(v_cache), n_tokens, _p(ref_queries), _p(q), nq, lr, _p(loss),
                             _p(grad), _p(fit_ws), fit_ws_bytes, _s(stream)))


def zha_debug_check(t, stream=None) -> int:
    v = ctypes.c_uint32()
    _check(_lib.zha_debug_check(t, ctypes.byref(v), _s(stream)))
    return int(v.value)


def zha_debug_checks_compiled() -> int:
    return int(_lib.zha_debug_checks_compiled())


def zha_num_tokens(t) -> int:
    return int(_lib.zha_num_tokens(t))


def zha_destroy(t):
    _check(_lib.zha_destroy(t))


def zha_status_string(s: int) -> str:
    return _lib.zha_status_string(int(s)).decode()


def zha_last_error() -> str:
    return (_lib.zha_last_error() or b"").decode()


class Tree:
    """One ZHA index over caller-owned caches: owns the device workspace (a torch tensor)."""

    def __init__(self, cfg: zha_config, device="cuda"):
        self.cfg = cfg
        nbytes = zha_workspace_bytes(cfg)
        if nbytes == 0:
            # reproduce the validation error message
            h = ctypes.c_void_p()
            _check(_lib.zha_create(ctypes.byref(cfg), None, 0, ctypes.byref(h)))
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.handle = zha_create(cfg, self.workspace, nbytes)
        self.group = cfg.num_q_heads // cfg.num_kv_heads
        self._keep = []

    def build(self, K, V, n_tokens, refs, stream=None):
        self._keep = [K, V, refs]
        zha_tree_build(self.handle, K, V, n_tokens, refs, stream)

    def append(self, k_new, v_new, stream=None):
        zha_tree_append(self.handle, k_new, v_new, stream)

    def append_n(self, k_new, v_new, stream=None):
        """k_new, v_new: [Hkv, m, d] device tensors."""
        zha_tree_append_n(self.handle, k_new, v_new, k_new.shape[1], stream)

    def set_top_p_levels(self, p_levels=None):
        if p_levels is not None and len(p_levels) != self.cfg.levels:
            raise ValueError(f"need {self.cfg.levels} values, got {len(p_levels)}")
        zha_set_top_p_levels(self.handle, p_levels)

    def set_route_mode(self, mode: int):
        """0: the config's default, 1: union frontiers, 2: every level from the keys."""
        zha_set_route_mode(self.handle, mode)

    @property
    def route_mode(self) -> int:
        return zha_route_mode(self.handle)

    def decode(self, q, out=None, stats=None, stream=None):
        if out is None:
            out = torch.empty(self.cfg.num_q_heads, self.cfg.head_dim, dtype=torch.float32, device=q.device)
        zha_decode(self.handle, q, out, stats, stream)
        return out

    def prefill(self, k_new, v_new, q, out=None, stats=None, stream=None):
        """k_new, v_new: [Hkv, m, d]; q: [m, Hq, d]; returns out [m, Hq, d] float32."""
        m = k_new.shape[1]
        if out is None:
            out = torch.empty(m, self.cfg.num_q_heads, self.cfg.head_dim, dtype=torch.float32, device=q.device)
        zha_prefill(self.handle, k_new, v_new, q, out, m, stats, stream)
        return out

    def prefill_batched(self, k_new, v_new, q, batch: int, out=None, stream=None):
        """Batched causal prefill: k_new, v_new [Hkv, m, d]; q [m, Hq, d]; ``batch`` queries
        per sub-batch.  Returns out [m, Hq, d] float32.  The prefill workspace is kept on the
        tree (grown when a larger batch needs more)."""
        m = k_new.shape[1]
        need = zha_prefill_workspace_bytes(self.cfg, batch)
        if need == 0:
            raise ValueError(f"no prefill workspace for batch={batch}")
        ws = getattr(self, "_pf_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._pf_ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        if out is None:
            out = torch.empty(m, self.cfg.num_q_heads, self.cfg.head_dim, dtype=torch.float32, device=q.device)
        zha_prefill_batched(self.handle, k_new, v_new, q, out, m, batch, ws, ws.numel(), stream)
        self._pf_last = (m - batch * ((m - 1) // batch), self.n_tokens)
        return out

    def prefill_trace(self, level: int):
        """Scores [Hkv, P, n], kept bitmaps [Hkv, P, ceil(n/32)] (int32 words) and each
        query's own rightmost node [Hkv, mb, R, d + 2] (s, c, LSE per plane) of the last
        sub-batch of prefill_batched at ``level``, as CPU tensors, with (mb, N) of that
        sub-batch."""
        mb, n_end = self._pf_last
        c = self.cfg
        g = c.num_q_heads // c.num_kv_heads
        n = -(-n_end // c.block ** level)
        dev = self.workspace.device
        scores = torch.empty(c.num_kv_heads, mb * g, n, dtype=torch.float32, device=dev)
        kept = torch.empty(c.num_kv_heads, mb * g, (n + 31) // 32, dtype=torch.int32, device=dev)
        own = torch.empty(c.num_kv_heads, mb, c.num_ref, c.head_dim + 2, dtype=torch.float32, device=dev)
        zha_debug_prefill_trace(self.handle, level, scores, kept, own)
        return scores.cpu(), kept.cpu(), own.cpu(), mb, n_end

    def decode_dense(self, q, out=None, stream=None):
        if out is None:
            out = torch.empty(self.cfg.num_q_heads, self.cfg.head_dim, dtype=torch.float32, device=q.device)
        zha_decode_dense(self.handle, q, out, stream)
        return out

    def fit_step(self, K, V, n_tokens, refs, q, lr=0.0, grad=True, stream=None):
        """One fitting step of the reference queries: refs (float32 [Hkv, R, d]) are updated in
        place by refs -= lr * grad.  q: [nq, Hq, d] training queries.  The tree is left built
        over the rounded refs the loss was taken at.  Returns (loss [Hkv], grad [Hkv, R, d] or
        None), device tensors."""
        nq = q.shape[0]
        need = zha_fit_workspace_bytes(self.cfg, n_tokens, nq)
        if need == 0:
            raise ValueError(f"no fit workspace for n_tokens={n_tokens}, nq={nq}")
        ws = getattr(self, "_fit_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._fit_ws = torch.empty(need, dtype=torch.uint8, device=refs.device)
        loss = torch.empty(self.cfg.num_kv_heads, dtype=torch.float32, device=refs.device)
        g = torch.empty_like(refs) if grad else None
        self._keep = [K, V, refs, ws]
        zha_fit_step(self.handle, K, V, n_tokens, refs, q, nq, lr, loss, g, ws, ws.numel(), stream)
        return loss, g

    @property
    def n_tokens(self) -> int:
        return zha_num_tokens(self.handle)

    def nodes(self, level: int) -> int:
        n = self.n_tokens
        return -(-n // self.cfg.block ** level)

    def level(self, level: int):
        n = self.nodes(level)
        c = self.cfg
        s = torch.empty(c.num_kv_heads, n, c.num_ref, c.head_dim, dtype=torch.float32, device=self.workspace.device)
        cc = torch.empty(c.num_kv_heads, n, c.num_ref, dtype=torch.float32, device=self.workspace.device)
        zha_debug_level(self.handle, level, s, cc)
        return s, cc

    def router_planes(self, level: int):
        """The quantised copy of s that routing reads at ``level``: bf16 planes give a
        [Hkv, n, R, d] bfloat16 tensor; MX FP4 planes give (codes [Hkv, n, R, d/2] uint8,
        scales [Hkv, n, R, d/32] uint8)."""
        c = self.cfg
        n, dev = self.nodes(level), self.workspace.device
        if c.plane_dtype == ZHA_MXFP4:
            q = torch.empty(c.num_kv_heads, n, c.num_ref, c.head_dim // 2, dtype=torch.uint8, device=dev)
            x = torch.empty(c.num_kv_heads, n, c.num_ref, c.head_dim // 32, dtype=torch.uint8, device=dev)
            zha_debug_router_planes(self.handle, level, q, x)
            return q, x
        s = torch.empty(c.num_kv_heads, n, c.num_ref, c.head_dim, dtype=torch.bfloat16, device=dev)
        zha_debug_router_planes(self.handle, level, s)
        return s

    def trace(self, level: int):
        """Routing trace of the last decode at ``level`` (0 = kept level-1 blocks): per KV
        head (nodes, masks, scores [8, n], keep) as CPU tensors cut to the entry count."""
        c = self.cfg
        cap = self.nodes(max(level, 1))
        dev = self.workspace.device
        nodes = torch.empty(c.num_kv_heads, cap, dtype=torch.int32, device=dev)
        masks = torch.empty(c.num_kv_heads, cap, dtype=torch.int32, device=dev)
        scores = torch.empty(c.num_kv_heads, GMAX, cap, dtype=torch.float32, device=dev)
        keep = torch.empty(c.num_kv_heads, cap, dtype=torch.int32, device=dev)
        counts = torch.empty(c.num_kv_heads, dtype=torch.int32, device=dev)
        zha_debug_trace(self.handle, level, cap, nodes, masks, scores if level else None,
                        keep if level else None, counts)
        out = []
        for kv in range(c.num_kv_heads):
            n = int(counts[kv])
            out.append(dict(nodes=nodes[kv, :n].cpu(), masks=masks[kv, :n].cpu(),
                            scores=scores[kv, :, :n].cpu() if level else None,
                            keep=keep[kv, :n].cpu() if level else None))
        return out

    def route_level(self, level: int, q, frontiers, path: int = 0):
        """Teacher-forced routing of one level.  ``frontiers[kv]`` = (node ids ascending,
        head masks) as int tensors; ``path`` as zha_debug_route_level; returns the trace of
        that level."""
        c = self.cfg
        cap = max(1, self.nodes(level))
        dev = self.workspace.device
        nodes = torch.zeros(c.num_kv_heads, cap, dtype=torch.int32, device=dev)
        masks = torch.zeros(c.num_kv_heads, cap, dtype=torch.int32, device=dev)
        counts = torch.zeros(c.num_kv_heads, dtype=torch.int32, device=dev)
        for kv, (nd, mk) in enumerate(frontiers):
            n = len(nd)
            nodes[kv, :n] = torch.as_tensor(nd, dtype=torch.int32).to(dev)
            masks[kv, :n] = torch.as_tensor(mk, dtype=torch.int64).to(torch.int32).to(dev)
            counts[kv] = n
        zha_debug_route_level(self.handle, level, q, nodes, masks, counts, cap, path)
        return self.trace(level)

    def close(self):
        if getattr(self, "handle", None) is not None:
            zha_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
