"""Tree attention over a DFS-packed prefix tree on MI355X (gfx950).

Thin ctypes binding of ``libtree_attn.so`` (C ABI in ``include/tree_attn.h``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments, allocates outputs and workspaces with torch, and
passes torch's current HIP stream.  There is no fallback: if the library is
missing, every call raises.

Calls mirror the C names:

    plan = tree_plan(parent, seg_len)                     # host planner
    o, lse = tree_attn_fwd(plan, q, k, v, rope_base=1e4)  # q [N,Hq,d], k/v [N,Hkv,d]
    dq, dk, dv = tree_attn_bwd(plan, q, k, v, o, lse, do, rope_base=1e4)
    loss, dlogits, err = tree_weighted_nll(logits, labels, w)
    o, lse = tree_decode_splitkv(q, k, v, span_ptr, spans, max_len)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = ["TreeAttnError", "Plan", "Partition", "HipEvents", "tree_plan", "tree_partition", "tree_attn_fwd",
           "saturation_flag", "clear_saturation_flag", "scan_wait_timed_out",
           "tree_attn_bwd", "tree_partition_fwd", "tree_partition_bwd", "tree_weighted_nll", "tree_lmhead_nll",
           "Route", "tree_route", "tree_scan_fwd", "tree_scan_bwd", "tree_conv_fwd", "tree_conv_bwd",
           "tree_decode_splitkv", "library_path", "load_library", "TA_BLOCK_M", "TA_BLOCK_N", "TA_BLOCK_KV"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtree_attn.so")
TA_BLOCK_M, TA_BLOCK_N, TA_BLOCK_KV, TA_KV_SUB, TA_CHUNK_INTS = 32, 64, 128, 32, 16
TA_KPIECE_INTS, TA_KWAVE_INTS, TA_KV_PIECE_MIN = 32, 7, 32
TA_F32, TA_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "parent pointers contain a cycle",
           3: "size exceeds the int32 index range", 4: "out of memory or buffer too small",
           5: "unsupported configuration", 6: "HIP error"}


class TreeAttnError(RuntimeError):
    def __init__(self, call: str, status: int):
        super().__init__(f"{call} failed: {_STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


class _View(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_nodes", "n_tokens", "n_leaves", "max_pos", "block_m", "block_n", "block_kv",
        "n_qtiles", "n_chunks", "n_ktiles")] + \
        [(n, ctypes.c_int64) for n in ("n_flat", "visible_pairs", "computed_pairs_fwd", "computed_pairs_bwd")] + \
        [(n, ctypes.POINTER(ctypes.c_int32)) for n in (
            "dfs_order", "node_start", "node_sub_end", "pos", "g", "node_of", "sub_end", "anc_ptr", "anc",
            "fq_ptr", "fq_chunk", "fq_order", "bk")] + \
        [(n, ctypes.c_int32) for n in ("n_prefix_nodes", "q_start", "n_kpieces", "n_ksplit", "n_kslots",
                                        "kv_piece_cap")] + \
        [(n, ctypes.POINTER(ctypes.c_int32)) for n in ("kp", "kr")] + \
        [("n_dsblk", ctypes.c_int64)] + \
        [(n, ctypes.POINTER(ctypes.c_int32)) for n in ("dq_ptr", "dq_ent", "dq_order")]


class _PartView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_nodes", "n_parts", "max_local_tokens", "reserved")] + \
        [(n, ctypes.c_int64) for n in ("n_tokens", "naive_tokens")] + \
        [("part_of", ctypes.POINTER(ctypes.c_int32)), ("part_root", ctypes.POINTER(ctypes.c_int32)),
         ("part_parent", ctypes.POINTER(ctypes.c_int32)), ("n_prefix", ctypes.POINTER(ctypes.c_int32)),
         ("own_tokens", ctypes.POINTER(ctypes.c_int64))] + \
        [(n, ctypes.POINTER(ctypes.c_int32)) for n in (
            "local_ptr", "local_node", "local_parent", "local_len", "tok_ptr", "tok_idx")]


class _RouteView(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_tokens", "n_chunks", "chunk", "conv_k")] + \
        [(n, ctypes.POINTER(ctypes.c_int32)) for n in ("chunks", "cprev", "succ_ptr", "succ", "kid_ptr", "kid",
                                                         "order")]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtree_attn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise TreeAttnError("load_library", 6) from FileNotFoundError(
            f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pI32 = ctypes.POINTER(ctypes.c_int32)
    sigs = {
        "tree_plan": (I32, [pI32, pI32, I32, I32, I32, ctypes.POINTER(P)]),
        "tree_plan_ex": (I32, [pI32, pI32, I32, I32, I32, I32, ctypes.POINTER(P)]),
        "tree_plan_view": (I32, [P, ctypes.POINTER(_View)]),
        "tree_plan_device_bytes": (I32, [P, ctypes.POINTER(SZ)]),
        "tree_plan_upload": (I32, [P, P, SZ, P]),
        "tree_plan_free": (None, [P]),
        "tree_attn_ws_bytes": (I32, [P, I32, I32, I32, I32, I32, F32, ctypes.POINTER(SZ)]),
        "tree_attn_bwd_ws_budget": (I32, [P, I32, I32, I32, I32, F32, SZ, ctypes.POINTER(SZ), pI32]),
        "tree_attn_fwd": (I32, [P, P, I32, P, P, P, I32, I32, I32, F32, F32, P, P, P, SZ, P]),
        "tree_attn_bwd": (I32, [P, P, I32, P, P, P, P, P, P, I32, I32, I32, F32, F32, P, P, P, P, SZ, P]),
        "tree_nll_ws_bytes": (I32, [I32, I32, ctypes.POINTER(SZ)]),
        "tree_weighted_nll": (I32, [I32, P, P, P, I32, I32, I32, P, P, P, P, SZ, P]),
        "tree_decode_ws_bytes": (I32, [I32, I32, I32, I32, I32, ctypes.POINTER(SZ), pI32]),
        "tree_decode_splitkv": (I32, [I32, P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, P, P, P, SZ, P]),
        "tree_attn_fwd_ex": (I32, [P, P, I32, P, P, P, I32, I32, I32, F32, F32, P, P, P, SZ, P, I32, P]),
        "tree_attn_bwd_ex": (I32, [P, P, I32, P, P, P, P, P, P, I32, I32, I32, F32, F32, P, P, P, P, SZ, P, I32,
                                   P]),
        "tree_decode_splitkv_ex": (I32, [I32, P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, P, P, P, SZ, P, I32,
                                         P]),
        "tree_decode_splitkv_noalloc": (I32, [I32, P, P, P, P, P, I32, I32, I32, I32, I32, F32, I32, P, P, P]),
        "tree_partition": (I32, [pI32, pI32, I32, I64, I32, I32, ctypes.POINTER(P)]),
        "tree_partition_view": (I32, [P, ctypes.POINTER(_PartView)]),
        "tree_partition_plan": (I32, [P, I32, ctypes.POINTER(P)]),
        "tree_partition_device_bytes": (I32, [P, ctypes.POINTER(SZ)]),
        "tree_partition_upload": (I32, [P, P, SZ, P]),
        "tree_partition_free": (None, [P]),
        "tree_partition_ws_bytes": (I32, [P, I32, I32, I32, I32, I32, F32, ctypes.POINTER(SZ)]),
        "tree_partition_fwd": (I32, [P, P, I32, P, P, P, I32, I32, I32, F32, F32, P, P, P, SZ, P]),
        "tree_partition_bwd": (I32, [P, P, I32, P, P, P, P, P, P, I32, I32, I32, F32, F32, P, P, P, P, SZ, P]),
        "tree_lmhead_nll_ws_bytes": (I32, [I32, I32, I32, I32, I32, ctypes.POINTER(SZ)]),
        "tree_lmhead_nll": (I32, [I32, P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, P, P, SZ, P]),
        "tree_route": (I32, [P, I32, ctypes.POINTER(P)]),
        "tree_route_view": (I32, [P, ctypes.POINTER(_RouteView)]),
        "tree_route_device_bytes": (I32, [P, ctypes.POINTER(SZ)]),
        "tree_route_upload": (I32, [P, P, SZ, P]),
        "tree_route_free": (None, [P]),
        "tree_scan_ws_bytes": (I32, [P, I32, ctypes.POINTER(SZ)]),
        "tree_scan_fwd": (I32, [P, P, P, P, I32, P, P, SZ, P]),
        "tree_scan_bwd": (I32, [P, P, P, P, P, I32, P, P, P, SZ, P]),
        "tree_conv_ws_bytes": (I32, [P, I32, ctypes.POINTER(SZ)]),
        "tree_conv_fwd": (I32, [P, P, P, P, I32, P, P]),
        "tree_conv_bwd": (I32, [P, P, P, P, P, I32, P, P, P, SZ, P]),
        "ta_status_string": (ctypes.c_char_p, [I32]),
    }
    host_only = os.environ.get("TA_HOST_ONLY_LIBRARY") == "1"  # a planner-only build (sanitizer tests)
    for name, (res, args) in sigs.items():
        fn = getattr(L, name, None)
        if fn is None:
            if host_only:
                continue
            raise TreeAttnError("load_library", 6) from AttributeError(f"{_LIB_PATH} lacks {name}")
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(call, status):
    if status != 0:
        raise TreeAttnError(call, status)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Plan:
    """Host plan of a prefix tree (owned by the library; freed on deletion)."""

    def __init__(self, parent, seg_len, block_m: int = 0, block_n: int = 0, n_prefix_nodes: int = 0):
        L = load_library()
        parent, seg_len = _i32(parent), _i32(seg_len)
        if parent.ndim != 1 or parent.shape != seg_len.shape:
            raise ValueError("parent and seg_len must be 1-D arrays of equal length")
        self._lib = L
        self._ptr = ctypes.c_void_p()
        pI32 = ctypes.POINTER(ctypes.c_int32)
        _check("tree_plan", L.tree_plan_ex(parent.ctypes.data_as(pI32), seg_len.ctypes.data_as(pI32),
                                           int(parent.shape[0]), int(n_prefix_nodes), block_m, block_n,
                                           ctypes.byref(self._ptr)))
        self._owner = None
        self._load_view()

    @classmethod
    def _borrowed(cls, ptr, owner):
        """A view of a plan owned by another library object (kept alive by `owner`)."""
        self = cls.__new__(cls)
        self._lib = load_library()
        self._ptr = ctypes.c_void_p(ptr)
        self._owner = owner
        self._load_view()
        return self

    def _load_view(self):
        L = self._lib
        v = _View()
        _check("tree_plan_view", L.tree_plan_view(self._ptr, ctypes.byref(v)))
        self._v = v
        self._dev = {}
        for name in ("n_nodes", "n_tokens", "n_leaves", "max_pos", "block_m", "block_n", "block_kv",
                     "n_qtiles", "n_chunks", "n_ktiles", "n_flat", "visible_pairs",
                     "computed_pairs_fwd", "computed_pairs_bwd", "n_prefix_nodes", "q_start", "n_kpieces",
                     "n_ksplit", "n_kslots", "kv_piece_cap", "n_dsblk"):
            setattr(self, name, int(getattr(v, name)))

    def _arr(self, name, n):
        if n == 0:
            return np.zeros(0, np.int32)
        return np.ctypeslib.as_array(getattr(self._v, name), shape=(n,)).copy()

    def view(self) -> dict:
        """Copies of every plan table as numpy arrays."""
        n, N = self.n_nodes, self.n_tokens
        anc_ptr = self._arr("anc_ptr", n + 1)
        return dict(
            dfs_order=self._arr("dfs_order", n), node_start=self._arr("node_start", n),
            node_sub_end=self._arr("node_sub_end", n), pos=self._arr("pos", N), g=self._arr("g", N),
            node_of=self._arr("node_of", N), sub_end=self._arr("sub_end", N), anc_ptr=anc_ptr,
            anc=self._arr("anc", int(anc_ptr[-1])), fq_ptr=self._arr("fq_ptr", self.n_qtiles + 1),
            fq_chunk=self._arr("fq_chunk", self.n_chunks * TA_CHUNK_INTS).reshape(-1, TA_CHUNK_INTS),
            fq_order=self._arr("fq_order", self.n_qtiles), bk=self._arr("bk", self.n_ktiles * 4).reshape(-1, 4),
            kp=self._arr("kp", self.n_kpieces * TA_KPIECE_INTS).reshape(-1, TA_KPIECE_INTS),
            kr=self._arr("kr", self.n_ksplit * 4).reshape(-1, 4),
            dq_ptr=self._arr("dq_ptr", self.n_qtiles + 1),
            dq_ent=self._arr("dq_ent", int(self._arr("dq_ptr", self.n_qtiles + 1)[-1]) * 4).reshape(-1, 4),
            dq_order=self._arr("dq_order", self.n_qtiles))

    @property
    def handle(self):
        return self._ptr

    def device(self, device=None):
        """The plan's tables uploaded to device memory (a torch uint8 tensor, cached)."""
        import torch
        dev = torch.device(device if device is not None else "cuda")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        key = str(dev)
        if key not in self._dev:
            n = ctypes.c_size_t()
            _check("tree_plan_device_bytes", self._lib.tree_plan_device_bytes(self._ptr, ctypes.byref(n)))
            buf = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
            st = torch.cuda.current_stream(dev)
            _check("tree_plan_upload", self._lib.tree_plan_upload(self._ptr, ctypes.c_void_p(buf.data_ptr()),
                                                                   int(n.value), ctypes.c_void_p(st.cuda_stream)))
            st.synchronize()  # the host tables are pageable: finish the copy before returning
            self._dev[key] = buf
        return self._dev[key]

    def __del__(self):
        ptr = getattr(self, "_ptr", None)
        if ptr is not None and ptr.value and getattr(self, "_owner", None) is None:
            self._lib.tree_plan_free(ptr)
            self._ptr = None


def tree_plan(parent, seg_len, block_m: int = 0, block_n: int = 0, n_prefix_nodes: int = 0) -> Plan:
    """Plan of a prefix tree; n_prefix_nodes > 0 plans nodes 0..n-1 as a key-only ancestor chain
    (tree_plan_ex)."""
    return Plan(parent, seg_len, block_m, block_n, n_prefix_nodes)


class Partition:
    """Connected-subtree partition of a tree under a token capacity (tree_partition), with each
    partition's local plan (its root's ancestor chain as a key-only prefix)."""

    def __init__(self, parent, seg_len, capacity: int, block_m: int = 0, block_n: int = 0):
        L = load_library()
        parent, seg_len = _i32(parent), _i32(seg_len)
        if parent.ndim != 1 or parent.shape != seg_len.shape:
            raise ValueError("parent and seg_len must be 1-D arrays of equal length")
        self._lib = L
        self._ptr = ctypes.c_void_p()
        pI32 = ctypes.POINTER(ctypes.c_int32)
        _check("tree_partition", L.tree_partition(parent.ctypes.data_as(pI32), seg_len.ctypes.data_as(pI32),
                                                  int(parent.shape[0]), int(capacity), block_m, block_n,
                                                  ctypes.byref(self._ptr)))
        v = _PartView()
        _check("tree_partition_view", L.tree_partition_view(self._ptr, ctypes.byref(v)))
        self._v = v
        self._dev = {}
        for name in ("n_nodes", "n_parts", "max_local_tokens", "n_tokens", "naive_tokens"):
            setattr(self, name, int(getattr(v, name)))
        self.plans = []
        for i in range(self.n_parts):
            pp = ctypes.c_void_p()
            _check("tree_partition_plan", L.tree_partition_plan(self._ptr, i, ctypes.byref(pp)))
            self.plans.append(Plan._borrowed(pp.value, self) if pp.value else None)

    def _arr(self, name, n):
        if n == 0:
            return np.zeros(0, getattr(self._v, name)._type_)
        return np.ctypeslib.as_array(getattr(self._v, name), shape=(n,)).copy()

    def view(self) -> dict:
        """Copies of the partition tables as numpy arrays."""
        n, P = self.n_nodes, self.n_parts
        local_ptr = self._arr("local_ptr", P + 1)
        tok_ptr = self._arr("tok_ptr", P + 1)
        return dict(
            part_of=self._arr("part_of", n), part_root=self._arr("part_root", P),
            part_parent=self._arr("part_parent", P), n_prefix=self._arr("n_prefix", P),
            own_tokens=self._arr("own_tokens", P), local_ptr=local_ptr,
            local_node=self._arr("local_node", int(local_ptr[-1])),
            local_parent=self._arr("local_parent", int(local_ptr[-1])),
            local_len=self._arr("local_len", int(local_ptr[-1])), tok_ptr=tok_ptr,
            tok_idx=self._arr("tok_idx", int(tok_ptr[-1])))

    @property
    def handle(self):
        return self._ptr

    def device(self, device=None):
        """Every local plan and row map uploaded to device memory (a torch uint8 tensor, cached)."""
        import torch
        dev = torch.device(device if device is not None else "cuda")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        key = str(dev)
        if key not in self._dev:
            n = ctypes.c_size_t()
            _check("tree_partition_device_bytes",
                   self._lib.tree_partition_device_bytes(self._ptr, ctypes.byref(n)))
            buf = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
            st = torch.cuda.current_stream(dev)
            _check("tree_partition_upload", self._lib.tree_partition_upload(
                self._ptr, ctypes.c_void_p(buf.data_ptr()), int(n.value), ctypes.c_void_p(st.cuda_stream)))
            st.synchronize()  # the host tables are pageable: finish the copy before returning
            self._dev[key] = buf
        return self._dev[key]

    def __del__(self):
        ptr = getattr(self, "_ptr", None)
        if ptr is not None and ptr.value:
            self.plans = []
            self._lib.tree_partition_free(ptr)
            self._ptr = None


def tree_partition(parent, seg_len, capacity: int, block_m: int = 0, block_n: int = 0) -> Partition:
    """Cut a tree into connected subtrees of at most `capacity` own tokens (tree_partition)."""
    return Partition(parent, seg_len, capacity, block_m, block_n)


class Route:
    """Routing tables of a plan for recurrent layers (tree_route): scan chunks and conv context."""

    def __init__(self, plan: "Plan", conv_k: int = 4):
        L = load_library()
        self._lib = L
        self._plan = plan
        self._ptr = ctypes.c_void_p()
        _check("tree_route", L.tree_route(plan.handle, int(conv_k), ctypes.byref(self._ptr)))
        v = _RouteView()
        _check("tree_route_view", L.tree_route_view(self._ptr, ctypes.byref(v)))
        self._v = v
        self._dev = {}
        for name in ("n_tokens", "n_chunks", "chunk", "conv_k"):
            setattr(self, name, int(getattr(v, name)))

    def view(self) -> dict:
        def arr(name, n):
            return np.zeros(0, np.int32) if n == 0 else np.ctypeslib.as_array(getattr(self._v, name), shape=(n,)).copy()
        sp = arr("succ_ptr", self.n_tokens + 1)
        kp = arr("kid_ptr", self.n_chunks + 1)
        return dict(chunks=arr("chunks", 4 * self.n_chunks).reshape(-1, 4),
                    cprev=arr("cprev", self.n_tokens * (self.conv_k - 1)).reshape(self.n_tokens, self.conv_k - 1),
                    succ_ptr=sp, succ=arr("succ", int(sp[-1])),
                    kid_ptr=kp, kid=arr("kid", int(kp[-1])), order=arr("order", self.n_chunks))

    @property
    def handle(self):
        return self._ptr

    def device(self, device=None):
        import torch
        dev = torch.device(device if device is not None else "cuda")
        if dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        key = str(dev)
        if key not in self._dev:
            n = ctypes.c_size_t()
            _check("tree_route_device_bytes", self._lib.tree_route_device_bytes(self._ptr, ctypes.byref(n)))
            buf = torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)
            st = torch.cuda.current_stream(dev)
            _check("tree_route_upload", self._lib.tree_route_upload(self._ptr, ctypes.c_void_p(buf.data_ptr()),
                                                                     int(n.value), ctypes.c_void_p(st.cuda_stream)))
            st.synchronize()
            self._dev[key] = buf
        return self._dev[key]

    def __del__(self):
        ptr = getattr(self, "_ptr", None)
        if ptr is not None and ptr.value:
            self._lib.tree_route_free(ptr)
            self._ptr = None


def tree_route(plan, conv_k: int = 4) -> Route:
    return Route(plan, conv_k)


def _dt(t):
    import torch
    if t.dtype == torch.bfloat16:
        return TA_BF16
    if t.dtype == torch.float32:
        return TA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, shape, dtype, device):
    """Every tensor handed to the library (inputs, and outputs the caller
    supplies) must have exactly this shape and dtype, be contiguous and live
    on the call's device: the kernels take raw pointers."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")


def _events(events):
    """Optional stage-timing events: a HipEvents slice (see HipEvents.slice)."""
    if events is None:
        return ctypes.c_void_p(0), 0
    arr, n = events
    return ctypes.cast(arr, ctypes.c_void_p), n


class HipEvents:
    """A pool of hipEvent_t created through the HIP runtime, for the *_ex
    calls' stage timing (events must be recorded on the launch stream)."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        self.n = 0
        for i in range(n):
            e = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise TreeAttnError("hipEventCreate", 6)
            self.arr[i] = e.value
            self.n = i + 1

    def slice(self, start: int, count: int):
        base = ctypes.addressof(self.arr) + start * ctypes.sizeof(ctypes.c_void_p)
        return (ctypes.c_void_p(base), count)

    def elapsed_ms(self, a: int, b: int) -> float:
        self._hip.hipEventSynchronize(self.arr[b])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[a], self.arr[b]) != 0:
            raise TreeAttnError("hipEventElapsedTime", 6)
        return float(ms.value)

    def __del__(self):
        for i in range(getattr(self, "n", 0)):
            if self.arr[i]:
                self._hip.hipEventDestroy(self.arr[i])


def saturation_flag(ws) -> int:
    """The bf16 attention calls' saturation flag (the first int32 of their
    workspace): 1 when a Q or K value beyond the fp16 range was clamped since
    the flag was last cleared (a synchronising read)."""
    return int(ws[:4].view(__import__("torch").int32).item())


def clear_saturation_flag(ws) -> None:
    """Zero the saturation flag of a workspace (asynchronously, on the current stream)."""
    ws[:4].zero_()


def scan_wait_timed_out(ws) -> bool:
    """After tree_scan_fwd/bwd with workspace ws: whether a wait for a
    published value ran out (word 1 of the workspace; the outputs are then not
    valid).  A synchronising read."""
    return int(ws[4:8].view(__import__("torch").int32).item()) != 0


def _workspace(nbytes, device, ws):
    """A caller-supplied workspace must be a contiguous uint8 tensor on the
    call's device; one smaller than nbytes is replaced by a fresh buffer."""
    import torch
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous uint8 tensor")
        if not ws.is_cuda or ws.device != device:
            raise ValueError(f"ws must live on {device}")
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf[:min(nbytes, 4)].zero_()  # a fresh workspace starts with a clear saturation flag
    return buf, nbytes


def attn_ws_bytes(plan: Plan, op: int, dtype_code: int, Hq: int, Hkv: int, d: int, rope_base: float) -> int:
    n = ctypes.c_size_t()
    _check("tree_attn_ws_bytes", load_library().tree_attn_ws_bytes(plan.handle, op, dtype_code, Hq, Hkv, d,
                                                                    float(rope_base), ctypes.byref(n)))
    return int(n.value)


def tree_attn_fwd(plan: Plan, q, k, v, scale: float = 0.0, rope_base: float = 0.0, o=None, lse=None, ws=None,
                  events=None):
    """Forward tree attention.  q [N,Hq,d], k/v [N,Hkv,d] (bf16 or fp32) ->
    o [N,Hq,d] (same dtype), lse [Hq,N] fp32."""
    import torch
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if N != plan.n_tokens:
        raise ValueError(f"q has {N} tokens, the plan {plan.n_tokens}")
    for name, t, shp in (("q", q, (N, Hq, d)), ("k", k, (N, Hkv, d)), ("v", v, (N, Hkv, d))):
        _need(t, name, shp, q.dtype, dev)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(Hq, N, dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (N, Hq, d), q.dtype, dev)
    _need(lse, "lse", (Hq, N), torch.float32, dev)
    dt = _dt(q)
    wsb = attn_ws_bytes(plan, 0, dt, Hq, Hkv, d, rope_base)
    ws, wsn = _workspace(wsb, dev, ws)
    ev, nev = _events(events)
    _check("tree_attn_fwd", load_library().tree_attn_fwd_ex(
        plan.handle, _ptr(plan.device(dev)), dt, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, d, float(scale),
        float(rope_base), _ptr(o), _ptr(lse), _ptr(ws), wsn, ev, nev, _stream(q)))
    return o, lse


def bwd_ws_budget(plan: Plan, dtype_code: int, Hq: int, Hkv: int, d: int, rope_base: float, budget: int = 0):
    """(bytes, kv_heads_per_round) of the largest backward workspace within
    `budget` bytes (0: the library default, 8 GiB); raises when even the
    smallest workspace exceeds it."""
    n, h = ctypes.c_size_t(), ctypes.c_int32()
    _check("tree_attn_bwd_ws_budget", load_library().tree_attn_bwd_ws_budget(
        plan.handle, dtype_code, Hq, Hkv, d, float(rope_base), int(budget), ctypes.byref(n), ctypes.byref(h)))
    return int(n.value), int(h.value)


def tree_attn_bwd(plan: Plan, q, k, v, o, lse, dO, scale: float = 0.0, rope_base: float = 0.0,
                  dq=None, dk=None, dv=None, ws=None, events=None, recompute_dq: bool = False,
                  ws_budget: int = 0):
    """Backward of tree_attn_fwd -> (dq, dk, dv), overwritten, deterministic.
    Without a caller workspace the binding allocates the largest one within
    ws_budget bytes (0: the library default, 8 GiB): the full dS workspace
    when it fits, else the dS blocks of as many KV heads as fit (run in
    rounds), else the smallest one.  recompute_dq: use the smallest workspace,
    in which dQ recomputes S and dP instead of reading the dS blocks the dK/dV
    kernel stores (bf16)."""
    import torch
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if N != plan.n_tokens:
        raise ValueError(f"q has {N} tokens, the plan {plan.n_tokens}")
    for name, t, shp in (("q", q, (N, Hq, d)), ("k", k, (N, Hkv, d)), ("v", v, (N, Hkv, d)),
                         ("o", o, (N, Hq, d)), ("dO", dO, (N, Hq, d))):
        _need(t, name, shp, q.dtype, dev)
    _need(lse, "lse", (Hq, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", (N, Hq, d), q.dtype, dev)
    _need(dk, "dk", (N, Hkv, d), q.dtype, dev)
    _need(dv, "dv", (N, Hkv, d), q.dtype, dev)
    dt = _dt(q)
    if recompute_dq:
        wsb = attn_ws_bytes(plan, 2, dt, Hq, Hkv, d, rope_base)
    elif ws is not None:
        wsb = attn_ws_bytes(plan, 2, dt, Hq, Hkv, d, rope_base)  # a caller workspace: the call uses what fits
    else:
        wsb = bwd_ws_budget(plan, dt, Hq, Hkv, d, rope_base, ws_budget)[0]
    ws, wsn = _workspace(wsb, dev, ws)
    if recompute_dq:
        wsn = min(wsn, wsb)
    ev, nev = _events(events)
    _check("tree_attn_bwd", load_library().tree_attn_bwd_ex(
        plan.handle, _ptr(plan.device(dev)), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
        Hq, Hkv, d, float(scale), float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsn, ev, nev,
        _stream(q)))
    return dq, dk, dv


def partition_ws_bytes(part: Partition, op: int, dtype_code: int, Hq: int, Hkv: int, d: int,
                       rope_base: float) -> int:
    n = ctypes.c_size_t()
    _check("tree_partition_ws_bytes", load_library().tree_partition_ws_bytes(
        part.handle, op, dtype_code, Hq, Hkv, d, float(rope_base), ctypes.byref(n)))
    return int(n.value)


def tree_partition_fwd(part: Partition, q, k, v, scale: float = 0.0, rope_base: float = 0.0, o=None, lse=None,
                       ws=None):
    """tree_attn_fwd run one partition at a time through the gateway.  Same layouts as tree_attn_fwd."""
    import torch
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if N != part.n_tokens:
        raise ValueError(f"q has {N} tokens, the partition {part.n_tokens}")
    for name, t, shp in (("q", q, (N, Hq, d)), ("k", k, (N, Hkv, d)), ("v", v, (N, Hkv, d))):
        _need(t, name, shp, q.dtype, dev)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(Hq, N, dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (N, Hq, d), q.dtype, dev)
    _need(lse, "lse", (Hq, N), torch.float32, dev)
    dt = _dt(q)
    ws, wsn = _workspace(partition_ws_bytes(part, 0, dt, Hq, Hkv, d, rope_base), dev, ws)
    _check("tree_partition_fwd", load_library().tree_partition_fwd(
        part.handle, _ptr(part.device(dev)), dt, _ptr(q), _ptr(k), _ptr(v), Hq, Hkv, d, float(scale),
        float(rope_base), _ptr(o), _ptr(lse), _ptr(ws), wsn, _stream(q)))
    return o, lse


def tree_partition_bwd(part: Partition, q, k, v, o, lse, dO, scale: float = 0.0, rope_base: float = 0.0,
                       dq=None, dk=None, dv=None, ws=None):
    """Backward of tree_partition_fwd -> (dq, dk, dv), with the gateway gradients relayed in fp32."""
    import torch
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if N != part.n_tokens:
        raise ValueError(f"q has {N} tokens, the partition {part.n_tokens}")
    for name, t, shp in (("q", q, (N, Hq, d)), ("k", k, (N, Hkv, d)), ("v", v, (N, Hkv, d)),
                         ("o", o, (N, Hq, d)), ("dO", dO, (N, Hq, d))):
        _need(t, name, shp, q.dtype, dev)
    _need(lse, "lse", (Hq, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", (N, Hq, d), q.dtype, dev)
    _need(dk, "dk", (N, Hkv, d), q.dtype, dev)
    _need(dv, "dv", (N, Hkv, d), q.dtype, dev)
    dt = _dt(q)
    ws, wsn = _workspace(partition_ws_bytes(part, 1, dt, Hq, Hkv, d, rope_base), dev, ws)
    _check("tree_partition_bwd", load_library().tree_partition_bwd(
        part.handle, _ptr(part.device(dev)), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO),
        Hq, Hkv, d, float(scale), float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), wsn, _stream(q)))
    return dq, dk, dv


def lmhead_ws_bytes(N: int, V: int, Dm: int, need_grad: bool, vocab_chunk: int = 0) -> int:
    n = ctypes.c_size_t()
    _check("tree_lmhead_nll_ws_bytes", load_library().tree_lmhead_nll_ws_bytes(
        int(N), int(V), int(Dm), int(bool(need_grad)), int(vocab_chunk), ctypes.byref(n)))
    return int(n.value)


def tree_lmhead_nll(h, W, labels, w, ignore_index: int = -100, need_grad: bool = True, vocab_chunk: int = 0,
                    loss=None, lse=None, dh=None, dW=None, err_flag=None, ws=None):
    """Output layer + weighted NLL without the N x V logits.  h [N,Dm] bf16, W [V,Dm] bf16,
    labels [N] int32, w [N] fp32 -> (loss [1] fp32, lse [N] fp32, dh, dW (bf16, None without grad),
    err_flag [1] int32)."""
    import torch
    N, Dm = h.shape
    V = W.shape[0]
    dev = h.device
    _need(h, "h", (N, Dm), torch.bfloat16, dev)
    _need(W, "W", (V, Dm), torch.bfloat16, dev)
    _need(labels, "labels", (N,), torch.int32, dev)
    _need(w, "w", (N,), torch.float32, dev)
    loss = torch.zeros(1, dtype=torch.float32, device=dev) if loss is None else loss
    lse = torch.empty(N, dtype=torch.float32, device=dev) if lse is None else lse
    err_flag = torch.zeros(1, dtype=torch.int32, device=dev) if err_flag is None else err_flag
    _need(loss, "loss", (1,), torch.float32, dev)
    _need(lse, "lse", (N,), torch.float32, dev)
    _need(err_flag, "err_flag", (1,), torch.int32, dev)
    if need_grad:
        dh = torch.empty_like(h) if dh is None else dh
        dW = torch.empty_like(W) if dW is None else dW
        _need(dh, "dh", (N, Dm), torch.bfloat16, dev)
        _need(dW, "dW", (V, Dm), torch.bfloat16, dev)
    else:
        dh = dW = None
    ws, wsn = _workspace(lmhead_ws_bytes(N, V, Dm, need_grad, vocab_chunk), dev, ws)
    _check("tree_lmhead_nll", load_library().tree_lmhead_nll(
        TA_BF16, _ptr(h), _ptr(W), _ptr(labels), _ptr(w), N, V, Dm, int(ignore_index), int(vocab_chunk),
        _ptr(loss), _ptr(lse), _ptr(dh) if dh is not None else None, _ptr(dW) if dW is not None else None,
        _ptr(err_flag), _ptr(ws), wsn, _stream(h)))
    return loss, lse, dh, dW, err_flag


def _route_ws(fn, route, C):
    n = ctypes.c_size_t()
    _check(fn, getattr(load_library(), fn)(route.handle, int(C), ctypes.byref(n)))
    return int(n.value)


def _need_rows(route, name, t, C):
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (route.n_tokens, C):
        raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor of shape ({route.n_tokens}, {C})")


def tree_scan_fwd(route: Route, a, b, h=None, ws=None):
    """h_t = a_t * h_prev(t) + b_t along the tree (chunks start from the parent's end state)."""
    import torch
    C = a.shape[1]
    for name, t in (("a", a), ("b", b)):
        _need_rows(route, name, t, C)
    h = torch.empty_like(a) if h is None else h
    _need_rows(route, "h", h, C)
    ws, wsn = _workspace(_route_ws("tree_scan_ws_bytes", route, C), a.device, ws)
    _check("tree_scan_fwd", load_library().tree_scan_fwd(route.handle, _ptr(route.device(a.device)), _ptr(a), _ptr(b),
                                                         C, _ptr(h), _ptr(ws), wsn, _stream(a)))
    return h


def tree_scan_bwd(route: Route, a, h, dh, da=None, db=None, ws=None):
    import torch
    C = a.shape[1]
    for name, t in (("a", a), ("h", h), ("dh", dh)):
        _need_rows(route, name, t, C)
    da = torch.empty_like(a) if da is None else da
    db = torch.empty_like(a) if db is None else db
    _need_rows(route, "da", da, C)
    _need_rows(route, "db", db, C)
    ws, wsn = _workspace(_route_ws("tree_scan_ws_bytes", route, C), a.device, ws)
    _check("tree_scan_bwd", load_library().tree_scan_bwd(route.handle, _ptr(route.device(a.device)), _ptr(a), _ptr(h),
                                                         _ptr(dh), C, _ptr(da), _ptr(db), _ptr(ws), wsn, _stream(a)))
    return da, db


def tree_conv_fwd(route: Route, x, w, y=None):
    """y_t = sum_j w[:, j] * x_{prev^j(t)} along the tree path."""
    import torch
    C = x.shape[1]
    _need_rows(route, "x", x, C)
    _need(w, "w", (C, route.conv_k), torch.float32, x.device)
    y = torch.empty_like(x) if y is None else y
    _need_rows(route, "y", y, C)
    _check("tree_conv_fwd", load_library().tree_conv_fwd(route.handle, _ptr(route.device(x.device)), _ptr(x), _ptr(w),
                                                         C, _ptr(y), _stream(x)))
    return y


def tree_conv_bwd(route: Route, x, w, dy, dx=None, dw=None, ws=None):
    import torch
    C = x.shape[1]
    for name, t in (("x", x), ("dy", dy)):
        _need_rows(route, name, t, C)
    _need(w, "w", (C, route.conv_k), torch.float32, x.device)
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    _need_rows(route, "dx", dx, C)
    _need(dw, "dw", (C, route.conv_k), torch.float32, x.device)
    ws, wsn = _workspace(_route_ws("tree_conv_ws_bytes", route, C), x.device, ws)
    _check("tree_conv_bwd", load_library().tree_conv_bwd(route.handle, _ptr(route.device(x.device)), _ptr(x), _ptr(w),
                                                         _ptr(dy), C, _ptr(dx), _ptr(dw), _ptr(ws), wsn, _stream(x)))
    return dx, dw


def tree_weighted_nll(logits, labels, w, ignore_index: int = -100, need_grad: bool = True,
                      loss=None, dlogits=None, err_flag=None, ws=None):
    """sum_t w_t [y_t valid] (logsumexp(x_t) - x_t[y_t]) -> (loss [1] fp32, dlogits or None, err_flag [1] int32)."""
    import torch
    N, V = logits.shape
    dev = logits.device
    _need(logits, "logits", (N, V), torch.float32, dev)
    _need(labels, "labels", (N,), torch.int32, dev)
    _need(w, "w", (N,), torch.float32, dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    if need_grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    if err_flag is None:
        err_flag = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(loss, "loss", (1,), torch.float32, dev)
    _need(err_flag, "err_flag", (1,), torch.int32, dev)
    if need_grad:
        _need(dlogits, "dlogits", (N, V), torch.float32, dev)
    n = ctypes.c_size_t()
    L = load_library()
    _check("tree_nll_ws_bytes", L.tree_nll_ws_bytes(N, V, ctypes.byref(n)))
    ws, wsn = _workspace(int(n.value), dev, ws)
    _check("tree_weighted_nll", L.tree_weighted_nll(
        TA_F32, _ptr(logits), _ptr(labels), _ptr(w), N, V, int(ignore_index), _ptr(loss),
        _ptr(dlogits if need_grad else None), _ptr(err_flag), _ptr(ws), wsn, _stream(logits)))
    return loss, (dlogits if need_grad else None), err_flag


def decode_ws_bytes(B, Hq, d, max_len, n_splits=0):
    n = ctypes.c_size_t()
    s = ctypes.c_int32()
    _check("tree_decode_ws_bytes", load_library().tree_decode_ws_bytes(B, Hq, d, int(max_len), int(n_splits),
                                                                        ctypes.byref(n), ctypes.byref(s)))
    return int(n.value), int(s.value)


def _check_spans(span_ptr, spans, n_rows: int, max_len: int):
    """Host check of the decode span tables (one small device-to-host copy):
    span_ptr non-decreasing from 0 to the span count, every (start, len) span
    inside [0, n_rows), and every item's total length at most max_len."""
    sp = span_ptr.cpu().numpy().astype(np.int64)
    s = spans.cpu().numpy().astype(np.int64).reshape(-1, 2)
    if sp[0] != 0 or np.any(np.diff(sp) < 0) or sp[-1] > len(s):
        raise ValueError("span_ptr must rise from 0 to at most the number of spans")
    used = s[:sp[-1]]
    if np.any(used[:, 1] < 0) or np.any(used[:, 0] < 0) or np.any(used[:, 0] + used[:, 1] > n_rows):
        raise ValueError(f"a span lies outside the {n_rows} K/V rows")
    tot = np.add.reduceat(np.concatenate([used[:, 1], [0]]), sp[:-1]) if len(sp) > 1 else np.zeros(0)
    tot = np.where(np.diff(sp) > 0, tot, 0)
    if np.any(tot > max_len):
        raise ValueError(f"an item's spans add up to more than max_len = {max_len}")


def tree_decode_splitkv(q, k, v, span_ptr, spans, max_len: int, scale: float = 0.0, n_splits: int = 0,
                        o=None, lse=None, ws=None, events=None, check_spans: bool = True):
    """Split-KV single-query decode.  q [B,Hq,d] bf16; k/v [L,Hkv,d] bf16;
    span_ptr [B+1], spans [S,2] int32 on the device -> o [B,Hq,d], lse [B,Hq].
    check_spans: verify on the host (one synchronising copy of the two small
    tables) that every span lies inside k's rows and every item within
    max_len; with False the caller guarantees it, as the C call requires."""
    import torch
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _need(q, "q", (B, Hq, d), torch.bfloat16, dev)
    _need(k, "k", tuple(k.shape), torch.bfloat16, dev)
    _need(v, "v", tuple(k.shape), torch.bfloat16, dev)
    _need(span_ptr, "span_ptr", (B + 1,), torch.int32, dev)
    _need(spans, "spans", tuple(spans.shape), torch.int32, dev)
    if spans.dim() != 2 or spans.shape[1] != 2:
        raise ValueError("spans must have shape (S, 2)")
    if check_spans:
        _check_spans(span_ptr, spans, k.shape[0], max_len)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev) if lse is None else lse
    _need(o, "o", (B, Hq, d), torch.bfloat16, dev)
    _need(lse, "lse", (B, Hq), torch.float32, dev)
    wsb, _ = decode_ws_bytes(B, Hq, d, max_len, n_splits)
    ws, wsn = _workspace(wsb, dev, ws)
    ev, nev = _events(events)
    _check("tree_decode_splitkv", load_library().tree_decode_splitkv_ex(
        TA_BF16, _ptr(q), _ptr(k), _ptr(v), _ptr(span_ptr), _ptr(spans), B, Hq, Hkv, d, int(max_len),
        float(scale), int(n_splits), _ptr(o), _ptr(lse), _ptr(ws), wsn, ev, nev, _stream(q)))
    return o, lse


DECODE_SCRATCH_BYTES = 16 << 20  # TA_DECODE_SCRATCH_BYTES


def tree_decode_splitkv_noalloc(q, k, v, span_ptr, spans, max_len: int, o, lse, scale: float = 0.0,
                                n_splits: int = 0):
    """tree_decode_splitkv without any allocation, for graph capture and
    serving loops: the caller passes the outputs o [B,Hq,d] bf16 and lse
    [B,Hq] fp32, and the per-slice partials use the library's fixed scratch
    (DECODE_SCRATCH_BYTES per GPU; larger requests raise before any launch).
    Calls that overlap on one GPU share that scratch and race.  The span
    tables are not checked here (no host copy): the caller guarantees them."""
    import torch
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _need(q, "q", (B, Hq, d), torch.bfloat16, dev)
    _need(k, "k", tuple(k.shape), torch.bfloat16, dev)
    _need(v, "v", tuple(k.shape), torch.bfloat16, dev)
    _need(span_ptr, "span_ptr", (B + 1,), torch.int32, dev)
    _need(spans, "spans", tuple(spans.shape), torch.int32, dev)
    _need(o, "o", (B, Hq, d), torch.bfloat16, dev)
    _need(lse, "lse", (B, Hq), torch.float32, dev)
    need, _ = decode_ws_bytes(B, Hq, d, max_len, n_splits)
    if need > DECODE_SCRATCH_BYTES:
        raise ValueError(f"the decode partials need {need} bytes, more than the {DECODE_SCRATCH_BYTES}-byte "
                         "scratch of the allocation-free call")
    _check("tree_decode_splitkv_noalloc", load_library().tree_decode_splitkv_noalloc(
        TA_BF16, _ptr(q), _ptr(k), _ptr(v), _ptr(span_ptr), _ptr(spans), B, Hq, Hkv, d, int(max_len),
        float(scale), int(n_splits), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse
