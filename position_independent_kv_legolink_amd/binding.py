"""ctypes binding of libpiclink.so (include/piclink.h): argument marshalling only.

Every step of the link path runs in the library: page allocation, planning,
the scatter, attention and merge kernels. This module turns torch tensors into
device pointers and the current torch stream into a hipStream_t, and raises
on any non-OK status. PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libpiclink.so")

PIC_OK = 0
STATUS_NAMES = {-1: "PIC_ERR_INVALID", -2: "PIC_ERR_OOM", -3: "PIC_ERR_NOT_FOUND", -4: "PIC_ERR_EXISTS",
                -5: "PIC_ERR_DEVICE", -6: "PIC_ERR_WORKSPACE", -7: "PIC_ERR_STATE"}
DTYPES = {"bf16": 0, "f32": 1}

EXPORTS = ["pic_store_sizes", "pic_store_create", "pic_store_destroy", "pic_store_chunk",
           "pic_store_chunk_pages", "pic_store_release", "pic_store_evict", "pic_store_usage", "pic_store_stats",
           "pic_link_plan",
           "pic_plan_info", "pic_plan_export", "pic_plan_upload", "pic_link_attend", "pic_link_attend_layer",
           "pic_link_attend_static", "pic_link_decode", "pic_forward_workspace", "pic_link_forward", "pic_linear",
           "pic_rmsnorm",
           "pic_plan_free",
           "pic_profile_enable", "pic_profile_read", "pic_last_error"]


class PicError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class StoreConfig(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("max_position", ctypes.c_int32),
                ("key_layout", ctypes.c_int32), ("compile_offset", ctypes.c_int32),
                ("num_layers", ctypes.c_int32)]


# how stored keys carry position: pre-RoPE, or rotated at their position inside their segment
KEY_LAYOUTS = {"position_free": 0, "segment_rope": 1}


class ModelConfig(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("norm_eps", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("mlp_norm", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p)]


class Request(ctypes.Structure):
    _fields_ = [("has_prefix", ctypes.c_int32), ("prefix_id", ctypes.c_uint64),
                ("chunk_ids", ctypes.POINTER(ctypes.c_uint64)), ("n_chunks", ctypes.c_int32),
                ("suffix_len", ctypes.c_int32)]


class LinkOptions(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("block_level", ctypes.c_int32), ("pos_offset", ctypes.c_int32),
                ("recompute_all", ctypes.c_int32), ("split_pages", ctypes.c_int32),
                ("rope_keys", ctypes.c_int32), ("decode", ctypes.c_int32)]


class StoreUsage(ctypes.Structure):
    _fields_ = [("pages_total", ctypes.c_int64), ("pages_free", ctypes.c_int64), ("pages_chunks", ctypes.c_int64),
                ("pages_plans_only", ctypes.c_int64), ("chunks", ctypes.c_int64), ("plans", ctypes.c_int64),
                ("evictions", ctypes.c_int64)]


class PlanSizes(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("pages", ctypes.c_int64), ("private_pages", ctypes.c_int64),
                ("cow_pages", ctypes.c_int64), ("work_items", ctypes.c_int64),
                ("split_items", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("requests", ctypes.c_int64), ("rotated_pages", ctypes.c_int64), ("decode_items", ctypes.c_int64),
                ("table_bytes", ctypes.c_int64), ("partial_bytes", ctypes.c_int64),
                ("rotated_key_bytes", ctypes.c_int64), ("decode_partial_bytes", ctypes.c_int64)]


_lib = None


def lib():
    """Load libpiclink.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it first (python -c "
                               "'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIBRARY)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        P = ctypes.POINTER
        sig = {
            "pic_store_sizes": [P(StoreConfig), P(i64), P(i64)],
            "pic_store_create": [P(StoreConfig), vp, vp, vp, vp, P(vp)],
            "pic_store_destroy": [vp],
            "pic_store_chunk": [vp, u64, vp, vp, i32, vp],
            "pic_store_chunk_pages": [vp, u64, vp, i32, P(i32), P(i32)],
            "pic_store_release": [vp, u64],
            "pic_store_stats": [vp, P(i32), P(i32), P(i32)],
            "pic_store_evict": [vp, i32, P(i32)],
            "pic_store_usage": [vp, P(StoreUsage)],
            "pic_link_plan": [vp, P(Request), i32, P(LinkOptions), P(vp)],
            "pic_plan_info": [vp, P(PlanSizes)],
            "pic_plan_export": [vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "pic_plan_upload": [vp, vp, vp, i64, vp],
            "pic_link_attend": [vp, vp, vp, vp, vp, vp, vp, vp, i64, vp],
            "pic_link_attend_static": [vp, vp, vp, vp, vp, vp, vp, vp],
            "pic_link_attend_layer": [vp, vp, i32, vp, vp, vp, vp, vp, vp, i64, vp],
            "pic_forward_workspace": [vp, vp, P(ModelConfig), P(i64)],
            "pic_link_forward": [vp, vp, P(ModelConfig), vp, vp, vp, i64, vp],
            "pic_linear": [vp, vp, vp, i32, i32, i32, i32, vp, vp],
            "pic_rmsnorm": [vp, vp, vp, i32, i32, ctypes.c_float, vp],
            "pic_link_decode": [vp, vp, vp, vp, vp, vp, vp, vp, i64, vp],
            "pic_plan_free": [vp, vp],
            "pic_profile_enable": [vp, i32],
            "pic_profile_read": [vp, P(ctypes.c_double), P(i32)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        L.pic_last_error.argtypes = []
        L.pic_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != PIC_OK:
        raise PicError(status, lib().pic_last_error().decode())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_device(t, what):
    """Device memory the kernels read or write: a host tensor here would hand the GPU a host
    address, so it is refused before any library call."""
    if t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous device tensor")


def _nbytes(t):
    return t.numel() * t.element_size()


@dataclass
class LinkRequest:
    chunk_ids: list
    suffix_len: int = 0
    prefix_id: int | None = None


class Store:
    """Paged chunk-KV store over caller-owned torch device pools.

    With ``device=None`` the store holds metadata only (host planning, tests
    without a GPU). ``key_layout`` is "position_free" (stored keys are pre-RoPE)
    or "segment_rope" (a chunk's token j holds its key rotated at position
    ``compile_offset + j``: 0 for a chunk compiled from position 0, 4 for
    LegoLink-0's four dummy tokens).
    """

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, dtype,
                 rope_theta, max_position, device="cuda", key_layout="position_free", compile_offset=0,
                 num_layers=1):
        if key_layout not in KEY_LAYOUTS:
            raise ValueError(f"key_layout must be one of {sorted(KEY_LAYOUTS)}")
        self.cfg = StoreConfig(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, DTYPES[dtype],
                               float(rope_theta), max_position, KEY_LAYOUTS[key_layout], int(compile_offset),
                               int(num_layers))
        self.num_layers = max(1, int(num_layers))
        self.key_layout = key_layout
        self.dtype = dtype
        self.device = device
        self.k_pool = self.v_pool = self.rope_table = None
        L = lib()
        if device is not None:
            import torch
            pool_bytes, rope_bytes = ctypes.c_int64(), ctypes.c_int64()
            _check(L.pic_store_sizes(ctypes.byref(self.cfg), ctypes.byref(pool_bytes), ctypes.byref(rope_bytes)))
            tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
            shape = (num_pages, num_kv_heads, page_size, head_dim)
            if self.num_layers > 1:
                shape = (self.num_layers,) + shape
            self.k_pool = torch.empty(shape, dtype=tdt, device=device)
            self.v_pool = torch.empty(shape, dtype=tdt, device=device)
            self.rope_table = torch.empty((max_position, head_dim), dtype=torch.float32, device=device)
            assert self.k_pool.numel() * self.k_pool.element_size() == pool_bytes.value
            assert self.rope_table.numel() * 4 == rope_bytes.value
        h = ctypes.c_void_p()
        _check(L.pic_store_create(ctypes.byref(self.cfg), _ptr(self.k_pool), _ptr(self.v_pool),
                                  _ptr(self.rope_table), _stream() if device is not None else None,
                                  ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _check(lib().pic_store_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().pic_store_destroy(self.handle)
        except Exception:
            pass

    def store_chunk(self, chunk_id: int, k=None, v=None, n_tokens: int | None = None):
        """k, v: device tensors [n][Hkv][d] ([num_layers][n][Hkv][d] for a multi-layer store) of the
        store dtype, keys in the store's key form; or n_tokens only."""
        if k is not None:
            n_tokens = k.shape[1] if self.num_layers > 1 else k.shape[0]
            exp = (n_tokens, self.cfg.num_kv_heads, self.cfg.head_dim)
            if self.num_layers > 1:
                exp = (self.num_layers,) + exp
            if tuple(k.shape) != exp or tuple(v.shape) != exp or not k.is_contiguous() or not v.is_contiguous():
                raise ValueError(f"chunk K/V must be contiguous {exp}")
            if k.dtype != self.k_pool.dtype or v.dtype != self.k_pool.dtype:
                raise ValueError("chunk K/V dtype differs from the store's")
            _on_device(k, "chunk K")
            _on_device(v, "chunk V")
        _check(lib().pic_store_chunk(self.handle, chunk_id, _ptr(k), _ptr(v), int(n_tokens),
                                     _stream() if k is not None else None))

    def chunk_pages(self, chunk_id: int):
        n, t = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pic_store_chunk_pages(self.handle, chunk_id, None, 0, ctypes.byref(n), ctypes.byref(t)))
        out = np.zeros(n.value, dtype=np.int32)
        _check(lib().pic_store_chunk_pages(self.handle, chunk_id, out.ctypes.data_as(ctypes.c_void_p), n.value,
                                           ctypes.byref(n), ctypes.byref(t)))
        return out, t.value

    def release(self, chunk_id: int):
        _check(lib().pic_store_release(self.handle, chunk_id))

    def stats(self):
        f, c, p = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pic_store_stats(self.handle, ctypes.byref(f), ctypes.byref(c), ctypes.byref(p)))
        return dict(free_pages=f.value, chunks=c.value, plans=p.value)

    def evict(self, target_free_pages: int) -> int:
        """Release least recently used chunks until target_free_pages pages are free; returns how many."""
        n = ctypes.c_int32()
        _check(lib().pic_store_evict(self.handle, int(target_free_pages), ctypes.byref(n)))
        return n.value

    def usage(self):
        u = StoreUsage()
        _check(lib().pic_store_usage(self.handle, ctypes.byref(u)))
        return {f: getattr(u, f) for f, _ in StoreUsage._fields_}

    def link_plan(self, requests, *, k=0, block_level=False, pos_offset=0, recompute_all=False,
                  split_pages=0, rope_keys=0, decode=0):
        n = len(requests)
        reqs = (Request * max(n, 1))()
        keep = []
        for i, r in enumerate(requests):
            ids = (ctypes.c_uint64 * max(len(r.chunk_ids), 1))(*[int(c) for c in r.chunk_ids])
            keep.append(ids)
            reqs[i] = Request(0 if r.prefix_id is None else 1, 0 if r.prefix_id is None else int(r.prefix_id),
                              ctypes.cast(ids, ctypes.POINTER(ctypes.c_uint64)), len(r.chunk_ids),
                              int(r.suffix_len))
        opts = LinkOptions(int(k), int(bool(block_level)), int(pos_offset), int(bool(recompute_all)),
                           int(split_pages), int(rope_keys), int(decode))
        h = ctypes.c_void_p()
        _check(lib().pic_link_plan(self.handle, reqs, n, ctypes.byref(opts), ctypes.byref(h)))
        return Plan(self, h)

    def profile_enable(self, on=True):
        _check(lib().pic_profile_enable(self.handle, int(bool(on))))

    def profile_read(self):
        ms = (ctypes.c_double * 4)()
        calls = ctypes.c_int32()
        _check(lib().pic_profile_read(self.handle, ms, ctypes.byref(calls)))
        return dict(scatter_ms=ms[0], attention_ms=ms[1], merge_ms=ms[2], rotate_ms=ms[3], calls=calls.value)


class Plan:
    def __init__(self, store: Store, handle):
        self.store = store
        self.handle = handle
        s = PlanSizes()
        _check(lib().pic_plan_info(handle, ctypes.byref(s)))
        self.sizes = {f: getattr(s, f) for f, _ in PlanSizes._fields_}
        self.workspace = None

    @property
    def rows(self):
        return self.sizes["rows"]

    def export(self):
        s = self.sizes
        B = self.store.cfg.page_size
        a = dict(row_pos=np.zeros(s["rows"], np.int32), row_dst=np.zeros(s["rows"], np.int32),
                 block_table=np.zeros(s["pages"], np.int32), pos_map=np.zeros(s["pages"] * B, np.int32),
                 cu_rows=np.zeros(s["requests"] + 1, np.int32), cu_pages=np.zeros(s["requests"] + 1, np.int32),
                 cow_src=np.zeros(s["cow_pages"], np.int32), cow_dst=np.zeros(s["cow_pages"], np.int32))
        P = lambda x: x.ctypes.data_as(ctypes.c_void_p)
        _check(lib().pic_plan_export(self.handle, P(a["row_pos"]), P(a["row_dst"]), P(a["block_table"]),
                                     P(a["pos_map"]), P(a["cu_rows"]), P(a["cu_pages"]), P(a["cow_src"]),
                                     P(a["cow_dst"])))
        return a

    def upload(self, workspace=None):
        """Copy the plan's device tables into ``workspace`` (a uint8 device tensor; allocated if None)."""
        import torch
        if workspace is None:
            workspace = torch.empty(self.sizes["workspace_bytes"], dtype=torch.uint8, device=self.store.device)
        _on_device(workspace, "workspace")
        _check(lib().pic_plan_upload(self.store.handle, self.handle, _ptr(workspace),
                                     _nbytes(workspace), _stream()))
        self.workspace = workspace
        return workspace

    def free(self):
        if self.handle:
            _check(lib().pic_plan_free(self.store.handle, self.handle))
            self.handle = None


def link_attend(store: Store, plan: Plan, q_new, k_new, v_new, out=None, lse=None):
    """Run the link step; returns ``out`` [R][Hq][d] (and fills ``lse`` [R][Hq] if given)."""
    import torch
    c = store.cfg
    R = plan.rows
    tdt = store.k_pool.dtype
    for name, t, h in (("q_new", q_new, c.num_q_heads), ("k_new", k_new, c.num_kv_heads),
                       ("v_new", v_new, c.num_kv_heads)):
        if tuple(t.shape) != (R, h, c.head_dim) or t.dtype != tdt or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {tdt} device tensor of shape {(R, h, c.head_dim)}")
    if out is None:
        out = torch.empty((R, c.num_q_heads, c.head_dim), dtype=tdt, device=q_new.device)
    if tuple(out.shape) != (R, c.num_q_heads, c.head_dim) or out.dtype != tdt:
        raise ValueError("out has the wrong shape or dtype")
    _on_device(out, "out")
    if lse is not None:
        if tuple(lse.shape) != (R, c.num_q_heads) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 tensor [R][Hq]")
        _on_device(lse, "lse")
    if plan.workspace is None:
        # the library copies the plan's tables in itself when the workspace does not hold them
        plan.workspace = torch.empty(plan.sizes["workspace_bytes"], dtype=torch.uint8, device=q_new.device)
    ws = plan.workspace
    _on_device(ws, "workspace")
    _check(lib().pic_link_attend(store.handle, plan.handle, _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(out),
                                 _ptr(lse), _ptr(ws), _nbytes(ws), _stream()))
    return out


STATIC_SCRATCH_BYTES = 64 << 20


def _link_args(store: Store, plan: Plan, q_new, k_new, v_new, out, lse):
    import torch
    c = store.cfg
    R = plan.rows
    tdt = store.k_pool.dtype
    for name, t, h in (("q_new", q_new, c.num_q_heads), ("k_new", k_new, c.num_kv_heads),
                       ("v_new", v_new, c.num_kv_heads)):
        if tuple(t.shape) != (R, h, c.head_dim) or t.dtype != tdt or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {tdt} device tensor of shape {(R, h, c.head_dim)}")
    if out is None:
        out = torch.empty((R, c.num_q_heads, c.head_dim), dtype=tdt, device=q_new.device)
    if tuple(out.shape) != (R, c.num_q_heads, c.head_dim) or out.dtype != tdt:
        raise ValueError("out has the wrong shape or dtype")
    _on_device(out, "out")
    if lse is not None:
        if tuple(lse.shape) != (R, c.num_q_heads) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 tensor [R][Hq]")
        _on_device(lse, "lse")
    return out


def link_attend_static(store: Store, plan: Plan, q_new, k_new, v_new, out=None, lse=None):
    """The link step on the library's static device scratch instead of a workspace
    (pic_link_attend_static: allocates nothing when ``out`` is given). Plans whose workspace
    exceeds STATIC_SCRATCH_BYTES are refused. Returns ``out``."""
    out = _link_args(store, plan, q_new, k_new, v_new, out, lse)
    _check(lib().pic_link_attend_static(store.handle, plan.handle, _ptr(q_new), _ptr(k_new), _ptr(v_new), _ptr(out),
                                        _ptr(lse), _stream()))
    return out


def link_attend_layer(store: Store, plan: Plan, layer: int, q_new, k_new, v_new, out=None, lse=None):
    """The link step on one layer of a multi-layer store; returns ``out``."""
    import torch
    out = _link_args(store, plan, q_new, k_new, v_new, out, lse)
    if plan.workspace is None:
        plan.workspace = torch.empty(plan.sizes["workspace_bytes"], dtype=torch.uint8, device=q_new.device)
    ws = plan.workspace
    _on_device(ws, "workspace")
    _check(lib().pic_link_attend_layer(store.handle, plan.handle, int(layer), _ptr(q_new), _ptr(k_new), _ptr(v_new),
                                       _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), _stream()))
    return out


@dataclass
class Model:
    """Decoder layers around the link step: d_model = num_q_heads * head_dim, the MLP width
    d_ff, the RMSNorm epsilon, and per layer a dict of device bf16 weights attn_norm [d_model],
    w_qkv [(Hq + 2 Hkv) d][d_model], w_o [d_model][Hq d], mlp_norm [d_model],
    w_gate_up [2 d_ff][d_model] (rows alternate 32 gate and 32 up rows), w_down [d_model][d_ff]."""
    d_model: int
    d_ff: int
    norm_eps: float
    layers: list

    def config(self):
        return ModelConfig(int(self.d_model), int(self.d_ff), float(self.norm_eps))

    def weights(self):
        arr = (LayerWeights * len(self.layers))()
        for i, w in enumerate(self.layers):
            for name in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down"):
                t = w[name]
                _on_device(t, name)
                setattr(arr[i], name, t.data_ptr())
        return arr


def forward_workspace_bytes(store: Store, plan: Plan, model: Model) -> int:
    n = ctypes.c_int64()
    cfg = model.config()
    _check(lib().pic_forward_workspace(store.handle, plan.handle, ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def link_forward(store: Store, plan: Plan, model: Model, x, workspace=None):
    """The plan's selected rows through every layer of the store (pic_link_forward): ``x``
    [rows][d_model] bf16 on the device, overwritten with the last layer's output. Returns
    (x, workspace)."""
    import torch
    if len(model.layers) != store.num_layers:
        raise ValueError("one weight set per store layer")
    if tuple(x.shape) != (plan.rows, model.d_model) or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous bf16 tensor of shape {(plan.rows, model.d_model)}")
    _on_device(x, "x")
    need = forward_workspace_bytes(store, plan, model)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _on_device(workspace, "workspace")
    cfg = model.config()
    weights = model.weights()
    _check(lib().pic_link_forward(store.handle, plan.handle, ctypes.byref(cfg), weights, _ptr(x), _ptr(workspace),
                                  _nbytes(workspace), _stream()))
    return x, workspace


def linear(a, w, epilogue=0, residual=None, out=None):
    """out = a w^T (epilogue 0), + residual (1), or SiLU(gate) * up of w's interleaved rows (2);
    bf16 device tensors a [m][k], w [n][k]."""
    import torch
    m, k = a.shape
    n = w.shape[0]
    for name, t in (("a", a), ("w", w)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
        _on_device(t, name)
    if w.shape[1] != k:
        raise ValueError("a and w disagree on k")
    width = n // 2 if epilogue == 2 else n
    if out is None:
        out = torch.empty((m, width), dtype=torch.bfloat16, device=a.device)
    if tuple(out.shape) != (m, width) or out.dtype != torch.bfloat16:
        raise ValueError("out has the wrong shape or dtype")
    _on_device(out, "out")
    if residual is not None:
        if tuple(residual.shape) != (m, n) or residual.dtype != torch.bfloat16 or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous bf16 tensor [m][n]")
        _on_device(residual, "residual")
    _check(lib().pic_linear(_ptr(a), _ptr(w), _ptr(out), m, n, k, int(epilogue), _ptr(residual), _stream()))
    return out


def rmsnorm(x, w, eps, out=None):
    """x / sqrt(mean(x^2) + eps) * w per row, bf16 device tensors."""
    import torch
    rows, dm = x.shape
    for name, t in (("x", x), ("w", w)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
        _on_device(t, name)
    if out is None:
        out = torch.empty_like(x)
    _on_device(out, "out")
    _check(lib().pic_rmsnorm(_ptr(x), _ptr(w), _ptr(out), rows, dm, float(eps), _stream()))
    return out


def link_decode(store: Store, plan: Plan, q, k, v, out=None, lse=None):
    """One decode step after link_attend with the same plan and workspace: every request's new
    token ([n_req][Hq][d] queries, [n_req][Hkv][d] keys and values, pre-RoPE) attends over the
    request's linked cache and itself. Returns ``out`` [n_req][Hq][d]."""
    import torch
    c = store.cfg
    n = plan.sizes["requests"]
    tdt = store.k_pool.dtype
    for name, t, h in (("q", q, c.num_q_heads), ("k", k, c.num_kv_heads), ("v", v, c.num_kv_heads)):
        if tuple(t.shape) != (n, h, c.head_dim) or t.dtype != tdt or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {tdt} device tensor of shape {(n, h, c.head_dim)}")
    if out is None:
        out = torch.empty((n, c.num_q_heads, c.head_dim), dtype=tdt, device=q.device)
    if tuple(out.shape) != (n, c.num_q_heads, c.head_dim) or out.dtype != tdt:
        raise ValueError("out has the wrong shape or dtype")
    _on_device(out, "out")
    if lse is not None:
        if tuple(lse.shape) != (n, c.num_q_heads) or lse.dtype != torch.float32:
            raise ValueError("lse must be a float32 tensor [n_req][Hq]")
        _on_device(lse, "lse")
    if plan.workspace is None:
        raise RuntimeError("upload the plan and run link_attend before link_decode")
    ws = plan.workspace
    _check(lib().pic_link_decode(store.handle, plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                 _ptr(ws), _nbytes(ws), _stream()))
    return out
