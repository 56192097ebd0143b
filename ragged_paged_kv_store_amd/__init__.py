"""Python binding of librpkv.so (include/rpkv.h): argument marshalling only.

Every step of the path (planning, store_kv, attention tiles, split-KV chunks,
the merge) runs in the native library; this module converts torch tensors and
numpy arrays into pointers and sizes, keeps the caller's workspace large enough,
and raises on any non-OK status.  There is no fallback: if the built library is
missing, importing the package raises.

Layouts are those of the C header: q/out [T, Hq, D]; k/v [T, Hkv, D]; one
layer's pools [num_pages * page_size, Hkv, D]; page table [batch, cols] int32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "librpkv.so")

RPKV_OK = 0
STATUS = {0: "RPKV_OK", 1: "RPKV_ERR_INVALID_ARG", 2: "RPKV_ERR_UNSUPPORTED",
          3: "RPKV_ERR_WORKSPACE_TOO_SMALL", 4: "RPKV_ERR_NOT_PREPARED", 5: "RPKV_ERR_HIP",
          6: "RPKV_ERR_CAPACITY"}
BF16, F32 = 0, 1
KERNEL_KINDS = ("store", "prefill", "decode", "merge", "f32", "fused")

# every function include/rpkv.h declares
EXPORTS = (
    "rpkv_status_string", "rpkv_last_error", "rpkv_supports", "rpkv_plan_create",
    "rpkv_plan_destroy", "rpkv_plan_batch", "rpkv_prepare_metadata", "rpkv_workspace_bytes",
    "rpkv_last_indices", "rpkv_plan_get_info", "rpkv_plan_get_items", "rpkv_plan_get_token_list",
    "rpkv_store_kv", "rpkv_attend", "rpkv_forward", "rpkv_timing_enable", "rpkv_timing_collect",
    "rpkv_build_metadata", "rpkv_graph_decode_init", "rpkv_graph_decode_forward",
    "rpkv_prepare_metadata_csr", "rpkv_rewrite_block_table", "rpkv_plan_get_cascade_tree",
    "rpkv_check_slot_mapping", "rpkv_graph_decode_forward_noalloc", "rpkv_plan_summary",
)


class RpkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("max_tokens", ctypes.c_int64),
                ("max_pages_per_req", ctypes.c_int32), ("decode_max_rows", ctypes.c_int32),
                ("split_target", ctypes.c_int32), ("split_min_keys", ctypes.c_int32),
                ("prefix_detect_keys", ctypes.c_int32), ("tiles_per_block", ctypes.c_int32),
                ("check_slots", ctypes.c_int32)]


class PrefixGroup(ctypes.Structure):
    _fields_ = [("first_req", ctypes.c_int32), ("num_reqs", ctypes.c_int32),
                ("prefix_len", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("num_prefill_items", ctypes.c_int32), ("num_decode_items", ctypes.c_int32),
                ("num_cascade_items", ctypes.c_int32), ("num_merge_tokens", ctypes.c_int32),
                ("num_partials", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("decode_chunk", ctypes.c_int32), ("cascade_members", ctypes.c_int32),
                ("plan_host_us", ctypes.c_double), ("num_cascade_levels", ctypes.c_int32),
                ("cascade_depth", ctypes.c_int32), ("num_cascade_level_members", ctypes.c_int32),
                ("tiles_per_block", ctypes.c_int32), ("metadata_bytes", ctypes.c_int64),
                ("metadata_capacity_bytes", ctypes.c_int64), ("buffer_allocations", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class KernelTimes(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64 * 8), ("total_ms", ctypes.c_double * 8)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m ragged_paged_kv_store_amd.build_lib")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    sigs = {
        "rpkv_status_string": (ctypes.c_char_p, [i32]),
        "rpkv_last_error": (ctypes.c_char_p, []),
        "rpkv_supports": (i32, [P(Shape)]),
        "rpkv_plan_create": (i32, [P(Shape), P(vp)]),
        "rpkv_plan_destroy": (None, [vp]),
        "rpkv_plan_batch": (i32, [vp, i32, vp, vp, i32, vp, vp, i32]),
        "rpkv_prepare_metadata": (i32, [vp, i32, vp, vp, vp, i64, i32, vp, vp, i32, vp, sz, vp]),
        "rpkv_workspace_bytes": (i32, [vp, P(sz)]),
        "rpkv_last_indices": (i32, [vp, vp]),
        "rpkv_plan_get_info": (i32, [vp, P(PlanInfo)]),
        "rpkv_plan_get_items": (i32, [vp, i32, vp, i32, P(i32)]),
        "rpkv_plan_get_token_list": (i32, [vp, vp, i32, P(i32)]),
        "rpkv_plan_get_cascade_tree": (i32, [vp, i32, i32, vp, vp, vp, vp]),
        "rpkv_store_kv": (i32, [vp, vp, vp, vp, i64, vp, vp, vp]),
        "rpkv_attend": (i32, [vp, vp, vp, vp, vp, ctypes.c_float, vp]),
        "rpkv_forward": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp]),
        "rpkv_timing_enable": (i32, [vp, i32, i32]),
        "rpkv_timing_collect": (i32, [vp, P(KernelTimes)]),
        "rpkv_build_metadata": (i32, [i32, vp, vp, vp, vp, i64, i32, i32, i64] + [vp] * 7),
        "rpkv_graph_decode_init": (i32, [vp, i32, i32, i32]),
        "rpkv_prepare_metadata_csr": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]),
        "rpkv_rewrite_block_table": (i32, [i32, vp, i64, i32, i32, vp, i64, vp]),
        "rpkv_graph_decode_forward": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, vp,
                                            ctypes.c_float, vp]),
        "rpkv_check_slot_mapping": (i32, [vp, vp, i64]),
        "rpkv_plan_summary": (i32, [vp, ctypes.c_char_p, sz]),
        "rpkv_graph_decode_forward_noalloc": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                    vp, i64, i32, vp, ctypes.c_float, vp]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(st: int) -> None:
    if st != RPKV_OK:
        raise RpkvError(st, lib.rpkv_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(t) -> Optional[int]:
    """Device/host pointer of a torch tensor (or None)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def build_metadata(num_computed, n, block_tables, page_size: int, need_logits=None,
                   max_tokens: Optional[int] = None, out=None, stream=None):
    """rpkv_build_metadata on device tensors (int32 num_computed [B], n [B],
    block_tables [B, stride]; uint8 need_logits [B] or None).  Returns a dict of
    int32 device tensors: query_start_loc [B+1], seq_lens [B], positions and
    slot_mapping [max_tokens], logits_indices [B], counts [2] (N, number of
    logits indices).  `out` may pass preallocated tensors of those names (for
    graph capture); nothing is synchronised."""
    import torch
    B = int(num_computed.shape[0])
    for name, t in (("num_computed", num_computed), ("n", n), ("block_tables", block_tables)):
        if not t.is_cuda or t.dtype != torch.int32 or t.shape[0] != B:
            raise ValueError(f"{name}: int32 device tensor with {B} rows expected")
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables: 2-D with unit column stride expected")
    if need_logits is not None and (need_logits.dtype != torch.uint8 or need_logits.shape[0] != B
                                    or not need_logits.is_cuda):
        raise ValueError("need_logits: uint8 device tensor [B] expected")
    if max_tokens is None:
        max_tokens = int(n.sum().item())
    dev = num_computed.device
    o = dict(out or {})
    shapes = {"query_start_loc": B + 1, "seq_lens": B, "positions": max_tokens,
              "slot_mapping": max_tokens, "logits_indices": max(B, 1), "counts": 2}
    for k, sz in shapes.items():
        if k not in o:
            o[k] = torch.empty(max(sz, 1), dtype=torch.int32, device=dev)
        elif o[k].dtype != torch.int32 or o[k].numel() < sz or not o[k].is_contiguous():
            raise ValueError(f"out[{k}]: contiguous int32 with >= {sz} entries expected")
    st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(lib.rpkv_build_metadata(B, num_computed.data_ptr(), n.data_ptr(),
                                   None if need_logits is None else need_logits.data_ptr(),
                                   block_tables.data_ptr(), block_tables.stride(0),
                                   block_tables.shape[1], page_size, max_tokens,
                                   o["query_start_loc"].data_ptr(), o["seq_lens"].data_ptr(),
                                   o["positions"].data_ptr(), o["slot_mapping"].data_ptr(),
                                   o["logits_indices"].data_ptr(), o["counts"].data_ptr(), st))
    return o


def rewrite_block_table(table, factor: int, stream=None):
    """rpkv_rewrite_block_table: a [B, cols] int32 device table of blocks of
    `factor` kernel pages -> a new [B, cols*factor] table of kernel pages."""
    import torch
    if not (table.is_cuda and table.dtype == torch.int32 and table.dim() == 2 and
            table.stride(1) == 1):
        raise ValueError("table must be a 2-D int32 CUDA tensor with unit column stride")
    B, cols = table.shape
    out = torch.empty((B, cols * factor), dtype=torch.int32, device=table.device)
    _check(lib.rpkv_rewrite_block_table(B, table.data_ptr(), table.stride(0), cols, factor,
                                        out.data_ptr(), out.stride(0), _stream(stream)))
    return out


def supports(**kw) -> Tuple[bool, str]:
    s = make_shape(**kw)
    st = lib.rpkv_supports(ctypes.byref(s))
    return st == RPKV_OK, ("" if st == RPKV_OK else lib.rpkv_last_error().decode())


def make_shape(num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, dtype: int,
               max_batch: int, num_pages: int, max_tokens: int, max_pages_per_req: int,
               decode_max_rows: int = 0, split_target: int = 0, split_min_keys: int = 0,
               prefix_detect_keys: int = 0, tiles_per_block: int = 0,
               check_slots: int = 0) -> Shape:
    return Shape(num_q_heads, num_kv_heads, head_dim, page_size, dtype, max_batch, num_pages,
                 max_tokens, max_pages_per_req, decode_max_rows, split_target, split_min_keys,
                 prefix_detect_keys, tiles_per_block, check_slots)


class Plan:
    """One layer type's plan: prepare once per batch, then store/attend per layer."""

    def __init__(self, **shape_kw):
        self.shape = make_shape(**shape_kw)
        h = ctypes.c_void_p()
        _check(lib.rpkv_plan_create(ctypes.byref(self.shape), ctypes.byref(h)))
        self._h = h
        self.workspace = None      # torch uint8 device tensor, grown on demand
        self._pt = None            # keep the page table alive while prepared
        self.batch = 0
        self.num_tokens = 0

    # The C ABI takes plain pointers; these checks keep tensors of another shape,
    # dtype or device from ever reaching a kernel.
    def _dtype(self):
        import torch
        return torch.bfloat16 if self.shape.dtype == BF16 else torch.float32

    def _check_rows(self, name, t, heads, min_rows):
        if t is None:
            if min_rows > 0:
                raise ValueError(f"{name} is required")
            return
        sh = self.shape
        if not t.is_cuda or t.dtype != self._dtype() or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {self._dtype()} CUDA tensor")
        if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != sh.head_dim:
            raise ValueError(f"{name} must be [tokens, {heads}, {sh.head_dim}], got {tuple(t.shape)}")
        if t.shape[0] < min_rows:
            raise ValueError(f"{name} has {t.shape[0]} rows, the batch has {min_rows} tokens")

    def _check_pool(self, name, t):
        sh = self.shape
        want = sh.num_pages * sh.page_size * sh.num_kv_heads * sh.head_dim
        if t is None or not t.is_cuda or t.dtype != self._dtype() or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {self._dtype()} CUDA tensor")
        if t.numel() != want or t.shape[-1] != sh.head_dim or t.shape[-2] != sh.num_kv_heads:
            raise ValueError(f"{name} must hold [num_pages*page_size, Hkv, D] = "
                             f"[{sh.num_pages * sh.page_size}, {sh.num_kv_heads}, {sh.head_dim}]")

    def _check_slots(self, t, min_rows):
        import torch
        if t is None:
            if min_rows > 0:
                raise ValueError("slot_mapping is required")
            return
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous() or t.dim() != 1:
            raise ValueError("slot_mapping must be a contiguous int32 CUDA vector")
        if t.numel() < min_rows:
            raise ValueError("slot_mapping is shorter than the batch")

    def close(self):
        if getattr(self, "_h", None):
            lib.rpkv_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ per batch
    def plan_host(self, cu_q, cache_seqlens, page_table_cols: int, page_table_host=None,
                  groups: Sequence[Tuple[int, int, int]] = ()):
        """Host-only planning (no device work)."""
        cu = _i32(cu_q)
        sl = _i32(cache_seqlens)
        bs = len(sl)
        pth = None if page_table_host is None else _i32(page_table_host)
        if pth is not None:
            assert pth.shape == (bs, page_table_cols)
        garr = (PrefixGroup * max(len(groups), 1))(*[PrefixGroup(*g) for g in groups])
        _check(lib.rpkv_plan_batch(self._h, bs, cu.ctypes.data, sl.ctypes.data, page_table_cols,
                                   None if pth is None else pth.ctypes.data,
                                   ctypes.cast(garr, ctypes.c_void_p) if groups else None,
                                   len(groups)))
        self.batch = bs

    def prepare(self, cu_q, cache_seqlens, page_table, page_table_host=None,
                groups: Sequence[Tuple[int, int, int]] = (), stream=None):
        """prepare_metadata: plan on the host and upload the work partition.

        page_table: torch int32 device tensor [batch, cols] (row stride = its
        stride(0)).  The workspace is (re)allocated with torch when too small.
        """
        import torch
        cu = _i32(cu_q)
        sl = _i32(cache_seqlens)
        bs = len(sl)
        if not (page_table.is_cuda and page_table.dtype == torch.int32 and
                page_table.dim() == 2 and page_table.stride(1) == 1):
            raise ValueError("page_table must be a 2-D int32 CUDA tensor with unit column stride")
        if page_table.shape[0] < len(cache_seqlens):
            raise ValueError("page_table has fewer rows than the batch")
        cols = page_table.shape[1]
        pth = None if page_table_host is None else _i32(page_table_host)
        garr = (PrefixGroup * max(len(groups), 1))(*[PrefixGroup(*g) for g in groups])
        gptr = ctypes.cast(garr, ctypes.c_void_p) if groups else None
        s = _stream(stream)
        for _ in range(2):
            ws = self.workspace
            st = lib.rpkv_prepare_metadata(
                self._h, bs, cu.ctypes.data, sl.ctypes.data, page_table.data_ptr(),
                page_table.stride(0), cols, None if pth is None else pth.ctypes.data, gptr,
                len(groups), None if ws is None else ws.data_ptr(),
                0 if ws is None else ws.numel(), s)
            if st == 3:  # workspace too small: grow and plan again
                need = ctypes.c_size_t()
                _check(lib.rpkv_workspace_bytes(self._h, ctypes.byref(need)))
                self.workspace = torch.empty(int(need.value * 1.25) + 256, dtype=torch.uint8,
                                             device=page_table.device)
                continue
            _check(st)
            break
        self._pt = page_table
        self.batch = bs
        self.num_tokens = int(cu[-1]) if len(cu) else 0

    def prepare_csr(self, cu_q, page_indptr, last_page_len, page_indices, page_indices_host=None,
                    groups: Sequence[Tuple[int, int, int]] = (), stream=None):
        """prepare_metadata_csr: the page table as FlashInfer's (page_indices [K]
        int32 device tensor, page_indptr [B+1] and last_page_len [B] on the host)."""
        import torch
        cu = _i32(cu_q)
        ip = _i32(page_indptr)
        lp = _i32(last_page_len)
        bs = len(lp)
        if not (page_indices.is_cuda and page_indices.dtype == torch.int32 and
                page_indices.is_contiguous()):
            raise ValueError("page_indices must be a contiguous int32 CUDA tensor")
        if len(ip) != bs + 1 or (bs and page_indices.numel() < int(ip[-1])):
            raise ValueError("page_indptr must have batch+1 entries within page_indices")
        pih = None if page_indices_host is None else _i32(page_indices_host)
        garr = (PrefixGroup * max(len(groups), 1))(*[PrefixGroup(*g) for g in groups])
        gptr = ctypes.cast(garr, ctypes.c_void_p) if groups else None
        s = _stream(stream)
        for _ in range(2):
            ws = self.workspace
            st = lib.rpkv_prepare_metadata_csr(
                self._h, bs, cu.ctypes.data, ip.ctypes.data, lp.ctypes.data,
                page_indices.data_ptr(), None if pih is None else pih.ctypes.data, gptr,
                len(groups), None if ws is None else ws.data_ptr(),
                0 if ws is None else ws.numel(), s)
            if st == 3:
                need = ctypes.c_size_t()
                _check(lib.rpkv_workspace_bytes(self._h, ctypes.byref(need)))
                self.workspace = torch.empty(int(need.value * 1.25) + 256, dtype=torch.uint8,
                                             device=page_indices.device)
                continue
            _check(st)
            break
        self._pt = page_indices
        self.batch = bs
        self.num_tokens = int(cu[-1]) if len(cu) else 0

    def info(self) -> dict:
        inf = PlanInfo()
        _check(lib.rpkv_plan_get_info(self._h, ctypes.byref(inf)))
        return inf.as_dict()

    def summary(self) -> str:
        """One-line text summary of the last planned batch (rpkv_plan_summary)."""
        buf = ctypes.create_string_buffer(512)
        _check(lib.rpkv_plan_summary(self._h, buf, ctypes.sizeof(buf)))
        return buf.value.decode()

    def items(self, kind: int) -> np.ndarray:
        n = ctypes.c_int32()
        _check(lib.rpkv_plan_get_items(self._h, kind, None, 0, ctypes.byref(n)))
        out = np.zeros((max(n.value, 1), 8), np.int32)
        _check(lib.rpkv_plan_get_items(self._h, kind, out.ctypes.data, n.value, ctypes.byref(n)))
        return out[:n.value]

    def token_list(self) -> np.ndarray:
        n = ctypes.c_int32()
        _check(lib.rpkv_plan_get_token_list(self._h, None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib.rpkv_plan_get_token_list(self._h, out.ctypes.data, n.value, ctypes.byref(n)))
        return out[:n.value]

    def cascade_tree(self) -> list:
        """The last plan's shared-prefix levels, parents first: a list of dicts
        {"members": tuple of request indices, "prefix": keys, "parent": index or -1}."""
        inf = self.info()
        nl, nm = inf["num_cascade_levels"], inf["num_cascade_level_members"]
        par = np.zeros(max(nl, 1), np.int32)
        pre = np.zeros(max(nl, 1), np.int32)
        ind = np.zeros(nl + 1, np.int32)
        mem = np.zeros(max(nm, 1), np.int32)
        _check(lib.rpkv_plan_get_cascade_tree(self._h, nl, nm, par.ctypes.data, pre.ctypes.data,
                                              ind.ctypes.data, mem.ctypes.data))
        return [{"members": tuple(int(x) for x in mem[ind[k]:ind[k + 1]]),
                 "prefix": int(pre[k]), "parent": int(par[k])} for k in range(nl)]

    def last_indices(self) -> np.ndarray:
        out = np.zeros(max(self.batch, 1), np.int32)
        _check(lib.rpkv_last_indices(self._h, out.ctypes.data))
        return out[:self.batch]

    def check_slot_mapping(self, slots_host) -> None:
        """rpkv_check_slot_mapping on a host array: raises RpkvError
        (INVALID_ARG) on a duplicate or out-of-range slot."""
        s = _i32(slots_host).reshape(-1)
        _check(lib.rpkv_check_slot_mapping(self._h, s.ctypes.data if s.size else None, s.size))

    def workspace_bytes(self) -> int:
        need = ctypes.c_size_t()
        _check(lib.rpkv_workspace_bytes(self._h, ctypes.byref(need)))
        return int(need.value)

    # ------------------------------------------------------------ per layer
    def store_kv(self, k, v, slot_mapping, k_pool, v_pool, stream=None):
        n = int(slot_mapping.numel()) if slot_mapping is not None else 0
        self._check_slots(slot_mapping, n)
        self._check_rows("k", k, self.shape.num_kv_heads, n)
        self._check_rows("v", v, self.shape.num_kv_heads, n)
        self._check_pool("k_pool", k_pool)
        self._check_pool("v_pool", v_pool)
        _check(lib.rpkv_store_kv(self._h, _ptr(k), _ptr(v), _ptr(slot_mapping),
                                 int(slot_mapping.numel()) if slot_mapping is not None else 0,
                                 _ptr(k_pool), _ptr(v_pool), _stream(stream)))

    def attend(self, q, k_pool, v_pool, out, scale: float, stream=None):
        T = self.num_tokens
        if T > 0:
            self._check_rows("q", q, self.shape.num_q_heads, T)
            self._check_rows("out", out, self.shape.num_q_heads, T)
            self._check_pool("k_pool", k_pool)
            self._check_pool("v_pool", v_pool)
        _check(lib.rpkv_attend(self._h, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                               float(scale), _stream(stream)))

    def forward(self, q, k, v, slot_mapping, k_pool, v_pool, out, scale: float, stream=None):
        T = self.num_tokens
        if T > 0:
            self._check_slots(slot_mapping, T)
            self._check_rows("q", q, self.shape.num_q_heads, T)
            self._check_rows("out", out, self.shape.num_q_heads, T)
            self._check_rows("k", k, self.shape.num_kv_heads, T)
            self._check_rows("v", v, self.shape.num_kv_heads, T)
            self._check_pool("k_pool", k_pool)
            self._check_pool("v_pool", v_pool)
        _check(lib.rpkv_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(slot_mapping),
                                _ptr(k_pool), _ptr(v_pool), _ptr(out), float(scale),
                                _stream(stream)))

    # ---------------------------------------------- graph-capturable decode
    def graph_decode_init(self, max_batch: int, q_len: int, max_seq_len: int):
        _check(lib.rpkv_graph_decode_init(self._h, max_batch, q_len, max_seq_len))
        self._graph = (max_batch, q_len, max_seq_len)

    def graph_decode_forward(self, batch: int, q, k, v, slot_mapping, k_pool, v_pool, seq_lens,
                             page_table, out, scale: float, stream=None):
        """Capturable: every check here is on shapes only (no device reads)."""
        import torch
        if getattr(self, "_graph", None) is None:
            raise RpkvError(4, "graph_decode_init first")
        _, q_len, _ = self._graph
        T = batch * q_len
        self._check_slots(slot_mapping, T)
        self._check_rows("q", q, self.shape.num_q_heads, T)
        self._check_rows("out", out, self.shape.num_q_heads, T)
        self._check_rows("k", k, self.shape.num_kv_heads, T)
        self._check_rows("v", v, self.shape.num_kv_heads, T)
        self._check_pool("k_pool", k_pool)
        self._check_pool("v_pool", v_pool)
        if (not seq_lens.is_cuda or seq_lens.dtype != torch.int32 or seq_lens.numel() < batch
                or not seq_lens.is_contiguous()):
            raise ValueError("seq_lens: contiguous int32 device tensor with >= batch entries")
        if (not page_table.is_cuda or page_table.dtype != torch.int32 or page_table.dim() != 2
                or page_table.shape[0] < batch or page_table.stride(1) != 1):
            raise ValueError("page_table: int32 device tensor [>= batch, cols], unit column stride")
        _check(lib.rpkv_graph_decode_forward(
            self._h, batch, _ptr(q), _ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(k_pool),
            _ptr(v_pool), seq_lens.data_ptr(), page_table.data_ptr(), page_table.stride(0),
            page_table.shape[1], _ptr(out), float(scale), _stream(stream)))

    def graph_decode_forward_noalloc(self, batch: int, q_len: int, max_seq_len: int, q, k, v,
                                     slot_mapping, k_pool, v_pool, seq_lens, page_table, out,
                                     scale: float, stream=None):
        """rpkv_graph_decode_forward_noalloc: the graph-decode step with no
        graph_decode_init and no allocation (partials in the library's fixed
        device array).  Shape checks only (no device reads)."""
        import torch
        T = batch * q_len
        self._check_slots(slot_mapping, T)
        self._check_rows("q", q, self.shape.num_q_heads, T)
        self._check_rows("out", out, self.shape.num_q_heads, T)
        self._check_rows("k", k, self.shape.num_kv_heads, T)
        self._check_rows("v", v, self.shape.num_kv_heads, T)
        self._check_pool("k_pool", k_pool)
        self._check_pool("v_pool", v_pool)
        if (not seq_lens.is_cuda or seq_lens.dtype != torch.int32 or seq_lens.numel() < batch
                or not seq_lens.is_contiguous()):
            raise ValueError("seq_lens: contiguous int32 device tensor with >= batch entries")
        if (not page_table.is_cuda or page_table.dtype != torch.int32 or page_table.dim() != 2
                or page_table.shape[0] < batch or page_table.stride(1) != 1):
            raise ValueError("page_table: int32 device tensor [>= batch, cols], unit column stride")
        _check(lib.rpkv_graph_decode_forward_noalloc(
            self._h, batch, q_len, max_seq_len, _ptr(q), _ptr(k), _ptr(v), _ptr(slot_mapping),
            _ptr(k_pool), _ptr(v_pool), seq_lens.data_ptr(), page_table.data_ptr(),
            page_table.stride(0), page_table.shape[1], _ptr(out), float(scale), _stream(stream)))

    # ------------------------------------------------------- instrumentation
    def timing_enable(self, enable: bool, max_launches: int = 4096):
        _check(lib.rpkv_timing_enable(self._h, 1 if enable else 0, max_launches))

    def timing_collect(self) -> dict:
        kt = KernelTimes()
        _check(lib.rpkv_timing_collect(self._h, ctypes.byref(kt)))
        return {name: (int(kt.launches[i]), float(kt.total_ms[i]))
                for i, name in enumerate(KERNEL_KINDS)}
