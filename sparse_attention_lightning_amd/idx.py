"""Python binding of the C-ABI in ``include/idx.h`` (argument marshalling only).

The functions carry the C names.  They take torch tensors that already live on
the GPU, check dtype, device and layout (refusing, for example, int64 slot
tables or non-contiguous planes), pass raw device pointers and the current HIP
stream to ``libidx.so``, and raise :class:`IdxError` with the library's message
when it refuses a call.  Every step of the computation runs in the library's
HIP kernels; if the library is missing this module raises instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

import torch

LIB_PATH = Path(__file__).resolve().parent / "libidx.so"

IDX_OK, IDX_E_NULL, IDX_E_FORMAT, IDX_E_SHAPE, IDX_E_PACK = 0, -1, -2, -3, -4
IDX_E_TOPK, IDX_E_LAUNCH, IDX_E_ALIGN, IDX_E_MODE = -5, -6, -7, -8
IDX_K_BF16, IDX_K_FP8_E4M3, IDX_K_NVFP4 = 0, 1, 2
IDX_SCORE_MAX, IDX_SCORE_LSE = 0, 1
IDX_MAX_BLOCKS = 8192
IDX_MAX_REQ = 8192
IDX_MAX_REQ_ROWS = 65536
IDX_MAX_ROWS = 1 << 24
IDX_NOALLOC_MAX_SCORES = 4 << 20
IDX_ATTN_MAX_ROWS = 64
IDX_ATTN_MAX_DRAFT = 16
IDX_ATTN_MAX_IDS = 1024
IDX_ATTN_MAX_SPLITS = 64
IDX_FP4_FUSED_MAX_KEYS = 1024
EXPORTS = ("idx_fp4_store", "idx_score_packed", "idx_block_topk", "idx_step", "idx_last_error",
           "idx_step_noalloc", "idx_probe_read", "idx_sparse_attn", "idx_sparse_attn_workspace",
           "idx_score_packed_fp4", "idx_step_fp4")


class IdxError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class IdxParams(C.Structure):
    """Mirror of ``idx_params``."""
    _fields_ = [
        ("k_format", C.c_int32), ("n_req", C.c_int32), ("n_slot_rows", C.c_int32),
        ("packed_queries", C.c_int32), ("gqa", C.c_int32), ("head_dim", C.c_int32),
        ("block_size", C.c_int32), ("max_blocks", C.c_int32), ("topk", C.c_int32),
        ("init_blocks", C.c_int32), ("local_blocks", C.c_int32), ("score_mode", C.c_int32),
        ("sm_scale", C.c_float), ("reserved", C.c_int32),
        ("n_pages", C.c_int64),
        ("q", C.c_void_p), ("k", C.c_void_p), ("k_scale", C.c_void_p),
        ("req_slot", C.c_void_p), ("block_table", C.c_void_p), ("row_len", C.c_void_p),
        ("block_scores", C.c_void_p), ("topk_ids", C.c_void_p), ("topk_scores", C.c_void_p),
    ]


class IdxFp4NewKeys(C.Structure):
    """Mirror of ``idx_fp4_new_keys``."""
    _fields_ = [("staging_bf16", C.c_void_p), ("n_tokens", C.c_int64), ("staging_row_stride", C.c_int64),
                ("slot_mapping", C.c_void_p)]


class IdxAttnParams(C.Structure):
    """Mirror of ``idx_attn_params``."""
    _fields_ = [
        ("n_req", C.c_int32), ("n_slot_rows", C.c_int32), ("packed_queries", C.c_int32),
        ("kv_heads", C.c_int32), ("q_per_kv", C.c_int32), ("head_dim", C.c_int32),
        ("block_size", C.c_int32), ("max_blocks", C.c_int32), ("topk", C.c_int32),
        ("sm_scale", C.c_float), ("kv_format", C.c_int32), ("n_pages", C.c_int64),
        ("workspace_bytes", C.c_int64),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("req_slot", C.c_void_p), ("block_table", C.c_void_p), ("row_len", C.c_void_p),
        ("topk_ids", C.c_void_p), ("out", C.c_void_p), ("lse", C.c_void_p), ("workspace", C.c_void_p),
    ]


_lib: C.CDLL | None = None


def load(path: Path | str | None = None) -> C.CDLL:
    """Load ``libidx.so``; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"HIP library {p} is missing: build it with __graft_entry__.build()")
    lib = C.CDLL(str(p))
    for name in ("idx_score_packed", "idx_block_topk", "idx_step", "idx_step_noalloc"):
        fn = getattr(lib, name)
        fn.argtypes = [C.POINTER(IdxParams), C.c_void_p]
        fn.restype = C.c_int
    for name in ("idx_score_packed_fp4", "idx_step_fp4"):
        fn = getattr(lib, name)
        fn.argtypes = [C.POINTER(IdxParams), C.POINTER(IdxFp4NewKeys), C.c_void_p]
        fn.restype = C.c_int
    lib.idx_fp4_store.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_int64, C.c_void_p]
    lib.idx_fp4_store.restype = C.c_int
    lib.idx_last_error.argtypes = []
    lib.idx_last_error.restype = C.c_char_p
    lib.idx_probe_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int32, C.c_int32,
                                   C.c_void_p, C.c_int32, C.c_void_p]
    lib.idx_probe_read.restype = C.c_int
    lib.idx_sparse_attn.argtypes = [C.POINTER(IdxAttnParams), C.c_void_p]
    lib.idx_sparse_attn.restype = C.c_int
    lib.idx_sparse_attn_workspace.argtypes = [C.POINTER(IdxAttnParams)]
    lib.idx_sparse_attn_workspace.restype = C.c_int64
    if path is None:
        _lib = lib
    return lib


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(rc: int, lib: C.CDLL) -> None:
    if rc != IDX_OK:
        raise IdxError(rc, lib.idx_last_error().decode())


def _dev(t: torch.Tensor | None, name: str, dtypes, optional: bool = False) -> int | None:
    if t is None:
        if optional:
            return None
        raise TypeError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_K_DTYPES = {
    IDX_K_BF16: (torch.bfloat16,),
    IDX_K_FP8_E4M3: (torch.float8_e4m3fn, torch.uint8),
    IDX_K_NVFP4: (torch.uint8,),
}
_ROW_BYTES = {IDX_K_BF16: 256, IDX_K_FP8_E4M3: 128, IDX_K_NVFP4: 64}


def make_params(*, k_format: int, q: torch.Tensor, k: torch.Tensor | None,
                k_scale: torch.Tensor | None, req_slot: torch.Tensor,
                block_table: torch.Tensor | None, row_len: torch.Tensor,
                block_scores: torch.Tensor | None, topk_ids: torch.Tensor | None,
                topk_scores: torch.Tensor | None, packed_queries: int, gqa: int, topk: int,
                init_blocks: int, local_blocks: int, max_blocks: int | None = None,
                n_slot_rows: int | None = None, n_pages: int | None = None,
                score_mode: int = IDX_SCORE_MAX, sm_scale: float = 0.0) -> IdxParams:
    """Build the parameter block from tensors (sizes read from their shapes
    unless given).  ``score_mode`` IDX_SCORE_LSE takes ``sm_scale``.
    ``block_scores`` may be None for :func:`idx_step_noalloc` (which keeps
    them itself; then ``max_blocks`` comes from ``block_table`` or must be
    given).  The returned object keeps the tensors alive."""
    if k_format not in _K_DTYPES:
        raise ValueError(f"unknown k_format {k_format}")
    p = IdxParams()
    p.k_format = k_format
    p.packed_queries = packed_queries
    p.gqa = gqa
    p.head_dim = 128
    p.block_size = 128
    p.topk = topk
    p.init_blocks = init_blocks
    p.local_blocks = local_blocks
    p.score_mode = score_mode
    p.sm_scale = sm_scale
    p.q = _dev(q, "q", (torch.bfloat16,), optional=True)
    p.k = _dev(k, "k", _K_DTYPES[k_format], optional=True)
    p.k_scale = _dev(k_scale, "k_scale", (torch.uint8,), optional=True)
    p.req_slot = _dev(req_slot, "req_slot", (torch.int32,))
    p.block_table = _dev(block_table, "block_table", (torch.int32,), optional=True)
    p.row_len = _dev(row_len, "row_len", (torch.int32,))
    p.block_scores = _dev(block_scores, "block_scores", (torch.float32,), optional=True)
    p.topk_ids = _dev(topk_ids, "topk_ids", (torch.int32,), optional=True)
    p.topk_scores = _dev(topk_scores, "topk_scores", (torch.float32,), optional=True)
    p.n_req = req_slot.numel()
    if max_blocks is None:
        if block_table is not None:
            max_blocks = block_table.shape[-1]
        elif block_scores is not None:
            max_blocks = block_scores.numel() // max(1, p.n_req * packed_queries * gqa)
        else:
            raise ValueError("max_blocks is needed when neither block_table nor block_scores is given")
    p.max_blocks = max_blocks
    if n_slot_rows is None:
        n_slot_rows = block_table.shape[0] if block_table is not None else 0
    p.n_slot_rows = n_slot_rows
    if n_pages is None:
        n_pages = (k.numel() * k.element_size()) // (128 * _ROW_BYTES[k_format]) if k is not None else 0
    p.n_pages = n_pages
    rows = p.n_req * packed_queries * gqa
    if row_len.numel() != p.n_req * packed_queries:
        raise ValueError("row_len must have n_req * packed_queries entries")
    if block_scores is not None and block_scores.numel() < rows * max_blocks:
        raise ValueError("block_scores is smaller than n_req * P * H * max_blocks")
    if q is not None and q.numel() < rows * 128:
        raise ValueError("q is smaller than n_req * P * H * 128")
    if block_table is not None and block_table.numel() < n_slot_rows * max_blocks:
        raise ValueError("block_table is smaller than n_slot_rows * max_blocks")
    if k is not None and k.numel() * k.element_size() < n_pages * 128 * _ROW_BYTES[k_format]:
        raise ValueError("k is smaller than n_pages pages")
    if k_format == IDX_K_NVFP4 and k_scale is not None and k_scale.numel() < n_pages * 128 * 8:
        raise ValueError("k_scale is smaller than n_pages pages")
    for t, n in ((topk_ids, "topk_ids"), (topk_scores, "topk_scores")):
        if t is not None and t.numel() < rows * topk:
            raise ValueError(f"{n} is smaller than n_req * P * H * topk")
    p._keep = (q, k, k_scale, req_slot, block_table, row_len, block_scores, topk_ids, topk_scores)
    return p


def idx_score_packed(p: IdxParams, stream=None) -> None:
    lib = load()
    _check(lib.idx_score_packed(C.byref(p), _stream(stream)), lib)


def idx_block_topk(p: IdxParams, stream=None) -> None:
    lib = load()
    _check(lib.idx_block_topk(C.byref(p), _stream(stream)), lib)


def idx_step(p: IdxParams, stream=None) -> None:
    lib = load()
    _check(lib.idx_step(C.byref(p), _stream(stream)), lib)


def make_new_keys(staging: torch.Tensor, slot_mapping: torch.Tensor) -> IdxFp4NewKeys:
    """The step's new NVFP4 keys: ``staging`` bf16 [n_tokens, >=128] (row
    stride from the tensor) and ``slot_mapping`` int64 [n_tokens]."""
    if staging.dim() != 2 or staging.shape[1] < 128 or staging.stride(1) != 1:
        raise ValueError("staging must be [n_tokens, >=128] with unit element stride")
    if staging.device.type != "cuda" or staging.dtype != torch.bfloat16:
        raise TypeError("staging must be a bf16 GPU tensor")
    _dev(slot_mapping, "slot_mapping", (torch.int64,))
    if slot_mapping.numel() != staging.shape[0]:
        raise ValueError("slot_mapping needs one entry per staging row")
    nk = IdxFp4NewKeys(staging.data_ptr(), staging.shape[0], staging.stride(0), slot_mapping.data_ptr())
    nk._keep = (staging, slot_mapping)
    return nk


def idx_score_packed_fp4(p: IdxParams, keys: IdxFp4NewKeys, stream=None) -> None:
    """idx_fp4_store of ``keys`` into p's NVFP4 planes, then idx_score_packed
    (one launch when the score kernel takes the keys)."""
    lib = load()
    _check(lib.idx_score_packed_fp4(C.byref(p), C.byref(keys), _stream(stream)), lib)


def idx_step_fp4(p: IdxParams, keys: IdxFp4NewKeys, stream=None) -> None:
    """idx_score_packed_fp4 then idx_block_topk."""
    lib = load()
    _check(lib.idx_step_fp4(C.byref(p), C.byref(keys), _stream(stream)), lib)


def idx_step_noalloc(p: IdxParams, stream=None) -> None:
    """idx_step with the block scores kept in the library's own device array
    (``p`` built with ``block_scores=None``); allocates nothing."""
    lib = load()
    _check(lib.idx_step_noalloc(C.byref(p), _stream(stream)), lib)


def idx_probe_read(base: torch.Tensor, unit_bytes: int, units: torch.Tensor | None = None,
                   n_units: int | None = None, nt: bool = False, sink: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Measurement aid: stream ``base`` (a contiguous GPU tensor viewed as
    units of ``unit_bytes``) unit by unit, in the order of ``units`` (int32
    unit ids) or in address order.  Returns the sink words."""
    lib = load()
    if base.device.type != "cuda" or not base.is_contiguous():
        raise ValueError("base must be a contiguous GPU tensor")
    n_base = base.numel() * base.element_size() // unit_bytes
    up = None
    if units is not None:
        up = _dev(units, "units", (torch.int32,))
        n_units = units.numel() if n_units is None else n_units
    elif n_units is None:
        n_units = n_base
    if sink is None:
        sink = torch.empty(4096, dtype=torch.int32, device=base.device)
    rc = lib.idx_probe_read(base.data_ptr(), n_base, up, n_units, unit_bytes, int(nt), sink.data_ptr(),
                            sink.numel(), _stream(stream))
    _check(rc, lib)
    return sink


def idx_fp4_store(staging: torch.Tensor, slot_mapping: torch.Tensor, payload: torch.Tensor,
                  scales: torch.Tensor, stream=None) -> None:
    """Quantize ``staging`` (bf16 [n_tokens, >=128], row stride from the
    tensor) into ``payload`` (uint8 [n_slots, 64]) and ``scales`` (uint8
    [n_slots, 8]) at ``slot_mapping`` (int64 [n_tokens])."""
    lib = load()
    if staging.dim() != 2 or staging.shape[1] < 128 or staging.stride(1) != 1:
        raise ValueError("staging must be [n_tokens, >=128] with unit element stride")
    if staging.device.type != "cuda" or staging.dtype != torch.bfloat16:
        raise TypeError("staging must be a bf16 GPU tensor")
    _dev(slot_mapping, "slot_mapping", (torch.int64,))
    _dev(payload, "payload", (torch.uint8,))
    _dev(scales, "scales", (torch.uint8,))
    n_slots = payload.shape[0]
    if payload.shape != (n_slots, 64) or scales.shape != (n_slots, 8):
        raise ValueError("payload must be [n_slots, 64] and scales [n_slots, 8]")
    if slot_mapping.numel() != staging.shape[0]:
        raise ValueError("slot_mapping needs one entry per staging row")
    rc = lib.idx_fp4_store(staging.data_ptr(), staging.shape[0], staging.stride(0),
                           slot_mapping.data_ptr(), payload.data_ptr(), scales.data_ptr(),
                           n_slots, _stream(stream))
    _check(rc, lib)


def make_attn_params(*, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, req_slot: torch.Tensor,
                     block_table: torch.Tensor, row_len: torch.Tensor, topk_ids: torch.Tensor,
                     out: torch.Tensor, lse: torch.Tensor, sm_scale: float,
                     workspace: torch.Tensor | None = None, kv_format: int | None = None) -> IdxAttnParams:
    """Parameter block of the sparse attention from tensors: q [R*P, H, G,
    128] bf16, k [n_pages, H, 128, 128] and v [n_pages, H, 4, 128 dims, 32
    tokens] both bf16 or both fp8 e4m3 (float8_e4m3fn, or uint8 with
    ``kv_format`` given), topk_ids [R*P*H, topk] (or [R*P, H, topk]) int32,
    out like q, lse [R*P, H, G] fp32.  Without ``workspace`` one of the size
    the library asks for is allocated here (kept alive by the returned
    object)."""
    if q.dim() != 4 or q.shape[-1] != 128:
        raise ValueError("q must be [R*P, H, G, 128]")
    if k.dim() != 4 or k.shape[2:] != (128, 128) or v.shape != (k.shape[0], k.shape[1], 4, 128, 32):
        raise ValueError("k must be [n_pages, H, 128, 128] and v [n_pages, H, 4, 128, 32]")
    p = IdxAttnParams()
    n_req = req_slot.numel()
    rows, H, G = q.shape[0], q.shape[1], q.shape[2]
    if n_req == 0 or rows % n_req:
        raise ValueError("q rows must be n_req * packed_queries")
    P = rows // n_req
    if k.shape[1] != H:
        raise ValueError("k and q disagree on kv_heads")
    if row_len.numel() != rows:
        raise ValueError("row_len must have n_req * packed_queries entries")
    topk = topk_ids.numel() // max(1, rows * H)
    if topk_ids.numel() != rows * H * topk or out.shape != q.shape or lse.shape != q.shape[:3]:
        raise ValueError("topk_ids, out or lse has the wrong shape")
    p.n_req, p.packed_queries, p.kv_heads, p.q_per_kv = n_req, P, H, G
    p.head_dim = p.block_size = 128
    p.n_slot_rows, p.max_blocks = block_table.shape[0], block_table.shape[1]
    p.topk, p.sm_scale, p.n_pages = topk, sm_scale, k.shape[0]
    if kv_format is None:
        kv_format = IDX_K_FP8_E4M3 if k.dtype == torch.float8_e4m3fn else IDX_K_BF16
    if kv_format not in (IDX_K_BF16, IDX_K_FP8_E4M3) or v.dtype != k.dtype:
        raise ValueError("k and v must share one format: bf16 or fp8 e4m3")
    p.kv_format = kv_format
    p.q = _dev(q, "q", (torch.bfloat16,))
    p.k = _dev(k, "k", _K_DTYPES[kv_format])
    p.v = _dev(v, "v", _K_DTYPES[kv_format])
    p.req_slot = _dev(req_slot, "req_slot", (torch.int32,))
    p.block_table = _dev(block_table, "block_table", (torch.int32,))
    p.row_len = _dev(row_len, "row_len", (torch.int32,))
    p.topk_ids = _dev(topk_ids, "topk_ids", (torch.int32,))
    p.out = _dev(out, "out", (torch.bfloat16,))
    p.lse = _dev(lse, "lse", (torch.float32,))
    if workspace is None:
        need = idx_sparse_attn_workspace(p)
        if need > 0:
            workspace = torch.empty((need + 15) // 16 * 4, dtype=torch.float32, device=q.device)
    p.workspace = _dev(workspace, "workspace", (torch.float32, torch.uint8), optional=True)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p._keep = (q, k, v, req_slot, block_table, row_len, topk_ids, out, lse, workspace)
    return p


def idx_sparse_attn_workspace(p: IdxAttnParams) -> int:
    lib = load()
    n = lib.idx_sparse_attn_workspace(C.byref(p))
    if n < 0:
        raise IdxError(int(n), lib.idx_last_error().decode())
    return int(n)


def idx_sparse_attn(p: IdxAttnParams, stream=None) -> None:
    lib = load()
    _check(lib.idx_sparse_attn(C.byref(p), _stream(stream)), lib)
