"""ctypes binding of the C oracle (test infrastructure only).

Arrays are numpy arrays in host memory.  bf16 data travels as its raw 16-bit
patterns (``uint16``), fp8 and NVFP4 data as bytes (``uint8``).  The functions
mirror the GPU library's entry points with an ``oracle_`` prefix and return the
outputs as new numpy arrays.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

import numpy as np

from . import build as _build

K_BF16, K_FP8_E4M3, K_NVFP4 = 0, 1, 2
BYTES_PER_TOKEN = {K_BF16: 256, K_FP8_E4M3: 128, K_NVFP4: 64}


class OracleParams(C.Structure):
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


class OracleAttnParams(C.Structure):
    _fields_ = [
        ("n_req", C.c_int32), ("n_slot_rows", C.c_int32), ("packed_queries", C.c_int32),
        ("kv_heads", C.c_int32), ("q_per_kv", C.c_int32), ("head_dim", C.c_int32),
        ("block_size", C.c_int32), ("max_blocks", C.c_int32), ("topk", C.c_int32),
        ("sm_scale", C.c_float), ("kv_format", C.c_int32), ("n_pages", C.c_int64),
        ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p),
        ("req_slot", C.c_void_p), ("block_table", C.c_void_p), ("row_len", C.c_void_p),
        ("topk_ids", C.c_void_p), ("out", C.c_void_p), ("lse", C.c_void_p), ("out_abs", C.c_void_p),
    ]


_LIBS: dict[str, C.CDLL] = {}


def load(path: Path | str | None = None) -> C.CDLL:
    """Load (building first if needed) the oracle library at ``path``."""
    path = Path(path) if path is not None else _build.DEFAULT_LIB
    key = str(path)
    if key in _LIBS:
        return _LIBS[key]
    if not path.exists():
        _build.build(path)
    lib = C.CDLL(str(path))
    for name in ("oracle_score_packed", "oracle_block_topk", "oracle_step"):
        fn = getattr(lib, name)
        fn.argtypes = [C.POINTER(OracleParams)]
        fn.restype = C.c_int
    lib.oracle_sparse_attn.argtypes = [C.POINTER(OracleAttnParams)]
    lib.oracle_sparse_attn.restype = C.c_int
    lib.oracle_fp4_store.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_int64]
    lib.oracle_fp4_store.restype = C.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = C.c_int
    lib.oracle_set_threads.argtypes = [C.c_int]
    lib.oracle_set_threads.restype = C.c_int
    lib.oracle_fp8_value.argtypes = [C.c_uint8]
    lib.oracle_fp8_value.restype = C.c_double
    lib.oracle_e2m1_value.argtypes = [C.c_uint8]
    lib.oracle_e2m1_value.restype = C.c_double
    lib.oracle_e4m3_encode.argtypes = [C.c_float]
    lib.oracle_e4m3_encode.restype = C.c_uint8
    lib.oracle_e2m1_encode.argtypes = [C.c_float, C.c_float]
    lib.oracle_e2m1_encode.restype = C.c_uint8
    _LIBS[key] = lib
    return lib


def _ptr(a: np.ndarray | None) -> int | None:
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _arr(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


class Oracle:
    """One loaded oracle library (the product build, or a mutant)."""

    def __init__(self, path: Path | str | None = None):
        self.lib = load(path)

    def threads(self) -> int:
        return self.lib.oracle_threads()

    def set_threads(self, n: int) -> int:
        """Threads for later calls from this thread; returns the count before."""
        return self.lib.oracle_set_threads(n)

    # -- number formats --------------------------------------------------
    def fp8_value(self, code: int) -> float:
        return self.lib.oracle_fp8_value(code)

    def e2m1_value(self, code: int) -> float:
        return self.lib.oracle_e2m1_value(code)

    def e4m3_encode(self, t: float) -> int:
        return self.lib.oracle_e4m3_encode(t)

    def e2m1_encode(self, x: float, s: float) -> int:
        return self.lib.oracle_e2m1_encode(x, s)

    # -- NVFP4 store -------------------------------------------------------
    def fp4_store(self, staging_bits: np.ndarray, slot_mapping: np.ndarray,
                  payload: np.ndarray, scales: np.ndarray) -> None:
        """Quantize ``staging_bits`` (uint16 bf16 patterns, [n_tokens, >=128])
        into ``payload`` ([n_slots, 64] uint8) and ``scales`` ([n_slots, 8]
        uint8) in place."""
        staging_bits = _arr(staging_bits, np.uint16)
        slot_mapping = _arr(slot_mapping, np.int64)
        assert payload.dtype == np.uint8 and scales.dtype == np.uint8
        assert payload.flags["C_CONTIGUOUS"] and scales.flags["C_CONTIGUOUS"]
        n_slots = payload.shape[0]
        assert payload.shape == (n_slots, 64) and scales.shape == (n_slots, 8)
        n_tok = staging_bits.shape[0]
        stride = staging_bits.shape[1] if staging_bits.ndim == 2 else 128
        rc = self.lib.oracle_fp4_store(_ptr(staging_bits), n_tok, stride, _ptr(slot_mapping),
                                       _ptr(payload), _ptr(scales), n_slots)
        if rc:
            raise ValueError(f"oracle_fp4_store refused its arguments or ran out of memory ({rc})")

    # -- scoring and selection ---------------------------------------------
    def _params(self, a: dict, outs: dict) -> OracleParams:
        p = OracleParams()
        for f in ("k_format", "n_req", "n_slot_rows", "packed_queries", "gqa", "max_blocks",
                  "topk", "init_blocks", "local_blocks", "n_pages"):
            setattr(p, f, int(a[f]))
        p.score_mode = int(a.get("score_mode", 0))
        p.sm_scale = float(a.get("sm_scale", 0.0))
        p.head_dim = int(a.get("head_dim", 128))
        p.block_size = int(a.get("block_size", 128))
        p.q = _ptr(a["q"])
        p.k = _ptr(a["k"])
        p.k_scale = _ptr(a.get("k_scale"))
        p.req_slot = _ptr(a["req_slot"])
        p.block_table = _ptr(a["block_table"])
        p.row_len = _ptr(a["row_len"])
        p.block_scores = _ptr(outs["block_scores"])
        p.topk_ids = _ptr(outs["topk_ids"])
        p.topk_scores = _ptr(outs["topk_scores"])
        return p

    @staticmethod
    def _check(a: dict) -> dict:
        a = dict(a)
        a["q"] = _arr(a["q"], np.uint16)
        a["k"] = _arr(a["k"], np.uint16 if a["k_format"] == K_BF16 else np.uint8)
        if a.get("k_scale") is not None:
            a["k_scale"] = _arr(a["k_scale"], np.uint8)
        a["req_slot"] = _arr(a["req_slot"], np.int32)
        a["block_table"] = _arr(a["block_table"], np.int32)
        a["row_len"] = _arr(a["row_len"], np.int32)
        rows = a["n_req"] * a["packed_queries"]
        assert a["q"].size == rows * a["gqa"] * 128, "q shape"
        assert a["row_len"].size == rows and a["req_slot"].size == a["n_req"]
        assert a["block_table"].size == a["n_slot_rows"] * a["max_blocks"]
        bpt = BYTES_PER_TOKEN[a["k_format"]]
        assert a["k"].nbytes == a["n_pages"] * 128 * bpt, "k plane size"
        if a["k_format"] == K_NVFP4:
            assert a["k_scale"].nbytes == a["n_pages"] * 128 * 8, "scale plane size"
        return a

    def _outs(self, a: dict, block_scores: np.ndarray | None = None) -> dict:
        rows = a["n_req"] * a["packed_queries"] * a["gqa"]
        bs = (np.full((rows, a["max_blocks"]), np.nan, np.float32)
              if block_scores is None else _arr(block_scores, np.float32).copy())
        return {"block_scores": bs,
                "topk_ids": np.full((rows, a["topk"]), -7, np.int32),
                "topk_scores": np.full((rows, a["topk"]), np.nan, np.float32)}

    def score_packed(self, **a) -> dict:
        a = self._check(a)
        outs = self._outs(a)
        rc = self.lib.oracle_score_packed(C.byref(self._params(a, outs)))
        if rc:
            raise ValueError(f"oracle_score_packed refused its arguments or ran out of memory ({rc})")
        return {"block_scores": outs["block_scores"]}

    def block_topk(self, block_scores: np.ndarray, **a) -> dict:
        a = self._check(a)
        outs = self._outs(a, block_scores)
        rc = self.lib.oracle_block_topk(C.byref(self._params(a, outs)))
        if rc:
            raise ValueError(f"oracle_block_topk refused its arguments or ran out of memory ({rc})")
        return {"topk_ids": outs["topk_ids"], "topk_scores": outs["topk_scores"]}

    def step(self, **a) -> dict:
        a = self._check(a)
        outs = self._outs(a)
        rc = self.lib.oracle_step(C.byref(self._params(a, outs)))
        if rc:
            raise ValueError(f"oracle_step refused its arguments or ran out of memory ({rc})")
        return outs

    # -- sparse attention over the selected blocks ---------------------------
    def sparse_attn(self, **a) -> dict:
        """out [rows, H, G, 128], lse [rows, H, G] and out_abs (the weighted
        |V| that scales out's rounding error) as float32 arrays."""
        R, P, H, G = a["n_req"], a["packed_queries"], a["kv_heads"], a["q_per_kv"]
        MB, K, n_pages = a["max_blocks"], a["topk"], a["n_pages"]
        kv_format = int(a.get("kv_format", K_BF16))
        q = _arr(a["q"], np.uint16)
        kv_dtype = np.uint16 if kv_format == K_BF16 else np.uint8
        k = _arr(a["k"], kv_dtype)
        v = _arr(a["v"], kv_dtype)
        req_slot = _arr(a["req_slot"], np.int32)
        bt = _arr(a["block_table"], np.int32)
        row_len = _arr(a["row_len"], np.int32)
        ids = _arr(a["topk_ids"], np.int32)
        assert q.size == R * P * H * G * 128 and row_len.size == R * P and req_slot.size == R
        assert bt.size == a["n_slot_rows"] * MB and ids.size == R * P * H * K
        assert k.size == n_pages * H * 128 * 128 and v.size == k.size
        out = np.full((R * P, H, G, 128), np.nan, np.float32)
        lse = np.full((R * P, H, G), np.nan, np.float32)
        oabs = np.full_like(out, np.nan)
        pr = OracleAttnParams()
        for f in ("n_req", "n_slot_rows", "packed_queries", "kv_heads", "q_per_kv", "max_blocks", "topk",
                  "n_pages"):
            setattr(pr, f, int(a[f]))
        pr.head_dim, pr.block_size = 128, 128
        pr.sm_scale = float(a["sm_scale"])
        pr.kv_format = kv_format
        pr.q, pr.k, pr.v = _ptr(q), _ptr(k), _ptr(v)
        pr.req_slot, pr.block_table, pr.row_len, pr.topk_ids = _ptr(req_slot), _ptr(bt), _ptr(row_len), _ptr(ids)
        pr.out, pr.lse, pr.out_abs = _ptr(out), _ptr(lse), _ptr(oabs)
        rc = self.lib.oracle_sparse_attn(C.byref(pr))
        if rc:
            raise ValueError(f"oracle_sparse_attn refused its arguments or ran out of memory ({rc})")
        return {"out": out, "lse": lse, "out_abs": oabs}
