"""The C-ABI library without a GPU: it loads, exports every entry point that
include/idx.h declares, and refuses bad arguments with the documented codes
before touching the HIP runtime."""
from __future__ import annotations

import ctypes as C
import re
import subprocess
from pathlib import Path

import pytest

from sparse_attention_lightning_amd import idx as I

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def lib():
    if not I.LIB_PATH.exists():
        pytest.fail("libidx.so is not built (run __graft_entry__.build())")
    return I.load()


def declared_functions() -> list[str]:
    text = (ROOT / "include" / "idx.h").read_text()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\s*\*)\s*(idx_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(I.EXPORTS)


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def good_params() -> I.IdxParams:
    """Valid-looking parameters with dummy, never dereferenced pointers."""
    p = I.IdxParams()
    p.k_format, p.n_req, p.n_slot_rows = I.IDX_K_FP8_E4M3, 2, 4
    p.packed_queries, p.gqa, p.head_dim, p.block_size = 4, 4, 128, 128
    p.max_blocks, p.topk, p.init_blocks, p.local_blocks, p.n_pages = 16, 8, 1, 2, 64
    for i, f in enumerate(["q", "k", "k_scale", "req_slot", "block_table", "row_len",
                           "block_scores", "topk_ids", "topk_scores"]):
        setattr(p, f, 0x100000 * (i + 1))
    return p


REFUSALS = [
    ("k_format", 3, I.IDX_E_FORMAT),
    ("k_format", -1, I.IDX_E_FORMAT),
    ("head_dim", 64, I.IDX_E_SHAPE),
    ("block_size", 64, I.IDX_E_SHAPE),
    ("packed_queries", 0, I.IDX_E_SHAPE),
    ("gqa", I.IDX_MAX_REQ_ROWS // 4 + 1, I.IDX_E_PACK),
    ("packed_queries", I.IDX_MAX_REQ_ROWS // 4 + 1, I.IDX_E_PACK),
    ("n_req", I.IDX_MAX_ROWS // 16 + 1, I.IDX_E_PACK),
    ("n_req", -1, I.IDX_E_SHAPE),
    ("n_pages", -2, I.IDX_E_SHAPE),
    ("max_blocks", I.IDX_MAX_BLOCKS + 1, I.IDX_E_SHAPE),
    ("max_blocks", -1, I.IDX_E_SHAPE),
    ("reserved", 1, I.IDX_E_SHAPE),
    ("score_mode", 2, I.IDX_E_MODE),
    ("score_mode", -1, I.IDX_E_MODE),
    ("topk", 0, I.IDX_E_TOPK),
    ("topk", 2, I.IDX_E_TOPK),          # < init + local
    ("local_blocks", -1, I.IDX_E_TOPK),
    ("init_blocks", -2, I.IDX_E_TOPK),
    ("q", None, I.IDX_E_NULL),
    ("k", None, I.IDX_E_NULL),
    ("req_slot", None, I.IDX_E_NULL),
    ("row_len", None, I.IDX_E_NULL),
    ("block_table", None, I.IDX_E_NULL),
    ("block_scores", None, I.IDX_E_NULL),
    ("topk_ids", None, I.IDX_E_NULL),
    ("topk_scores", None, I.IDX_E_NULL),
    ("q", 0x100008, I.IDX_E_ALIGN),
    ("k", 0x100004, I.IDX_E_ALIGN),
]


@pytest.mark.parametrize("field,value,code", REFUSALS, ids=[f"{f}={v}" for f, v, _ in REFUSALS])
def test_step_refusals(lib, field, value, code):
    p = good_params()
    setattr(p, field, value)
    assert lib.idx_step(C.byref(p), None) == code
    assert lib.idx_last_error().decode() != ""


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan")])
def test_lse_needs_a_finite_positive_scale(lib, scale):
    p = good_params()
    p.score_mode = I.IDX_SCORE_LSE
    p.sm_scale = scale
    assert lib.idx_step(C.byref(p), None) == I.IDX_E_MODE
    assert lib.idx_score_packed(C.byref(p), None) == I.IDX_E_MODE
    p.score_mode = I.IDX_SCORE_MAX  # the scale is ignored for the max
    assert lib.idx_score_packed(C.byref(p), None) != I.IDX_E_MODE


def test_params_layout_matches_header(tmp_path):
    """The ctypes mirror has the C struct's size and field offsets (gcc reads
    include/idx.h)."""
    names = [f for f, _ in I.IdxParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "idx.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(idx_params));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(idx_params, {n}));\n' for n in names)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(I.IdxParams)
    assert got[1:] == [getattr(I.IdxParams, n).offset for n in names]


def test_attn_params_layout_matches_header(tmp_path):
    names = [f for f, _ in I.IdxAttnParams._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "idx.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(idx_attn_params));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(idx_attn_params, {n}));\n' for n in names)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(I.IdxAttnParams)
    assert got[1:] == [getattr(I.IdxAttnParams, n).offset for n in names]


def good_attn_params() -> I.IdxAttnParams:
    p = I.IdxAttnParams()
    p.n_req, p.n_slot_rows, p.packed_queries, p.kv_heads, p.q_per_kv = 2, 4, 4, 2, 4
    p.head_dim = p.block_size = 128
    p.max_blocks, p.topk, p.sm_scale, p.n_pages = 16, 8, 0.125, 64
    p.workspace_bytes = 1 << 30
    for i, f in enumerate(["q", "k", "v", "req_slot", "block_table", "row_len", "topk_ids", "out", "lse",
                           "workspace"]):
        setattr(p, f, 0x100000 * (i + 1))
    return p


ATTN_REFUSALS = [
    ("head_dim", 64, I.IDX_E_SHAPE),
    ("block_size", 256, I.IDX_E_SHAPE),
    ("packed_queries", 0, I.IDX_E_SHAPE),
    ("kv_heads", 0, I.IDX_E_SHAPE),
    ("q_per_kv", 0, I.IDX_E_SHAPE),
    ("q_per_kv", 17, I.IDX_E_PACK),          # 4 * 17 rows > 64
    ("packed_queries", 17, I.IDX_E_PACK),    # more than 16 draft rows
    ("n_req", -1, I.IDX_E_SHAPE),
    ("n_req", I.IDX_MAX_REQ + 1, I.IDX_E_SHAPE),
    ("max_blocks", I.IDX_MAX_BLOCKS + 1, I.IDX_E_SHAPE),
    ("n_pages", -1, I.IDX_E_SHAPE),
    ("topk", 0, I.IDX_E_TOPK),
    ("topk", I.IDX_ATTN_MAX_IDS // 4 + 1, I.IDX_E_TOPK),
    ("sm_scale", 0.0, I.IDX_E_MODE),
    ("sm_scale", float("inf"), I.IDX_E_MODE),
    ("sm_scale", float("nan"), I.IDX_E_MODE),
    ("kv_format", I.IDX_K_NVFP4, I.IDX_E_FORMAT),
    ("kv_format", -1, I.IDX_E_FORMAT),
    ("q", None, I.IDX_E_NULL),
    ("v", None, I.IDX_E_NULL),
    ("topk_ids", None, I.IDX_E_NULL),
    ("lse", None, I.IDX_E_NULL),
    ("block_table", None, I.IDX_E_NULL),
    ("v", 0x100008, I.IDX_E_ALIGN),
    ("workspace", 0x100004, I.IDX_E_ALIGN),
    ("workspace_bytes", 16, I.IDX_E_SHAPE),
]


@pytest.mark.parametrize("field,value,code", ATTN_REFUSALS, ids=[f"{f}={v}" for f, v, _ in ATTN_REFUSALS])
def test_attn_refusals(lib, field, value, code):
    p = good_attn_params()
    setattr(p, field, value)
    assert lib.idx_sparse_attn(C.byref(p), None) == code, lib.idx_last_error().decode()
    assert lib.idx_last_error().decode() != ""


def test_attn_workspace_query(lib):
    p = good_attn_params()
    assert lib.idx_sparse_attn_workspace(C.byref(p)) > 0
    p.q_per_kv = 17
    assert lib.idx_sparse_attn_workspace(C.byref(p)) == I.IDX_E_PACK
    assert lib.idx_sparse_attn_workspace(None) == I.IDX_E_NULL


def test_null_params(lib):
    assert lib.idx_step(None, None) == I.IDX_E_NULL
    assert lib.idx_score_packed(None, None) == I.IDX_E_NULL
    assert lib.idx_block_topk(None, None) == I.IDX_E_NULL
    assert lib.idx_sparse_attn(None, None) == I.IDX_E_NULL


def test_entry_specific_requirements(lib):
    p = good_params()
    p.k_format = I.IDX_K_NVFP4
    p.k_scale = None
    assert lib.idx_score_packed(C.byref(p), None) == I.IDX_E_NULL   # scoring needs scales
    p = good_params()
    p.topk_ids = None
    assert lib.idx_block_topk(C.byref(p), None) == I.IDX_E_NULL    # selection needs outputs
    p = good_params()
    p.k_format = I.IDX_K_NVFP4
    p.k_scale = 0x100001
    assert lib.idx_score_packed(C.byref(p), None) == I.IDX_E_ALIGN


EMPTY_NULLS = [  # (sizes that empty some arrays, the pointers that may then be NULL)
    (dict(n_pages=0), ["k", "k_scale"]),
    (dict(max_blocks=0), ["block_scores", "block_table"]),
    (dict(n_slot_rows=0), ["block_table"]),
    (dict(n_req=0), ["q", "req_slot", "row_len", "block_scores", "topk_ids", "topk_scores"]),
]


@pytest.mark.parametrize("sizes,nulls", EMPTY_NULLS, ids=[next(iter(s)) for s, _ in EMPTY_NULLS])
def test_empty_arrays_may_be_null(lib, sizes, nulls):
    """A pointer is required only where its array has elements.  The call is
    made to fail a later check (a misaligned pointer) so that nothing runs:
    IDX_E_ALIGN shows that every NULL check passed."""
    p = good_params()
    p.k_format = I.IDX_K_NVFP4
    for f, v in sizes.items():
        setattr(p, f, v)
    for f in nulls:
        setattr(p, f, None)
    if "q" in nulls:
        p.k = 0x100004
    else:
        p.q = 0x100008
    assert lib.idx_step(C.byref(p), None) == I.IDX_E_ALIGN, lib.idx_last_error().decode()
    # the same NULLs with the sizes left non-zero are refused
    q = good_params()
    q.k_format = I.IDX_K_NVFP4
    for f in nulls:
        setattr(q, f, None)
    assert lib.idx_step(C.byref(q), None) == I.IDX_E_NULL


FP4_REFUSALS = [
    dict(stride=100, code=I.IDX_E_SHAPE),
    dict(stride=130, code=I.IDX_E_SHAPE),
    dict(n_tokens=-1, code=I.IDX_E_SHAPE),
    dict(n_slots=-1, code=I.IDX_E_SHAPE),
    dict(payload=None, code=I.IDX_E_NULL),
    dict(slot_mapping=None, code=I.IDX_E_NULL),
    dict(staging=0x200008, code=I.IDX_E_ALIGN),
    dict(scales=0x500004, code=I.IDX_E_ALIGN),
]


@pytest.mark.parametrize("case", FP4_REFUSALS, ids=lambda c: ",".join(f"{k}" for k in c if k != "code"))
def test_fp4_store_refusals(lib, case):
    a = dict(staging=0x200000, n_tokens=10, stride=128, slot_mapping=0x300000, payload=0x400000,
             scales=0x500000, n_slots=10)
    a.update({k: v for k, v in case.items() if k != "code"})
    rc = lib.idx_fp4_store(a["staging"], a["n_tokens"], a["stride"], a["slot_mapping"],
                           a["payload"], a["scales"], a["n_slots"], None)
    assert rc == case["code"]


def test_fp4_store_empty_is_ok(lib):
    assert lib.idx_fp4_store(None, 0, 128, None, None, None, 0, None) == I.IDX_OK


def test_binding_constants_match_header():
    text = (ROOT / "include" / "idx.h").read_text()
    for name in ("IDX_MAX_BLOCKS", "IDX_MAX_REQ", "IDX_MAX_REQ_ROWS"):
        m = re.search(rf"#define\s+{name}\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(I, name), name
    m = re.search(r"#define\s+IDX_MAX_ROWS\s+\(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == I.IDX_MAX_ROWS
    for name in ("IDX_ATTN_MAX_ROWS", "IDX_ATTN_MAX_DRAFT", "IDX_ATTN_MAX_IDS", "IDX_ATTN_MAX_SPLITS"):
        m = re.search(rf"#define\s+{name}\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(I, name), name
    m = re.search(r"#define\s+IDX_NOALLOC_MAX_SCORES\s+\((\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == I.IDX_NOALLOC_MAX_SCORES
    enums = dict((k, int(v)) for k, v in re.findall(r"(IDX_\w+)\s*=\s*(-?\d+)", text))
    for k, v in enums.items():
        assert getattr(I, k) == v, k


def test_noalloc_refusals(lib):
    """idx_step_noalloc keeps the block scores itself: a caller buffer is
    refused, as is a step whose block scores exceed its array; the other
    checks are idx_step's."""
    p = good_params()
    assert lib.idx_step_noalloc(C.byref(p), None) == I.IDX_E_SHAPE     # block_scores given
    assert "NULL" in lib.idx_last_error().decode()
    p.block_scores = None
    p.head_dim = 64
    assert lib.idx_step_noalloc(C.byref(p), None) == I.IDX_E_SHAPE     # idx_step's checks apply
    p = good_params()
    p.block_scores = None
    p.topk_ids = None
    assert lib.idx_step_noalloc(C.byref(p), None) == I.IDX_E_NULL
    p = good_params()
    p.block_scores = None
    p.max_blocks = I.IDX_MAX_BLOCKS
    p.n_req = I.IDX_NOALLOC_MAX_SCORES // (16 * I.IDX_MAX_BLOCKS) + 1  # one request too many
    assert lib.idx_step_noalloc(C.byref(p), None) == I.IDX_E_SHAPE
    assert "exceeds" in lib.idx_last_error().decode()
    assert lib.idx_step_noalloc(None, None) == I.IDX_E_NULL


PROBE_REFUSALS = [
    dict(unit_bytes=512, code=I.IDX_E_SHAPE),
    dict(unit_bytes=3072, code=I.IDX_E_SHAPE),
    dict(unit_bytes=1 << 21, code=I.IDX_E_SHAPE),
    dict(n_units=-1, code=I.IDX_E_SHAPE),
    dict(n_base=0, code=I.IDX_E_SHAPE),
    dict(n_sink=0, code=I.IDX_E_SHAPE),
    dict(base=None, code=I.IDX_E_NULL),
    dict(sink=None, code=I.IDX_E_NULL),
    dict(base=0x200008, code=I.IDX_E_ALIGN),
]


@pytest.mark.parametrize("case", PROBE_REFUSALS, ids=lambda c: ",".join(f"{k}={v}" for k, v in c.items() if k != "code"))
def test_probe_refusals(lib, case):
    a = dict(base=0x200000, n_base=64, units=None, n_units=64, unit_bytes=16384, nt=0, sink=0x300000, n_sink=256)
    a.update({k: v for k, v in case.items() if k != "code"})
    rc = lib.idx_probe_read(a["base"], a["n_base"], a["units"], a["n_units"], a["unit_bytes"], a["nt"],
                            a["sink"], a["n_sink"], None)
    assert rc == case["code"]


def test_last_error_is_per_thread(lib):
    """A refusal on one host thread leaves another thread's message alone."""
    import threading
    seen = {}

    def refuse():
        p = good_params()
        p.head_dim = 64
        seen["rc"] = lib.idx_step(C.byref(p), None)
        seen["msg"] = lib.idx_last_error().decode()

    def fresh():
        seen["other"] = lib.idx_last_error().decode()

    t = threading.Thread(target=refuse)
    t.start()
    t.join()
    u = threading.Thread(target=fresh)
    u.start()
    u.join()
    assert seen["rc"] == I.IDX_E_SHAPE and "head_dim" in seen["msg"]
    assert seen["other"] == ""


def test_new_keys_layout_matches_header(tmp_path):
    names = [f for f, _ in I.IdxFp4NewKeys._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "idx.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(idx_fp4_new_keys));\n'
                   + "".join(f'  printf("%zu\\n", offsetof(idx_fp4_new_keys, {n}));\n' for n in names)
                   + '  printf("%d\\n", IDX_FP4_FUSED_MAX_KEYS);\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", f"-I{ROOT / 'include'}", str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == C.sizeof(I.IdxFp4NewKeys)
    assert got[1:-1] == [getattr(I.IdxFp4NewKeys, n).offset for n in names]
    assert got[-1] == I.IDX_FP4_FUSED_MAX_KEYS


def good_fp4_step() -> tuple:
    p = good_params()
    p.k_format = I.IDX_K_NVFP4
    nk = I.IdxFp4NewKeys(0x900000, 256, 128, 0xA00000)
    return p, nk


FP4_STEP_REFUSALS = [
    ("p", "k_format", I.IDX_K_FP8_E4M3, I.IDX_E_FORMAT),
    ("p", "k_format", I.IDX_K_BF16, I.IDX_E_FORMAT),
    ("p", "k_scale", 0x100004, I.IDX_E_ALIGN),     # 8-byte alignment for the store's scale words
    ("p", "topk", 0, I.IDX_E_TOPK),                 # the step's own checks still apply
    ("k", "n_tokens", -1, I.IDX_E_SHAPE),
    ("k", "staging_row_stride", 100, I.IDX_E_SHAPE),
    ("k", "staging_row_stride", 130, I.IDX_E_SHAPE),
    ("k", "staging_bf16", None, I.IDX_E_NULL),
    ("k", "slot_mapping", None, I.IDX_E_NULL),
    ("k", "staging_bf16", 0x900008, I.IDX_E_ALIGN),
]


@pytest.mark.parametrize("which,field,value,code", FP4_STEP_REFUSALS,
                         ids=[f"{w}.{f}={v}" for w, f, v, _ in FP4_STEP_REFUSALS])
def test_fp4_step_refusals(lib, which, field, value, code):
    p, nk = good_fp4_step()
    setattr(p if which == "p" else nk, field, value)
    assert lib.idx_step_fp4(C.byref(p), C.byref(nk), None) == code
    assert lib.idx_last_error().decode() != ""
    assert lib.idx_score_packed_fp4(C.byref(p), C.byref(nk), None) == code


def test_fp4_step_needs_keys(lib):
    p, _ = good_fp4_step()
    assert lib.idx_step_fp4(C.byref(p), None, None) == I.IDX_E_NULL
    assert lib.idx_score_packed_fp4(C.byref(p), None, None) == I.IDX_E_NULL
