"""Sparse attention over the selected blocks: the HIP path (through the C-ABI)
against the CPU oracle on an MI355X, with K/V in bf16 and in fp8 e4m3.

Acceptance (derived from the arithmetic: P in bf16 for the PV product, out
rounded to bf16, scores in fp32):
* out: |g - o| <= 2^-8 * (out_abs + |o|) + 1e-6 per element, where out_abs =
  sum_t w_t |v_t| is the oracle's weighted |V|;
* lse: |g - o| <= 1e-4 * max(1, |o|);
* NaN rows, and rows with out = 0 and lse = -inf, exactly where the oracle
  has them.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import conftest
import harness as Hn
import pins
from sparse_attention_lightning_amd import idx as I
from sparse_attention_lightning_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not Hn.gpu_ok(), reason="needs an MI355X (gfx950)")]

SCALE = pins.ATTN_SCALE
KVF = pytest.mark.parametrize("kvf", [W.K_BF16, W.K_FP8_E4M3], ids=["bf16kv", "fp8kv"])


def say(*a):
    print("[case]", *a, flush=True)


def gpu_attn(w: W.Workload, at: W.AttnInputs, ids, sm_scale: float = SCALE) -> dict:
    ids_t = ids if isinstance(ids, torch.Tensor) else torch.as_tensor(np.ascontiguousarray(ids), device="cuda")
    out = torch.full_like(at.q, float("nan"))
    lse = torch.full(at.q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    p = I.make_attn_params(q=at.q, k=at.k, v=at.v, req_slot=w.req_slot, block_table=w.block_table,
                           row_len=w.row_len, topk_ids=ids_t.contiguous(), out=out, lse=lse, sm_scale=sm_scale)
    I.idx_sparse_attn(p)
    torch.cuda.synchronize()
    return {"out": out.float().cpu().numpy(), "lse": lse.cpu().numpy()}


def assert_attn(g: dict, o: dict, what: str = "attn") -> None:
    go, oo, oa = g["out"].astype(np.float64), o["out"].astype(np.float64), o["out_abs"].astype(np.float64)
    gl, ol = g["lse"].astype(np.float64), o["lse"].astype(np.float64)
    assert go.shape == oo.shape and gl.shape == ol.shape
    assert np.array_equal(np.isnan(gl), np.isnan(ol)), f"{what}: NaN rows differ"
    assert np.array_equal(np.isneginf(gl), np.isneginf(ol)), f"{what}: empty rows differ"
    assert np.array_equal(np.isnan(go), np.isnan(oo)), f"{what}: NaN outputs differ"
    empty = np.isneginf(ol)
    assert (go[empty] == 0).all(), f"{what}: an empty row's output is not 0"
    f = np.isfinite(oo)
    err = np.abs(go[f] - oo[f]) - (2.0 ** -8 * (oa[f] + np.abs(oo[f])) + 1e-6)
    if err.size:
        i = int(np.argmax(err))
        assert err[i] <= 0, f"{what}: out off by {np.abs(go[f] - oo[f])[i]:.3g} at flat {i} (bound {err[i]:.3g} over)"
    fl = np.isfinite(ol)
    el = np.abs(gl[fl] - ol[fl]) / np.maximum(np.abs(ol[fl]), 1.0)
    assert el.size == 0 or el.max() <= 1e-4, f"{what}: lse rel err {el.max():.3g}"


# ---------------------------------------------------------------------------
# small shapes, random selections (with repeated and ignored ids)
# ---------------------------------------------------------------------------
SHAPES = [  # (P, H, G, lens, topk, pads)
    (4, 4, 4, [0, 130, 700, 1500, 3000], 8, 1),
    (1, 1, 1, [1, 128, 129, 5000], 5, 0),
    (2, 3, 8, [640, 260], 6, 1),
    (16, 1, 1, [513, 2049], 4, 0),
    (3, 2, 5, [90, 1030, 40], 7, 2),
    (4, 2, 2, [20000], 64, 0),
    # more than one 16-row tile a (request, KV head): 20, 32, 48 and 64 rows
    (5, 2, 4, [300, 2600], 6, 1),
    (4, 2, 8, [0, 130, 5000], 8, 1),
    (3, 2, 16, [700, 1500], 5, 0),
    (4, 1, 16, [129, 9000], 12, 1),
    (16, 1, 4, [2049, 600], 4, 0),
]


@KVF
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_attn_small_shapes(oracle, shape, kvf):
    P, H, G, lens, topk, pads = SHAPES[shape]
    say("attn small", SHAPES[shape], "kv format", kvf)
    w = W.make(name="attn", R=len(lens), P=P, H=H, k_format=W.K_BF16, req_len=lens, topk=topk, init_blocks=1,
               local_blocks=1, seed=700 + shape, pads=pads, pad_len=4000, device="cuda")
    at = W.make_attn(w, G, kv_format=kvf)
    wc = W.make(name="attn", R=len(lens), P=P, H=H, k_format=W.K_BF16, req_len=lens, topk=topk, init_blocks=1,
                local_blocks=1, seed=700 + shape, pads=pads, pad_len=4000)  # CPU copy of the tables
    ids = pins.random_selection(wc, np.random.default_rng(710 + shape), topk=topk)
    a = W.attn_oracle_args(w, at, ids, SCALE)
    assert_attn(gpu_attn(w, at, ids), oracle.sparse_attn(**a), f"shape {shape}")


@KVF
def test_attn_after_the_step(oracle, kvf):
    """The indexer step's own selection feeds the attention (the verify
    pipeline: score -> top-k -> attention)."""
    say("attn after idx_step, kv format", kvf)
    w = W.make(name="pipe", R=4, P=4, H=4, k_format=W.K_FP8_E4M3, req_len=[3000, 9000, 200, 17000], topk=16,
               init_blocks=1, local_blocks=2, seed=720, pads=1, pad_len=5000, device="cuda")
    at = W.make_attn(w, 4, kv_format=kvf)
    outs = Hn.gpu_outputs(w)
    I.idx_step(Hn.gpu_params(w, outs))
    g = gpu_attn(w, at, outs["topk_ids"])
    a = W.attn_oracle_args(w, at, outs["topk_ids"], SCALE)
    assert_attn(g, oracle.sparse_attn(**a), "after the step")


@pytest.mark.parametrize("scale", [1e-3, 1.0, 10.0])
def test_attn_scales(oracle, scale):
    say("attn scale", scale)
    w = W.make(name="sc", R=2, P=4, H=2, k_format=W.K_BF16, req_len=[1000, 2600], topk=6, init_blocks=1,
               local_blocks=1, seed=730, device="cuda")
    wc = W.make(name="sc", R=2, P=4, H=2, k_format=W.K_BF16, req_len=[1000, 2600], topk=6, init_blocks=1,
                local_blocks=1, seed=730)
    at = W.make_attn(w, 4)
    ids = pins.random_selection(wc, np.random.default_rng(731), topk=6)
    assert_attn(gpu_attn(w, at, ids, scale), oracle.sparse_attn(**W.attn_oracle_args(w, at, ids, scale)),
                f"scale {scale}")


@KVF
def test_attn_bad_pages_and_empty_rows(oracle, kvf):
    """A selected block on a page outside the pool makes exactly the rows
    that see it NaN; rows of length 0, rows selecting nothing and graph pads
    get 0 and -inf."""
    say("attn bad pages, kv format", kvf)
    lens = [700, 1500, 0, 300]
    w = W.make(name="bad", R=4, P=4, H=2, k_format=W.K_BF16, req_len=lens, topk=6, init_blocks=1,
               local_blocks=1, seed=740, pads=1, pad_len=900, device="cuda")
    wc = W.make(name="bad", R=4, P=4, H=2, k_format=W.K_BF16, req_len=lens, topk=6, init_blocks=1,
                local_blocks=1, seed=740, pads=1, pad_len=900)
    at = W.make_attn(w, 3, kv_format=kvf)
    ids = pins.random_selection(wc, np.random.default_rng(741), topk=6)
    ids[3 * 4 + 1, 0] = -1  # request 3, draft row 1, head 0 selects nothing
    s1 = int(wc.req_slot[1])
    w.block_table[s1, int(ids[1 * 4 + 3, 1][0])] = w.n_pages + 9
    w.block_table[s1, 0] = -5
    a = W.attn_oracle_args(w, at, ids, SCALE)
    o = oracle.sparse_attn(**a)
    assert np.isnan(o["lse"]).any() and np.isneginf(o["lse"]).any()
    assert_attn(gpu_attn(w, at, ids), o, "bad pages")


def test_attn_degenerate(oracle):
    say("attn degenerate")
    # only graph pads
    w = W.make(name="pads", R=0, P=2, H=2, k_format=W.K_BF16, req_len=[], topk=3, init_blocks=1, local_blocks=1,
               seed=750, pads=3, pad_len=600, device="cuda")
    at = W.make_attn(w, 2)
    ids = np.zeros((w.n_req * 2 * 2, 3), np.int32)
    g = gpu_attn(w, at, ids)
    assert (g["out"] == 0).all() and np.isneginf(g["lse"]).all()
    # a table with no block column: nothing can be selected
    w = W.make(name="mb0", R=2, P=1, H=1, k_format=W.K_BF16, req_len=[0, 0], topk=2, init_blocks=1, local_blocks=1,
               seed=751, device="cuda", max_blocks=0)
    at = W.make_attn(w, 2)
    g = gpu_attn(w, at, np.zeros((2, 2), np.int32))
    assert (g["out"] == 0).all() and np.isneginf(g["lse"]).all()


@KVF
def test_attn_repeated_calls_are_identical(oracle, kvf):
    """The same inputs give bit-identical outputs over repeated launches (no
    state is carried in the workspace between calls)."""
    say("attn repeat, kv format", kvf)
    w = W.make(name="rep", R=3, P=4, H=4, k_format=W.K_BF16, req_len=[4000, 800, 12000], topk=12, init_blocks=1,
               local_blocks=2, seed=760, device="cuda")
    wc = W.make(name="rep", R=3, P=4, H=4, k_format=W.K_BF16, req_len=[4000, 800, 12000], topk=12, init_blocks=1,
                local_blocks=2, seed=760)
    at = W.make_attn(w, 4, kv_format=kvf)
    ids = pins.random_selection(wc, np.random.default_rng(761), topk=12)
    first = gpu_attn(w, at, ids)
    for _ in range(20):
        again = gpu_attn(w, at, ids)
        assert np.array_equal(first["out"], again["out"], equal_nan=True)
        assert np.array_equal(first["lse"], again["lse"], equal_nan=True)


def test_attn_unsplit_batch(oracle):
    """A batch of (request, KV head) items that fills the device on its own
    is not split: the partial kernel writes the output, no merge runs and no
    workspace is needed."""
    say("attn unsplit batch")
    R = 80
    lens = [int(x) for x in np.random.default_rng(790).integers(0, 3000, size=R)]
    w = W.make(name="unsplit", R=R, P=2, H=4, k_format=W.K_BF16, req_len=lens, topk=5, init_blocks=1,
               local_blocks=1, seed=791, pads=2, pad_len=800, device="cuda")
    wc = W.make(name="unsplit", R=R, P=2, H=4, k_format=W.K_BF16, req_len=lens, topk=5, init_blocks=1,
                local_blocks=1, seed=791, pads=2, pad_len=800)
    at = W.make_attn(w, 8)
    ids = pins.random_selection(wc, np.random.default_rng(792), topk=5)
    out = torch.empty_like(at.q)
    lse = torch.empty(at.q.shape[:3], dtype=torch.float32, device="cuda")
    p = I.make_attn_params(q=at.q, k=at.k, v=at.v, req_slot=w.req_slot, block_table=w.block_table,
                           row_len=w.row_len, topk_ids=torch.as_tensor(ids, device="cuda"), out=out, lse=lse,
                           sm_scale=SCALE)
    assert I.idx_sparse_attn_workspace(p) == 0 and p.workspace is None
    from test_gpu_parity import _graph_kernel_nodes
    assert _graph_kernel_nodes(lambda: I.idx_sparse_attn(p)) == 1
    assert_attn(gpu_attn(w, at, ids), oracle.sparse_attn(**W.attn_oracle_args(w, at, ids, SCALE)), "unsplit")


@KVF
@pytest.mark.parametrize("case", range(32))
def test_attn_random_shapes(oracle, case, kvf):
    """Seeded random shapes: draft rows, KV heads, query heads a KV head
    (P G <= 64: one to four 16-row tiles), request lengths (some 0, some straddling block ends),
    selection sizes, graph pads, repeated and ignored ids."""
    rng = np.random.default_rng(900 + case)
    P = int(rng.integers(1, 9))
    G = int(rng.integers(1, 64 // P + 1))
    H = int(rng.integers(1, 5))
    R = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.choice([0, 1, 127, 128, 129, 700, 2048, 5000, 20000], size=R)]
    topk = int(rng.integers(4, 40))
    pads = int(rng.integers(0, 3))
    say("attn random", case, dict(P=P, G=G, H=H, R=R, lens=lens, topk=topk, pads=pads, kv_format=kvf))
    kw = dict(name="rand", R=R, P=P, H=H, k_format=W.K_BF16, req_len=lens, topk=topk, init_blocks=1,
              local_blocks=1, seed=910 + case, pads=pads, pad_len=int(rng.integers(1, 3000)))
    w = W.make(**kw, device="cuda")
    wc = W.make(**kw)
    at = W.make_attn(w, G, kv_format=kvf)
    ids = pins.random_selection(wc, np.random.default_rng(920 + case), topk=topk)
    scale = float(np.float32(rng.choice([0.05, SCALE, 0.5])))
    assert_attn(gpu_attn(w, at, ids, scale), oracle.sparse_attn(**W.attn_oracle_args(w, at, ids, scale)),
                f"random case {case}")


@KVF
def test_attn_graph_replays(oracle, kvf):
    """idx_sparse_attn captured once in a HIP graph and replayed after new
    queries, values, lengths and selections are written into the captured
    buffers equals the eager call on every replay (the workspace needs no
    clearing between replays)."""
    say("attn graph replays, kv format", kvf)
    kw = dict(name="gr", R=3, P=4, H=2, k_format=W.K_BF16, req_len=[3000, 9000, 400], topk=24, init_blocks=1,
              local_blocks=1, seed=930)
    w, wc = W.make(**kw, device="cuda"), W.make(**kw)
    at = W.make_attn(w, 4, kv_format=kvf)
    ids = torch.as_tensor(pins.random_selection(wc, np.random.default_rng(931), topk=24), device="cuda")
    out = torch.empty_like(at.q)
    lse = torch.empty(at.q.shape[:3], dtype=torch.float32, device="cuda")
    p = I.make_attn_params(q=at.q, k=at.k, v=at.v, req_slot=w.req_slot, block_table=w.block_table,
                           row_len=w.row_len, topk_ids=ids, out=out, lse=lse, sm_scale=SCALE)
    assert p.workspace is not None  # split: partials and a merge in the graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        I.idx_sparse_attn(p)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        I.idx_sparse_attn(p)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(932)
    base_len = w.row_len.clone()
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        at.q.copy_(torch.randn(at.q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        at.v.copy_(torch.randn(at.v.shape, generator=gen, device="cuda").to(at.v.dtype))
        w.row_len.copy_(torch.clamp(base_len - 301 * rep, min=0))
        ids.copy_(torch.as_tensor(pins.random_selection(wc, np.random.default_rng(940 + rep), topk=24), device="cuda"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"out": out.float().cpu().numpy(), "lse": lse.cpu().numpy()}
        eager = gpu_attn(w, at, ids)
        assert np.array_equal(got["out"], eager["out"], equal_nan=True), f"replay {rep}: out"
        assert np.array_equal(got["lse"], eager["lse"], equal_nan=True), f"replay {rep}: lse"
    assert_attn(got, oracle.sparse_attn(**W.attn_oracle_args(w, at, ids, SCALE)), "graph replay")


def test_attn_launch_count():
    from test_gpu_parity import _graph_kernel_nodes
    say("attn launch count")
    # few items with long selections: split, so partials and a merge (two launches)
    w = W.make(name="lc", R=3, P=4, H=2, k_format=W.K_BF16, req_len=[4000, 9000, 0], topk=32, init_blocks=1,
               local_blocks=1, seed=770, device="cuda")
    at = W.make_attn(w, 4)
    ids = torch.zeros((w.rows, 32), dtype=torch.int32, device="cuda")
    out = torch.empty_like(at.q)
    lse = torch.empty(at.q.shape[:3], dtype=torch.float32, device="cuda")
    p = I.make_attn_params(q=at.q, k=at.k, v=at.v, req_slot=w.req_slot, block_table=w.block_table,
                           row_len=w.row_len, topk_ids=ids, out=out, lse=lse, sm_scale=SCALE)
    assert I.idx_sparse_attn_workspace(p) > 0
    assert _graph_kernel_nodes(lambda: I.idx_sparse_attn(p)) == 2


# ---------------------------------------------------------------------------
# full size: the decode workloads' selections over bf16 K/V pools of their
# size (sampled requests against the oracle, on a compacted pool of just the
# pages those requests select)
# ---------------------------------------------------------------------------
def _subset(w: W.Workload, at: W.AttnInputs, ids: np.ndarray, reqs) -> tuple[dict, np.ndarray]:
    P, H = w.packed_queries, w.gqa
    bt = w.block_table.cpu().numpy()
    slots = w.req_slot.cpu().numpy()
    lens = w.row_len.cpu().numpy()
    K = ids.shape[-1]
    ids3 = ids.reshape(w.n_req * P, H, K)
    need = set()
    for r in reqs:
        s = int(slots[r])
        if not (0 <= s < w.n_slot_rows):
            continue
        for j in range(P):
            nb = (int(lens[r * P + j]) + 127) // 128
            for h in range(H):
                for b in ids3[r * P + j, h]:
                    if 0 <= b < nb and 0 <= bt[s, b] < w.n_pages:
                        need.add(int(bt[s, b]))
    pages = np.array(sorted(need), dtype=np.int64)
    remap = {int(p_): i for i, p_ in enumerate(pages)}
    n_slot = len(reqs)
    bt_sub = np.full((n_slot, w.max_blocks), -1, np.int32)
    req_slot = np.zeros(len(reqs), np.int32)
    for i, r in enumerate(reqs):
        s = int(slots[r])
        if not (0 <= s < w.n_slot_rows):
            req_slot[i] = n_slot + i  # still a graph pad
            continue
        req_slot[i] = i
        bt_sub[i] = [remap.get(int(x), -1) if x >= 0 else -1 for x in bt[s]]
    rows = np.concatenate([np.arange(r * P, r * P + P) for r in reqs])
    pg = torch.as_tensor(pages if len(pages) else np.zeros(1, np.int64), device="cuda")

    def u16(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    def kv(t):  # raw bytes of a K or V pool in its format
        return u16(t) if at.kv_format == W.K_BF16 else t.contiguous().cpu().view(torch.uint8).numpy()

    kv_dt = np.uint16 if at.kv_format == W.K_BF16 else np.uint8
    kk = kv(at.k.index_select(0, pg)) if len(pages) else np.zeros((1, H, 128, 128), kv_dt)
    vv = kv(at.v.index_select(0, pg)) if len(pages) else np.zeros((1, H, 4, 128, 32), kv_dt)
    q = u16(at.q)[rows]
    a = dict(n_req=len(reqs), n_slot_rows=n_slot, packed_queries=P, kv_heads=H, q_per_kv=at.q_per_kv,
             max_blocks=w.max_blocks, topk=K, sm_scale=SCALE, n_pages=max(1, len(pages)), kv_format=at.kv_format,
             q=np.ascontiguousarray(q),
             k=np.ascontiguousarray(kk), v=np.ascontiguousarray(vv), req_slot=req_slot, block_table=bt_sub,
             row_len=np.ascontiguousarray(lens[rows].astype(np.int32)),
             topk_ids=np.ascontiguousarray(ids3[rows].reshape(-1, K)))
    return a, rows


@pytest.mark.parametrize("cfg,reqs,kvf,G", [(3, "all", W.K_BF16, 4), (4, "all", W.K_BF16, 4),
                                            (3, "all", W.K_FP8_E4M3, 4), (3, "all", W.K_FP8_E4M3, 16)],
                         ids=["524k_fp8", "150k_nvfp4", "524k_fp8_fp8kv", "524k_fp8_fp8kv_g16"])
def test_attn_full_size(oracle, cfg, reqs, kvf, G):
    """Every row of the 524K workload (its 32 requests and 3 graph pads:
    about 8 GB of selected bf16 K/V pages go to the oracle, 4 GB in fp8) and
    of the 150K one (64 requests, about 16 GB), against the oracle."""
    w = W.config(cfg, device="cuda")
    if reqs == "all":
        reqs = list(range(w.n_req))
    say("attn full size", W.CONFIG_NAMES[cfg], "kv format", kvf, "query heads a KV head", G, "requests", reqs)
    if w.k_format == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
    outs = Hn.gpu_outputs(w)
    I.idx_step(Hn.gpu_params(w, outs))
    at = W.make_attn(w, G, kv_format=kvf)
    g = gpu_attn(w, at, outs["topk_ids"])
    ids = outs["topk_ids"].cpu().numpy()
    a, rows = _subset(w, at, ids, reqs)
    o = oracle.sparse_attn(**a)
    assert_attn({"out": g["out"][rows], "lse": g["lse"][rows]}, o, f"full size {W.CONFIG_NAMES[cfg]}")
    # every real row saw something; pads none
    real = np.arange(w.n_real * w.packed_queries)
    assert np.isfinite(g["lse"][real]).all() and np.isneginf(g["lse"][w.n_real * w.packed_queries:]).all()
    conftest.REPORT.append(f"sparse attention {w.name} ({'fp8' if kvf else 'bf16'} K/V, {G} query heads a KV head): "
                           f"{len(reqs)} of {w.n_req} requests compared ({len(rows) * w.gqa * G} query heads)")
    del at
    torch.cuda.empty_cache()
