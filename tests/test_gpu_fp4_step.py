"""The NVFP4 step with its new keys (idx_step_fp4 / idx_score_packed_fp4)
against idx_fp4_store followed by idx_step, on the GPU: the pool bytes and the
outputs must be identical, whether the score launch stores the keys itself or
a store launch runs first; and against the oracle.

The other keys of the pool are stored first; the new keys' slots still hold
the workload's poison (code 7, scale 448) when the step starts, so a key the
score kernel read before writing it would win its block."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import harness as Hn
from sparse_attention_lightning_amd import idx as I
from sparse_attention_lightning_amd import workloads as W

pytestmark = pytest.mark.gpu

LSE = dict(score_mode=I.IDX_SCORE_LSE, sm_scale=float(np.float32(128 ** -0.5)))


def say(*a):
    print(*a, flush=True)


def new_key_rows(w: W.Workload, every: int = 1) -> np.ndarray:
    """Staging rows of each real request's last packed_queries tokens (of
    every ``every``-th request)."""
    ends = np.cumsum(w.group_len()[: w.n_real].astype(np.int64))
    P = min(w.packed_queries, 4)
    rows = [np.arange(max(e - P, 0), e) for r, e in enumerate(ends) if r % every == 0]
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


def setup_pool(w: W.Workload, new_rows: np.ndarray):
    """Every other staging key stored; the new ones left as the fill."""
    keep = np.ones(w.staging.shape[0], bool)
    keep[new_rows] = False
    idx = torch.as_tensor(np.nonzero(keep)[0], device="cuda")
    I.idx_fp4_store(w.staging.index_select(0, idx).contiguous(), w.slot_mapping.index_select(0, idx).contiguous(),
                    w.k, w.k_scale)
    torch.cuda.synchronize()


def step_both(w: W.Workload, staging: torch.Tensor, slots: torch.Tensor, **mode):
    """The same step twice on copies of the pool: store then step, and the
    fused call.  Returns (reference, fused), each the outputs and the planes."""
    res = []
    for fused in (False, True):
        k, ks = w.k.clone(), w.k_scale.clone()
        outs = Hn.gpu_outputs(w)
        p = Hn.gpu_params(w, outs, k=k, k_scale=ks, **mode)
        if fused:
            I.idx_step_fp4(p, I.make_new_keys(staging, slots))
        else:
            I.idx_fp4_store(staging, slots, k, ks)
            I.idx_step(p)
        torch.cuda.synchronize()
        r = {key: v.cpu().numpy() for key, v in outs.items()}
        r["payload"], r["scales"] = k.cpu().numpy(), ks.cpu().numpy()
        res.append(r)
    return res


def assert_identical(ref: dict, got: dict, what: str):
    for key in ("payload", "scales", "block_scores", "topk_ids", "topk_scores"):
        assert np.array_equal(ref[key], got[key], equal_nan=True), f"{what}: {key} differs"


def keys_of(w: W.Workload, rows: np.ndarray, extra_slots=()):
    """Staging rows and slots of the new keys, plus keys at ``extra_slots``
    (their staging rows taken from the start of the pool's staging)."""
    st = w.staging[torch.as_tensor(rows, device="cuda")] if len(rows) else w.staging[:0]
    sl = w.slot_mapping[torch.as_tensor(rows, device="cuda")] if len(rows) else w.slot_mapping[:0]
    if extra_slots:
        st = torch.cat([st, w.staging[: len(extra_slots)]])
        sl = torch.cat([sl, torch.as_tensor(np.asarray(extra_slots, np.int64), device="cuda")])
    return st.contiguous(), sl.contiguous()


SHAPES = {
    # (R, P, H, lens, topk, init, local, pads, every): one tile a request
    "small": (3, 4, 4, [700, 2048, 33], 6, 1, 2, 1, 1),
    "one_block_requests": (3000, 1, 4, [100] * 3000, 1, 1, 0, 0, 3),   # shares span several rounds
    "sorted_rounds": (8, 4, 4, [140000] * 8, 16, 1, 2, 0, 1),           # rounds of >= 32 pages (pool order)
    "many_rows": (2, 5, 4, [3000, 900], 5, 1, 2, 1, 1),                # 20 rows a request: a store launch first
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("mode", ["max", "lse"])
def test_fp4_step_equals_store_then_step(shape, mode):
    R, P, H, lens, topk, init, local, pads, every = SHAPES[shape]
    say("fp4 step", shape, mode)
    w = W.make(name="fs_" + shape, R=R, P=P, H=H, k_format=W.K_NVFP4, req_len=lens, topk=topk, init_blocks=init,
               local_blocks=local, seed=1200 + len(shape), pads=pads, pad_len=900, device="cuda")
    rows = new_key_rows(w, every)
    setup_pool(w, rows)
    gap = w.extra["gap_pages"]
    extra = [-1, w.n_pages * 128, w.n_pages * 128 + 5]  # skipped slots
    if len(gap):
        extra += [int(gap[0]) * 128 + 3, int(gap[-1]) * 128 + 127]  # pages no request reads
    st, sl = keys_of(w, rows, extra)
    assert st.shape[0] <= I.IDX_FP4_FUSED_MAX_KEYS
    ref, got = step_both(w, st, sl, **(LSE if mode == "lse" else {}))
    assert_identical(ref, got, f"{shape} {mode}")


def test_fp4_step_many_keys_take_a_store_launch():
    """More keys than the score launch takes: a store launch runs first, with
    the same result."""
    say("fp4 step, many keys")
    w = W.make(name="fs_many", R=1200, P=1, H=4, k_format=W.K_NVFP4, req_len=[300] * 1200, topk=2, init_blocks=1,
               local_blocks=1, seed=1230, device="cuda")
    rows = new_key_rows(w)
    assert len(rows) > I.IDX_FP4_FUSED_MAX_KEYS
    setup_pool(w, rows)
    st, sl = keys_of(w, rows)
    ref, got = step_both(w, st, sl)
    assert_identical(ref, got, "many keys")
    from test_gpu_parity import _graph_kernel_nodes
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)
    assert _graph_kernel_nodes(lambda: I.idx_step_fp4(p, I.make_new_keys(st, sl))) == 3


def test_fp4_step_one_launch_fewer(oracle):
    """The score launch stores the keys: the step is two launches (scoring,
    selection), and it matches the oracle over the whole pool."""
    say("fp4 step launch count and oracle")
    w = W.make(name="fs_lc", R=4, P=4, H=4, k_format=W.K_NVFP4, req_len=[5000, 300, 9000, 1], topk=8, init_blocks=1,
               local_blocks=2, seed=1240, pads=1, pad_len=700, device="cuda")
    rows = new_key_rows(w)
    setup_pool(w, rows)
    st, sl = keys_of(w, rows)
    from test_gpu_parity import _graph_kernel_nodes
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)
    nk = I.make_new_keys(st, sl)
    assert _graph_kernel_nodes(lambda: I.idx_step_fp4(p, nk)) == 2
    assert _graph_kernel_nodes(lambda: I.idx_score_packed_fp4(p, nk)) == 1
    outs = Hn.gpu_outputs(w)
    I.idx_step_fp4(Hn.gpu_params(w, outs), nk)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in outs.items()}
    payload, scales = Hn.oracle_pool(oracle, w)
    assert np.array_equal(w.k.cpu().numpy(), payload) and np.array_equal(w.k_scale.cpu().numpy(), scales)
    a = w.oracle_args(payload, scales)
    Hn.assert_parity(g, oracle.step(**a), a)


def test_fp4_step_repeats_are_identical():
    """Repeated fused steps over the same keys give the same bytes and outputs."""
    say("fp4 step repeats")
    w = W.make(name="fs_rep", R=6, P=4, H=4, k_format=W.K_NVFP4, req_len=[3000, 12000, 700, 40000, 128, 129],
               topk=10, init_blocks=1, local_blocks=2, seed=1250, device="cuda")
    rows = new_key_rows(w)
    setup_pool(w, rows)
    st, sl = keys_of(w, rows)
    nk = I.make_new_keys(st, sl)
    first = None
    for _ in range(10):
        outs = Hn.gpu_outputs(w)
        I.idx_step_fp4(Hn.gpu_params(w, outs), nk)
        torch.cuda.synchronize()
        r = {k: v.cpu().numpy() for k, v in outs.items()}
        r["payload"], r["scales"] = w.k.cpu().numpy(), w.k_scale.cpu().numpy()
        if first is None:
            first = r
        assert_identical(first, r, "repeat")


@pytest.mark.parametrize("mode", ["max", "lse"])
def test_workload_4_fused_store(oracle, mode):
    """The ~150K NVFP4 workload at full size with the step's 256 new keys
    stored by the score launch: every slot of both planes and every row
    against the oracle."""
    say("workload 64req_150k_nvfp4, fused store of the step's keys", mode)
    w = W.config(4, device="cuda")
    rows = new_key_rows(w)
    setup_pool(w, rows)
    st, sl = keys_of(w, rows)
    outs = Hn.gpu_outputs(w)
    m = LSE if mode == "lse" else {}
    I.idx_step_fp4(Hn.gpu_params(w, outs, **m), I.make_new_keys(st, sl))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in outs.items()}
    from test_gpu_parity import _oracle_pool_full
    payload, scales = _oracle_pool_full(oracle, w)
    assert np.array_equal(w.k.cpu().numpy(), payload), "payload bytes differ"
    assert np.array_equal(w.k_scale.cpu().numpy(), scales), "scale bytes differ"
    a = dict(w.oracle_args(payload, scales), **m)
    Hn.assert_parity(g, oracle.step(**a), a)


def test_fp4_step_graph_replays():
    """idx_step_fp4 captured once in a HIP graph and replayed after new key
    values are written into the captured staging buffer equals, on every
    replay, the store then the step run eagerly on a copy of the pool."""
    say("fp4 step graph replays")
    w = W.make(name="fs_graph", R=5, P=4, H=4, k_format=W.K_NVFP4, req_len=[4000, 900, 15000, 60, 2100],
               topk=8, init_blocks=1, local_blocks=2, seed=1260, pads=1, pad_len=800, device="cuda")
    rows = new_key_rows(w)
    setup_pool(w, rows)
    st, sl = keys_of(w, rows)
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)
    nk = I.make_new_keys(st, sl)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        I.idx_step_fp4(p, nk)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        I.idx_step_fp4(p, nk)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1261)
    for rep in range(4):
        st.copy_(torch.randn(st.shape, generator=gen, device="cuda").to(torch.bfloat16) * (1 + rep))
        k0, ks0 = w.k.clone(), w.k_scale.clone()
        for v in outs.values():
            v.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {key: v.cpu().numpy() for key, v in outs.items()}
        got["payload"], got["scales"] = w.k.cpu().numpy(), w.k_scale.cpu().numpy()
        ref_outs = Hn.gpu_outputs(w)
        I.idx_fp4_store(st, sl, k0, ks0)
        I.idx_step(Hn.gpu_params(w, ref_outs, k=k0, k_scale=ks0))
        torch.cuda.synchronize()
        ref = {key: v.cpu().numpy() for key, v in ref_outs.items()}
        ref["payload"], ref["scales"] = k0.cpu().numpy(), ks0.cpu().numpy()
        assert_identical(ref, got, f"replay {rep}")
