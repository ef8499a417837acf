"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI,
run the oracle on the same seeded inputs, and compare with the acceptance
rule.

Acceptance (GPU vs oracle):
* NVFP4 store bytes: bit-exact on every slot.
* block scores: |g - o| <= 2e-3 * max(|o|, 1) wherever the oracle is finite;
  -inf and NaN exactly where the oracle has them.
* ids: identical, unless the oracle's k-th and (k+1)-th best non-forced
  scores (k = topk - |forced|) differ by less than 1e-4 relative; then the
  sets must have the same size, hold every forced block, and every id in the
  symmetric difference must score within 1e-4 relative of the k-th.
"""
from __future__ import annotations

import numpy as np
import torch

from sparse_attention_lightning_amd import idx as I
from sparse_attention_lightning_amd import workloads as W

SCORE_RTOL = 2e-3
TIE_RTOL = 1e-4


def gpu_ok() -> bool:
    if not torch.cuda.is_available():
        return False
    return torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
def gpu_outputs(w: W.Workload, fill: float = float("nan")) -> dict:
    dev = w.q.device
    rows = w.rows
    return {
        "block_scores": torch.full((rows, w.max_blocks), fill, dtype=torch.float32, device=dev),
        "topk_ids": torch.full((rows, w.topk), -7, dtype=torch.int32, device=dev),
        "topk_scores": torch.full((rows, w.topk), fill, dtype=torch.float32, device=dev),
    }


def gpu_params(w: W.Workload, outs: dict, k=None, k_scale=None, score_mode: int = I.IDX_SCORE_MAX,
               sm_scale: float = 0.0) -> I.IdxParams:
    return I.make_params(
        k_format=w.k_format, q=w.q, k=w.k if k is None else k,
        k_scale=w.k_scale if k_scale is None else k_scale, req_slot=w.req_slot,
        block_table=w.block_table, row_len=w.row_len, block_scores=outs["block_scores"],
        topk_ids=outs["topk_ids"], topk_scores=outs["topk_scores"],
        packed_queries=w.packed_queries, gqa=w.gqa, topk=w.topk, init_blocks=w.init_blocks,
        local_blocks=w.local_blocks, max_blocks=w.max_blocks, n_slot_rows=w.n_slot_rows,
        n_pages=w.n_pages, score_mode=score_mode, sm_scale=sm_scale)


def gpu_fp4_store(w: W.Workload) -> None:
    """Quantize the workload's staging keys into its NVFP4 planes on the GPU."""
    I.idx_fp4_store(w.staging, w.slot_mapping, w.k, w.k_scale)


def gpu_step(w: W.Workload, **mode) -> dict:
    """idx_step on the workload; ``mode``: score_mode / sm_scale."""
    outs = gpu_outputs(w)
    I.idx_step(gpu_params(w, outs, **mode))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in outs.items()}


# ---------------------------------------------------------------------------
# oracle side
# ---------------------------------------------------------------------------
def oracle_pool(o, w: W.Workload, tokens: np.ndarray | None = None):
    """NVFP4 planes written by the oracle's own store from the staging keys
    (only the staging rows in ``tokens`` if given), starting from the
    workload's initial fill."""
    payload = np.full((w.n_pages * 128, 64), W.POISON_FP4_PAYLOAD, np.uint8)
    scales = np.full((w.n_pages * 128, 8), W.POISON_FP4_SCALE, np.uint8)
    st = w.staging.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    sm = w.slot_mapping.cpu().numpy()
    if tokens is not None:
        st, sm = st[tokens], sm[tokens]
    o.fp4_store(np.ascontiguousarray(st), np.ascontiguousarray(sm), payload, scales)
    return payload, scales


def subset_args(a: dict, reqs, P: int, H: int) -> dict:
    """Oracle arguments restricted to the requests ``reqs`` (same pool)."""
    reqs = np.asarray(reqs)
    q = a["q"].reshape(a["n_req"], P * H, 128)[reqs].reshape(-1, H, 128)
    rl = a["row_len"].reshape(a["n_req"], P)[reqs].reshape(-1)
    return dict(a, n_req=len(reqs), q=np.ascontiguousarray(q),
                req_slot=np.ascontiguousarray(a["req_slot"][reqs]), row_len=np.ascontiguousarray(rl))


def subset_rows_args(a: dict, req: int, qrows, P: int, H: int) -> dict:
    """Oracle arguments for request ``req`` alone, restricted to its query rows
    ``qrows`` (each with all H heads; the same pool, slot and lengths), as a
    request of len(qrows) packed rows."""
    qrows = np.asarray(qrows)
    q = a["q"].reshape(a["n_req"], P, H, 128)[req, qrows].reshape(-1, H, 128)
    rl = a["row_len"].reshape(a["n_req"], P)[req, qrows]
    return dict(a, n_req=1, packed_queries=len(qrows), q=np.ascontiguousarray(q),
                req_slot=np.ascontiguousarray(a["req_slot"][req:req + 1]), row_len=np.ascontiguousarray(rl))


def rows_of(reqs, rows_per_req: int) -> np.ndarray:
    reqs = np.asarray(reqs)
    return (reqs[:, None] * rows_per_req + np.arange(rows_per_req)[None, :]).reshape(-1)


# ---------------------------------------------------------------------------
# comparison
# ---------------------------------------------------------------------------
def assert_scores(g: np.ndarray, o: np.ndarray, what: str = "block scores") -> None:
    assert g.shape == o.shape, (g.shape, o.shape)
    on, gn = np.isnan(o), np.isnan(g)
    oi, gi = np.isinf(o), np.isinf(g)
    assert np.array_equal(on, gn), f"{what}: NaN positions differ ({np.argwhere(on != gn)[:3]})"
    assert np.array_equal(oi, gi), f"{what}: inf positions differ ({np.argwhere(oi != gi)[:3]})"
    assert np.array_equal(g[gi], o[oi]), f"{what}: inf signs differ"
    f = ~(on | oi)
    err = np.abs(g[f].astype(np.float64) - o[f]) / np.maximum(np.abs(o[f].astype(np.float64)), 1.0)
    if err.size:
        worst = int(np.argmax(err))
        assert err.max() <= SCORE_RTOL, f"{what}: max rel err {err.max():.3g} at flat {worst}"


def _forced(nb: int, init: int, local: int) -> set:
    return set(range(min(init, nb))) | set(range(max(nb - local, 0), nb))


def assert_ids(g_ids: np.ndarray, o_ids: np.ndarray, o_bs: np.ndarray, nbs: np.ndarray,
               topk: int, init: int, local: int) -> int:
    """Compare selections row by row; returns the number of rows that differ
    inside the near-tie allowance."""
    relaxed = 0
    for r in range(g_ids.shape[0]):
        if np.array_equal(g_ids[r], o_ids[r]):
            continue
        nb = int(nbs[r])
        assert nb > topk, f"row {r}: nb={nb} <= topk but ids differ"
        F = _forced(nb, init, local)
        k = topk - len(F)
        free = np.array([b for b in range(nb) if b not in F])
        s = o_bs[r, free].astype(np.float64)
        order = np.lexsort((free, -np.nan_to_num(s, nan=-np.inf)))
        ok_, ok1 = s[order[k - 1]], s[order[k]]
        gap = abs(ok_ - ok1)
        assert gap < TIE_RTOL * max(abs(ok_), abs(ok1)), \
            f"row {r}: ids differ but oracle k-th/k+1-th gap {gap:.3g} is not a near tie"
        gs, os_ = set(g_ids[r][g_ids[r] >= 0].tolist()), set(o_ids[r][o_ids[r] >= 0].tolist())
        assert len(gs) == len(os_) == topk and F <= gs, f"row {r}: size or forced set wrong"
        for b in gs ^ os_:
            assert abs(o_bs[r, b] - ok_) <= TIE_RTOL * max(abs(ok_), 1e-30), f"row {r}: id {b}"
        relaxed += 1
    return relaxed


def row_blocks(a: dict) -> np.ndarray:
    """nb of every output row (0 for graph pads), from the oracle arguments."""
    P, H, MB = a["packed_queries"], a["gqa"], a["max_blocks"]
    ln = np.clip(a["row_len"].astype(np.int64), 0, MB * 128)
    nb = (ln + 127) // 128
    pad = (a["req_slot"] < 0) | (a["req_slot"] >= a["n_slot_rows"])
    nb = np.where(np.repeat(pad, P), 0, nb)
    return np.repeat(nb, H)


def assert_parity(g: dict, o: dict, a: dict) -> int:
    assert_scores(g["block_scores"], o["block_scores"])
    n = assert_ids(g["topk_ids"], o["topk_ids"], o["block_scores"], row_blocks(a), a["topk"],
                   a["init_blocks"], a["local_blocks"])
    # scores of the selected ids are the GPU's own block scores
    rows = np.arange(g["topk_ids"].shape[0])[:, None]
    sel = g["topk_ids"] >= 0
    bs = g["block_scores"]
    if bs.shape[1] == 0:  # no block column: nothing can be selected
        bs = np.full((bs.shape[0], 1), -np.inf, dtype=np.float32)
    want = np.where(sel, bs[rows, np.maximum(g["topk_ids"], 0)], -np.inf)
    assert np.array_equal(g["topk_scores"], want, equal_nan=True), "topk_scores != block scores"
    return n
