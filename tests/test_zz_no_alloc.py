"""idx_step_noalloc (the block scores in the library's own device array)
against idx_step (a caller buffer), through the C-ABI: two calls in a row,
the second on a smaller step, each bit-identical to idx_step on the same
inputs, and the smaller one also against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import harness as Hn
from sparse_attention_lightning_amd import idx as I
from sparse_attention_lightning_amd import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not Hn.gpu_ok(), reason="needs an MI355X (gfx950)")]


def say(*a):
    print("[case]", *a, flush=True)


def _noalloc(w: W.Workload, **mode) -> dict:
    outs = {"topk_ids": torch.full((w.rows, w.topk), -7, dtype=torch.int32, device="cuda"),
            "topk_scores": torch.full((w.rows, w.topk), np.nan, dtype=torch.float32, device="cuda")}
    p = I.make_params(k_format=w.k_format, q=w.q, k=w.k, k_scale=w.k_scale, req_slot=w.req_slot,
                      block_table=w.block_table, row_len=w.row_len, block_scores=None, **outs,
                      packed_queries=w.packed_queries, gqa=w.gqa, topk=w.topk,
                      init_blocks=w.init_blocks, local_blocks=w.local_blocks,
                      max_blocks=w.max_blocks, n_slot_rows=w.n_slot_rows, n_pages=w.n_pages, **mode)
    I.idx_step_noalloc(p)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in outs.items()}


def _same(a: dict, b: dict) -> None:
    assert np.array_equal(a["topk_ids"], b["topk_ids"]), "ids differ from idx_step"
    assert np.array_equal(a["topk_scores"], b["topk_scores"], equal_nan=True), "scores differ from idx_step"


def test_noalloc_matches_idx_step_twice(oracle):
    # 1: the 32-request x 524K fp8 step with graph pads (2.29 M block scores)
    say("noalloc: 32req_524k_fp8_3pads")
    big = W.config(3, device="cuda")
    g_big = _noalloc(big)
    _same(g_big, Hn.gpu_step(big))
    del big
    torch.cuda.empty_cache()
    # 2: a smaller step right after it (the array still holds the first
    # call's scores past this step's extent)
    say("noalloc: small fp8 step after it")
    w = W.make(name="noalloc_small", R=5, P=4, H=4, k_format=W.K_FP8_E4M3,
               req_len=[0, 130, 2000, 5000, 777], topk=6, init_blocks=1, local_blocks=2, seed=41,
               pads=1, pad_len=3000, device="cuda")
    g = _noalloc(w)
    ref = Hn.gpu_step(w)
    _same(g, ref)
    a = w.oracle_args()
    o = oracle.step(**a)
    Hn.assert_parity(dict(ref), o, a)
    # and the lse reduction through the same array
    say("noalloc: small step, lse")
    lse = dict(score_mode=I.IDX_SCORE_LSE, sm_scale=0.125)
    _same(_noalloc(w, **lse), Hn.gpu_step(w, **lse))


def test_noalloc_refuses_a_step_too_large():
    say("noalloc: refusal")
    w = W.make(name="noalloc_big", R=1, P=4, H=4, k_format=W.K_BF16, req_len=[300], topk=4,
               init_blocks=1, local_blocks=1, seed=42, max_blocks=I.IDX_MAX_BLOCKS, device="cuda")
    rows = (I.IDX_NOALLOC_MAX_SCORES // (16 * I.IDX_MAX_BLOCKS)) + 1
    q = torch.zeros((rows * 4, 4, 128), dtype=torch.bfloat16, device="cuda")
    outs = {"topk_ids": torch.empty((rows * 16, 4), dtype=torch.int32, device="cuda"),
            "topk_scores": torch.empty((rows * 16, 4), dtype=torch.float32, device="cuda")}
    p = I.make_params(k_format=W.K_BF16, q=q, k=w.k, k_scale=None,
                      req_slot=w.req_slot.repeat(rows), block_table=w.block_table,
                      row_len=w.row_len.repeat(rows), block_scores=None, **outs, packed_queries=4, gqa=4,
                      topk=4, init_blocks=1, local_blocks=1, max_blocks=I.IDX_MAX_BLOCKS)
    with pytest.raises(I.IdxError) as e:
        I.idx_step_noalloc(p)
    assert e.value.code == I.IDX_E_SHAPE and "exceeds" in str(e.value)
