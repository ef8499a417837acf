"""Brute-force reference for tiny inputs (fp64, numpy), independent of the oracle.

It decodes K through torch's own dtype conversions (bf16, float8_e4m3fn) or
takes an already exact value pool, scores every visible token of every row one
block at a time with a numpy matmul, reduces a block with numpy's max or
scipy's logsumexp, and selects blocks by one full sort with the key (not
forced, NaN last, -score, id).  The oracle uses none of this: it
decodes the bits itself, accumulates dots in a loop and selects with a
forced-flag pass plus a sort of the remaining blocks.
"""
from __future__ import annotations

import math

import numpy as np
import torch
from scipy.special import logsumexp

K_BF16, K_FP8_E4M3, K_NVFP4 = 0, 1, 2


def pool_values(k_format: int, k: np.ndarray) -> np.ndarray:
    """Dequantize a bf16 or fp8 K plane to float64 [tokens, 128] via torch."""
    if k_format == K_BF16:
        t = torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).view(torch.bfloat16)
    elif k_format == K_FP8_E4M3:
        t = torch.from_numpy(np.ascontiguousarray(k).view(np.uint8)).view(torch.float8_e4m3fn)
    else:
        raise ValueError("NVFP4 pools are given to the brute force as exact values")
    return t.to(torch.float64).numpy().reshape(-1, 128)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def step(a: dict, pool: np.ndarray) -> dict:
    """Block scores and forced top-k for argument dict ``a`` (oracle layout),
    with K given as float64 values per pool token."""
    R, P, H = a["n_req"], a["packed_queries"], a["gqa"]
    MB, K = a["max_blocks"], a["topk"]
    init, local = a["init_blocks"], a["local_blocks"]
    lse = a.get("score_mode", 0) == 1
    scale = float(a.get("sm_scale", 0.0))
    q = bf16_values(a["q"]).reshape(R * P * H, 128)
    bt = a["block_table"].reshape(a["n_slot_rows"], MB)
    rows = R * P * H
    bs = np.full((rows, MB), -np.inf, dtype=np.float32)
    ids = np.full((rows, K), -1, dtype=np.int32)
    sc = np.full((rows, K), -np.inf, dtype=np.float32)
    for r in range(R):
        slot = int(a["req_slot"][r])
        if not (0 <= slot < a["n_slot_rows"]):
            continue
        for i in range(P * H):
            o = r * P * H + i
            n = int(min(max(int(a["row_len"][r * P + i // H]), 0), MB * 128))
            nb = math.ceil(n / 128)
            for b in range(nb):
                page = int(bt[slot, b])
                if not (0 <= page < a["n_pages"]):
                    bs[o, b] = np.nan
                    continue
                t0 = page * 128
                toks = pool[t0: t0 + min(128, n - 128 * b)]
                s = toks @ q[o]
                bs[o, b] = np.float32(logsumexp(scale * s) if lse else s.max())

            def key(b):
                forced = b < init or b >= nb - local
                s = float(bs[o, b])
                return (not forced, math.isnan(s), 0.0 if math.isnan(s) else -s, b)

            chosen = sorted(sorted(range(nb), key=key)[:K])
            ids[o, : len(chosen)] = chosen
            sc[o, : len(chosen)] = bs[o, chosen]
    return {"block_scores": bs, "topk_ids": ids, "topk_scores": sc}


def select(block_scores: np.ndarray, nb: np.ndarray, topk: int, init: int, local: int):
    """Selection alone, on given float32 block scores [rows, MB] and per-row
    block counts."""
    rows = block_scores.shape[0]
    ids = np.full((rows, topk), -1, dtype=np.int32)
    sc = np.full((rows, topk), -np.inf, dtype=np.float32)
    for o in range(rows):
        n = int(nb[o])

        def key(b):
            forced = b < init or b >= n - local
            s = float(block_scores[o, b])
            return (not forced, math.isnan(s), 0.0 if math.isnan(s) else -s, b)

        chosen = sorted(sorted(range(n), key=key)[:topk])
        ids[o, : len(chosen)] = chosen
        sc[o, : len(chosen)] = block_scores[o, chosen]
    return ids, sc
