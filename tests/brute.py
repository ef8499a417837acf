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


# ---------------------------------------------------------------------------
# sparse attention over the selected blocks
# ---------------------------------------------------------------------------
def _attn_rows(a: dict):
    """Yield (row, h, g, visible token list as (page, t), bad) per query head."""
    R, P, H, G, MB, K = a["n_req"], a["packed_queries"], a["kv_heads"], a["q_per_kv"], a["max_blocks"], a["topk"]
    bt = a["block_table"].reshape(a["n_slot_rows"], MB)
    ids = a["topk_ids"].reshape(R * P, H, K)
    for row in range(R * P):
        r = row // P
        slot = int(a["req_slot"][r])
        pad = not (0 <= slot < a["n_slot_rows"])
        n = int(min(max(int(a["row_len"][row]), 0), MB * 128))
        for h in range(H):
            toks, bad = [], False
            if not pad:
                chosen = sorted({int(b) for b in ids[row, h] if 0 <= b < math.ceil(n / 128)})
                for b in chosen:
                    page = int(bt[slot, b])
                    if not (0 <= page < a["n_pages"]):
                        bad = True
                        continue
                    toks += [(page, t) for t in range(min(128, n - 128 * b))]
            for g in range(G):
                yield row, h, g, toks, bad


def kv_values(a: dict, arr: np.ndarray) -> np.ndarray:
    """A main K or V pool as float64, decoded by torch (bf16 or float8_e4m3fn)."""
    if a.get("kv_format", K_BF16) == K_FP8_E4M3:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.uint8)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    return bf16_values(arr)


def sparse_attn(a: dict) -> dict:
    """fp64 reference: for each query head, scipy's softmax and logsumexp over
    the scaled dots with the visible tokens of its selected blocks (numpy
    gathers and matmuls), then the weighted sum of their V columns."""
    from scipy.special import logsumexp, softmax
    R, P, H, G = a["n_req"], a["packed_queries"], a["kv_heads"], a["q_per_kv"]
    q = bf16_values(a["q"]).reshape(R * P, H, G, 128)
    k = kv_values(a, a["k"]).reshape(a["n_pages"], H, 128, 128)
    v = kv_values(a, a["v"]).reshape(a["n_pages"], H, 4, 128, 32)   # [page][h][token / 32][dim][token % 32]
    scale = float(np.float32(a["sm_scale"]))  # the softmax scale crosses the interface as fp32
    out = np.zeros((R * P, H, G, 128))
    lse = np.full((R * P, H, G), -np.inf)
    for row, h, g, toks, bad in _attn_rows(a):
        if bad:
            out[row, h, g], lse[row, h, g] = np.nan, np.nan
            continue
        if not toks:
            continue
        pg = np.array([p for p, _ in toks])
        tt = np.array([t for _, t in toks])
        s = scale * (k[pg, h, tt, :] @ q[row, h, g])
        out[row, h, g] = softmax(s) @ v[pg, h, tt // 32, :, tt % 32]
        lse[row, h, g] = logsumexp(s)
    return {"out": out, "lse": lse}


def sparse_attn_loops(a: dict) -> dict:
    """The same in plain Python loops and math.exp (tiny inputs only)."""
    R, P, H, G = a["n_req"], a["packed_queries"], a["kv_heads"], a["q_per_kv"]
    q = bf16_values(a["q"]).reshape(R * P, H, G, 128).tolist()
    k = kv_values(a, a["k"]).reshape(a["n_pages"], H, 128, 128)
    v = kv_values(a, a["v"]).reshape(a["n_pages"], H, 4, 128, 32)
    out = [[[[0.0] * 128 for _ in range(G)] for _ in range(H)] for _ in range(R * P)]
    lse = [[[-math.inf] * G for _ in range(H)] for _ in range(R * P)]
    for row, h, g, toks, bad in _attn_rows(a):
        if bad:
            out[row][h][g] = [math.nan] * 128
            lse[row][h][g] = math.nan
            continue
        if not toks:
            continue
        s = []
        for p_, t in toks:
            kr = k[p_, h, t].tolist()
            s.append(float(np.float32(a["sm_scale"])) * sum(x * y for x, y in zip(q[row][h][g], kr)))
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        o = [0.0] * 128
        for wi, (p_, t) in zip(w, toks):
            col = v[p_, h, t // 32, :, t % 32].tolist()
            for d in range(128):
                o[d] += wi * col[d]
        out[row][h][g] = [x / tot for x in o]
        lse[row][h][g] = m + math.log(tot)
    return {"out": np.array(out), "lse": np.array(lse)}
