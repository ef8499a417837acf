"""Pins of the CPU oracle: checks against facts other than the oracle itself.

Every ``pin_*`` function takes an :class:`oracle.binding.Oracle` and raises
``AssertionError`` when the oracle disagrees with what the pages and the
mathematics fix:

* library routines: torch's float8_e4m3fn decode;
* exact rational arithmetic: E4M3 scale and E2M1 code rounding, exhaustively;
* hand-worked examples and the page's boundary case (``tests/golden``);
* brute force on tiny inputs (``brute.py``);
* invariants: packed == per-row, masking, slot/page permutation, graph pads,
  forced blocks present, NVFP4 == bf16 of the dequantized values.

``test_oracle_pins.py`` runs them on the oracle; ``test_oracle_mutants.py``
runs them on copies with one planted mistake each and requires a failure.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import brute
from sparse_attention_lightning_amd import workloads as W

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def e2m1_table() -> dict[int, float]:
    out = {}
    for line in (GOLDEN / "e2m1_values.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            out[int(c)] = float(v)
    return out


def fp8_values_torch() -> np.ndarray:
    """Value of every e4m3fn byte, via torch's own conversion."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_bits(values) -> np.ndarray:
    t = torch.as_tensor(np.asarray(values, dtype=np.float64)).to(torch.bfloat16)
    out = t.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(t.to(torch.float64).numpy(), np.asarray(values, dtype=np.float64)), \
        "value not exact in bf16"
    return out


def unpack_codes(payload: np.ndarray) -> np.ndarray:
    """Codes of each element: the even element sits in the low nibble (ATOM
    PR 2745, Summary)."""
    lo = payload & 0x0F
    hi = payload >> 4
    return np.stack([lo, hi], axis=-1).reshape(payload.shape[0], -1)


def same(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(a, b, equal_nan=True)


def assert_close_scores(got: np.ndarray, want: np.ndarray, what: str) -> None:
    gi, wi = np.isinf(got), np.isinf(want)
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gi, wi) and np.array_equal(gn, wn), f"{what}: inf/nan layout differs"
    assert np.array_equal(got[gi], want[wi]), f"{what}: inf signs differ"
    f = ~(gi | gn)
    err = np.abs(got[f].astype(np.float64) - want[f]) / np.maximum(np.abs(want[f]), 1.0)
    assert err.size == 0 or err.max() <= 1e-6, f"{what}: max rel err {err.max():.3g}"


def small_workload(k_format: int, seed: int, pads: int = 0, R_lens=(0, 300, 1022, 3000),
                   topk: int = 5, local: int = 2) -> W.Workload:
    return W.make(name="pin", R=len(R_lens), P=4, H=4, k_format=k_format, req_len=list(R_lens),
                  topk=topk, init_blocks=1, local_blocks=local, seed=seed, pads=pads,
                  pad_len=2000)


def exact_fp4_staging(w: W.Workload, seed: int) -> np.ndarray:
    """Overwrite the workload's staging keys with values NVFP4 holds exactly:
    per 16-group a scale s and codes c, value e2m1(c) * s, with one element at
    6 s so that amax / 6 = s.  Returns the float64 values [n_tokens, 128]."""
    rng = np.random.default_rng(seed)
    tab = e2m1_table()
    fp8 = fp8_values_torch()
    n = w.staging.shape[0]
    sb = rng.integers(0x28, 0x48, size=(n, 8))             # scales around 2^-2 .. 2^2
    codes = rng.integers(0, 16, size=(n, 8, 16))
    codes[:, :, 0] = np.where(rng.random((n, 8)) < 0.5, 7, 15)  # one +-6 s per group
    lut = np.array([tab[c] for c in range(16)])
    vals = lut[codes] * fp8[sb][:, :, None]
    vals = vals.reshape(n, 128)
    w.staging.copy_(torch.from_numpy(bf16_bits(vals).view(np.int16)).view(torch.bfloat16))
    return vals


def oracle_fp4_pool(o, w: W.Workload) -> tuple[np.ndarray, np.ndarray]:
    payload = w.k.numpy().copy()
    scales = w.k_scale.numpy().copy()
    stag = w.staging.contiguous().view(torch.int16).numpy().view(np.uint16)
    o.fp4_store(stag, w.slot_mapping.numpy(), payload, scales)
    return payload, scales


def exact_pool_from_staging(w: W.Workload, vals: np.ndarray) -> np.ndarray:
    pool = np.full((w.n_pages * 128, 128), np.nan)
    pool[w.slot_mapping.numpy()] = vals
    return pool


def compare_step(got: dict, want: dict, what: str) -> None:
    assert_close_scores(got["block_scores"], want["block_scores"], what + " block scores")
    assert np.array_equal(got["topk_ids"], want["topk_ids"]), what + ": ids differ"
    assert_close_scores(got["topk_scores"], want["topk_scores"], what + " top-k scores")


def topk_args(nb: np.ndarray, MB: int, topk: int, init: int, local: int, rng) -> dict:
    """Arguments for block_topk alone: one request per row (P = H = 1)."""
    R = len(nb)
    lens = np.where(nb > 0, nb * 128 - rng.integers(0, 128, size=R), 0).astype(np.int32)
    return dict(k_format=W.K_BF16, n_req=R, n_slot_rows=R, packed_queries=1, gqa=1,
                max_blocks=MB, topk=topk, init_blocks=init, local_blocks=local, n_pages=0,
                q=np.zeros((R, 128), np.uint16), k=np.zeros(0, np.uint16),
                req_slot=np.arange(R, dtype=np.int32),
                block_table=np.zeros((R, MB), np.int32), row_len=lens)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def pin_fp8_decode(o) -> None:
    """All 256 e4m3fn bytes decode to torch's float8_e4m3fn value."""
    ref = fp8_values_torch()
    got = np.array([o.fp8_value(c) for c in range(256)])
    assert same(got, ref), "fp8 decode differs from torch float8_e4m3fn"
    # each value is exact in bf16 (the exact widening the pages rely on)
    finite = ref[np.isfinite(ref)]
    assert np.array_equal(torch.tensor(finite).to(torch.bfloat16).double().numpy(), finite)


def pin_e2m1_decode(o) -> None:
    tab = e2m1_table()
    for c in range(16):
        v = o.e2m1_value(c)
        assert v == tab[c] and math.copysign(1, v) == math.copysign(1, tab[c]), c


def pin_golden_store(o) -> None:
    """Hand-worked NVFP4 groups (tests/golden/fp4_store_examples.txt)."""
    groups, scales, codes, bytes_ = [], [], [], []
    for line in (GOLDEN / "fp4_store_examples.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        a, b, c, d = [x.split() for x in line.split("|")]
        groups.append([float(x) for x in a])
        scales.append(int(b[0], 16))
        codes.append([int(x) for x in c])
        bytes_.append([int(x, 16) for x in d])
    n = len(groups)
    vals = np.zeros((n, 8, 16))
    vals[:, 0, :] = groups               # each example is group 0 of its own token
    stag = bf16_bits(vals.reshape(n, 128))
    payload = np.full((n, 64), 0x5A, np.uint8)
    sc = np.full((n, 8), 0x5A, np.uint8)
    o.fp4_store(stag, np.arange(n, dtype=np.int64), payload, sc)
    assert np.array_equal(sc[:, 0], scales), f"scale bytes {sc[:, 0]} != {scales}"
    assert np.array_equal(unpack_codes(payload)[:, :16], np.array(codes)), "codes differ"
    assert np.array_equal(payload[:, :8], np.array(bytes_, np.uint8)), "payload bytes differ"
    # the all-zero groups 1..7: scale 0, codes 0
    assert not sc[:, 1:].any() and not payload[:, 8:].any()


def pin_fp4_roundtrip(o) -> None:
    """Every code at every positive finite scale: the store returns the scale
    byte and codes, and the oracle's decode (read through one-hot queries)
    returns the exact values; every value is exact in bf16."""
    tab = e2m1_table()
    fp8 = fp8_values_torch()
    order = [7, 1, 2, 3, 4, 5, 6, 0, 8, 9, 10, 11, 12, 13, 14, 15]
    sbs = list(range(1, 0x7F))                        # 126 positive finite scales
    ng = len(sbs)
    n_tok = (ng + 7) // 8
    vals = np.zeros((n_tok * 8, 16))
    for g, sb in enumerate(sbs):
        vals[g] = [tab[c] * fp8[sb] for c in order]
    vals = vals.reshape(n_tok, 128)
    stag = bf16_bits(vals)
    payload = np.zeros((n_tok, 64), np.uint8)
    scales = np.zeros((n_tok, 8), np.uint8)
    o.fp4_store(stag, np.arange(n_tok, dtype=np.int64), payload, scales)
    got_sc = scales.reshape(-1)[:ng]
    assert np.array_equal(got_sc, sbs), "scale byte lost in the round trip"
    got_codes = unpack_codes(payload).reshape(-1, 16)[:ng]
    assert np.array_equal(got_codes, np.tile(order, (ng, 1))), "codes lost in the round trip"
    # decode: token t sits at offset 0 of page t; 128 one-hot heads read it back
    R = n_tok
    pay = np.zeros((R * 128, 64), np.uint8)
    ksc = np.zeros((R * 128, 8), np.uint8)
    pay[np.arange(R) * 128] = payload
    ksc[np.arange(R) * 128] = scales
    q = np.tile(bf16_bits(np.eye(128)), (R, 1))
    a = dict(k_format=W.K_NVFP4, n_req=R, n_slot_rows=R, packed_queries=1, gqa=128,
             max_blocks=1, topk=1, init_blocks=1, local_blocks=0, n_pages=R, q=q, k=pay,
             k_scale=ksc, req_slot=np.arange(R, dtype=np.int32),
             block_table=np.arange(R, dtype=np.int32).reshape(R, 1),
             row_len=np.ones(R, np.int32))
    back = o.score_packed(**a)["block_scores"].reshape(R, 128)
    assert np.array_equal(back.astype(np.float64), vals), "decode does not return the values"


def pin_scale_rounding(o) -> None:
    """The group scale is the E4M3 value nearest to amax / 6 (ties to the even
    code, clamped at 448), for every finite non-negative bf16 amax, against
    exact rational arithmetic."""
    fp8 = fp8_values_torch()
    grid = [Fraction(float(fp8[c])) for c in range(0x7F)]  # codes 0..0x7E, ascending
    bits = np.arange(0, 0x7F80, dtype=np.uint32)          # +0 .. largest finite bf16
    amax = (bits << 16).astype(np.uint32).view(np.float32)
    want = np.empty(len(bits), np.uint8)
    import bisect
    for i, a in enumerate(amax):
        t = Fraction(float(a)) / 6
        if t >= 448:
            want[i] = 0x7E
            continue
        lo = bisect.bisect_right(grid, t) - 1
        if grid[lo] == t:
            want[i] = lo
            continue
        dl, dh = t - grid[lo], grid[lo + 1] - t
        want[i] = lo if dl < dh else lo + 1 if dh < dl else (lo if lo % 2 == 0 else lo + 1)
    n = len(bits)
    n_tok = (n + 7) // 8
    g = np.zeros((n_tok * 8, 16), np.uint16)
    g[:n, 0] = bits.astype(np.uint16)
    payload = np.zeros((n_tok, 64), np.uint8)
    scales = np.zeros((n_tok, 8), np.uint8)
    o.fp4_store(g.reshape(n_tok, 128), np.arange(n_tok, dtype=np.int64), payload, scales)
    got = scales.reshape(-1)[:n]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} scale bytes wrong, e.g. amax={amax[bad[0]]!r}"


def _exact_codes(x_bits: np.ndarray, s_val: float) -> np.ndarray:
    """E2M1 code of x / s by exact integer comparison with the midpoints of the
    e2m1 grid (golden table), ties to the even code, saturating at 6."""
    tab = e2m1_table()
    mags = [tab[c] for c in range(8)]
    mid4 = [int((mags[k] + mags[k + 1]) * 2) for k in range(7)]   # 4 x midpoint
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fx, ex = np.frexp(np.abs(x))
    X = np.rint(fx * 256).astype(np.int64)
    a = ex.astype(np.int64) - 8
    fs, es = math.frexp(s_val)
    S, b = int(round(fs * 16)), es - 4
    assert S * 2.0 ** b == s_val
    e = a - b
    mag = np.zeros(len(x), np.int64)
    for k, m4 in enumerate(mid4):
        lhs = np.where(e >= 0, (4 * X) << np.minimum(np.maximum(e, 0), 12), 4 * X)
        rhs = np.where(e >= 0, m4 * S, (m4 * S) << np.minimum(np.maximum(-e, 0), 12))
        mag += (lhs > rhs) | ((lhs == rhs) & (k % 2 == 1))
    sign = (x_bits >> 15).astype(np.int64)
    return (mag | (sign << 3)).astype(np.uint8)


def pin_code_rounding(o) -> None:
    """Every bf16 x with |x| <= 6 s at every positive finite scale s: the code
    equals exact-rational round-half-even of x / s (groups [6 s, x...], so
    the scale is s exactly)."""
    fp8 = fp8_values_torch()
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    posv = (pos << 16).view(np.float32)
    groups, expect, scale_want = [], [], []
    for sb in range(1, 0x7F):
        s = float(fp8[sb])
        lead = bf16_bits([6 * s])[0]
        sel = pos[posv <= 6 * s].astype(np.uint16)
        xs = np.concatenate([sel, sel | 0x8000])
        pad = (-len(xs)) % 15
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 15)
        grp = np.concatenate([np.full((len(xs), 1), lead, np.uint16), xs], axis=1)
        groups.append(grp)
        expect.append(_exact_codes(grp.reshape(-1), s).reshape(-1, 16))
        scale_want.append(np.full(len(grp), sb, np.uint8))
    groups = np.concatenate(groups)
    expect = np.concatenate(expect)
    scale_want = np.concatenate(scale_want)
    n = len(groups)
    padg = (-n) % 8
    groups = np.concatenate([groups, np.zeros((padg, 16), np.uint16)])
    n_tok = len(groups) // 8
    payload = np.zeros((n_tok, 64), np.uint8)
    scales = np.zeros((n_tok, 8), np.uint8)
    o.fp4_store(groups.reshape(n_tok, 128), np.arange(n_tok, dtype=np.int64), payload, scales)
    got_sc = scales.reshape(-1)[:n]
    assert np.array_equal(got_sc, scale_want), "scale of a [6s, ...] group is not s"
    got = unpack_codes(payload).reshape(-1, 16)[:n]
    bad = np.argwhere(got != expect)
    assert bad.size == 0, f"{len(bad)} codes differ from exact rounding, first at {bad[0]}"


# ---------------------------------------------------------------------------
# scoring and selection
# ---------------------------------------------------------------------------
def pin_bruteforce_bf16(o) -> None:
    w = small_workload(W.K_BF16, seed=11, pads=1)
    a = w.oracle_args()
    compare_step(o.step(**a), brute.step(a, brute.pool_values(W.K_BF16, a["k"])), "bf16")


def pin_bruteforce_fp8(o) -> None:
    w = small_workload(W.K_FP8_E4M3, seed=12, pads=1)
    a = w.oracle_args()
    compare_step(o.step(**a), brute.step(a, brute.pool_values(W.K_FP8_E4M3, a["k"])), "fp8")


def pin_bruteforce_fp4(o) -> None:
    w = small_workload(W.K_NVFP4, seed=13, pads=1)
    vals = exact_fp4_staging(w, seed=13)
    payload, scales = oracle_fp4_pool(o, w)
    a = w.oracle_args(payload, scales)
    compare_step(o.step(**a), brute.step(a, exact_pool_from_staging(w, vals)), "nvfp4")


def pin_bruteforce_lse(o) -> None:
    """lse block scores against scipy's logsumexp over the visible tokens (the
    sglang PR 45451 Accuracy Tests check the lse of the selected blocks)."""
    for fmt, seed in ((W.K_BF16, 15), (W.K_FP8_E4M3, 16)):
        w = small_workload(fmt, seed=seed, pads=1)
        a = dict(w.oracle_args(), score_mode=1, sm_scale=0.3)
        compare_step(o.step(**a), brute.step(a, brute.pool_values(fmt, a["k"])), f"lse {fmt}")


def pin_lse_closed_form(o) -> None:
    """A block whose visible tokens all hold the same key has lse =
    c * q.k + ln(visible tokens); checked on every valid block, partial last
    blocks included."""
    w = small_workload(W.K_BF16, seed=17, R_lens=(300, 1022, 129))
    a = dict(w.oracle_args(), score_mode=1, sm_scale=0.125)
    k = a["k"].reshape(w.n_pages, 128, 128).copy()
    k[:] = k[:, :1, :]  # every token of a page repeats the page's first key
    a["k"] = k.reshape(-1, 128)
    got = o.score_packed(**a)["block_scores"]
    q = brute.bf16_values(a["q"]).reshape(-1, 128)
    kv = brute.bf16_values(k[:, 0, :])
    bt = a["block_table"].reshape(a["n_slot_rows"], -1)
    rows = 16
    checked = 0
    for r in range(w.n_req):
        slot = int(a["req_slot"][r])
        for i in range(rows):
            n = int(a["row_len"][r * 4 + i // 4])
            for b in range((n + 127) // 128):
                vis = min(128, n - 128 * b)
                want = 0.125 * float(q[r * rows + i] @ kv[bt[slot, b]]) + np.log(vis)
                g = float(got[r * rows + i, b])
                assert abs(g - want) <= 1e-6 * max(abs(want), 1.0), (r, i, b, g, want)
                checked += 1
    assert checked > 100


def pin_lse_bounds(o) -> None:
    """c * max <= lse <= c * max + ln(visible tokens) on every valid block,
    with the max from the max mode of the same oracle."""
    w = small_workload(W.K_FP8_E4M3, seed=18)
    a = w.oracle_args()
    mx = o.score_packed(**a)["block_scores"].astype(np.float64)
    ls = o.score_packed(**dict(a, score_mode=1, sm_scale=0.7))["block_scores"].astype(np.float64)
    assert np.array_equal(np.isinf(mx), np.isinf(ls)), "lse and max disagree on which blocks are empty"
    f = np.isfinite(mx)
    lens = np.repeat(a["row_len"].astype(np.int64), 4).reshape(-1, 1)
    vis = np.clip(lens - 128 * np.arange(mx.shape[1])[None, :], 0, 128)
    tol = 1e-6 * np.maximum(np.abs(ls), 1.0)
    assert np.all(ls[f] >= 0.7 * mx[f] - tol[f]), "lse below c * max"
    assert np.all(ls[f] <= 0.7 * mx[f] + np.log(vis[f]) + tol[f]), "lse above c * max + ln n"


def pin_fp4_equals_bf16_of_dequant(o) -> None:
    """NVFP4 scoring equals bf16 scoring fed the dequantized keys, bit for bit
    (ATOM PR 2745, Validation: e2m1 x E4M3 values are exact in bf16)."""
    w = small_workload(W.K_NVFP4, seed=14)
    vals = exact_fp4_staging(w, seed=14)
    payload, scales = oracle_fp4_pool(o, w)
    a4 = w.oracle_args(payload, scales)
    pool = np.full((w.n_pages * 128, 128), 8192.0)
    pool[w.slot_mapping.numpy()] = vals
    a16 = dict(a4, k_format=W.K_BF16, k=bf16_bits(pool), k_scale=None)
    r4, r16 = o.step(**a4), o.step(**a16)
    for key in r4:
        assert same(r4[key], r16[key]), f"nvfp4 and bf16-of-dequant differ in {key}"


def pin_topk_textbook(o) -> None:
    """With no forced blocks, selection is numpy's stable argsort of -score."""
    rng = np.random.default_rng(21)
    MB, topk = 50, 7
    nb = rng.integers(0, MB + 1, size=64)
    bs = rng.standard_normal((64, MB)).astype(np.float32)
    bs[:, 1::3] = bs[:, ::3][:, : bs[:, 1::3].shape[1]]   # plant exact ties
    a = topk_args(nb, MB, topk, 0, 0, rng)
    got = o.block_topk(bs, **a)
    for r in range(64):
        n = nb[r]
        want = np.arange(n) if n <= topk else np.sort(np.argsort(-bs[r, :n], kind="stable")[:topk])
        row = got["topk_ids"][r]
        assert np.array_equal(row[: len(want)], want) and (row[len(want):] == -1).all(), r


def pin_topk_bruteforce(o) -> None:
    """Forced top-k against one full sort, on scores with many exact ties and
    a few NaN (NaN ranks below every number)."""
    rng = np.random.default_rng(22)
    MB, topk = 40, 8
    for init, local in [(0, 0), (1, 0), (0, 2), (1, 2), (3, 1), (2, 6)]:
        nb = rng.integers(0, MB + 1, size=80)
        bs = rng.choice(np.array([-1.0, 0.0, 0.5, 1.0, 2.0], np.float32), size=(80, MB))
        bs[rng.random((80, MB)) < 0.03] = np.nan
        a = topk_args(nb, MB, topk, init, local, rng)
        got = o.block_topk(bs, **a)
        ids, sc = brute.select(bs, nb, topk, init, local)
        assert np.array_equal(got["topk_ids"], ids), (init, local)
        assert same(got["topk_scores"], sc), (init, local)


def _check_invariants(a: dict, res: dict) -> None:
    P, H, K = a["packed_queries"], a["gqa"], a["topk"]
    init, local, MB = a["init_blocks"], a["local_blocks"], a["max_blocks"]
    for r in range(a["n_req"]):
        pad = not (0 <= a["req_slot"][r] < a["n_slot_rows"])
        for i in range(P * H):
            o = r * P * H + i
            ids = res["topk_ids"][o]
            n = min(max(int(a["row_len"][r * P + i // H]), 0), MB * 128)
            nb = 0 if pad else (n + 127) // 128
            sel = ids[ids >= 0]
            assert (ids[len(sel):] == -1).all() and np.isneginf(res["topk_scores"][o][len(sel):]).all()
            assert np.all(np.diff(sel) > 0), "ids not ascending"
            if nb <= K:
                assert np.array_equal(sel, np.arange(nb)), "nb <= topk must select every block"
            else:
                forced = set(range(min(init, nb))) | set(range(max(nb - local, 0), nb))
                assert forced <= set(sel.tolist()), "forced block missing"
                assert len(sel) == K
            assert same(res["topk_scores"][o][: len(sel)], res["block_scores"][o][sel])


def pin_topk_invariants(o) -> None:
    for fmt, seed in [(W.K_BF16, 31), (W.K_FP8_E4M3, 32)]:
        w = small_workload(fmt, seed, pads=1, topk=6, local=3)
        a = w.oracle_args()
        _check_invariants(a, o.step(**a))


def pin_exact_tie(o) -> None:
    """Two blocks with bit-identical pages tie exactly; with one free slot the
    lower block id wins."""
    w = W.make(name="tie", R=2, P=4, H=4, k_format=W.K_BF16, req_len=[2000, 2500], topk=4,
               init_blocks=1, local_blocks=2, seed=41)
    b1, b2 = 3, 9
    a = w.oracle_args()
    k = a["k"].reshape(w.n_pages, 128, 128)
    bt = a["block_table"]
    s0 = a["req_slot"][0]
    p1, p2 = bt[s0, b1], bt[s0, b2]
    kv = torch.from_numpy(k[p1].view(np.int16)).view(torch.bfloat16) * 8   # exact
    k[p1] = kv.view(torch.int16).numpy().view(np.uint16)
    k[p2] = k[p1]
    res = o.step(**a)
    for i in range(16):
        bs = res["block_scores"][i]
        assert bs[b1] == bs[b2]
        ids = set(res["topk_ids"][i].tolist())
        assert b1 in ids and b2 not in ids, f"row {i}: tie not resolved to the lower id"


def pin_straddle(o) -> None:
    """Rows ending at 32767..32770 (tests/golden/straddle_32767.txt)."""
    gold = []
    for line in (GOLDEN / "straddle_32767.txt").read_text().splitlines():
        if line.strip() and not line.startswith("#"):
            f = line.split()
            gold.append((int(f[0]), int(f[1]), int(f[2]),
                         [int(x) for x in f[3].split(",")], [int(x) for x in f[4].split(",")]))
    for fmt, local in [(W.K_BF16, 2), (W.K_FP8_E4M3, 2), (W.K_FP8_E4M3, 0)]:
        w = W.make(name="straddle", R=4, P=4, H=2, k_format=fmt, req_len=[32767] * 4, topk=8,
                   init_blocks=1, local_blocks=local, seed=51 + fmt + local)
        a = w.oracle_args()
        res = o.step(**a)
        compare_step(res, brute.step(a, brute.pool_values(fmt, a["k"])), "straddle")
        for r in range(4):
            for i in range(8):
                ln, nb, last, f2, f0 = gold[i // 2]
                o_ = r * 8 + i
                assert int(a["row_len"][r * 4 + i // 2]) == ln
                bs = res["block_scores"][o_]
                assert np.isfinite(bs[:nb]).all() and np.isneginf(bs[nb:]).all(), "block count"
                forced = f2 if local == 2 else f0
                assert set(forced) <= set(res["topk_ids"][o_].tolist()), "forced set"


def pin_packed_equals_per_row(o) -> None:
    """Scoring a request's rows packed gives exactly what scoring each
    (draft row, head) as its own request gives (sglang PR 45451 and 42614:
    packed max scores and IDs equal the per-row kernel's)."""
    for fmt, seed in [(W.K_BF16, 61), (W.K_FP8_E4M3, 62)]:
        w = small_workload(fmt, seed, pads=1)
        a = w.oracle_args()
        R, P, H = a["n_req"], a["packed_queries"], a["gqa"]
        per = dict(a, n_req=R * P * H, packed_queries=1, gqa=1,
                   q=a["q"].reshape(R * P * H, 128),
                   req_slot=np.repeat(a["req_slot"], P * H),
                   row_len=np.repeat(a["row_len"], H))
        rp, rr = o.step(**a), o.step(**per)
        for key in rp:
            assert same(rp[key], rr[key]), f"packed != per-row in {key}"


def pin_many_rows_equal_per_row(o) -> None:
    """Requests with many query rows (a prefill chunk: row j sees L + j
    tokens, 4 heads, 300 rows a request) score exactly as each row run as its
    own request, and the max scores match the brute force."""
    w = W.make(name="pin_rows", R=2, P=75, H=4, k_format=W.K_FP8_E4M3, req_len=[700, 2000], topk=5,
               init_blocks=1, local_blocks=2, seed=63, pads=1, pad_len=500)
    a = w.oracle_args()
    R, P, H = a["n_req"], a["packed_queries"], a["gqa"]
    per = dict(a, n_req=R * P * H, packed_queries=1, gqa=1, q=a["q"].reshape(R * P * H, 128),
               req_slot=np.repeat(a["req_slot"], P * H), row_len=np.repeat(a["row_len"], H))
    rp, rr = o.step(**a), o.step(**per)
    for key in rp:
        assert same(rp[key], rr[key]), f"many rows != per-row in {key}"
    compare_step(rp, brute.step(a, brute.pool_values(W.K_FP8_E4M3, a["k"])), "many rows")


def _token_loc(a: dict, r: int, pos: int) -> int:
    slot = a["req_slot"][r]
    page = a["block_table"][slot, pos // 128]
    return int(page) * 128 + pos % 128


def pin_masking(o) -> None:
    """Keys a row cannot see never change its results: poison the tokens past
    the shortest row of each request; that row's outputs stay the same and the
    longest row's change."""
    for fmt, seed in [(W.K_BF16, 71), (W.K_FP8_E4M3, 72)]:
        w = small_workload(fmt, seed)
        a = w.oracle_args()
        base = o.step(**a)
        k = a["k"].reshape(-1, 128).copy()
        big = bf16_bits([8192.0])[0] if fmt == W.K_BF16 else W.POISON_FP8_CODE
        for r, L in enumerate(w.req_len):
            for pos in range(int(L), int(L) + 3):
                k[_token_loc(a, r, pos)] = big
        res = o.step(**dict(a, k=k.reshape(a["k"].shape)))
        P, H = 4, 4
        changed = False
        for r, L in enumerate(w.req_len):
            for i in range(P * H):
                o_ = r * P * H + i
                if i // H == 0:
                    for key in res:
                        assert same(res[key][o_], base[key][o_]), f"row saw masked keys ({key})"
                elif i // H == 3 and L > 0:
                    changed |= not same(res["block_scores"][o_], base["block_scores"][o_])
        assert changed, "poisoned keys were not visible to the longer rows"


def pin_slot_permutation(o) -> None:
    """Relabelling request slots and physical pages changes no output
    (sglang PR 42614: K is addressed through the slot table)."""
    w = small_workload(W.K_FP8_E4M3, 81)
    a = w.oracle_args()
    rng = np.random.default_rng(82)
    sigma = rng.permutation(a["n_slot_rows"]).astype(np.int32)
    pi = rng.permutation(a["n_pages"]).astype(np.int32)
    bt = a["block_table"]
    bt2 = np.full_like(bt, -1)
    for s in range(a["n_slot_rows"]):
        row = bt[s]
        bt2[sigma[s]] = np.where(row >= 0, pi[np.maximum(row, 0)], -1)
    k = a["k"].reshape(a["n_pages"], 128, 128)
    k2 = np.empty_like(k)
    k2[pi] = k
    a2 = dict(a, req_slot=sigma[a["req_slot"]], block_table=bt2, k=k2.reshape(a["k"].shape))
    r1, r2 = o.step(**a), o.step(**a2)
    for key in r1:
        assert same(r1[key], r2[key]), f"slot/page relabelling changed {key}"


def pin_graph_pads(o) -> None:
    """Graph-pad requests (slot past the request table) emit sentinels and
    leave the real rows bit-identical (sglang PR 42614, Modifications 1)."""
    w = small_workload(W.K_BF16, 91, pads=2)
    a = w.oracle_args()
    R, P, H = w.n_real, 4, 4
    real = dict(a, n_req=R, q=a["q"][: R * P], req_slot=a["req_slot"][:R],
                row_len=a["row_len"][: R * P])
    full, part = o.step(**a), o.step(**real)
    n = R * P * H
    for key in full:
        assert same(full[key][:n], part[key]), f"pads changed real rows ({key})"
    assert np.isneginf(full["block_scores"][n:]).all()
    assert (full["topk_ids"][n:] == -1).all() and np.isneginf(full["topk_scores"][n:]).all()


def pin_bad_page_ids(o) -> None:
    """A visible block whose page id lies outside [0, n_pages) (negative, one
    past the pool, far past it) is not read: every row that sees it scores
    NaN, rows that do not see it keep -inf, every other block is bit-equal to
    the run with valid ids, and selection ranks the NaN below every number.
    This is the library's stated rule for bad tables (the pages give none);
    it is checked against the brute force and against the valid-table run,
    for the max and the lse."""
    for fmt, mode in ((W.K_BF16, {}), (W.K_FP8_E4M3, {}),
                      (W.K_FP8_E4M3, {"score_mode": 1, "sm_scale": 0.2})):
        # request 2's rows see 3070..3073 tokens: 24, 24, 24 and 25 blocks
        w = small_workload(fmt, seed=95, R_lens=(300, 1022, 3070), topk=6, local=1)
        a = dict(w.oracle_args(), **mode)
        base = o.step(**a)
        bt = a["block_table"].copy()
        s1, s2 = int(a["req_slot"][1]), int(a["req_slot"][2])
        bad = {(1, 2): a["n_pages"] + 5, (1, 7): a["n_pages"],   # block 7: the last of request 1
               (2, 0): -3, (2, 10): 1 << 30, (2, 24): a["n_pages"]}  # block 24: seen by row 3 only
        for (r, b), pg in bad.items():
            bt[(s1, s2)[r - 1], b] = pg
        a2 = dict(a, block_table=bt)
        got = o.step(**a2)
        compare_step(got, brute.step(a2, brute.pool_values(fmt, a["k"])), f"bad pages {fmt} {mode}")
        bs, bs0 = got["block_scores"], base["block_scores"]
        P, H = 4, 4
        want = bs0.copy()
        for (r, b), _ in bad.items():
            for i in range(P * H):
                L = int(a["row_len"][r * P + i // H])
                if b < (L + 127) // 128:
                    want[r * P * H + i, b] = np.nan
        assert same(bs, want), f"bad pages {fmt} {mode}: block scores are not NaN exactly where seen"
        # row 3 of request 2 sees block 24 (NaN); rows 0..2 do not (-inf)
        assert np.isnan(bs[2 * 16 + 12: 2 * 16 + 16, 24]).all()
        assert np.isneginf(bs[2 * 16: 2 * 16 + 12, 24]).all()
        # a NaN block is taken only when forced (block 0, block 24 as row 3's local window)
        for o_ in range(bs.shape[0]):
            for b in got["topk_ids"][o_][got["topk_ids"][o_] >= 0]:
                if np.isnan(bs[o_, b]):
                    nb = int(np.isfinite(bs0[o_]).sum())
                    assert b < 1 or b >= nb - 1 or nb <= 6, f"row {o_} selected NaN block {b}"


# ---------------------------------------------------------------------------
# sparse attention over the selected blocks
# ---------------------------------------------------------------------------
ATTN_SCALE = float(np.float32(128 ** -0.5))  # an fp32 number, as the interface carries it


def attn_workload(seed: int, lens=(0, 130, 700, 1500), P: int = 3, H: int = 2, G: int = 3, pads: int = 1,
                  kv_format: int = W.K_BF16):
    w = W.make(name="attn", R=len(lens), P=P, H=H, k_format=W.K_BF16, req_len=list(lens), topk=4,
                init_blocks=1, local_blocks=1, seed=seed, pads=pads, pad_len=900)
    return w, W.make_attn(w, G, seed=seed + 1, kv_format=kv_format)


def random_selection(w, rng, topk: int, messy: bool = True) -> np.ndarray:
    """Per (draft row, KV head) a random set of the row's blocks, ascending,
    padded with -1; with ``messy`` some rows also list an id twice, an id
    past the row's blocks and one past max_blocks (all to be ignored)."""
    rows = w.n_req * w.packed_queries
    lens = w.row_len.numpy()
    ids = np.full((rows, w.gqa, topk), -1, np.int32)
    for row in range(rows):
        nb = (int(lens[row]) + 127) // 128
        for h in range(w.gqa):
            n = int(min(nb, rng.integers(1, topk - 2))) if nb else 0
            chosen = np.sort(rng.choice(nb, size=n, replace=False)) if n else np.zeros(0, int)
            ids[row, h, :n] = chosen
            if messy and n and rng.random() < 0.6:
                ids[row, h, n:n + 3] = [chosen[0], nb + 1, w.max_blocks + 7][: topk - n]
    return ids


def assert_attn_close(got: dict, want: dict, what: str, rtol: float = 1e-6) -> None:
    for key in ("out", "lse"):
        g = np.asarray(got[key], np.float64)
        x = np.asarray(want[key], np.float64)
        assert g.shape == x.shape, (what, key, g.shape, x.shape)
        assert np.array_equal(np.isnan(g), np.isnan(x)), f"{what} {key}: NaN layout differs"
        assert np.array_equal(np.isinf(g), np.isinf(x)), f"{what} {key}: inf layout differs"
        f = np.isfinite(x)
        err = np.abs(g[f] - x[f]) / np.maximum(np.abs(x[f]), 1e-3)
        assert err.size == 0 or err.max() <= rtol, f"{what} {key}: max rel err {err.max():.3g}"


def pin_attn_bruteforce(o) -> None:
    """Oracle against scipy's softmax / logsumexp and numpy gathers over the
    visible tokens of each row's selected blocks: random selections (with
    duplicates, ids past the row and past max_blocks), partial last blocks,
    several KV heads and query heads a KV head, a graph pad."""
    w, at = attn_workload(611)
    ids = random_selection(w, np.random.default_rng(612), topk=6)
    a = W.attn_oracle_args(w, at, ids, ATTN_SCALE)
    assert_attn_close(o.sparse_attn(**a), brute.sparse_attn(a), "attn brute force")


def pin_attn_fp8(o) -> None:
    """fp8 e4m3 K/V: the oracle against brute force over torch's float8_e4m3fn
    decode, and equal (bit for bit) to the bf16 path given the same values
    widened to bf16, which holds every e4m3 value exactly (3 mantissa bits,
    exponents 2^-9 to 2^8)."""
    w, at = attn_workload(615, kv_format=W.K_FP8_E4M3)
    ids = random_selection(w, np.random.default_rng(616), topk=6)
    a = W.attn_oracle_args(w, at, ids, ATTN_SCALE)
    got = o.sparse_attn(**a)
    assert_attn_close(got, brute.sparse_attn(a), "attn fp8 brute force")
    wide = W.AttnInputs(at.q_per_kv, at.q, at.k.to(torch.bfloat16), at.v.to(torch.bfloat16), at.seed)
    ref = o.sparse_attn(**W.attn_oracle_args(w, wide, ids, ATTN_SCALE))
    for key in ("out", "lse"):
        assert np.array_equal(got[key], ref[key], equal_nan=True), f"attn fp8 vs widened bf16: {key}"


def pin_attn_loops(o) -> None:
    """The same against plain Python loops and math.exp on a tiny case."""
    w, at = attn_workload(621, lens=(40, 200), P=2, H=2, G=2, pads=0)
    ids = random_selection(w, np.random.default_rng(622), topk=4)
    a = W.attn_oracle_args(w, at, ids, 0.3)
    assert_attn_close(o.sparse_attn(**a), brute.sparse_attn_loops(a), "attn loops")


def pin_attn_dense(o) -> None:
    """Every block selected: causal attention over the whole visible context,
    from torch's scaled_dot_product_attention in float64 with each row's
    length mask (and torch.logsumexp for the lse)."""
    w, at = attn_workload(631, lens=(129, 300, 1022), P=4, H=2, G=2, pads=0)
    R, P, H, G = w.n_req, 4, 2, 2
    lens = w.row_len.numpy()
    nbmax = int((lens.max() + 127) // 128)
    ids = np.full((R * P, H, nbmax), -1, np.int32)
    for row in range(R * P):
        nb = (int(lens[row]) + 127) // 128
        ids[row, :, :nb] = np.arange(nb)
    a = W.attn_oracle_args(w, at, ids, ATTN_SCALE)
    got = o.sparse_attn(**a)
    k64 = at.k.to(torch.float64)
    v64 = at.v.to(torch.float64)
    q64 = at.q.to(torch.float64)
    bt = w.block_table.numpy()
    for r in range(R):
        slot = int(w.req_slot[r])
        L = int(lens[r * P: r * P + P].max())
        pages = torch.as_tensor(bt[slot, : (L + 127) // 128].astype(np.int64))
        for h in range(H):
            kc = k64[pages, h].reshape(-1, 128)[:L]                       # [L, 128] in position order
            vc = v64[pages, h].permute(0, 1, 3, 2).reshape(-1, 128)[:L]   # [L, 128] in position order
            for j in range(P):
                row = r * P + j
                mask = torch.arange(L) < int(lens[row])
                qq = q64[row, h][None, :, None, :]                        # [1, G, 1, 128]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, kc[None, None].expand(1, G, L, 128), vc[None, None].expand(1, G, L, 128),
                    attn_mask=mask[None, None, None, :], scale=ATTN_SCALE)[0, :, 0, :]
                s = ATTN_SCALE * (q64[row, h] @ kc.T)
                lse = torch.logsumexp(s.masked_fill(~mask[None, :], -math.inf), dim=1)
                assert_attn_close({"out": got["out"][row, h], "lse": got["lse"][row, h]},
                                  {"out": ref.numpy(), "lse": lse.numpy()}, f"dense row {row} head {h}")


def pin_attn_closed_forms(o) -> None:
    """(1) The same V column for every token: the output is that column,
    exactly, whatever the weights.  (2) The same key for every token: the
    weights are uniform, so the output is the mean of the visible selected V
    columns and lse = c q.k0 + ln n.  (3) A row of one token: its V column,
    lse = c q.k."""
    rng = np.random.default_rng(641)
    w, at = attn_workload(641)
    ids = random_selection(w, rng, topk=6, messy=False)
    R, P, H, G = w.n_req, w.packed_queries, w.gqa, at.q_per_kv
    col = torch.randn(128, generator=torch.Generator().manual_seed(642)).to(torch.bfloat16)
    v_const = at.v.clone()
    v_const[:] = col[None, None, None, :, None]
    res = o.sparse_attn(**W.attn_oracle_args(w, W.AttnInputs(G, at.q, at.k, v_const, at.seed), ids, ATTN_SCALE))
    lens = w.row_len.numpy()
    for row in range(R * P):
        r = row // P
        real = r < w.n_real and lens[row] > 0
        for h in range(H):
            if real and (ids[row, h] >= 0).any():
                assert np.array_equal(res["out"][row, h], np.broadcast_to(col.float().numpy(), (G, 128))), \
                    f"constant V: row {row} head {h}"
            else:
                assert (res["out"][row, h] == 0).all() and np.isneginf(res["lse"][row, h]).all()
    # (2) equal keys
    k0 = torch.randn(128, generator=torch.Generator().manual_seed(643)).to(torch.bfloat16)
    k_eq = at.k.clone()
    k_eq[:] = k0
    res = o.sparse_attn(**W.attn_oracle_args(w, W.AttnInputs(G, at.q, k_eq, at.v, at.seed), ids, ATTN_SCALE))
    v64 = at.v.to(torch.float64).numpy()
    bt = w.block_table.numpy()
    q64 = at.q.to(torch.float64).numpy()
    for row in range(R * P):
        r = row // P
        if r >= w.n_real or lens[row] == 0:
            continue
        for h in range(H):
            cols = []
            for b in sorted(set(ids[row, h][ids[row, h] >= 0].tolist())):
                page = bt[int(w.req_slot[r]), b]
                cols += [v64[page, h, t // 32, :, t % 32] for t in range(min(128, int(lens[row]) - 128 * b))]
            n = len(cols)
            s0 = ATTN_SCALE * (q64[row, h] @ k0.double().numpy())
            assert_attn_close({"out": res["out"][row, h], "lse": res["lse"][row, h]},
                              {"out": np.broadcast_to(np.mean(cols, axis=0), (G, 128)), "lse": s0 + math.log(n)},
                              f"equal keys row {row} head {h}", rtol=1e-5)
    # (3) one visible token
    w1, at1 = attn_workload(644, lens=(1, 1), P=1, H=2, G=3, pads=0)
    ids1 = np.zeros((2, 2, 1), np.int32)
    res = o.sparse_attn(**W.attn_oracle_args(w1, at1, ids1, ATTN_SCALE))
    bt1 = w1.block_table.numpy()
    for r in range(2):
        page = bt1[int(w1.req_slot[r]), 0]
        for h in range(2):
            want = at1.v[page, h, 0, :, 0].float().numpy()
            assert np.array_equal(res["out"][r, h], np.broadcast_to(want, (3, 128))), "one token: V column"
            s = ATTN_SCALE * (at1.q[r, h].double().numpy() @ at1.k[page, h, 0].double().numpy())
            assert np.allclose(res["lse"][r, h], s, rtol=1e-6, atol=1e-6), "one token: lse"


def pin_attn_invariants(o) -> None:
    """Reordered, duplicated and ignored ids change nothing; neither do the
    K and V of unselected blocks and of tokens past a row's length; graph
    pads give 0 and -inf; a selected block on a page outside the pool makes
    exactly the rows that see it NaN."""
    rng = np.random.default_rng(651)
    w, at = attn_workload(651)
    ids = random_selection(w, rng, topk=7, messy=False)
    a = W.attn_oracle_args(w, at, ids, ATTN_SCALE)
    base = o.sparse_attn(**a)
    shuffled = ids.copy()
    for row in range(ids.shape[0]):
        for h in range(ids.shape[1]):
            sel = ids[row, h][ids[row, h] >= 0]
            extra = [-1, w.max_blocks, 99999] + (list(sel[:1]) if len(sel) else [])
            lst = list(rng.permutation(sel)) + extra
            shuffled[row, h] = (lst + [-1] * 7)[:7]
    got = o.sparse_attn(**dict(a, topk_ids=shuffled))
    for key in base:
        assert same(got[key], base[key]), f"id order / duplicates / ignored ids changed {key}"
    # poison what no row of that head may use: unselected blocks, tokens past each row
    k2, v2 = at.k.clone(), at.v.clone()
    bt = w.block_table.numpy()
    lens = w.row_len.numpy()
    P = w.packed_queries
    for r in range(w.n_real):
        slot = int(w.req_slot[r])
        nbg = (int(lens[r * P: r * P + P].max()) + 127) // 128
        for h in range(w.gqa):
            used = set(ids[r * P: r * P + P, h][ids[r * P: r * P + P, h] >= 0].tolist())
            for b in range(nbg):
                if b not in used:
                    k2[bt[slot, b], h] = 7
                    v2[bt[slot, b], h] = -5000
    res = o.sparse_attn(**W.attn_oracle_args(w, W.AttnInputs(at.q_per_kv, at.q, k2, v2, at.seed), ids, ATTN_SCALE))
    for key in base:
        assert same(res[key], base[key]), f"unselected blocks changed {key}"
    n_real_rows = w.n_real * P
    assert (base["out"][n_real_rows:] == 0).all() and np.isneginf(base["lse"][n_real_rows:]).all(), "pads"
    # a selected block on a bad page
    bt_bad = bt.copy()
    row, h = 3 * P - 1, 1            # request 2's longest row, head 1
    b = int(ids[row, h][0])
    bt_bad[int(w.req_slot[2]), b] = w.n_pages + 3
    res = o.sparse_attn(**dict(a, block_table=np.ascontiguousarray(bt_bad)))
    for rr in range(ids.shape[0]):
        for hh in range(w.gqa):
            sees = (rr // P == 2 and b in ids[rr, hh].tolist() and 128 * b < lens[rr])
            if sees:
                assert np.isnan(res["out"][rr, hh]).all() and np.isnan(res["lse"][rr, hh]).all(), (rr, hh)
            else:
                assert same(res["out"][rr, hh], base["out"][rr, hh]), (rr, hh)
    assert np.isnan(res["lse"][row, h]).all()


PINS = [
    pin_fp8_decode, pin_e2m1_decode, pin_golden_store, pin_fp4_roundtrip,
    pin_bruteforce_bf16, pin_bruteforce_fp8, pin_bruteforce_fp4, pin_fp4_equals_bf16_of_dequant,
    pin_bruteforce_lse, pin_lse_closed_form, pin_lse_bounds,
    pin_topk_textbook, pin_topk_bruteforce, pin_topk_invariants, pin_exact_tie, pin_straddle,
    pin_packed_equals_per_row, pin_many_rows_equal_per_row, pin_masking, pin_slot_permutation,
    pin_graph_pads, pin_bad_page_ids,
    pin_attn_bruteforce, pin_attn_fp8, pin_attn_loops, pin_attn_dense, pin_attn_closed_forms, pin_attn_invariants,
    pin_scale_rounding, pin_code_rounding,
]
