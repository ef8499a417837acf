"""HIP path vs the CPU oracle on an MI355X (through the C-ABI).

Small cases are compared in full.  The five decode workloads run at full size
in the launch configuration the benchmark times and are compared in full too:
every row of every request, graph pads included, and every byte of the NVFP4
planes.  The prefill workload is compared on every one of its 32,768 rows too,
plus properties that hold at any size.
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


def say(*a):
    print("[case]", *a, flush=True)


# ---------------------------------------------------------------------------
# small shapes, full comparison
# ---------------------------------------------------------------------------
SHAPES = [  # (P, H, lens of the requests, topk, init, local, pads)
    (4, 2, [1000, 1500], 4, 1, 1, 0),                  # the tiny workload's shape
    (4, 4, [0, 1, 127, 128, 300, 1022, 3000], 5, 1, 2, 2),
    (1, 1, [5, 129, 2000], 3, 1, 1, 1),
    (2, 8, [640, 700], 6, 2, 0, 0),
    (1, 16, [4095, 77], 8, 0, 3, 1),
    (16, 1, [513, 2049], 7, 1, 2, 0),
    (3, 5, [260, 1031, 30], 4, 1, 3, 1),
]


@pytest.mark.parametrize("fmt", [W.K_BF16, W.K_FP8_E4M3, W.K_NVFP4], ids=["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("shape", range(len(SHAPES)))
def test_small_shapes(oracle, fmt, shape):
    P, H, lens, topk, init, local, pads = SHAPES[shape]
    say("small", fmt, SHAPES[shape])
    w = W.make(name="small", R=len(lens), P=P, H=H, k_format=fmt, req_len=lens, topk=topk,
               init_blocks=init, local_blocks=local, seed=100 + shape, pads=pads,
               pad_len=4096, device="cuda")
    if fmt == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        payload, scales = Hn.oracle_pool(oracle, w)
        assert np.array_equal(w.k.cpu().numpy(), payload), "fp4 payload bytes differ"
        assert np.array_equal(w.k_scale.cpu().numpy(), scales), "fp4 scale bytes differ"
        a = w.oracle_args(payload, scales)
    else:
        a = w.oracle_args()
    g = Hn.gpu_step(w)
    o = oracle.step(**a)
    Hn.assert_parity(g, o, a)


def test_tiny_workload(oracle):
    say("tiny workload, full comparison")
    w = W.config(0, device="cuda")
    a = w.oracle_args()
    g, o = Hn.gpu_step(w), oracle.step(**a)
    Hn.assert_parity(g, o, a)
    assert np.array_equal(g["topk_ids"], o["topk_ids"])


def test_invalid_page_ids(oracle):
    """Page ids outside the pool are not read; the rows that see the block
    get NaN, and selection ranks NaN below every number."""
    say("invalid page ids")
    w = W.make(name="badpage", R=3, P=4, H=4, k_format=W.K_FP8_E4M3, req_len=[900, 1500, 400],
               topk=4, init_blocks=1, local_blocks=1, seed=7, device="cuda")
    bt = w.block_table
    s0, s1 = int(w.req_slot[0]), int(w.req_slot[1])
    bt[s0, 2] = w.n_pages + 5
    bt[s1, 0] = -3
    bt[s1, 11] = 1 << 30
    a = w.oracle_args()
    g, o = Hn.gpu_step(w), oracle.step(**a)
    Hn.assert_parity(g, o, a)
    assert np.isnan(g["block_scores"][:16, 2]).all() and np.isnan(g["block_scores"][16:32, 0]).all()


# ---------------------------------------------------------------------------
# NVFP4 store
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("copies", [1, 2], ids=["eight_lanes", "four_lanes"])
def test_fp4_store_exhaustive_rounding(oracle, copies):
    """Every bf16 x with |x| <= 6 s at every positive finite E4M3 scale s
    (4.2M values) stored by the GPU and by the oracle: identical bytes.  The
    set is 39,162 keys; twice over (78,324) it goes through the kernel that
    stores 65,536 keys or more four lanes a key."""
    say("fp4 store exhaustive rounding set", copies)
    fp8 = pins.fp8_values_torch()
    pos = np.arange(0, 0x7F80, dtype=np.uint32)
    posv = (pos << 16).view(np.float32)
    groups = []
    for sb in range(1, 0x7F):
        s = float(fp8[sb])
        lead = pins.bf16_bits([6 * s])[0]
        sel = pos[posv <= 6 * s].astype(np.uint16)
        xs = np.concatenate([sel, sel | 0x8000])
        xs = np.concatenate([xs, np.zeros((-len(xs)) % 15, np.uint16)]).reshape(-1, 15)
        groups.append(np.concatenate([np.full((len(xs), 1), lead, np.uint16), xs], axis=1))
    # also every amax (scale rounding), one group each
    amax = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    g2 = np.zeros((len(amax), 16), np.uint16)
    g2[:, 0] = amax
    groups.append(g2)
    groups = np.concatenate(groups)
    groups = np.concatenate([groups, np.zeros(((-len(groups)) % 8, 16), np.uint16)])
    st = np.concatenate([groups.reshape(-1, 128)] * copies)
    n = st.shape[0]
    perm = np.random.default_rng(3).permutation(n).astype(np.int64)   # scattered slots
    pay_o = np.full((n, 64), 0x5A, np.uint8)
    sc_o = np.full((n, 8), 0x5A, np.uint8)
    oracle.fp4_store(st, perm, pay_o, sc_o)
    stg = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).cuda()
    pay_g = torch.full((n, 64), 0x5A, dtype=torch.uint8, device="cuda")
    sc_g = torch.full((n, 8), 0x5A, dtype=torch.uint8, device="cuda")
    I.idx_fp4_store(stg, torch.from_numpy(perm).cuda(), pay_g, sc_g)
    torch.cuda.synchronize()
    assert np.array_equal(sc_g.cpu().numpy(), sc_o), "scale bytes differ"
    assert np.array_equal(pay_g.cpu().numpy(), pay_o), "payload bytes differ"


@pytest.mark.parametrize("n", [3000, 80000], ids=["eight_lanes", "four_lanes"])
def test_fp4_store_skips_and_strides(oracle, n):
    """Negative and out-of-range slots are skipped (their bytes keep the
    fill); a staging row stride larger than 128 is honoured.  Both store
    kernels (four lanes a key from 65,536 keys)."""
    say("fp4 store skip/stride", n)
    n_slots = n - 500
    rng = np.random.default_rng(5)
    big = torch.randn(n, 200, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    st = big[:, :128]
    slots = np.concatenate([rng.permutation(n_slots).astype(np.int64), np.full(n - n_slots, -1)])
    slots[rng.random(n) < 0.05] = -9
    slots[rng.random(n) < 0.05] = n_slots + 17
    pay_o = np.full((n_slots, 64), 0x33, np.uint8)
    sc_o = np.full((n_slots, 8), 0x33, np.uint8)
    st_np = np.ascontiguousarray(st.view(torch.int16).numpy().view(np.uint16))
    oracle.fp4_store(st_np, slots, pay_o, sc_o)
    pay_g = torch.full((n_slots, 64), 0x33, dtype=torch.uint8, device="cuda")
    sc_g = torch.full((n_slots, 8), 0x33, dtype=torch.uint8, device="cuda")
    big_g = big.cuda()
    I.idx_fp4_store(big_g[:, :128], torch.from_numpy(slots).cuda(), pay_g, sc_g)
    torch.cuda.synchronize()
    assert np.array_equal(pay_g.cpu().numpy(), pay_o) and np.array_equal(sc_g.cpu().numpy(), sc_o)


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------
def test_packed_equals_per_row():
    """Each (draft row, head) run as its own request gives bit-identical
    block scores and ids (sglang PR 45451: packed max scores equal the
    per-row kernel's)."""
    for fmt in (W.K_BF16, W.K_FP8_E4M3):
        say("packed == per-row", fmt)
        w = W.make(name="pk", R=4, P=4, H=4, k_format=fmt, req_len=[0, 300, 1022, 3000], topk=5,
                   init_blocks=1, local_blocks=2, seed=61, pads=1, pad_len=2000, device="cuda")
        g = Hn.gpu_step(w)
        R, P, H = w.n_req, 4, 4
        per = W.Workload(**{**w.__dict__})
        per.n_req, per.packed_queries, per.gqa = R * P * H, 1, 1
        per.q = w.q.reshape(R * P * H, 1, 128).contiguous()
        per.req_slot = w.req_slot.repeat_interleave(P * H).contiguous()
        per.row_len = w.row_len.repeat_interleave(H).contiguous()
        gp = Hn.gpu_step(per)
        for key in g:
            assert np.array_equal(g[key], gp[key], equal_nan=True), f"packed != per-row ({key})"


def test_batch_invariance():
    """A probe request's outputs do not depend on the other requests of the
    launch (alone, with others, with pads) (ATOM PR 2485, Why / Test)."""
    say("batch invariance")
    base = W.make(name="bi", R=6, P=4, H=4, k_format=W.K_FP8_E4M3,
                  req_len=[2000, 50, 7000, 333, 4100, 1], topk=6, init_blocks=1, local_blocks=2,
                  seed=71, pads=2, pad_len=3000, device="cuda")
    full = Hn.gpu_step(base)
    rows = 16
    for probe in (0, 2, 4):
        for others in ([], [1], [3, 5], [1, 3, 5, 6, 7]):
            sel = [probe] + others
            sub = W.Workload(**{**base.__dict__})
            idx_t = torch.as_tensor(sel, device="cuda")
            sub.n_req = len(sel)
            sub.q = base.q.reshape(base.n_req, rows, 128)[idx_t].reshape(-1, 4, 128).contiguous()
            sub.req_slot = base.req_slot[idx_t].contiguous()
            sub.row_len = base.row_len.reshape(base.n_req, 4)[idx_t].reshape(-1).contiguous()
            g = Hn.gpu_step(sub)
            for key in full:
                assert np.array_equal(g[key][:rows], full[key][probe * rows:(probe + 1) * rows],
                                      equal_nan=True), (probe, others, key)


def test_masked_keys_never_seen():
    """Poisoning keys past the shortest row changes nothing for that row."""
    say("masking")
    w = W.make(name="mask", R=4, P=4, H=4, k_format=W.K_BF16, req_len=[0, 300, 1022, 3000],
               topk=5, init_blocks=1, local_blocks=2, seed=81, device="cuda")
    base = Hn.gpu_step(w)
    bt = w.block_table.cpu().numpy()
    slots = w.req_slot.cpu().numpy()
    for r, L in enumerate(w.req_len):
        for pos in range(int(L), int(L) + 3):
            page = int(bt[slots[r], pos // 128])
            w.k[page * 128 + pos % 128] = 8192.0
    res = Hn.gpu_step(w)
    for r in range(4):
        o0 = r * 16
        for key in res:
            assert np.array_equal(res[key][o0:o0 + 4], base[key][o0:o0 + 4], equal_nan=True)


def test_exact_tie_lower_id():
    """Bit-identical pages tie exactly; with one free slot the lower id wins."""
    say("exact tie")
    w = W.make(name="tie", R=2, P=4, H=4, k_format=W.K_BF16, req_len=[2000, 2500], topk=4,
               init_blocks=1, local_blocks=2, seed=41, device="cuda")
    b1, b2 = 3, 9
    s0 = int(w.req_slot[0])
    p1, p2 = int(w.block_table[s0, b1]), int(w.block_table[s0, b2])
    kv = w.k.view(w.n_pages, 128, 128)
    kv[p1] *= 8
    kv[p2] = kv[p1]
    g = Hn.gpu_step(w)
    for i in range(16):
        assert g["block_scores"][i, b1] == g["block_scores"][i, b2]
        ids = set(g["topk_ids"][i].tolist())
        assert b1 in ids and b2 not in ids


@pytest.mark.parametrize("R", [48, 1100], ids=["wg_per_row", "wave_per_row"])
def test_topk_synthetic_scores_exact(oracle, R):
    """Selection alone on the same fp32 scores (many exact ties, NaN, -0):
    ids and scores identical to the oracle's.  1,100 rows of at most 1,024
    blocks take the one-wave-per-row kernel and 1,100 rows of 1,025 to 2,048
    blocks the workgroup kernel with 256 threads; 48 rows the workgroup kernel
    with 512 threads (4 blocks a thread up to 2,048 blocks, 8 up to 4,096, 16
    beyond)."""
    rng = np.random.default_rng(9)
    for MB, topk, init, local in [(40, 8, 1, 2), (300, 64, 1, 2), (1000, 64, 0, 0), (8192, 64, 3, 5),
                                  (700, 1, 1, 0), (50, 50, 2, 2), (1024, 64, 1, 2), (2048, 64, 1, 2),
                                  (2052, 100, 2, 3), (4096, 64, 1, 2), (1190, 64, 1, 2)]:
        say("topk synthetic", R, MB, topk, init, local)
        nb = rng.integers(0, MB + 1, size=R)
        nb[:3] = [MB, topk, topk + 1]
        vals = np.array([-1.0, 0.0, -0.0, 0.5, 1.0, 2.0, np.nan, -np.inf], np.float32)
        bs = rng.choice(vals, size=(R, MB), p=[.2, .1, .1, .2, .2, .14, .03, .03]).astype(np.float32)
        bs[R // 2:] = rng.standard_normal((R - R // 2, MB)).astype(np.float32)
        a = pins.topk_args(nb, MB, topk, init, local, rng)
        o = oracle.block_topk(bs, **a)
        dev = "cuda"
        outs = {"block_scores": torch.from_numpy(bs).to(dev),
                "topk_ids": torch.full((R, topk), -7, dtype=torch.int32, device=dev),
                "topk_scores": torch.full((R, topk), 7.0, dtype=torch.float32, device=dev)}
        p = I.make_params(k_format=W.K_BF16, q=None, k=None, k_scale=None,
                          req_slot=torch.from_numpy(a["req_slot"]).to(dev), block_table=None,
                          row_len=torch.from_numpy(a["row_len"]).to(dev), packed_queries=1, gqa=1,
                          topk=topk, init_blocks=init, local_blocks=local, max_blocks=MB,
                          n_slot_rows=R, n_pages=0, **outs)
        I.idx_block_topk(p)
        torch.cuda.synchronize()
        assert np.array_equal(outs["topk_ids"].cpu().numpy(), o["topk_ids"])
        assert np.array_equal(outs["topk_scores"].cpu().numpy(), o["topk_scores"], equal_nan=True)


def test_fp4_equals_bf16_of_dequant():
    """NVFP4 scoring equals bf16 scoring fed the dequantized keys (ATOM PR
    2745, Validation): ids identical, scores within fp32 summation noise."""
    say("nvfp4 == bf16 of dequant")
    w = W.make(name="x", R=4, P=4, H=4, k_format=W.K_NVFP4, req_len=[0, 300, 1022, 3000], topk=5,
               init_blocks=1, local_blocks=2, seed=14, device="cuda")
    vals = pins.exact_fp4_staging(w, seed=14)   # exactly representable keys
    Hn.gpu_fp4_store(w)
    g4 = Hn.gpu_step(w)
    pool = np.full((w.n_pages * 128, 128), 8192.0)
    pool[w.slot_mapping.cpu().numpy()] = vals
    w16 = W.Workload(**{**w.__dict__})
    w16.k_format = W.K_BF16
    w16.k = torch.from_numpy(pins.bf16_bits(pool).view(np.int16)).view(torch.bfloat16).cuda()
    w16.k_scale = None
    g16 = Hn.gpu_step(w16)
    assert np.array_equal(g4["topk_ids"], g16["topk_ids"])
    a, b = g4["block_scores"], g16["block_scores"]
    f = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), f)
    assert np.max(np.abs(a[f] - b[f]) / np.maximum(np.abs(b[f]), 1)) <= 1e-5


@pytest.mark.parametrize("mode", ["max", "lse"])
@pytest.mark.parametrize("P,H", [(4, 4), (40, 4)], ids=["one_tile", "many_rows"])
def test_repeat_launches_identical(P, H, mode):
    """Repeated launches give bit-identical outputs (the graph-replay
    analogue of sglang PR 45451's tests), in both kernels and both score
    modes (the many-rows lse fold keeps a base per row across blocks)."""
    say("determinism", P, H, mode)
    m = LSE if mode == "lse" else {}
    w = W.make(name="det", R=5, P=P, H=H, k_format=W.K_FP8_E4M3, req_len=[100, 900, 4000, 1, 2222],
               topk=8, init_blocks=1, local_blocks=2, seed=91, device="cuda")
    first = Hn.gpu_step(w, **m)
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs, **m)
    for _ in range(50):
        I.idx_step(p)
    torch.cuda.synchronize()
    for key in first:
        assert np.array_equal(outs[key].cpu().numpy(), first[key], equal_nan=True)


# ---------------------------------------------------------------------------
# many requests: a workgroup's share spans several rounds (a round touches at
# most 8 requests), up to the request-count limit
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R,maxlen,fmt", [(2000, 1000, W.K_FP8_E4M3), (I.IDX_MAX_REQ - 2, 300, W.K_BF16)],
                         ids=["2000req", "max_req"])
def test_many_requests(oracle, R, maxlen, fmt):
    say("many requests", R, maxlen, fmt)
    rng = np.random.default_rng(R)
    lens = rng.integers(1, maxlen + 1, size=R)
    w = W.make(name="many", R=R, P=1, H=1, k_format=fmt, req_len=lens, topk=3, init_blocks=1,
               local_blocks=1, seed=R, pads=2, pad_len=maxlen, device="cuda")
    assert w.n_req <= I.IDX_MAX_REQ
    a = w.oracle_args()
    g = Hn.gpu_step(w)
    o = oracle.step(**a)
    Hn.assert_parity(g, o, a)


def test_shares_longer_than_a_round(oracle):
    """More than 768 pages per workgroup: a share runs as several rounds."""
    R, L = 50, 4000 * 128
    say("long shares", R, L)
    w = W.make(name="long", R=R, P=4, H=4, k_format=W.K_FP8_E4M3, req_len=np.full(R, L - 3),
               topk=64, init_blocks=1, local_blocks=2, seed=77, device="cuda")
    assert w.pool_pages_used() > 256 * 768
    a = w.oracle_args()
    g = Hn.gpu_step(w)
    sample = [0, 24, 49]
    sub = Hn.subset_args(a, sample, 4, 4)
    o = oracle.step(**sub)
    Hn.assert_parity({k: v[Hn.rows_of(sample, 16)] for k, v in g.items()}, o, sub)


# ---------------------------------------------------------------------------
# the five workloads at full size, in the benchmark's launch configuration:
# every row of every request (graph pads included) against the oracle, and
# for NVFP4 every byte of both planes
# ---------------------------------------------------------------------------
_POOLS: dict = {}


def _oracle_pool_full(oracle, w):
    """The oracle's NVFP4 planes for all of the workload's staging keys (one
    store per workload and session: the max and lse tests share it)."""
    key = (w.name, w.seed)
    if key not in _POOLS:
        _POOLS.clear()
        _POOLS[key] = Hn.oracle_pool(oracle, w)
    return _POOLS[key]


def _full(oracle, idx, local_blocks=None, **mode):
    say("workload", W.CONFIG_NAMES[idx], "local", local_blocks, mode, "every row")
    w = W.config(idx, device="cuda", local_blocks=local_blocks)
    if w.k_format == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        payload, scales = _oracle_pool_full(oracle, w)
        # every slot: written ones bit-exact, the rest still hold their fill
        assert np.array_equal(w.k.cpu().numpy(), payload), "fp4 payload bytes differ"
        assert np.array_equal(w.k_scale.cpu().numpy(), scales), "fp4 scale bytes differ"
        say("fp4 store: all", w.slot_mapping.numel(), "keys identical")
        a = w.oracle_args(payload, scales)
    else:
        a = w.oracle_args()
    a = dict(a, **mode)
    g = Hn.gpu_step(w, **mode)
    o = oracle.step(**a)
    relaxed = Hn.assert_parity(g, o, a)
    nbs = Hn.row_blocks(a)
    msg = (f"{w.name} local={w.local_blocks} {mode.get('score_mode', 0) and 'lse' or 'max'}: "
           f"{g['topk_ids'].shape[0]} rows compared, {relaxed} near-tie rows")
    say(msg)
    conftest.REPORT.append(msg)
    assert np.isneginf(g["block_scores"][nbs == 0]).all()
    return g, relaxed


def test_workload_1_bf16_131k(oracle):
    _full(oracle, 1)


@pytest.mark.parametrize("local", [2, 0])
def test_workload_2_fp8_straddle(oracle, local):
    g, _ = _full(oracle, 2, local_blocks=local)
    # the straddling requests: rows end at 32767..32770 -> 256/256/257/257 blocks
    for r in range(4):
        for j, nb in enumerate([256, 256, 257, 257]):
            for h in range(4):
                row = g["block_scores"][r * 16 + j * 4 + h]
                assert np.isfinite(row[:nb]).all() and np.isneginf(row[nb:]).all()


def test_workload_3_fp8_524k_pads(oracle):
    g, _ = _full(oracle, 3)
    pads = g["topk_ids"][32 * 16:]
    assert (pads == -1).all() and np.isneginf(g["block_scores"][32 * 16:]).all()


def test_workload_3_shares_do_not_change_results():
    """Shares this long follow the XCDs' rates measured on the previous
    launch, so repeated steps cut the pages differently; every output stays
    bit-identical."""
    say("workload", W.CONFIG_NAMES[3], "repeated steps")
    w = W.config(3, device="cuda")
    first = Hn.gpu_step(w)
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)
    for _ in range(4):
        I.idx_step(p)
    torch.cuda.synchronize()
    for key in first:
        assert np.array_equal(outs[key].cpu().numpy(), first[key], equal_nan=True), key


def test_workload_4_nvfp4_150k(oracle):
    _full(oracle, 4)


# ---------------------------------------------------------------------------
# lse block scores (sglang PR 45451, Accuracy Tests: the selected-block scores
# are checked as the max and as the lse)
# ---------------------------------------------------------------------------
LSE = dict(score_mode=I.IDX_SCORE_LSE, sm_scale=float(1 / np.sqrt(128)))


@pytest.mark.parametrize("fmt", [W.K_BF16, W.K_FP8_E4M3, W.K_NVFP4], ids=["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("shape", [1, 2, 4, 6])
def test_lse_small_shapes(oracle, fmt, shape):
    P, H, lens, topk, init, local, pads = SHAPES[shape]
    say("lse small", fmt, SHAPES[shape])
    w = W.make(name="lse", R=len(lens), P=P, H=H, k_format=fmt, req_len=lens, topk=topk,
               init_blocks=init, local_blocks=local, seed=200 + shape, pads=pads,
               pad_len=4096, device="cuda")
    if fmt == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        a = w.oracle_args(*Hn.oracle_pool(oracle, w))
    else:
        a = w.oracle_args()
    a = dict(a, **LSE)
    Hn.assert_parity(Hn.gpu_step(w, **LSE), oracle.step(**a), a)


@pytest.mark.parametrize("P,H", [(4, 4), (20, 2)], ids=["one_tile", "many_rows"])
@pytest.mark.parametrize("scale", [1e-6, 0.01, 1.0, 4.0, 1000.0])
def test_lse_scales(oracle, scale, P, H):
    """Small and large softmax scales (a large one makes the block's max term
    dominate, far past where exp of the raw terms would overflow; a small one
    sums 128 terms of nearly equal size)."""
    say("lse scale", scale, P, H)
    w = W.make(name="lse_scale", R=3, P=P, H=H, k_format=W.K_FP8_E4M3, req_len=[5000, 129, 2000],
               topk=6, init_blocks=1, local_blocks=2, seed=303, device="cuda")
    mode = dict(score_mode=I.IDX_SCORE_LSE, sm_scale=scale)
    a = dict(w.oracle_args(), **mode)
    Hn.assert_parity(Hn.gpu_step(w, **mode), oracle.step(**a), a)


def test_lse_invalid_page_ids(oracle):
    say("lse invalid page ids")
    w = W.make(name="lse_badpage", R=2, P=4, H=4, k_format=W.K_BF16, req_len=[900, 1500],
               topk=4, init_blocks=1, local_blocks=1, seed=8, device="cuda")
    w.block_table[int(w.req_slot[0]), 3] = w.n_pages + 1
    w.block_table[int(w.req_slot[1]), 0] = -1
    a = dict(w.oracle_args(), **LSE)
    g, o = Hn.gpu_step(w, **LSE), oracle.step(**a)
    assert np.isnan(o["block_scores"]).any()
    Hn.assert_parity(g, o, a)


def test_lse_workload_3_fp8_524k_pads(oracle):
    g, _ = _full(oracle, 3, **LSE)
    assert (g["topk_ids"][32 * 16:] == -1).all() and np.isneginf(g["block_scores"][32 * 16:]).all()


def test_lse_workload_4_nvfp4_150k(oracle):
    _full(oracle, 4, **LSE)


def _full_prefill(oracle, **mode):
    """The prefill workload at full size in the bench's launch configuration:
    the oracle scores every query row of every request (32,768 rows), each
    compared with the acceptance rule, and every row's selection is checked
    for validity as well."""
    say("workload", W.CONFIG_NAMES[5], mode, "every row")
    w = W.config(5, device="cuda")
    a = dict(w.oracle_args(), **mode)
    g = Hn.gpu_step(w, **mode)
    o = oracle.step(**a)
    relaxed = Hn.assert_parity(g, o, a)
    msg = (f"{w.name} local={w.local_blocks} {mode.get('score_mode', 0) and 'lse' or 'max'}: "
           f"{g['topk_ids'].shape[0]} rows compared, {relaxed} near-tie rows")
    say(msg)
    conftest.REPORT.append(msg)
    nbs = Hn.row_blocks(a)
    ids = g["topk_ids"]
    taken = (ids >= 0).sum(axis=1)
    assert np.array_equal(taken, np.minimum(nbs, w.topk)), "selection sizes"
    assert np.all(np.diff(ids, axis=1)[ids[:, 1:] >= 0] > 0), "taken ids ascending and distinct"
    assert np.all(ids[nbs > 0, 0] == 0), "block 0 (init) is always taken"
    last = np.take_along_axis(ids, np.maximum(taken - 1, 0)[:, None], axis=1)[:, 0]
    assert np.array_equal(last, nbs - 1), "the row's last block (local) is always taken"


def test_max_blocks_limit(oracle):
    """A request at the block limit: its longest row sees exactly
    IDX_MAX_BLOCKS * 128 tokens (1,048,576), beside a short one."""
    say("max blocks", I.IDX_MAX_BLOCKS)
    lmax = I.IDX_MAX_BLOCKS * 128
    w = W.make(name="maxblocks", R=2, P=4, H=4, k_format=W.K_FP8_E4M3, req_len=[lmax - 3, 5000], topk=64,
               init_blocks=1, local_blocks=2, seed=81, device="cuda")
    assert w.max_blocks == I.IDX_MAX_BLOCKS
    a = w.oracle_args()
    Hn.assert_parity(Hn.gpu_step(w), oracle.step(**a), a)


def test_max_blocks_limit_many_rows(oracle):
    """The many-rows kernel at the block limit: 20 rows of one request whose
    longest row sees 1,048,576 tokens, so its blocks are cut into chunks."""
    say("max blocks, many rows", I.IDX_MAX_BLOCKS)
    P, lmax = 20, I.IDX_MAX_BLOCKS * 128
    w = W.make(name="maxblocks_rows", R=2, P=P, H=1, k_format=W.K_FP8_E4M3,
               req_len=[lmax - P - 2, 3000], topk=64, init_blocks=1, local_blocks=2, seed=83,
               device="cuda")
    assert w.max_blocks == I.IDX_MAX_BLOCKS
    a = w.oracle_args()
    Hn.assert_parity(Hn.gpu_step(w), oracle.step(**a), a)


def test_max_rows_per_request(oracle):
    """One request at the rows limit: packed_queries x gqa = IDX_MAX_REQ_ROWS
    (16,384 causal query rows x 4 heads); sampled query rows against the
    oracle, every row's selection checked."""
    say("max rows a request", I.IDX_MAX_REQ_ROWS)
    P, H = I.IDX_MAX_REQ_ROWS // 4, 4
    w = W.make(name="maxrows", R=1, P=P, H=H, k_format=W.K_BF16, req_len=[300], topk=8,
               init_blocks=1, local_blocks=2, seed=82, device="cuda")
    a = w.oracle_args()
    g = Hn.gpu_step(w)
    qrows = [0, 1, 511, 512, 8191, 8192, P - 2, P - 1]
    sub = Hn.subset_rows_args(a, 0, qrows, P, H)
    rows = (np.asarray(qrows)[:, None] * H + np.arange(H)[None, :]).reshape(-1)
    Hn.assert_parity({k: v[rows] for k, v in g.items()}, oracle.step(**sub), sub)
    nbs = Hn.row_blocks(a)
    ids = g["topk_ids"]
    assert np.array_equal((ids >= 0).sum(axis=1), np.minimum(nbs, w.topk))
    assert np.all(np.diff(ids, axis=1)[ids[:, 1:] >= 0] > 0), "taken ids ascending and distinct"


def test_workload_5_prefill_32k_fp8(oracle):
    _full_prefill(oracle)


def test_lse_workload_5_prefill_32k_fp8(oracle):
    _full_prefill(oracle, **LSE)


# ---------------------------------------------------------------------------
# more than 16 rows a request: tiles of 16 rows, 64 sharing each K page (the
# prefill scorer of ATOM PR 2745's Summary; wide packs).  Row j of a request
# sees L + j tokens, which is the causal length of a prefill chunk's rows.
# ---------------------------------------------------------------------------
ROW_SHAPES = [  # (P, H, lens of the requests, topk, init, local, pads)
    (5, 4, [300, 1022, 3000], 5, 1, 2, 1),      # 20 rows: one item, a partial wave
    (32, 1, [129, 4000], 4, 1, 1, 0),           # 32 rows, one head
    (100, 4, [5000, 64, 700], 8, 1, 2, 1),      # 400 rows: 7 row groups, causal extents
    (3, 7, [2047, 2048, 2049], 6, 0, 3, 0),     # 21 rows, seven heads
]


@pytest.mark.parametrize("mode", ["max", "lse"])
@pytest.mark.parametrize("fmt", [W.K_BF16, W.K_FP8_E4M3, W.K_NVFP4], ids=["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("shape", range(len(ROW_SHAPES)))
def test_many_rows_shapes(oracle, fmt, shape, mode):
    P, H, lens, topk, init, local, pads = ROW_SHAPES[shape]
    say("many rows", fmt, mode, ROW_SHAPES[shape])
    w = W.make(name="rows", R=len(lens), P=P, H=H, k_format=fmt, req_len=lens, topk=topk,
               init_blocks=init, local_blocks=local, seed=400 + shape, pads=pads,
               pad_len=3000, device="cuda")
    if fmt == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        a = w.oracle_args(*Hn.oracle_pool(oracle, w))
    else:
        a = w.oracle_args()
    m = LSE if mode == "lse" else {}
    a = dict(a, **m)
    Hn.assert_parity(Hn.gpu_step(w, **m), oracle.step(**a), a)


def test_many_rows_equal_per_row():
    """A request's 200 rows give bit-identical outputs to each row run as its
    own request through the one-tile kernel."""
    say("many rows == per-row")
    w = W.make(name="rows_pr", R=2, P=50, H=4, k_format=W.K_FP8_E4M3, req_len=[900, 3000], topk=5,
               init_blocks=1, local_blocks=2, seed=71, pads=1, pad_len=2000, device="cuda")
    g = Hn.gpu_step(w)
    R, P, H = w.n_req, 50, 4
    per = W.Workload(**{**w.__dict__})
    per.n_req, per.packed_queries, per.gqa = R * P * H, 1, 1
    per.q = w.q.reshape(R * P * H, 1, 128).contiguous()
    per.req_slot = w.req_slot.repeat_interleave(P * H).contiguous()
    per.row_len = w.row_len.repeat_interleave(H).contiguous()
    gp = Hn.gpu_step(per)
    for key in g:
        assert np.array_equal(g[key], gp[key], equal_nan=True), f"many rows != per-row ({key})"


@pytest.mark.parametrize("mb", [48, 272])
def test_many_rows_output_layouts(oracle, mb):
    """The many-rows kernel's block-score writes: with max_blocks a multiple
    of 16 the scores leave in whole 64-byte granules staged in LDS, chunk
    boundaries rounded to four blocks and odd chunks walking backwards; the
    same step into a block-score array one float off 16-byte alignment takes
    the value-by-value path.  Both equal the oracle and each other bit for
    bit, with -inf past each row group's extent (prefill-like causal rows,
    a short request, a graph pad)."""
    say("many rows output layouts, max_blocks", mb)
    kw = dict(name="layout", R=3, P=64, H=4, k_format=W.K_FP8_E4M3, req_len=[1000, 5000, 60], topk=8,
              init_blocks=1, local_blocks=2, seed=560 + mb, pads=1, pad_len=2000, max_blocks=mb)
    w = W.make(**kw, device="cuda")
    aligned = Hn.gpu_step(w)
    # the same into views one float past 16-byte alignment
    rows = w.rows
    big = torch.full((rows * mb + 4,), float("nan"), dtype=torch.float32, device="cuda")
    outs = {"block_scores": big[1:1 + rows * mb].view(rows, mb),
            "topk_ids": torch.full((rows, w.topk), -7, dtype=torch.int32, device="cuda"),
            "topk_scores": torch.full((rows, w.topk), float("nan"), dtype=torch.float32, device="cuda")}
    assert outs["block_scores"].data_ptr() % 16 == 4
    I.idx_step(Hn.gpu_params(w, outs))
    torch.cuda.synchronize()
    shifted = {k: v.cpu().numpy() for k, v in outs.items()}
    for key in aligned:
        assert np.array_equal(aligned[key], shifted[key], equal_nan=True), key
    a = w.oracle_args()
    Hn.assert_parity(aligned, oracle.step(**a), a)


def test_many_rows_granule_chunks(oracle):
    """Row groups whose block chunks are dealt whole 64-byte granules: 1,024
    block columns over few row groups make chunks of 16 to 64 blocks, so the
    chunk boundaries fall between granules.  Extents of 1,021..1,024 blocks
    (64 granules), of 319..322 (20 and 21 granules, unequal shares, a
    partial last granule padded with -inf) and of 16..19 (one or two
    granules: most chunks empty), and a graph pad.  Sampled query rows of
    every request against the oracle; every block column of every row is
    written (no NaN fill left); aligned and misaligned block-score arrays
    agree bit for bit."""
    say("many rows, granule-aligned chunks")
    P, H, mb = 512, 4, 1024
    lens = [1020 * 128 - 126, 318 * 128 - 126, 1900]
    w = W.make(name="gran", R=3, P=P, H=H, k_format=W.K_FP8_E4M3, req_len=lens, topk=8,
               init_blocks=1, local_blocks=2, seed=575, pads=1, pad_len=3000, max_blocks=mb, device="cuda")
    g = Hn.gpu_step(w)
    assert not np.isnan(g["block_scores"]).any(), "a block column left unwritten"
    a = w.oracle_args()
    ends = [(128 * gi + 127) * H for gi in range(4)]  # each row group's longest row
    assert list(Hn.row_blocks(a)[ends]) == [1021, 1022, 1023, 1024]
    assert list(Hn.row_blocks(a)[[P * H + e for e in ends]]) == [319, 320, 321, 322]
    qrows = [0, 1, 127, 128, 255, 256, 300, 383, 384, 510, 511]
    for req in range(3):
        sub = Hn.subset_rows_args(a, req, qrows, P, H)
        rows = (req * P * H + np.asarray(qrows)[:, None] * H + np.arange(H)[None, :]).reshape(-1)
        Hn.assert_parity({k: v[rows] for k, v in g.items()}, oracle.step(**sub), sub)
    pad_rows = slice(3 * P * H, 4 * P * H)
    sub = Hn.subset_rows_args(a, 3, qrows, P, H)
    rows = (3 * P * H + np.asarray(qrows)[:, None] * H + np.arange(H)[None, :]).reshape(-1)
    Hn.assert_parity({k: v[rows] for k, v in g.items()}, oracle.step(**sub), sub)
    assert np.all(g["block_scores"][pad_rows] == -np.inf)
    big = torch.full((w.rows * mb + 4,), float("nan"), dtype=torch.float32, device="cuda")
    outs = {"block_scores": big[1:1 + w.rows * mb].view(w.rows, mb),
            "topk_ids": torch.full((w.rows, w.topk), -7, dtype=torch.int32, device="cuda"),
            "topk_scores": torch.full((w.rows, w.topk), float("nan"), dtype=torch.float32, device="cuda")}
    I.idx_step(Hn.gpu_params(w, outs))
    torch.cuda.synchronize()
    for key, v in outs.items():
        assert np.array_equal(g[key], v.cpu().numpy(), equal_nan=True), key


def test_many_rows_invalid_pages(oracle):
    say("many rows, invalid page ids")
    w = W.make(name="rows_bad", R=2, P=40, H=2, k_format=W.K_BF16, req_len=[1500, 900], topk=4,
               init_blocks=1, local_blocks=1, seed=72, device="cuda")
    w.block_table[int(w.req_slot[0]), 4] = w.n_pages + 9
    w.block_table[int(w.req_slot[1]), 0] = -5
    a = w.oracle_args()
    g, o = Hn.gpu_step(w), oracle.step(**a)
    assert np.isnan(o["block_scores"]).any()
    Hn.assert_parity(g, o, a)


# ---------------------------------------------------------------------------
# degenerate steps: rows with nothing visible, a call with no request, an
# empty K pool
# ---------------------------------------------------------------------------
DEGENERATE = [  # (R, P, H, lens of the requests, pads, pad_len, max_blocks)
    (3, 1, 4, [0, 0, 0], 0, 0, None),       # every row empty, no block column
    (3, 1, 4, [0, 0, 0], 0, 0, 6),          # every row empty, six block columns
    (0, 2, 2, [], 2, 700, None),            # graph pads only
    (1, 2, 2, [0], 3, 2000, None),          # an empty request beside pads
    (2, 1, 20, [0, 0], 1, 300, 3),          # many-rows kernel, no row sees a token
    (1, 32, 1, [0], 1, 500, None),          # many-rows kernel, rows of 0..31 tokens
    (0, 4, 4, [], 0, 0, None),              # no request at all
]


@pytest.mark.parametrize("fmt", [W.K_BF16, W.K_FP8_E4M3, W.K_NVFP4], ids=["bf16", "fp8", "nvfp4"])
@pytest.mark.parametrize("shape", range(len(DEGENERATE)))
def test_degenerate_steps(oracle, fmt, shape):
    R, P, H, lens, pads, pad_len, mb = DEGENERATE[shape]
    say("degenerate", fmt, DEGENERATE[shape])
    w = W.make(name="degenerate", R=R, P=P, H=H, k_format=fmt, req_len=lens, topk=4,
               init_blocks=1, local_blocks=2, seed=500 + shape, pads=pads, pad_len=pad_len,
               max_blocks=mb, device="cuda")
    if fmt == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        a = w.oracle_args(*Hn.oracle_pool(oracle, w))
    else:
        a = w.oracle_args()
    for m in ({}, LSE):
        a_m = dict(a, **m)
        g, o = Hn.gpu_step(w, **m), oracle.step(**a_m)
        for key in g:
            assert g[key].shape == o[key].shape, key
        Hn.assert_parity(g, o, a_m)
        assert np.array_equal(g["topk_ids"], o["topk_ids"])


def test_no_request_calls_each_entry_point():
    """A call over zero requests (every array empty, every pointer NULL) is
    accepted by all three entry points and launches nothing."""
    say("no request, each entry point")
    w = W.make(name="none", R=0, P=4, H=4, k_format=W.K_FP8_E4M3, req_len=[], topk=4,
               init_blocks=1, local_blocks=2, seed=510, device="cuda")
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)
    assert p.n_req == 0 and not p.q and not p.req_slot and not p.block_scores
    for call in (I.idx_score_packed, I.idx_block_topk, I.idx_step):
        call(p)
    torch.cuda.synchronize()


@pytest.mark.parametrize("P,H", [(1, 4), (20, 1)], ids=["one_tile", "many_rows"])
@pytest.mark.parametrize("fmt", [W.K_FP8_E4M3, W.K_NVFP4], ids=["fp8", "nvfp4"])
def test_empty_k_pool(oracle, fmt, P, H):
    """n_pages = 0 with NULL pool pointers: nothing is read, every visible
    block of a real request is NaN and the rest -inf."""
    say("empty K pool", fmt, P, H)
    w = W.make(name="no_pages", R=2, P=P, H=H, k_format=fmt, req_len=[300, 1000], topk=4,
               init_blocks=1, local_blocks=2, seed=511, pads=1, pad_len=500, device="cuda")
    w.k, w.n_pages = w.k[:0], 0
    if fmt == W.K_NVFP4:
        w.k_scale = w.k_scale[:0]
    assert w.k.data_ptr() == 0
    a = w.oracle_args()
    for m in ({}, LSE):
        a_m = dict(a, **m)
        g, o = Hn.gpu_step(w, **m), oracle.step(**a_m)
        assert np.isnan(o["block_scores"]).any() and not np.isfinite(o["block_scores"]).any()
        Hn.assert_parity(g, o, a_m)
        assert np.array_equal(g["topk_ids"], o["topk_ids"])


# ---------------------------------------------------------------------------
# graph capture: one captured step replayed with new device-side data
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [W.K_FP8_E4M3, W.K_NVFP4], ids=["fp8", "nvfp4"])
@pytest.mark.parametrize("P,H", [(4, 4), (20, 2)], ids=["one_tile", "many_rows"])
def test_graph_replays(oracle, P, H, fmt):
    """idx_step (after idx_fp4_store of the keys, for NVFP4) captured once in a
    HIP graph and replayed after new query values, new keys, shorter row
    lengths and a request turned into a graph pad are written into the
    captured buffers (eager work between replays) equals the eager calls on
    every replay, and the oracle on the last."""
    say("graph replays", P, H, fmt)
    w = W.make(name="graph", R=3, P=P, H=H, k_format=fmt, req_len=[700, 2500, 40],
               topk=5, init_blocks=1, local_blocks=2, seed=520 + P, pads=1, pad_len=3000,
               device="cuda")
    fp4 = fmt == W.K_NVFP4
    outs = Hn.gpu_outputs(w)
    p = Hn.gpu_params(w, outs)

    def step():
        if fp4:
            Hn.gpu_fp4_store(w)
        I.idx_step(p)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # first call (launch sizes queried) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(521)
    base_len = w.row_len.clone()
    for rep in range(4):
        outs["block_scores"].fill_(float("nan"))
        outs["topk_scores"].fill_(float("nan"))
        outs["topk_ids"].fill_(-7)
        w.q.copy_(torch.randn(w.q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        if fp4:
            w.staging.copy_(torch.randn(w.staging.shape, generator=gen, device="cuda").to(torch.bfloat16))
        w.row_len.copy_(torch.clamp(base_len - 97 * rep, min=0))  # lengths only shrink
        if rep == 3:
            w.req_slot[1] = -1
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {k: v.cpu().numpy() for k, v in outs.items()}
        if fp4:
            Hn.gpu_fp4_store(w)  # the same keys again: the pool is unchanged
        eager = Hn.gpu_step(w)
        for key in got:
            assert np.array_equal(got[key], eager[key], equal_nan=True), f"replay {rep}: {key}"
    a = w.oracle_args(*Hn.oracle_pool(oracle, w)) if fp4 else w.oracle_args()
    if fp4:
        assert np.array_equal(w.k.cpu().numpy(), a["k"]) and np.array_equal(w.k_scale.cpu().numpy(), a["k_scale"])
    o = oracle.step(**a)
    Hn.assert_parity(got, o, a)
    assert np.array_equal(got["topk_ids"], o["topk_ids"])


def _graph_kernel_nodes(fn) -> int:
    """Kernel nodes of a HIP graph captured from ``fn()`` (the calls are
    made once outside the capture first, so launch sizes are known)."""
    import ctypes as C
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(graph):
        fn()
    hip = C.CDLL("libamdhip64.so.7")  # the runtime torch has loaded (same soname)
    h = C.c_void_p(graph.raw_cuda_graph())
    n = C.c_size_t(0)
    assert hip.hipGraphGetNodes(h, None, C.byref(n)) == 0
    nodes = (C.c_void_p * max(1, n.value))()
    assert hip.hipGraphGetNodes(h, nodes, C.byref(n)) == 0
    kernels = 0
    for i in range(n.value):
        t = C.c_int(-1)
        assert hip.hipGraphNodeGetType(C.c_void_p(nodes[i]), C.byref(t)) == 0
        kernels += t.value == 0  # hipGraphNodeTypeKernel
    return kernels


@pytest.mark.parametrize("P,H", [(4, 4), (24, 4)], ids=["packed", "many_rows"])
def test_launch_count(P, H):
    """One packed scoring launch per step (the analogue of sglang PR 45451's
    verify test, which counts one packed launch per verify forward): scoring
    is one kernel, selection one, the step two, whatever the request count,
    formats and graph pads; the NVFP4 store is one."""
    say("launch count", P, H)
    for fmt in (W.K_BF16, W.K_FP8_E4M3, W.K_NVFP4):
        w = W.make(name="launches", R=6, P=P, H=H, k_format=fmt, req_len=[700, 2500, 40, 0, 9000, 131],
                   topk=5, init_blocks=1, local_blocks=2, seed=530, pads=2, pad_len=3000, device="cuda")
        outs = Hn.gpu_outputs(w)
        p = Hn.gpu_params(w, outs)
        assert _graph_kernel_nodes(lambda: I.idx_score_packed(p)) == 1
        assert _graph_kernel_nodes(lambda: I.idx_block_topk(p)) == 1
        assert _graph_kernel_nodes(lambda: I.idx_step(p)) == 2
        if fmt == W.K_NVFP4:
            assert _graph_kernel_nodes(lambda: Hn.gpu_fp4_store(w)) == 1


@pytest.mark.parametrize("unit_bytes", [1024, 16384, 32768])
def test_read_probe_reads_every_unit(unit_bytes):
    """The plain-read probe the benchmark's read ceiling comes from loads
    every byte of the units it is given: the XOR of its per-workgroup words
    equals the XOR of those units' 32-bit words (a unit listed twice
    cancels); ids outside the buffer read unit 0."""
    say("read probe", unit_bytes)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    n_base = (64 << 20) // unit_bytes
    base = torch.randint(-2**31, 2**31 - 1, (n_base * unit_bytes // 4,), generator=gen,
                         dtype=torch.int32, device="cuda")
    words = base.view(n_base, unit_bytes // 4).cpu().numpy().view(np.uint32)
    rng = np.random.default_rng(78)
    units = rng.integers(0, n_base, size=3 * n_base // 2).astype(np.int32)
    units[::97] = n_base + 5  # out of range: unit 0
    for ids in (None, units):
        sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        I.idx_probe_read(base, unit_bytes, None if ids is None else torch.as_tensor(ids, device="cuda"),
                         sink=sink)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        eff = np.arange(n_base) if ids is None else np.where(ids >= n_base, 0, ids)
        counts = np.bincount(eff, minlength=n_base) % 2
        want = np.bitwise_xor.reduce(words[counts == 1].reshape(-1)) if counts.any() else np.uint32(0)
        assert got == want, (unit_bytes, ids is None)


def test_host_threads_and_streams():
    """Four host threads, each with its own stream and workload, call
    idx_step together (ctypes drops the GIL for the call); every output equals
    the same workload's call made alone."""
    import threading
    say("host threads x streams")
    shapes = [(4, 4, W.K_FP8_E4M3), (20, 2, W.K_BF16), (1, 8, W.K_FP8_E4M3), (64, 1, W.K_BF16)]
    ws = [W.make(name=f"thr{i}", R=3, P=P, H=H, k_format=f, req_len=[900, 2100, 300], topk=5,
                 init_blocks=1, local_blocks=2, seed=530 + i, pads=1, pad_len=1000, device="cuda")
          for i, (P, H, f) in enumerate(shapes)]
    alone = [Hn.gpu_step(w) for w in ws]
    outs = [[Hn.gpu_outputs(w) for _ in range(5)] for w in ws]
    streams = [torch.cuda.Stream() for _ in ws]
    torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            for o in outs[i]:
                I.idx_step(Hn.gpu_params(ws[i], o), streams[i])
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(ws))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, w in enumerate(ws):
        for o in outs[i]:
            for key, v in o.items():
                assert np.array_equal(v.cpu().numpy(), alone[i][key], equal_nan=True), (i, key)


# ---------------------------------------------------------------------------
# seeded random shapes: every path (one tile, many rows, both top-k kernels),
# format and reduction, with lengths from empty to 20,000 tokens
# ---------------------------------------------------------------------------
def _random_case(seed: int) -> dict:
    rng = np.random.default_rng(9000 + seed)
    P = int(rng.choice([1, 2, 4, 5, 8, 16, 17, 33, 64]))
    H = int(rng.integers(1, 9)) if P <= 16 else int(rng.integers(1, 3))
    R = int(rng.integers(1, 6))
    lens = rng.integers(0, int(rng.choice([600, 6000, 20000])), size=R)  # > 64 blocks: workgroup top-k
    lens[rng.random(R) < 0.2] = 0
    topk = int(rng.integers(1, 17))
    init = int(rng.integers(0, min(3, topk) + 1))
    local = int(rng.integers(0, topk - init + 1)) if rng.random() < 0.7 else 0
    return dict(P=P, H=H, R=R, lens=lens.tolist(), topk=topk, init=init, local=min(local, 4),
                pads=int(rng.integers(0, 3)), fmt=int(rng.integers(0, 3)),
                lse=bool(rng.random() < 0.4), scale=float(rng.choice([0.02, 1 / np.sqrt(128), 0.5])))


@pytest.mark.parametrize("seed", range(256))
def test_random_shapes(oracle, seed):
    c = _random_case(seed)
    say("random", seed, c)
    w = W.make(name="random", R=c["R"], P=c["P"], H=c["H"], k_format=c["fmt"], req_len=c["lens"],
               topk=c["topk"], init_blocks=c["init"], local_blocks=c["local"], seed=600 + seed,
               pads=c["pads"], pad_len=2500, device="cuda")
    if c["fmt"] == W.K_NVFP4:
        Hn.gpu_fp4_store(w)
        a = w.oracle_args(*Hn.oracle_pool(oracle, w))
    else:
        a = w.oracle_args()
    m = dict(score_mode=I.IDX_SCORE_LSE, sm_scale=c["scale"]) if c["lse"] else {}
    a = dict(a, **m)
    Hn.assert_parity(Hn.gpu_step(w, **m), oracle.step(**a), a)
