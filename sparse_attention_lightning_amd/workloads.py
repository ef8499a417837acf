"""Seeded synthetic inputs for the packed indexer step.

This module draws inputs only: lengths, slot and page tables, N(0,1) queries
and keys, poison values.  It holds none of the method's arithmetic (no
dequantization, dot products, block maxima or selection), so both the GPU
library's tests and the CPU oracle can consume what it makes.

The workloads stand in for the shapes the pages measure on:
  * sglang PR 45451, Speed Tests: index step at 16 requests x 131K and
    32 requests x 524K with 4 EAGLE3 draft rows, bf16 and fp8 index K;
  * sglang PR 42614, Accuracy Tests: 4 requests x 4 draft rows whose rows end
    at 32767..32770 (256- and 257-block rows in one tile), request slots that
    are permuted, gapped and never equal to a row or group index, and graph
    pad slots past the request table;
  * ROCm/ATOM PR 2745, Validation: NVFP4 index keys at batch 64, ~150K context.
Real index keys and the pages' datasets are not available; N(0,1) values give
the same shapes and bytes moved.

Structural draws use ``numpy.random.default_rng(seed)``; bulk values use a
``torch.Generator`` seeded with the same number on the chosen device (so CPU
and GPU draws differ; every consumer of one Workload sees the same bytes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

K_BF16, K_FP8_E4M3, K_NVFP4 = 0, 1, 2
FORMAT_NAMES = {K_BF16: "bf16", K_FP8_E4M3: "fp8_e4m3", K_NVFP4: "nvfp4"}
BYTES_PER_TOKEN = {K_BF16: 256, K_FP8_E4M3: 128, K_NVFP4: 72}
BLOCK = 128
D = 128

# Poison written where no row may look: gap pages and the tail of each
# request's last page.  Large enough to win every block max if it leaked.
POISON_BF16 = 1.0e4
POISON_FP8_CODE = 0x7E        # 448, the largest finite e4m3fn value
POISON_FP4_PAYLOAD = 0x77     # code 7 (+6) in both nibbles
POISON_FP4_SCALE = 0x7E       # scale 448


@dataclass
class Workload:
    name: str
    k_format: int
    n_req: int                 # including graph pads
    n_real: int
    packed_queries: int
    gqa: int
    max_blocks: int
    topk: int
    init_blocks: int
    local_blocks: int
    n_slot_rows: int
    n_pages: int
    seed: int
    q: torch.Tensor            # bf16 [n_req*P, H, 128]
    k: torch.Tensor            # bf16 / float8_e4m3fn [n_pages*128, 128]; uint8 [n_pages*128, 64]
    k_scale: torch.Tensor | None   # uint8 [n_pages*128, 8] for NVFP4
    req_slot: torch.Tensor     # int32 [n_req]
    block_table: torch.Tensor  # int32 [n_slot_rows, max_blocks]
    row_len: torch.Tensor      # int32 [n_req*P]
    req_len: np.ndarray        # L_r of each real request (row j sees L_r + j)
    staging: torch.Tensor | None = None       # NVFP4: bf16 [n_tokens, 128]
    slot_mapping: torch.Tensor | None = None  # NVFP4: int64 [n_tokens]
    extra: dict = field(default_factory=dict)

    # -- sizes ------------------------------------------------------------
    @property
    def rows(self) -> int:
        return self.n_req * self.packed_queries * self.gqa

    def group_len(self) -> np.ndarray:
        """Longest row of every request (pads included)."""
        rl = self.row_len.cpu().numpy().reshape(self.n_req, self.packed_queries)
        return rl.max(axis=1)

    def k_tokens(self) -> int:
        """Tokens of K a packed step must read: the longest row of every real
        request (pads read nothing)."""
        return int(self.group_len()[: self.n_real].astype(np.int64).sum())

    def pool_pages_used(self) -> int:
        g = self.group_len()[: self.n_real].astype(np.int64)
        return int(((g + BLOCK - 1) // BLOCK).sum())

    # -- host copies for the CPU oracle -----------------------------------
    def oracle_args(self, k_payload: np.ndarray | None = None,
                    k_scale: np.ndarray | None = None) -> dict:
        """Keyword arguments of the oracle's entry points (numpy, host).

        For NVFP4 the caller passes the payload and scale planes the oracle's
        own store produced from ``staging``."""
        def u16(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        def u8(t):
            return t.detach().cpu().contiguous().view(torch.uint8).numpy()

        a = dict(k_format=self.k_format, n_req=self.n_req, n_slot_rows=self.n_slot_rows,
                 packed_queries=self.packed_queries, gqa=self.gqa, max_blocks=self.max_blocks,
                 topk=self.topk, init_blocks=self.init_blocks, local_blocks=self.local_blocks,
                 n_pages=self.n_pages, q=u16(self.q),
                 req_slot=self.req_slot.cpu().numpy().astype(np.int32),
                 block_table=self.block_table.cpu().numpy().astype(np.int32),
                 row_len=self.row_len.cpu().numpy().astype(np.int32))
        if self.k_format == K_BF16:
            a["k"] = u16(self.k)
        elif self.k_format == K_FP8_E4M3:
            a["k"] = u8(self.k)
        else:
            a["k"] = k_payload if k_payload is not None else u8(self.k)
            a["k_scale"] = k_scale if k_scale is not None else u8(self.k_scale)
        return a


def _slot_table(rng: np.random.Generator, R: int, P: int) -> tuple[int, np.ndarray]:
    """Permuted, gapped request slots: no request's slot equals its group index
    r or any of its row indices r*P + j.  The table has 2R + 5 rows, grown by P
    until every request has at least R free candidates."""
    n_slot_rows = 2 * R + 5
    while n_slot_rows - (P + 1) < R:
        n_slot_rows += P
    for _ in range(100000):
        slots = rng.permutation(n_slot_rows)[:R]
        bad = False
        for r, s in enumerate(slots):
            if s == r or (r * P <= s < r * P + P):
                bad = True
                break
        if not bad:
            return n_slot_rows, slots.astype(np.int32)
    raise RuntimeError("no slot permutation satisfies the constraints")


def _randn_into(dst: torch.Tensor, gen: torch.Generator, chunk_rows: int = 1 << 17) -> None:
    """Fill a [N, 128] tensor with N(0,1) draws cast (round to nearest even)
    to its dtype, a chunk at a time."""
    n = dst.shape[0]
    for s in range(0, n, chunk_rows):
        e = min(n, s + chunk_rows)
        x = torch.randn((e - s, dst.shape[1]), generator=gen, device=dst.device,
                        dtype=torch.float32)
        dst[s:e].copy_(x.to(dst.dtype))


def make(*, name: str, R: int, P: int, H: int, k_format: int, req_len, topk: int,
         init_blocks: int, local_blocks: int, seed: int, slots: str = "permuted",
         pads: int = 0, pad_len: int = 0, max_blocks: int | None = None,
         device: str | torch.device = "cpu", rng: np.random.Generator | None = None,
         poison: bool = True) -> Workload:
    """Build one workload.  Row j of request r sees ``req_len[r] + j`` tokens."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    device = torch.device(device)
    req_len = np.asarray(req_len, dtype=np.int64)
    assert req_len.shape == (R,)
    lmax = req_len + (P - 1)
    nbg = (lmax + BLOCK - 1) // BLOCK
    if pads:
        pad_nb = (pad_len + BLOCK - 1) // BLOCK
        mb_needed = int(max(nbg.max(initial=0), pad_nb))
    else:
        mb_needed = int(nbg.max(initial=0))
    max_blocks = mb_needed if max_blocks is None else max_blocks
    assert max_blocks >= mb_needed

    if slots == "identity":
        n_slot_rows, req_slot = R, np.arange(R, dtype=np.int32)
        n_pages = R * max_blocks
        page_of = [np.arange(nbg[r], dtype=np.int64) + r * max_blocks for r in range(R)]
    elif slots == "permuted":
        n_slot_rows, req_slot = _slot_table(rng, R, P)
        used = int(nbg.sum())
        n_pages = max(1, math.ceil(1.25 * used))
        perm = rng.permutation(n_pages).astype(np.int64)
        page_of, o = [], 0
        for r in range(R):
            page_of.append(perm[o:o + nbg[r]])
            o += nbg[r]
    else:
        raise ValueError(slots)

    bt = np.full((n_slot_rows, max_blocks), -1, dtype=np.int32)
    for r in range(R):
        bt[req_slot[r], : nbg[r]] = page_of[r]
    row_len = (req_len[:, None] + np.arange(P)[None, :]).reshape(-1)
    if pads:
        req_slot = np.concatenate([req_slot, n_slot_rows + np.arange(pads, dtype=np.int32)])
        row_len = np.concatenate([row_len, np.full(pads * P, pad_len, dtype=np.int64)])
    n_req = R + pads

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    q = torch.empty((n_req * P, H, D), dtype=torch.bfloat16, device=device)
    _randn_into(q.view(-1, D), gen)

    # tokens that no row may see: whole gap pages, and each last page's tail
    used_pages = np.zeros(n_pages, dtype=bool)
    tails = []  # (page, first poisoned offset)
    for r in range(R):
        used_pages[page_of[r]] = True
        rem = int(lmax[r] - (nbg[r] - 1) * BLOCK)
        if nbg[r] and rem < BLOCK:
            tails.append((int(page_of[r][-1]), rem))
    gap_pages = np.nonzero(~used_pages)[0]

    staging = slot_mapping = k_scale = None
    if k_format in (K_BF16, K_FP8_E4M3):
        dt = torch.bfloat16 if k_format == K_BF16 else torch.float8_e4m3fn
        k = torch.empty((n_pages * BLOCK, D), dtype=dt, device=device)
        _randn_into(k, gen)
        if poison:
            pv = (torch.tensor(POISON_BF16, dtype=torch.bfloat16) if k_format == K_BF16
                  else torch.tensor([POISON_FP8_CODE], dtype=torch.uint8).view(dt)[0])
            kv = k.view(n_pages, BLOCK, D)
            if len(gap_pages):
                kv[torch.as_tensor(gap_pages, device=device)] = pv.to(device)
            for pg, off in tails:
                kv[pg, off:] = pv.to(device)
    elif k_format == K_NVFP4:
        k = torch.full((n_pages * BLOCK, 64), POISON_FP4_PAYLOAD, dtype=torch.uint8,
                       device=device)
        k_scale = torch.full((n_pages * BLOCK, 8), POISON_FP4_SCALE, dtype=torch.uint8,
                             device=device)
        n_tok = int(lmax.sum())
        staging = torch.empty((n_tok, D), dtype=torch.bfloat16, device=device)
        _randn_into(staging, gen)
        sm = np.empty(n_tok, dtype=np.int64)
        o = 0
        for r in range(R):
            t = np.arange(lmax[r], dtype=np.int64)
            sm[o:o + lmax[r]] = page_of[r][t // BLOCK] * BLOCK + t % BLOCK
            o += lmax[r]
        slot_mapping = torch.as_tensor(sm, device=device)
    else:
        raise ValueError(k_format)

    return Workload(
        name=name, k_format=k_format, n_req=n_req, n_real=R, packed_queries=P, gqa=H,
        max_blocks=max_blocks, topk=topk, init_blocks=init_blocks, local_blocks=local_blocks,
        n_slot_rows=n_slot_rows, n_pages=n_pages, seed=seed, q=q, k=k, k_scale=k_scale,
        req_slot=torch.as_tensor(req_slot.astype(np.int32), device=device),
        block_table=torch.as_tensor(bt, device=device),
        row_len=torch.as_tensor(row_len.astype(np.int32), device=device),
        req_len=req_len, staging=staging, slot_mapping=slot_mapping,
        extra={"gap_pages": gap_pages, "tails": tails, "page_of": page_of})


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
CONFIG_NAMES = {
    0: "tiny_2req_bf16",
    1: "16req_131k_bf16",
    2: "16req_131k_fp8_straddle",
    3: "32req_524k_fp8_3pads",
    4: "64req_150k_nvfp4",
    5: "4req_2k_prefill_32k_fp8",
}


def config(idx: int, device: str | torch.device = "cpu", local_blocks: int | None = None,
           n_real: int | None = None, k_format: int | None = None) -> Workload:
    """Workload ``idx`` (0..5) with seed 1000 + idx.

    ``local_blocks`` overrides the forced local window (the 0 variant of the
    straddling fp8 workload).  ``n_real`` keeps the first ``n_real`` request
    lengths of the same draw (slot and page tables are drawn for the smaller
    table); it makes bounded samples for CPU timing.  ``k_format`` stores the
    keys in another format at the same shape (the name says which), e.g. the
    64-request ~150K workload with fp8 keys beside its NVFP4 ones."""
    seed = 1000 + idx
    rng = np.random.default_rng(seed)
    if idx == 0:
        lens = np.array([1000, 1500])
        kw = dict(R=2, P=4, H=2, k_format=K_BF16, topk=4, init_blocks=1, local_blocks=1,
                  slots="identity")
    elif idx in (1, 2):
        lens = rng.integers(122880, 131069, size=16, endpoint=True)
        if idx == 2:
            lens[:4] = 32767  # rows end at 32767..32770: 256 and 257 blocks in one tile
        kw = dict(R=16, P=4, H=4, k_format=K_BF16 if idx == 1 else K_FP8_E4M3, topk=64,
                  init_blocks=1, local_blocks=2, max_blocks=1024)
    elif idx == 3:
        lens = rng.integers(491520, 524285, size=32, endpoint=True)
        kw = dict(R=32, P=4, H=4, k_format=K_FP8_E4M3, topk=64, init_blocks=1,
                  local_blocks=2, pads=3, pad_len=524288, max_blocks=4096)
    elif idx == 4:
        lens = rng.integers(138240, 168957, size=64, endpoint=True)
        kw = dict(R=64, P=4, H=4, k_format=K_NVFP4, topk=64, init_blocks=1, local_blocks=2,
                  max_blocks=1320)
    elif idx == 5:
        # prefill chunks: 2,048 query rows a request at causal lengths L..L+2047
        lens = rng.integers(30720, 30720 + 2048, size=4, endpoint=True)
        kw = dict(R=4, P=2048, H=4, k_format=K_FP8_E4M3, topk=64, init_blocks=1, local_blocks=2,
                  max_blocks=272)
    else:
        raise ValueError(idx)
    if local_blocks is not None:
        kw["local_blocks"] = local_blocks
    if n_real is not None:
        lens = lens[:n_real]
        kw["R"] = n_real
    name = CONFIG_NAMES[idx]
    if k_format is not None and k_format != kw["k_format"]:
        short = {K_BF16: "bf16", K_FP8_E4M3: "fp8", K_NVFP4: "nvfp4"}
        name = name.replace(short[kw["k_format"]], short[k_format], 1)
        kw["k_format"] = k_format
    return make(name=name, req_len=lens, seed=seed, device=device, rng=rng, **kw)


# ---------------------------------------------------------------------------
# Inputs of the sparse attention that follows selection
# ---------------------------------------------------------------------------
POISON_ATTN_V = 1.0e4   # V where no row may look: a leaked token moves its row's output by ~1e4 / n
POISON_ATTN_V_FP8 = 448.0  # the same for fp8 K/V (the largest e4m3 value)


@dataclass
class AttnInputs:
    q_per_kv: int
    q: torch.Tensor     # bf16 [n_req*P, H, G, 128]: query head g of KV head h of each draft row
    k: torch.Tensor     # bf16 or float8_e4m3fn [n_pages, H, 128 tokens, 128]
    v: torch.Tensor     # like k: [n_pages, H, 4, 128 dims, 32 tokens] (each 32-token quarter of a page-head transposed)
    seed: int
    kv_format: int = K_BF16


def make_attn(w: Workload, q_per_kv: int, seed: int | None = None, poison: bool = True,
              kv_format: int = K_BF16) -> AttnInputs:
    """Seeded N(0,1) attention queries, keys and values over the workload's
    page pool (the same pages, slots and row lengths as its index K; the KV
    heads are the workload's gqa index heads), K and V stored in bf16 or cast
    (round to nearest even) to fp8 e4m3.  Gap pages and the tail of each
    request's last page get K = 0 and a large V (1e4 in bf16, 448 in fp8), so
    a token no row may see would move that row's output by far more than any
    tolerance."""
    seed = w.seed + 500 if seed is None else seed
    dev = w.q.device
    H, n_pages = w.gqa, w.n_pages
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    q = torch.empty((w.n_req * w.packed_queries, H, q_per_kv, D), dtype=torch.bfloat16, device=dev)
    _randn_into(q.view(-1, D), gen)
    kv_dtype = torch.bfloat16 if kv_format == K_BF16 else torch.float8_e4m3fn
    k = torch.empty((n_pages, H, BLOCK, D), dtype=kv_dtype, device=dev)
    _randn_into(k.view(-1, D), gen)
    v = torch.empty((n_pages, H, 4, D, BLOCK // 4), dtype=kv_dtype, device=dev)
    _randn_into(v.view(-1, D), gen)
    pv = POISON_ATTN_V if kv_format == K_BF16 else POISON_ATTN_V_FP8
    if poison:
        gap = w.extra["gap_pages"]
        if len(gap):
            gi = torch.as_tensor(gap, device=dev)
            k[gi] = 0
            v[gi] = pv
        for pg, off in w.extra["tails"]:
            k[pg, :, off:, :] = 0
            for u in range(4):  # tokens >= off of each 32-token quarter
                start = max(0, off - 32 * u)
                if start < 32:
                    v[pg, :, u, :, start:] = pv
    return AttnInputs(q_per_kv=q_per_kv, q=q, k=k, v=v, seed=seed, kv_format=kv_format)


def attn_oracle_args(w: Workload, at: AttnInputs, topk_ids, sm_scale: float) -> dict:
    """Keyword arguments of the oracle's sparse attention (numpy, host) for
    the selection ``topk_ids`` ([n_req*P*H, topk] int32, numpy or torch)."""
    def u16(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    def kv(t):
        return u16(t) if at.kv_format == K_BF16 else t.detach().cpu().contiguous().view(torch.uint8).numpy()

    ids = topk_ids.detach().cpu().numpy() if isinstance(topk_ids, torch.Tensor) else np.asarray(topk_ids)
    ids = np.ascontiguousarray(ids.astype(np.int32).reshape(w.n_req * w.packed_queries * w.gqa, -1))
    return dict(n_req=w.n_req, n_slot_rows=w.n_slot_rows, packed_queries=w.packed_queries,
                kv_heads=w.gqa, q_per_kv=at.q_per_kv, max_blocks=w.max_blocks, topk=ids.shape[1],
                sm_scale=sm_scale, n_pages=w.n_pages, kv_format=at.kv_format, q=u16(at.q), k=kv(at.k), v=kv(at.v),
                req_slot=w.req_slot.cpu().numpy().astype(np.int32),
                block_table=w.block_table.cpu().numpy().astype(np.int32),
                row_len=w.row_len.cpu().numpy().astype(np.int32), topk_ids=ids)
