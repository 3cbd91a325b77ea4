"""Token -> expert routing tables (oracle side, test infrastructure).

What is computed, and where the pages describe it:
* Per-expert hit counts: "MegaMoE" walk-through section 4.2 step 1 (each
  token's top-k experts counted per expert); reading notes, "dispatch inside
  the kernel", first step (only valid experts are counted).
* Block-padded layout: "fused MoE in practice" (stmoonar.pages.dev), section 2
  "schedule tables": hits sorted by expert into one buffer, each expert's row
  count rounded up to the GEMM row block, a prefix sum of the padded counts;
  the slot table [T, k] mapping token t's j-th hit to its row; ``pull_order``
  = tokens sorted by their smallest slot; ``slack`` = padding rows per row
  block (the counter seed: slack plus real arrivals fills the block).
* Pool capacity: the SymmBuffer page (backyes.github.io, section 6.2 "pool
  capacity"): align(tokens * min(k, E_local) + E_local * (block_m - 1), block_m),
  taken here with one rank.  The min(k, E_local) factor assumes a token never
  names one expert twice; this library accepts repeated ids (each one is a
  hit), so it uses k in place of min(k, E_local).  The two agree whenever
  k <= E_local.
* Inverse table (row -> token, top-k slot): the token source metadata of the
  reading notes ("the target process pulls tokens") restricted to one GPU.

Readings where the pages leave a choice open:
* A hit (t, j) is valid iff 0 <= topk_idx[t, j] - expert_begin < E; other ids
  (negative, other GPUs' experts) are dropped without error.
* Within one expert, rows go in ascending flat hit order t*k + j (stable); the
  pages' own kernels use atomics whose order is not fixed, and the practice
  page builds its tables with one stable sort, which is what is taken here.
* Padding rows carry row_token = row_topk = -1.  Rows at or beyond R_pad (the
  padded total) are not part of the result.
* pull_order lists the tokens with at least one valid hit, ascending by their
  smallest slot; entries at or beyond n_pull are not part of the result.

Two implementations: ``plan_naive`` (plain loops, small inputs) and
``plan_ref`` (vectorised stable argsort).  Tests require them to agree
element by element and check the invariants the practice page lists.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def capacity_rows(num_tokens: int, topk: int, num_experts: int, block_m: int) -> int:
    """Worst-case padded row count: the SymmBuffer page's pool formula with one rank,
    with k in place of min(k, E) so that repeated ids within a token stay in bounds."""
    raw = num_tokens * topk + num_experts * (block_m - 1)
    return (raw + block_m - 1) // block_m * block_m


@dataclass
class Plan:
    counts: np.ndarray        # int32 [E]
    offsets: np.ndarray       # int32 [E+1], padded prefix sum
    slot: np.ndarray          # int32 [T, k], -1 for invalid hits
    row_token: np.ndarray     # int32 [R_pad]
    row_topk: np.ndarray      # int32 [R_pad]
    block_expert: np.ndarray  # int32 [R_pad / bm]
    slack: np.ndarray         # int32 [R_pad / bm]
    pull_order: np.ndarray    # int32 [n_pull]
    num_valid: int            # N
    r_pad: int                # R_pad
    n_pull: int
    n_blocks: int
    capacity: int


def _valid_local(topk_idx: np.ndarray, num_experts: int, expert_begin: int):
    ids = np.asarray(topk_idx, dtype=np.int64)
    local = ids - expert_begin
    valid = (local >= 0) & (local < num_experts)
    return local, valid


def plan_naive(topk_idx, num_experts: int, expert_begin: int, block_m: int) -> Plan:
    """Plain loops over tokens and top-k slots; meant for small inputs."""
    ids = np.asarray(topk_idx, dtype=np.int64)
    T, k = ids.shape
    E, bm = num_experts, block_m
    counts = [0] * E
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j]) - expert_begin
            if 0 <= e < E:
                counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        padded = (counts[e] + bm - 1) // bm * bm
        offsets[e + 1] = offsets[e] + padded
    r_pad = offsets[E]
    slot = [[-1] * k for _ in range(T)]
    row_token = [-1] * r_pad
    row_topk = [-1] * r_pad
    fill = [0] * E
    for t in range(T):                       # ascending flat index t*k + j
        for j in range(k):
            e = int(ids[t, j]) - expert_begin
            if 0 <= e < E:
                r = offsets[e] + fill[e]
                fill[e] += 1
                slot[t][j] = r
                row_token[r] = t
                row_topk[r] = j
    n_blocks = r_pad // bm
    block_expert = [0] * n_blocks
    slack = [0] * n_blocks
    for e in range(E):
        for b in range(offsets[e] // bm, offsets[e + 1] // bm):
            block_expert[b] = e
    for b in range(n_blocks):
        slack[b] = sum(1 for r in range(b * bm, (b + 1) * bm) if row_token[r] < 0)
    firsts = []
    for t in range(T):
        s = [slot[t][j] for j in range(k) if slot[t][j] >= 0]
        if s:
            firsts.append((min(s), t))
    firsts.sort()
    pull_order = [t for _, t in firsts]
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return Plan(i32(counts), i32(offsets), i32(slot).reshape(T, k), i32(row_token), i32(row_topk),
                i32(block_expert), i32(slack), i32(pull_order), sum(counts), r_pad,
                len(pull_order), n_blocks, capacity_rows(T, k, E, bm))


def plan_ref(topk_idx, num_experts: int, expert_begin: int, block_m: int) -> Plan:
    """Vectorised twin of ``plan_naive``: one stable argsort plus scatters."""
    ids = np.asarray(topk_idx, dtype=np.int64)
    T, k = ids.shape
    E, bm = num_experts, block_m
    local, valid = _valid_local(ids, E, expert_begin)
    flat_e = local.reshape(-1)
    flat_v = valid.reshape(-1)
    hits = np.nonzero(flat_v)[0]             # flat hit indices t*k + j, ascending
    he = flat_e[hits]
    counts = np.bincount(he, minlength=E).astype(np.int64)
    padded = (counts + bm - 1) // bm * bm
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    r_pad = int(offsets[E])
    order = np.argsort(he, kind="stable")    # hits grouped by expert, flat order kept
    sorted_e = he[order]
    starts = np.zeros(E + 1, dtype=np.int64)
    starts[1:] = np.cumsum(counts)
    rank = np.arange(order.size) - starts[sorted_e]
    rows = offsets[sorted_e] + rank
    flat_slot = np.full(T * k, -1, dtype=np.int64)
    flat_slot[hits[order]] = rows
    row_token = np.full(r_pad, -1, dtype=np.int64)
    row_topk = np.full(r_pad, -1, dtype=np.int64)
    row_token[rows] = hits[order] // k
    row_topk[rows] = hits[order] % k
    n_blocks = r_pad // bm
    block_expert = np.repeat(np.arange(E), padded // bm)
    filled = (row_token >= 0).reshape(n_blocks, bm).sum(axis=1) if n_blocks else np.zeros(0, np.int64)
    slack = bm - filled
    slot = flat_slot.reshape(T, k)
    has = (slot >= 0).any(axis=1)
    min_slot = np.where(slot >= 0, slot, np.iinfo(np.int64).max).min(axis=1)
    toks = np.nonzero(has)[0]
    pull_order = toks[np.argsort(min_slot[toks], kind="stable")]
    i32 = lambda a: np.asarray(a, dtype=np.int32)
    return Plan(i32(counts), i32(offsets), i32(slot), i32(row_token), i32(row_topk),
                i32(block_expert), i32(slack), i32(pull_order), int(hits.size), r_pad,
                int(pull_order.size), n_blocks, capacity_rows(T, k, E, bm))
