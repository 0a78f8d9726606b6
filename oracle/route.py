"""Router and dispatch: logits, softmax, top-k, histogram, prefix scan,
stable permutation, tile map.

Test infrastructure only (see the package docstring).

Perplexity, "Optimizing on-device inference for Apple Silicon":

* "Qwen 创建了三种不同的工作负载形状": the router scores 256 experts per token
  and keeps 8; a shared expert processes every token.  The pages do not say
  how the 8 gates are formed.  Reading taken (the plainest one consistent
  with "softmax over 256 logits, top-8, renormalized gates"): softmax over
  all E logits, keep the top-k probabilities, divide them by their sum.
  Equal probabilities are broken toward the lower expert index; the k ids
  are listed in that order (gates descending).  A per-expert logit bias,
  when present, is added to the logits and so enters both the choice and
  the gate values.
* "将专家路由保留在 GPU 上": after the top-8 choice a histogram counts the
  assignments of every expert, a prefix scan turns the counts into start
  offsets, a scatter places the rows into their expert groups, and a block
  map lists the fixed-size matrix tiles the grouped GEMM must process.
  Reading taken for the scatter order (the page only says rows are placed
  into their groups): stable, i.e. inside one expert's group the
  assignments keep ascending order of a = t * topk + j.
* "使瓦片大小与专家负载相匹配": each expert's rows are cut into tiles of a
  fixed number of rows; the last tile of an expert may be partial and an
  expert with no rows has no tile.  The section's point is that the tile
  height should follow the load.  Reading taken for the two-height map the
  grouped GEMM runs on (load_matched_tile_map): an expert's rows go into
  tall tiles while a full tall tile remains, the rest into short tiles;
  all tall tiles are listed first.
"""
from __future__ import annotations

import numpy as np


def router_logits(H, Wr, logit_bias=None) -> np.ndarray:
    """float64 [T][E] = H [T][D] @ Wr [D][E] (+ logit_bias [E])."""
    L = np.asarray(H).astype(np.float64) @ np.asarray(Wr).astype(np.float64)
    if logit_bias is not None:
        L = L + np.asarray(logit_bias).astype(np.float64)[None, :]
    return L


def softmax(logits) -> np.ndarray:
    """Row-wise softmax in float64, computed with the row maximum subtracted."""
    L = np.asarray(logits, dtype=np.float64)
    z = L - L.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def topk_route(logits, topk: int):
    """ids int32 [T][topk] and gates float64 [T][topk].

    The probabilities are ordered by (probability descending, expert index
    ascending); the first ``topk`` are kept and renormalized to sum to 1.
    """
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    if not (1 <= topk <= E):
        raise ValueError("need 1 <= topk <= E")
    p = softmax(L)
    ids = np.empty((T, topk), dtype=np.int32)
    gates = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        order = np.argsort(-p[t], kind="stable")  # stable: ties keep lower index first
        sel = order[:topk]
        ids[t] = sel
        gates[t] = p[t, sel] / p[t, sel].sum()
    return ids, gates


def topk_near_ties(logits, topk: int, tau: float) -> np.ndarray:
    """bool [T][topk]: True where the j-th largest logit lies within ``tau`` of
    its neighbour in the descending order (the (j-1)-th or (j+1)-th, the
    latter including the first unchosen one).  Such positions can be decided
    either way by a computation whose logits carry an error below tau/2."""
    L = np.asarray(logits, dtype=np.float64)
    T, E = L.shape
    srt = -np.sort(-L, axis=1)
    m = min(topk + 1, E)
    gaps = srt[:, : m - 1] - srt[:, 1:m]  # gap between position j and j+1
    near = np.zeros((T, topk), dtype=bool)
    for j in range(topk):
        if j < m - 1:
            near[:, j] |= gaps[:, j] < tau
        if j > 0:
            near[:, j] |= gaps[:, j - 1] < tau
    return near


def histogram(ids, E: int) -> np.ndarray:
    """int32 [E]: counts[e] = number of assignments (t, j) with ids[t][j] == e."""
    ids = np.asarray(ids).ravel()
    counts = np.zeros(E, dtype=np.int64)
    for e in ids:
        counts[e] += 1
    return counts.astype(np.int32)


def exclusive_scan(counts) -> np.ndarray:
    """int32 [E + 1]: offsets[0] = 0, offsets[e + 1] = offsets[e] + counts[e]."""
    counts = np.asarray(counts, dtype=np.int64)
    offsets = np.zeros(counts.shape[0] + 1, dtype=np.int64)
    for e in range(counts.shape[0]):
        offsets[e + 1] = offsets[e] + counts[e]
    return offsets.astype(np.int32)


def stable_permutation(ids, E: int):
    """sorted_assign int32 [T*topk] and its inverse pos int32 [T*topk].

    sorted_assign lists the assignments a = t * topk + j grouped by expert in
    expert order, ascending a inside each group; pos[a] is the row of
    assignment a in that order.
    """
    flat = np.asarray(ids).ravel().astype(np.int64)
    offsets = exclusive_scan(histogram(flat, E)).astype(np.int64)
    fill = offsets[:-1].copy()
    sorted_assign = np.empty(flat.shape[0], dtype=np.int64)
    for a, e in enumerate(flat):  # ascending a: stable by construction
        sorted_assign[fill[e]] = a
        fill[e] += 1
    pos = np.empty_like(sorted_assign)
    pos[sorted_assign] = np.arange(flat.shape[0])
    return sorted_assign.astype(np.int32), pos.astype(np.int32)


def tile_map(counts, tile_rows: int) -> np.ndarray:
    """int32 [ntiles][3]: (expert, first row, rows) for every tile of at most
    ``tile_rows`` rows, experts in order, tiles in row order inside each
    expert."""
    counts = np.asarray(counts, dtype=np.int64)
    offsets = exclusive_scan(counts).astype(np.int64)
    tiles = []
    for e in range(counts.shape[0]):
        start = 0
        while start < counts[e]:
            rows = min(tile_rows, counts[e] - start)
            tiles.append((e, offsets[e] + start, rows))
            start += tile_rows
    return np.asarray(tiles, dtype=np.int32).reshape(-1, 3)


def load_matched_tile_map(counts, small_rows: int, big_rows: int) -> np.ndarray:
    """int32 [ntiles][4]: (expert, first row, rows, height).

    Each expert's rows, in row order, are cut into tiles of exactly
    ``big_rows`` rows while at least ``big_rows`` remain, and the remainder
    into tiles of at most ``small_rows`` rows.  The map lists every tall tile
    first (experts ascending, rows ascending), then every short tile (same
    order).  ``height`` is the tile height the tile is computed with
    (``big_rows`` or ``small_rows``); rows <= height.
    """
    counts = np.asarray(counts, dtype=np.int64)
    offsets = exclusive_scan(counts).astype(np.int64)
    tall, short = [], []
    for e in range(counts.shape[0]):
        start = 0
        while counts[e] - start >= big_rows:
            tall.append((e, offsets[e] + start, big_rows, big_rows))
            start += big_rows
        while start < counts[e]:
            rows = min(small_rows, counts[e] - start)
            short.append((e, offsets[e] + start, rows, small_rows))
            start += small_rows
    return np.asarray(tall + short, dtype=np.int32).reshape(-1, 4)
