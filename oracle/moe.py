"""CPU oracle of the MoE layout steps around the grouped GEMMs -- TEST
INFRASTRUCTURE ONLY (same rules as the rest of ``oracle``).

The steps follow the MoE flow of the kwkr.cn DeepGEMM usage article
(section 3.2: order tokens by expert index, count the tokens of each
expert; section 4.3: sort, count, run the grouped GEMM, put the outputs back
in token order) together with the two grouped layouts of "DeepSeek
open-source week, day 3: DeepGEMM" (contiguous layout: experts' rows
concatenated along M with an alignment requirement; masked layout: a fixed
slot per expert plus a tensor of valid counts).

Readings where the pages leave the step open (each pinned by a test):
  * the order of the tokens of one expert is their original order (a stable
    sort), so every layout below is unique;
  * contiguous layout: each expert's rows start at a multiple of `align`
    (the grouped GEMM's 128-row block); the padding rows of an expert carry
    its index, rows past the last expert carry -1 (a skipped block);
  * masked layout: an expert keeps at most `max_m` tokens, in token order;
    the rest are not placed (destination -1);
  * an expert index outside [0, G) routes a token nowhere.

Everything here is plain numpy written from those definitions.
"""
from __future__ import annotations

import numpy as np


def _ceil_to(v: np.ndarray, align: int) -> np.ndarray:
    return (v + align - 1) // align * align


def moe_counts(expert_idx, num_groups: int) -> np.ndarray:
    """counts[g] = number of tokens whose expert index is g."""
    e = np.asarray(expert_idx, np.int64)
    counts = np.zeros(num_groups, np.int64)
    for g in range(num_groups):
        counts[g] = int(np.count_nonzero(e == g))
    return counts


def moe_ranks(expert_idx, num_groups: int) -> np.ndarray:
    """rank[t] = number of tokens before t with the same expert (-1 when t
    routes nowhere)."""
    e = np.asarray(expert_idx, np.int64)
    rank = np.full(e.size, -1, np.int64)
    for g in range(num_groups):
        hit = e == g
        rank[hit] = np.cumsum(hit)[hit] - 1
    return rank


def moe_layout_contiguous(expert_idx, num_groups: int, m_rows: int, align: int = 128):
    """Contiguous (MoE prefill) layout.  Returns (counts [G], offsets [G+1],
    dst_row [T], m_indices [m_rows]), all int32:
        offsets[g + 1] = offsets[g] + ceil(counts[g] / align) * align,
        dst_row[t]     = offsets[e[t]] + rank[t],
        m_indices[r]   = g for offsets[g] <= r < offsets[g + 1], else -1."""
    e = np.asarray(expert_idx, np.int64)
    counts = moe_counts(e, num_groups)
    offsets = np.zeros(num_groups + 1, np.int64)
    offsets[1:] = np.cumsum(_ceil_to(counts, align))
    if offsets[-1] > m_rows:
        raise ValueError("m_rows is smaller than the laid-out rows")
    rank = moe_ranks(e, num_groups)
    dst = np.full(e.size, -1, np.int64)
    routed = rank >= 0
    dst[routed] = offsets[e[routed]] + rank[routed]
    m_indices = np.full(m_rows, -1, np.int64)
    for g in range(num_groups):
        m_indices[offsets[g]:offsets[g + 1]] = g
    return (counts.astype(np.int32), offsets.astype(np.int32), dst.astype(np.int32),
            m_indices.astype(np.int32))


def moe_layout_masked(expert_idx, num_groups: int, max_m: int):
    """Masked (MoE decode) layout.  Returns (counts [G], dst_row [T],
    masked_m [G]), int32:  dst_row[t] = e[t] * max_m + rank[t] when
    rank[t] < max_m, else -1;  masked_m[g] = min(counts[g], max_m)."""
    e = np.asarray(expert_idx, np.int64)
    counts = moe_counts(e, num_groups)
    rank = moe_ranks(e, num_groups)
    dst = np.full(e.size, -1, np.int64)
    keep = (rank >= 0) & (rank < max_m)
    dst[keep] = e[keep] * max_m + rank[keep]
    masked_m = np.minimum(counts, max_m)
    return counts.astype(np.int32), dst.astype(np.int32), masked_m.astype(np.int32)


def moe_contiguous_rows(num_tokens: int, num_groups: int, align: int = 128) -> int:
    """Rows that always suffice for the contiguous layout: every expert adds
    at most align - 1 padding rows."""
    return int(_ceil_to(np.int64(num_tokens + num_groups * (align - 1)), align))


def moe_scatter_rows(q, scales, dst_row, out_rows: int, rows_per_group: int, q_out, scales_out):
    """Moves token t's codes q[t] and its row of scales (logical [T][KG])
    to row dst_row[t] of the laid-out operand.  `scales_out` is logical
    [out_rows][KG]; rows of `q_out` / `scales_out` no token lands on keep
    their contents.  (`rows_per_group` only fixes the device layout of the
    scales; the logical result does not depend on it.)"""
    del rows_per_group
    dst = np.asarray(dst_row, np.int64)
    for t in range(dst.size):
        d = dst[t]
        if 0 <= d < out_rows:
            q_out[d] = q[t]
            scales_out[d] = scales[t]
    return q_out, scales_out


def moe_gather_rows(y, dst_row, n: int):
    """out[t] = y[dst_row[t]] (BF16 bit patterns); zeros where dst_row[t] < 0."""
    dst = np.asarray(dst_row, np.int64)
    out = np.zeros((dst.size, n), np.uint16)
    for t in range(dst.size):
        if dst[t] >= 0:
            out[t] = y[dst[t]]
    return out
