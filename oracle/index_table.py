"""Chunk-index table and its static bound, written as plain loops.

Test infrastructure: see the package docstring.

Source: FLA issue 1155, "[RFC] Graph capture support for prefill and
training", section "Core design":
  * NT_max = cdiv(T_max, 64) + N_max - 1 bounds the chunk count of any batch of
    at most T_max tokens in at most N_max sequences.
  * The table has a fixed shape [NT_max, 2]; each used slot holds (sequence id,
    position of the chunk inside its sequence); unused slots hold a sentinel.
  * cu_seqlens is padded to N_max + 1 entries with zero-length sequences.
Readings (the page does not fix them): the second column is the 0-based chunk
number within the sequence (first token = bos + 64 * c); the sentinel is
(-1, -1); used slots come first, in (sequence, chunk) order.
"""

from __future__ import annotations


def cdiv(a: int, b: int) -> int:
    return -(-a // b)


def nt_max(t_max: int, n_max: int, chunk: int = 64) -> int:
    """Static upper bound on the number of chunks (FLA RFC, "Core design")."""
    return cdiv(t_max, chunk) + n_max - 1


def chunk_count(cu_seqlens, chunk: int = 64) -> int:
    return sum(cdiv(cu_seqlens[i + 1] - cu_seqlens[i], chunk) for i in range(len(cu_seqlens) - 1))


def chunk_index_table(cu_seqlens, nt_cap: int, chunk: int = 64):
    """Fill a [nt_cap][2] table by walking every sequence's chunks in order."""
    table = []
    for s in range(len(cu_seqlens) - 1):
        length = cu_seqlens[s + 1] - cu_seqlens[s]
        for c in range(cdiv(length, chunk)):
            table.append([s, c])
    if len(table) > nt_cap:
        raise ValueError("more chunks than table slots")
    while len(table) < nt_cap:
        table.append([-1, -1])
    return table
