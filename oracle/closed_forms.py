"""Closed forms for KV memory accounting (test infrastructure; see oracle/__init__).

[P3] "Equations and derivations":
  Eq. (1)  M_KV = 2 * L * n * h_KV * d_h * b   (factor 2 = key and value,
           b = bytes per scalar; block tables, workspace and padding excluded)
  Eq. (2)  A_B(n) = B * ceil(n / B),  W_B(n) = A_B(n) - n
           (a fixed reservation of M slots wastes M - n instead)
  Eq. (3)  U = sum_i n_i / sum_i B * ceil(n_i / B)   (slot utilisation only)
The guide's captions are printed before each formula and run into the next
number; caption k is read as belonging to the formula that follows it.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Iterable


def kv_bytes(num_layers: int, num_tokens: int, num_kv_heads: int, head_dim: int, bytes_per_scalar: int) -> int:
    """Eq. (1) of [P3]: bytes of K and V for ``num_tokens`` tokens."""
    return 2 * num_layers * num_tokens * num_kv_heads * head_dim * bytes_per_scalar


def blocks_for(n: int, block_size: int) -> int:
    """Number of blocks a sequence of ``n`` tokens occupies: ceil(n / B) ([P3] section 2)."""
    if n < 0 or block_size <= 0:
        raise ValueError("n >= 0 and B > 0 required")
    return -(-n // block_size)


def allocated_slots(n: int, block_size: int) -> int:
    """Eq. (2) of [P3]: A_B(n) = B * ceil(n / B)."""
    return block_size * blocks_for(n, block_size)


def tail_waste(n: int, block_size: int) -> int:
    """Eq. (2) of [P3]: W_B(n) = A_B(n) - n (at most B - 1)."""
    return allocated_slots(n, block_size) - n


def fixed_reservation_slots(lengths: Iterable[int], max_len: int) -> int:
    """Slots reserved when every request reserves ``max_len`` contiguous slots ([P3] Eq. (2) caption)."""
    lengths = list(lengths)
    if any(n > max_len for n in lengths):
        raise ValueError("a length exceeds the reservation")
    return max_len * len(lengths)


def utilisation(lengths: Iterable[int], block_size: int) -> Fraction:
    """Eq. (3) of [P3] as an exact fraction: sum n_i / sum A_B(n_i)."""
    lengths = list(lengths)
    return Fraction(sum(lengths), sum(allocated_slots(n, block_size) for n in lengths))


def fixed_utilisation(lengths: Iterable[int], max_len: int) -> Fraction:
    """Slot utilisation of a fixed ``max_len`` reservation: sum n_i / (M * count)."""
    lengths = list(lengths)
    return Fraction(sum(lengths), fixed_reservation_slots(lengths, max_len))
