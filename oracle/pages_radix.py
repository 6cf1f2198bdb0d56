"""The TopK article's radix-select method, restated step by step in plain Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  This is the second,
independent route to the selected set: where ``topk_oracle.c`` sorts by float
comparison, this module follows the article's five named steps (section 02 of
"How to Use FlagOS's New Triton-TLE Language to Build a TopK Selector Faster
Than FlashInfer"):

1. mapping     - each float becomes an unsigned integer whose order is the
                 float order (``float_to_ordered_u32``);
2. binning     - the integer is cut into digits from the most significant end;
                 the article's worked pseudocode uses decimal digits, so this
                 restatement does too (``highest_power_of_10`` gives the place
                 value of the leading decimal digit; the article's example maps
                 839 to 100);
3. histogram   - count how many surviving candidates fall in each digit value;
4. threshold   - walk the digit values from 9 down to 0 to find the one holding
                 the element of the wanted rank, keep only that bucket, and
                 continue with the next lower digit;
5. collection  - with T, the k-th largest value, known: take every element
                 above T, then elements equal to T in scan (index) order until
                 k are held.

With the pseudocode's need_sorted option the collected output is then sorted
in descending order (``radix_topk_sorted``).

Pure-Python loops: meant for rows of a few thousand elements at most.
Readings where the article leaves a step open:
- the pseudocode works on non-negative integers; it is applied here to the
  mapped keys, which are non-negative by construction;
- ``highest_power_of_10(0)`` is undefined in the article; it is taken as 1 so a
  row whose largest key is 0 still runs one (trivial) digit round;
- -0.0 is mapped to the key of +0.0 (the two compare equal as floats, so they
  must tie); NaN keys are not produced (NaN is outside the contract);
- the descending sort of need_sorted is taken as stable: equal values keep the
  order in which the collection took them, which is index order.
"""

from __future__ import annotations

import struct
from typing import List, Sequence, Tuple


def float_to_ordered_u32(x: float) -> int:
    """Mapping step: an unsigned 32-bit key with key(a) < key(b) iff a < b for
    non-NaN float32 values a, b, and key(-0.0) == key(+0.0)."""
    (bits,) = struct.unpack("<I", struct.pack("<f", x))
    if bits == 0x80000000:  # -0.0 ties with +0.0
        bits = 0
    if bits & 0x80000000:
        # negative: larger magnitude must give a smaller key -> complement
        return (~bits) & 0xFFFFFFFF
    # non-negative: shift above every negative key
    return bits | 0x80000000


def highest_power_of_10(m: int) -> int:
    """Place value of the leading decimal digit of m (839 -> 100).  For m == 0
    the article gives no value; 1 is used."""
    p = 1
    while p * 10 <= m:
        p *= 10
    return p


def radix_select_kth_largest(keys: Sequence[int], k: int) -> int:
    """The k-th largest of ``keys`` (k counts from 1, with multiplicity), by
    decimal-digit histograms from the most significant digit down."""
    if not 1 <= k <= len(keys):
        raise ValueError("k out of range")
    candidates = list(keys)
    rank = k - 1  # zero-based rank among the candidates, counted from the top
    place = highest_power_of_10(max(candidates))
    while place > 0:
        count = [0] * 10
        for key in candidates:
            count[(key // place) % 10] += 1
        above = 0
        chosen = None
        for d in range(9, -1, -1):
            if rank < above + count[d]:
                chosen = d
                rank -= above
                break
            above += count[d]
        candidates = [key for key in candidates if (key // place) % 10 == chosen]
        place //= 10
    # every candidate left agrees on every digit: they are all equal
    return candidates[0]


def radix_topk_indices(values: Sequence[float], k: int) -> Tuple[List[int], int]:
    """Collection step on one row: indices of every value above the threshold,
    then of values equal to it in index order until k are held.  Returns the
    indices (in collection order) and the threshold key."""
    keys = [float_to_ordered_u32(v) for v in values]
    t = radix_select_kth_largest(keys, k)
    out = [i for i, key in enumerate(keys) if key > t]
    need = k - len(out)
    for i, key in enumerate(keys):
        if need == 0:
            break
        if key == t:
            out.append(i)
            need -= 1
    return out, t


def radix_topk_row(values: Sequence[float], k: int, length: int = None) -> List[int]:
    """One output row under the selector's contract: the valid prefix of
    ``length`` positions (all when None) is selected from; when fewer than k
    positions are valid they are all returned and the row is padded with -1."""
    L = len(values) if length is None else max(0, min(int(length), len(values)))
    if L <= k:
        return list(range(L)) + [-1] * (k - L)
    out, _ = radix_topk_indices(values[:L], k)
    return out


def radix_topk_sorted(values: Sequence[float], k: int) -> List[int]:
    """need_sorted: the collected indices sorted by value, largest first; a
    stable sort, so equal values stay in collection (= index) order."""
    out, _ = radix_topk_indices(values, k)
    keys = [float_to_ordered_u32(v) for v in values]
    return sorted(out, key=lambda i: keys[i], reverse=True)
