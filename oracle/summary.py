"""The stable key-block summary and its merge, written out literally.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

Page "Stable summary of an attention key block", Definition:
* for a nonempty key set S of one query row i, the summary is the triple
  (m, l, z): m is the largest score over S, l is the sum over S of
  exp(s_j - m), and z is the same exponential weights applied to the value
  rows and summed;
* the empty set has its own state with no numeric coordinates (BOTTOM here);
* two summaries of disjoint nonempty sets merge by taking the larger m as the
  new shift and rescaling each side's l and z by exp(old m - new m) before
  adding;
* dividing z by l gives the attention output over S.

The definition gives the merge only for two nonempty sets.  Reading adopted
for the empty state: it is the identity of the merge, since the union of the
empty set with T is T.

The exponential is a parameter so that the same literal code can run in
float64 (``math.exp``) or in mpmath.
"""

from __future__ import annotations

import math

BOTTOM = None  # the state of the empty key set: no maximum, no coordinates


def summary(scores, values, key_set, exp=math.exp):
    """(m, l, z) over the keys in ``key_set`` (BOTTOM if it is empty).

    scores: sequence of s_ij for one query row i (indexable by key j);
    values: sequence of value rows v_j (each a sequence of numbers).
    """
    key_set = list(key_set)
    if not key_set:
        return BOTTOM
    m = max(scores[j] for j in key_set)
    dim = len(values[key_set[0]])
    l = 0
    z = [0] * dim
    for j in key_set:
        w = exp(scores[j] - m)
        l = l + w
        for e in range(dim):
            z[e] = z[e] + w * values[j][e]
    return (m, l, z)


def merge(a, b, exp=math.exp):
    """The merge of two summaries of disjoint key sets."""
    if a is BOTTOM:
        return b
    if b is BOTTOM:
        return a
    m_a, l_a, z_a = a
    m_b, l_b, z_b = b
    m = max(m_a, m_b)
    fa = exp(m_a - m)
    fb = exp(m_b - m)
    l = fa * l_a + fb * l_b
    z = [fa * za + fb * zb for za, zb in zip(z_a, z_b)]
    return (m, l, z)


def finalize(state):
    """Attention output over the summarised set: z divided by l."""
    if state is BOTTOM:
        raise ValueError("the empty key set has no attention output")
    _, l, z = state
    return [ze / l for ze in z]


def fold(scores, values, blocks, tree, exp=math.exp):
    """Merge the summaries of ``blocks`` following the bracketing ``tree``.

    blocks: list of key lists (disjoint); tree: either an int (index of a
    block) or a pair (left_tree, right_tree).
    """
    if isinstance(tree, int):
        return summary(scores, values, blocks[tree], exp=exp)
    left, right = tree
    return merge(fold(scores, values, blocks, left, exp),
                 fold(scores, values, blocks, right, exp), exp=exp)
