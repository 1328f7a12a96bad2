"""Nested shared prefixes (a beam tree) made from a workload whose sequences
share one flat prefix, by repointing block-table entries at other full blocks
of that prefix.  The oracle reads the same tables, so any rewrite that keeps
every entry inside the context on a fully written block is a valid batch.
"""

import numpy as np


def two_levels(tables, groups, common):
    """Sequences in `groups` (lists of sequence indices, each list sharing its
    own prefix) all take the first `common` entries of the first group's
    leader: one root group over everything, each old group a child of it."""
    t = tables.copy()
    lead = groups[0][0]
    for g in groups:
        for b in g:
            t[b, :common] = tables[lead, :common]
    return t


def three_levels(tables, seqs, prefix):
    """Twelve sequences `seqs` sharing `prefix` blocks become a three-level
    tree: all twelve share blocks [0, 8); seqs[0:6] share [0, 20) and
    seqs[6:12] share [0, prefix) with blocks 8.. taken in reverse order;
    within the first six, seqs[3:6] take blocks 20.. in reverse order."""
    assert len(seqs) == 12 and prefix > 20
    t = tables.copy()
    lead = seqs[0]
    rev_hi = tables[lead, 8:prefix][::-1]
    rev_lo = tables[lead, 20:prefix][::-1]
    for b in seqs[6:]:
        t[b, 8:prefix] = rev_hi
    for b in seqs[3:6]:
        t[b, 20:prefix] = rev_lo
    return t


def random_tree(tables, seqs, prefix, rng, lo=0, depth=0, max_depth=3):
    """Split `seqs` (sharing tables[s, :prefix]) into a random nested tree, in
    place: at a random block k past `lo`, a random tail of the list takes the
    blocks k..prefix-1 of its first member's row in reverse order (a different
    id at k, still full blocks of the prefix), and both parts split again."""
    if depth >= max_depth or len(seqs) < 4 or prefix - lo < 12:
        return
    k = int(rng.integers(lo + 1, prefix - 8))
    cut = int(rng.integers(2, len(seqs) - 1))
    head, tail = seqs[:cut], seqs[cut:]
    row = tables[tail[0], k:prefix][::-1].copy()
    for b in tail:
        tables[b, k:prefix] = row
    random_tree(tables, head, prefix, rng, k, depth + 1, max_depth)
    random_tree(tables, tail, prefix, rng, k, depth + 1, max_depth)
