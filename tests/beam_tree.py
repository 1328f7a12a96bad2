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
