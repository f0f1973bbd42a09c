"""Group-by-expert permutation of the routed slots (oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Page "MoE推理优化实战：4bit存储+INT8计算的W4A8路线解析", §1: routing dispatch and
result combination are overheads of their own; the permutation is the dispatch
step that gathers every expert's rows together.

Slots are numbered s = t * k + j (token t, choice j).  Definition:

* counts[e] = number of slots routed to expert e;
* offsets = [0, cumsum(counts)] (E + 1 entries);
* perm[p] = the slot at position p, positions sorted by expert and, inside
  one expert, by slot number (a stable order);
* inv[s] = the position of slot s (perm[inv[s]] = s).

Pinned by (tests/test_oracle_permute.py): equality with numpy's stable
argsort and bincount, and the invariants (sum of counts = T k, perm a
bijection, ids[perm] non-decreasing, slot order increasing inside an expert).
"""
import numpy as np


def permute(ids, num_experts):
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1)
    counts = np.zeros(num_experts, dtype=np.int64)
    for e in flat:                       # plain histogram
        counts[e] += 1
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    for e in range(num_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for s, e in enumerate(flat):         # slots in increasing order -> stable
        perm[fill[e]] = s
        fill[e] += 1
    inv = np.empty_like(perm)
    inv[perm] = np.arange(flat.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv.astype(np.int32))
