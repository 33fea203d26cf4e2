"""Host-side description of prompt sharing for paged_attention_decode_shared.

Groups of sequences forked from one prompt share the physical blocks of it:
their block tables hold the same block ids at the same leading entries. For
each group this finds P, the number of tokens those shared leading blocks
hold (whole blocks, within every member's context, a multiple of 16), and
lays out the arrays the shared-prefix decode takes. Groups wider than the
kernel's member limit are split into several groups with the same prefix.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from ._binding import MAX_GROUP_MEMBERS

TILE = 16


def shared_prefix_groups(block_tables: np.ndarray, context_lens: np.ndarray, groups: Sequence[Sequence[int]],
                         block_size: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """(group_members int32 [G, 8], group_prefix int32 [G], seq_starts int32
    [S], max_prefix_len) for the given groups of sequence ids."""
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    S = lens.shape[0]
    seen = set()
    members, prefix = [], []
    for grp in groups:
        grp = [int(s) for s in grp]
        if not grp:
            continue
        if any(s < 0 or s >= S or s in seen for s in grp) or len(set(grp)) != len(grp):
            raise ValueError("groups must hold distinct valid sequence ids, each in one group")
        seen.update(grp)
        rows = tables[grp]
        same = (rows == rows[0]).all(axis=0)
        shared_blocks = int(np.argmin(same)) if not same.all() else rows.shape[1]
        full_blocks = int(lens[grp].min()) // block_size  # blocks every member has filled
        p = min(shared_blocks, full_blocks) * block_size
        p -= p % TILE
        for first in range(0, len(grp), MAX_GROUP_MEMBERS):
            part = grp[first:first + MAX_GROUP_MEMBERS]
            members.append(part + [-1] * (MAX_GROUP_MEMBERS - len(part)))
            prefix.append(p)
    starts = np.zeros(S, np.int32)
    for row, p in zip(members, prefix):
        for s in row:
            if s >= 0:
                starts[s] = p
    gm = np.array(members, np.int32).reshape(-1, MAX_GROUP_MEMBERS)
    gp = np.array(prefix, np.int32)
    return gm, gp, starts, int(gp.max()) if gp.size else 0
