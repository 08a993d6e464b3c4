"""Route / sort-by-expert table (oracle; test infrastructure only)."""
from __future__ import annotations

import numpy as np


def route_prep(topk_ids: np.ndarray, E: int):
    """Group the (token, slot) pairs by expert.

    Pair id p = t*k + j for topk_ids[t, j] (megamoe_rm.cu, route_prep: a pair
    is identified by token*topk + k).  An id of -1 means "no expert" and is
    skipped (megamoe_rm.cu, route_prep and combine).  Any other id outside
    [0, E) is also skipped and counted in n_invalid (reading: the pages define
    only -1).

    Within one expert the pairs keep ascending pair-id order: megamoe_rm.cu's
    route_prep gives each pair the rank among earlier pairs with the same
    expert, so the table is unique.  offsets is the exclusive prefix over
    experts, [E+1] entries with rows offsets[e]..offsets[e+1] belonging to
    expert e (the total_tokens_including_expert table of CUTLASS discussion
    #2855).

    Returns (offsets int32 [E+1], sorted_pair_ids int32 [P] (-1 past
    offsets[E]), pair_to_sorted int32 [P] (-1 for skipped pairs), n_invalid).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    P = ids.size
    valid = (ids >= 0) & (ids < E)
    n_invalid = int(np.count_nonzero((ids != -1) & ~valid))
    counts = np.bincount(ids[valid], minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    vp = np.nonzero(valid)[0]                        # valid pair ids, ascending
    srt = vp[np.argsort(ids[vp], kind="stable")]     # by expert, then pair id
    sorted_pair_ids = np.full(P, -1, np.int32)
    sorted_pair_ids[: srt.size] = srt
    pair_to_sorted = np.full(P, -1, np.int32)
    pair_to_sorted[srt] = np.arange(srt.size, dtype=np.int32)
    return offsets, sorted_pair_ids, pair_to_sorted, n_invalid
