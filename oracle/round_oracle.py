"""Round structure from token IDs: the plain definition, on the host.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing in the product
path).  It shares no code with the library's round planner.

Sources ("notes" is the TokenDance deep-dive page "TokenDance: Scaling
Multi-Agent LLM Serving via Collective KV Cache Sharing", "blog" the Chinese
blog summary of the same paper):

* notes, Summary "Method" and §4 "Key Innovations" (Round-Aware Prompt
  Interface): the application marks logical block boundaries with a reserved
  separator token, and the runtime identifies blocks shared across agents by
  hashing segment content instead of position-based chunks.
* notes, §2a (end-to-end data flow and its stage table): prompt assembly
  with separators, then segment hashing (tokens to segment IDs), then
  grouping of compatible requests; Figure 1: the same content sits at
  different absolute positions in different agents' prompts.
* notes, §5 "Scheduling": requests join one group only under compatibility
  constraints (same cached span, disjoint slot mappings); otherwise they
  degrade to per-request reuse.
* blog §4.1: the separator token (<TTSEP>) between blocks.

Readings where the pages leave a step open:

* A segment is a maximal run of non-separator tokens; separators belong to
  no segment and count as private tokens; empty runs are not segments.
* Two segments are one block exactly when their token sequences are equal
  (content identity; a hash only indexes it).  Block IDs are dense, in order
  of first appearance scanning requests, then segments, in order.
* A block is shared when it appears in at least ``min_share`` distinct
  requests (``min_share <= 0``: in every request).  In one request only its
  first occurrence is the shared copy; later repeats are private.
* A request's cached span is the set of shared blocks it holds.  Requests
  are grouped by equal cached span, so every member holds every block of the
  group and the shared region has the same length in all of them; its total
  prompt length may differ (Figure 1's unequal histories are the case the
  method exists for).  With slot ranges given, a request joins the first
  group of its span (lowest first member) none of whose members' ranges
  intersects its own, else it opens a new group.  Groups are numbered by
  their first member.
* A group's canonical block order is the order of first appearance in its
  first member.  ``blk_start`` is the prefix sum of block lengths,
  ``src_pos[b] = blk_start[b]`` (the cached K of a block is taken at its
  canonical position), ``dst_pos[i][b]`` is the offset of block b's shared
  copy in member i, ``priv_len[i]`` the member's other tokens.
* ``token_map[r][p]`` is the canonical index of token p of request r in its
  group's shared region, or -1 for a private token.

Pins (tests/test_round_plan.py): four hand-worked rounds with literal expected
layouts (slot splits, min_share, a private repeat, leading and doubled
separators), separator edge cases, and brute-force restatements of every rule
above on seeded random rounds (itertools.groupby runs, holder counts, content
at every dst_pos, first occurrences, token maps, priv_len, slot
disjointness, greedy placement).  No function here is "parity unpinned".
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


def segments(tokens: Sequence[int], sep: int) -> List[Tuple[int, int]]:
    """(start, length) of every maximal run of non-separator tokens."""
    out = []
    start = None
    for p, tok in enumerate(tokens):
        if tok == sep:
            if start is not None:
                out.append((start, p - start))
                start = None
        elif start is None:
            start = p
    if start is not None:
        out.append((start, len(tokens) - start))
    return out


def _overlap(a: Tuple[int, int], b: Tuple[int, int]) -> bool:
    """Half-open ranges [a0, a1) and [b0, b1) share a slot."""
    return a[0] < b[1] and b[0] < a[1]


def round_plan(requests: Sequence[Sequence[int]], sep: int, min_share: int = 0,
               slots: Optional[Sequence[Tuple[int, int]]] = None) -> Dict:
    """Groups, per-group layouts and per-request token maps of one round."""
    R = len(requests)
    reqs = [list(map(int, r)) for r in requests]
    need = R if min_share <= 0 else min_share

    # content identity: dense IDs in order of first appearance
    ids: Dict[Tuple[int, ...], int] = {}
    seg_of = []      # per request: [(start, length, id)]
    holders = []     # per id: set of requests holding it
    lengths = []     # per id: token count
    for r, toks in enumerate(reqs):
        lst = []
        for start, n in segments(toks, sep):
            key = tuple(toks[start:start + n])
            if key not in ids:
                ids[key] = len(ids)
                holders.append(set())
                lengths.append(n)
            c = ids[key]
            holders[c].add(r)
            lst.append((start, n, c))
        seg_of.append(lst)
    shared = [len(h) >= need for h in holders]

    # each request's shared copies: first occurrence of every shared block
    first: List[Dict[int, int]] = []
    order: List[List[int]] = []
    for r in range(R):
        f: Dict[int, int] = {}
        o: List[int] = []
        for start, n, c in seg_of[r]:
            if shared[c] and c not in f:
                f[c] = start
                o.append(c)
        first.append(f)
        order.append(o)

    # grouping by cached span, splitting on intersecting slot ranges
    groups: List[List[int]] = []
    by_span: Dict[frozenset, List[int]] = {}
    request_group = [-1] * R
    for r in range(R):
        span = frozenset(first[r])
        placed = False
        for g in by_span.get(span, []):
            if slots is None or not any(_overlap(slots[r], slots[m]) for m in groups[g]):
                groups[g].append(r)
                request_group[r] = g
                placed = True
                break
        if not placed:
            by_span.setdefault(span, []).append(len(groups))
            request_group[r] = len(groups)
            groups.append([r])

    out_groups = []
    token_maps = [[-1] * len(reqs[r]) for r in range(R)]
    for g, members in enumerate(groups):
        blocks = order[members[0]]
        blk_start = [0]
        for c in blocks:
            blk_start.append(blk_start[-1] + lengths[c])
        T = blk_start[-1]
        dst = [[first[r][c] for c in blocks] for r in members]
        priv = [len(reqs[r]) - T for r in members]
        for i, r in enumerate(members):
            for b, c in enumerate(blocks):
                for j in range(lengths[c]):
                    token_maps[r][dst[i][b] + j] = blk_start[b] + j
        out_groups.append(dict(agents=list(members), seg_ids=list(blocks), blk_start=blk_start,
                               src_pos=blk_start[:-1], dst_pos=dst, priv_len=priv))
    return dict(groups=out_groups, request_group=request_group, token_maps=token_maps,
                n_segments=len(ids))
