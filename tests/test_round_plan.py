"""Round structure from token IDs (host side): the oracle against hand-worked
examples and brute-force invariants, then the library's planner against the
oracle, exactly.

The worked examples follow the pages' prompt shape (TokenDance notes §2a:
a prompt is the round's outputs plus the agent's own history, joined with
separators; Figure 1: the same outputs at different offsets in each agent's
prompt).  Their expected layouts below were derived by hand from the
definitions in ``oracle/round_oracle.py``.
"""

import ctypes
import itertools
import os

import numpy as np
import pytest

import oracle as O
from collective_kv_cache_amd import tdx

SEP = 0
O_A, O_B, O_C = [11, 12, 13], [21, 22], [31, 32, 33, 34]
R0 = [101, 102, SEP] + O_A + [SEP] + O_B + [SEP] + O_C
R1 = [111, SEP] + O_C + [SEP] + O_A + [SEP] + O_B
R2 = [121, 122, 123, SEP] + O_B + [SEP] + O_C + [SEP] + O_A + [SEP]
R3 = [SEP] + O_A + [SEP, SEP] + O_B + [SEP] + O_A  # leading and doubled separators, a repeat

MAP0 = [-1, -1, -1, 0, 1, 2, -1, 3, 4, -1, 5, 6, 7, 8]
MAP1 = [-1, -1, 5, 6, 7, 8, -1, 0, 1, 2, -1, 3, 4]
MAP2 = [-1, -1, -1, -1, 3, 4, -1, 5, 6, 7, 8, -1, 0, 1, 2, -1]
ABC = dict(seg_ids=[1, 2, 3], blk_start=[0, 3, 5, 9], src_pos=[0, 3, 5])

WORKED = [
    # three agents, every output shared by all: one group, T = 9
    (([R0, R1, R2],), {},
     dict(groups=[dict(agents=[0, 1, 2], **ABC, dst_pos=[[3, 7, 10], [7, 11, 2], [12, 4, 7]],
                       priv_len=[5, 4, 7])],
          request_group=[0, 0, 0], token_maps=[MAP0, MAP1, MAP2])),
    # slot ranges: R1 intersects R0, so it opens a second group; R2 meets R0
    # only at a boundary (half-open ranges) and joins the first
    (([R0, R1, R2],), dict(slots=[(0, 100), (50, 150), (100, 200)]),
     dict(groups=[dict(agents=[0, 2], **ABC, dst_pos=[[3, 7, 10], [12, 4, 7]], priv_len=[5, 7]),
                  dict(agents=[1], seg_ids=[3, 1, 2], blk_start=[0, 4, 7, 9], src_pos=[0, 4, 7],
                       dst_pos=[[2, 7, 11]], priv_len=[4])],
          request_group=[0, 1, 0],
          token_maps=[MAP0, [-1, -1, 0, 1, 2, 3, -1, 4, 5, 6, -1, 7, 8], MAP2])),
    # min_share = 2: O_C (held by 3 of 4) is shared, R3 lacks it and forms
    # its own group; R3's second O_A is a private repeat
    (([R0, R1, R2, R3],), dict(min_share=2),
     dict(groups=[dict(agents=[0, 1, 2], **ABC, dst_pos=[[3, 7, 10], [7, 11, 2], [12, 4, 7]],
                       priv_len=[5, 4, 7]),
                  dict(agents=[3], seg_ids=[1, 2], blk_start=[0, 3, 5], src_pos=[0, 3],
                       dst_pos=[[1, 6]], priv_len=[7])],
          request_group=[0, 0, 0, 1],
          token_maps=[MAP0, MAP1, MAP2, [-1, 0, 1, 2, -1, -1, 3, 4, -1, -1, -1, -1]])),
    # shared by every request: O_C drops out, one group of four
    (([R0, R1, R2, R3],), {},
     dict(groups=[dict(agents=[0, 1, 2, 3], seg_ids=[1, 2], blk_start=[0, 3, 5], src_pos=[0, 3],
                       dst_pos=[[3, 7], [7, 11], [12, 4], [1, 6]], priv_len=[9, 8, 11, 7])],
          request_group=[0, 0, 0, 0],
          token_maps=[[-1, -1, -1, 0, 1, 2, -1, 3, 4, -1, -1, -1, -1, -1],
                      [-1, -1, -1, -1, -1, -1, -1, 0, 1, 2, -1, 3, 4],
                      [-1, -1, -1, -1, 3, 4, -1, -1, -1, -1, -1, -1, 0, 1, 2, -1],
                      [-1, 0, 1, 2, -1, -1, 3, 4, -1, -1, -1, -1]])),
]


def _lists(plan):
    """A plan (oracle lists or library arrays) as plain lists."""
    def conv(x):
        return x.tolist() if isinstance(x, np.ndarray) else x
    return dict(groups=[{k: conv(v) for k, v in g.items()} for g in plan["groups"]],
                request_group=conv(plan["request_group"]),
                token_maps=[conv(m) for m in plan["token_maps"]])


@pytest.mark.parametrize("case", range(len(WORKED)))
def test_oracle_worked_examples(case):
    args, kw, want = WORKED[case]
    got = _lists(O.round_plan(*args, SEP, **kw))
    assert got == want


def test_oracle_segments_edge_cases():
    assert O.segments([], SEP) == []
    assert O.segments([SEP, SEP], SEP) == []
    assert O.segments([5], SEP) == [(0, 1)]
    assert O.segments([SEP, 5, 6, SEP, SEP, 7, SEP], SEP) == [(1, 2), (5, 1)]
    assert O.segments([4, 4, SEP, 4], SEP) == [(0, 2), (3, 1)]


# ---- seeded random rounds and a brute-force check of every definition -------

def random_round(rng, R):
    pool = [rng.integers(1, 6, size=int(rng.integers(1, 5))).tolist() for _ in range(int(rng.integers(1, 7)))]
    reqs = []
    for _ in range(R):
        parts = []
        if rng.random() < 0.8:
            parts.append(rng.integers(1000, 1010, size=int(rng.integers(0, 5))).tolist())
        for c in rng.permutation(len(pool))[: int(rng.integers(0, len(pool) + 1))]:
            parts.append(pool[int(c)])
        if rng.random() < 0.3:
            parts.append(pool[int(rng.integers(len(pool)))])
        toks = []
        for p in parts:
            toks += [SEP] * int(rng.integers(0, 3)) + p  # no separator: two parts merge into one segment
        toks += [SEP] * int(rng.integers(0, 2))
        reqs.append(toks)
    return reqs


def random_slots(rng, R):
    b = rng.integers(0, 40, size=R)
    return [(int(x), int(x + rng.integers(0, 15))) for x in b]


def runs(tokens):
    """(start, content) of every maximal run of non-separator tokens."""
    out, p = [], 0
    for is_sep, grp in itertools.groupby(tokens, key=lambda t: t == SEP):
        g = list(grp)
        if not is_sep:
            out.append((p, tuple(g)))
        p += len(g)
    return out


def check_plan(reqs, plan, min_share, slots):
    R = len(reqs)
    need = R if min_share <= 0 else min_share
    rs = [runs(r) for r in reqs]
    holders = {}
    for r in range(R):
        for _, c in rs[r]:
            holders.setdefault(c, set()).add(r)
    span = [frozenset(c for _, c in rs[r] if len(holders[c]) >= need) for r in range(R)]
    seen = set()
    groups = plan["groups"]
    assert [g["agents"][0] for g in groups] == sorted(g["agents"][0] for g in groups)
    for gi, g in enumerate(groups):
        members = g["agents"]
        assert members == sorted(members)
        bs = g["blk_start"]
        T = bs[-1]
        first = members[0]
        contents = [tuple(reqs[first][g["dst_pos"][0][b]: g["dst_pos"][0][b] + bs[b + 1] - bs[b]])
                    for b in range(len(bs) - 1)]
        assert g["src_pos"] == bs[:-1]
        if g["dst_pos"]:
            # blocks in order of first appearance in the first member
            assert g["dst_pos"][0] == sorted(g["dst_pos"][0])
        for i, r in enumerate(members):
            assert r not in seen
            seen.add(r)
            assert plan["request_group"][r] == gi
            assert span[r] == span[first] == frozenset(contents)
            starts = {}
            for s, c in rs[r]:
                starts.setdefault(c, s)  # first occurrence
            m = plan["token_maps"][r]
            assert len(m) == len(reqs[r])
            want = [-1] * len(reqs[r])
            for b, c in enumerate(contents):
                d = g["dst_pos"][i][b]
                assert d == starts[c]
                for j in range(len(c)):
                    want[d + j] = bs[b] + j
            assert m == want
            assert g["priv_len"][i] == len(reqs[r]) - T
        if slots is not None:
            for a, b in itertools.combinations(members, 2):
                assert not (slots[a][0] < slots[b][1] and slots[b][0] < slots[a][1])
    assert seen == set(range(R))
    # greedy placement: an earlier group of the same span was refused only
    # because one of its members (placed before r) intersects r's slots
    for r in range(R):
        gi = plan["request_group"][r]
        for gj, g in enumerate(groups[:gi]):
            if g["agents"][0] < r and span[g["agents"][0]] == span[r]:
                assert slots is not None
                assert any(slots[m][0] < slots[r][1] and slots[r][0] < slots[m][1]
                           for m in g["agents"] if m < r)


@pytest.mark.parametrize("seed", range(40))
def test_oracle_brute_force_invariants(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.integers(1, 8))
    reqs = random_round(rng, R)
    min_share = int(rng.integers(-1, R + 2))
    slots = random_slots(rng, R) if seed % 2 else None
    plan = _lists(O.round_plan(reqs, SEP, min_share=min_share, slots=slots))
    check_plan(reqs, plan, min_share, slots)


# ---- the library's planner ----------------------------------------------------

needs_lib = pytest.mark.skipif(not os.path.exists(tdx.LIB_PATH), reason="libtdx.so not built")


@needs_lib
@pytest.mark.parametrize("case", range(len(WORKED)))
def test_library_worked_examples(case):
    args, kw, want = WORKED[case]
    assert _lists(tdx.round_plan(*args, SEP, **kw)) == want


@needs_lib
@pytest.mark.parametrize("seed", range(200))
def test_library_matches_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.integers(1, 12))
    reqs = random_round(rng, R)
    min_share = int(rng.integers(-1, R + 2))
    slots = random_slots(rng, R) if seed % 3 == 0 else None
    got = _lists(tdx.round_plan(reqs, SEP, min_share=min_share, slots=slots))
    assert got == _lists(O.round_plan(reqs, SEP, min_share=min_share, slots=slots))


@needs_lib
def test_library_all_gather_round_at_scale():
    # 64 agents, 32 shared outputs of 100-300 tokens in per-agent orders,
    # private histories of 500-4000 tokens: one group, layout as defined
    rng = np.random.default_rng(7)
    outs = [rng.integers(1, 150000, size=int(rng.integers(100, 301))).tolist() for _ in range(32)]
    reqs = []
    for i in range(64):
        toks = rng.integers(150000, 152000, size=int(rng.integers(500, 4001))).tolist()
        for b in rng.permutation(32):
            toks += [SEP] + outs[int(b)]
        reqs.append(toks)
    got = _lists(tdx.round_plan(reqs, SEP))
    assert len(got["groups"]) == 1 and got["groups"][0]["blk_start"][-1] == sum(map(len, outs))
    check_plan(reqs, got, 0, None)
    assert got == _lists(O.round_plan(reqs, SEP))


@needs_lib
def test_library_rejects_bad_arguments():
    L = tdx.lib()
    h = ctypes.c_void_p()
    toks = np.array([1, 2, 0, 3], np.int32)
    off = np.array([0, 2, 4], np.int64)
    P = lambda a: ctypes.c_void_p(a.ctypes.data)  # noqa: E731
    assert L.tdx_round_plan_build(P(toks), P(off), 2, 0, 0, None, None, None) == tdx.TDX_EINVAL
    assert L.tdx_round_plan_build(P(toks), P(off), 0, 0, 0, None, None, ctypes.byref(h)) == tdx.TDX_EINVAL
    assert h.value is None
    bad = np.array([0, 3, 2], np.int64)
    assert L.tdx_round_plan_build(P(toks), P(bad), 2, 0, 0, None, None, ctypes.byref(h)) == tdx.TDX_EINVAL
    assert "non-decreasing" in L.tdx_last_error().decode()
    assert L.tdx_round_plan_build(None, P(off), 2, 0, 0, None, None, ctypes.byref(h)) == tdx.TDX_EINVAL
    sb, se = np.array([5, 0], np.int64), np.array([4, 1], np.int64)
    assert L.tdx_round_plan_build(P(toks), P(off), 2, 0, 0, P(sb), None, ctypes.byref(h)) == tdx.TDX_EINVAL
    assert L.tdx_round_plan_build(P(toks), P(off), 2, 0, 0, P(sb), P(se), ctypes.byref(h)) == tdx.TDX_EINVAL
    assert L.tdx_round_plan_n_groups(None) == tdx.TDX_EINVAL
    assert L.tdx_round_plan_build(P(toks), P(off), 2, 0, 0, None, None, ctypes.byref(h)) == tdx.TDX_OK
    try:
        assert L.tdx_round_plan_n_groups(h) == 1  # nothing shared by both: one group, empty span
        assert L.tdx_round_plan_group_dims(h, 1, None, None, None) == tdx.TDX_EINVAL
        assert L.tdx_round_plan_group(h, -1, None, None, None, None, None, None) == tdx.TDX_EINVAL
        assert L.tdx_round_plan_request(h, 2, None, None) == tdx.TDX_EINVAL
    finally:
        L.tdx_round_plan_free(h)


@needs_lib
def test_library_empty_requests_and_no_sharing():
    got = _lists(tdx.round_plan([[], [SEP, SEP], [7]], SEP))
    # no block is held by all three: every request has the empty span -> one group, T = 0
    assert got["groups"] == [dict(agents=[0, 1, 2], seg_ids=[], blk_start=[0], src_pos=[],
                                  dst_pos=[[], [], []], priv_len=[0, 2, 1])]
    assert got["token_maps"] == [[], [-1, -1], [-1]]
