"""Pins for the oracle's work lists (jaehun.me section 3.4 "Work scheduling": an item is
256 consecutive queries of one document, its cost the number of key blocks it visits,
items sorted by descending cost and assigned in alternating directions; the backward
orders key tiles by descending cost.  agihunt.info: the list for 131,072 one-token
documents)."""
import numpy as np

from precision_causal_attention_token_amd import workloads


def _check(orc, cu, G=7):
    L = np.diff(cu).astype(np.int64)
    for kind, size in ((0, 256), (1, 128)):
        items = orc.worklist(cu, kind, G)
        n_expect = int(((L + size - 1) // size).sum())
        assert items.shape == (n_expect, 4)                               # W1: item count
        # W2: closed-form total cost.  fwd: doc with n items and m = ceil(L/128) key tiles
        # costs 2 + 4 + ... + 2(n-1) + m = n(n-1) + m ; bwd: m + (m-1) + ... + 1.
        m = (L + 127) // 128
        n = (L + 255) // 256
        total = (n * (n - 1) + m)[L > 0].sum() if kind == 0 else (m * (m + 1) // 2).sum()
        assert items[:, 2].sum() == total
        # W3: a permutation of the enumeration, non-increasing cost; among equal costs the
        # documents longer than 8 tokens first, then the shorter ones (one item each, at the
        # end of the list), each in enumeration order
        enum = [(k, b) for k in range(len(L)) for b in range(int((L[k] + size - 1) // size))]
        assert sorted(map(tuple, items[:, :2].tolist())) == enum
        assert np.all(np.diff(items[:, 2]) <= 0)
        small = L[items[:, 0]] <= 8
        n_small = int(((L >= 1) & (L <= 8)).sum())
        assert orc.small_docs(cu) == n_small
        assert not small[:len(items) - n_small].any() and small[len(items) - n_small:].all()
        for c in np.unique(items[:, 2]):
            for sm in (False, True):
                sel = items[(items[:, 2] == c) & (small == sm), :2]
                keys = sel[:, 0].astype(np.int64) * 1_000_000 + sel[:, 1]
                assert np.all(np.diff(keys) > 0)
        # each item's cost against its own definition (brute force over its keys)
        for doc, blk, cost, _ in items[:50]:
            Ld = int(L[doc])
            if kind == 0:
                qs = range(256 * blk, min(256 * (blk + 1), Ld))
                visited = {j // 128 for i in qs for j in range(0, i + 1, 127)} | {i // 128 for i in qs}
                assert cost == len(visited)
            else:
                assert cost == len(range(128 * blk, Ld, 128))
        # serpentine tags
        idx = np.arange(len(items))
        r, w = idx // G, idx % G
        assert np.array_equal(items[:, 3], np.where(r % 2 == 0, w, G - 1 - w))


def test_random_small(orc):
    for seed in range(8):
        lens = workloads.random_lengths(3000, 1, 700, seed=seed)
        if seed % 2:
            lens[1] = 0  # an empty document
        _check(orc, workloads.cu_seqlens(lens))


def test_lognormal_workload(orc):
    _check(orc, workloads.cu_seqlens(workloads.doc_lengths("lognormal")))


def test_extreme_packing_lists(orc):
    """W4: one 131072-token document -> forward costs 1024, 1022, ..., 2; 131072 one-token
    documents -> 131072 cost-1 items in enumeration order."""
    one = workloads.cu_seqlens([131072])
    f = orc.worklist(one, 0, 256)
    assert np.array_equal(f[:, 2], np.arange(1024, 0, -2))
    assert np.array_equal(f[:, 1], np.arange(511, -1, -1))
    b = orc.worklist(one, 1, 256)
    assert np.array_equal(b[:, 2], np.arange(1024, 0, -1))
    toks = workloads.cu_seqlens([1] * 131072)
    for kind in (0, 1):
        t = orc.worklist(toks, kind, 256)
        assert len(t) == 131072 and np.all(t[:, 2] == 1)
        assert np.array_equal(t[:, 0], np.arange(131072)) and not t[:, 1].any()


def test_schedule_rule(orc):
    """[J] §3.4 "Work scheduling": non-causal calls switch to dynamic assignment when the longest
    document is at least 4x the average.  Hand-worked cases: the pages' skewed mix (one 8192-token
    document and 224 of 256: longest 8192 against an average of 291), equal lengths, the boundary
    on both sides (longest exactly 4x the average, and one token short), empty documents counted
    in the average, no documents; causal kinds never."""
    cases = [([8192] + [256] * 224, 1), ([512] * 4, 0), ([8, 0, 0, 0], 1), ([7, 1, 0, 0], 0),
             ([12, 1, 1, 1, 0, 0, 0, 0, 0, 0, 0, 0], 1), ([3, 3, 3, 3], 0), ([], 0), ([0, 0], 0)]
    for lens, want in cases:
        cu = workloads.cu_seqlens(lens)
        for kind in (0, 1):
            assert orc.schedule_dynamic(cu, kind) == 0, (lens, kind)
        for kind in (2, 3):
            assert orc.schedule_dynamic(cu, kind) == want, (lens, kind)


def test_small_documents_last(orc):
    """W5: a hand-worked list.  Lengths 40, 5, 200, 1, 9, 0, 8, 129: documents 1, 3 and 6
    have at most 8 tokens, so their single cost-1 items close each list, after the cost-1
    items of documents 0 and 4 (and, backward, of the last key tiles of documents 2 and 7)."""
    cu = workloads.cu_seqlens([40, 5, 200, 1, 9, 0, 8, 129])
    want = {
        0: [(2, 0, 2), (7, 0, 2), (0, 0, 1), (4, 0, 1), (1, 0, 1), (3, 0, 1), (6, 0, 1)],
        1: [(2, 0, 2), (7, 0, 2), (0, 0, 1), (2, 1, 1), (4, 0, 1), (7, 1, 1), (1, 0, 1), (3, 0, 1), (6, 0, 1)],
        2: [(2, 0, 2), (7, 0, 2), (0, 0, 1), (4, 0, 1), (1, 0, 1), (3, 0, 1), (6, 0, 1)],
        3: [(2, 0, 2), (2, 1, 2), (7, 0, 2), (7, 1, 2), (0, 0, 1), (4, 0, 1), (1, 0, 1), (3, 0, 1), (6, 0, 1)],
    }
    for kind, ref in want.items():
        items = orc.worklist(cu, kind, 3)
        assert [tuple(x) for x in items[:, :3].tolist()] == ref, kind
        assert items[:, 3].tolist() == [0, 1, 2, 2, 1, 0, 0, 1, 2][:len(ref)]
    assert orc.small_docs(cu) == 3
