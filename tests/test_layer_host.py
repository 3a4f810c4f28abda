"""Host-side scheduling of the decode layer: which rows of a step go to the
prefill kernel (runs of at least two consecutive positions of one request) and
which stay decode rows.  No GPU."""
import numpy as np

from invariant_rmsnorm_bi_amd.layer import DecodeLayer


def _tabs(ids, width=4):
    return np.stack([np.full(width, i, dtype=np.int32) for i in ids])


def test_segments_split_prompt_chunks_from_decode_rows():
    bt = _tabs([0, 1, 2, 9, 9, 9, 5])
    assert DecodeLayer.segments(bt, [5, 9, 2, 0, 1, 2, 7]) == [(0, 3, -1), (3, 6, 0), (6, 7, -1)]


def test_segments_need_one_request_and_consecutive_positions():
    # consecutive positions of different requests, and one request's rows out of
    # order or repeated, are decode rows
    assert DecodeLayer.segments(_tabs([1, 2, 3]), [4, 5, 6]) == [(0, 3, -1)]
    assert DecodeLayer.segments(_tabs([1, 1, 1]), [4, 3, 3]) == [(0, 3, -1)]
    # two chunks of one request split by another request's row
    assert DecodeLayer.segments(_tabs([7, 7, 8, 7, 7]), [10, 11, 3, 12, 13]) == \
        [(0, 2, 10), (2, 3, -1), (3, 5, 12)]


def test_segments_cover_every_row_once():
    rng = np.random.default_rng(3)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        req = rng.integers(0, 3, B)
        pos = rng.integers(0, 6, B)
        segs = DecodeLayer.segments(_tabs(req), pos)
        assert segs[0][0] == 0 and segs[-1][1] == B
        for (a, b, p), (a2, _, _) in zip(segs, segs[1:] + [(B, B, -1)]):
            assert a < b == a2
            if p >= 0:
                assert b - a >= 2 and p == pos[a]
                assert (req[a:b] == req[a]).all() and (np.diff(pos[a:b]) == 1).all()
        # no two adjacent decode segments
        assert all(not (s[2] < 0 and t[2] < 0) for s, t in zip(segs, segs[1:]))
