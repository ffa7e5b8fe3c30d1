"""Pins of the attention-sink protection in the oracle cache (by hand: which
tokens end up protected, and that nothing else changes)."""
import numpy as np

import oracle as O


def test_sink_protection_by_hand():
    g = np.random.default_rng(3)
    B, H, D = 3, 2, 64
    k = g.standard_normal((B, 70, H, D)).astype(np.float32)
    v = g.standard_normal((B, 70, H, D)).astype(np.float32)
    plain = O.OracleCache(B, H, D, 2, 2, 32)
    sink = O.OracleCache(B, H, D, 2, 2, 32, protect_sink=True)
    prot = [np.array([5, 40]), np.array([0, 3]), np.array([], np.int64)]
    for c in (plain, sink):
        c.commit(0, k, v, ntok=[70, 33, 0], prot=prot)           # sequence 2 commits nothing yet
    assert sink.protected(0, 0)[0].tolist() == [0, 5, 40]        # the sink joins the list
    assert sink.protected(0, 1)[0].tolist() == [0, 3]            # already listed: not twice
    assert sink.protected(0, 2)[0].tolist() == []
    # the plain cache with the sink listed by hand is the same cache
    ref = O.OracleCache(B, H, D, 2, 2, 32)
    ref.commit(0, k, v, ntok=[70, 33, 0], prot=[np.array([0, 5, 40]), np.array([0, 3]), np.array([], np.int64)])
    for b in range(B):
        if sink.nslots(0, b):
            assert np.array_equal(sink.records(0, b), ref.records(0, b))
    # later commits, the first one of sequence 2, the suffix and a reset
    for c in (sink,):
        c.commit(0, k[:, :10], v[:, :10], ntok=[10, 10, 10])
        c.commit(1, k[:, :10], v[:, :10])
    assert sink.protected(0, 0)[0].tolist() == [0, 5, 40]        # position 70: not a sequence start
    assert sink.protected(0, 2)[0].tolist() == [0]               # sequence 2 starts now
    assert sink.protected(1, 0)[0].tolist() == []                # the suffix holds no sink
    sink.commit(0, k[:, :4], v[:, :4], reset=True)
    assert [sink.protected(0, b)[0].tolist() for b in range(B)] == [[0], [0], [0]]
