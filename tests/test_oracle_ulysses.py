"""Pins for the Ulysses simulation: over any number of ranks that divides the
heads, the sharded computation (head-sharded cache, sequence-sharded video
rows, all-to-all both ways, gather) equals the unsharded attention; the pure
data movement round-trips; and plausible bookkeeping slips are caught."""
import importlib

import numpy as np
import pytest

import oracle
from tests.pins import random_bits

uly = importlib.import_module("oracle.ulysses")


def _inputs(seed=0, H=8, hd=16, n_video=13, n_audio=3, cap=48, length=40, head=11):
    rng = np.random.default_rng(seed)
    n_q = n_video + n_audio
    return dict(q=random_bits(rng, (n_q, H, hd)), ring_k=random_bits(rng, (H, cap, hd)),
                ring_v=random_bits(rng, (H, cap, hd)), length=length, head=head,
                k_u=random_bits(rng, (n_q, H, hd)), v_u=random_bits(rng, (n_q, H, hd)),
                n_video=n_video)


def _sharded_error(P, **kw):
    x = _inputs(**kw)
    want = oracle.attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                            x["k_u"], x["v_u"])
    got = oracle.ulysses_attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                                   x["k_u"], x["v_u"], x["n_video"], P)
    return float(np.max(np.abs(got - want)))


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_sharded_equals_global_attention(P):
    assert _sharded_error(P) <= 1e-15


def test_ragged_shards_and_no_audio():
    assert _sharded_error(4, n_video=5, n_audio=0) <= 1e-15      # 5 rows over 4 ranks
    assert _sharded_error(2, n_video=1, n_audio=4) <= 1e-15      # one rank has no video


def test_exchanges_round_trip():
    rng = np.random.default_rng(1)
    H, n_video, n_audio, P = 8, 11, 2, 4
    x = rng.standard_normal((n_video + n_audio, H, 3))
    shards = uly.shard_sequence(x, n_video, P)
    per_head = uly.seq_to_head(shards, n_video, P, H)
    for r, t in enumerate(per_head):               # every token, this rank's heads
        h0, h1 = uly.head_range(H, P, r)
        assert np.array_equal(t, x[:, h0:h1])
    back = uly.head_to_seq(per_head, n_video, P, H)
    assert all(np.array_equal(a, b) for a, b in zip(back, shards))
    assert np.array_equal(uly.gather_sequence(back, n_video, P), x)


def test_heads_must_divide():
    with pytest.raises(ValueError):
        uly.head_range(8, 3, 0)


def test_reversed_rank_order_is_caught(monkeypatch):
    # mistake: the sequence -> head exchange stacks the video shards in reverse
    orig = uly.seq_to_head

    def reversed_order(shards, n_video, P, H):
        out = orig(shards, n_video, P, H)
        chunks = uly.video_chunks(n_video, P)
        res = []
        for t in out:
            parts = [t[lo:hi] for lo, hi in chunks][::-1]
            res.append(np.concatenate(parts + [t[n_video:]]))
        return res
    monkeypatch.setattr(uly, "seq_to_head", reversed_order)
    assert _sharded_error(4) > 1e-3


def test_audio_counted_per_rank_is_caught(monkeypatch):
    # mistake: every rank's audio rows are gathered as keys, P copies of them
    orig = uly.seq_to_head

    def audio_from_all(shards, n_video, P, H):
        out = orig(shards, n_video, P, H)
        n_audio = shards[0].shape[0] - (uly.video_chunks(n_video, P)[0][1])
        return [np.concatenate([t] + [t[n_video:]] * (P - 1)) if n_audio else t for t in out]
    monkeypatch.setattr(uly, "seq_to_head", audio_from_all)
    x = _inputs()
    got = uly.ulysses_attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                                x["k_u"], x["v_u"], x["n_video"], 4)
    want = oracle.attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                            x["k_u"], x["v_u"])
    assert got.shape != want.shape or np.max(np.abs(got - want)) > 1e-3


def test_wrong_head_offset_is_caught(monkeypatch):
    # mistake: every rank uses the first head range of the cache
    monkeypatch.setattr(uly, "head_range", lambda H, P, r: (0, H // P) if H % P == 0 else None)
    x = _inputs()
    got = uly.ulysses_attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                                x["k_u"], x["v_u"], x["n_video"], 4)
    want = oracle.attention(x["q"], x["ring_k"], x["ring_v"], x["length"], x["head"],
                            x["k_u"], x["v_u"])
    assert np.max(np.abs(got - want)) > 1e-3
