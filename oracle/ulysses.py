"""Oracle: Ulysses-style context parallel attention over P performer ranks,
simulated on one host (no communication library: the exchanges are array
re-arrangements).

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the performer is a group of GPUs in Ulysses-style context parallel;
every rank keeps a pre-sharded local K/V cache, the long video latent sequence
is split along its tokens over the ranks, and around the attention of the
denoiser an all-to-all exchange moves the data between the sequence dimension
and the head dimension so that the result equals global attention; after
denoising a gather reassembles the sequence.  The short audio latent sequence
is not split: every rank handles it on its own
[Wan-Streamer v0.2: Higher Resolution, Same Latency (nanless digest),
方法概述和架构 and its summary].

Readings where the pages are silent:
* rank r owns heads [r H / P, (r + 1) H / P) (P divides H) and the video rows
  of the r-th of P contiguous, near-equal chunks (numpy's array_split); every
  rank holds all audio rows;
* the cache is pre-sharded by head, so rank r's ring is the head range of the
  full ring and needs no exchange;
* sequence -> head: rank r receives, for its heads, the video rows of every
  rank in rank order, followed by the audio rows (from its own copy);
* head -> sequence: rank r receives, for all heads, the outputs of its video
  rows and of all audio rows.
"""
from __future__ import annotations

import numpy as np

from .attention import attention


def video_chunks(n_video: int, P: int):
    """Row ranges [lo, hi) of the P video shards."""
    bounds = np.cumsum([0] + [len(c) for c in np.array_split(np.arange(n_video), P)])
    return [(int(bounds[r]), int(bounds[r + 1])) for r in range(P)]


def head_range(H: int, P: int, r: int):
    if H % P:
        raise ValueError(f"{P} ranks do not divide {H} heads")
    return r * H // P, (r + 1) * H // P


def shard_sequence(x, n_video: int, P: int):
    """Per rank: its video rows followed by all audio rows, all heads."""
    return [np.concatenate([x[lo:hi], x[n_video:]]) for lo, hi in video_chunks(n_video, P)]


def seq_to_head(shards, n_video: int, P: int, H: int):
    """All-to-all: rank r gets every rank's video rows (in rank order) of its
    heads, then the audio rows of its heads from its own shard."""
    chunks = video_chunks(n_video, P)
    out = []
    for r in range(P):
        h0, h1 = head_range(H, P, r)
        video = [shards[s][:hi - lo, h0:h1] for s, (lo, hi) in enumerate(chunks)]
        audio = shards[r][chunks[r][1] - chunks[r][0]:, h0:h1]
        out.append(np.concatenate(video + [audio]))
    return out


def head_to_seq(per_rank, n_video: int, P: int, H: int):
    """All-to-all back: rank r gets, for all heads, the rows of its video
    shard and all audio rows."""
    chunks = video_chunks(n_video, P)
    out = []
    for r, (lo, hi) in enumerate(chunks):
        parts = []
        for s in range(P):
            # rank s holds rows [all video in rank order, audio] of its heads
            parts.append(np.concatenate([per_rank[s][lo:hi], per_rank[s][n_video:]]))
        out.append(np.concatenate(parts, axis=1))
    return out


def gather_sequence(shards, n_video: int, P: int):
    """Gather after denoising: the video rows of every rank in order, then the
    audio rows (identical on every rank; rank 0's copy)."""
    chunks = video_chunks(n_video, P)
    video = [shards[r][:hi - lo] for r, (lo, hi) in enumerate(chunks)]
    return np.concatenate(video + [shards[0][chunks[0][1] - chunks[0][0]:]])


def ulysses_attention(q, ring_k, ring_v, length: int, head: int, k_u, v_u, n_video: int, P: int):
    """Attention of the unit's queries computed the Ulysses way over P ranks.
    q, k_u, v_u: [n_q][H][hd] bf16 bits (video rows first); ring_k/ring_v:
    [H][cap][hd] (the full ring; rank r uses its head range).  Returns O
    [n_q][H][hd] float64, gathered."""
    H = q.shape[1]
    qs, ks, vs = (shard_sequence(t, n_video, P) for t in (q, k_u, v_u))
    qh, kh, vh = (seq_to_head(t, n_video, P, H) for t in (qs, ks, vs))
    per_rank = []
    for r in range(P):
        h0, h1 = head_range(H, P, r)
        per_rank.append(attention(qh[r], ring_k[h0:h1], ring_v[h0:h1], length, head, kh[r], vh[r]))
    return gather_sequence(head_to_seq(per_rank, n_video, P, H), n_video, P)
