"""Python mirror of the paged decode's split plan and workspace layout, written from the
library's documented interface (include/mla_decode.h: mla_plan_paged,
mla_paged_workspace_bytes, mla_paged_decode_partials), for bit-exact checks of the
integer work the decode launch does on the device.  Test infrastructure only.

The plan: request b holds tiles(b) = ceil(n_b / T) tiles of T tokens (T = 64 for the FP8
cache formats, 32 for the others; with a sliding window, counted from the tile holding its
first visible token) and costs tiles(b) + C when it has any, C = 8 for T = 64 and 10 for
T = 32 (the segment overhead in tiles).  On the cost axis each request is its C-unit overhead
part followed by its tiles; range w of the NS ranges covers the cost interval
[w W / NS, (w + 1) W / NS) of the total cost W and takes the tiles that fall in it.  A
range that covers parts of several requests runs one segment per request; segment
(w, b) writes partial slot w + b.  seg_first[b] and seg_last[b] are the first and last
range that touch request b, and info[0] = W.

Workspace: o_part [slots][rows][512] fp32, lse_part [slots][rows] fp32, seg_first [B],
seg_last [B] int32, info [64] int32, each section starting on a 256-byte boundary, with
slots = NS + B - 1 and rows = q_len * H.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TILE = 32
SEGMENT_COST = {32: 10, 64: 8}  # per-segment overhead in tiles, by tile size


def tile_tokens(fmt: int) -> int:
    """Tokens per tile of a cache format: 64 for FP8 (formats 1 and 3), else 32."""
    return 64 if fmt in (1, 3) else 32


def segment_cost(tile: int) -> int:
    return SEGMENT_COST[tile]


def _round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def workspace_layout(B: int, q_len: int, H: int, num_splits: int) -> dict:
    rows = q_len * H
    slots = num_splits + B - 1
    o_off = 0
    lse_off = _round_up(slots * rows * 512 * 4, 256)
    first_off = lse_off + _round_up(slots * rows * 4, 256)
    last_off = first_off + _round_up(B * 4, 256)
    info_off = last_off + _round_up(B * 4, 256)
    return dict(rows=rows, slots=slots, o_off=o_off, lse_off=lse_off, first_off=first_off, last_off=last_off,
                info_off=info_off, total=info_off + 256)


@dataclass
class Segment:
    w: int        # range
    b: int        # request
    slot: int     # w + b
    t0: int       # first token (request-relative)
    t1: int       # one past the last token, clipped to the request's length


def plan(seq_lens, max_len: int, num_splits: int, q_len: int = 1, window: int = 0, tile: int = TILE):
    """Returns (segments, seg_first, seg_last, W): the segments in range order, the
    first / last range per request (-1 where the request has no tiles), and the total
    cost."""
    n = [min(max(int(x), 0), max_len) for x in seq_lens]
    B = len(n)
    sc = segment_cost(tile)

    def first_tile(nb):
        return max(nb - q_len - window + 1, 0) // tile if window > 0 else 0

    tiles = [(-(-nb // tile)) - first_tile(nb) if nb > 0 else 0 for nb in n]
    cost = [t + sc if t > 0 else 0 for t in tiles]
    W = sum(cost)
    T = sum(tiles)
    cstart = np.concatenate([[0], np.cumsum(cost)]).astype(np.int64)
    tstart = np.concatenate([[0], np.cumsum(tiles)]).astype(np.int64)

    def locate(c):
        # the request whose cost span holds c, its first tile, and the tile c maps to
        for b in range(B):
            if cost[b] and c < cstart[b] + cost[b]:
                return b, int(tstart[b]), int(tstart[b] + max(c - cstart[b] - sc, 0))
        raise AssertionError("cost position past the batch")

    segs = []
    seg_first = [-1] * B
    seg_last = [-1] * B
    if W == 0:
        return segs, seg_first, seg_last, W
    for w in range(num_splits):
        lo = (w * W) // num_splits
        hi = ((w + 1) * W) // num_splits
        b, base, t0 = locate(lo)
        t1 = T if hi >= W else locate(hi)[2]
        t = t0
        while t < t1:
            nb = tiles[b]
            if base + nb <= t:
                base += nb
                b += 1
                continue
            seg_end = min(t1, base + nb)
            tf = first_tile(n[b])
            segs.append(Segment(w, b, w + b, (t - base + tf) * tile, min((seg_end - base + tf) * tile, n[b])))
            if t == base:
                seg_first[b] = w
            if seg_end == base + nb:
                seg_last[b] = w
            t = seg_end
            base += nb
            b += 1
    return segs, seg_first, seg_last, W
