"""The host replay of the balanced schedule covers every tile exactly once (CPU)."""

import pytest

from gpu_helpers import balanced_pieces


@pytest.mark.parametrize("ctx,stok,Hkv,G", [
    ((37, 100), 0, 1, 512), ((0, 5, 64, 65), 0, 2, 7), ((4000, 0, 1, 33), 4, 8, 512),
    ((131072, 40211), 0, 8, 512), ((0, 0), 3, 2, 5), ((1,), 0, 1, 1),
])
def test_pieces_tile_the_space_once(ctx, stok, Hkv, G):
    pieces = balanced_pieces(ctx, stok, Hkv, G)
    seen = {}
    for g, b, hk, j, seg, whole in pieces:
        assert seg >= 1
        for t in range(j, j + seg):
            key = (b, hk, t)
            assert key not in seen
            seen[key] = g
    want = {(b, hk, t) for b, c in enumerate(ctx) for hk in range(Hkv)
            for t in range(-(-(c + stok) // 32))}
    assert set(seen) == want
    # Slots b*Hkv + hk + g of partial pieces never collide.
    slots = [b * Hkv + hk + g for g, b, hk, j, seg, whole in pieces if not whole]
    assert len(slots) == len(set(slots))
    assert all(0 <= s < len(ctx) * Hkv + G for s in slots)
