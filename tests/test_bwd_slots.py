"""The backward's workspace slots of band key tiles (no GPU).

The tiled backward of the window + global pattern gives every (query tile,
band key tile) pair a workspace slot for its dK/dV share; the reduce kernel
sums a key tile's slots. The tile sets below are the kernels' own integer
arithmetic (64-row query tiles over the last Nq positions of a request of L
keys, a query tile's band from the key tile of its first row's window start
to the key tile of its last row, global tiles excluded); a slot index that
two query tiles of one key tile share would make one share replace the
other. The slot count per band key tile is window // 64 + 3.
"""


def _tiles_seen(L, Nq, window, n_global):
    """{band key tile: [query tiles that see it]} as the tile kernel visits them."""
    pbase = L - Nq
    ntiles_all = (L + 63) // 64
    gt = (min(n_global, L) + 63) // 64
    seen = {}
    for qt in range((Nq + 63) // 64):
        q0 = qt * 64
        nrows = min(64, Nq - q0)
        first, last = pbase + q0, pbase + q0 + nrows - 1
        last_tile = min(ntiles_all - 1, last // 64)
        wt = max(0, first - window + 1) // 64
        for t in range(max(gt, wt), last_tile + 1):
            seen.setdefault(t, []).append(qt)
    return seen


def _collides(seen, key):
    return any(len({key(qt, t) for qt in qts}) != len(qts) for t, qts in seen.items())


def test_query_tile_residue_never_collides():
    for window in list(range(1, 200, 3)) + [255, 256, 257, 511, 512, 513, 1000]:
        nslot = window // 64 + 3
        for ctx in (100, 320, 700):
            for L in range(1, ctx + 1, 13):
                for Nq in sorted({1, 33, 64, 65, 96, 128, L}):
                    if Nq > L:
                        continue
                    for n_global in (0, 3, 64):
                        seen = _tiles_seen(L, Nq, window, n_global)
                        assert all(len(q) <= nslot for q in seen.values()), (window, L, Nq)
                        assert not _collides(seen, lambda qt, t: qt % nslot), (window, L, Nq, n_global)


def test_distance_from_last_tile_collides_on_a_short_last_query_tile():
    # requests of 300 keys, 96 query rows, window 20: rows 204..267 and
    # 268..299 both end in key tile 4, so "last tile - t" names one slot twice
    seen = _tiles_seen(300, 96, 20, 3)
    pbase, ntiles_all = 300 - 96, (300 + 63) // 64

    def last_tile(qt):
        nrows = min(64, 96 - 64 * qt)
        return min(ntiles_all - 1, (pbase + 64 * qt + nrows - 1) // 64)

    assert last_tile(0) == last_tile(1) == 4
    assert _collides(seen, lambda qt, t: last_tile(qt) - t)
    assert not _collides(seen, lambda qt, t: qt % (20 // 64 + 3))
