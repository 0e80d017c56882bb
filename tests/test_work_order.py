"""The prefill's workgroup order (the XCD-aware, longest-tiles-first map from
a linear workgroup id to (sequence, q head, query tile)) is a bijection of
[0, batch * hq * ntiles) for every shape: no tile is run twice or skipped.
The map is restated here from the kernel's description: ids are dealt to
the 8 XCDs round robin; with kv heads a multiple of 8, XCD x takes the kv
heads congruent to x mod 8 and runs its share in blocks of tblk tiles (the
tiles with the most keys first), stream by stream, the q heads of one kv head
side by side; otherwise tiles with the most keys go first over all
(sequence, head) pairs."""
import pytest


def work_item(batch, hq, hkv, tblk, ntiles, lin):
    if hkv % 8 == 0:
        grp = hq // hkv
        xcd, j = lin & 7, lin >> 3
        nstream = batch * (hkv >> 3)
        tb = max(1, min(tblk, ntiles))
        blk = j // (nstream * tb * grp)
        t0 = blk * tb
        tl = min(tb, ntiles - t0)
        r = j - blk * (nstream * tb * grp)
        st, r2 = divmod(r, tl * grp)
        t = r2 // grp
        b = st % batch
        h = (xcd + 8 * (st // batch)) * grp + (r2 - t * grp)
        return b, h, t0 + t
    nbh = batch * hq
    bh = lin % nbh
    return bh // hq, bh % hq, lin // nbh


@pytest.mark.parametrize("batch,hq,hkv", [(1, 8, 8), (3, 32, 8), (8, 32, 8), (2, 64, 16), (5, 16, 16),
                                          (4, 12, 4), (1, 2, 2), (7, 6, 3)])
@pytest.mark.parametrize("ntiles", [1, 2, 3, 7, 33])
@pytest.mark.parametrize("per_cu", [1, 2, 3, 4])
def test_prefill_work_order_is_a_bijection(batch, hq, hkv, ntiles, per_cu):
    # the launcher's choice: the workgroups resident on one XCD (32 CUs times
    # the kernel's occupancy) divided by the group size
    tblk = max(1, 32 * per_cu // (hq // hkv))
    n = batch * hq * ntiles
    seen = set()
    for lin in range(n):
        b, h, ty = work_item(batch, hq, hkv, tblk, ntiles, lin)
        assert 0 <= b < batch and 0 <= h < hq and 0 <= ty < ntiles
        seen.add((b, h, ty))
    assert len(seen) == n


def test_longest_tiles_start_first_on_each_xcd():
    # 8 kv heads: along each XCD's own order of ids the block of tiles (tile
    # index counted from the sequence end, divided by the block size) never
    # decreases, so the tiles with the most keys are dealt first
    batch, hq, hkv, ntiles = 3, 32, 8, 9
    tblk = 96 // (hq // hkv)
    for xcd in range(8):
        blocks = [work_item(batch, hq, hkv, tblk, ntiles, lin)[2] // tblk
                  for lin in range(xcd, batch * hq * ntiles, 8)]
        assert all(blocks[i] <= blocks[i + 1] for i in range(len(blocks) - 1))
