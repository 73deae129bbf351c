"""GPU map parity: the task -> tile map computed by the kernels' own device
scheduler (bst_tile_map / bst_grouped_tile_map) must equal the oracle's map
bit for bit, for every direction, offset, tile, remap and grid."""
import itertools

import numpy as np
import pytest

from gpu_util import say, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # (batch, M, N, tile)
    (1, 200, 136, (64, 64)),          # tails workload
    (1, 1024, 1024, (256, 128)),      # fp16 2k workload
    (1, 1024, 2048, (256, 256)),      # mxfp8 workload (fp8 tile)
    (16, 512, 768, (128, 192)),       # bf16 batch workload
    (3, 1000, 700, (128, 128)),
    (1, 1, 1, (64, 64)),
    (2, 4097, 63, (128, 256)),
]


def _ab(tile):
    return 5 if tile == (256, 256) else 1     # int8 has the 256x256 tile


@pytest.mark.parametrize("batch,M,N,tile", CASES)
def test_map_matches_oracle(orc, batch, M, N, tile):
    import block_swizzle_tile_amd as bst
    for off, d, remap, grid in itertools.product([1, 2, 3, 4, 8, 1000], ["zn", "nz", "raster"],
                                                 [0, 1], [0, 7]):
        say("map", batch, M, N, tile, off, d, remap, grid)
        s = bst.make_sched(tile=tile, offset=off, direction=d, xcd_remap=remap, grid=grid)
        got = bst.tile_map(batch, M, N, s, ab=_ab(tile)).cpu().numpy()
        want = orc.tile_map(batch, M, N, tile[0], tile[1], off, d)
        assert np.array_equal(got[:, :5].astype(np.uint32), want), (off, d, remap, grid)
        assert np.all(got[:, 5] == 0)
        assert np.all((got[:, 6] >= 0) & (got[:, 6] < 8))


def test_remap_places_contiguous_tasks_on_one_xcd(orc):
    """With the renumbering on, the tasks each XCD runs form one contiguous
    range of task indices (checked through the XCC id each workgroup reports).

    The renumbering rests on the hardware dealing workgroups out to the 8
    XCDs round-robin (workgroup w on XCD w mod 8), which is checked first
    with the renumbering off; if the device places workgroups otherwise the
    premise does not hold and the test is skipped with that reason."""
    import block_swizzle_tile_amd as bst
    base = dict(tile=(128, 128), offset=2, direction="zn", grid=256)
    hw = bst.tile_map(1, 2048, 2048, bst.make_sched(xcd_remap=0, **base)).cpu().numpy()
    assert sorted(hw[:, 7].tolist()) == list(range(256))     # one task per workgroup
    if not np.array_equal(hw[:, 6], hw[:, 7] % 8):
        pytest.skip("workgroups are not dealt out to XCDs round-robin on this device: %s"
                    % hw[:16, 6].tolist())
    got = bst.tile_map(1, 2048, 2048, bst.make_sched(xcd_remap=1, **base)).cpu().numpy()
    wg, xcc = got[:, 7], got[:, 6]
    assert sorted(wg.tolist()) == list(range(256))
    say("xcc per task", xcc.tolist())
    # every XCD runs 32 tasks, and its tasks are consecutive: along the task
    # order the XCC id changes exactly 7 times, in increasing order
    assert np.all(np.bincount(xcc, minlength=8) == 32)
    changes = np.flatnonzero(np.diff(xcc) != 0)
    assert changes.size == 7, changes
    assert np.all(np.diff(xcc[np.concatenate([[0], changes + 1])]) > 0)
    # and the renumbering itself: logical index l of XCD x = x * 32 + w // 8
    assert np.array_equal(np.arange(256), (wg % 8) * 32 + wg // 8)


@pytest.mark.parametrize("tile", [(64, 64), (128, 128), (256, 256)])
@pytest.mark.parametrize("d", ["zn", "nz", "raster"])
def test_grouped_map_matches_oracle(orc, tile, d):
    import block_swizzle_tile_amd as bst
    from block_swizzle_tile_amd import inputs
    for gm in [inputs.group_sizes(), np.array([0, 300, 5, 0, 129, 64, 1], np.int32),
               np.array([0], np.int32), np.array([7], np.int32)]:
        N = 4096 if gm.sum() == 8192 else 200
        for off in [1, 3]:
            say("grouped map", tile, d, gm.tolist(), off)
            s = bst.make_sched(tile=tile, offset=off, direction=d)
            got = bst.grouped_tile_map(to_gpu(gm, "i32"), int(gm.sum()), N, s).cpu().numpy()
            want = orc.grouped_tile_map(gm, N, tile[0], tile[1], off, d)
            T = want.shape[0]
            assert np.array_equal(got[:T, :6].astype(np.uint32), want)
            assert np.all(got[T:] == -1)
