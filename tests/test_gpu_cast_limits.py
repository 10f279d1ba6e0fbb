"""Col casts of a tall tensor: more than 65,535 tiles of 256 rows (the 2D
launch limit a one-workgroup-per-tile col cast would hit), with and without
the fused amax, alone and with the row copy from the same read.  The first
and last 4,096 rows of each copy are checked against the oracle's cast with
the same scale; the amax is exact.
"""
import numpy as np
import pytest
import torch

import precision_block_scaled_amd as P
from oracle import recipes as R
from tests.gpu_util import to_gpu_bf16, to_np_f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("both", [False, True])
@pytest.mark.parametrize("fused_amax", [False, True])
def test_col_cast_more_than_65535_row_tiles(fused_amax, both):
    rows, cols = 256 * 65537 + 16, 16               # 65,538 row tiles, the last one ragged
    rng = np.random.default_rng(99)
    x = (rng.integers(0x3000, 0x4700, (rows, cols), dtype=np.uint16)
         | (rng.integers(0, 2, (rows, cols), dtype=np.uint16) << 15))
    x[rows - 3, 5] = 0x4780                         # the maximum sits in the last tile
    s = np.float32(0.5)
    scale = torch.tensor([s], dtype=torch.float32, device="cuda")
    amax = torch.full((1,), -1.0, device="cuda") if fused_amax else None
    out = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    row = torch.empty((rows, cols), dtype=torch.uint8, device="cuda") if both else None
    rec = P.PBS_RECIPE_FP8_DELAYED if fused_amax else P.PBS_RECIPE_FP8_CURRENT
    mask = P.PBS_ROW | P.PBS_COL if both else P.PBS_COL
    P.pbs_cast(rec, to_gpu_bf16(x), rows, cols, P.PBS_FMT_E4M3, mask, 0, 0, 0, scale, amax, row, None, out,
               None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    got_row = row.cpu().numpy() if both else None
    for sl in (slice(0, 4096), slice(rows - 4096, rows)):
        want = R.cast_pertensor(x[sl], s, "e4m3", "col")
        bad = np.argwhere(got[:, sl] != want)
        assert len(bad) == 0, f"{len(bad)} codes differ in rows {sl}, first at {tuple(bad[0])}"
        if both:
            assert (got_row[sl] == want.T).all(), f"row copy differs in rows {sl}"
    if fused_amax:
        assert to_np_f32(amax)[0] == R.amax(x)
