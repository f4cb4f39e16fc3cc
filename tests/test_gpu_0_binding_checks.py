"""The Python binding refuses caller-supplied buffers of the wrong shape, and
vbs of the wrong length, before any call into the library: the C ABI writes
the full output extent, so a short buffer would be written past its end."""
import pytest
import torch

import video_dit_block_amd as vsa

pytestmark = pytest.mark.gpu


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device="cuda")


def _i(*shape):
    return torch.zeros(shape, dtype=torch.int32, device="cuda")


def test_short_buffers_are_refused():
    T, H, W, NH, D = 5, 6, 7, 2, 64          # 8 cubes, 512 tiled rows
    x = _bf(1, T * H * W, NH, D)
    with pytest.raises(ValueError, match="out"):
        vsa.tile(x, T, H, W, out=_bf(1, 511, NH, D))
    with pytest.raises(ValueError, match="vbs"):
        vsa.tile(x, T, H, W, vbs=_i(7))
    qt = _bf(1, 512, NH, D)
    with pytest.raises(ValueError, match="out"):
        vsa.untile(qt, T, H, W, out=_bf(1, T * H * W - 1, NH, D))
    with pytest.raises(ValueError, match="vbs"):
        vsa.select(qt, qt, _i(7), 3)
    with pytest.raises(ValueError, match="out"):
        vsa.select(qt, qt, _i(8), 3, out=_i(1, NH, 8, 2))
    with pytest.raises(ValueError, match="out"):
        vsa.select_noalloc(qt, qt, _i(8), 3, out=_i(1, NH, 7, 3))
    with pytest.raises(ValueError, match="vbs"):
        vsa.select_cdf(qt, qt, _i(9), 3, 0.9)
    with pytest.raises(ValueError, match="out"):
        vsa.fwd(qt, qt, qt, _i(1, NH, 8, 3), _i(8), out=_bf(1, 448, NH, D))
    with pytest.raises(ValueError, match="vbs"):
        vsa.coarse(qt, qt, qt, _i(4))
    torch.cuda.synchronize()
