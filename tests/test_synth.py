"""CPU checks of the seeded input generator (moe_synth): reproducibility,
independence of the tensors' streams, the f16 rounding of block scales and
offsets, the block byte layout, and the moments of every distribution."""
import numpy as np
import pytest
import torch

import moe_synth as S


def test_seeds_reproduce_and_separate():
    wl = S.WORKLOADS["tiny"]
    a, b = S.make_layer(wl, layer=0), S.make_layer(wl, layer=0)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    c = S.make_layer(wl, layer=1)
    assert not torch.equal(a["router_w"], c["router_w"])
    assert not torch.equal(a["gate_exps"], a["up_exps"])  # distinct tensor names draw distinct streams
    assert torch.equal(S.make_x(wl, 3, layer=2, step=1), S.make_x(wl, 3, layer=2, step=1))
    assert not torch.equal(S.make_x(wl, 3, layer=2, step=1), S.make_x(wl, 3, layer=2, step=2))
    # the seed hash depends on every part of its key
    keys = {S.seed_for(m, w, l, t) for m in (0, 1) for w in ("a", "b") for l in (0, 1) for t in ("x", "y")}
    assert len(keys) == 16


@pytest.mark.parametrize("qt", [S.Q4_0, S.Q4_1, S.Q8_0])
def test_block_scales_are_f16_round_to_nearest_even(qt):
    # redraw the uniform f32 values from the same generator stream and round them with numpy (IEEE
    # round-to-nearest-even): the stored f16 bits must be exactly those
    n, seed, lo, hi = 4096, 1234, 0.001, 0.02
    blocks = S.q4_blocks(n, qt, "cpu", seed, lo, hi).numpy()
    g = torch.Generator().manual_seed(seed)
    d32 = (torch.rand(n, generator=g) * (hi - lo) + lo).numpy()
    assert np.array_equal(blocks[:, 0:2].copy().view(np.uint16).ravel(), d32.astype(np.float16).view(np.uint16))
    if qt == S.Q4_1:
        m32 = (torch.rand(n, generator=g) * (hi - lo) + lo).numpy()
        assert np.array_equal(blocks[:, 2:4].copy().view(np.uint16).ravel(),
                              m32.astype(np.float16).view(np.uint16))
    assert blocks.shape == (n, S.BLOCK_BYTES[qt])


def test_distribution_moments():
    n = 1 << 16
    b = S.q4_blocks(n, S.Q4_1, "cpu", 7, 0.001, 0.02).numpy()
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    m = b[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    for v in (d, m):
        assert v.min() >= 0.001 - 1e-6 and v.max() <= 0.02 + 1e-5
        assert abs(v.mean() - 0.0105) < 2e-4            # U(0.001, 0.02): mean 0.0105
        assert abs(v.std() - 0.019 / 12 ** 0.5) < 2e-4  # sd 0.00548
    nib = b[:, 4:].ravel()
    lo, hi = nib & 15, nib >> 4
    for q in (lo, hi):
        freq = np.bincount(q, minlength=16) / q.size
        assert np.abs(freq - 1 / 16).max() < 0.003
    wl = S.WORKLOADS["flint"]
    x = S.make_x(wl, 64).numpy().ravel()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    r = S.normal((256, 2048), 0.05, "cpu", 11).numpy().ravel()
    assert abs(r.mean()) < 1e-3 and abs(r.std() - 0.05) < 5e-4


def test_wide_variants():
    # signed scales and offsets, f16-subnormal scales, and +-30 input outliers, at their stated rates
    wl = S.Workload("w", 256, 8, 2, 64, 32, S.Q4_1, signed_scales=True, subnormal_frac=0.1, x_outlier_frac=0.02)
    b = S.make_layer(wl, 0)["gate_exps"].reshape(-1, 20).numpy()
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    m = b[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert 0.45 < (d < 0).mean() < 0.55 and 0.45 < (m < 0).mean() < 0.55
    sub = np.abs(d) < 2.0 ** -14
    assert 0.08 < sub.mean() < 0.12 and np.all(d[sub] != 0)
    x = S.make_x(wl, 64).numpy()
    out = np.abs(x) == 30.0
    assert 0.015 < out.mean() < 0.025
    assert np.array_equal(x[~out], S.make_x(S.Workload("w", 256, 8, 2, 64, 32), 64).numpy()[~out])


def test_centred_offsets():
    # centred Q4_1 blocks: m = -c d with c ~ U(7, 8), rounded to f16, so the block's values straddle zero;
    # d keeps its U(lo, hi) draw and the nibbles their uniform bytes (the same stream as without centring)
    n = 1 << 14
    b = S.q4_blocks(n, S.Q4_1, "cpu", 5, 0.001, 0.02, centred=True).numpy()
    plain = S.q4_blocks(n, S.Q4_1, "cpu", 5, 0.001, 0.02).numpy()
    assert np.array_equal(b[:, 0:2], plain[:, 0:2]) and np.array_equal(b[:, 4:], plain[:, 4:])
    d = b[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    m = b[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    c = -m / d
    assert c.min() >= 7.0 - 1e-2 and c.max() <= 8.0 + 1e-2
    assert abs(c.mean() - 7.5) < 0.02
    # the mean weight of a block, d * 7.5 + m, is centred on zero
    assert abs((d * 7.5 + m).mean()) < 2e-4
    # Q4_0 and Q8_0 blocks carry no offset: centring leaves them as they are
    for qt in (S.Q4_0, S.Q8_0):
        assert np.array_equal(S.q4_blocks(256, qt, "cpu", 5, centred=True).numpy(),
                              S.q4_blocks(256, qt, "cpu", 5).numpy())
