"""Input generators: determinism, shapes, densities, token-order properties."""

import numpy as np
import torch

import synth


def test_tiny_workload_recipe():
    w = synth.make_workload("tiny")
    assert w.q.shape == (1, 1024, 64) and w.q.dtype == torch.bfloat16
    assert w.mask.shape == (1, 16, 16)
    assert int(w.mask[0, 7].sum()) == 0
    diag = torch.diagonal(w.mask[0])
    assert int(diag.sum()) == 15          # all but the fully masked block 7
    assert 0.4 < float(w.mask.float().mean()) < 0.65
    w2 = synth.make_workload("tiny")
    assert torch.equal(w.q, w2.q) and torch.equal(w.mask, w2.mask) and torch.equal(w.x0, w2.x0)
    assert float(w.x0.min()) >= -1.0 and float(w.x0.max()) < 1.0


def test_layer16k_density_and_padding():
    w = synth.make_workload("layer16k", heads=3)
    assert w.q.shape == (3, 16384, 128)
    dens = float(w.mask.float().mean())
    assert 0.17 < dens < 0.23
    nnz = w.mask.sum(-1)
    assert int(nnz.min()) >= 9 and int(nnz.max()) > 2 * int(nnz.min())
    assert torch.all(torch.diagonal(w.mask, dim1=1, dim2=2) == 1)


def test_wan_shape_padding_and_topk():
    w = synth.make_workload("wan75k", heads=2)
    assert w.seq_len == 75600 and w.q.shape == (2, 75648, 128)
    assert torch.all(w.q[:, 75600:] == 0) and torch.all(w.v[:, 75600:] == 0)
    nb = 591
    assert w.mask.shape == (2, nb, nb)
    for h in range(2):
        nnz = w.mask[h].sum(-1)
        assert torch.all(torch.diagonal(w.mask[h]) == 1)
        # k per head in [30, 147], plus the diagonal when it is not among the top k
        assert 30 <= int(nnz.min()) and int(nnz.max()) <= 148
        assert int(nnz.max()) - int(nnz.min()) <= 1


def test_video_hilbert_order_is_a_local_bijection():
    """The curve runs over the whole (t, y, x) box: a bijection whose steps join face
    neighbours almost everywhere (odd side lengths force a few diagonal steps of two
    cells), and whose 128-token blocks are compact in all three axes, not planar."""
    o = synth.video_hilbert_order(33, 45, 80)
    assert np.array_equal(np.sort(o), np.arange(33 * 45 * 80))
    t, y, x = o // 3600, (o % 3600) // 80, o % 80
    dt, dy, dx = np.abs(np.diff(t)), np.abs(np.diff(y)), np.abs(np.diff(x))
    step = dt + dy + dx
    assert step.max() <= 2 and max(dt.max(), dy.max(), dx.max()) <= 2
    assert (step == 1).mean() >= 0.9
    assert o[0] == 0                        # the curve enters at the origin corner
    ext = np.array([[np.ptp(a[i:i + 128]) + 1 for a in (t, y, x)]
                    for i in range(0, o.size - 127, 128)])
    assert ext[:, 0].mean() > 3             # blocks span several frames ...
    assert ext.max() <= 16                  # ... and stay compact in space and time
    for dims in ((80, 45, 33), (7, 5, 3), (1, 9, 4), (12, 1, 1), (2, 2, 2), (16, 16, 16)):
        cells = synth.gilbert3d(*dims)
        assert len(set(cells)) == len(cells) == dims[0] * dims[1] * dims[2]
        assert all(0 <= c[i] < dims[i] for c in cells for i in range(3))
    # power-of-two cubes and flat boxes: every step is a unit step, as in Hilbert's curve
    for dims in ((8, 8, 8), (80, 45, 1), (2, 2, 1), (4, 4, 4)):
        c = np.array(synth.gilbert3d(*dims))
        if dims == (8, 8, 8) or dims == (4, 4, 4):
            assert np.abs(np.diff(c, axis=0)).sum(1).max() <= 2
        else:
            assert np.all(np.abs(np.diff(c, axis=0)).sum(1) == 1)
    for w_, h_ in ((80, 45), (7, 5), (1, 9), (12, 1)):
        cells = synth.gilbert2d(w_, h_)
        assert len(set(cells)) == w_ * h_
        assert np.all(np.abs(np.diff(np.array(cells), axis=0)).sum(1) == 1)


def test_random_tiny_case():
    w = synth.random_tiny_case(3, heads=2, seq_len=300, block=64, empty_rows=(1,))
    assert w.q.shape == (2, 320, 64)
    assert int(w.mask[:, 1].sum()) == 0
    assert torch.all(w.q[:, 300:] == 0)


def test_random_mask_density_and_diagonal():
    w = synth.make_workload("random20", heads=2, grid=(3, 45, 80))
    m = w.mask
    nb = m.shape[1]
    assert torch.all(torch.diagonal(m, dim1=1, dim2=2) == 1)
    dens = m.float().mean().item()
    assert abs(dens - (0.2 + 0.8 / nb)) < 0.03, dens


def test_long_wan_geometry():
    # 401 frames at 720x1280: (401 - 1) / 4 + 1 = 101 latent frames, and 720 / 16 by
    # 1280 / 16 = 45 x 80 tokens per frame (8x spatial compression, 2x2 patches)
    cfg = synth.get_config("wan364k")
    assert cfg.seq_len == 363600 and cfg.num_blocks == 2841 and cfg.padded_len == 363648
    assert cfg.heads == 40 and cfg.head_dim == 128 and cfg.mask == "topk"


def test_wide_range_case_spans_the_softmax_bounds():
    """The wide-range inputs do what their GPU test needs: some query row's block
    maximum rises by more than 2^32 (32 log2 units) over an earlier block of its list,
    and some kept block lies more than 96 log2 units below its row's final maximum."""
    import math

    import numpy as np

    w = synth.wide_range_case(7, heads=2, seq_len=1000, head_dim=128, block=128)
    q = w.q.float().numpy().astype(np.float64)
    k = w.k.float().numpy().astype(np.float64)
    m = w.mask.numpy()
    H, mb, b, L = m.shape[0], m.shape[1], w.block, w.seq_len
    l2 = w.scale / math.log(2.0)
    rise = below = 0.0
    for h in range(H):
        s = q[h, :L] @ k[h, :L].T * l2
        for u in range(mb):
            rows = s[u * b:min(L, (u + 1) * b)]
            cols = np.nonzero(m[h, u])[0]
            if len(cols) < 2:
                continue
            bmax = np.stack([rows[:, v * b:min(L, (v + 1) * b)].max(axis=1) for v in cols], 1)
            run = np.maximum.accumulate(bmax, axis=1)
            rise = max(rise, float((bmax[:, 1:] - run[:, :-1]).max()))
            below = max(below, float((run[:, -1:] - bmax).max()))
    assert rise > 32.0
    assert below > 96.0
