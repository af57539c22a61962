"""The seeded input generator: determinism, thread-count independence,
bf16 rounding and the tile-centroid value model."""
import numpy as np

import zebra_synth as zs


def test_bf16_round_to_nearest_even():
    # bf16 keeps 7 mantissa bits: the spacing just above 1 is 2^-7
    x = np.array([1.0, 1.0 + 2 ** -7, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8, -2.5, 0.0,
                  1.0 + 2 ** -8 + 2 ** -20], np.float32)
    b = zs.f32_to_bf16(x)
    back = zs.bf16_to_f32(b)
    # ties go to the even mantissa: 1 + 3*2^-8 -> 1 + 2^-6, 1 + 2^-8 -> 1
    assert back.tolist() == [1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -6, 1.0, -2.5, 0.0, 1.0 + 2 ** -7]


def test_deterministic_and_thread_independent():
    L = zs.CONFIGS["2views_16x16"]
    a = zs.stage_inputs(L, seed=0, threads=1)
    b = zs.stage_inputs(L, seed=0, threads=4)
    c = zs.stage_inputs(L, seed=1, threads=2)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and x.shape == (522, 1, 64)
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    s1 = zs.stage_inputs(L, seed=0, stage=1)
    assert not np.array_equal(a[1], s1[1])


def test_tile_centroid_model():
    L = zs.Layout(4, 5, 16, 16, heads=2)
    q, k, v = (zs.bf16_to_f32(x).astype(np.float64) for x in zs.stage_inputs(L, seed=3))
    tpf = L.tokens_per_frame
    # keys of one 8x8 block of one frame share a centroid: their spread is
    # the 0.5-scaled noise, much smaller than the spread across blocks
    blk = [5 + r * 16 + c for r in range(8) for c in range(8)]
    kk = k[blk, 0]
    assert kk.std(axis=0).mean() < 0.7
    assert np.abs(kk.mean(axis=0)).mean() > 0.3
    # queries of frame 1 follow the mean centroid of frames 0 and 2
    q1 = q[[tpf + x for x in blk], 0].mean(axis=0)
    kc = 0.75 * (kk.mean(axis=0) + k[[2 * tpf + x for x in blk], 0].mean(axis=0))
    assert np.corrcoef(q1, kc)[0, 1] > 0.95
    assert abs(v.mean()) < 0.05 and abs(v.std() - 1) < 0.05


def test_affine_and_rows():
    L = zs.CONFIGS["32views"]
    W, b = zs.affine_params(L, seed=0)
    assert W.shape == (16, 64, 64) and b.shape == (16, 64)
    assert np.abs(np.diagonal(W, axis1=1, axis2=2) - 1).max() < 0.05
    rows = zs.sample_rows(L, 2048, seed=0, special_frames=4)
    assert rows.shape == (2048, 2) and len({tuple(r) for r in rows}) == 2048
    tpf = L.tokens_per_frame
    spec = rows[(rows[:, 1] % tpf) < L.specials]
    assert len(spec) >= 4 * 5 * 16
    assert np.array_equal(rows, zs.sample_rows(L, 2048, seed=0, special_frames=4))


def test_device_generator_model_and_determinism():
    """The torch-drawn variant (used where every stage of a long schedule
    needs fresh inputs) follows the same tile-centroid model: keys of a block
    share a centroid, queries follow the neighbouring frames' centroids,
    specials and values are unit normal; it is deterministic per (seed,
    stage) and bf16-rounded."""
    import torch
    L = zs.Layout(4, 5, 16, 16, heads=2)
    q, k, v = zs.stage_inputs_device(L, seed=3, device="cpu")
    q2, _, _ = zs.stage_inputs_device(L, seed=3, device="cpu")
    q3, _, _ = zs.stage_inputs_device(L, seed=3, stage=1, device="cpu")
    assert q.dtype == torch.int16 and q.shape == (L.tokens, 2, 64)
    assert torch.equal(q, q2) and not torch.equal(q, q3)
    f = lambda t: zs.bf16_to_f32(t.numpy().view(np.uint16)).astype(np.float64)  # noqa: E731
    q, k, v = f(q), f(k), f(v)
    tpf = L.tokens_per_frame
    blk = [5 + r * 16 + c for r in range(8) for c in range(8)]
    kk = k[blk, 0]
    assert kk.std(axis=0).mean() < 0.7 and np.abs(kk.mean(axis=0)).mean() > 0.3
    q1 = q[[tpf + x for x in blk], 0].mean(axis=0)
    kc = 0.75 * (kk.mean(axis=0) + k[[2 * tpf + x for x in blk], 0].mean(axis=0))
    assert np.corrcoef(q1, kc)[0, 1] > 0.95
    assert abs(v.mean()) < 0.05 and abs(v.std() - 1) < 0.05
    spec = q[[f * tpf + s for f in range(4) for s in range(5)]]
    assert abs(spec.std() - 1) < 0.15
    mu = zs.calib_mean(L, seed=3, stage=2)
    assert mu.shape == (2, 64) and mu.dtype == np.float32 and np.abs(mu).max() < 0.06
