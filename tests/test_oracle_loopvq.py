"""Pins of oracle/loopvq.py (joint vector quantization across loop steps)."""
import numpy as np
import pytest

from oracle import loopvq as ov

torch = pytest.importorskip("torch")


def test_planted_codeword_fixes_the_joint_order():
    """Loop r's channels [4j, 4j+4) sit at positions [4r, 4r+4) of group j's
    joint vector: the codeword built that way is chosen, a decoy with the
    loops swapped is not, and decoding loop r returns loop r's channels."""
    R, T, D = 2, 1, 8
    x = np.zeros((R, T, D))
    x[0, 0] = [1, 2, 3, 4, 5, 6, 7, 8]
    x[1, 0] = [10, 20, 30, 40, 50, 60, 70, 80]
    cb = np.full((D // 4, 256, 4 * R), 1000.0)
    cb[0, 17] = [1, 2, 3, 4, 10, 20, 30, 40]         # group 0: loop 0 then loop 1
    cb[0, 5] = [10, 20, 30, 40, 1, 2, 3, 4]          # decoy: loops swapped
    cb[1, 200] = [5, 6, 7, 8, 50, 60, 70, 80]
    cb[1, 3] = [5, 6, 7, 8, 50, 60, 70, 81]          # one unit off
    idx = ov.encode(x, cb)
    assert idx.tolist() == [[17, 200]]
    assert ov.decode_loop(idx, cb, 0).tolist() == [[1, 2, 3, 4, 5, 6, 7, 8]]
    assert ov.decode_loop(idx, cb, 1).tolist() == [[10, 20, 30, 40, 50, 60, 70, 80]]


def test_codebook_holding_every_vector_is_lossless():
    rng = np.random.default_rng(3)
    R, T, D = 4, 40, 16
    x = rng.normal(size=(R, T, D)).astype(np.float16).astype(np.float64)
    jv = ov.joint_vectors(x)                           # [T][G][16]
    cb = rng.normal(10.0, 1.0, size=(D // 4, 256, 4 * R))
    cb[:, 100:100 + T, :] = jv.transpose(1, 0, 2)
    idx = ov.encode(x, cb)
    assert np.array_equal(idx, np.broadcast_to(100 + np.arange(T)[:, None], idx.shape))
    for r in range(R):
        assert np.array_equal(ov.decode_loop(idx, cb, r), x[r])


def test_ties_take_the_lowest_index_and_scaling_is_neutral():
    rng = np.random.default_rng(4)
    R, T, D = 2, 30, 8
    x = rng.normal(size=(R, T, D))
    cb = rng.normal(size=(D // 4, 256, 4 * R))
    cb[:, 201] = cb[:, 7]                              # duplicate codewords
    idx = ov.encode(x, cb)
    assert not np.any(idx == 201)
    assert np.array_equal(idx, ov.encode(2.0 * x, 2.0 * cb))
    d = ov.distances(x, cb)
    assert np.all(np.take_along_axis(d, idx[..., None], -1)[..., 0] <= d.min(-1))


def test_attend_matches_sdpa():
    rng = np.random.default_rng(5)
    T, D = 77, 16
    k = rng.normal(size=(T, D))
    v = rng.normal(size=(T, D))
    q = rng.normal(size=D)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=0.3)[0, 0, 0].numpy()
    assert np.allclose(ov.attend(q, k, v, 0.3), want, rtol=1e-12, atol=1e-12)
    assert np.array_equal(ov.attend(q, k[:0], v[:0]), np.zeros(D))
