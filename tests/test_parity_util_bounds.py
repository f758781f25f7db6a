"""The end-to-end bound of the GPU parity tests (parity_util.decoder_bound) bounds what a
latent difference becomes in the restored, rotated K|V (review page section 2.5: the
decoder is linear; section 2.1: RoPE rotates key pairs (j, j + D/2))."""

import numpy as np

from oracle import OracleCodec
from oracle.codec import linear_decoder, rope_rotate
from parity_util import decoder_bound
from synth import codec_weights


def test_decoder_bound_holds_and_is_reached_per_pair():
    N, D, d_c = 3, 16, 32
    W = codec_weights(2 * N * D, 64, d_c, np.random.default_rng(3), "f32")
    codec = OracleCodec(N, D, 64, d_c, 4, 4, 32, "f32", 1e4, W)
    rng = np.random.default_rng(4)
    dz = rng.standard_normal((200, d_c)) * np.exp(rng.uniform(-8, 0, (200, 1)))
    pos = rng.integers(0, 100000, 200)
    diff = linear_decoder(dz, W["Wd"])
    diff[:, : codec.dk] = rope_rotate(diff[:, : codec.dk], pos, N, D, 1e4)
    b = decoder_bound(codec, dz)
    assert np.all(np.abs(diff) <= b * (1 + 1e-12))
    # at position 0 (no rotation) a one-hot latent difference reaches |W_d| on the V half
    e = np.zeros((1, d_c))
    e[0, 5] = 2.0
    np.testing.assert_allclose(decoder_bound(codec, e)[0, codec.dk:], 2 * np.abs(W["Wd"][5, codec.dk:]))
