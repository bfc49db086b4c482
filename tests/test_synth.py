"""The seeded input generator (CPU only)."""
import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library for Philox4x32-10.
    assert synth.philox4x32_10([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert synth.philox4x32_10([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6,
                                                                       0x6D5451FD]
    assert synth.philox4x32_10([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_normals_moments():
    z = synth.normals(7, 1, 100_000)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 1) < 0.02
    assert abs(np.mean(z ** 4) - 3) < 0.1


def test_rows_are_index_addressable_and_deterministic():
    w = synth.WORKLOADS["c2"].scaled(N=5000)
    full = synth.points(w)
    parts = np.concatenate([synth.points(w, 0, 1234), synth.points(w, 1234, 3766)])
    assert np.array_equal(full, parts)
    assert np.array_equal(full, synth.points(w))
    single = synth.points(w, 4321, 1)
    assert np.array_equal(single[0], full[4321])


def test_mixture_shapes():
    w = synth.WORKLOADS["c1"]
    X, comp = synth.points(w, with_components=True)
    assert X.dtype == np.float32 and X.shape == (16384, 32)
    cen = synth.centers(w)
    resid = X - cen[comp]
    assert abs(resid.std() - 1.0) < 0.02          # sigma = 1
    assert abs(cen.std() - 2.0) < 0.15            # centres ~ N(0, 4I)
    counts = np.bincount(comp, minlength=64)
    assert counts.min() > 150 and counts.max() < 370  # equal weights: 256 each on average
    w3 = synth.WORKLOADS["c3"].scaled(N=4000)
    X3 = synth.bf16_bits_to_f32(synth.points(w3)).astype(np.float64)
    assert np.allclose(np.linalg.norm(X3, axis=1), 1.0, atol=1e-2)  # unit vectors (bf16 rounding)


def test_zipf_weights():
    w = synth.WORKLOADS["c4"].scaled(N=200_000)
    _, comp = synth.points(w, with_components=True)
    cdf = synth.zipf_cdf(4096, 1.2)
    assert abs(cdf[0] - 0.215) < 0.002            # top component holds ~21.5% of the mass
    frac0 = np.mean(comp == 0)
    assert abs(frac0 - cdf[0]) < 0.005


def test_sample_indices():
    idx = synth.sample_indices(9, 1000, 300)
    assert len(set(idx.tolist())) == 300 and idx.min() >= 0 and idx.max() < 1000
    assert np.array_equal(idx, synth.sample_indices(9, 1000, 300))
    full = synth.sample_indices(3, 50, 50)
    assert sorted(full.tolist()) == list(range(50))


def test_init_centroids_are_data_rows():
    w = synth.WORKLOADS["c2"].scaled(N=3000, K=40)
    X = synth.points(w)
    C0 = synth.init_centroids(w, X)
    idx = synth.init_indices(w)
    assert np.array_equal(C0, synth.bf16_bits_to_f32(X[idx]))
    assert np.array_equal(C0, synth.init_centroids(w))  # regenerated row by row
