"""The stored oracle outputs in tests/golden/fullsize_oracle.npz and vae_oracle.npz:
present, finite, of the shapes their workloads give, and tied to the current input
recipe by the checksums that the scripts beside them record (a change to the seeded input generators
or to a workload's recipe fails here, on the CPU, before a GPU run compares against stale
values)."""
import importlib.util
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _mkg():
    spec = importlib.util.spec_from_file_location("mkg", os.path.join(HERE, "golden", "make_fullsize_golden.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_stored_full_size_outputs_match_their_input_recipes():
    mkg = _mkg()
    g = np.load(os.path.join(HERE, "golden", "fullsize_oracle.npz"))
    cases = {
        "d1536": (mkg.cd_inputs(192, 192), (2, 4, 192, 192)),
        "c1024_mx": (mkg.cd_inputs(128, 128), (2, 4, 128, 128)),
        "c1024_mx_ulp": (mkg.ulp_up(mkg.cd_inputs(128, 128)), (2, 4, 128, 128)),
        "e1024_b8": (mkg.e_inputs(), (len(mkg.E_SAMPLES), 4, 128, 128)),
    }
    for name, (inputs, shape) in cases.items():
        assert name in g.files, name
        a = g[name]
        assert a.shape == shape and a.dtype == np.float32 and np.isfinite(a).all(), name
        np.testing.assert_array_equal(g[name + "_checksum"], mkg.checksum(*inputs), err_msg=name)


def test_ulp_twin_differs_from_its_base_by_one_ulp_in_the_latents_only():
    mkg = _mkg()
    lat, taus, text, mask = mkg.cd_inputs(128, 128)
    lat2, taus2, text2, mask2 = mkg.ulp_up((lat, taus, text, mask))
    assert (lat2 > lat).all()
    np.testing.assert_array_equal(lat2, np.nextafter(lat, np.float32(np.inf)))
    assert taus2 is taus and text2 is text and mask2 is mask


def test_stored_vae_decode_matches_its_latent():
    spec = importlib.util.spec_from_file_location("mkv", os.path.join(HERE, "golden", "make_vae_golden.py"))
    mkv = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mkv)
    g = np.load(os.path.join(HERE, "golden", "vae_oracle.npz"))
    assert float(mkv.latent().astype(np.float64).sum()) == float(g["full1024_checksum"])
    assert g["full1024_center"].shape == (3, 256, 256) and g["full1024_corners"].shape == (4, 3, 64, 64)
    for k in ("full1024_center", "full1024_corners", "full1024_mean"):
        assert np.isfinite(g[k]).all(), k
