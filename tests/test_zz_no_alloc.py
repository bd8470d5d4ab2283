"""rgc_apply_noalloc, the normalized update for callers that cannot allocate:
the same kernels as rgc_apply with the workspace in the library's static
device scratch. Called through the C ABI; its weights and stats must equal
rgc_apply's bit for bit on the same inputs (the parity bar for this entry
point is rgc_apply's own, which the parity tests hold against the oracle),
over calls in a row on one device, each later one with a smaller input, so
that a call sees what the previous one left in the shared scratch."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as orc
from rank_randomized_gradient_amd import rgc, synth
from parity_tools import assert_update_close

pytestmark = pytest.mark.gpu

bits = synth.to_numpy_bits


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rgc.load_library()
    return torch.device("cuda", 0)


def _inputs(d, k, r, seed):
    w = synth.normal_bf16((d, k), 0.02, seed=seed)
    c = synth.normal_f32((d, r), 1e-2, seed=seed + 1)
    p = orc.qr_projection(seed, k, r) if r <= 128 else orc.rademacher_projection(seed, k, r)
    return w, c, synth.from_numpy_bits(p)


# larger first, then smaller: the Gram-form norms (r <= 128), then the
# rebuilt-H norms (r > 128), then the smallest shape
SEQUENCE = [(6144, 2048, 64), (2048, 2048, 128), (264, 1048, 192), (256, 512, 16)]


def test_noalloc_matches_rgc_apply_in_a_row(dev):
    lib = rgc.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for d, k, r in SEQUENCE:
        w, c, p = _inputs(d, k, r, d + k + r)
        seed, tau = 0xC0FFEE + d, 1e-3
        cg, pg = c.to(dev), p.to(dev)
        w_ref, w_na = w.clone().to(dev), w.clone().to(dev)
        st_ref, st_na = torch.zeros(4, device=dev), torch.zeros(4, device=dev)
        rgc.rgc_apply(w_ref, cg, pg, tau, seed, stats=st_ref)
        status = lib.rgc_apply_noalloc(w_na.data_ptr(), k, cg.data_ptr(), pg.data_ptr(), d, k, r, tau, seed,
                                       st_na.data_ptr(), stream)
        assert status == 0, lib.rgc_status_string(status)
        torch.cuda.synchronize()
        assert torch.equal(w_ref.view(torch.int16), w_na.view(torch.int16)), (d, k, r)
        assert torch.equal(st_ref, st_na), (d, k, r)
        ref_w, ref_stats = orc.apply_update(bits(w), c.numpy(), bits(p), tau, seed)
        np.testing.assert_allclose(st_na.cpu().numpy()[:3], ref_stats[:3], rtol=1e-5)
        abs_terms = np.abs(c.numpy().astype(np.float64)) @ np.abs(orc.bf16_to_f64(bits(p))).T
        assert_update_close(bits(w_na), ref_w, ref_stats[2], abs_terms, what=f"noalloc W {d}x{k}x{r}")


def test_noalloc_zero_sketch_then_update(dev):
    """A skipped update (zero sketch) followed by a real one on the same scratch."""
    d, k, r = 256, 512, 16
    w, c, p = _inputs(d, k, r, 7)
    pg = p.to(dev)
    wg = w.clone().to(dev)
    st = torch.zeros(4, device=dev)
    rgc.rgc_apply_noalloc(wg, torch.zeros(d, r, device=dev), pg, 1e-3, 1, stats=st)
    torch.cuda.synchronize()
    assert st.cpu().numpy()[3] == 1 and np.array_equal(bits(wg), bits(w))
    w_ref = w.clone().to(dev)
    rgc.rgc_apply(w_ref, c.to(dev), pg, 1e-3, 2)
    rgc.rgc_apply_noalloc(wg, c.to(dev), pg, 1e-3, 2, stats=st)
    torch.cuda.synchronize()
    assert torch.equal(w_ref.view(torch.int16), wg.view(torch.int16))
