"""Host-side bookkeeping of the sketched linear layer (CPU only: no kernel
runs). The carried weight norm must be streamed again (fresh) whenever the
weights may have changed outside the layer's own carried updates."""
import torch

from rank_randomized_gradient_amd import SketchedLinear


def _layer():
    return SketchedLinear(64, 32, 16, device="cpu", carry_norm=True)


def test_new_layer_streams_the_norm():
    assert _layer()._norm_is_stale()


def test_version_counter_marks_the_norm_stale():
    layer = _layer()
    # as after a carried update: the buffer holds ||W||^2 of the weights as they stand
    layer._norm_fresh = False
    layer._norm_version = layer.weight._version
    assert not layer._norm_is_stale()
    with torch.no_grad():
        layer.weight.mul_(2)
    assert layer._norm_is_stale()


def test_load_state_dict_marks_the_norm_stale():
    layer = _layer()
    sd = layer.state_dict()
    layer._norm_fresh = False
    layer._norm_version = layer.weight._version
    layer.load_state_dict(sd)
    assert layer._norm_fresh and layer._norm_is_stale()


def test_invalidate_marks_the_norm_stale():
    layer = _layer()
    layer._norm_fresh = False
    layer._norm_version = layer.weight._version
    layer.invalidate_weight_norm()
    assert layer._norm_is_stale()
