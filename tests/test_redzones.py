"""The red-zone helper of the GPU tests, exercised on host tensors: a write
one element past either end of a buffer is reported, writes inside it are
not, and the zones of a buffer are forgotten after a check."""
import pytest

torch = pytest.importorskip("torch")

import redzones  # noqa: E402


def _zone_base():
    return redzones._live[-1][0]


def test_writes_inside_the_buffer_pass():
    t = redzones.poisoned((3, 5), torch.int32, 0x5A, "cpu")
    assert t.shape == (3, 5) and t.dtype == torch.int32
    assert (t.view(torch.uint8) == 0x5A).all()
    t.fill_(7)
    redzones.check()


@pytest.mark.parametrize("where", ["one_past_the_end", "one_before_the_start"])
def test_writes_just_outside_are_reported(where):
    t = redzones.poisoned(10, torch.float32, 0x11, "cpu")
    base = _zone_base()
    g = redzones.GUARD
    if where == "one_past_the_end":
        base[g + t.numel() * 4] = 0
        side = "after"
    else:
        base[g - 1] = 0
        side = "before"
    with pytest.raises(AssertionError, match=f"1 bytes changed {side} the buffer"):
        redzones.check()
    redzones.check()   # forgotten once checked


def test_empty_buffer_has_zones():
    t = redzones.poisoned((0, 4), torch.int32, 0x5A, "cpu")
    assert t.numel() == 0
    _zone_base()[redzones.GUARD] = 1   # the first byte after an empty buffer
    with pytest.raises(AssertionError, match="after the buffer"):
        redzones.check()
