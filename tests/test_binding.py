"""Host-side checks of the Python binding that run before any GPU call: an
``out`` or ``workspace`` that cannot hold the result is refused with
ValueError (the C ABI cannot see a tensor's extent, only its row stride)."""

import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def rts():
    import row_top_select_amd
    return row_top_select_amd


def test_topk_rows_out_too_small(rts):
    x = torch.zeros((4, 100), dtype=torch.float32)
    with pytest.raises(ValueError, match="at least"):
        rts.topk_rows(x, 8, out=torch.empty((1, 8), dtype=torch.int32))     # too few rows
    with pytest.raises(ValueError, match="at least"):
        rts.topk_rows(x, 8, out=torch.empty((4, 7), dtype=torch.int32))     # too few columns
    with pytest.raises(ValueError, match="unit column stride"):
        rts.topk_rows(x, 8, out=torch.empty((8, 4), dtype=torch.int32).t())
    with pytest.raises(TypeError):
        rts.topk_rows(x, 8, out=torch.empty((4, 8), dtype=torch.int64))


def test_topk_rows_workspace_must_be_a_tensor(rts):
    x = torch.zeros((4, 100), dtype=torch.float32)
    with pytest.raises(ValueError, match="workspace"):
        rts.topk_rows(x, 8, workspace=bytearray(64))


def test_topk_rows_rejects_host_tensors(rts):
    # shapes are fine: the call reaches the device-pointer marshalling and stops there
    with pytest.raises(ValueError, match="GPU tensor"):
        rts.topk_rows(torch.zeros((4, 100)), 8)
