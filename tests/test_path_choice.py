"""Host-side choice between the shared-dS and the recompute path (CPU only)."""
import pytest

from flashattention_backward_pass_bwd_amd import _lib, api

GB = 1 << 30


@pytest.mark.parametrize("dtype,ws,free,want", [
    (_lib.FA_DTYPE_BF16, 8 * GB, 280 * GB, True),     # the long workload's 8.7 GB on an idle 288 GB device
    (_lib.FA_DTYPE_BF16, 8 * GB, 16 * GB, True),      # exactly half of the free memory
    (_lib.FA_DTYPE_BF16, 8 * GB + 1, 16 * GB, False),  # just over half: recompute instead
    (_lib.FA_DTYPE_BF16, 300 * GB, 280 * GB, False),   # more than the device holds
    (_lib.FA_DTYPE_BF16, 0, 280 * GB, False),          # nothing visible: no workspace to share
    (_lib.FA_DTYPE_F32, 1, 280 * GB, False),           # fp32 has no shared-dS path
])
def test_shared_ds_only_when_the_workspace_fits(dtype, ws, free, want):
    assert api.use_shared_ds(dtype, ws, free) is want


def test_fraction_is_stated_and_applied():
    assert 0 < api.DS_WORKSPACE_FRACTION <= 1
    assert api.use_shared_ds(_lib.FA_DTYPE_BF16, 3 * GB, 10 * GB, fraction=0.3)
    assert not api.use_shared_ds(_lib.FA_DTYPE_BF16, 3 * GB + 1, 10 * GB, fraction=0.3)
