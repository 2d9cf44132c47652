"""The reference streaming copy (the bandwidth yardstick of the bench line):
every byte arrives, nothing past the end is written, bad arguments are
refused before any launch."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 48, (1 << 20) + 16, 3 * 4096 * 257 + 32])
def test_copy_reference_copies_every_byte(nbytes):
    import torch
    import moe_expert_token_amd as ms
    rng = np.random.default_rng(nbytes)
    src_h = rng.integers(0, 256, size=nbytes + 64, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    ms.moe_shuffle_copy_reference(src, dst, nbytes)
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got[:nbytes], src_h[:nbytes])
    assert (got[nbytes:] == 0xA5).all()  # nothing past the end


def test_copy_reference_rejects_bad_arguments():
    import torch
    import moe_expert_token_amd as ms
    a = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    b = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(ms.MoeShuffleError) as e:
        ms.moe_shuffle_copy_reference(a, b, 24)
    assert e.value.code == ms.E_ALIGN
    with pytest.raises(ms.MoeShuffleError) as e:
        ms.moe_shuffle_copy_reference(a[8:], b, 16)
    assert e.value.code == ms.E_ALIGN
    with pytest.raises(ms.MoeShuffleError) as e:
        ms.moe_shuffle_copy_reference(a, a[16:], 64)
    assert e.value.code == ms.E_INVALID_ARG
    ms.moe_shuffle_copy_reference(a, b, 0)
    torch.cuda.synchronize()
