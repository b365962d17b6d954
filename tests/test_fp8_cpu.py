"""Host-side validation of the FP8 key entry points (no call here reaches a
kernel launch)."""

import pytest

K = pytest.importorskip("kv_cache_quantization_codec_amd")
B = K.binding
E = {name: code for code, name in B.STATUS_NAMES.items()}
FAKE = 0x10000


@pytest.mark.parametrize("name", ["kivi_fp8_encode", "kivi_fp8_decode"])
@pytest.mark.parametrize("args,status", [
    ((FAKE, 2, 64, 12, 1024, FAKE, 1024), "KIVI_E_HEAD_DIM"),
    ((FAKE, 2, 64, 264, 1 << 15, FAKE, 1 << 15), "KIVI_E_HEAD_DIM"),
    ((FAKE, -1, 64, 128, 8192, FAKE, 8192), "KIVI_E_SHAPE"),
    ((FAKE, 2, 64, 128, 8176, FAKE, 8192), "KIVI_E_SHAPE"),      # stride < n_tokens * D
    ((FAKE, 2, 64, 128, 8192, FAKE, 8200), "KIVI_E_ALIGN"),      # stride not a multiple of 16
    ((FAKE, 2, 1 << 29, 128, 1 << 36, FAKE, 1 << 36), "KIVI_E_SHAPE"),   # index range
    ((0, 2, 64, 128, 8192, FAKE, 8192), "KIVI_E_NULL"),
    ((FAKE, 2, 64, 128, 8192, 0, 8192), "KIVI_E_NULL"),
    ((FAKE + 8, 2, 64, 128, 8192, FAKE, 8192), "KIVI_E_ALIGN"),
    ((0, 0, 64, 128, 8192, 0, 8192), "KIVI_OK"),                 # no slices: nothing touched
    ((0, 2, 0, 128, 0, 0, 0), "KIVI_OK"),                        # no tokens
])
def test_fp8_argument_errors(name, args, status):
    assert getattr(B.lib(), name)(*args, None) == E[status]
