"""The allocation-free int8 GEMV (qmm_gemv_i8_noalloc) against the entry
point it stands in for (qmm_gemv_i8 with a caller workspace): same kernels,
so the outputs must agree bit for bit.  Two calls in a row on the library's
scratch, the second smaller than the first, so the second runs on a scratch
that still holds the first call's larger quantization."""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gguf_block_quantized_kind_amd as qmm  # noqa: E402

from test_gpu_parity import SENTINEL, dev, filled, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qmm.load_library()


def with_workspace(kind, P, x, M, N, K):
    ws = torch.empty(qmm.qmm_gemv_i8_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
    y = filled((M, N))
    qmm.qmm_gemv_i8(kind, P, x, y, M, N, K, ws)
    return host(y)


def without_workspace(kind, P, x, M, N, K):
    y = filled((M, N))
    qmm.qmm_gemv_i8_noalloc(kind, P, x, y, M, N, K)
    return host(y)


@pytest.mark.parametrize("kind", ["Q8_0", "Q4_0", "MXFP4"])
@pytest.mark.parametrize("xdt", ["f32", "f16"])
def test_noalloc_matches_the_workspace_entry_point(kind, xdt):
    g = wl.rng("gpu_noalloc", f"{kind}_{xdt}")
    dt = np.float16 if xdt == "f16" else np.float32
    # The largest M * K the scratch holds, then a smaller and ragged call.
    for M, N, K in ((8, 1040, 32768), (3, 300, 1024)):
        W = wl.random_weights(kind, N, K, g)
        P = qmm.repack(kind, dev(W), N, K)
        x = dev(wl.activations((M, K), dt, g))
        got = without_workspace(kind, P, x, M, N, K)
        want = with_workspace(kind, P, x, M, N, K)
        assert not np.any(got == SENTINEL), f"M={M} K={K}: outputs not written"
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"M={M} N={N} K={K}"


def test_noalloc_rejects_a_size_beyond_its_scratch():
    M, N, K = 8, 64, 32768 + 256
    W = wl.random_weights("Q8_0", N, K, wl.rng("gpu_noalloc", "big"))
    P = qmm.repack("Q8_0", dev(W), N, K)
    x = dev(np.zeros((M, K), dtype=np.float32))
    y = filled((M, N))
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_gemv_i8_noalloc("Q8_0", P, x, y, M, N, K)
    assert "exceeds" in str(e.value)
    assert np.all(host(y) == SENTINEL)
