"""The measurement probes (include/mla.h, mla_probe_*) on the GPU: they run,
and the LDS read probe reads exactly the bytes it documents.

Each workgroup of the LDS probe fills its 96 KB of LDS with word i =
i * 2654435761 (mod 2^32); lane l of wave w then reads, eight times per
iteration, W bytes at w * 8192 + j * (64 W) + l * W (j = 0..7) and XORs the
32-bit sum of the words it read into its output.  With one iteration the
output is therefore a closed form of (w, l), computed here on the host; with
two iterations every term appears twice and the output is zero.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import torch  # noqa: F401
    import mla_latent_kv_26_amd as m
    return m


def lds_expected(width, iterations, threads=512):
    out = np.zeros(threads, np.uint64)
    for tid in range(threads):
        w, l = tid >> 6, tid & 63
        x = 0
        for _ in range(iterations):
            for j in range(8):
                byte = w * 8192 + j * 64 * width + l * width
                words = [((byte // 4 + k) * 2654435761) & 0xFFFFFFFF for k in range(width // 4)]
                x ^= sum(words) & 0xFFFFFFFF
        out[tid] = x
    return out.astype(np.uint32)


@pytest.mark.parametrize("width", [16, 8])
@pytest.mark.parametrize("iterations", [1, 2, 3])
def test_lds_probe_reads_the_documented_bytes(m, width, iterations):
    import torch
    sink = m.mla_probe_sink()
    sink.zero_()
    nbytes = m.mla_probe_lds_read(width, iterations, sink)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert nbytes == cus * 8 * iterations * 8 * 64 * width
    got = sink[: cus * 512 * 4].view(torch.int32).cpu().numpy().view(np.uint32).reshape(cus, 512)
    want = lds_expected(width, iterations)
    for blk in (0, cus // 2, cus - 1):
        np.testing.assert_array_equal(got[blk], want)


def test_hbm_and_mfma_probes_run(m):
    import torch
    sink = m.mla_probe_sink()
    buf = torch.ones(64 * 36864, dtype=torch.uint8, device="cuda")
    m.mla_probe_hbm_read(buf, 0, sink)
    m.mla_probe_hbm_read(buf, 1, sink)
    flops = m.mla_probe_mfma(8, 10, sink)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 10 * 4 * 32768
    out = sink[: 8 * 256 * 4].view(torch.float32).cpu().numpy()
    assert np.all(np.isfinite(out))
