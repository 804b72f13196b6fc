"""The MFMA rate probe (c3_probe_mfma_rate) does the work it is timed for: every wave's 64 lane
sums equal the closed form iterations * 8 * (S0 + S1), with S_s = sum over k of (sum over the 32
rows of X_s[.][k]) * (sum over the 32 columns of Y_s[k][.]) for the probe's operands: exactly for
the small-integer operands (every product and partial sum is an integer below 2^24), within fp32
rounding for the random ones; and the same bits on every run."""
import numpy as np
import pytest




def probe_bits(seed):
    """The probe's random bf16 operand for a seed, as float64 (same formula as the kernel)."""
    h = (np.asarray(seed, dtype=np.uint64) * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)
    bits = ((h >> np.uint64(31)) << np.uint64(15)) | \
        ((np.uint64(125) + ((h >> np.uint64(20)) & np.uint64(3))) << np.uint64(7)) | \
        (h & np.uint64(0x7F))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def closed_form_per_wave(iterations: int, random: int) -> float:
    i = np.arange(32)
    k = np.arange(16)
    total = 0.0
    for s in (0, 1):
        if random:
            X = probe_bits(i[:, None] * 16 + k[None, :] + s * 512 + 1)            # [i][k]
            Y = probe_bits(k[:, None] * 32 + i[None, :] + s * 512 + 1025)         # [k][j]
        else:
            X = (((i[:, None] * 31 + k[None, :] * 17 + s * 7 + 3) % 5) - 2).astype(np.float64)
            Y = (((k[:, None] * 13 + i[None, :] * 29 + s * 11 + 1) % 5) - 2).astype(np.float64)
        total += float(np.dot(X.sum(axis=0), Y.sum(axis=1)))
    return iterations * 8 * total


def test_closed_form_reference_on_tiny_matrices():
    """The host reference (sum of all entries of X_s . Y_s) against explicit products."""
    i = np.arange(32)
    k = np.arange(16)
    for random in (0, 1):
        want = 0.0
        for s in (0, 1):
            if random:
                X = probe_bits(i[:, None] * 16 + k[None, :] + s * 512 + 1)
                Y = probe_bits(k[:, None] * 32 + i[None, :] + s * 512 + 1025)
            else:
                X = (((i[:, None] * 31 + k[None, :] * 17 + s * 7 + 3) % 5) - 2).astype(float)
                Y = (((k[:, None] * 13 + i[None, :] * 29 + s * 11 + 1) % 5) - 2).astype(float)
            want += (X @ Y).sum()
        assert closed_form_per_wave(1, random) == pytest.approx(8 * want, rel=1e-12)


@pytest.mark.gpu
@pytest.mark.parametrize("n_wg,iters,random", [(8, 100, 0), (256, 1000, 0), (3, 262144, 0),
                                               (8, 100, 1), (256, 1000, 1)])
def test_mfma_probe_closed_form(c3gpu, n_wg, iters, random):
    import torch

    print(f"MFMA probe {n_wg} workgroups x {iters} iterations, random={random}", flush=True)
    out = torch.full((n_wg * 256,), float("nan"), dtype=torch.float64, device="cuda:0")
    c3gpu.c3_probe_mfma_rate(out, n_wg, iters, random)
    torch.cuda.synchronize()
    per_wave = out.cpu().numpy().reshape(n_wg * 4, 64).sum(axis=1)
    want = closed_form_per_wave(iters, random)
    if random:
        np.testing.assert_allclose(per_wave, want, rtol=1e-3)
    else:
        assert np.all(per_wave == want), (per_wave[:4], want)
    again = torch.empty_like(out)
    c3gpu.c3_probe_mfma_rate(again, n_wg, iters, random)
    torch.cuda.synchronize()
    assert torch.equal(out, again)


@pytest.mark.gpu
def test_mfma_probe_arguments(c3gpu):
    import torch

    out = torch.empty(256, dtype=torch.float64, device="cuda:0")
    for n_wg, iters, random in ((0, 10, 1), (1, 0, 1), (1, 262145, 0), (65537, 10, 1), (1, 10, 2)):
        with pytest.raises(c3gpu.C3Error) as e:
            c3gpu.c3_probe_mfma_rate(out, n_wg, iters, random)
        assert e.value.status == c3gpu.C3_E_INVALID
