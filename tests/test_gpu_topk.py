"""Exact parity of the selection's per-group top-k (mcs_topk_rows, the kernel
mcs_select runs on its key scores) with the oracle's top-k on the same
float32 rows: every kept index set must be identical, ties to the lower index.

The rows reach each of the kernel's paths: the sampled band (the usual case,
DiT-shaped rows), the band's fallback when its sample misjudges the k-th score
(rows whose sampled lines hold only zeros), the fallbacks' two-read,
three-read and all-global variants (the k-th score's first-pass bin holding
at most 2048, at most 4096, or more scores), rows longer than the band's
131072 keys, ragged lengths, ties, zeros and subnormals, and k = 1 and k = n.
"""

import numpy as np
import pytest
import torch

import oracle.mcs_oracle as orc

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sample_lines(n):
    """32-key lines the kernel's band samples: one per stratum, at a hashed
    position (mirrors the kernel's rule, so that a test row can hide from it)."""
    nlines = -(-n // 32)
    nls = min(128, nlines)
    out = []
    for i in range(nls):
        a, b = i * nlines // nls, (i + 1) * nlines // nls
        out.append(a + (((i * 2654435761) & 0xFFFFFFFF) >> 7) % (b - a))
    return np.array(out, np.int64)


def dit_rows(rows, n, rng):
    """Key-score-like rows: a heavy-tailed background plus a few spatially
    clustered bumps (a group attends to tokens near it)."""
    out = np.empty((rows, n), np.float32)
    j = np.arange(n, dtype=np.float64)
    for r in range(rows):
        x = np.exp(rng.normal(size=n) * 1.2 - 9.0)
        for _ in range(rng.integers(1, 4)):
            c, w = rng.uniform(0, n), rng.uniform(n / 400, n / 40)
            x += rng.uniform(1e-4, 1e-2) * np.exp(-0.5 * ((j - c) / w) ** 2)
        out[r] = x
    return out


def hidden_bin_rows(rows, n, in_bin, k, rng):
    """Rows whose band sample sees only zeros (so the band misses and the
    fallback runs) and whose k-th score lies in a first-pass bin of about
    in_bin scores: in_bin scores in [1, 1.25) (one bin), the others in
    [0.01, 0.5), the sampled lines zero."""
    out = np.empty((rows, n), np.float32)
    lines = sample_lines(n)
    mask = np.zeros(n, bool)
    for ln in lines:
        mask[32 * ln:32 * ln + 32] = True
    free = np.nonzero(~mask)[0]
    for r in range(rows):
        x = rng.uniform(0.01, 0.5, size=n).astype(np.float32)
        hot = rng.choice(free, size=in_bin, replace=False)
        x[hot] = rng.uniform(1.0, 1.25, size=in_bin).astype(np.float32)
        x[mask] = 0.0
        out[r] = x
    assert k < in_bin
    return out


def run_rows(x, k, ld=None):
    rows, n = x.shape
    ld = ld or -(-n // 4) * 4
    buf = torch.zeros((max(rows, 1), ld), dtype=torch.float32)
    buf[:rows, :n] = torch.from_numpy(x)
    dev = buf.cuda()[:rows, :n]
    out = mcs.topk_rows(dev, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(x, k, what, ld=None):
    print(f"[case] top-k rows {what}: rows={x.shape[0]} n={x.shape[1]} k={k}", flush=True)
    got = run_rows(x, k, ld)
    for r in range(x.shape[0]):
        ref, _ = orc.topk_select(x[r].astype(np.float64), k)
        assert np.array_equal(got[r], ref), (
            f"{what} row {r}: first differences at {np.nonzero(got[r] != ref)[0][:8]}")


def test_dit_rows_video_layer_shape():
    _need_gpu()
    rng = np.random.default_rng(11)
    check(dit_rows(48, 24960, rng), 2496, "video layer (24960 keys, 10%)")


def test_dit_rows_long_and_asset_shapes():
    _need_gpu()
    rng = np.random.default_rng(12)
    check(dit_rows(12, 75600, rng), 3776, "long video layer (75600 keys, 5%)")
    check(dit_rows(12, 32768, rng), 8192, "asset layer (32768 keys, 25%)")
    check(dit_rows(12, 32768, rng), 2048, "asset layer (32768 keys, 6.25%)")


@pytest.mark.parametrize("in_bin,k", [(1500, 1000), (3000, 2000), (6000, 4000)])
def test_band_fallback_paths(in_bin, k):
    _need_gpu()
    rng = np.random.default_rng(13 + in_bin)
    check(hidden_bin_rows(6, 20000, in_bin, k, rng), k, f"hidden sample, k-th bin ~{in_bin}")


def test_uniform_ragged_and_long_rows():
    _need_gpu()
    rng = np.random.default_rng(14)
    check(rng.random((8, 24961), dtype=np.float32), 100, "uniform, ragged length")
    check(rng.random((4, 24961), dtype=np.float32), 2500, "uniform, ragged length, padded stride", ld=25088)
    check(rng.random((3, 131072), dtype=np.float32), 13107, "uniform, longest band row")
    check(rng.random((2, 140001), dtype=np.float32), 5000, "uniform, longer than the band's rows")
    check(rng.random((4, 5000), dtype=np.float32), 4999, "uniform, all but one")


def test_ties_zeros_and_subnormals():
    _need_gpu()
    rng = np.random.default_rng(15)
    check((rng.integers(0, 8, size=(6, 4096)) * 0.125).astype(np.float32), 409, "eight distinct values")
    check(np.ones((3, 16384), np.float32), 300, "all equal")
    x = rng.random((4, 10000), dtype=np.float32)
    x[:, ::3] = 0.0
    x[:, 1::7] = np.float32(1e-40)  # subnormal
    x[:, 2::11] = np.float32(3e-39)
    check(x, 6000, "zeros and subnormals around the k-th score")
    check(np.zeros((2, 3000), np.float32), 1500, "all zero")


@pytest.mark.parametrize("n", [1, 3, 31, 33, 100, 4095, 4097])
def test_short_rows_k1_and_kn(n):
    _need_gpu()
    rng = np.random.default_rng(16 + n)
    x = rng.random((3, n), dtype=np.float32)
    check(x, 1, f"n={n}, k=1")
    check(x, n, f"n={n}, k=n")
    if n > 2:
        check(x, n // 2, f"n={n}, k=n/2")


def test_rejects_bad_rows():
    _need_gpu()
    x = torch.zeros((2, 30), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        mcs.topk_rows(x, 3)  # row stride 30 is not a multiple of 4
    y = torch.zeros((2, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(mcs._lib.McsError):
        mcs.topk_rows(y, 33)  # k > n
