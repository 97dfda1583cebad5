"""GPU sign-hash keys on queries whose projections float32 arithmetic cannot
decide: sums that cancel to zero, to a remainder below float32's precision,
beyond float32's range, or into its subnormal range.  The key is defined by
the float64 sum in dimension order (oracle.hash_keys), so the permutation
must still match the oracle's bit for bit."""

import numpy as np
import pytest
import torch

import oracle.mcs_oracle as orc
from mcs_inputs import round_bf16

pytestmark = pytest.mark.gpu

mcs = pytest.importorskip("sparse_attention_diffusion_mcs_amd")

# three consecutive query values against projection entries (1, 1, -1); the
# float64 sum in order is the middle value (or, for the first pattern row
# below, the first), which float32 loses
PATTERNS = [
    (1.0, 2.0 ** -30, 1.0),          # 2^-30: float32 rounds 1 + 2^-30 to 1, sum 0
    (1.0, -2.0 ** -30, 1.0),         # -2^-30
    (1.0, 0.0, 1.0),                 # exactly 0: bit 0
    (2.0 ** -30, 1.0, 1.0),          # 2^-30 + 1 - 1: float32 sum 0
    (1.0, 2.0 ** -20, 1.0),          # representable, but below the decision threshold
    (2.0 ** 100, 2.0 ** 70, 2.0 ** 100),     # squares beyond float32's range
    (2.0 ** -120, 2.0 ** -130, 2.0 ** -120),  # subnormal remainder
]


def fp32_sum(x, r):
    """Sequential float32 fused multiply-add sum; exact in float64 for the
    values used here, so rounding each step to float32 is the fused result."""
    acc = np.float32(0.0)
    for a, b in zip(x, r):
        acc = np.float32(np.float64(acc) + np.float64(a) * np.float64(b))
    return acc


def problem(d, n, seed, bf16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d)).astype(np.float32)
    proj = rng.standard_normal((8, d)).astype(np.float32)
    rows = []
    for b in range(8):
        proj[b, 3 * b:3 * b + 3] = (1.0, 1.0, -1.0)
        for pat in PATTERNS:
            rows.append((b, pat))
    pos = rng.choice(n, size=len(rows), replace=False)
    for (b, pat), i in zip(rows, pos):
        q[i] = 0.0
        q[i, 3 * b:3 * b + 3] = pat
    if bf16:
        q = round_bf16(q)
    return q, proj, list(zip(rows, pos))


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (64, "fp32"), (128, "fp32")])
def test_hash_keys_float32_cannot_decide(d, dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H, n, G = 2, 640, 64
    bf16 = dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    qs, projs = [], None
    crafted = []
    for h in range(H):
        q, proj, rows = problem(d, n, 100 + h, bf16)
        if projs is None:
            projs = proj
        qs.append(q)
        crafted.append(rows)
    # one projection matrix for both heads (the second head's crafted rows
    # were placed against the first head's patterns, which are the same)
    print(f"[hash] d={d} {dtype}: {len(PATTERNS) * 8} crafted rows per head", flush=True)
    q_dev = torch.from_numpy(np.stack(qs)).to("cuda").to(tdt).contiguous()
    rng = np.random.default_rng(7)
    k_dev = torch.from_numpy(rng.standard_normal((H, n, d)).astype(np.float32)).to("cuda").to(tdt)
    v_dev = torch.from_numpy(rng.standard_normal((H, n, d)).astype(np.float32)).to("cuda").to(tdt)
    meta, _ = mcs.select(q_dev, k_dev, v_dev, G, [64] * H, projs, scale=1.0 / np.sqrt(d))
    torch.cuda.synchronize()
    perm = meta.perm.cpu().numpy()
    lost = 0
    for h in range(H):
        keys = orc.hash_keys(qs[h], projs)
        assert np.array_equal(perm[h], orc.group_permutation(keys)), f"head {h}: perm differs from the oracle's"
        for (b, pat), i in crafted[h]:
            bit = (int(keys[i]) >> b) & 1
            s32 = fp32_sum(qs[h][i], projs[b])
            lost += int((s32 > 0) != bool(bit))
    # the case only tests something if float32 alone gets some of these bits wrong
    assert lost >= 3 * H, f"only {lost} crafted bits differ between float32 and float64 sums"
