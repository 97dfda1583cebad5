"""Generator G: seeded DiT-shaped attention inputs.

The pages (the MC-Sparse abstract, "MC-Sparse: Deconstructing and Closing the
Dense-Sparse Attention Gap in Diffusion Transformers", and the blog summary
"MC-Sparse: three failure modes, one fix") measure on a video DiT and a 3D
asset DiT whose weights and data are not available.  These synthetic inputs
stand in for them: attention logits follow 3D token locality, queries and keys
carry a shared per-head rotation, values are Gaussian, and every later
denoising step perturbs the step-0 tensors with fresh Gaussian drift.

Recipe (all random draws are float32 standard normals from numpy's PCG64,
seeded by SeedSequence([seed, workload_id, stream, head, step])):

* grid (T, Y, X), N = T*Y*X, token i <-> (t, y, x) in raster order
  i = (t*Y + y)*X + x;
* position embedding P_i in R^d: sin/cos features of t, y and x with widths
  d/4, 3d/8, 3d/8; an axis of width w uses frequencies 10000^(-m/(w/2)),
  m = 0..w/2-1, laid out as [sin(u*w_0..), cos(u*w_0..)]; so |P_i|^2 = d/2;
* per head h: W_h = orthogonal factor of a QR of a Gaussian d x d matrix with
  the signs fixed so that diag(R) > 0;
  Q = 3 P W_h + 0.5 E_Q,  K = 3 P W_h + 0.5 E_K,  V = E_V;
* joint video + text sequences (the joint attention of MM-DiT blocks, whose
  text tokens are appended to the latent tokens): L text tokens follow the
  N_v grid tokens, each with an embedding T_j = sqrt(d/2) * u_j / |u_j|,
  u_j a Gaussian vector (stream 9, shared by all heads), in place of P;
  they enter Q, K and V exactly as grid tokens do;
* step t > 0: X_t = X_0 + delta * t * E_t with E_t freshly drawn per step,
  per tensor and per head (not a random walk);
* the float32 master is rounded to bfloat16 (round to nearest even) for the
  bf16 workloads; both sides receive exactly the same rounded values.
"""

from __future__ import annotations

import numpy as np

STREAM_W, STREAM_EQ, STREAM_EK, STREAM_EV = 0, 1, 2, 3
STREAM_DQ, STREAM_DK, STREAM_DV = 4, 5, 6
STREAM_PROJ, STREAM_KEEP = 7, 8
STREAM_TEXT = 9

_DRIFT_STREAMS = (STREAM_DQ, STREAM_DK, STREAM_DV)


def rng(seed: int, workload_id: int, stream: int, head: int = 0, step: int = 0) -> np.random.Generator:
    """Independent generator per (seed, workload, stream, head, step)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, workload_id, stream, head, step])))


def _normal(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def position_embedding(grid, d: int) -> np.ndarray:
    """3D sin/cos position features, float32 [N, d], raster order over (t, y, x)."""
    if d % 8 != 0:
        raise ValueError("head_dim must be a multiple of 8")
    T, Y, X = grid
    widths = (d // 4, 3 * d // 8, 3 * d // 8)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    coords = (t.reshape(-1), y.reshape(-1), x.reshape(-1))
    parts = []
    for u, w in zip(coords, widths):
        half = w // 2
        omega = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
        ang = u.astype(np.float64)[:, None] * omega[None, :]
        parts.append(np.sin(ang))
        parts.append(np.cos(ang))
    return np.concatenate(parts, axis=1).astype(np.float32)


def text_embedding(seed: int, workload_id: int, n_text: int, d: int) -> np.ndarray:
    """Embeddings of n_text text tokens, float32 [n_text, d], each of squared
    norm d/2 (that of every grid token's position embedding) in a Gaussian
    random direction."""
    u = _normal(rng(seed, workload_id, STREAM_TEXT), (n_text, d)).astype(np.float64)
    u *= np.sqrt(d / 2.0) / np.maximum(np.linalg.norm(u, axis=1, keepdims=True), 1e-300)
    return u.astype(np.float32)


def token_embedding(grid, d: int, n_text: int = 0, seed: int = 0, workload_id: int = 0) -> np.ndarray:
    """Embedding of every token of a sequence: the grid tokens in raster order
    (position_embedding), then n_text text tokens (text_embedding)."""
    pos = position_embedding(grid, d)
    if n_text <= 0:
        return pos
    return np.concatenate([pos, text_embedding(seed, workload_id, n_text, d)], axis=0)


def head_rotation(seed: int, workload_id: int, head: int, d: int) -> np.ndarray:
    """Haar-random orthogonal d x d matrix for one head (float32)."""
    a = _normal(rng(seed, workload_id, STREAM_W, head), (d, d)).astype(np.float64)
    qm, rm = np.linalg.qr(a)
    qm = qm * np.sign(np.diag(rm))[None, :]
    return qm.astype(np.float32)


def head_base(seed: int, workload_id: int, head: int, grid, d: int, pos: np.ndarray | None = None):
    """Step-0 float32 masters (Q0, K0, V0) of one head, each [N, d]."""
    if pos is None:
        pos = position_embedding(grid, d)
    n = pos.shape[0]
    w = head_rotation(seed, workload_id, head, d)
    pw = 3.0 * (pos.astype(np.float64) @ w.astype(np.float64))
    q = (pw + 0.5 * _normal(rng(seed, workload_id, STREAM_EQ, head), (n, d))).astype(np.float32)
    k = (pw + 0.5 * _normal(rng(seed, workload_id, STREAM_EK, head), (n, d))).astype(np.float32)
    v = _normal(rng(seed, workload_id, STREAM_EV, head), (n, d))
    return q, k, v


def head_step(base, seed: int, workload_id: int, head: int, step: int, delta: float, bf16: bool):
    """Inputs of one head at denoising step `step`, as float32 arrays.

    base = head_base(...) masters.  step 0 returns the (rounded) masters;
    step t > 0 adds delta * t * fresh Gaussian noise to each tensor.
    """
    out = []
    for x0, stream in zip(base, _DRIFT_STREAMS):
        if step == 0 or delta == 0.0:
            x = x0
        else:
            e = _normal(rng(seed, workload_id, stream, head, step), x0.shape)
            x = (x0 + np.float32(delta * step) * e).astype(np.float32)
        out.append(round_bf16(x) if bf16 else np.ascontiguousarray(x, dtype=np.float32))
    return tuple(out)


def hash_projections(seed: int, workload_id: int, d: int, bits: int = 8) -> np.ndarray:
    """Random projection directions, float32 [bits, d], shared by all heads."""
    return _normal(rng(seed, workload_id, STREAM_PROJ), (bits, d))


def keep_draw(seed: int, workload_id: int, heads: int, choices) -> np.ndarray:
    """Per-head keep fraction drawn uniformly from `choices` (float64 [heads])."""
    g = rng(seed, workload_id, STREAM_KEEP)
    pick = g.integers(0, len(choices), size=heads)
    return np.asarray(choices, dtype=np.float64)[pick]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)
