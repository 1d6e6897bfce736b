"""Seeded synthetic workloads for joint RoPE attention.

This module only builds inputs: shapes, token segments, position ids and
seeded random Q/K/V.  It holds none of the attention arithmetic, so both the
oracle (tests) and the HIP path (binding, bench) can draw the same inputs.

Workload structure follows the FLUX 3 Image Klein pages:
  * one joint sequence ordered text, noisy image, then references (Hugging
    Face blog "Welcome FLUX.3 Image Klein in Diffusers", Architecture section);
  * one token per 16x16 pixel patch, so a 1024^2 image is a 64x64 grid of
    4,096 tokens (same page, "The VAE and Tokenization");
  * a 1024^2 reference adds 4,096 tokens per transformer call (techbeat story,
    Summary);  width 3072 = 24 heads x 128 (blog, "The Qwen3-VL Text Encoder");
  * "up to 4K" resolution (model README, Model overview table) -> 256x256.

Position ids are three-axis integers: text token i -> (i, 0, 0), image token
at grid (r, c) -> (0, r, c), reference k = 1..R at (r, c) -> (k, r, c).

Random draws: one numpy PCG64 generator per call, seeded with the config's
seed, draws float32 standard normals for Q, then K, then V (each [B, N, H, D]),
multiplies by sigma and rounds to bfloat16 with round-to-nearest-even done on
the bit pattern.  For the FP8 workload each (tensor, batch, head) slice is then
scaled by s = absmax / 448 (s = 1 for an all-zero slice) and rounded to OCP
e4m3 ("e4m3fn") codes with saturation at +-448; the codes and the float32
scales are the inputs.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Segment:
    kind: str          # "text", "image" or "ref"
    rows: int          # text: token count; image/ref: grid rows
    cols: int = 1      # image/ref: grid cols
    index: int = 0     # ref: 1-based reference number (third-axis offset)

    @property
    def tokens(self) -> int:
        return self.rows * self.cols if self.kind != "text" else self.rows


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    segments: Tuple[Segment, ...]
    sigma: float
    fp8: bool
    seed: int
    description: str
    # Share of a per-(batch, head) direction u common to all of Q and K:
    # q = sigma (a u + sqrt(1 - a^2) z).  With a > 0 the rotary embedding makes
    # scores depend mostly on relative position (local attention).  0: plain
    # Gaussian Q and K.
    coherence: float = 0.0

    @property
    def tokens(self) -> int:
        return sum(s.tokens for s in self.segments)

    @property
    def segment_tokens(self) -> List[int]:
        return [s.tokens for s in self.segments]

    @property
    def axes_dim(self) -> Tuple[int, int, int]:
        return default_axes_dim(self.head_dim)

    def flops(self) -> float:
        """Algorithmic matrix flops of one call: QK^T and PV, 2 flops per MAC."""
        n = self.tokens
        return 4.0 * self.batch * self.heads * n * n * self.head_dim


def default_axes_dim(head_dim: int) -> Tuple[int, int, int]:
    """Split of head_dim over the three position axes: (D/4, 3D/8, 3D/8)."""
    if head_dim % 16:
        raise ValueError("head_dim must be a multiple of 16")
    return (head_dim // 4, 3 * head_dim // 8, 3 * head_dim // 8)


def _text(n):
    return Segment("text", n)


def _img(r, c):
    return Segment("image", r, c)


def _ref(k, r, c):
    return Segment("ref", r, c, k)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", 1, 2, 64, (_text(16), _img(8, 8)), 1.0, False, 1,
                 "tiny: 16 text + 8x8 image tokens (80), 2 heads, head_dim 64"),
        Workload("t2i1024", 1, 24, 128, (_text(512), _img(64, 64)), 0.5, False, 2,
                 "1024^2 text-to-image: 512 text + 64x64 image tokens (4,608), 24 heads, head_dim 128"),
        Workload("edit1024", 1, 24, 128, (_text(512), _img(64, 64), _ref(1, 64, 64)), 0.5, False, 3,
                 "1024^2 single-reference edit: 512 text + 4,096 image + 4,096 reference tokens (8,704)"),
        Workload("gen2048r2", 1, 24, 128,
                 (_text(512), _img(128, 128), _ref(1, 64, 64), _ref(2, 64, 64)), 0.5, False, 4,
                 "2048^2 with two 1024^2 references: 512 + 16,384 + 2x4,096 tokens (25,088)"),
        Workload("gen4k_fp8", 1, 24, 128, (_text(512), _img(256, 256)), 0.5, True, 5,
                 "4K generation, e4m3 Q/K/V with per-head scales: 512 + 256x256 tokens (66,048)"),
        Workload("edit1024_local", 1, 24, 128, (_text(512), _img(64, 64), _ref(1, 64, 64)), 1.5, False, 6,
                 "edit-call tokens (8,704) with position-local attention (sigma 1.5; Q and K share a "
                 "per-head direction, coherence 0.9): input for tile-sparse attention", 0.9),
    ]
}


def custom_workload(name: str, batch: int, heads: int, head_dim: int,
                     segments: Sequence[Segment], sigma: float = 0.5,
                     fp8: bool = False, seed: int = 0) -> Workload:
    return Workload(name, batch, heads, head_dim, tuple(segments), sigma, fp8, seed, name)


def position_ids(segments: Sequence[Segment]) -> np.ndarray:
    """[N, 3] int32 position ids for text / image / reference segments."""
    out = []
    t0 = 0
    for s in segments:
        if s.kind == "text":
            ids = np.zeros((s.rows, 3), np.int32)
            ids[:, 0] = np.arange(t0, t0 + s.rows, dtype=np.int32)
            t0 += s.rows
        else:
            r, c = np.meshgrid(np.arange(s.rows, dtype=np.int32),
                               np.arange(s.cols, dtype=np.int32), indexing="ij")
            ids = np.stack([np.full(r.size, s.index, np.int32), r.ravel(), c.ravel()], axis=1)
        out.append(ids.astype(np.int32))
    return np.ascontiguousarray(np.concatenate(out, axis=0))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _round(x: np.ndarray, sigma: float) -> np.ndarray:
    """sigma * x (float32) rounded to bf16 bits."""
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return f32_to_bf16_bits(x)


def quantize_e4m3_per_head(x_bf16_bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-(batch, head) absmax scaling and RNE rounding to e4m3fn codes.

    x: [B, N, H, D] bf16 bits.  Returns (codes uint8 [B, N, H, D],
    scales float32 [B, H]).  The rounding itself is torch's float8_e4m3fn cast;
    values are clamped to +-448 first because that cast does not saturate.
    """
    import torch

    x = torch.from_numpy(bf16_bits_to_f32(x_bf16_bits))
    absmax = x.abs().amax(dim=(1, 3))                       # [B, H]
    scale = torch.where(absmax > 0, absmax / E4M3_MAX, torch.ones_like(absmax))
    y = (x / scale[:, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), scale.numpy().astype(np.float32)


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray                  # [B,N,H,D] uint16 (bf16 bits) or uint8 (e4m3 codes)
    k: np.ndarray
    v: np.ndarray
    pos: np.ndarray                # [N,3] int32
    segment_tokens: List[int]
    scales: Optional[np.ndarray]   # [3,B,H] float32 for fp8, else None

    def sha256(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k, self.v, self.pos) + ((self.scales,) if self.scales is not None else ()):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def make_inputs(w: Workload, seed: Optional[int] = None, sigma: Optional[float] = None) -> Inputs:
    seed = w.seed if seed is None else seed
    sigma = w.sigma if sigma is None else sigma
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (w.batch, w.tokens, w.heads, w.head_dim)
    zq = rng.standard_normal(shape, dtype=np.float32)
    zk = rng.standard_normal(shape, dtype=np.float32)
    zv = rng.standard_normal(shape, dtype=np.float32)
    if w.coherence:
        a = np.float32(w.coherence)
        b = np.float32(np.sqrt(1.0 - w.coherence * w.coherence))
        u = rng.standard_normal((w.batch, 1, w.heads, w.head_dim), dtype=np.float32)
        zq = a * u + b * zq
        zk = a * u + b * zk
    q, k, v = (_round(z, sigma) for z in (zq, zk, zv))
    pos = position_ids(w.segments)
    scales = None
    if w.fp8:
        q, sq = quantize_e4m3_per_head(q)
        k, sk = quantize_e4m3_per_head(k)
        v, sv = quantize_e4m3_per_head(v)
        scales = np.ascontiguousarray(np.stack([sq, sk, sv]).astype(np.float32))
    return Inputs(w, q, k, v, pos, w.segment_tokens, scales)
