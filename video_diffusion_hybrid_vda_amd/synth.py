"""Seeded synthetic inputs for the Video DeltaNet hybrid attention forward.

This module only draws random tensors of the right shapes and value ranges;
it holds none of the method's arithmetic.  Both the HIP path (through the
binding) and the CPU oracle are fed from it, so they see bit-identical inputs.

Shapes follow the statement of the problem: Q/K/V are laid out as
[batch, heads, frames, tokens_per_frame, head_dim]; per-frame decay gamma and
write strength beta are [batch, heads, frames]; the layer input x is
token-major [batch, frames*tokens_per_frame, heads*head_dim]; weights are
[D_in, D_out] row-major (y = x @ W).

Value recipe (the pages publish no activations or weights, so these stand in
for the MiniMax H3 768p workload): Q, V, x ~ N(0, 1); K ~ N(0, 1) with every
token row scaled to unit L2 norm (the caller-side normalisation the operator
assumes); beta ~ U(beta_lo, beta_hi); gamma ~ U(gamma_lo, gamma_hi); gate and
output-projection weights ~ N(0, w_std^2); RMSNorm weight = 1.
Draw order is fixed: q, k, v, x, beta, gamma, w_gs, w_gl, w_os, w_ol.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class VdnConfig:
    batch: int
    heads: int
    head_dim: int
    frames: int
    tokens_per_frame: int
    dtype: str = "bf16"          # "f32" or "bf16" storage for q/k/v/x/weights
    chunk_frames: int = 5        # latent frames per VAE temporal chunk
    window_chunks: int = 1       # +-chunks of the sliding window
    anchor_first: bool = True
    anchor_last: bool = True
    beta_lo: float = 0.1
    beta_hi: float = 1.0
    gamma_lo: float = 0.9
    gamma_hi: float = 1.0
    w_std: float = 0.02
    rms_eps: float = 1e-6
    seed: int = 0
    name: str = ""
    context_tokens: int = 0      # text/audio tokens after the video tokens

    @property
    def model_dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def seq_len(self) -> int:
        """Rows per (batch, head): video tokens, then context tokens."""
        return self.frames * self.tokens_per_frame + self.context_tokens

    @property
    def video_len(self) -> int:
        return self.frames * self.tokens_per_frame

    def replace(self, **kw) -> "VdnConfig":
        return dataclasses.replace(self, **kw)


# The five workloads of the operator's statement (tiny fp32 layer, VDA-only
# scan, 42-frame layer, 102-frame headline layer, batch-2 length sweep).
CONFIGS = {
    1: VdnConfig(1, 1, 32, 10, 16, dtype="f32", beta_lo=0.0, beta_hi=1.0, seed=0,
                 name="tiny fp32 layer B1 H1 d32 T10 N16"),
    2: VdnConfig(1, 8, 64, 42, 1560, dtype="bf16", seed=1,
                 name="VDA scan B1 H8 d64 T42 N1560"),
    3: VdnConfig(1, 24, 128, 42, 4032, dtype="bf16", seed=2,
                 name="hybrid layer B1 H24 d128 T42 N4032"),
    4: VdnConfig(1, 24, 128, 102, 4032, dtype="bf16", seed=3,
                 name="hybrid layer B1 H24 d128 T102 N4032"),
    5: VdnConfig(2, 24, 128, 102, 4032, dtype="bf16", seed=4,
                 name="hybrid layer B2 H24 d128 T{42,62,82,102} N4032"),
}


def make_inputs(cfg: VdnConfig, device="cpu", with_layer: bool = True) -> dict:
    """Draw every input of one hybrid-attention call.

    Returns a dict of torch tensors on `device`: q, k, v (cfg.dtype) of shape
    [B, H, T, N, d], or [B, H, T*N + n_ctx, d] when cfg.context_tokens > 0
    (context rows after the video rows, drawn like them), gamma, beta
    (float32), and when `with_layer`: x [B, T*N + n_ctx, D], w_gs, w_gl, w_os,
    w_ol (cfg.dtype) and rms_w (float32).  Random numbers are drawn in float32 from
    a torch.Generator seeded with cfg.seed on `device`, then rounded once to
    the storage dtype (round to nearest even for bf16).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    dt = DTYPES[cfg.dtype]
    B, H, T, N, d = cfg.batch, cfg.heads, cfg.frames, cfg.tokens_per_frame, cfg.head_dim
    D, L = cfg.model_dim, cfg.seq_len

    def randn(*shape, std=1.0):
        t = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        return t.mul_(std) if std != 1.0 else t

    def uniform(lo, hi, *shape):
        t = torch.rand(*shape, generator=gen, device=dev, dtype=torch.float32)
        return t.mul_(hi - lo).add_(lo)

    out = {}
    qkv_shape = (B, H, T, N, d) if cfg.context_tokens == 0 else (B, H, L, d)
    out["q"] = randn(*qkv_shape).to(dt)
    k = randn(*qkv_shape)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    out["k"] = k.to(dt)
    del k
    out["v"] = randn(*qkv_shape).to(dt)
    x = randn(B, L, D).to(dt) if with_layer else None
    out["beta"] = uniform(cfg.beta_lo, cfg.beta_hi, B, H, T).contiguous()
    out["gamma"] = uniform(cfg.gamma_lo, cfg.gamma_hi, B, H, T).contiguous()
    if with_layer:
        out["x"] = x
        for name in ("w_gs", "w_gl", "w_os", "w_ol"):
            out[name] = randn(D, D, std=cfg.w_std).to(dt)
        out["rms_w"] = torch.ones(D, device=dev, dtype=torch.float32)
    return out


def sample_tokens(cfg: VdnConfig, count: int, seed: int = 1234) -> list:
    """Query tokens to check at full size: the first/last token of every
    anchor frame and chunk edge, the ragged last chunk, random video tokens,
    and the first, middle and last context token if there are any."""
    T, N, C = cfg.frames, cfg.tokens_per_frame, cfg.chunk_frames
    picks = {0, N - 1, N, T * N - 1, (T - 1) * N, (T - 1) * N - 1}
    for c in range(0, T, C):
        picks.add(c * N)
        picks.add(max(c * N - 1, 0))
    g = torch.Generator().manual_seed(seed)
    extra = torch.randint(0, T * N, (max(count - len(picks), 0),), generator=g).tolist()
    picks.update(extra)
    if cfg.context_tokens > 0:   # first, middle and last context token
        L = T * N
        picks.update({L, L + cfg.context_tokens // 2, L + cfg.context_tokens - 1})
    return sorted(p for p in picks if 0 <= p < cfg.seq_len)
