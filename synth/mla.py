"""Seeded synthetic inputs for the MLA attention sub-layer.

Shapes and distributions only (no arithmetic of the layer).  Recipe:

* x ~ N(0, 1) bf16 [T, d]; the input RMSNorm weight gamma = 1, or
  ~ N(1, gamma_std) bf16 for parity cases; the two latent-norm weights the same;
* the five projection matrices ~ N(0, 0.02) in nn.Linear [out, in] layout,
  stored as e4m3 codes with one fp32 scale per 128x128 block (scale = block
  amax / 448, codes = torch's float8_e4m3fn cast of the clamped quotient; a
  partial last row block, as in the 576-row key-value down-projection, takes
  the amax of its rows);
* the cache prefix (positions below each sequence's cached length): the
  normalised latent ~ N(0, 1) rounded to bf16 and block-quantised per 1x128
  the same way, the rotated positional key ~ N(0, 1.7) in bf16 (the spread a
  7168-wide N(0, 0.02) projection of a unit-RMS input has).  Positions at and
  past the cached length are left zero; the layer writes the new ones.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from .gen import _randn, block_quantize_weight

ROLE_MLA_X, ROLE_MLA_W, ROLE_MLA_NORM, ROLE_MLA_CACHE, ROLE_MLA_LEN = 21, 22, 23, 24, 25
FP8_MAX = 448.0
MATS = ("w_qa", "w_qb", "w_kva", "w_kvb", "w_o")


@dataclass(frozen=True)
class MLAShape:
    name: str
    n_seq: int
    n_new: int
    cached: tuple            # cached length of each sequence (len n_seq)
    max_len: int
    d_model: int = 7168
    n_heads: int = 64
    q_lora: int = 1536
    kv_lora: int = 512
    qk_nope: int = 128
    qk_rope: int = 64
    v_head: int = 128
    rope_theta: float = 50000.0
    rope_factor: float = 32.0
    rope_orig_len: int = 4096
    beta_fast: float = 1.0
    beta_slow: float = 1.0
    mscale_all_dim: float = 1.0
    rms_eps: float = 1e-6
    x_std: float = 1.0
    weight_std: float = 0.02
    gamma_std: float = 0.0
    rope_key_std: float = 1.7

    @property
    def tokens(self) -> int:
        return self.n_seq * self.n_new

    def weight_shapes(self) -> dict:
        H = self.n_heads
        return {"w_qa": (self.q_lora, self.d_model),
                "w_qb": (H * (self.qk_nope + self.qk_rope), self.q_lora),
                "w_kva": (self.kv_lora + self.qk_rope, self.d_model),
                "w_kvb": (H * (self.qk_nope + self.v_head), self.kv_lora),
                "w_o": (self.d_model, H * self.v_head)}


# One K2 attention layer, decode: 64 sequences of 4096 cached positions, one new
# token each (the batch of the MoE decode step).
MLA_K2_DECODE = MLAShape("mla_k2_decode", n_seq=64, n_new=1, cached=(4096,) * 64, max_len=4097)
# Prefill: 2 sequences x 4096 new positions from an empty cache (the batch of
# the MoE prefill step).
MLA_K2_PREFILL = MLAShape("mla_k2_prefill", n_seq=2, n_new=4096, cached=(0, 0), max_len=4096)


def small_mla(n_seq=3, n_new=1, cached=(0, 5, 300), max_len=320, d_model=512, n_heads=16,
              q_lora=256, **kw) -> MLAShape:
    """A small layer with the kernels' fixed head widths (latent 512, 128 + 64
    query/key features, 128 value features)."""
    return MLAShape("small_mla", n_seq=n_seq, n_new=n_new, cached=tuple(cached), max_len=max_len,
                    d_model=d_model, n_heads=n_heads, q_lora=q_lora, **kw)


@dataclass
class MLAInputs:
    shape: MLAShape
    x: torch.Tensor                 # [T, d] bf16
    norm_w: torch.Tensor            # [d] bf16
    g_qa: torch.Tensor              # [q_lora] bf16
    g_kva: torch.Tensor             # [kv_lora] bf16
    w: dict                         # name -> uint8 codes [out, in]; "s" + name[1:] -> fp32 scales
    cached_len: torch.Tensor        # [S] int32
    cache_codes: torch.Tensor       # [S, max_len, 512] uint8
    cache_scales: torch.Tensor      # [S, max_len, 4] fp32
    cache_rope: torch.Tensor        # [S, max_len, 64] bf16

    def fresh_cache(self):
        """Copies of the cache tensors (a call writes the new positions)."""
        return self.cache_codes.clone(), self.cache_scales.clone(), self.cache_rope.clone()


def _quant_rows(w: torch.Tensor):
    """[N, K] fp32 -> codes [N, K], scales [ceil(N/128), K/128]; a partial last
    row block is quantised over its own rows (zero padding leaves amax as is)."""
    n, k = w.shape
    npad = (n + 127) // 128 * 128
    if npad != n:
        w = torch.cat([w, torch.zeros((npad - n, k), dtype=w.dtype, device=w.device)])
    codes, scales = block_quantize_weight(w)
    return codes[:n].contiguous(), scales


def _gamma(shape, n, seed, idx, device):
    if shape.gamma_std == 0.0:
        return torch.ones(n, dtype=torch.bfloat16, device=device)
    return (_randn((n,), shape.gamma_std, device, seed, ROLE_MLA_NORM, idx) + 1.0).to(torch.bfloat16)


def generate_mla(shape: MLAShape, seed: int = 0, device="cpu",
                 weights_from: Optional[MLAInputs] = None) -> MLAInputs:
    """Seeded inputs for ``shape``; ``weights_from`` reuses another workload's
    weights and norm weights (same layer dimensions)."""
    assert len(shape.cached) == shape.n_seq
    assert all(c + shape.n_new <= shape.max_len for c in shape.cached)
    T, d, R = shape.tokens, shape.d_model, shape.kv_lora
    x = _randn((T, d), shape.x_std, device, seed, ROLE_MLA_X).to(torch.bfloat16)
    if weights_from is not None:
        b = weights_from.shape
        assert (b.d_model, b.n_heads, b.q_lora) == (shape.d_model, shape.n_heads, shape.q_lora)
        w, norm_w, g_qa, g_kva = (weights_from.w, weights_from.norm_w, weights_from.g_qa,
                                  weights_from.g_kva)
    else:
        w = {}
        for i, (name, shp) in enumerate(shape.weight_shapes().items()):
            full = _randn(shp, shape.weight_std, device, seed, ROLE_MLA_W, i)
            w[name], w["s" + name[1:]] = _quant_rows(full)
            del full
        norm_w = _gamma(shape, d, seed, 0, device)
        g_qa = _gamma(shape, shape.q_lora, seed, 1, device)
        g_kva = _gamma(shape, R, seed, 2, device)
    S, L = shape.n_seq, shape.max_len
    cached = torch.tensor(shape.cached, dtype=torch.int32, device=device)
    codes = torch.zeros((S, L, R), dtype=torch.uint8, device=device)
    scales = torch.ones((S, L, R // 128), dtype=torch.float32, device=device)
    rope = torch.zeros((S, L, shape.qk_rope), dtype=torch.bfloat16, device=device)
    for s_ in range(S):
        n = int(shape.cached[s_])
        if n == 0:
            continue
        c = _randn((n, R), 1.0, device, seed, ROLE_MLA_CACHE, s_, 0).to(torch.bfloat16).float()
        blk = c.view(n, R // 128, 128)
        amax = blk.abs().amax(dim=2)
        sc = torch.where(amax == 0, torch.ones_like(amax), amax / FP8_MAX)
        q = (blk / sc[:, :, None]).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
        codes[s_, :n] = q.view(torch.uint8).view(n, R)
        scales[s_, :n] = sc
        rope[s_, :n] = _randn((n, shape.qk_rope), shape.rope_key_std, device, seed, ROLE_MLA_CACHE,
                              s_, 1).to(torch.bfloat16)
    return MLAInputs(shape, x, norm_w, g_qa, g_kva, w, cached, codes, scales, rope)
