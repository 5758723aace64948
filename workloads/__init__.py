"""Seeded synthetic inputs for MLA ragged prefill and merge_state.

This module only draws random numbers and lays them out. It holds none of
the attention arithmetic, so both the HIP path and the fp64 oracle can take
their inputs from it without sharing any of the method.

Shapes follow the DeepSeek-V3/R1 MLA prefill described on the pages:
  * "[DeepseekR1] How ragged prefill manage kv_cache?" (sglang issue 3849):
    query/key head dim 192 (128 NoPE + 64 RoPE), value/output head dim 128,
    and a compressed cache of 512 latent dims plus 64 RoPE dims per token.
  * "vllm.v1.attention.backends.mla.prefill.flashinfer" (FlashInferPrefillBackend
    / finalize_attention_metadata): ragged qo_indptr / kv_indptr, NHD tensors,
    one causal pass over the new tokens and one non-causal pass per context
    chunk indexed by chunked_context.cu_seq_lens[i].

A workload is defined by its seed and by the torch device its generator runs
on: `torch.Generator(device).manual_seed(seed)`. CPU and GPU generators give
different numbers for the same seed, so a parity check always hands the very
same bytes to both sides (the oracle reads a host copy of what the GPU used).

Draw order for each named workload: lengths, then Q, K, V; the chunked-prefill
workload then draws each context chunk's K and V; the decompression workload
draws c_kv, k_rope, W_UK, W_UV, then Q.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

DQK = 192          # 128 NoPE + 64 RoPE
DVO = 128
D_NOPE = 128
D_ROPE = 64
D_LATENT = 512


def default_sm_scale() -> float:
    return DQK ** -0.5


@dataclass
class PrefillInputs:
    """One ragged prefill pass: NHD tensors plus host int32 indptrs."""
    q: torch.Tensor                    # [Tq, H, 192]
    k: torch.Tensor                    # [Tk, H, 192]
    v: torch.Tensor                    # [Tk, H, 128]
    qo_indptr: List[int]
    kv_indptr: List[int]
    num_heads: int
    causal: bool
    sm_scale: float

    @property
    def batch(self) -> int:
        return len(self.qo_indptr) - 1


@dataclass
class ChunkedInputs:
    """New tokens (causal over themselves) plus prefix context chunks."""
    main: PrefillInputs
    chunks: List[PrefillInputs] = field(default_factory=list)


@dataclass
class AbsorbedInputs:
    """Weight-absorbed MLA over the latent cache: absorbed queries and the
    shared cache rows (c_kv | k_rope)."""
    q: torch.Tensor                    # [Tq, H, 576]
    kv: torch.Tensor                   # [Tk, 576]
    qo_indptr: List[int]
    kv_indptr: List[int]
    num_heads: int
    causal: bool
    sm_scale: float


@dataclass
class DecompressInputs:
    c_kv: torch.Tensor                 # [T, 512]
    k_rope: torch.Tensor               # [T, 64]
    w_uk: torch.Tensor                 # [512, H*128]
    w_uv: torch.Tensor                 # [512, H*128]
    q: torch.Tensor                    # [T, H, 192]
    indptr: List[int]
    num_heads: int
    sm_scale: float


@dataclass
class LatentPrefillInputs:
    """A ragged prefill whose K/V come from the latent cache: c_kv, k_rope and
    the up-projections, with separate query and key lengths."""
    c_kv: torch.Tensor                 # [Tk, 512]
    k_rope: torch.Tensor               # [Tk, 64]
    w_uk: torch.Tensor                 # [512, H*128]
    w_uv: torch.Tensor                 # [512, H*128]
    q: torch.Tensor                    # [Tq, H, 192]
    qo_indptr: List[int]
    kv_indptr: List[int]
    num_heads: int
    causal: bool
    sm_scale: float


def indptr_from_lengths(lengths) -> List[int]:
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn(shape, gen: torch.Generator, dtype: torch.dtype, device, std: float = 1.0,
          chunk_elems: int = 1 << 28) -> torch.Tensor:
    """N(0, std^2) drawn in fp32 and rounded to `dtype` (round-to-nearest-even
    for bf16), filled in slices so the fp32 temporary stays bounded."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    pos = 0
    while pos < n:
        m = min(chunk_elems, n - pos)
        t = torch.randn(m, generator=gen, dtype=torch.float32, device=device)
        if std != 1.0:
            t.mul_(std)
        flat[pos:pos + m].copy_(t)
        pos += m
    return out


def ragged_inputs(lengths_q, lengths_kv, num_heads: int, dtype: torch.dtype, seed: int,
                  causal: bool = True, device="cpu", sm_scale: Optional[float] = None,
                  gen: Optional[torch.Generator] = None) -> PrefillInputs:
    """Q, K, V ~ N(0,1) for a ragged batch with the given per-sequence lengths."""
    g = gen if gen is not None else _gen(seed, device)
    qo = indptr_from_lengths(lengths_q)
    kv = indptr_from_lengths(lengths_kv)
    q = randn((qo[-1], num_heads, DQK), g, dtype, device)
    k = randn((kv[-1], num_heads, DQK), g, dtype, device)
    v = randn((kv[-1], num_heads, DVO), g, dtype, device)
    return PrefillInputs(q, k, v, qo, kv, num_heads, causal,
                         default_sm_scale() if sm_scale is None else sm_scale)


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def tiny_fp32(device="cpu") -> PrefillInputs:
    """3 sequences of lengths 1, 17, 64 (qo = kv), 4 heads, fp32, causal, seed 1."""
    return ragged_inputs([1, 17, 64], [1, 17, 64], 4, torch.float32, seed=1,
                         causal=True, device=device)


def deepseek_v3_lengths(seed: int = 2) -> List[int]:
    g = _gen(seed, "cpu")
    return [int(x) for x in torch.randint(256, 4097, (16,), generator=g)]


def deepseek_v3_batch(device="cpu", num_heads: int = 128) -> PrefillInputs:
    """16 sequences, qo = kv ~ U[256, 4096], 128 heads, bf16, causal, seed 2.

    The lengths are drawn on a CPU generator so they are the same on every
    device; the tensors are drawn on `device`."""
    lens = deepseek_v3_lengths(2)
    g = _gen(2, device)
    return ragged_inputs(lens, lens, num_heads, torch.bfloat16, seed=2, causal=True,
                         device=device, gen=g)


def chunked_prefill(device="cpu", num_requests: int = 8, new_tokens: int = 2048,
                    prefix: int = 8192, num_chunks: int = 2, num_heads: int = 128,
                    dtype=torch.bfloat16, seed: int = 3) -> ChunkedInputs:
    """New tokens attend causally to themselves; the prefix is split into
    `num_chunks` context chunks attended non-causally; seed 3."""
    g = _gen(seed, device)
    lens = [new_tokens] * num_requests
    main = ragged_inputs(lens, lens, num_heads, dtype, seed, causal=True, device=device, gen=g)
    per_chunk = prefix // num_chunks
    chunks = []
    for _ in range(num_chunks):
        kv = indptr_from_lengths([per_chunk] * num_requests)
        k = randn((kv[-1], num_heads, DQK), g, dtype, device)
        v = randn((kv[-1], num_heads, DVO), g, dtype, device)
        chunks.append(PrefillInputs(main.q, k, v, main.qo_indptr, kv, num_heads, False,
                                    main.sm_scale))
    return ChunkedInputs(main, chunks)


def skewed_lengths(seed: int = 4, n: int = 64, lo: int = 16, hi: int = 32768,
                   cap: int = 262144) -> List[int]:
    """Log-uniform lengths on [lo, hi], total capped at `cap`.

    Cap rule: if the sum exceeds the cap, scale every length by cap/sum,
    floor, clamp to >= lo, then take any remaining excess off the longest."""
    g = _gen(seed, "cpu")
    u = torch.rand(n, generator=g, dtype=torch.float64)
    lens = [int(math.floor(math.exp(math.log(lo) + float(x) * (math.log(hi) - math.log(lo)))))
            for x in u]
    lens = [min(max(x, lo), hi) for x in lens]
    total = sum(lens)
    if total > cap:
        f = cap / total
        lens = [max(lo, int(math.floor(x * f))) for x in lens]
        excess = sum(lens) - cap
        while excess > 0:
            i = max(range(n), key=lambda j: lens[j])
            take = min(excess, lens[i] - lo)
            lens[i] -= take
            excess -= take
    return lens


def skewed_batch(device="cpu", num_heads: int = 128) -> PrefillInputs:
    lens = skewed_lengths(4)
    g = _gen(4, device)
    return ragged_inputs(lens, lens, num_heads, torch.bfloat16, seed=4, causal=True,
                         device=device, gen=g)


def decompress_batch(device="cpu", num_seqs: int = 8, seq_len: int = 4096,
                     num_heads: int = 128, seed: int = 5) -> DecompressInputs:
    """Latent cache c_kv [T,512], shared k_rope [T,64], W_UK/W_UV [512, H*128]
    ~ N(0, 1/512), then Q [T,H,192]; all bf16; seed 5."""
    g = _gen(seed, device)
    t = num_seqs * seq_len
    bf = torch.bfloat16
    c_kv = randn((t, D_LATENT), g, bf, device)
    k_rope = randn((t, D_ROPE), g, bf, device)
    std = 1.0 / math.sqrt(D_LATENT)
    w_uk = randn((D_LATENT, num_heads * D_NOPE), g, bf, device, std=std)
    w_uv = randn((D_LATENT, num_heads * DVO), g, bf, device, std=std)
    q = randn((t, num_heads, DQK), g, bf, device)
    return DecompressInputs(c_kv, k_rope, w_uk, w_uv, q,
                            indptr_from_lengths([seq_len] * num_seqs), num_heads,
                            default_sm_scale())


def latent_prefill_inputs(lengths_q, lengths_kv, num_heads: int, seed: int, causal: bool = True,
                          device="cpu") -> LatentPrefillInputs:
    """The decompression workload's distributions (c_kv, k_rope ~ N(0,1),
    W_UK, W_UV ~ N(0, 1/512), Q ~ N(0,1), all bf16, drawn in that order) for
    a ragged batch with separate query and key lengths."""
    g = _gen(seed, device)
    qo = indptr_from_lengths(lengths_q)
    kv = indptr_from_lengths(lengths_kv)
    bf = torch.bfloat16
    c_kv = randn((kv[-1], D_LATENT), g, bf, device)
    k_rope = randn((kv[-1], D_ROPE), g, bf, device)
    std = 1.0 / math.sqrt(D_LATENT)
    w_uk = randn((D_LATENT, num_heads * D_NOPE), g, bf, device, std=std)
    w_uv = randn((D_LATENT, num_heads * DVO), g, bf, device, std=std)
    q = randn((qo[-1], num_heads, DQK), g, bf, device)
    return LatentPrefillInputs(c_kv, k_rope, w_uk, w_uv, q, qo, kv, num_heads, causal,
                               default_sm_scale())


def absorbed_inputs(lengths_q, lengths_kv, num_heads: int, seed: int, causal: bool = True,
                    device="cpu", sm_scale: Optional[float] = None) -> AbsorbedInputs:
    """Absorbed queries q [Tq,H,576] and latent cache rows kv [Tk,576], both
    N(0,1) rounded to bf16; drawn in that order. The score scale defaults
    to 1/sqrt(192), the head dim the absorbed scores stand in for."""
    g = _gen(seed, device)
    qo = indptr_from_lengths(lengths_q)
    kv = indptr_from_lengths(lengths_kv)
    dk = D_LATENT + D_ROPE
    q = randn((qo[-1], num_heads, dk), g, torch.bfloat16, device)
    c = randn((kv[-1], dk), g, torch.bfloat16, device)
    return AbsorbedInputs(q, c, qo, kv, num_heads, causal,
                          default_sm_scale() if sm_scale is None else sm_scale)


def absorbed_batch(device="cpu", num_heads: int = 128) -> AbsorbedInputs:
    """The DeepSeek-V3 batch lengths (16 seqs U[256,4096], seed 2) through the
    absorbed path: causal, bf16, seed 6."""
    lens = deepseek_v3_lengths()
    return absorbed_inputs(lens, lens, num_heads, seed=6, causal=True, device=device)


def merge_inputs(num_tokens: int, num_heads: int, dtype: torch.dtype, seed: int,
                 device="cpu", neg_inf_frac: float = 0.0):
    """Two (O, LSE) partial states. O ~ N(0,1); LSE ~ N(0, 4) so the two weights
    vary widely. A fraction of rows gets LSE = -inf on one or both sides (an
    empty key split), chosen by a seeded draw."""
    g = _gen(seed, device)
    o_a = randn((num_tokens, num_heads, DVO), g, dtype, device)
    o_b = randn((num_tokens, num_heads, DVO), g, dtype, device)
    lse_a = randn((num_tokens, num_heads), g, torch.float32, device, std=2.0)
    lse_b = randn((num_tokens, num_heads), g, torch.float32, device, std=2.0)
    if neg_inf_frac > 0:
        sel = torch.rand((num_tokens, num_heads), generator=g, device=device)
        lse_a[sel < neg_inf_frac / 3] = float("-inf")
        lse_b[(sel >= neg_inf_frac / 3) & (sel < 2 * neg_inf_frac / 3)] = float("-inf")
        both = (sel >= 2 * neg_inf_frac / 3) & (sel < neg_inf_frac)
        lse_a[both] = float("-inf")
        lse_b[both] = float("-inf")
        # an empty split leaves O = 0 on that side
        o_a[torch.isinf(lse_a)] = 0
        o_b[torch.isinf(lse_b)] = 0
    return o_a, lse_a, o_b, lse_b


WORKLOADS = {
    "tiny_fp32": "3 seqs {1,17,64}, 4 heads, fp32, causal",
    "deepseek_v3_batch": "16 seqs U[256,4096], 128 heads, bf16, causal",
    "chunked_prefill": "8 x (2048 new causal + 2 x 4096 context non-causal), 128 heads, bf16, merged",
    "skewed_batch": "64 seqs log-uniform [16,32768], total <= 262144, 128 heads, bf16, causal",
    "decompress_batch": "8 x 4096 tokens, latent 512 -> 128 heads via W_UK/W_UV, then causal prefill",
    "absorbed_batch": "16 seqs U[256,4096] (seed 2), 128 heads, absorbed q [T,H,576] over kv [T,576], bf16, causal",
}
