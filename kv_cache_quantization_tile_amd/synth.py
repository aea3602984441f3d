"""Seeded synthetic KV-cache workloads.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic, so the CPU oracle and the HIP path can both be fed from it.

The workloads stand in for the pages' own measurement (a Qwen3-32B-class model serving
long-context bursts, README "Quick start" and intro): same attention shape (64 query heads,
8 KV heads, head_dim 128, float16) and the same context lengths, synthetic values.

Every generator takes a torch device; large workloads are drawn directly on the GPU.
The same seed gives different numbers on different devices, so a caller that compares two
implementations copies one draw to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

HEAD_DIM = 128
TILE = 128


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _student_t(shape, nu: float, g, device):
    """Student-t(nu) = Z / sqrt(W / nu) with W ~ chi^2(nu) = 2 Gamma(nu / 2)."""
    z = _randn(shape, g, device)
    alpha = torch.full(shape, nu / 2.0, device=device, dtype=torch.float32)
    w = 2.0 * torch._standard_gamma(alpha, generator=g)
    return z / torch.sqrt(w / nu)


def _lognormal(n, sigma, g, device):
    return torch.empty(n, device=device, dtype=torch.float32).log_normal_(0.0, sigma, generator=g)


def _outlier_channels(n_out, g, device):
    return torch.randperm(HEAD_DIM, generator=g, device=device)[:n_out]


def round_to_tile(length: float) -> int:
    """128 * round(length / 128), ties rounded up."""
    return TILE * int(math.floor(length / TILE + 0.5))


@dataclass
class Workload:
    """A paged KV workload: prompt tokens to quantize, a block table, decode steps.

    k_src / v_src: [T_total, Hkv, 128] float16, the prompt tokens of all sequences
    concatenated (sequence b starts at token seq_start[b]).
    Full prompt tiles are listed in tile_src_token (first source token of the tile) and
    tile_dst_page (page id); page p of sequence b is block_table[b, p].
    """
    name: str
    hq: int
    hkv: int
    k_src: torch.Tensor
    v_src: torch.Tensor
    seq_start: list
    prompt_lens: list
    block_table: torch.Tensor          # int32 [B, max_pages]
    num_pages: int                     # pages allocated for prompts
    free_pages: list                   # page ids left for tiles filled during decode
    tile_src_token: torch.Tensor       # int64 [n_tiles]
    tile_dst_page: torch.Tensor        # int32 [n_tiles]
    n_iters: int = 8
    decode_steps: int = 1
    append: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.prompt_lens)

    def step_inputs(self, step: int, device=None):
        """Query (and appended token) of decode step `step`, drawn from its own seed."""
        device = device or self.k_src.device
        g = _gen(self.seed * 1000 + 17 + step, device)
        q = _randn((self.batch, self.hq, HEAD_DIM), g, device).to(torch.float16)
        if not self.append:
            return q, None, None
        kn = self._token_dist("k", (self.batch, self.hkv, HEAD_DIM), g, device)
        vn = self._token_dist("v", (self.batch, self.hkv, HEAD_DIM), g, device)
        return q, kn.to(torch.float16), vn.to(torch.float16)

    def _token_dist(self, which, shape, g, device):
        dist = self.extra.get("dist", "normal")
        if dist == "t3":
            return _student_t(shape, 3.0, g, device)
        if dist == "cfg4":
            x = _randn(shape, g, device)
            if which == "k":
                x = x * self.extra["k_chan_scale"].to(device)[None]
            return x
        return _randn(shape, g, device)


def _paged(name, hq, hkv, k_src, v_src, lens, g, device, permute_pages, spare_per_seq,
           **kw) -> Workload:
    """Lay prompts out in pages: sequence b's full prompt tiles get the next page ids of a
    (optionally random) permutation of all pages; `spare_per_seq` pages per sequence are
    kept free for tiles that fill during decode."""
    starts, s = [], 0
    for L in lens:
        starts.append(s)
        s += L
    n_prompt_pages = sum(L // TILE for L in lens)
    total_pages = n_prompt_pages + spare_per_seq * len(lens)
    if permute_pages:
        order = torch.randperm(total_pages, generator=g, device=device).cpu().tolist()
    else:
        order = list(range(total_pages))
    width = max(L // TILE for L in lens) + spare_per_seq + 1
    bt = torch.full((len(lens), width), -1, dtype=torch.int32)
    src_tok, dst_page = [], []
    nxt = 0
    for b, L in enumerate(lens):
        for p in range(L // TILE):
            bt[b, p] = order[nxt]
            src_tok.append(starts[b] + p * TILE)
            dst_page.append(order[nxt])
            nxt += 1
    return Workload(name=name, hq=hq, hkv=hkv, k_src=k_src, v_src=v_src, seq_start=starts,
                    prompt_lens=list(lens), block_table=bt.to(device), num_pages=total_pages,
                    free_pages=order[nxt:],
                    tile_src_token=torch.tensor(src_tok, dtype=torch.int64, device=device),
                    tile_dst_page=torch.tensor(dst_page, dtype=torch.int32, device=device),
                    **kw)


def single_tile(device="cpu", seed: int = 0) -> Workload:
    """One KV head, one 128-token tile; K and V N(0,1) with 4 outlier channels x20 each;
    one N(0,1) query; 8 Sinkhorn iterations.

    Draw order: K values, K outlier channels, V values, V outlier channels, query.
    """
    g = _gen(seed, device)
    k = _randn((TILE, HEAD_DIM), g, device)
    k[:, _outlier_channels(4, g, device)] *= 20.0
    v = _randn((TILE, HEAD_DIM), g, device)
    v[:, _outlier_channels(4, g, device)] *= 20.0
    q = _randn((1, 1, HEAD_DIM), g, device)
    w = _paged("single_tile", 1, 1, k.to(torch.float16)[:, None, :],
               v.to(torch.float16)[:, None, :], [TILE], g, device, False, 0,
               n_iters=8, decode_steps=1, seed=seed)
    w.extra["q0"] = q.to(torch.float16)
    return w


def _magnitude_channels(tokens, hkv, g, device, sigma, n_out, mult):
    """Per (KV head): channel magnitudes lognormal(0, sigma), n_out outlier channels x mult,
    times N(0,1) values."""
    out = torch.empty((tokens, hkv, HEAD_DIM), dtype=torch.float16, device=device)
    for h in range(hkv):
        mag = _lognormal(HEAD_DIM, sigma, g, device)
        mag[_outlier_channels(n_out, g, device)] *= mult
        out[:, h, :] = (_randn((tokens, HEAD_DIM), g, device) * mag[None, :]).to(torch.float16)
    return out


def one_layer(device="cpu", seed: int = 1, context: int = 16384) -> Workload:
    """One decoder layer with Qwen3-32B-like GQA: 64 query / 8 KV heads, batch 1, 16384
    tokens; per (KV head, tensor) channel magnitudes lognormal(0,1), 2% (3) outlier channels
    x10, times N(0,1); contiguous pages; one decode step (no append)."""
    g = _gen(seed, device)
    k = _magnitude_channels(context, 8, g, device, 1.0, 3, 10.0)
    v = _magnitude_channels(context, 8, g, device, 1.0, 3, 10.0)
    return _paged("one_layer_16k", 64, 8, k, v, [context], g, device, False, 0,
                  n_iters=8, decode_steps=1, seed=seed)


def uneven_tokens(device="cpu", seed: int = 5, context: int = 4096, hkv: int = 8,
                  sigma: float = 1.0) -> Workload:
    """Channel structure of `one_layer` (lognormal(0,1) channel magnitudes, 3 outlier channels
    x10) times per-token magnitudes lognormal(0, sigma): a cache whose token scales are
    uneven. 8 query heads per KV head, batch 1, contiguous pages, one decode step."""
    g = _gen(seed, device)
    k = _magnitude_channels(context, hkv, g, device, 1.0, 3, 10.0)
    v = _magnitude_channels(context, hkv, g, device, 1.0, 3, 10.0)
    for dst in (k, v):
        tok = _lognormal(context * hkv, sigma, g, device).view(context, hkv, 1)
        dst.copy_((dst.float() * tok).to(torch.float16))
    return _paged("uneven_tokens", 8 * hkv, hkv, k, v, [context], g, device, False, 0,
                  n_iters=8, decode_steps=1, seed=seed)


def batched_paged(device="cpu", seed: int = 2, batch: int = 32, lo: int = 4096,
                  hi: int = 32768, steps: int = 16, lens=None) -> Workload:
    """Batched paged decode: context lengths uniform in [lo, hi] rounded to 128, pages
    placed by a random permutation, K/V Student-t(3); `steps` decode steps that append one
    token per sequence into an fp16 staging tile (quantized each time it fills)."""
    g = _gen(seed, device)
    if lens is None:
        u = torch.rand(batch, generator=g, device=device, dtype=torch.float64).cpu()
        lens = [round_to_tile(lo + (hi - lo) * float(x)) for x in u]
    T = sum(lens)
    k = _student_t((T, 8, HEAD_DIM), 3.0, g, device).to(torch.float16)
    v = _student_t((T, 8, HEAD_DIM), 3.0, g, device).to(torch.float16)
    spare = steps // TILE + 1
    return _paged("batched_paged", 64, 8, k, v, lens, g, device, True, spare,
                  n_iters=8, decode_steps=steps, append=True, seed=seed,
                  extra={"dist": "t3"})


def long_context(device="cpu", seed: int = 3, context: int = 131072, steps: int = 64) -> Workload:
    """Batch 1, 131072 tokens, 64 / 8 heads; K with per-channel lognormal(0,1.5) scales and
    1% (1) outlier channel x50 per KV head, V N(0,1); `steps` decode steps with append."""
    g = _gen(seed, device)
    kscale = torch.empty((8, HEAD_DIM), dtype=torch.float32, device=device)
    for h in range(8):
        mag = _lognormal(HEAD_DIM, 1.5, g, device)
        mag[_outlier_channels(1, g, device)] *= 50.0
        kscale[h] = mag
    k = (_randn((context, 8, HEAD_DIM), g, device) * kscale[None]).to(torch.float16)
    v = _randn((context, 8, HEAD_DIM), g, device).to(torch.float16)
    spare = steps // TILE + 1
    return _paged("long_context_128k", 64, 8, k, v, [context], g, device, False, spare,
                  n_iters=8, decode_steps=steps, append=True, seed=seed,
                  extra={"dist": "cfg4", "k_chan_scale": kscale})


def prefill_burst(device="cpu", seed: int = 4, batch: int = 64, context: int = 16384,
                  n_iters: int = 8) -> Workload:
    """64 sequences x 16384 tokens, 8 KV heads; even KV heads N(0,1), odd KV heads
    Student-t(2.5), for K and V; then one batched decode step (no append)."""
    g = _gen(seed, device)
    T = batch * context
    k = torch.empty((T, 8, HEAD_DIM), dtype=torch.float16, device=device)
    v = torch.empty((T, 8, HEAD_DIM), dtype=torch.float16, device=device)
    for h in range(8):
        for dst in (k, v):
            if h % 2 == 0:
                dst[:, h, :] = _randn((T, HEAD_DIM), g, device).to(torch.float16)
            else:
                dst[:, h, :] = _student_t((T, HEAD_DIM), 2.5, g, device).to(torch.float16)
    return _paged("prefill_burst", 64, 8, k, v, [context] * batch, g, device, False, 0,
                  n_iters=n_iters, decode_steps=1, seed=seed)


def tile_batch(n_tiles: int, device="cpu", seed: int = 11, dist: str = "mixed", return_kinds=False):
    """[n_tiles, 128 tokens, 128 channels] float16 tiles for quantizer tests; with
    dist == 'mixed' a rotation of N(0,1), Student-t(3), lognormal channel magnitudes with
    outlier channels, a large offset with small noise, large magnitudes, and N(0,1)."""
    g = _gen(seed, device)
    x = _randn((n_tiles, TILE, HEAD_DIM), g, device)
    if dist == "mixed":
        for i in range(n_tiles):
            kind = i % 6
            if kind == 1:
                x[i] = _student_t((TILE, HEAD_DIM), 3.0, g, device)
            elif kind == 2:
                mag = _lognormal(HEAD_DIM, 1.0, g, device)
                mag[_outlier_channels(3, g, device)] *= 10.0
                x[i] = x[i] * mag[None, :]
            elif kind == 3:
                x[i] = x[i] * 0.05 + 5.0
            elif kind == 4:
                x[i] = x[i] * 300.0
    kinds = [i % 6 if dist == "mixed" else 0 for i in range(n_tiles)]
    return (x.to(torch.float16), kinds) if return_kinds else x.to(torch.float16)


# tile_batch kind whose rotated channel 0 is a large offset over small noise: the stage-3
# normalization is ill-conditioned on it (near-constant rows after the first column step)
OFFSET_TILE_KIND = 3
