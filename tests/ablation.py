"""Error ablation of the KVarN quantizer on synthetic caches: an experiment, not a parity test.

What each stage of the method buys, measured on the seeded synthetic workloads:

* one step: relative error of the dequantized keys and values, and of the attention output
  against exact float64 attention over the float16 cache, for the quantizer with and without
  the channel rotation ([README] "How KVarN works", stage 2) and with 0 to 8 normalization
  iterations (stage 3);
* token scales: the relative error of each cached token's magnitude, | ||x_hat_t|| / ||x_t|| - 1 |,
  the quantity [hypho] ("the paper's core finding") names as the driver of error accumulation
  over decode steps;
* many steps: a toy autoregressive loop. Each step's attention output feeds (weakly) the next
  query and fully the next appended key / value token. It runs once on the exact cache and
  once on a quantized one. The divergence of the two trajectories stands in for that error
  accumulation. There is no model here: the loop's maps are fixed random rotations, so only
  the propagation of cache error is modelled.

The oracle supplies every variant (float64). With --gpu, the HIP kernels supply the variants
the method itself covers (rotation on, N = 0 .. 8) through the C ABI.

Test infrastructure (it imports the oracle): run as `python -m tests.ablation [--gpu]`.
"""
from __future__ import annotations

import argparse
import json
import math
import time

import numpy as np

from oracle import kvarn_oracle as O

SOFTMAX_SCALE = 1.0 / math.sqrt(128.0)

# (label, channel rotation, normalization iterations, key bits, value bits, group size); the
# last rows are the other presets' code widths (kvarn_k2v2_g128, kvarn_k4v4_g128) and group
# size 64 (kvarn_k4v2_g64, kvarn_k2v2_g64) at N = 8
VARIANTS = (
    ("RTN only", False, 0, 4, 2, 128),
    ("rotation + RTN", True, 0, 4, 2, 128),
    ("normalization (N=8) + RTN", False, 8, 4, 2, 128),
    ("KVarN N=1", True, 1, 4, 2, 128),
    ("KVarN N=2", True, 2, 4, 2, 128),
    ("KVarN N=4", True, 4, 4, 2, 128),
    ("KVarN N=8", True, 8, 4, 2, 128),
    ("KVarN N=8, k2v2", True, 8, 2, 2, 128),
    ("KVarN N=8, k4v4", True, 8, 4, 4, 128),
    ("KVarN N=8, g64", True, 8, 4, 2, 64),
    ("KVarN N=8, k2v2 g64", True, 8, 2, 2, 64),
)


def dequantized(x_tc: np.ndarray, kind: int, rotate: bool, n_iters: int, k_bits: int = 4,
                v_bits: int = 2, group: int = 128) -> np.ndarray:
    """x_tc: [T, 128] float16 tokens of one KV head, T a multiple of 128. Returns the oracle's
    quantized-then-dequantized tokens [T, 128], float64."""
    t = x_tc.shape[0]
    tiles = np.asarray(x_tc, np.float16).reshape(t // 128, 128, 128)      # [tile, token, channel]
    x = np.swapaxes(tiles, -1, -2)                                         # channels x tokens
    d = O.quantize_tiles(x, kind, n_iters, rotate_channels=rotate, k_bits=k_bits, v_bits=v_bits,
                         group=group)
    xh = O.dequantize_tiles(d["codes"], d["r"], d["s"], d["scale"], d["zero"], kind,
                            rotate_channels=rotate, group=group)
    return np.swapaxes(xh, -1, -2).reshape(t, 128)


def attention_heads(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Softmax attention of query rows q [G, 128] over k, v [T, 128], float64."""
    z = SOFTMAX_SCALE * (q @ k.T)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def row_rel_err(a: np.ndarray, b: np.ndarray) -> float:
    """Mean over rows of ||a - b|| / ||b||."""
    return float(np.mean(np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)))


def frob_rel_err(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def caches(k: np.ndarray, v: np.ndarray, variants=VARIANTS) -> dict:
    """Dequantized prompt caches per variant: {label: (k_hat, v_hat)}, each [T, Hkv, 128]."""
    out = {}
    for label, rot, n, kb, vb, gs in variants:
        kh = np.stack([dequantized(k[:, g], O.KIND_K, rot, n, kb, vb, gs) for g in range(k.shape[1])], 1)
        vh = np.stack([dequantized(v[:, g], O.KIND_V, rot, n, kb, vb, gs) for g in range(v.shape[1])], 1)
        out[label] = (kh, vh)
    return out


def token_scale_err(xh: np.ndarray, x: np.ndarray) -> float:
    """Mean over tokens (and KV heads) of | ||xh_t|| / ||x_t|| - 1 |; x, xh [T, Hkv, 128]."""
    n = np.linalg.norm(x, axis=-1)
    ok = n > 0
    return float(np.mean(np.abs(np.linalg.norm(xh, axis=-1)[ok] / n[ok] - 1.0)))


def grouped_queries(q_sets: np.ndarray) -> np.ndarray:
    """[S, Hq, 128] query sets -> [Hq * S, 128] rows ordered by KV head (8 query heads per KV
    head), so that the rows of KV head g are [g * 8 S, (g + 1) * 8 S)."""
    s_, hq, _ = q_sets.shape
    hkv = hq // 8
    return np.ascontiguousarray(q_sets.reshape(s_, hkv, 8, 128).transpose(1, 0, 2, 3)).reshape(-1, 128)


def single_step(k: np.ndarray, v: np.ndarray, q: np.ndarray, cache: dict) -> dict:
    """k, v: [T, Hkv, 128] float16 prompt; q: [R, 128] float16 query rows, R / Hkv consecutive
    rows per KV head (grouped_queries); cache from caches().
    Returns {label: {"k", "v", "attn", "k_tok", "v_tok"}}: relative errors of K and V
    (Frobenius per KV head, averaged), of the attention output (per query head, averaged) and
    of the token magnitudes (token_scale_err)."""
    hkv = k.shape[1]
    g_sz = q.shape[0] // hkv
    kf, vf, qf = (np.asarray(a, np.float16).astype(np.float64) for a in (k, v, q))
    exact = [attention_heads(qf[g * g_sz:(g + 1) * g_sz], kf[:, g], vf[:, g]) for g in range(hkv)]
    out = {}
    for label, (kh, vh) in cache.items():
        ek = np.mean([frob_rel_err(kh[:, g], kf[:, g]) for g in range(hkv)])
        ev = np.mean([frob_rel_err(vh[:, g], vf[:, g]) for g in range(hkv)])
        ea = np.mean([row_rel_err(attention_heads(qf[g * g_sz:(g + 1) * g_sz], kh[:, g], vh[:, g]),
                                  exact[g]) for g in range(hkv)])
        out[label] = {"k": float(ek), "v": float(ev), "attn": float(ea),
                      "k_tok": token_scale_err(kh, kf), "v_tok": token_scale_err(vh, vf)}
    return out


class ToyLoop:
    """The toy autoregressive loop. Per step, with o the attention output per query head:
      next query  q = sqrt(1 - a^2) xi + a sqrt(128) unit(Rq o), xi ~ N(0, 1) shared by both
      runs, a = FEEDBACK (weak, so that the loop itself does not amplify differences);
      appended key and value of KV head g, with u = mean of o over g's query heads:
      k = sk (.) sqrt(128) unit(Rk u), v = sv (.) sqrt(128) unit(Rv u), sk, sv the prompt's
      per-channel standard deviations; all rounded to float16 as a cache would hold them.
    Rq, Rk, Rv are fixed random orthogonal matrices."""

    FEEDBACK = 0.25

    def __init__(self, k: np.ndarray, v: np.ndarray, seed: int):
        rng = np.random.default_rng(seed)
        self.rq, self.rk, self.rv = (np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(3))
        kf = np.asarray(k, np.float16).astype(np.float64)
        vf = np.asarray(v, np.float16).astype(np.float64)
        self.sk = kf.std(axis=0)        # [Hkv, 128]
        self.sv = vf.std(axis=0)
        self.noise_seed = seed + 1

    @staticmethod
    def _unit(x):
        return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-300)

    def next_inputs(self, o: np.ndarray, xi: np.ndarray):
        """o: [Hq, 128] attention output -> (q [Hq,128], k_new [Hkv,128], v_new [Hkv,128]),
        float16-rounded float64."""
        hkv = self.sk.shape[0]
        r128 = math.sqrt(128.0)
        a = self.FEEDBACK
        q = math.sqrt(1.0 - a * a) * xi + a * r128 * self._unit(o @ self.rq.T)
        u = o.reshape(hkv, -1, 128).mean(axis=1)
        kn = self.sk * r128 * self._unit(u @ self.rk.T)
        vn = self.sv * r128 * self._unit(u @ self.rv.T)
        f16 = lambda a: a.astype(np.float16).astype(np.float64)
        return f16(q), f16(kn), f16(vn)

    def noises(self, steps: int, hq: int):
        rng = np.random.default_rng(self.noise_seed)
        return [rng.standard_normal((hq, 128)) for _ in range(steps)]


def _attend_all(q, ks, vs, g_sz):
    """q [Hq,128]; ks, vs [T, Hkv, 128] -> o [Hq, 128]."""
    hkv = ks.shape[1]
    return np.concatenate([attention_heads(q[g * g_sz:(g + 1) * g_sz], ks[:, g], vs[:, g])
                           for g in range(hkv)], 0)


def divergence(k, v, q0, cache: dict, steps: int, seed: int = 7) -> dict:
    """Runs the toy loop on the exact prompt and on each cache variant for `steps` steps
    (appended tokens stay float16, as in a staging tile). Returns {label: [d_0 .. d_{steps-1}]},
    d_s = mean over query heads of ||o_quant - o_exact|| / ||o_exact|| at step s."""
    loop = ToyLoop(k, v, seed)
    hq, hkv = q0.shape[0], k.shape[1]
    g_sz = hq // hkv
    kf, vf = (np.asarray(a, np.float16).astype(np.float64) for a in (k, v))
    xis = loop.noises(steps, hq)
    # exact trajectory
    ke, ve, q = kf, vf, np.asarray(q0, np.float16).astype(np.float64)
    exact = []
    for s in range(steps):
        o = _attend_all(q, ke, ve, g_sz)
        exact.append(o)
        q, kn, vn = loop.next_inputs(o, xis[s])
        ke = np.concatenate([ke, kn[None]], 0)
        ve = np.concatenate([ve, vn[None]], 0)
    out = {}
    for label, (kh, vh) in cache.items():
        kq, vq, q = kh, vh, np.asarray(q0, np.float16).astype(np.float64)
        d = []
        for s in range(steps):
            o = _attend_all(q, kq, vq, g_sz)
            d.append(row_rel_err(o, exact[s]))
            q, kn, vn = loop.next_inputs(o, xis[s])
            kq = np.concatenate([kq, kn[None]], 0)
            vq = np.concatenate([vq, vn[None]], 0)
        out[label] = d
    return out


# ----------------------------------------------------------------------------- HIP kernels

def _exact_attention_torch(q, k, v, g_sz):
    """q [B, Hq, 128], k, v [T, Hkv, 128] (one sequence per b: k[b]) -> [B, Hq, 128] float64."""
    import torch
    hkv = k.shape[1]
    qq = q.double().view(q.shape[0], hkv, g_sz, 128)
    z = SOFTMAX_SCALE * torch.einsum("bgjc,tgc->bgjt", qq, k.double())
    p = torch.softmax(z, dim=-1)
    return torch.einsum("bgjt,tgc->bgjc", p, v.double()).reshape(q.shape[0], -1, 128)


def kernel_attn_errors(k, v, q_sets, n_list=(0, 1, 2, 4, 8)) -> dict:
    """The HIP kernels (kvarn_quantize_kv_tiles + kvarn_decode_attention through the C ABI) on
    one cache: k, v [T, Hkv, 128] float16 torch tensors on the GPU (T a multiple of 128),
    q_sets [S, Hq, 128] (decoded as S sequences sharing the cache's pages). Returns
    {"KVarN N=n": mean attention rel err against exact float64 attention}."""
    import torch
    from kv_cache_quantization_tile_amd import kvarn as K
    dev = k.device
    T, hkv = k.shape[0], k.shape[1]
    n_t = T // 128
    S = q_sets.shape[0]
    g_sz = q_sets.shape[1] // hkv
    q1 = q_sets.to(torch.float16).contiguous()
    exact = _exact_attention_torch(q1, k, v, g_sz)
    tok = torch.arange(n_t, dtype=torch.int64, device=dev) * 128
    page = torch.arange(n_t, dtype=torch.int32, device=dev)
    bt = page.view(1, n_t).repeat(S, 1).contiguous()
    sl = torch.full((S,), T, dtype=torch.int32, device=dev)
    out = {}
    for n in n_list:
        params = K.params_from_dtype("kvarn_k4v2_g128", n)
        kp = K.new_pool(n_t, hkv, K.KIND_K)
        vp = K.new_pool(n_t, hkv, K.KIND_V)
        K.quantize_kv_tiles(params, k.contiguous(), v.contiguous(), tok, page, kp, vp)
        o = K.decode_attention(params, q1, kp, vp, bt, sl, T).double()
        torch.cuda.synchronize()
        out[f"KVarN N={n}"] = ((o - exact).norm(dim=-1) / exact.norm(dim=-1)).mean().item()
    return out


# ----------------------------------------------------------------------------- report

def _table(rows: dict, cols) -> str:
    head = "| variant | " + " | ".join(c for c, _ in cols) + " |\n|---|" + "---|" * len(cols) + "\n"
    body = "".join(f"| {label} | " + " | ".join(f(v) for _, f in cols) + " |\n" for label, v in rows.items())
    return head + body


def main(argv=None):
    from kv_cache_quantization_tile_amd import synth
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--tokens", type=int, default=2048, help="prompt tokens per workload (oracle part)")
    ap.add_argument("--kv-heads", type=int, default=2, help="KV heads per workload (oracle part)")
    ap.add_argument("--steps", type=int, default=64, help="toy loop steps")
    ap.add_argument("--query-sets", type=int, default=8, help="query sets (8 rows per KV head each)")
    ap.add_argument("--gpu", action="store_true", help="also run the kernels at full size")
    ap.add_argument("--out", default=None, help="write the results as JSON here")
    args = ap.parse_args(argv)
    t0 = time.perf_counter()
    res = {}
    makers = {
        "one_layer (channel outliers x10)": lambda: synth.one_layer("cpu", context=args.tokens),
        "long_context keys (lognormal(0,1.5) + outlier x50)": lambda: synth.long_context("cpu", context=args.tokens),
        "uneven token scales (lognormal(0,1) per token)": lambda: synth.uneven_tokens("cpu", context=args.tokens),
        "Student-t(3)": lambda: synth.batched_paged("cpu", batch=1, lens=[args.tokens]),
    }
    for name, make in makers.items():
        w = make()
        k = w.k_src[:, :args.kv_heads].numpy()
        v = w.v_src[:, :args.kv_heads].numpy()
        q_sets = np.stack([w.step_inputs(i, "cpu")[0][0, :8 * args.kv_heads].numpy()
                           for i in range(args.query_sets)])
        cache = caches(k, v)
        one = single_step(k, v, grouped_queries(q_sets), cache)
        div = divergence(k, v, q_sets[0], cache, args.steps)
        res[name] = {"single_step": one, "divergence": div}
        if args.gpu:
            import torch
            kern = kernel_attn_errors(torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                                      torch.from_numpy(q_sets).cuda())
            res[name]["kernels"] = kern
            for lab, e in kern.items():   # the kernels at N = 0 are rotation + RTN
                one["rotation + RTN" if lab == "KVarN N=0" else lab]["attn_kernel"] = e
        print(f"\n### {name}: {args.tokens} tokens x {args.kv_heads} KV heads, "
              f"{8 * args.query_sets} query rows per KV head\n")
        rows = {lab: {**one[lab], "d": div[lab]} for lab in one}
        last = args.steps - 1
        cols = [("K rel err", lambda r: f"{r['k']:.4f}"), ("V rel err", lambda r: f"{r['v']:.4f}"),
                ("K token-scale err", lambda r: f"{r['k_tok']:.4f}"),
                ("V token-scale err", lambda r: f"{r['v_tok']:.4f}"),
                ("attn rel err", lambda r: f"{r['attn']:.4f}")]
        if args.gpu:
            cols.append(("attn rel err, kernels", lambda r: f"{r['attn_kernel']:.4f}" if "attn_kernel" in r else "-"))
        cols += [("loop d_0", lambda r: f"{r['d'][0]:.4f}"),
                 (f"loop d_{last // 2}", lambda r: f"{r['d'][last // 2]:.4f}"),
                 (f"loop d_{last}", lambda r: f"{r['d'][last]:.4f}")]
        print(_table(rows, cols), flush=True)
    if args.gpu:
        import torch
        for name, make in (("one_layer_16k", lambda: synth.one_layer("cuda")),
                           ("long_context_128k", lambda: synth.long_context("cuda"))):
            w = make()
            q_sets = torch.stack([w.step_inputs(i)[0][0] for i in range(args.query_sets)])
            g = kernel_attn_errors(w.k_src, w.v_src, q_sets)
            res["kernels, full " + name] = g
            print(f"\n### kernels, full {name} ({w.k_src.shape[0]} tokens, {w.hkv} KV heads, one decode step)\n")
            print(_table({lab: e for lab, e in g.items()}, [("attn rel err", lambda e: f"{e:.4f}")]), flush=True)
    print(f"\n({time.perf_counter() - t0:.1f} s)")
    if args.out:
        with open(args.out, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
