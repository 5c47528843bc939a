"""Benchmark of the decode MoE layer on one MI355X.

Workload (one "step" = one decode MoE layer call: route, gate/up, down):
a Flint-shaped layer (hidden 2048, 256 routed experts + 1 shared, expert
intermediate 512, sigmoid top-6, NVFP4 weights with BF16 activations) at
batch 1, with 32 independently seeded layer copies rotated call by call so
that the weights come from HBM, not from the 256 MB cache.  Weights and the
per-step activations are generated and repacked on the GPU before timing.

Reported (one JSON line):
  value        algorithmic HBM bytes per step / time per step, in TB/s: the
               selected experts' packed gate/up/down bytes (counted from the
               returned expert indices), the router matrix, and the
               activations in and out
  roofline     the dominant kernel: at batch 1 the whole layer is one launch
               (flint_b1_kernel), so its algorithmic bytes per launch over
               its average duration (HIP events around the graph replays on
               the launch stream) against 8 TB/s, and against the best rate
               of a plain read of the same number of bytes
               (flint_stream_read); the three-kernel path's per-stage times
               are reported beside
  cpu_baseline the float64 NumPy oracle on a bounded sample of the same
               workload, on the host, with all of its threads and with one
  batch8       the same layer at batch 8 (up to 48 distinct experts), one
               launch of flint_b8_kernel per layer
  decode_step  the 49-sublayer decode step (47 MoE + 2 dense, RMSNorm,
               residual) at batch 1, NVFP4 and BF16 weights
  prefill      8,192 tokens through one layer: TFLOP/s against the BF16
               MFMA peak, for i.i.d. and for skewed (correlated) tokens
  lm_head      an NVFP4 LM-head GEMV (2048 -> 150,144, 173 MB) through
               flint_dense_gemv at batch 1 and 8: TB/s against 8 TB/s
  qk_norm_rope_kv  the fused per-head Q/K RMSNorm + RoPE + KV-cache write
               (flint_qk_norm_rope_kv) for 8 and 8,192 tokens
  decode_attention  decode attention with learned sinks
               (flint_decode_attention): a 100K-context full layer at batch
               1 and a 513-token window layer at batch 1 and 8
The timed calls are replays of a HIP graph of back-to-back layer calls (host
launch cost is not on the clock), on activations and layer copies that the
warm-up calls did not use; the decode error word is checked after them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402
import w4a16_moe_decode_amd as fm  # noqa: E402

METRIC = "MoE-layer decode µs & achieved HBM TB/s (batch 1, 8); prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
N_COPIES = 32


def build_copies(shape: gen.MoeShape, n_copies: int, seed: int, device):
    """n_copies independently seeded packed layers, generated on the GPU."""
    layers, host_src0 = [], None
    for c in range(n_copies):
        src = gen.moe_layer_source(shape, gen.seed_for(seed, "copy", c), device)
        layers.append(fm.pack_moe_layer(src.router, src.gate, src.up, src.down, src.gscale,
                                        src.sh_gate, src.sh_up, src.sh_down, src.sh_gscale,
                                        src.layout, device))
        if c == 0:      # the oracle baseline runs on exactly copy 0's bytes
            host_src0 = gen.MoeLayerSource(**{
                k: (v.cpu() if isinstance(v, torch.Tensor) else v)
                for k, v in src.__dict__.items()})
        del src
    torch.cuda.synchronize()
    return layers, host_src0


def expert_bytes(shape: gen.MoeShape):
    H, I, SI = shape.hidden, shape.inter, shape.shared_inter
    per = lambda r, c: r * c // 2 + r * c // 16
    return {"gate_up": 2 * per(I, H), "down": per(H, I),
            "sh_gate_up": 2 * per(SI, H), "sh_down": per(H, SI)}


def step_bytes(shape: gen.MoeShape, batch: int, n_distinct: int):
    """Algorithmic HBM bytes of one decode call and of its gate/up kernel."""
    eb = expert_bytes(shape)
    router = shape.n_experts * shape.hidden * 2
    act = 2 * batch * shape.hidden * 2
    gu = n_distinct * eb["gate_up"] + eb["sh_gate_up"] + batch * shape.hidden * 2
    total = n_distinct * (eb["gate_up"] + eb["down"]) + eb["sh_gate_up"] + eb["sh_down"] + router + act
    return total, gu


class Bench:
    def __init__(self, layers, shape, batch, n_steps, seed):
        self.layers, self.shape, self.batch = layers, shape, batch
        self.runners = [fm.DecodeRunner(L, shape.top_k, 0) for L in layers]
        ws = self.runners[0].ws
        for r in self.runners:
            r.ws = ws                       # one workspace for the whole stream
        dev = layers[0].router.device
        n = max(n_steps, len(layers))
        self.x = gen.activations(gen.seed_for(seed, "x", batch), n * batch, shape.hidden, dev
                                 ).view(n, batch, shape.hidden)
        self.out = torch.empty_like(self.x)
        self.idx = torch.zeros((n, batch, shape.top_k), dtype=torch.int32, device=dev)
        self.w = torch.zeros((n, batch, shape.top_k), dtype=torch.float32, device=dev)

    def call(self, i):
        r = self.runners[i % len(self.runners)]
        r(self.x[i], out=self.out[i], topk_idx=self.idx[i], topk_w=self.w[i])

    def graph(self, n_steps, first=0):
        """A graph of calls first .. first + n_steps - 1 (call i: activations
        i, layer copy i mod copies)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(first, first + min(n_steps, 3)):     # eager warm-up before capture
                self.call(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(first, first + n_steps):
                self.call(i)
        return g

    def distinct(self, n_steps, first=0):
        idx = self.idx[first:first + n_steps].cpu()
        return [len(set(idx[i].reshape(-1).tolist())) for i in range(n_steps)]

    def stage_times(self, n_launch=256, ws_per_copy=4, flags=fm.FLINT_SPLIT):
        """Average duration of each stage, from HIP events around a graph of
        back-to-back launches of that stage alone on the launch stream.  Each
        launch uses its own (layer copy, workspace) pair holding a routing
        computed from its own activations, so consecutive launches read
        different experts of different copies (about 1 GB touched per pass,
        well past the 256 MB cache)."""
        pairs = []
        for k in range(ws_per_copy):
            for c, L in enumerate(self.layers):
                r = fm.DecodeRunner(L, self.shape.top_k, flags)
                i = (k * len(self.layers) + c) % self.x.shape[0]
                r(self.x[i], out=self.out[i], topk_idx=self.idx[i], topk_w=self.w[i])
                pairs.append((r, i))
        torch.cuda.synchronize()
        res = []
        for st in range(3):
            def body(st=st):
                for j in range(n_launch):
                    r, i = pairs[j % len(pairs)]
                    r.stage(st, self.x[i], self.out[i], self.idx[i], self.w[i])
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                body()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                body()
            g.replay()
            res.append(timed(g) / n_launch * 1e6)
            del g
        del pairs
        return res


def bench_step(args, dev, batch=1, n_moe=47, n_dense=2, reps=20):
    """The decode step over the MoE part of the model: 47 MoE sublayers
    (Flint shape, own seeded weights, 21.4 GB NVFP4) and 2 dense SwiGLU
    sublayers (intermediate 5632), pre-norm RMSNorm, residual in place; then
    the same step with BF16 weights (the exact dequantisation, 76 GB)."""
    shape = gen.SHAPE_FLINT
    layers, gmo, dl, gde = [], [], [], []
    for l in range(n_moe):
        src = gen.moe_layer_source(shape, gen.seed_for(args.seed, "step-moe", l), dev)
        layers.append(fm.pack_moe_layer(src.router, src.gate, src.up, src.down, src.gscale,
                                        src.sh_gate, src.sh_up, src.sh_down, src.sh_gscale,
                                        src.layout, dev))
        gmo.append(gen.rmsnorm_gamma(gen.seed_for(args.seed, "step-gm", l), shape.hidden, dev))
        del src
    for l in range(n_dense):
        g, u, d, ts = gen.dense_mlp_source(shape.hidden, gen.DENSE_INTER,
                                           gen.seed_for(args.seed, "step-dense", l), dev)
        dl.append(fm.pack_dense_mlp(g, u, d, ts, device=dev))
        gde.append(gen.rmsnorm_gamma(gen.seed_for(args.seed, "step-gd", l), shape.hidden, dev))
    torch.cuda.synchronize()
    eb = expert_bytes(shape)
    dense_bytes = sum(D.gu_codes.numel() + D.gu_scales.numel() + D.d_codes.numel() + D.d_scales.numel()
                      for D in dl)
    out = {}
    for wbf16 in (False, True):
        if wbf16:
            for L in layers:
                L.add_bf16()
            for D in dl:
                D.add_bf16()
            torch.cuda.synchronize()
        step = fm.DecodeStep(layers, gmo, dl, gde, shape.top_k, wbf16=wbf16)
        x0 = gen.activations(gen.seed_for(args.seed, "step-x"), batch, shape.hidden, dev)
        x = x0.clone()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(x)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                step(x)
        g.replay()
        x.copy_(x0)
        secs = timed(g) / reps
        idx = torch.stack([step.routing(l, batch)[0].reshape(-1) for l in range(n_moe)]).cpu()
        distinct = [len(set(idx[l].tolist())) for l in range(n_moe)]
        mult = 2.0 / (0.5 + 1.0 / 16) if wbf16 else 1.0      # bf16 bytes per weight vs nvfp4
        nb = sum(mult * (d * (eb["gate_up"] + eb["down"]) + eb["sh_gate_up"] + eb["sh_down"])
                 + shape.n_experts * shape.hidden * 2 + 4 * batch * shape.hidden for d in distinct)
        nb += mult * dense_bytes
        key = "bf16" if wbf16 else "nvfp4"
        out[key] = {"us_per_step": round(secs * 1e6, 2), "tokens_per_s": round(batch / secs, 1),
                    "tb_s": round(nb / secs / 1e12, 4), "bytes_per_step": int(nb)}
        print(f"[bench] decode step {key}: {secs * 1e6:.1f} us/step, {batch / secs:.0f} tok/s, "
              f"{nb / secs / 1e12:.3f} TB/s", file=sys.stderr, flush=True)
        del g, step
    out.update({"layers": n_moe + n_dense, "moe_layers": n_moe, "dense_layers": n_dense, "batch": batch,
                "dense_inter": gen.DENSE_INTER})
    return out


LM_HEAD_VOCAB = 150144


def bench_lm_head(dev, seed, n_copies=3, reps=30):
    """An NVFP4 LM-head GEMV (hidden 2048 -> 150,144 vocabulary rows, 173 MB
    of packed weights) through flint_dense_gemv at batch 1 and 8, rotating
    n_copies independently seeded matrices (519 MB, past the 256 MB cache)."""
    rows, cols = LM_HEAD_VOCAB, 2048
    mats = []
    for c in range(n_copies):
        src = gen.nvfp4_source(gen.seed_for(seed, "lm-head", c), 1, rows, cols, dev)
        mats.append(fm.repack_matrices(src))
        del src
    gs = torch.tensor([1 / 64, 0, 0, 0], dtype=torch.float32, device=dev)
    nbytes = rows * cols // 2 + rows * cols // 16
    out = {"rows": rows, "cols": cols, "weight_bytes": nbytes, "copies": n_copies}
    for batch in (1, 8):
        x = gen.activations(gen.seed_for(seed, "lm-x", batch), batch, cols, dev)
        y = torch.empty((batch, rows), dtype=torch.bfloat16, device=dev)

        def body(n):
            for i in range(n):
                c, s = mats[i % n_copies]
                fm.flint_dense_gemv(c, s, gs, None, rows, cols, 0, x, batch, y, fm.FLINT_EPI_NONE)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            body(n_copies)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(reps)
        g.replay()
        secs = timed(g) / reps
        b = nbytes + 2 * batch * (rows + cols)
        out[f"batch{batch}"] = {"us": round(secs * 1e6, 2), "tb_s": round(b / secs / 1e12, 3),
                                "frac_hbm_peak": round(b / secs / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] lm head batch {batch}: {secs * 1e6:.1f} us, {b / secs / 1e12:.3f} TB/s",
              file=sys.stderr, flush=True)
        del g
    del mats
    return out


def bench_attn_prep(dev, seed, reps=50):
    """The fused per-head Q/K RMSNorm + RoPE + KV-cache write
    (flint_qk_norm_rope_kv) at the Flint attention shape (GQA 32/4, d 128):
    8 decode tokens, and 8,192 prefill tokens over 3 rotating input copies
    (each 84 MB in, 84 MB out).  Bytes: projection rows and table rows read,
    q rows and K/V cache rows written."""
    sh = gen.ATTN_FLINT
    D = sh.head_dim
    table = gen.rope_table(600, D, device=dev)
    gq = gen.rmsnorm_gamma(gen.seed_for(seed, "attn-gq"), D, dev)
    gk = gen.rmsnorm_gamma(gen.seed_for(seed, "attn-gk"), D, dev)
    shape = fm.FlintAttnShape(sh.n_q_heads, sh.n_kv_heads, D, fm.FLINT_ATTN_ROPE, 1e-6)
    out = {"shape": "32 q / 4 kv heads, d 128, RoPE"}
    for T, n_copies in ((8, 1), (8192, 3)):
        g = torch.Generator(device="cpu").manual_seed(gen.seed_for(seed, "attn", T))
        sets = []
        for c in range(n_copies):
            qkv = gen.attn_rows(gen.seed_for(seed, "attn-qkv", T, c), T, sh, dev)
            pos = torch.randint(0, 600, (T,), generator=g, dtype=torch.int32).to(dev)
            slots = torch.randperm(max(T, 1024), generator=g)[:T].to(torch.int32).to(dev)
            kc = torch.empty((max(T, 1024), sh.n_kv_heads, D), dtype=torch.bfloat16, device=dev)
            vc = torch.empty_like(kc)
            q = torch.empty((T, sh.n_q_heads, D), dtype=torch.bfloat16, device=dev)
            sets.append((qkv, pos, slots, kc, vc, q))

        def body(n):
            for i in range(n):
                qkv, pos, slots, kc, vc, q = sets[i % n_copies]
                fm.flint_qk_norm_rope_kv(shape, qkv, T, pos, table, 600, slots, kc, vc, kc.shape[0], gq, gk, q)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            body(n_copies)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            body(reps)
        gr.replay()
        secs = timed(gr) / reps
        nb = T * ((sh.n_q_heads + 2 * sh.n_kv_heads) * D * 2 + D * 4 + 8 + sh.n_q_heads * D * 2
                  + 2 * sh.n_kv_heads * D * 2)
        out[f"tokens{T}"] = {"us": round(secs * 1e6, 2), "tb_s": round(nb / secs / 1e12, 3),
                             "frac_hbm_peak": round(nb / secs / 1e9 / HBM_PEAK_GBS, 4)}
        print(f"[bench] q/k norm + rope + kv write, {T} tokens: {secs * 1e6:.2f} us, "
              f"{nb / secs / 1e12:.3f} TB/s", file=sys.stderr, flush=True)
        del gr, sets
    return out


def bench_attn_decode(dev, seed):
    """Decode attention with learned sinks (flint_decode_attention) at the
    Flint attention shape (GQA 32/4, d 128), one query per sequence:
    a full-context (NoPE) layer at 100K context, batch 1 (the pages' decode
    measurement context), and a 513-token window layer at batch 1 and 8.
    Each case rotates independently drawn KV caches whose total passes the
    256 MB cache.  Bytes: the attended K and V rows, q and the output."""
    n_q, n_kv, d = 32, 4, 128
    shape = fm.FlintAttnShape(n_q, n_kv, d, 0, 0.0)
    scale = 1.0 / math.sqrt(d)
    out = {"shape": "32 q / 4 kv heads, d 128, learned sinks"}
    for name, batch, L, window, n_copies in (("full_100k_b1", 1, 100000, 0, 3),
                                             ("window513_b1", 1, 100000, 513, 320),
                                             ("window513_b8", 8, 100000, 513, 40)):
        ring = window if window else L
        cases = [gen.decode_attn_case(gen.seed_for(seed, "attn-dec", name, c), n_q, n_kv, [L] * batch, ring, dev,
                                      gap=0) for c in range(n_copies)]
        wsb = fm.flint_decode_attention_workspace_bytes(shape, window, batch, L)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        o = torch.empty((batch, n_q, d), dtype=torch.bfloat16, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        reps = max(30, n_copies)

        def body(n):
            for i in range(n):
                c = cases[i % n_copies]
                fm.flint_decode_attention(shape, window, ring, scale, c.q, batch, c.k_cache, c.v_cache, c.n_rows,
                                          c.seq_base, c.seq_len, L, c.sinks, o, ws if wsb else None, wsb, err)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            body(n_copies)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            body(reps)
        gr.replay()
        secs = timed(gr) / reps
        if int(err.item()) != 0:
            raise RuntimeError(f"decode attention {name}: error word set")
        span = min(L, window) if window else L
        nb = batch * (span * n_kv * d * 2 * 2 + 2 * n_q * d * 2)
        out[name] = {"us": round(secs * 1e6, 2), "tb_s": round(nb / secs / 1e12, 3),
                     "frac_hbm_peak": round(nb / secs / 1e9 / HBM_PEAK_GBS, 4), "bytes": nb,
                     "batch": batch, "context": L, "window": window}
        print(f"[bench] decode attention {name}: {secs * 1e6:.2f} us, {nb / secs / 1e12:.3f} TB/s",
              file=sys.stderr, flush=True)
        del gr, cases
        torch.cuda.empty_cache()
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(shape: gen.MoeShape, T: int) -> float:
    H, E, I, SI, K = shape.hidden, shape.n_experts, shape.inter, shape.shared_inter, shape.top_k
    return 2.0 * T * (H * E + K * 3 * I * H + 3 * SI * H)


def bench_prefill(layer, shape, seed, T=8192, reps=4, tiled=True, warm=16, timed_reps=16):
    """The 8,192-token prefill through one Flint-shaped layer (NVFP4), for
    i.i.d. tokens and for correlated tokens whose routing is skewed.  With
    ``tiled`` the weights are also given in the prefill layout
    (flint_moe_prefill_tiled; regrouped once, outside the timed region)."""
    out = {}
    runner = fm.PrefillRunner(layer, shape.top_k, T, 0, tiled=tiled)
    dev = layer.router.device
    idx = torch.zeros((T, shape.top_k), dtype=torch.int32, device=dev)
    w = torch.zeros((T, shape.top_k), dtype=torch.float32, device=dev)
    for kind in ("iid", "correlated"):
        x = gen.activations(gen.seed_for(seed, "prefill", kind), T, shape.hidden, dev, kind)
        y = torch.empty_like(x)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            runner(x, y, idx, w)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                runner(x, y, idx, w)
        # Warm-up replays: the first few milliseconds of prefill work in a
        # process run up to 15 % slower than the rest.
        for _ in range(warm):
            g.replay()
        each, total = timed_replays(g, timed_reps)
        secs = total / (timed_reps * reps)
        hist = torch.bincount(idx.reshape(-1).long(), minlength=shape.n_experts).float()
        fl = prefill_flops(shape, T)
        out[kind] = {"us": round(secs * 1e6, 1), "tflops": round(fl / secs / 1e12, 1),
                     "frac_mfma_peak": round(fl / secs / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "us_replays_p10_p50_p90": [round(v / reps * 1e6, 1) for v in percentiles(each)],
                     "hist_max_over_mean": round(float(hist.max() / hist.mean()), 2)}
        print(f"[bench] prefill {kind}: {secs * 1e6:.1f} us, {fl / secs / 1e12:.1f} TFLOP/s, "
              f"hist max/mean {out[kind]['hist_max_over_mean']}", file=sys.stderr, flush=True)
        del g
    out.update({"tokens": T, "gflop": round(prefill_flops(shape, T) / 1e9, 2),
                "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "dtype": "bf16 mfma (nvfp4 weights decoded to bf16 in registers)",
                "weights": "prefill layout (flint_moe_prefill_tiled)" if tiled else "packed planes (flint_moe_prefill)"})
    return out


def timed_replays(graph, reps):
    """Seconds of each of `reps` back-to-back replays (HIP events on the
    launch stream between them), and of all of them together."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for r in range(reps):
        graph.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    each = [ev[r].elapsed_time(ev[r + 1]) * 1e-3 for r in range(reps)]
    return each, ev[0].elapsed_time(ev[reps]) * 1e-3


def percentiles(xs):
    ys = sorted(xs)
    def q(f):
        return ys[min(len(ys) - 1, int(round(f * (len(ys) - 1))))]
    return q(0.1), q(0.5), q(0.9)


def read_ceiling(dev, nbytes, n_bufs=None, reps=50):
    """The best rate of flint_stream_read over a few launch shapes for a read
    of nbytes (rotating buffers totalling > 600 MB, past the 256 MB cache)."""
    nbytes = int(nbytes) // 16 * 16
    n_bufs = n_bufs or max(2, int(600e6 // nbytes) + 1)
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n_bufs)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    n16 = nbytes // 16
    shapes = [(256, 8, (n16 + 2047) // 2048), (64, 8, (n16 + 511) // 512), (512, 8, 256), (512, 16, 256),
              (768, 27, 256), (1024, 16, 512)]
    best = None
    for threads, loads, blocks in shapes:
        def body(n):
            for i in range(n):
                fm.flint_stream_read(bufs[i % n_bufs], nbytes, threads, loads, blocks, sink)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            body(n_bufs)
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body(reps)
        g.replay()
        secs = timed(g) / reps
        if best is None or secs < best[0]:
            best = (secs, threads, loads, blocks)
        del g
    del bufs
    secs, threads, loads, blocks = best
    return {"bytes": nbytes, "us": round(secs * 1e6, 2), "tb_s": round(nbytes / secs / 1e12, 3),
            "frac_hbm_peak": round(nbytes / secs / 1e9 / HBM_PEAK_GBS, 4),
            "launch": f"{blocks} x {threads} threads, {loads} 16-byte loads per thread per pass"}


def timed(graph, reps=1):
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e-3     # seconds


def host_cpu():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "model": model}


def cpu_baseline(layer_src, shape, budget_s: float):
    """The oracle (float64 NumPy) on batch-1 calls of copy 0 until the time
    budget is spent, with all of the host's threads and with one thread;
    TB/s of algorithmic bytes, like the GPU value."""
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from _parity import oracle_experts
    from oracle import moe

    def run(threads):
        with threadpool_limits(threads):
            torch.set_num_threads(threads)
            t_start = time.perf_counter()
            n, nbytes = 0, 0
            while time.perf_counter() - t_start < budget_s:
                ex = oracle_experts(layer_src)    # decode from the source bytes every call
                x = gen.numpy_f64(gen.activations(gen.seed_for(0, "cpu", n), 1, shape.hidden))
                _, r = moe.moe_layer(x, ex, shape.top_k, False)
                nbytes += step_bytes(shape, 1, len(set(r.idx.reshape(-1).tolist())))[0]
                n += 1
            el = time.perf_counter() - t_start
        return n, nbytes, el

    host = host_cpu()
    n_all = host["cpu_count"] or 1
    n, nbytes, el = run(n_all)
    n1, nbytes1, el1 = run(1)
    torch.set_num_threads(n_all)
    return {"value": nbytes / el / 1e12, "unit": "TB/s", "cores": n_all, "kind": "oracle",
            "sample": f"{n} batch-1 decode calls of one Flint-shaped layer (copy 0), {el:.1f} s, "
                      f"float64 NumPy, {n_all} threads",
            "us_per_layer": el / n * 1e6,
            "one_thread": {"value": nbytes1 / el1 / 1e12, "cores": 1, "us_per_layer": el1 / n1 * 1e6,
                           "sample": f"{n1} calls, {el1:.1f} s"},
            "host": host}


CSRC = os.path.join(ROOT, "w4a16_moe_decode_amd", "csrc")
# per kernel: the committed counter summary and the sources it was taken from
TRAFFIC = {
    "flint_b1_kernel": (os.path.join(ROOT, "profiles", "flint_b1_kernel_decode_b1_hbm_traffic.txt"),
                        ("flint_b1.hip", "flint_common.hpp", "fused_common.hpp", "common.hpp")),
    "flint_b8_kernel": (os.path.join(ROOT, "profiles", "flint_b8_kernel_decode_b8_hbm_traffic.txt"),
                        ("flint_b8.hip", "flint_common.hpp", "fused_common.hpp", "common.hpp")),
}


def kernel_source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of a kernel from its committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    plain copy of known size), or None when the kernel's source has changed
    since the counters were taken."""
    path, files = TRAFFIC[kernel]
    try:
        with open(path) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    if kv.get("kernel_source_sha256_16", "").strip() != kernel_source_digest(files):
        return None
    return {"bytes_per_launch": float(kv["hbm_bytes_per_launch"]),
            "read_bytes": float(kv["read_bytes_per_launch"]),
            "write_bytes": float(kv["write_bytes_per_launch"]),
            "algorithmic_bytes_per_launch": float(kv["algorithmic_bytes_per_launch"])}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048,
                    help="timed layer calls: replays of a graph of --graph-calls calls")
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--graph-calls", type=int, default=64)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=N_COPIES)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-batch8", action="store_true")
    ap.add_argument("--no-step", action="store_true", help="skip the 49-layer decode step")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8,192-token prefill")
    ap.add_argument("--no-lm-head", action="store_true", help="skip the NVFP4 LM-head GEMV")
    ap.add_argument("--no-attn", action="store_true", help="skip the fused Q/K norm + RoPE + KV write")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="first run a plain elementwise copy (fp32 negate) of this many MiB three "
                         "times, so that a counter run can scale FETCH_SIZE / WRITE_SIZE by it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode layer is replicated per GPU; see the sharding notes)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    fm.lib()
    dev = torch.device("cuda:0")
    shape = gen.SHAPE_FLINT
    if args.calibration_copy_mib > 0:
        src = torch.ones(args.calibration_copy_mib << 18, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)     # reads and writes calibration_copy_mib MiB each
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] generating {args.copies} layer copies on the GPU", file=sys.stderr, flush=True)
    layers, src0 = build_copies(shape, args.copies, args.seed, dev)

    G = args.graph_calls
    reps = max(1, args.steps // G)
    steps = reps * G
    res = {}
    for batch in ([1] if args.no_batch8 else [1, 8]):
        # warm-up calls 0 .. W-1 and timed calls W .. W+G-1 use different
        # activations (and so different experts) of the rotating copies
        b = Bench(layers, shape, batch, args.warmup + G, args.seed)
        gw = b.graph(args.warmup, 0)
        gt = b.graph(G, args.warmup)
        gw.replay()
        each, secs = timed_replays(gt, reps)
        err = fm.decode_error_word(b.runners[0])
        if err != 0:
            raise SystemExit(f"decode error word {err} after the timed batch-{batch} calls")
        dist = b.distinct(G, args.warmup)
        nb_graph = sum(step_bytes(shape, batch, d)[0] for d in dist)
        nbytes = nb_graph * reps
        gu_bytes = sum(step_bytes(shape, batch, d)[1] for d in dist) / len(dist)
        p10, p50, p90 = percentiles([e / G * 1e6 for e in each])
        st_us = b.stage_times()
        res[batch] = dict(secs=secs, nbytes=nbytes, gu_bytes=gu_bytes, stage_us=st_us,
                          distinct=sum(dist) / len(dist), pct=(p10, p50, p90),
                          path=fm.flint_moe_decode_path(b.runners[0].shape, batch))
        print(f"[bench] batch {batch}: {secs / steps * 1e6:.2f} us/layer (replays p10/p50/p90 "
              f"{p10:.2f}/{p50:.2f}/{p90:.2f}), {nbytes / secs / 1e12:.3f} TB/s, split-path stages "
              f"{['%.2f' % s for s in st_us]} us, distinct experts {res[batch]['distinct']:.2f}",
              file=sys.stderr, flush=True)
        del b, gw, gt

    ceil = {}
    for batch, r in res.items():
        ceil[batch] = read_ceiling(dev, r["nbytes"] / steps)
        print(f"[bench] plain read of {ceil[batch]['bytes'] / 1e6:.1f} MB: {ceil[batch]['us']} us, "
              f"{ceil[batch]['tb_s']} TB/s ({ceil[batch]['launch']})", file=sys.stderr, flush=True)

    r1 = res[1]
    us = r1["secs"] / steps * 1e6
    gu_us = r1["stage_us"][1]
    # batch 1 runs as one kernel launch per layer: the dominant (only) kernel
    # is the single-launch layer, timed by the graph of back-to-back calls
    achieved = r1["nbytes"] / r1["secs"] / 1e9
    traffic = measured_traffic("flint_b1_kernel")
    line = {
        "metric": METRIC,
        "value": round(r1["nbytes"] / r1["secs"] / 1e12, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "flint_moe_decode_layer", "hidden": shape.hidden,
                   "routed_experts": shape.n_experts, "shared_experts": 1,
                   "expert_inter": shape.inter, "top_k": shape.top_k, "batch": 1,
                   "weights": "nvfp4 (e2m1 + ue4m3/16 + fp32 per expert)", "activations": "bf16",
                   "layer_copies": args.copies, "parallelism": "single-gpu"},
        "us_per_layer": round(us, 3),
        "us_per_layer_replays_p10_p50_p90": [round(v, 3) for v in r1["pct"]],
        "tokens_per_s_per_layer": round(1e6 / us, 1),
        "timing": f"{reps} timed replays of a graph of {G} back-to-back calls (calls {args.warmup}.."
                  f"{args.warmup + G - 1}: activations and layer copies not used by the {args.warmup} "
                  f"warm-up calls); HIP events on the launch stream; percentiles of the per-replay means",
        "split_path_stage_us": {"route": round(r1["stage_us"][0], 3), "gate_up": round(gu_us, 3),
                                "down": round(r1["stage_us"][2], 3)},
        "roofline": {"bound": "hbm", "kernel": "flint_b1_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "traffic_read_write": [traffic["read_bytes"], traffic["write_bytes"]] if traffic else None,
                     "algorithmic_bytes_per_launch": round(r1["nbytes"] / steps),
                     "read_ceiling": ceil[1],
                     "frac_of_read_ceiling": round(achieved / 1e3 / ceil[1]["tb_s"], 4)},
    }
    if 8 in res:
        r8 = res[8]
        us8 = r8["secs"] / steps * 1e6
        a8 = r8["nbytes"] / r8["secs"] / 1e9
        line["batch8"] = {"us_per_layer": round(us8, 3),
                          "us_per_layer_replays_p10_p50_p90": [round(v, 3) for v in r8["pct"]],
                          "tb_s": round(a8 / 1e3, 4),
                          "kernel": "flint_b8_kernel" if r8["path"] == fm.FLINT_PATH_SINGLE_BATCH else "three kernels",
                          "frac_hbm_peak": round(a8 / HBM_PEAK_GBS, 4),
                          "read_ceiling": ceil[8],
                          "frac_of_read_ceiling": round(a8 / 1e3 / ceil[8]["tb_s"], 4),
                          "tokens_per_s_per_layer": round(8e6 / us8, 1),
                          "distinct_experts": round(r8["distinct"], 2),
                          "algorithmic_bytes_per_call": round(r8["nbytes"] / steps),
                          "traffic": (measured_traffic("flint_b8_kernel") or {}).get("bytes_per_launch"),
                          "split_path_stage_us": [round(v, 3) for v in r8["stage_us"]]}
    if not args.no_prefill:
        line["prefill"] = bench_prefill(layers[0], shape, args.seed)
    if not args.no_attn:
        line["qk_norm_rope_kv"] = bench_attn_prep(dev, args.seed)
        line["decode_attention"] = bench_attn_decode(dev, args.seed)
    if not args.no_lm_head:
        line["lm_head"] = bench_lm_head(dev, args.seed)
    if not args.no_step:
        del layers
        torch.cuda.empty_cache()
        line["decode_step"] = bench_step(args, dev)
    if not args.no_cpu:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(src0, shape, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
