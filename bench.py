"""Link-step benchmark on one MI355X.

A step is one pass of the whole link path over one batch: link_plan (host),
plan upload, copy-on-write scatter, key rotation (when the plan rotates keys
ahead of attention), attention, and split merge. The default workload is the
50,304-token request (64-token prefix + 98 x 512-token chunks + 64-token
suffix, LegoLink-32, Llama-3-8B layer shape, bf16). Its chunk KV and new rows
are seeded synthetic data, resident in HBM before timing starts.

Output: one JSON line with the step throughput (algorithmic TFLOP/s; steps
back to back as a serving loop runs them, each step's table upload on a copy
stream into the other of two workspaces, overlapping the previous step's
kernels), the attention kernel's roofline position (timed live with HIP events on the
stream it runs on), the link latency (each step alone between
synchronisations: 10th, 50th and 90th percentile), the same step with the
256 MiB MALL evicted before each step ("cold"), decode after link, the dense
full-recompute comparator on the same inputs, and the fp64 CPU oracle timed
on a bounded sample of rows.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-dense]
                    [--cold-steps N] [--rope-keys 0|1|2] [--key-layout L] [--split-pages P]
"""
from __future__ import annotations

import argparse
import dataclasses
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "link-step attention TFLOP/s + HBM GB/s (% MI355X peak); link latency @50k tok"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
DECODE_WARMUP, DECODE_STEPS = 3, 20
DECODE_SLOTS = DECODE_WARMUP + DECODE_STEPS
KERNEL_SOURCE = os.path.join(ROOT, "position_independent_kv_legolink_amd", "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def algorithmic_counts(cfg, export, sizes, n_tokens_per_request):
    """FLOP (QK^T + PV over unmasked keys) and HBM bytes of one link call."""
    d, hq, hkv = cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    elem = 2 if cfg.dtype == "bf16" else 4
    flop = 0
    kv_bytes = 0
    cu = export["cu_rows"]
    for r in range(len(cu) - 1):
        pos = export["row_pos"][cu[r]:cu[r + 1]].astype(np.int64)
        if pos.size == 0:
            continue
        first = int(export["pos_map"][export["cu_pages"][r] * cfg.page_size])
        keys = pos - first + 1                      # tokens at positions <= p
        flop += int(4 * d * hq * keys.sum())
        kv_bytes += int(keys.max()) * hkv * d * elem * 2
    R = sizes["rows"]
    q_out = 2 * R * hq * d * elem
    new_kv = 2 * R * hkv * d * elem
    page_bytes = hkv * cfg.page_size * d * elem
    private = 2 * sizes["private_pages"] * page_bytes
    cow = 2 * sizes["cow_pages"] * page_bytes
    attn_bytes = kv_bytes + q_out
    total = attn_bytes + new_kv + private + cow
    return flop, attn_bytes, total


class LinkJob:
    """Store, requests and device tensors of one workload."""

    def __init__(self, cfg, *, dense_pages=0, rope_keys=0, split_pages=0, key_layout="position_free"):
        import torch

        import position_independent_kv_legolink_amd as pic
        from workloads import gen

        self.cfg = cfg
        self.pic = pic
        self.torch = torch
        draws = gen.request_chunks(cfg)
        chunk_ids = sorted({c for ids in draws for c in ids})
        B = cfg.page_size
        pages = len(chunk_ids) * -(-cfg.chunk_len // B) + len(draws) * (-(-cfg.prefix_len // B))
        private = len(draws) * (cfg.chunks_per_request * -(-max(cfg.k, B if cfg.block_level else 0) // B)
                                + -(-cfg.suffix_len // B))
        self.n_tokens = cfg.prefix_len + cfg.chunks_per_request * cfg.chunk_len + cfg.suffix_len
        # room for the decode measurement's plan: its private pages plus DECODE_SLOTS decode slots per
        # request, and the RoPE rows of those positions
        decode_pages = private + len(draws) * (-(-DECODE_SLOTS // B) + 1)
        self.store = pic.Store(num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads, head_dim=cfg.head_dim,
                               page_size=B, num_pages=pages + private + max(dense_pages, decode_pages) + 64,
                               dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                               max_position=self.n_tokens + DECODE_SLOTS + 1, key_layout=key_layout)
        self.key_layout = key_layout
        self.tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        t = time.time()
        for c in chunk_ids:
            k, v = gen.chunk_kv(cfg, c)
            self.store.store_chunk(c, self._dev(k), self._dev(v))
        self.requests = []
        for r, ids in enumerate(draws):
            pid = None
            if cfg.prefix_len:
                pid = cfg.prefix_id(r)
                k, v = gen.prefix_kv(cfg, r)
                self.store.store_chunk(pid, self._dev(k), self._dev(v))
            self.requests.append(pic.LinkRequest(ids, cfg.suffix_len, pid))
        torch.cuda.synchronize()
        log(f"stored {len(chunk_ids)} chunks in {time.time() - t:.1f}s")
        self.plan_kw = dict(k=cfg.k, block_level=cfg.block_level, rope_keys=rope_keys, split_pages=split_pages)
        plan = self.store.link_plan(self.requests, **self.plan_kw)
        self.sizes = dict(plan.sizes)
        self.export = plan.export()
        cu = self.export["cu_rows"]
        qs, ks, vs = [], [], []
        for r in range(len(self.requests)):
            q, k, v = gen.new_rows(cfg, r, int(cu[r + 1] - cu[r]))
            qs.append(q), ks.append(k), vs.append(v)
        self.q = self._dev(np.concatenate(qs))
        self.k = self._dev(np.concatenate(ks))
        self.v = self._dev(np.concatenate(vs))
        self.workspace = torch.empty(self.sizes["workspace_bytes"], dtype=torch.uint8, device="cuda")
        self.out = torch.empty((self.sizes["rows"], cfg.num_q_heads, cfg.head_dim), dtype=self.tdt, device="cuda")
        plan.free()

    def _dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to("cuda", self.tdt).contiguous()

    def step(self):
        plan = self.store.link_plan(self.requests, **self.plan_kw)
        plan.upload(self.workspace)
        self.pic.link_attend(self.store, plan, self.q, self.k, self.v, out=self.out)
        plan.free()

    def step_pipelined(self):
        """One step as a serving loop runs them back to back: the same planning, upload and link
        call, with the upload on a copy stream into the other of two workspaces, so that the
        table copy overlaps the previous step's kernels instead of standing between them (the
        upload still waits for the step that last used that workspace, and the link call for
        the upload)."""
        torch = self.torch
        if not hasattr(self, "_pipe"):
            self._pipe = dict(ws=[self.workspace, torch.empty_like(self.workspace)], copy=torch.cuda.Stream(),
                              done=[None, None], k=0)
        pp = self._pipe
        k = pp["k"]
        pp["k"] ^= 1
        plan = self.store.link_plan(self.requests, **self.plan_kw)
        compute = torch.cuda.current_stream()
        with torch.cuda.stream(pp["copy"]):
            if pp["done"][k] is not None:
                pp["copy"].wait_event(pp["done"][k])
            plan.upload(pp["ws"][k])
            uploaded = torch.cuda.Event()
            uploaded.record(pp["copy"])
        compute.wait_event(uploaded)
        self.pic.link_attend(self.store, plan, self.q, self.k, self.v, out=self.out)
        done = torch.cuda.Event()
        done.record(compute)
        pp["done"][k] = done
        plan.free()


class NoGC:
    """Python's cyclic collector is off inside timed regions: one full collection over the
    objects a workload's setup leaves (about 170,000 for the 64-request workload) stalls the host
    for 40-65 ms, which a 10-step interval would count as 4-6 ms per step."""

    def __enter__(self):
        self.was = gc.isenabled()
        gc.disable()

    def __exit__(self, *exc):
        if self.was:
            gc.enable()


def time_steps(job, steps, warmup):
    """Throughput: steps back to back, each table upload overlapping the previous step's kernels
    (LinkJob.step_pipelined). Returns ms per step and the per-kernel profile."""
    torch = job.torch
    for _ in range(warmup):
        job.step_pipelined()
    torch.cuda.synchronize()
    job.store.profile_enable(True)
    torch.cuda.synchronize()
    with NoGC():
        t0 = time.perf_counter()
        for _ in range(steps):
            job.step_pipelined()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    prof = job.store.profile_read()
    job.store.profile_enable(False)
    return (t1 - t0) * 1e3 / steps, prof


def time_steps_no_events(job, steps):
    """The same steps without the per-kernel events: each event pair costs the GPU about 5 us,
    which matters for the short workloads."""
    torch = job.torch
    torch.cuda.synchronize()
    with NoGC():
        t0 = time.perf_counter()
        for _ in range(steps):
            job.step_pipelined()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps


def time_steps_latency(job, steps):
    """Link latency: each step (planning on the host, table upload and the kernels) timed alone
    between synchronisations, so nothing overlaps it. Returns the per-step times in ms."""
    torch = job.torch
    times = []
    with NoGC():
        for _ in range(steps):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            job.step()
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
    return times


def percentiles(times):
    a = np.asarray(times, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def time_steps_cold(job, steps, evict_mib=512):
    """Each step after a write of evict_mib MiB of scratch (the 256 MiB MALL holds none of the
    link step's data afterwards), timed on its own between synchronisations; the eviction is
    outside the timed interval. Returns (ms of each step, per-kernel profile)."""
    torch = job.torch
    scratch = torch.empty(evict_mib << 20, dtype=torch.uint8, device="cuda")
    job.store.profile_enable(True)
    times = []
    for i in range(steps):
        scratch.fill_(i & 0xff)
        torch.cuda.synchronize()
        with NoGC():
            t0 = time.perf_counter()
            job.step()
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
    prof = job.store.profile_read()
    job.store.profile_enable(False)
    del scratch
    return times, prof


def decode_measure(job, steps=DECODE_STEPS, warmup=DECODE_WARMUP):
    """Decode after link on the same requests: a plan with warmup + steps decode slots per
    request, one link call (it rotates the keys), then consecutive decode steps, the last
    `steps` timed with HIP events on the stream they run on (each appends its token). Bytes per
    step: every request's logical K' and V pages (shared pages count once per request that reads
    them) plus the new tokens' q, k, v and outputs."""
    torch, cfg = job.torch, job.cfg
    kw = dict(job.plan_kw)
    kw["rope_keys"] = 0
    plan = job.store.link_plan(job.requests, decode=warmup + steps, **kw)
    ws = torch.empty(plan.sizes["workspace_bytes"], dtype=torch.uint8, device="cuda")
    plan.upload(ws)
    job.pic.link_attend(job.store, plan, job.q, job.k, job.v)
    n = len(job.requests)
    g = np.random.default_rng(7)
    mk = lambda h: torch.from_numpy(g.standard_normal((n, h, cfg.head_dim), dtype=np.float32)).to(
        "cuda", job.tdt).contiguous()
    q, k, v = mk(cfg.num_q_heads), mk(cfg.num_kv_heads), mk(cfg.num_kv_heads)
    out = torch.empty_like(q)
    for _ in range(warmup):
        job.pic.link_decode(job.store, plan, q, k, v, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with NoGC():
        e0.record()
        for _ in range(steps):
            job.pic.link_decode(job.store, plan, q, k, v, out=out)
        e1.record()
        e1.synchronize()
    ms = e0.elapsed_time(e1) / steps
    elem = 2 if cfg.dtype == "bf16" else 4
    page_bytes = cfg.num_kv_heads * cfg.page_size * cfg.head_dim * elem
    nbytes = 2 * plan.sizes["pages"] * page_bytes + n * (2 * cfg.num_q_heads + 2 * cfg.num_kv_heads) * cfg.head_dim * elem
    items = plan.sizes["decode_items"]
    ws_mb = plan.sizes["workspace_bytes"] / 1e6
    rot_mb = plan.sizes["rotated_key_bytes"] / 1e6
    # decode reads the link call's rotated copy when it made one, else rotates the pool's keys
    keys = "rotated copy" if plan.sizes["rotated_pages"] else "pool, rotated in the kernel"
    plan.free()
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"requests": n, "ms": round(ms, 4), "work_items": items, "algorithmic_mb": round(nbytes / 1e6, 1),
            "gbps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
            "workspace_mb": round(ws_mb, 1), "rotated_keys_mb": round(rot_mb, 1), "keys": keys}


def model_measure(cfg, shape_name="llama3_8b", steps=5, warmup=2, gemm_reps=10):
    """TTFT-shaped latency: the request's selected rows through every layer of a Llama-3-8B-shaped
    model with seeded random weights (pic_link_forward: per layer RMSNorm, QKV projection, the
    link step over that layer's cached K/V, output projection, RMSNorm, gate/up + SwiGLU, down
    projection), each forward timed alone with HIP events after resetting the rows' hidden states.
    The layers' cached K/V and weights are drawn on the GPU (torch's seeded generator). The hand-
    written GEMM is also timed on its own at each projection shape of the layer."""
    import torch

    import position_independent_kv_legolink_amd as pic
    from workloads import MODEL_SHAPES, gen

    shape = MODEL_SHAPES[shape_name]
    L, dff, eps = shape.n_layers, shape.d_ff, shape.norm_eps
    hq, hkv, hd, B = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    dm, qd, kvd = hq * hd, hq * hd, hkv * hd
    draws = gen.request_chunks(cfg)
    chunk_ids = sorted({c for ids in draws for c in ids})
    n_tokens = cfg.prefix_len + cfg.chunks_per_request * cfg.chunk_len + cfg.suffix_len
    pages = len(chunk_ids) * -(-cfg.chunk_len // B) + len(draws) * (-(-cfg.prefix_len // B))
    private = len(draws) * (cfg.chunks_per_request * -(-max(cfg.k, B if cfg.block_level else 0) // B)
                            + -(-cfg.suffix_len // B))
    store = pic.Store(num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, page_size=B, num_pages=pages + private + 16,
                      dtype="bf16", rope_theta=cfg.rope_theta, max_position=n_tokens + 1, num_layers=L)
    g = torch.Generator(device="cuda")
    g.manual_seed(shape.weight_seed)

    def randn(*size, scale=1.0):
        return (torch.randn(*size, generator=g, device="cuda", dtype=torch.float32) * scale).to(torch.bfloat16)

    requests = []
    for c in chunk_ids:
        store.store_chunk(c, randn(L, cfg.chunk_len, hkv, hd, scale=cfg.kv_scale),
                          randn(L, cfg.chunk_len, hkv, hd, scale=cfg.kv_scale))
    for r, ids in enumerate(draws):
        pid = None
        if cfg.prefix_len:
            pid = cfg.prefix_id(r)
            store.store_chunk(pid, randn(L, cfg.prefix_len, hkv, hd, scale=cfg.kv_scale),
                              randn(L, cfg.prefix_len, hkv, hd, scale=cfg.kv_scale))
        requests.append(pic.LinkRequest(ids, cfg.suffix_len, pid))
    layers = []
    for _ in range(L):
        layers.append(dict(attn_norm=(1.0 + 0.1 * randn(dm).float()).to(torch.bfloat16),
                           w_qkv=randn(qd + 2 * kvd, dm, scale=dm ** -0.5), w_o=randn(dm, qd, scale=qd ** -0.5),
                           mlp_norm=(1.0 + 0.1 * randn(dm).float()).to(torch.bfloat16),
                           w_gate_up=randn(2 * dff, dm, scale=dm ** -0.5), w_down=randn(dm, dff, scale=dff ** -0.5)))
    model = pic.Model(d_model=dm, d_ff=dff, norm_eps=eps, layers=layers)
    plan = store.link_plan(requests, k=cfg.k, block_level=cfg.block_level)
    R = plan.rows
    x0 = randn(R, dm)
    x = torch.empty_like(x0)
    ws = torch.empty(pic.forward_workspace_bytes(store, plan, model), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    times = []
    with NoGC():
        for i in range(warmup + steps):
            x.copy_(x0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pic.link_forward(store, plan, model, x, workspace=ws)
            e1.record()
            e1.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
    assert torch.isfinite(x.float()).all(), "non-finite hidden states"
    ms = float(np.median(times))
    # the projections alone, at the layer's shapes (same kernel, same grid)
    a_dm, a_q, a_ff = randn(R, dm), randn(R, qd), randn(R, dff)
    gemms = {"qkv": (a_dm, layers[0]["w_qkv"], 0), "o": (a_q, layers[0]["w_o"], 1),
             "gate_up_swiglu": (a_dm, layers[0]["w_gate_up"], 2), "down": (a_ff, layers[0]["w_down"], 1)}
    gemm_out = {}
    gemm_ms_total, gemm_flop_total = 0.0, 0.0
    for name, (a, w, epi) in gemms.items():
        res = torch.empty((R, w.shape[0]), dtype=torch.bfloat16, device="cuda") if epi == 1 else None
        out = torch.empty((R, w.shape[0] // 2 if epi == 2 else w.shape[0]), dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            pic.linear(a, w, epi, residual=res, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(gemm_reps):
            pic.linear(a, w, epi, residual=res, out=out)
        e1.record()
        e1.synchronize()
        gms = e0.elapsed_time(e1) / gemm_reps
        flop = 2.0 * R * w.shape[0] * w.shape[1]
        gemm_ms_total += gms
        gemm_flop_total += flop
        gemm_out[name] = {"m": R, "n": int(w.shape[0]), "k": int(w.shape[1]), "ms": round(gms, 4),
                          "tflops": round(flop / (gms * 1e-3) / 1e12, 1),
                          "frac": round(flop / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    ex = plan.export()
    attn_flop = 0.0
    for r in range(len(requests)):
        p = ex["row_pos"][ex["cu_rows"][r]:ex["cu_rows"][r + 1]].astype(np.float64)
        attn_flop += 4.0 * hd * hq * float(np.sum(p + 1))     # positions start at 0
    layer_flop = gemm_flop_total + attn_flop
    plan.free()
    store.close()
    gemm_tflops = gemm_flop_total / (gemm_ms_total * 1e-3) / 1e12
    return {"model": shape_name, "layers": L, "d_model": dm, "d_ff": dff, "rows": R, "tokens_per_request": n_tokens,
            "ms": round(ms, 3), "ms_p10_p90": [round(float(np.quantile(times, 0.1)), 3),
                                               round(float(np.quantile(times, 0.9)), 3)],
            "ms_per_layer": round(ms / L, 4), "gflop_per_layer": round(layer_flop / 1e9, 1),
            "tflops": round(L * layer_flop / (ms * 1e-3) / 1e12, 1),
            "gemm": gemm_out, "gemm_ms_per_layer": round(gemm_ms_total, 4),
            "gemm_tflops": round(gemm_tflops, 1), "gemm_frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
            "weights": "random N(0, 1/fan_in), bf16", "data": "synthetic"}


def dense_comparator(job, reps=3):
    """Full recompute of every token (prefix and suffix included) on the same inputs.

    Every token's K/V is the linked cache's (cached chunk rows, with the link's
    recomputed rows in place), so the dense output at the link's selected rows
    must equal the link output; the largest difference is reported.
    """
    from workloads import gen

    torch, cfg = job.torch, job.cfg
    plan = job.store.link_plan(job.requests, k=cfg.k, recompute_all=True, rope_keys=job.plan_kw["rope_keys"])
    sizes, ex = dict(plan.sizes), plan.export()
    R = sizes["rows"]
    B = cfg.page_size
    k_all = torch.empty((R, cfg.num_kv_heads, cfg.head_dim), dtype=job.tdt, device="cuda")
    v_all = torch.empty_like(k_all)
    link_rows = []          # dense row index of every link row, in link order
    lcu = job.export["cu_rows"]
    at = 0
    for r, req in enumerate(job.requests):
        segs = ([("p", req.prefix_id, cfg.prefix_len, 0)] if req.prefix_id is not None else []) + \
               [("c", c, cfg.chunk_len, min(B, cfg.chunk_len) if cfg.block_level else min(cfg.k, cfg.chunk_len))
                for c in req.chunk_ids] + ([("s", None, cfg.suffix_len, cfg.suffix_len)] if cfg.suffix_len else [])
        lr = int(lcu[r])
        for kind, cid, length, rec in segs:
            if kind == "s":
                kk = job.k[lr:lr + rec]
                vv = job.v[lr:lr + rec]
            else:
                ck, cv = gen.prefix_kv(cfg, r) if kind == "p" else gen.chunk_kv(cfg, cid)
                kk, vv = job._dev(ck), job._dev(cv)
                kk[:rec] = job.k[lr:lr + rec]
                vv[:rec] = job.v[lr:lr + rec]
            k_all[at:at + length] = kk
            v_all[at:at + length] = vv
            link_rows.extend(range(at, at + rec))
            lr += rec
            at += length
    assert at == R
    g = gen.rng(cfg.seed, gen.KIND_Q_ALL, 0)
    q = job._dev(g.standard_normal((R, cfg.num_q_heads, cfg.head_dim), dtype=np.float32) * cfg.q_scale)
    idx = torch.tensor(link_rows, dtype=torch.long, device="cuda")
    q[idx] = job.q
    ws = torch.empty(sizes["workspace_bytes"], dtype=torch.uint8, device="cuda")
    out = torch.empty((R, cfg.num_q_heads, cfg.head_dim), dtype=job.tdt, device="cuda")
    plan.upload(ws)
    job.pic.link_attend(job.store, plan, q, k_all, v_all, out=out)
    torch.cuda.synchronize()
    job.store.profile_enable(True)
    with NoGC():
        t0 = time.perf_counter()
        for _ in range(reps):
            job.pic.link_attend(job.store, plan, q, k_all, v_all, out=out)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / reps
    prof = job.store.profile_read()
    job.store.profile_enable(False)
    flop, attn_bytes, _ = algorithmic_counts(cfg, ex, sizes, job.n_tokens)
    plan.free()
    job.step()
    torch.cuda.synchronize()
    diff = float((out[idx].float() - job.out.float()).abs().max())
    del q, k_all, v_all, ws, out
    attn_ms = prof["attention_ms"] / max(prof["calls"], 1)
    res = dict(rows=R, gflop=round(flop / 1e9, 1), ms=round(wall, 4), attention_ms=round(attn_ms, 4),
               attention_tflops=round(flop / attn_ms / 1e9, 2), max_abs_diff_at_link_rows=diff)
    if job.key_layout != "position_free":
        # every token enters as a new, position-free row here, while the cached keys of this
        # store are compiled from position 0: the timing holds, the comparison does not
        res["max_abs_diff_at_link_rows"] = None
        res["note"] = "cached keys re-entered as new rows without undoing their rotation: no output comparison"
    return res


def cpu_baseline(cfg, target_s, key_layout="position_free"):
    """The fp64 oracle on a bounded, evenly spread sample of the same workload's rows."""
    from oracle import link as olink
    from oracle import plan as oplan
    from workloads import gen

    draws = gen.request_chunks(cfg)
    segs = oplan.link_segments(prefix_id=cfg.prefix_id(0) if cfg.prefix_len else None, prefix_len=cfg.prefix_len,
                               chunk_ids=draws[0], chunk_lens=[cfg.chunk_len] * len(draws[0]),
                               suffix_len=cfg.suffix_len, k=cfg.k, block_level=cfg.block_level,
                               page_size=cfg.page_size)
    cached = {c: gen.chunk_kv(cfg, c) for c in set(draws[0])}
    if cfg.prefix_len:
        cached[cfg.prefix_id(0)] = gen.prefix_kv(cfg, 0)
    pos = np.asarray(oplan.selected_positions(segs), dtype=np.int64)
    R = len(pos)
    q, k, v = gen.new_rows(cfg, 0, R)
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # calibrate on a few rows (two probe sizes remove the fixed cost of building the merged
    # cache and rotating every key), then take as many evenly spread rows as fit the target
    times = []
    for n_probe in (4, 12):
        probe = np.linspace(0, R - 1, n_probe).astype(np.int64)
        t = time.perf_counter()
        olink.link_attention(segs, cached, q, k, v, cfg.rope_theta, rows=probe, key_layout=key_layout)
        times.append(time.perf_counter() - t)
    per_row = max((times[1] - times[0]) / 8, 1e-6)
    n = int(max(4, min(R, (target_s - times[0]) / per_row)))
    rows = np.unique(np.linspace(0, R - 1, n).astype(np.int64))
    t = time.perf_counter()
    olink.link_attention(segs, cached, q, k, v, cfg.rope_theta, rows=rows, key_layout=key_layout)
    dt = time.perf_counter() - t
    first = segs[0].start
    flop = int(4 * cfg.head_dim * cfg.num_q_heads * (pos[rows] - first + 1).sum())
    return dict(value=round(flop / dt / 1e12, 6), unit="TFLOP/s", cores=cores, kind="oracle",
                sample=f"{len(rows)} of {R} selected rows of request 0, evenly spread over positions, all "
                       f"{cfg.num_q_heads} heads, fp64 with explicit loops; {dt:.1f} s")


def traffic_from_profiles(workload, key_layout="position_free"):
    """HBM bytes per attention launch from the committed counter summary, if it is current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        t = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if (t.get("kernel_source_sha256_16") != kernel_hash() or t.get("workload") != workload
            or t.get("key_layout", "position_free") != key_layout):
        return None
    return t.get("hbm_bytes_per_launch")


def _counter_rows(directory, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    out = []
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def summarize_traffic(fetch_dir, write_dir, copy_mib, workload, out_json, key_layout="position_free"):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch) into HBM bytes per
    attention launch, each scaled by what the same counter reads for the calibration copy."""
    copy_bytes = copy_mib * (1 << 20)
    res = {"workload": workload, "key_layout": key_layout, "kernel_source_sha256_16": kernel_hash(),
           "copy_bytes": copy_bytes}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        rows = _counter_rows(d, counter)
        attn = [v for k, v in rows if "link_attention" in k]
        copy = [v for k, v in rows if "elementwise" in k.lower() or "mul" in k.lower()]
        if not attn or not copy:
            raise SystemExit(f"{counter}: need attention and calibration-copy dispatches in {d}")
        attn_kib = sum(attn) / len(attn)
        copy_kib = max(copy)
        scale = copy_bytes / (copy_kib * 1024.0)
        res[f"{name}_kib_per_dispatch"] = round(attn_kib, 1)
        res[f"copy_{name}_kib"] = round(copy_kib, 1)
        res[f"{name}_scale"] = round(scale, 4)
        res[f"{name}_bytes_per_launch"] = int(attn_kib * 1024 * scale)
    res["hbm_bytes_per_launch"] = res["fetch_bytes_per_launch"] + res["write_bytes_per_launch"]
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first; the GPU needs about 50 ms of load to reach its steady clocks")
    ap.add_argument("--workload", default="long50k_k32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps, each after evicting the MALL, reported under 'cold' (0: none)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-after-link measurement")
    ap.add_argument("--no-model", action="store_true",
                    help="skip the 32-layer forward (TTFT-shaped latency) of the request's selected rows")
    ap.add_argument("--rope-keys", type=int, default=0, choices=(0, 1, 2),
                    help="key rotation: 0 automatic, 1 inside attention, 2 once ahead of attention")
    ap.add_argument("--key-layout", default="position_free", choices=("position_free", "segment_rope"),
                    help="stored key form: pre-RoPE, or rotated at the position inside the segment "
                         "(a chunk compiled from position 0)")
    ap.add_argument("--value-scale", type=float, default=1.0,
                    help="scale the workload's synthetic Q, K and V by this factor (0: all zeros); the MFMA "
                         "clock depends on the operand values, so this shows how much of the attention time "
                         "is power rather than schedule")
    ap.add_argument("--split-pages", type=int, default=0,
                    help="KV pages per attention work item: 0 automatic, > 0 at most that many, "
                         "< 0 only where the kernel's limit requires")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size per step (counter calibration runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) into per-launch HBM bytes")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE)
    args = ap.parse_args()
    if args.traffic_from:
        summarize_traffic(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib or 256, args.workload,
                          args.traffic_out, args.key_layout)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the link step of one request batch runs on one MI355X "
              f"here (asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import CONFIGS

    import position_independent_kv_legolink_amd as pic
    pic.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = CONFIGS[args.workload]
    if args.value_scale != 1.0:
        cfg = dataclasses.replace(cfg, q_scale=cfg.q_scale * args.value_scale,
                                  kv_scale=cfg.kv_scale * args.value_scale)
    dense_pages = 0 if args.no_dense else (-(-(cfg.prefix_len + cfg.chunks_per_request * cfg.chunk_len +
                                                 cfg.suffix_len) // cfg.page_size)) * cfg.n_requests
    job = LinkJob(cfg, dense_pages=dense_pages, rope_keys=args.rope_keys, split_pages=args.split_pages,
                  key_layout=args.key_layout)
    # the setup's objects are never garbage: keep the collector from scanning them again
    gc.collect()
    gc.freeze()
    flop, attn_bytes, total_bytes = algorithmic_counts(cfg, job.export, job.sizes, job.n_tokens)
    # page sharing: logical pages the requests read vs the distinct physical pages behind them
    elem = 2 if cfg.dtype == "bf16" else 4
    page_bytes = cfg.num_kv_heads * cfg.page_size * cfg.head_dim * elem
    logical = int(job.sizes["pages"])
    distinct = int(np.unique(job.export["block_table"]).size)
    # live device bytes of the link step: the K/V pages it reads (each distinct page once) plus the
    # plan's workspace, whose rotated keys are a per-request copy of every logical key page
    unique_kv = 2 * distinct * page_bytes
    ws = job.sizes["workspace_bytes"]
    kv_pages = {"logical": logical, "distinct": distinct, "sharing_ratio": round(logical / max(distinct, 1), 3),
                "unique_kv_mb": round(unique_kv / 1e6, 1),
                "logical_kv_mb": round(2 * logical * page_bytes / 1e6, 1),
                "workspace_mb": round(ws / 1e6, 1),
                "rotated_keys_mb": round(job.sizes["rotated_key_bytes"] / 1e6, 1),
                "partials_mb": round(job.sizes["partial_bytes"] / 1e6, 1),
                "live_mb": round((unique_kv + ws) / 1e6, 1),
                "live_saving": round(2 * logical * page_bytes / max(unique_kv + ws, 1), 3)}
    t = time.perf_counter()
    for _ in range(10):
        job.store.link_plan(job.requests, **job.plan_kw).free()
    plan_ms = (time.perf_counter() - t) * 1e3 / 10
    log(f"{cfg.name}: rows {job.sizes['rows']}, pages {job.sizes['pages']}, work items {job.sizes['work_items']} "
        f"({job.sizes['split_items']} split), {flop / 1e9:.1f} GFLOP, {total_bytes / 1e6:.1f} MB")

    copy_src = copy_dst = None
    if args.copy_probe_mib:
        copy_src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        copy_dst = torch.empty_like(copy_src)

    # the kernel durations come from a run with the library's per-kernel events; the step time from
    # the same steps without them (each event pair costs the GPU a few microseconds)
    ms_step_events, prof = time_steps(job, args.steps, args.warmup)
    ms_step = time_steps_no_events(job, args.steps)
    lat = time_steps_latency(job, args.steps)
    latency = dict(steps=len(lat), **percentiles(lat))
    if copy_src is not None:
        # a plain elementwise kernel that reads and writes copy_probe_mib MiB each
        for _ in range(args.steps):
            torch.mul(copy_src, 1.0, out=copy_dst)
        torch.cuda.synchronize()
    calls = max(prof["calls"], 1)
    attn_ms = prof["attention_ms"] / calls
    # with keys rotated ahead the scatter runs inside the rotation's launch: the profile's scatter
    # interval holds no kernel then (only the cost of its events), and its rotation interval both
    fused = job.sizes["rotated_pages"] > 0
    scatter_ms = 0.0 if fused else prof["scatter_ms"] / calls
    merge_ms = prof["merge_ms"] / calls
    rotate_ms = prof["rotate_ms"] / calls
    link_ms = scatter_ms + rotate_ms + attn_ms + merge_ms
    log(f"step {ms_step:.3f} ms; scatter {scatter_ms:.4f} key rotation {rotate_ms:.4f} attention {attn_ms:.4f} "
        f"merge {merge_ms:.4f} ms")
    # key rotation pass: every rotated page's keys read and written, its cos/sin rows read once (one
    # row per slot for position-free keys, one per page for keys rotated inside their segment)
    rot_pages = job.sizes["rotated_pages"]
    cs_rows = cfg.page_size if args.key_layout == "position_free" else 1
    rot_bytes = rot_pages * (2 * cfg.num_kv_heads * cfg.page_size * cfg.head_dim * elem
                             + cs_rows * cfg.head_dim * 4)
    if fused:
        # and the scatter's: the new rows read, the private pages written, their copy-on-write rows read
        page_b = cfg.num_kv_heads * cfg.page_size * cfg.head_dim * elem
        rot_bytes += (2 * job.sizes["rows"] * cfg.num_kv_heads * cfg.head_dim * elem
                      + 2 * (job.sizes["private_pages"] + job.sizes["cow_pages"]) * page_b)

    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flop / (attn_ms * 1e-3) / 1e12
    roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=traffic_from_profiles(cfg.name, args.key_layout))

    cold = None
    if args.cold_steps > 0:
        c_times, c_prof = time_steps_cold(job, args.cold_steps)
        c_ms = float(np.mean(c_times))
        cc = max(c_prof["calls"], 1)
        c_attn = c_prof["attention_ms"] / cc
        cold = {"steps": args.cold_steps, "evict_mib": 512, "ms_per_step": round(c_ms, 4), **percentiles(c_times),
                "attention_ms": round(c_attn, 4), "attention_tflops": round(flop / (c_attn * 1e-3) / 1e12, 2),
                "rotate_ms": round(c_prof["rotate_ms"] / cc, 4),
                "scatter_ms": 0.0 if fused else round(c_prof["scatter_ms"] / cc, 4),
                "merge_ms": round(c_prof["merge_ms"] / cc, 4)}
        log(f"cold (MALL evicted before each step, steps not overlapped with planning): {cold}")
        # the same kernel with its K/V out of the MALL: launches of the cold leg
        achieved_cold = flop / (c_attn * 1e-3) / 1e12
        roofline["achieved_cold"] = round(achieved_cold, 2)
        roofline["frac_cold"] = round(achieved_cold / peak, 4)

    decode = None
    if not args.no_decode and cfg.dtype == "bf16":
        decode = decode_measure(job)
        log(f"decode after link: {decode}")

    model = None
    if not args.no_model and cfg.dtype == "bf16":
        model = model_measure(cfg)
        log(f"32-layer forward: {model}")

    dense = None
    if not args.no_dense:
        dense = dense_comparator(job)
        dense["link_speedup"] = round(dense["ms"] / link_ms, 2)
        log(f"dense full recompute: {dense}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds, args.key_layout)
        log(f"cpu oracle: {cpu}")

    result = {
        "metric": METRIC,
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_events": round(ms_step_events, 4),
        "step_pipeline": "table upload on a copy stream into the other of two workspaces, overlapping the "
                         "previous step's kernels; link_latency_wall_ms times steps alone",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens_per_request": job.n_tokens, "requests": cfg.n_requests,
                   "selected_rows": job.sizes["rows"], "q_heads": cfg.num_q_heads, "kv_heads": cfg.num_kv_heads,
                   "head_dim": cfg.head_dim, "page_size": cfg.page_size, "k": cfg.k,
                   "block_level": cfg.block_level, "key_layout": args.key_layout, "parallelism": "single GPU",
                   **({"value_scale": args.value_scale} if args.value_scale != 1.0 else {})},
        "link_latency_ms": round(link_ms, 4),
        "link_latency_wall_ms": latency,
        "attention_ms": round(attn_ms, 4),
        "scatter_ms": round(scatter_ms, 4),
        "merge_ms": round(merge_ms, 4),
        "keys_rotated_ahead": rot_pages > 0,
        "scatter_in_rotation": fused,
        "rotate_ms": round(rotate_ms, 4),
        "rotate_gbps": round(rot_bytes / (rotate_ms * 1e-3) / 1e9, 1) if rotate_ms > 0 else None,
        "link_plan_host_ms": round(plan_ms, 4),
        "kv_pages": kv_pages,
        "algorithmic_gflop": round(flop / 1e9, 3),
        "algorithmic_mb": round(total_bytes / 1e6, 2),
        "hbm_gbps": round(total_bytes / (link_ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(total_bytes / (link_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "mfma_frac_step": round(flop / (ms_step * 1e-3) / 1e12 / peak, 4),
        "roofline": roofline,
        "cold": cold,
        "decode": decode,
        "model_forward": model,
        "dense_comparator": dense,
        "cpu_baseline": cpu,
        "kernel_source_sha256_16": kernel_hash(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
