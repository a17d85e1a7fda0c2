#!/usr/bin/env python3
"""Benchmark of the multi-row verify pass on one MI355X.

Workload (one "step"): the dense 27B-class MLP verify slice -- gate/up W4
5120 -> 17408, SiLU * up, down W4 17408 -> 5120, group 64 -- over R = 16 draft
lanes, through the library's verify_mlp_w4 entry point (W4 kernel for gate and
up in one launch, split reduce fused with SiLU * up, W4 kernel for down, split
reduce).  The weights are packed once at load (w4_pack, an exact byte
reordering with the same byte count), outside the timed region, like any
model load; inputs are resident in HBM before timing; the weights rotate over
several copies (> 2 x 256 MB in total) so the 256 MB Infinity Cache cannot
serve them.

Printed: one JSON line with the metric (algorithmic HBM GB/s of the verify
pass), the per-R sweep (R = 1, 2, 4, 8, 16), the dominant kernel's roofline
and the CPU oracle's time on a bounded sample of the same workload.  The step
time comes from HIP events recorded on the stream the path runs on, around
the whole timed region.  The W4 kernel's launch duration comes from the
library's timing hook: each workgroup stamps the device wall clock at its
start and at its end, and a launch lasts from its first start to its last end
(HIP events around single launches add the event packets' own overhead, about
a quarter of a 20 us launch).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4 verify-pass HBM GB/s (% of peak) at R=1..16; exact accepted tok/s"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--R", type=int, default=16)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the LM-head, MoE and decoder legs")
    ap.add_argument("--legs", default="lm_head,moe,formats,decoder_4096,decoder_32768,prefill",
                    help="comma list of the legs to run after the MLP slice")
    ap.add_argument("--legs-only", action="store_true",
                    help="run only the legs named by --legs (no MLP slice, no headline line): "
                         "for profiling one leg at a time")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (checked against eager)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 512 MiB five times (the known-size "
                         "reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def mlp_bytes(R, H, I, G):
    """Algorithmic bytes of the three W4 linears: weights + x in + y out each."""
    def lin(K, N):
        return N * K * 0.5 + 4.0 * N * (K // G) + 2.0 * R * K + 4.0 * R * N
    return 2 * lin(H, I) + lin(I, H)


# The sources that define the W4 kernels whose HBM traffic the committed
# counters measure (kernel code, launch plans, layouts, shared helpers).
W4_SOURCES = ("w4_verify.hip", "w4_kernel.h", "w4_layout.h", "ev_internal.h")


def source_hash():
    h = hashlib.sha256()
    for f in W4_SOURCES:
        with open(os.path.join(ROOT, "exact_speculative_decoding_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM traffic per W4 launch from committed rocprofv3 counter runs, valid
    only while the W4 kernel sources are unchanged since the counters were
    taken."""
    p = os.path.join(ROOT, "profiles", "w4_verify_mlp_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(d, R):
    """The oracle as it stands on this host: one whole R-row pass of the MLP
    slice (rows one at a time, OpenMP over output columns), in the same unit;
    then the same pass on one thread."""
    import oracle
    nb = mlp_bytes(R, d["H"], d["I"], d["G"])
    threads = int(oracle.num_threads())
    t0 = time.perf_counter()
    oracle.mlp(d["x"][:R], d["gate"], d["up"], d["down"], d["G"])
    dt = time.perf_counter() - t0
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.mlp(d["x"][:R], d["gate"], d["up"], d["down"], d["G"])
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"one {R}-row pass of the MLP slice (all three W4 linears and the glue)",
            "one_thread": {"value": round(nb / dt1 / 1e9, 4), "seconds": round(dt1, 2),
                           "ms_per_row": round(1e3 * dt1 / R, 1)},
            "cpu_model": cpu_model()}


def cpu_sampler(syn, R=16, V=151936):
    """The oracle's keyed sample (top-20, top-p 0.95, T 0.7) of R rows of
    the LM head's vocabulary, per row."""
    import numpy as np
    import oracle
    g = np.random.default_rng(1003)
    logits = syn.logits(g, R, V, scale=3.0)
    pos = np.arange(R, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.sample_rows(logits, pos, 0.7, 20, 0.95, 42)
    dt = time.perf_counter() - t0
    return {"kind": "oracle", "ms_per_row": round(1e3 * dt / R, 2), "rows": R, "V": V}


def cpu_moe(syn, R=16):
    """The oracle's MoE layer (128 experts, top 8, 2048 <-> 768, G 32) on R
    rows, per row."""
    import oracle
    d = syn.moe()
    t0 = time.perf_counter()
    oracle.moe(d["x"][:R], d["rho"][:R], d["top"], d["G"], d["gate"], d["up"], d["down"])
    dt = time.perf_counter() - t0
    return {"kind": "oracle", "ms_per_row": round(1e3 * dt / R, 1), "rows": R,
            "sample": f"one {R}-row MoE layer pass"}


# The pages' own decode figures, end to end on other hardware (context only:
# whole models with trained drafters, not this verify pass).
PAGES_CONTEXT = [
    {"what": "Qwen3.8-27B + DFlash2 drafter, code prompts, sampled, one stream",
     "tok_s": 49.6, "vs": "vLLM MTP=3: 17.7 tok/s", "hardware": "1x DGX Spark (GB10)",
     "source": "TensorFold README, DGX Spark table; 650 Group, 'TensorFold: the contract is what it does not change'"},
    {"what": "Nemotron 3.5 Lightning 30B-A3B, short answer with thinking",
     "tok_s": "188-206", "vs": "mlx_lm: 138 tok/s", "hardware": "Apple M5 Max, 128 GB",
     "source": "blog 'TensorFold: The engine that makes local LLMs 2-3x faster', section 'The numbers'"},
]


def stream_ceiling(ev, dev, stream, reps=20):
    """The practical ceiling next to the nominal peak: a plain streaming read
    (the library's read probe) of the two W4 launch sizes of the MLP slice,
    timed like the W4 launches.  Launches rotate over disjoint regions of a
    1 GiB buffer, so the 256 MB MALL holds none of them."""
    import torch
    buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    gbs = {}
    for nb in (50405376, 100810752):  # down; gate + up
        nreg = buf.numel() // nb
        region = lambda i: buf[(i % nreg) * nb:(i % nreg + 1) * nb]
        for i in range(3):
            ev.read_probe(region(i), sink, stream)
        torch.cuda.synchronize()
        ev.w4_timing_read()
        ev.w4_timing(True)
        for i in range(reps):
            ev.read_probe(region(i), sink, stream)
        torch.cuda.synchronize()
        ev.w4_timing(False)
        n, ms, by = ev.w4_timing_read()
        gbs[f"{nb / 1e6:.1f} MB"] = round(by / (ms * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return {"kernel": "plain grid-stride read (1024 x 256 threads, 16-byte loads)", "unit": "GB/s",
            "GB_s": gbs, "frac_of_peak": {k: round(v / HBM_PEAK_GBS, 3) for k, v in gbs.items()}}


def _event_time(stream, fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _prewarm(fn, ms=30.0, min_steps=200):
    """Untimed steps until `ms` of wall time and `min_steps` have passed: the
    part reaches its steady rate only after ~10 ms of streaming work."""
    import time
    import torch
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms or i < min_steps:
        for _ in range(50):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def leg_lm_head(ev, syn, to_dev, stream, steps):
    """LM head + sampler (5120 -> 151936, G 64): W4 logits of R hidden rows, then
    the keyed sample (T 0.7, top-k 20, top-p 0.95), per R."""
    import torch
    d = syn.lm_head()
    K, V, G = d["K"], d["V"], d["G"]
    copies = [ev.w4_pack(*(to_dev(a) for a in d["w"]), G) for _ in range(2)]  # 2 x 437.6 MB
    h = to_dev(d["h"])
    y = torch.empty((16, V), dtype=torch.float32, device="cuda")
    ws = torch.empty(ev.verify_linear_w4_workspace(K, V, G), dtype=torch.uint8, device="cuda")
    sws = torch.empty(ev.keyed_sample_workspace(V), dtype=torch.uint8, device="cuda")
    tok = torch.empty(16, dtype=torch.int32, device="cuda")
    out = {}
    for R in (1, 2, 4, 8, 16):
        pos = torch.arange(R, dtype=torch.int64, device="cuda")

        def step(i):
            ev.verify_linear_w4(h[:R], copies[i % 2], y=y[:R], ws=ws, stream=stream)
            ev.keyed_sample(y[:R], pos, 0.7, 20, 0.95, 42, tokens=tok[:R], ws=sws, stream=stream)
        if R == 1:
            _prewarm(step)  # the first point of the leg starts from an idle part
        ms = _event_time(stream, step, steps, 100)  # ~10 ms: the part's steady rate
        by = V * K * 0.5 + 4.0 * V * (K // G) + 2.0 * R * K + 4.0 * R * V * 2  # logits written + read
        out[str(R)] = {"us_per_pass": round(ms * 1e3, 2), "GB_s": round(by / (ms * 1e-3) / 1e9, 1),
                       "pct_hbm_peak": round(100 * by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
                       "lanes_per_s": round(R / (ms * 1e-3), 1)}
    del copies
    return {"workload": "LM head 5120 -> 151936 W4 G64 + keyed sample", "per_R": out}


def leg_moe(ev, syn, to_dev, stream, steps, n_stacks=12, n_rho=64):
    """MoE verify layer (hidden 2048, 128 experts, top 8, I 768, G 32), per R;
    bytes = the touched experts' weights (read once) + x + y.  Step i uses
    expert stack i % 12 (12 packed copies, 4.5 GB) and router-logit set
    i % 64, so the touched experts change every step and a stack comes back
    only after twelve steps, more than the 256 MB Infinity Cache holds even at
    R = 1 (8 experts, 23.6 MB a step)."""
    import numpy as np
    import torch
    d = syn.moe()
    H, I, E, top, G = d["H"], d["I"], d["E"], d["top"], d["G"]
    std = {m: tuple(to_dev(a) for a in d[m]) for m in ("gate", "up", "down")}
    stacks = [tuple(ev.w4_pack_stack(*std[m], G) for m in ("gate", "up", "down")) for _ in range(n_stacks)]
    del std
    g = np.random.default_rng(1014)
    rho = torch.from_numpy(g.standard_normal((n_rho, 16, E), dtype=np.float32)).cuda()
    x = to_dev(d["x"])
    ws = torch.empty(ev.verify_moe_w4_workspace(H, I, E, top, G), dtype=torch.uint8, device="cuda")
    y = torch.empty((16, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((n_rho, 16, top), dtype=torch.int32, device="cuda")
    per_expert = 3 * (I * H * 0.5 + 4.0 * I * (H // G))
    out = {}
    for R in (1, 2, 4, 8, 16):
        # the routing of every router set, read back once (untimed)
        g0, u0, d0 = stacks[0]
        for j in range(n_rho):
            ev.verify_moe_w4(x[:R], rho[j, :R].contiguous(), g0, u0, d0, top, y=y[:R], expert_ids=ids[j, :R],
                             ws=ws, stream=stream)
        torch.cuda.synchronize()
        touched = [len(np.unique(ids[j, :R].cpu().numpy())) for j in range(n_rho)]
        rho_r = [rho[j, :R].contiguous() for j in range(n_rho)]

        def step(i):
            gg, uu, dd = stacks[i % n_stacks]
            ev.verify_moe_w4(x[:R], rho_r[i % n_rho], gg, uu, dd, top, y=y[:R], ws=ws, stream=stream)
        n = max(steps, n_rho)
        if R == 1:
            _prewarm(step)  # the first point of the leg starts from an idle part
        ms = _event_time(stream, step, n, 200)  # ~10 ms of warm-up: the part's steady rate
        experts = sum(touched[i % n_rho] for i in range(n)) / n
        by = experts * per_expert + 2.0 * R * H + 4.0 * R * H
        out[str(R)] = {"us_per_pass": round(ms * 1e3, 2), "experts_mean": round(experts, 2),
                       "GB_s": round(by / (ms * 1e-3) / 1e9, 1),
                       "pct_hbm_peak": round(100 * by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}
    del stacks
    torch.cuda.empty_cache()
    return {"workload": "MoE layer H2048 E128 top8 I768 W4 G32", "weight_rotation":
            f"{n_stacks} expert stacks x {n_rho} router sets", "per_R": out}


def leg_decoder(ev, syn, C, n_tokens=512, R=8, p_draft=0.65, cpu_steps=0):
    """The 8-layer decoder: serial decoding (R = 1) of n_tokens, then drafted
    decoding with R - 1 drafts a round that match the serial transcript with
    probability p_draft; exact accepted tok/s = committed tokens / wall time
    (host drafter and the one read-back per round included)."""
    import numpy as np
    import torch
    from exact_speculative_decoding_amd.loop import decode, rows_after_probe, token_sha
    d = syn.decoder(C=C)
    cfg = d["cfg"]
    pos0, V = cfg["prefill"], cfg["vocab"]
    samp = (0.7, 20, 0.95, 42)

    def run(m, Rr, drafter):
        def fn(tokens, pos):
            return m.verify_step_host(tokens, pos, *samp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        toks, rounds = decode(fn, d["first_token"], pos0, n_tokens, Rr, drafter)
        torch.cuda.synchronize()
        return toks, rounds, time.perf_counter() - t0

    m = ev.load_decoder(cfg, d["w"], d["kc"], d["vc"])
    kc0, vc0 = m.k_cache.clone(), m.v_cache.clone()
    run(m, 1, lambda p, c: [])  # warm-up
    m.k_cache.copy_(kc0)
    m.v_cache.copy_(vc0)
    serial, _, t_serial = run(m, 1, lambda p, c: [])
    m.k_cache.copy_(kc0)
    m.v_cache.copy_(vc0)
    # the load-time exactness check on the live shapes: draft only if R-row
    # passes reproduce one-row steps here (it writes slots the decode rewrites)
    probe_words = []

    def probe(r):
        toks = torch.tensor([d["first_token"]] + serial[:r - 1], dtype=torch.int32, device="cuda")
        probe_words.append(m.verify_probe(toks, pos0, *samp))
        return probe_words[-1]
    R_used = rows_after_probe(probe, R)
    m.k_cache.copy_(kc0)
    m.v_cache.copy_(vc0)
    drafted, rounds, t_drafted = run(m, R_used, syn.transcript_drafter(serial, pos0 + 1, p_draft, 21, V))
    w_bytes = sum(np.asarray(d["w"][k]).nbytes for k in d["w"] if k.endswith(("_q", "_s", "_b")))
    kv_round = 2 * cfg["layers"] * cfg["kv_heads"] * (pos0 + n_tokens // 2) * cfg["head_dim"] * 2
    per_round = n_tokens / rounds
    roof = per_round * HBM_PEAK_GBS * 1e9 / (w_bytes + kv_round)
    tps = n_tokens / t_drafted
    cpu = None
    if cpu_steps:  # run after every GPU leg (see run_legs), so its threads disturb none
        cpu = lambda: cpu_decoder(d, C, cpu_steps, serial, samp)
    return {"workload": f"8-layer decoder H2048 16/4 heads MLP6144 V32768 W4 G64, cache {C}",
            "tokens": n_tokens, "R": R_used, "probe_mismatch_words": probe_words[0],
            "draft_match": p_draft, "rounds": rounds,
            "tokens_per_round": round(per_round, 3), "identical_to_serial": drafted == serial,
            "token_sha": {"drafted": token_sha(drafted), "serial": token_sha(serial)},
            "accepted_tok_s": round(tps, 1), "serial_tok_s": round(n_tokens / t_serial, 1),
            "ms_per_round": round(1e3 * t_drafted / rounds, 3),
            "bytes_per_round": int(w_bytes + kv_round),
            "roofline_tok_s": round(roof, 1), "pct_roofline": round(100 * tps / roof, 2),
            **({"cpu_baseline": cpu} if cpu else {})}


def cpu_decoder(d, C, cpu_steps, serial, samp):
    """The oracle's serial steps of the decoder from the GPU run's start, on
    the host cores, and whether they sample the GPU's serial tokens."""
    import oracle
    cfg = d["cfg"]
    pos0 = cfg["prefill"]
    om = oracle.Decoder(cfg, d["w"], d["kc"], d["vc"])
    tok = d["first_token"]
    oracle_tokens = []
    t0 = time.perf_counter()
    for i in range(cpu_steps):
        _, tok, _ = om.step(tok, pos0 + i, *samp)
        oracle_tokens.append(tok)
    dt = time.perf_counter() - t0
    return {"kind": "oracle", "tokens": cpu_steps, "ms_per_token": round(1e3 * dt / cpu_steps, 1),
            "matches_gpu_serial": [int(t) for t in oracle_tokens] == serial[:cpu_steps],
            "tok_s": round(cpu_steps / dt, 3), "cores": int(oracle.num_threads()),
            "sample": f"{cpu_steps} serial steps of the 8-layer decoder, cache {C}"}


def leg_formats(ev, syn, to_dev, stream, steps):
    """The W4 kernel on the two 4-bit formats, one linear at a time: affine
    uint4 (fp16 scale and bias per 64) and NVFP4-style (E2M1 codes, E4M3 scale
    per 16, tensor scale), both 0.5625 bytes a weight, for the slice's two
    matrix shapes, four rotating copies each; kernel-only GB/s from the
    per-workgroup stamps (the split sums excluded), per R."""
    import numpy as np
    import torch
    out = {}
    g = np.random.default_rng(1011)
    for K, N in ((5120, 17408), (17408, 5120)):
        aff = [ev.w4_pack(*(to_dev(a) for a in syn.w4_matrix(g, N, K, 64)), 64) for _ in range(4)]
        q, s, st = syn.nvfp4_matrix(g, N, K)
        fp4 = [ev.nvfp4_pack(to_dev(q), to_dev(s), st) for _ in range(4)]
        x = to_dev(syn.activations(g, 16, K))
        y = torch.empty((16, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(ev.verify_linear_w4_workspace(K, N, 64), 1), dtype=torch.uint8, device="cuda")
        row = {}
        for R in (1, 16):
            for name, mats, fn in (("affine_g64", aff, ev.verify_linear_w4), ("nvfp4", fp4, ev.verify_linear_nvfp4)):
                for i in range(200):
                    fn(x[:R], mats[i % 4], y=y[:R], ws=ws, stream=stream)
                torch.cuda.synchronize()
                ev.w4_timing_read()
                ev.w4_timing(True)
                for i in range(steps):
                    fn(x[:R], mats[i % 4], y=y[:R], ws=ws, stream=stream)
                torch.cuda.synchronize()
                ev.w4_timing(False)
                n, ms, by = ev.w4_timing_read()
                row.setdefault(name, {})[str(R)] = {"kernel_us": round(1e3 * ms / n, 2),
                                                    "GB_s": round(by / (ms * 1e-3) / 1e9, 1),
                                                    "frac": round(by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        out[f"{K}->{N}"] = row
        del aff, fp4
        torch.cuda.empty_cache()
    return {"workload": "one W4 linear, affine G64 vs NVFP4, kernel only", "shapes": out}


def leg_prefill(ev, syn, C=4096, P=3584, grid=2048, reps=3):
    """Grid-aligned chunked prefill of a P-token prompt into the 8-layer
    decoder's cache (passes of at most 16 rows, never across a multiple of 16
    or of the 2,048-token grid).  Bytes per pass: the layers' W4 weights plus
    the cache entries read (attention over the slots before each pass's rows)."""
    import numpy as np
    import torch
    d = syn.decoder(C=C, prefill=0)
    cfg = d["cfg"]
    m = ev.load_decoder(cfg, d["w"], d["kc"], d["vc"])
    prompt = torch.from_numpy(np.random.default_rng(7).integers(0, cfg["vocab"], P).astype(np.int32)).cuda()
    m.prefill(prompt[:64], 0, grid)  # warm-up (captures the pass graphs)
    torch.cuda.synchronize()
    t = []
    for _ in range(reps):
        t0 = time.perf_counter()
        m.prefill(prompt, 0, grid)
        torch.cuda.synchronize()
        t.append(time.perf_counter() - t0)
    dt = min(t)
    w_layers = sum(np.asarray(d["w"][k]).nbytes for k in d["w"]
                   if k.endswith(("_q", "_s", "_b")) and not k.startswith("lm"))
    passes = P // 16
    kv = sum(2 * cfg["layers"] * cfg["kv_heads"] * (16 * i + 16) * cfg["head_dim"] * 2 for i in range(passes))
    by = passes * w_layers + kv
    roof = P * HBM_PEAK_GBS * 1e9 / by
    tps = P / dt
    return {"workload": f"prefill of a {P}-token prompt, 8-layer decoder H2048, cache {C}, grid {grid}",
            "ms": round(1e3 * dt, 2), "tok_s": round(tps, 1), "passes": passes,
            "roofline_tok_s": round(roof, 1), "pct_roofline": round(100 * tps / roof, 2)}


def run_legs(args, ev, syn, to_dev, stream):
    """The legs named by --legs, in a fixed order, each timed on its own."""
    legs, want = {}, set(args.legs.split(","))
    leg_steps = max(args.steps, 100)  # a leg point over a few ms, not a 1-2 ms window
    runs = [("lm_head", "lm_head_sampler", lambda: leg_lm_head(ev, syn, to_dev, stream, leg_steps)),
            ("moe", "moe_layer", lambda: leg_moe(ev, syn, to_dev, stream, leg_steps)),
            ("formats", "formats", lambda: leg_formats(ev, syn, to_dev, stream, args.steps)),
            ("decoder_4096", "decoder_4096",
             lambda: leg_decoder(ev, syn, 4096, cpu_steps=0 if args.no_cpu_baseline else 24)),
            ("decoder_32768", "decoder_32768",
             lambda: leg_decoder(ev, syn, 32768, cpu_steps=0 if args.no_cpu_baseline else 16)),
            ("prefill", "prefill_4096", lambda: leg_prefill(ev, syn))]
    for name, key, fn in runs:
        if name in want:
            legs[key] = fn()
            print(f"# {key} leg done", file=sys.stderr, flush=True)
    # the oracle timings of the decoder legs, after all GPU timing
    for key, leg in legs.items():
        if callable(leg.get("cpu_baseline")):
            leg["cpu_baseline"] = leg["cpu_baseline"]()
    return legs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path's multi-GPU sharding is a design, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_speculative_decoding_amd as ev
    import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.calibrate_copy:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                          "launches": 5}), flush=True)
        return

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    if args.legs_only:
        print(json.dumps({"legs": run_legs(args, ev, syn, to_dev, torch.cuda.current_stream())}), flush=True)
        return

    d = syn.mlp()
    H, I, G = d["H"], d["I"], d["G"]

    copies = []
    for c in range(args.copies):
        mats = []
        for m in ("gate", "up", "down"):
            q, s, b = (to_dev(a) for a in d[m])
            mats.append(ev.w4_pack(q, s, b, G))
            del q, s, b
        copies.append(tuple(mats))
    torch.cuda.synchronize()
    x_all = to_dev(d["x"])
    ws = torch.empty(ev.verify_mlp_w4_workspace(H, I, G), dtype=torch.uint8, device=dev)
    y = torch.empty((16, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream() if args.graph else torch.cuda.current_stream()

    def eager(i, R):
        gate, up, down = copies[i % len(copies)]
        ev.verify_mlp_w4(x_all[:R], gate, up, down, y=y[:R], ws=ws, stream=stream)

    graphs = {}

    def step(i, R):
        if not args.graph:
            return eager(i, R)
        key = (i % len(copies), R)
        if key not in graphs:
            # capture on a side stream, then check that replays reproduce eager bits
            eager(i, R)
            torch.cuda.synchronize()
            ref = y[:R].clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                eager(i, R)
            for _ in range(3):
                y.zero_()
                g.replay()
                torch.cuda.synchronize()
                if not torch.equal(y[:R].view(torch.int32), ref.view(torch.int32)):
                    raise RuntimeError("graph replay differs from eager")
            graphs[key] = g
        graphs[key].replay()

    def timed(R, steps, warmup):
        for i in range(warmup):
            step(i, R)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step(i, R)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def step_percentiles(R, steps):
        """p10 / p50 / p90 of single steps, each between two events (which add
        their own overhead; the headline uses one bracket around all steps)."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            step(i, R)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        t = sorted(1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        pick = lambda f: round(t[min(steps - 1, int(f * (steps - 1) + 0.5))], 2)
        return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}

    R = args.R
    torch.cuda.set_stream(stream)
    # Untimed pre-warm before the warm-up steps, whatever --warmup says: the
    # part reaches its steady streaming rate only after ~10 ms of this work.
    torch.cuda.synchronize()
    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < 0.03 or n_pre < 300:
        for _ in range(50):
            step(n_pre, R)
            n_pre += 1
        torch.cuda.synchronize()
    prewarm = {"steps": n_pre, "ms": round(1e3 * (time.perf_counter() - t_pre), 1)}
    ms = timed(R, args.steps, args.warmup)
    gbs = mlp_bytes(R, H, I, G) / (ms * 1e-3) / 1e9
    print(f"# R={R}: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    pct = step_percentiles(R, args.steps)

    per_r = {}
    sweep_steps = max(args.steps, 100)  # ~4 ms a point: a short window is at the mercy of clock noise
    if not args.no_sweep:
        for r in (1, 2, 4, 8, 16):
            m = timed(r, sweep_steps, 50)
            g = mlp_bytes(r, H, I, G) / (m * 1e-3) / 1e9
            per_r[str(r)] = {"us_per_pass": round(m * 1e3, 2), "GB_s": round(g, 1),
                             "pct_hbm_peak": round(100 * g / HBM_PEAK_GBS, 1),
                             "lanes_per_s": round(r / (m * 1e-3), 1)}
            print(f"# R={r}: {m * 1e3:.1f} us/pass, {g:.0f} GB/s", file=sys.stderr, flush=True)

    # dominant kernel: the W4 kernel (both W4 launches of the slice), each
    # launch timed by the device wall-clock stamps of its workgroups, over as
    # many steps again; at the config's R, then at every R of the sweep
    def kernel_roofline(r, steps):
        torch.cuda.synchronize()
        ev.w4_timing_read()
        ev.w4_timing(True)
        for i in range(steps):
            eager(i, r)
        torch.cuda.synchronize()
        ev.w4_timing(False)
        n_launch, k_ms, k_bytes = ev.w4_timing_read()
        k_gbs = k_bytes / (k_ms * 1e-3) / 1e9
        return n_launch, k_ms, k_bytes, k_gbs

    n_launch, k_ms, k_bytes, k_gbs = kernel_roofline(R, args.steps)
    traffic = load_traffic()
    roofline = {"kernel": "w4_sk_kernel", "bound": "hbm", "achieved": round(k_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k_gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic, "R": R, "launches": n_launch,
                "avg_launch_us": round(1e3 * k_ms / max(n_launch, 1), 2),
                "algorithmic_bytes_per_launch": round(k_bytes / max(n_launch, 1))}
    if not args.no_sweep:
        roofline["per_R"] = {}
        for r in (1, 2, 4, 8, 16):
            nl, kms, kby, kg = kernel_roofline(r, sweep_steps)
            roofline["per_R"][str(r)] = {"achieved": round(kg, 1), "frac": round(kg / HBM_PEAK_GBS, 4),
                                         "avg_launch_us": round(1e3 * kms / max(nl, 1), 2),
                                         "algorithmic_bytes_per_launch": round(kby / max(nl, 1))}

    out = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dense 27B-class MLP verify slice: gate/up W4 5120->17408, "
                               "SiLU*up, down W4 17408->5120, group 64",
                   "R": R, "launch": "hip graph replay" if args.graph else "eager", "H": H, "I": I, "G": G, "weight_copies": args.copies,
                   "weight_bytes_per_copy": int(mlp_bytes(0, H, I, G))},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "prewarm": prewarm,
        "lanes_per_s": round(R / (ms * 1e-3), 1),
        "step_us_percentiles": pct,
        "per_R": per_r,
        "roofline": roofline,
    }
    if not args.no_legs:
        out["stream_ceiling"] = stream_ceiling(ev, dev, stream)
        print("# stream ceiling done", file=sys.stderr, flush=True)
    if not args.no_legs:
        legs = run_legs(args, ev, syn, to_dev, stream)
        out["legs"] = legs
        if "decoder_4096" in legs:
            out["exact_accepted_tok_s"] = legs["decoder_4096"]["accepted_tok_s"]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, R)
        out["cpu_baseline"]["sampler"] = cpu_sampler(syn)
        out["cpu_baseline"]["moe_layer"] = cpu_moe(syn)
        for leg in ("decoder_4096", "decoder_32768"):
            if leg in out.get("legs", {}):
                out["cpu_baseline"][leg] = out["legs"][leg].pop("cpu_baseline")
    out["pages_context"] = PAGES_CONTEXT
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
