"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = the whole hot path on one batch of synthetic input resident in HBM:
sliding-tile mask (if the workload has one) -> NABLA mask (pool + select, OR'd with
the sliding-tile mask) -> kv lists (CSR) -> block-sparse attention forward.

Prints ONE JSON line. `value` is the effective attention throughput of the whole step:
kept-tile FLOPs (4 * 64 * 64 * D per kept 64x64 tile) / step time. The roofline object
is for the dominant kernel (the attention kernel), timed with HIP events on the stream
it runs on; `cpu_baseline` times the fp64 oracle on a bounded sample of the same work.

    python bench.py [--steps K] [--warmup W] [--config 3] [--dense] [--dense-reps R] [--no-cpu-baseline]
    python bench.py --sweep [--config 5]    (threshold sweep table, bf16 and fp8 Q/K)

The default workload is the 14B 720p shape (40 heads, 21x45x80 grid, NABLA thr 0.2); the
line also carries dense attention of the same shape (the same kernel over an all-ones
mask, timed after the sparse launches) and its speedup.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (published)
FP8_PEAK_TFLOPS = 5033.2       # MI355X dense fp8 MFMA (published)
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E (published)
PEAK_CLOCK_MHZ = 2400.0        # the engine clock the published MFMA peaks are quoted at
LLC_BYTES = 256 << 20           # MI355X last-level (Infinity) cache


def _flops_per_tile(D):
    return 4.0 * 64 * 64 * D


def _measured_traffic(workload, fp8=False, dense=False):
    """HBM bytes per attention launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None when the kernel source has
    changed since they were taken or the workload was not profiled."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["attn_fwd"]
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
        entry = rec["workloads"][workload]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if hashlib.sha256(src).hexdigest()[:16] != entry["sha256_prefix"] or fp8 or dense:
        return None
    return entry["traffic_bytes_per_launch"]


def run_gpu(cfg, steps, warmup, thr, dense=False, fp8=False, graph=True, csr_step=False, dense_reps=0,
            rotate=False):
    import torch
    import block_sparse_attention_mask_amd as bsa
    from synth import make_inputs

    bsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(cfg, seed=0, device=dev)
    qa, ka, qs, ks = q, k, None, None
    if fp8:
        # fp8 e4m3 Q/K with per-block scales, produced inside each step by the library
        # (from the mask build's own read of Q and K when there is an adaptive mask)
        qa, ka = torch.empty(q.shape, dtype=torch.uint8, device=dev), torch.empty(k.shape, dtype=torch.uint8, device=dev)
        qs = torch.empty(cfg.B, cfg.H, cfg.nb, dtype=torch.float32, device=dev)
        ks = torch.empty(cfg.B, cfg.H, cfg.nb, dtype=torch.float32, device=dev)
    signs = None
    if rotate:
        # incoherent processing: random signs of the Hadamard rotation, drawn once
        from synth import make_signs
        signs = make_signs(cfg.D, seed=0)

    def quantize_qk():
        if rotate:
            bsa.quantize_fp8_blocks_rotated(q, signs, False, out=(qa, qs))
            bsa.quantize_fp8_blocks_rotated(k, signs, True, out=(ka, ks))
        else:
            bsa.quantize_fp8_blocks(q, out=(qa, qs))
            bsa.quantize_fp8_blocks(k, out=(ka, ks))
    nb, S = cfg.nb, cfg.S
    use_nabla = (thr is not None) and not dense
    plane = torch.empty(nb, nb, dtype=torch.uint8, device=dev)
    mask = torch.empty(cfg.B, cfg.H, nb, nb, dtype=torch.uint8, device=dev)
    ones = torch.ones(nb, nb, dtype=torch.uint8, device=dev)
    rows = cfg.B * cfg.H * nb
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(rows * nb, dtype=torch.int32, device=dev)
    out = torch.empty_like(v)
    import ctypes
    shp = bsa.Shape(cfg.B, cfg.H, S, cfg.S_valid, cfg.D, 64)
    lib = bsa.load()
    csr_ws = torch.empty(max(256, lib.csr_workspace_size(cfg.B, cfg.H, nb)), dtype=torch.uint8, device=dev)
    attn_ws = torch.empty(max(256, lib.attn_csr_workspace_size(ctypes.byref(shp), bsa._dtype_code(qa))),
                          dtype=torch.uint8, device=dev)
    n_slots = lib.attn_work_order_slots(ctypes.byref(shp))
    work_order = torch.empty(n_slots, dtype=torch.int32, device=dev) if n_slots > 0 else None
    # short rows: the kv lists (and the work order) come out of the mask build's own
    # launch, and attention reads them there; no compaction pass over the mask
    fused = use_nabla and not fp8 and nb <= 256 and not csr_step
    if fused:
        kv_len = torch.empty(rows, dtype=torch.int32, device=dev)
        kv_idx = torch.empty(rows, nb, dtype=torch.int32, device=dev)
        lists_ws = bsa.nabla_lists_workspace(q, cfg.S_valid)
        sta_kw = {} if cfg.sta is None else dict(grid=cfg.grid, tile=cfg.sta.tile, window=cfg.sta.window,
                                                  order=cfg.order, order_tile=cfg.order_tile)

    st = {}

    def phase_mask():
        m = mask
        if fused:
            # the attention kernel derives its work order from kv_len itself
            bsa.nabla_build_mask_lists(q, k, thr, s_valid=cfg.S_valid, out=(mask, kv_len, kv_idx, None),
                                       ws=lists_ws, **sta_kw)
            st["m"], st["wo"] = m, None
            return
        if use_nabla and not fp8 and cfg.sta is not None:
            # NABLA OR sliding tiles in one call (the rule inside the selection where the
            # layout allows it)
            bsa.nabla_build_mask_sta(q, k, thr, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                     order_tile=cfg.order_tile, s_valid=cfg.S_valid, out=mask)
            st["m"] = m
            return
        if cfg.sta is not None and not dense:
            bsa.sta_build_mask(S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                               order_tile=cfg.order_tile, device=dev, out=plane)
        if use_nabla and fp8 and rotate:
            bsa.nabla_build_mask_fp8_rotated(q, k, thr, signs, or_mask=plane if cfg.sta is not None else None,
                                             out=mask, q8_out=(qa, qs), k8_out=(ka, ks))
        elif use_nabla and fp8:
            bsa.nabla_build_mask_fp8(q, k, thr, or_mask=plane if cfg.sta is not None else None, out=mask,
                                     q8_out=(qa, qs), k8_out=(ka, ks))
        elif use_nabla:
            bsa.nabla_build_mask(q, k, thr, or_mask=plane if cfg.sta is not None else None, out=mask)
        else:
            m = ones if dense else plane
            if fp8:
                quantize_qk()
        st["m"] = m

    def phase_csr():
        if fused:
            return      # built by the mask phase
        # kv lists, and the attention work order where the shape has one (one call)
        st["rp"], st["ci"] = bsa.mask_to_csr(st["m"], B=cfg.B, H=cfg.H, row_ptr=row_ptr, col_idx=col_idx, ws=csr_ws,
                                             work_order=work_order)
        st["wo"] = work_order

    def phase_attn():
        if fused:
            bsa.block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, s_valid=cfg.S_valid, out=out, ws=attn_ws,
                                            work_order=st["wo"])
            return
        bsa.block_sparse_attn_fwd_csr(qa, ka, v, st["rp"], st["ci"], s_valid=cfg.S_valid, q_scale=qs, k_scale=ks,
                                      out=out, ws=attn_ws, work_order=st["wo"])

    def step(ev=None):
        for x, fn in enumerate((phase_mask, phase_csr, phase_attn)):
            if ev is not None:
                ev[x].record()
            fn()
        if ev is not None:
            ev[3].record()
        return st["m"], (kv_len if fused else st["rp"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if graph:
        # one step captured as a HIP graph (the library allocates nothing, never syncs
        # and records no memset), replayed once per timed step: the kernels and their
        # order are the eager step's, without the host's per-launch overhead
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        ref = out.clone()            # the eager step's output (also with no warmup steps)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            m_g, rp_g = step()

        def run():
            g.replay()
            return m_g, rp_g
    # timed region: whole steps back to back, events only at its two ends
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_all0.record()
    for s in range(steps):
        m, rp = run()
    t_all1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = t_all0.elapsed_time(t_all1)
    if graph and not torch.equal(out, ref):
        raise RuntimeError("graph replay output differs from the eager step")
    # phase breakdown in a second pass of the same steps, with events between the phases
    # (each event adds a few microseconds of its own, so it is kept out of the timed region)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for s in range(steps):
        step(evs[s])
    torch.cuda.synchronize()
    per_step = sorted(e[0].elapsed_time(e[3]) for e in evs)
    eager_ms = {name: sum(e[x].elapsed_time(e[x + 1]) for e in evs) / steps
                for x, name in enumerate(("mask", "csr", "attn"))}
    # Device time of each phase: in the eager pass the host's marshalling of a call can
    # leave the GPU idle after a phase event, and the event pair counts that. Here the
    # phase runs `steps` times back to back after one call queued ahead, one event pair
    # around them: the host stays ahead of the GPU, so the pair sees the kernels and the
    # gaps between them only. (A HIP graph of the repeated calls reads higher at the
    # 2B-DiT shape: 238 us per attention launch against 222-224 us in the kernel trace.)
    def phase_ms(fn):
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        fn()
        p0.record()
        for _ in range(steps):
            fn()
        p1.record()
        torch.cuda.synchronize()
        return p0.elapsed_time(p1) / steps

    mask_ms, csr_ms = phase_ms(phase_mask), phase_ms(phase_csr)
    with _SclkSampler() as clk_attn:      # the shader clock while the attention repeats run
        attn_ms = phase_ms(phase_attn)
    kept = int(rp.sum().item()) if fused else int(rp[-1].item())
    # attention launches so far (warm-ups, timed steps, the eager pass, the phase repeats);
    # a kernel trace of this run splits its attention dispatches at this count
    n_attn = warmup + (1 if graph else 0) + steps + steps + steps + 1
    dense_ms = None
    clk_dense = None
    if dense_reps and not dense:
        # dense attention of the same shape: the same kernel and call over an all-ones mask,
        # after the sparse launches (one warm-up, then dense_reps timed back to back)
        ones_rp, ones_ci = bsa.mask_to_csr(ones, B=cfg.B, H=cfg.H, row_ptr=row_ptr, col_idx=col_idx, ws=csr_ws)
        qd, kd = qa, ka
        if fp8:
            quantize_qk()

        def dense_attn():
            bsa.block_sparse_attn_fwd_csr(qd, kd, v, ones_rp, ones_ci, s_valid=cfg.S_valid, q_scale=qs, k_scale=ks,
                                          out=out, ws=attn_ws)
        dense_attn()
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with _SclkSampler() as clk_dense:
            d0.record()
            for _ in range(dense_reps):
                dense_attn()
            d1.record()
            torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / dense_reps
    return dict(ms_per_step=ms_total / steps, wall_s=wall, mask_ms=mask_ms, csr_ms=csr_ms, attn_ms=attn_ms,
                dense_ms=dense_ms, sclk_attn=clk_attn.summary(), sclk_dense=clk_dense.summary() if clk_dense else None,
                attn_launches={"sparse": n_attn, "dense": (1 + dense_reps) if dense_ms else 0},
                eager_phase_ms=eager_ms, kv_lists="from the mask build" if fused else "compaction launch",
                step_ms_median=per_step[len(per_step) // 2], step_ms_min=per_step[0],
                kept_tiles=kept, kept_fraction=kept / (cfg.B * cfg.H * nb * nb), mask=m.cpu() if use_nabla else None,
                q=q, k=k, v=v, qa=qa, ka=ka, qs=qs, ks=ks)


class _SclkSampler:
    """Samples the shader clock the driver reports (pp_dpm_sclk, the starred level) from a host
    thread while the block runs; summary() gives the median, min and max in MHz of the card
    with the highest median (the busy one), or None where the file is not readable."""

    def __init__(self, period_s=0.02):
        import glob
        self.files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.period = period_s
        self.samples = {f: [] for f in self.files}

    def _read(self, f):
        try:
            with open(f) as fh:
                for ln in fh:
                    if "*" in ln:
                        return float(ln.split(":", 1)[1].lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _loop(self):
        while not self._stop.is_set():
            for f in self.files:
                v = self._read(f)
                if v is not None:
                    self.samples[f].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._loop, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join()

    def summary(self):
        best = None
        for f, v in self.samples.items():
            if v:
                v = sorted(v)
                cur = {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v)}
                if best is None or cur["median"] > best["median"]:
                    best = cur
        return best


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def run_cpu_baseline(cfg, thr, budget_s=15.0):
    """The fp64 oracle (as it stands) on a bounded sample: whole heads, mask + attention."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    from synth import make_inputs, get_config
    c1 = get_config(cfg.cid, heads=min(cfg.H, 2))
    q, k, v = make_inputs(c1, seed=0, device="cpu")
    plane = None
    if cfg.sta is not None:
        plane = oracle.sta_block_mask(cfg.grid, cfg.order, cfg.order_tile, cfg.sta.tile, cfg.sta.window, 64, cfg.S)
    flops, heads, blocks_done = 0.0, 0, 0
    t_mask = t_attn = 0.0
    t0 = time.perf_counter()
    for h in range(c1.H):
        qh, kh, vh = (x[0, h].double().numpy() for x in (q, k, v))
        tm = time.perf_counter()
        if thr is not None:
            keep, _, _ = oracle.nabla_mask(qh, kh, 64, thr)
            if plane is not None:
                keep = keep | plane
        else:
            keep = plane
        t_mask += time.perf_counter() - tm
        # attention on as many query blocks as the budget allows (whole head when possible)
        for i0 in range(0, cfg.nb, 32):
            blocks = list(range(i0, min(cfg.nb, i0 + 32)))
            ta = time.perf_counter()
            oracle.block_sparse_attention(qh, kh, vh, keep, 64, cfg.S_valid, q_blocks=blocks)
            t_attn += time.perf_counter() - ta
            flops += keep[blocks].sum() * _flops_per_tile(cfg.D)
            blocks_done += len(blocks)
            if time.perf_counter() - t0 > budget_s:
                break
        heads += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    per_block = t_attn / max(blocks_done, 1)
    full = t_mask / heads * cfg.B * cfg.H + per_block * cfg.B * cfg.H * cfg.nb
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "cpu_model": _cpu_model(),
            "kind": "oracle",
            "oracle_s_per_head_mask": round(t_mask / heads, 4), "oracle_s_per_query_block": round(per_block, 6),
            "extrapolated_full_oracle_s": round(full, 1),
            "sample": f"{cfg.name}: NABLA/STA mask of {heads} head(s) + attention of {blocks_done} query blocks "
                      f"in fp64 numpy ({dt:.1f} s)"}


def run_backward(cfg, steps, warmup, thr, cpu_baseline=True):
    """Backward pass (dq, dk, dv) of the block-sparse attention for the config's mask.

    The mask, the forward output and lse are built once; the timed region is K calls
    of block_sparse_attn_bwd (delta pre-pass, both index lists, dK/dV and dQ kernels).
    Effective TFLOP/s counts the usual five 64x64xD products per kept tile (S, dP, dV,
    dK, dQ = 2.5x the forward's flops); the kernels compute S and dP twice (once for
    dK/dV, once for dQ), which that count leaves out."""
    import torch
    import block_sparse_attention_mask_amd as bsa
    from synth import make_inputs

    bsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(cfg, seed=0, device=dev)
    do = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(1)).to(torch.bfloat16).to(dev)
    plane = None
    if cfg.sta is not None:
        plane = bsa.sta_build_mask(cfg.S, cfg.S_valid, cfg.grid, cfg.sta.tile, cfg.sta.window, order=cfg.order,
                                   order_tile=cfg.order_tile, device=dev)
    mask = bsa.nabla_build_mask(q, k, thr, or_mask=plane) if thr is not None else plane
    o, lse = bsa.block_sparse_attn_fwd(q, k, v, mask, s_valid=cfg.S_valid, return_lse=True)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    import ctypes
    shp = bsa.Shape(cfg.B, cfg.H, cfg.S, cfg.S_valid, cfg.D, 64)
    ws = torch.empty(max(256, bsa.load().attn_bwd_workspace_size(ctypes.byref(shp))), dtype=torch.uint8, device=dev)

    def bwd():
        bsa.block_sparse_attn_bwd(q, k, v, o, do, lse, mask, s_valid=cfg.S_valid, out=grads, ws=ws)

    def fwd():
        bsa.block_sparse_attn_fwd(q, k, v, mask, s_valid=cfg.S_valid, return_lse=True)

    res = {}
    for name, fn in (("bwd", bwd), ("fwd", fwd)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    m = mask.expand(cfg.B, cfg.H, cfg.nb, cfg.nb) if mask.dim() == 2 else mask
    kept = int(m.sum().item())
    fpt = _flops_per_tile(cfg.D)
    tf = 2.5 * kept * fpt / (res["bwd"] * 1e-3) / 1e12
    line = {
        "metric": "sparse attn backward effective TFLOP/s (kept tiles, 5 products per tile)",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(res["bwd"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Q/K/V with smooth positional term; dO ~ N(0,1))",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "S": cfg.S, "S_valid": cfg.S_valid, "D": cfg.D,
                   "thr": thr, "sta": cfg.sta is not None, "pass": "backward"},
        "fwd_ms_same_call_path": round(res["fwd"], 4), "bwd_over_fwd": round(res["bwd"] / res["fwd"], 3),
        "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4), "kept_tiles": kept,
        "kept_fraction": round(kept / (cfg.B * cfg.H * cfg.nb * cfg.nb), 5),
    }
    if cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline_bwd(cfg, m[0].cpu().numpy().astype(bool))
    print(json.dumps(line), flush=True)


def run_cpu_baseline_bwd(cfg, keep0, budget_s=15.0):
    """The fp64 gradient oracle (as it stands) on a bounded sample: runs of 8 query blocks
    of head 0 with their dq (the oracle then forms S, P V, dP and dS K for those rows:
    4 of the 64x64xD products per kept tile), until the budget is spent."""
    import numpy as np
    import oracle
    from synth import make_inputs, get_config
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    c1 = get_config(cfg.cid, heads=1)
    q, k, v = make_inputs(c1, seed=0, device="cpu")
    qh, kh, vh = (x[0, 0].double().numpy() for x in (q, k, v))
    do = np.random.default_rng(1).standard_normal((cfg.S, cfg.D))
    flops, blocks_done = 0.0, 0
    t0 = time.perf_counter()
    for i0 in range(0, cfg.nb, 8):
        blocks = list(range(i0, min(cfg.nb, i0 + 8)))
        oracle.block_sparse_attention_bwd(qh, kh, vh, do, keep0[0], 64, cfg.S_valid, q_blocks=blocks, kv_blocks=[])
        flops += 2.0 * keep0[0][blocks].sum() * _flops_per_tile(cfg.D)
        blocks_done += len(blocks)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{cfg.name}: dq of {blocks_done} query blocks of head 0 in fp64 numpy ({dt:.1f} s; "
                      f"4 products per kept tile)"}


def run_reorder(cfg, steps, warmup):
    """Token reordering of Q at the config's shape: row-major -> tile-major (the config's
    sliding tile, else 4 x 8 x 8) and back; HBM roofline (every row read and written once)."""
    import torch
    import block_sparse_attention_mask_amd as bsa
    from synth import make_inputs

    bsa.load()
    dev = torch.device("cuda:0")
    q, _, _ = make_inputs(cfg, seed=0, device=dev)
    tile = cfg.sta.tile if cfg.sta is not None else (4, 8, 8)
    y = torch.empty_like(q)
    z = torch.empty_like(q)
    res = {}
    for name, fn in (("forward", lambda: bsa.token_reorder(q, cfg.grid, "tile", tile, out=y)),
                     ("inverse", lambda: bsa.token_reorder(y, cfg.grid, "tile", tile, inverse=True, out=z))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    if not torch.equal(z[:, :, :cfg.S_valid], q[:, :, :cfg.S_valid]):
        raise RuntimeError("reorder round trip failed")
    nbytes = 2 * q.numel() * q.element_size()
    gbps = nbytes / (res["forward"] * 1e-3) / 1e9
    print(json.dumps({"metric": "token reorder GB/s (read + write of every row)", "value": round(gbps, 1),
                      "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
                      "ms_per_step": round(res["forward"], 4), "higher_is_better": True, "scaling": "weak",
                      "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": cfg.name, "grid": list(cfg.grid), "tile": list(tile), "B": cfg.B,
                                 "H": cfg.H, "S": cfg.S, "D": cfg.D},
                      "inverse_ms": round(res["inverse"], 4),
                      "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                   "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                                   "kernel": "token_reorder_kernel", "per_launch_bytes": nbytes}}), flush=True)


def run_topk_compare(cfg, steps, warmup, thr):
    """CDF thresholding vs Top-k at equal average retained blocks (the comparison of the
    NABLA review's Appendix C): k = the CDF mask's mean kept count per row. For each
    scorer: mask-build time, kept fraction, attention time, and the L1 distance of
    sampled query blocks' attention output from dense attention (fp64 oracle)."""
    import numpy as np
    import torch
    import oracle
    import block_sparse_attention_mask_amd as bsa
    from synth import make_inputs

    bsa.load()
    dev = torch.device("cuda:0")
    q, k, v = make_inputs(cfg, seed=0, device=dev)
    cdf = bsa.nabla_build_mask(q, k, thr)
    kk = int(round(cdf.float().sum(-1).mean().item()))
    builders = {"cdf": lambda: bsa.nabla_build_mask(q, k, thr, out=cdf),
                "topk": lambda: bsa.nabla_build_mask_topk(q, k, kk)}
    heads, blocks = [0, cfg.H - 1], [0, cfg.nb // 3, 2 * cfg.nb // 3]
    dense = {}
    for h in heads:
        qd, kd, vd = (x[0, h].double().cpu().numpy() for x in (q, k, v))
        dense[h] = oracle.block_sparse_attention(qd, kd, vd, np.ones((cfg.nb, cfg.nb), bool), 64, cfg.S_valid,
                                                 q_blocks=blocks)[0]
    for name, build in builders.items():
        for _ in range(warmup):
            m = build()
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        for _ in range(steps):
            m = build()
        e[1].record()
        for _ in range(steps):
            bsa.block_sparse_attn_fwd(q, k, v, m, s_valid=cfg.S_valid)
        e[2].record()
        torch.cuda.synchronize()
        mask_ms, attn_ms = e[0].elapsed_time(e[1]) / steps, e[1].elapsed_time(e[2]) / steps
        mk = m.cpu().numpy().astype(bool)
        l1 = []
        for h in heads:
            qd, kd, vd = (x[0, h].double().cpu().numpy() for x in (q, k, v))
            O = oracle.block_sparse_attention(qd, kd, vd, mk[0, h], 64, cfg.S_valid, q_blocks=blocks)[0]
            rows = np.concatenate([np.arange(i * 64, min((i + 1) * 64, cfg.S_valid)) for i in blocks])
            l1.append(np.abs(O[rows] - dense[h][rows]).sum(axis=1).mean())
        kept = int(mk.sum())
        print(json.dumps({"compare": "cdf_vs_topk", "workload": cfg.name, "scorer": name, "thr": thr, "topk": kk,
                          "kept_fraction": round(kept / mk.size, 5), "mask_ms": round(mask_ms, 4),
                          "attn_ms": round(attn_ms, 4),
                          "attn_tflops": round(kept * _flops_per_tile(cfg.D) / (attn_ms * 1e-3) / 1e12, 1),
                          "mean_row_l1_vs_dense": float(np.mean(l1))}), flush=True)


def run_sweep(cfg_id, steps, warmup):
    """Threshold sweep (the combined-sweep workload): for each thr, with bf16 and with fp8
    Q/K, the kept fraction, step and attention time, effective TFLOP/s over kept tiles,
    speedup over dense attention of the same shape, the error of sampled query blocks
    against the fp64 oracle with the same mask, and how far that oracle output lies from
    the fp64 dense output (what the sparsification itself changes). Prints a markdown
    table and one JSON line per row."""
    import numpy as np
    import torch
    import oracle
    import block_sparse_attention_mask_amd as bsa
    from synth import get_config, make_inputs

    cfg = get_config(cfg_id)
    fpt = _flops_per_tile(cfg.D)
    q, k, v = make_inputs(cfg, seed=0, device="cuda:0")
    heads = [0, cfg.H - 1]
    blocks = [0, cfg.nb // 2, cfg.nb - 1]                  # includes the partly padded last block
    rows = []
    for fp8 in (False, True):
        peak = BF16_PEAK_TFLOPS if not fp8 else 4.0 / (2.0 / FP8_PEAK_TFLOPS + 2.0 / BF16_PEAK_TFLOPS)
        dense = run_gpu(cfg, steps, warmup, None, dense=True, fp8=fp8)
        dense_tf = dense["kept_tiles"] * fpt / (dense["attn_ms"] * 1e-3) / 1e12
        rows.append({"qk": "fp8" if fp8 else "bf16", "thr": "dense", "kept_fraction": 1.0,
                     "step_ms": dense["attn_ms"], "attn_ms": dense["attn_ms"], "attn_tflops": dense_tf,
                     "frac_peak": dense_tf / peak, "speedup_vs_dense": 1.0, "attn_speedup_vs_dense": 1.0,
                     "max_err": None, "mean_err": None,
                     "sampled_kept_blocks": None, "max_sparsify_err": None})
        for thr in cfg.thrs:
            r = run_gpu(cfg, steps, warmup, thr, fp8=fp8)
            qa, ka, qs, ks = r["qa"], r["ka"], r["qs"], r["ks"]      # the step's own fp8 codes (or bf16 q, k)
            tf = r["kept_tiles"] * fpt / (r["attn_ms"] * 1e-3) / 1e12
            # error of sampled query blocks against the fp64 oracle, with the GPU's mask
            mask = r["mask"].to("cuda:0")
            out = bsa.block_sparse_attn_fwd(qa, ka, v, mask, s_valid=cfg.S_valid, q_scale=qs, k_scale=ks)
            torch.cuda.synchronize()
            errs, sparsify = [], []
            for h in heads:
                if fp8:
                    qd = (qa[0, h].view(torch.float8_e4m3fn).double().view(cfg.nb, 64, cfg.D) * qs[0, h].double()[:, None, None]).view(cfg.S, cfg.D)
                    kd = (ka[0, h].view(torch.float8_e4m3fn).double().view(cfg.nb, 64, cfg.D) * ks[0, h].double()[:, None, None]).view(cfg.S, cfg.D)
                else:
                    qd, kd = q[0, h].double(), k[0, h].double()
                O, _ = oracle.block_sparse_attention(qd.cpu().numpy(), kd.cpu().numpy(), v[0, h].double().cpu().numpy(),
                                                     r["mask"][0, h].numpy().astype(bool), 64, cfg.S_valid, q_blocks=blocks)
                Od, _ = oracle.block_sparse_attention(qd.cpu().numpy(), kd.cpu().numpy(), v[0, h].double().cpu().numpy(),
                                                      np.ones((cfg.nb, cfg.nb), bool), 64, cfg.S_valid, q_blocks=blocks)
                for i in blocks:
                    sl = slice(i * 64, min((i + 1) * 64, cfg.S_valid))
                    errs.append(np.abs(out[0, h, sl].double().cpu().numpy() - O[sl]))
                    sparsify.append(np.abs(O[sl] - Od[sl]))
            e = np.concatenate([x.ravel() for x in errs])
            sp = np.concatenate([x.ravel() for x in sparsify])
            sampled_kept = int(sum(int(r["mask"][0, h, i].sum()) for h in heads for i in blocks))
            rows.append({"qk": "fp8" if fp8 else "bf16", "thr": thr, "kept_fraction": r["kept_fraction"],
                         "step_ms": r["ms_per_step"], "attn_ms": r["attn_ms"], "attn_tflops": tf,
                         "frac_peak": tf / peak, "speedup_vs_dense": dense["attn_ms"] / r["ms_per_step"],
                         "attn_speedup_vs_dense": dense["attn_ms"] / r["attn_ms"],
                         "max_err": float(e.max()), "mean_err": float(e.mean()), "sampled_kept_blocks": sampled_kept,
                         "max_sparsify_err": float(sp.max())})
    print(f"| Q/K | thr | kept | step ms | attn ms | attn TFLOP/s | of peak | speedup vs dense (step) "
          f"| speedup vs dense (attention) | max err | mean err | kv blocks of the sampled rows "
          f"| max oracle sparse - dense |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for x in rows:
        err = "" if x["max_err"] is None else f"{x['max_err']:.2e} | {x['mean_err']:.2e}"
        print(f"| {x['qk']} | {x['thr']} | {100 * x['kept_fraction']:.1f}% | {x['step_ms']:.2f} | {x['attn_ms']:.2f} | "
              f"{x['attn_tflops']:.0f} | {100 * x['frac_peak']:.1f}% | {x['speedup_vs_dense']:.2f}x | "
              f"{x['attn_speedup_vs_dense']:.2f}x | "
              f"{err if err else '- | -'} | {x['sampled_kept_blocks'] if x['sampled_kept_blocks'] is not None else '-'} | "
              f"{'-' if x['max_sparsify_err'] is None else format(x['max_sparsify_err'], '.2e')} |")
    for x in rows:
        print(json.dumps({"sweep": cfg.name, **{kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in x.items()}}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload 1-5 (default 3, the 14B 720p shape)")
    ap.add_argument("--dense-reps", type=int, default=3,
                    help="timed launches of dense attention (all-ones mask, same kernel) after the sparse ones; "
                         "0 skips the dense comparison")
    ap.add_argument("--thr", type=float, default=None, help="NABLA threshold (default: the config's first)")
    ap.add_argument("--fp8", action="store_true", help="fp8 e4m3 Q/K with per-block scales (config 5 run)")
    ap.add_argument("--rotate", action="store_true",
                    help="with --fp8: Hadamard rotation of Q and K before the quantisation (incoherent processing)")
    ap.add_argument("--dense", action="store_true", help="all-ones mask (dense comparison)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--csr-step", action="store_true",
                    help="kv lists from a compaction launch over the mask instead of from the mask build")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as a HIP graph (checked against the eager step) instead of eager launches")
    ap.add_argument("--topk-compare", action="store_true",
                    help="CDF vs Top-k masks at equal average kept blocks (default config 3)")
    ap.add_argument("--reorder", action="store_true",
                    help="time the token reordering (row-major -> tile-major and back) at the config's shape")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dq, dk, dv) of the config instead of the forward step")
    ap.add_argument("--sweep", action="store_true",
                    help="threshold sweep of the config (default 5) with bf16 and fp8 Q/K: table, not the bench line")
    ap.add_argument("--kv-chunk", type=int, default=0, metavar="W",
                    help="attention over the kv-chunked walk with chunks of W key blocks (bsa_set_attn_kv_chunk); "
                         "attn_ms then includes the combine launch")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (the path shards by "
              f"(batch, head) with no communication, see the design notes)", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        run_sweep(args.config if args.config != 3 else 5, min(args.steps, 5), min(args.warmup, 2))
        return
    if args.topk_compare:
        from synth import get_config
        cfg = get_config(args.config)
        run_topk_compare(cfg, min(args.steps, 5), min(args.warmup, 2), args.thr or cfg.thrs[0])
        return
    if args.reorder:
        from synth import get_config
        run_reorder(get_config(args.config), args.steps, args.warmup)
        return
    if args.backward:
        from synth import get_config
        cfg = get_config(args.config)
        thr = args.thr if args.thr is not None else (cfg.thrs[0] if cfg.thrs else None)
        run_backward(cfg, args.steps, args.warmup, thr, cpu_baseline=not args.no_cpu_baseline)
        return
    from synth import get_config
    cfg = get_config(args.config)
    thr = args.thr if args.thr is not None else (cfg.thrs[0] if cfg.thrs else None)
    if args.kv_chunk:
        import block_sparse_attention_mask_amd as bsa
        bsa.set_attn_kv_chunk(args.kv_chunk)
    if args.rotate and not args.fp8:
        ap.error("--rotate needs --fp8")
    r = run_gpu(cfg, args.steps, args.warmup, thr, dense=args.dense, fp8=args.fp8, graph=args.graph,
                csr_step=args.csr_step, dense_reps=args.dense_reps, rotate=args.rotate)
    fpt = _flops_per_tile(cfg.D)
    kept_flops = r["kept_tiles"] * fpt
    attn_tflops = kept_flops / (r["attn_ms"] * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS
    if args.fp8:
        peak = 4.0 / (2.0 / FP8_PEAK_TFLOPS + 2.0 / BF16_PEAK_TFLOPS)   # fp8 QK^T + bf16 PV
    qk_bytes = 2 * cfg.B * cfg.H * cfg.S * cfg.D * (4 if cfg.dtype == "f32" else 2)
    mask_bytes = qk_bytes + cfg.B * cfg.H * cfg.nb * cfg.nb
    line = {
        "metric": "sparse attn effective TFLOP/s (kept tiles) + % bf16 MFMA peak; mask build GB/s",
        "value": round(kept_flops / (r["ms_per_step"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16" if args.fp8 else cfg.dtype,
        "data": "synthetic (seeded Q/K/V with smooth positional term)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "S": cfg.S, "S_valid": cfg.S_valid, "D": cfg.D,
                   "grid": list(cfg.grid), "token_order": cfg.order, "thr": thr,
                   "sta": None if cfg.sta is None else {"tile": list(cfg.sta.tile), "window": list(cfg.sta.window)},
                   "dense": args.dense, "fp8_qk": args.fp8, "fp8_rotation": args.rotate,
                   "launch": "hip_graph" if args.graph else "eager", "kv_chunk": args.kv_chunk or None},
        "attn_ms": round(r["attn_ms"], 4), "mask_ms": round(r["mask_ms"], 4), "csr_ms": round(r["csr_ms"], 4),
        "kv_lists": r["kv_lists"],
        # per-step spread and phase times from the eager pass with events between the phases
        "step_ms_median_eager": round(r["step_ms_median"], 4), "step_ms_min_eager": round(r["step_ms_min"], 4),
        "eager_phase_ms": {k: round(x, 4) for k, x in r["eager_phase_ms"].items()},
        "attn_tflops": round(attn_tflops, 2), "attn_frac_bf16_peak": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
        "mask_build_gbps": round(mask_bytes / (r["mask_ms"] * 1e-3) / 1e9, 1) if thr is not None else None,
        "mask_build_frac_hbm": round(mask_bytes / (r["mask_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        if thr is not None else None,
        # Q and K of back-to-back steps stay in the 256 MB last-level cache when they fit
        # in it: the mask-build rate is then not an HBM rate
        "mask_build_llc_resident": qk_bytes <= LLC_BYTES if thr is not None else None,
        "kept_fraction": round(r["kept_fraction"], 5), "kept_tiles": r["kept_tiles"],
        "attn_launches": r["attn_launches"],
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": round(peak, 1), "unit": "TFLOP/s",
                     "frac": round(attn_tflops / peak, 4),
                     "traffic": None if args.kv_chunk else _measured_traffic(cfg.name, args.fp8, args.dense),
                     "kernel": "attn_fwd_kernel", "per_launch_flops": kept_flops},
    }
    if r["dense_ms"]:
        dense_flops = cfg.B * cfg.H * cfg.nb * cfg.nb * fpt
        dense_tf = dense_flops / (r["dense_ms"] * 1e-3) / 1e12
        line["dense"] = {"attn_ms": round(r["dense_ms"], 4), "tflops": round(dense_tf, 2),
                         "frac_peak": round(dense_tf / peak, 4),
                         "speedup_step_vs_dense": round(r["dense_ms"] / r["ms_per_step"], 3),
                         "speedup_attn_vs_dense": round(r["dense_ms"] / r["attn_ms"], 3),
                         "reps": args.dense_reps}
    # The published peaks assume the 2400 MHz peak engine clock; the clock the part holds
    # under this load is lower, and the MFMA rate scales with it.
    if r["sclk_attn"]:
        ca = r["sclk_attn"]
        sc = {"source": "pp_dpm_sclk", "peak_assumes_mhz": PEAK_CLOCK_MHZ,
              "attn_mhz": ca, "attn_frac_of_peak_at_clock": round(attn_tflops / (peak * ca["median"] / PEAK_CLOCK_MHZ), 4)}
        if r["dense_ms"] and r["sclk_dense"]:
            cd = r["sclk_dense"]
            sc["dense_mhz"] = cd
            sc["dense_frac_of_peak_at_clock"] = round(line["dense"]["tflops"] / (peak * cd["median"] / PEAK_CLOCK_MHZ), 4)
        line["shader_clock"] = sc
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(cfg, None if args.dense else thr)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
