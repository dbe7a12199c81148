#!/usr/bin/env python3
"""Benchmark of the replay-free verify hot path on one MI355X.

A step is one pass of the whole path over one block: verify (short FIR,
outer FIR, modal IIR scan, split-K causal block attention over the KV
prefix), accept, and slice.  Default workload: the long-context layer --
d = 4096, 3/128 FIR taps, 16 poles, 32 heads x 128, a 262144-token bf16 KV
prefix, gamma = 12 (13 block positions), greedy acceptance with drafts
agreeing for a Geometric(0.7) prefix.  Inputs are resident in HBM before the
timed region starts.

Prints ONE JSON line (metric, value = verified block-positions per second,
roofline of the prefix-attention kernel, CPU oracle baseline, ...).

    python bench.py [--steps K] [--warmup W] [--config long262k|long262k_g6|mid8k|multi4x4|wide131k]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
WORKLOAD_NAMES = {
    "long262k": "long-context verify: d=4096, FIR 3/128 taps, 16 poles, 32x128 heads, 262144-token bf16 KV prefix, gamma=12, greedy",
    "long262k_g6": "long-context verify: d=4096, FIR 3/128 taps, 16 poles, 32x128 heads, 262144-token bf16 KV prefix, gamma=6, greedy",
    "mid8k": "mid-size verify: d=4096, FIR 3/128 taps, 16 poles, 32x128 heads, 8192-token bf16 KV prefix, gamma=12, sampling T=1",
    "multi4x4": "batched multi-candidate verify: 4 sequences x 4 candidates, KV prefixes 16384/32768/51200/65536, gamma=12, sampling",
    "wide131k": "wide layer: d=8192, FIR 3/128 taps, 16 poles, 64x128 heads, 131072-token bf16 KV prefix, gamma=12, greedy",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_stream_long262k_traffic.json")


def traffic_file(cfg_name: str) -> str:
    """Counter summary of the prefix-streaming kernel for one workload."""
    return os.path.join(ROOT, "profiles", f"verify_stream_{cfg_name}_traffic.json")


def _hip():
    lib = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch already loaded
    lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return lib


def _events(hip, n):
    evs = (ctypes.c_void_p * n)()
    for i in range(n):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs[i] = e
    return evs


def _ms(hip, a, b) -> float:
    out = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
    return float(out.value)


def verify_alg_bytes(cfg, kv_lens) -> int:
    """Bytes the verify must move: KV prefix once per sequence, block tensors, conv/IIR state and weights."""
    act = 2 if cfg.act == "bf16" else 4
    nq = cfg.nb * cfg.nc * cfg.P
    H, Dh, d, N = cfg.heads, cfg.head_dim, cfg.d, cfg.poles
    kv = sum(2 * H * L * Dh * act for L in kv_lens)
    attn_io = 4 * nq * H * Dh * act                                   # q, block k, block v in; o out
    conv = (nq * d * act                                              # x
            + cfg.nb * ((cfg.taps_short - 1) * d * act + (cfg.taps_outer - 1) * d * 4 + d * N * 4)  # windows, IIR
            + (cfg.taps_short + cfg.taps_outer) * d * 4 + 3 * d * N * 4                              # weights
            + nq * d * 4 + nq * d * N * 4 + nq * d * act)            # f, s, y out
    return kv + attn_io + conv


def stream_kernel_name(cfg) -> str:
    """The kernel that streams the KV prefix for this workload."""
    return "k_verify_stream" if cfg.act == "bf16" else "k_attn_prefix_f32"


def stream_alg_bytes(cfg, kv_lens) -> int:
    """Bytes the prefix-streaming kernel must move: the KV prefix once per sequence and the queries.

    512 B per (key, head) of the prefix (Dh bf16 K + Dh bf16 V), read once per sequence for all
    nc * P queries; the conv/IIR scan, the causal block part and the combine run in the finish kernel.
    """
    act = 2 if cfg.act == "bf16" else 4
    nq = cfg.nb * cfg.nc * cfg.P
    return sum(2 * cfg.heads * L * cfg.head_dim * act for L in kv_lens) + nq * cfg.heads * cfg.head_dim * act


VERIFY_SOURCES = ("stream_one.hip", "prefix_tile.h", "worklist.h", "hci_internal.h")
PREFILL_SOURCES = ("prefill.hip", "slice.hip", "hci_internal.h")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_long262k_traffic.json")


def _kernel_sha(sources=VERIFY_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "hybrid_conv_iir_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(cfg_name, path=TRAFFIC_FILE, sources=VERIFY_SOURCES, prompt=None):
    """Counter-measured HBM bytes per launch, or None once the kernel sources changed since."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != _kernel_sha(sources) or t.get("config") != cfg_name:
        return None
    if prompt is not None and t.get("prompt") != prompt:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(cfg, case_np, heads, reps):
    """The fp64 oracle as it stands, timed on this host on a bounded sample of the workload.

    The sample is one (sequence, candidate) block's verify -> accept -> slice with attention over
    `heads`, repeated `reps` times; time is scaled to all heads and all blocks of the workload.
    """
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    layer = oracle.Layer.from_dict(case_np["params"])
    small, bn, ri = case_np["small"], case_np["blk"], case_np["ri"]
    b, c = 0, 0
    x, q, k, v = bn["x"][b, c], bn["q"][b, c][:, heads], bn["k"][b, c][:, heads], bn["v"][b, c][:, heads]
    st = oracle.SeqState(small["short_win"][b], small["outer_win"][b], small["iir"][b],
                         [case_np["kpre"]], [case_np["vpre"]])
    t_conv = t_attn = t_acc = t_slice = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        f = oracle.depthwise_fir(x, st.short_win, layer.w_short)
        g = oracle.depthwise_fir(f, st.outer_win, layer.w_outer)
        s, y = oracle.modal_iir(g, st.iir, layer.lam, layer.beta, layer.c)
        t1 = time.perf_counter()
        oracle.block_attention(q, k, v, st.k_blocks, st.v_blocks)
        t2 = time.perf_counter()
        if cfg.mode == "greedy":
            kk, _, _ = oracle.greedy_accept(ri["target_logits"][b, c], ri["drafts"][b, c])
        else:
            kk, _, _ = oracle.rejection_accept(ri["target_logits"][b, c], ri["draft_logits"][b, c],
                                               ri["drafts"][b, c], ri["uniforms"][b, c], cfg.temperature)
        t3 = time.perf_counter()
        oracle.slice_state(st, x, {"f": f, "s": s}, k, v, kk)
        t4 = time.perf_counter()
        t_conv += t1 - t0
        t_attn += t2 - t1
        t_acc += t3 - t2
        t_slice += t4 - t3
    scale = cfg.heads / len(heads)
    blocks = cfg.nb * cfg.nc          # the sample is one (sequence, candidate) block
    measured = t_conv + t_attn + t_acc + t_slice
    est = (t_conv + t_attn * scale + t_acc + t_slice) / reps * blocks
    return {
        "value": round(cfg.nb * cfg.nc * cfg.P / est, 3),
        "unit": "verified block-positions/s",
        "cores": int(cores),
        "blas_threads": int(blas_threads),
        "threads_note": ("cores = host cores available to the process; the oracle's FIR, IIR, softmax and "
                         "acceptance loops run on one thread, only its matrix products use the BLAS threads"),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, verify->accept->slice of one block with attention over {len(heads)} of "
                   f"{cfg.heads} heads, {reps} repetitions (timed {measured:.1f} s"
                   f"{'; attention time scaled x%g to all heads' % scale if scale != 1 else ''}"
                   f"{'; x%d blocks' % blocks if blocks > 1 else ''})"),
        "seconds_per_step_est": round(est, 3),
    }



def prefill_alg_flops(cfg, T) -> float:
    """FIR then IIR as written, per position and channel: a multiply and an add per short and outer
    tap; per pole two multiplies and an add for the state update and a multiply-add for the readout."""
    return float(cfg.nb) * T * cfg.d * (2 * cfg.taps_short + 2 * cfg.taps_outer + 5 * cfg.poles)


def prefill_alg_bytes(cfg, T, want_y) -> float:
    """Prompt x, K/V rows in, K/V rows appended to the cache, outputs y if wanted, and the committed
    windows and IIR state read and written."""
    act = 2 if cfg.act == "bf16" else 4
    per_pos = cfg.d * act + 4 * cfg.heads * cfg.head_dim * act + (cfg.d * act if want_y else 0)
    state = 2 * cfg.d * ((cfg.taps_short - 1) * act + (cfg.taps_outer - 1) * 4 + cfg.poles * 4)
    weights = cfg.d * (cfg.taps_short + cfg.taps_outer + 2 * cfg.poles) * 4
    return float(cfg.nb) * (T * per_pos + state) + weights


def bench_prefill(args, cfg, hip):
    """Prompt -> committed state: chunked FIR + IIR scan, carry scan, window commit, KV append."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci, synth
    T, W, K = args.prompt, args.warmup, args.steps
    cfg = synth.scaled(cfg, kv_lens=(0,) * cfg.nb)
    lay = dv.DeviceLayer(cfg, synth.make_layer(cfg))
    st = dv.DeviceState(lay, cfg.nb, (T + 31) // 32 * 32)
    small = synth.make_state_small(cfg)
    pr = synth.prompt(cfg, T, device="cuda")
    at = hci.act_torch_dtype(lay.act)
    y = torch.empty((cfg.nb, T, cfg.d), dtype=at, device="cuda")
    ws = torch.empty(hci.prefill_workspace_bytes(lay.c, cfg.nb, T, True), dtype=torch.uint8, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream

    def one(with_y, evs=None):
        st.load_small(small)
        st.kv_len.zero_()
        if evs is not None:
            hip.hipEventRecord(evs[0], sp)
        hci.prefill(lay.c, st.c, cfg.nb, T, 0, pr["x"], pr["k"], pr["v"], y if with_y else None, ws)
        if evs is not None:
            hip.hipEventRecord(evs[1], sp)

    res = {}
    for with_y in (False, True):
        for _ in range(W):
            one(with_y)
        evsets = [_events(hip, 2) for _ in range(K)]
        for i in range(K):
            one(with_y, evsets[i])
        torch.cuda.synchronize()
        res[with_y] = float(np.median([_ms(hip, e[0], e[1]) for e in evsets]))
    # the practical copy ceiling beside the 8 TB/s read peak: a 1 GiB device-to-device copy by
    # hci_probe_copy (read + write bytes / its best time), the pattern the KV append follows
    csrc = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cdst = torch.empty_like(csrc)
    pe = _events(hip, 2)
    copy_ms = []
    for _ in range(4):
        hip.hipEventRecord(pe[0], sp)
        hci.probe_copy(cdst, csrc)
        hip.hipEventRecord(pe[1], sp)
        hip.hipEventSynchronize(pe[1])
        copy_ms.append(_ms(hip, pe[0], pe[1]))
    copy_gbs = 2.0 * csrc.numel() * 4 / (min(copy_ms[1:]) * 1e-3) / 1e9
    del csrc, cdst
    t_state = res[False] * 1e-3
    flops = prefill_alg_flops(cfg, T)
    achieved = flops / t_state / 1e12
    alg = prefill_alg_bytes(cfg, T, False)
    gbs = alg / t_state / 1e9
    out = {
        "metric": "prefill positions/sec per layer (prompt -> committed state)",
        "value": round(cfg.nb * T / t_state, 1),
        "unit": "positions/s",
        "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(res[False], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) prompt)",
        "config": {"workload": f"prefill of a {T}-token prompt into one hybrid layer "
                               f"(d={cfg.d}, FIR {cfg.taps_short}/{cfg.taps_outer} taps, {cfg.poles} poles, "
                               f"{cfg.heads}x{cfg.head_dim} heads)", "prompt": T, "nb": cfg.nb},
        "ms_with_outputs_y": round(res[True], 4),
        "hbm_GBs_with_outputs_y": round(prefill_alg_bytes(cfg, T, True) / (res[True] * 1e-3) / 1e9, 1),
        "fir_iir_TFLOPs_equivalent": round(achieved, 2),
        "hbm_probe_copy_GBs": round(copy_gbs, 1),
        "roofline": {"kernel": "hci_prefill, all launches (scan, state, KV append)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 4),
                     "traffic": _traffic(cfg.name, PREFILL_TRAFFIC_FILE, PREFILL_SOURCES, T),
                     "alg_bytes_per_launch": alg},
    }
    print(json.dumps(out), flush=True)


def bench_linear(args, hip):
    """y = x W for the verified block's rows: every weight byte read once per call (HBM-bound)."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import hci, synth
    M, K, N = (int(v) for v in args.linear_shape.split(","))
    x = synth.dense((M, K), 1.0, 1, device="cuda")
    w = synth.dense((K, N), K ** -0.5, 2, device="cuda")
    wps = []
    for _ in range(4):          # rotate weights so no call finds the previous one's bytes in the 256 MB MALL
        wp = torch.empty(hci.linear_packed_elems(K, N), dtype=torch.bfloat16, device="cuda")
        hci.linear_pack(w, wp)
        wps.append(wp)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    for i in range(args.warmup):
        hci.linear(x, wps[i % 4], N, y)
    evs = [_events(hip, 2) for _ in range(args.steps)]
    for i in range(args.steps):
        hip.hipEventRecord(evs[i][0], sp)
        hci.linear(x, wps[i % 4], N, y)
        hip.hipEventRecord(evs[i][1], sp)
    torch.cuda.synchronize()
    ms = float(np.median([_ms(hip, e[0], e[1]) for e in evs]))
    # the practical floor for the same bytes: the streaming read probe over the same four weight
    # copies in turn, one launch each, timed the same way
    sink = torch.empty(hci.probe_sink_words(), dtype=torch.float32, device="cuda")
    for i in range(args.warmup):
        hci.probe_read(wps[i % 4], sink)
    pevs = [_events(hip, 2) for _ in range(args.steps)]
    for i in range(args.steps):
        hip.hipEventRecord(pevs[i][0], sp)
        hci.probe_read(wps[i % 4], sink)
        hip.hipEventRecord(pevs[i][1], sp)
    torch.cuda.synchronize()
    read_ms = float(np.median([_ms(hip, e[0], e[1]) for e in pevs]))
    alg = 2.0 * (K * N + M * K + M * N)
    gbs = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": "dense projection rows/sec (weights streamed once per call)",
        "value": round(M / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) rows, N(0,1/K) weights)",
        "config": {"workload": f"y = x W with x {M}x{K}, W {K}x{N} bf16 (a block of {M} rows through a "
                               f"{K}->{N} projection)", "M": M, "K": K, "N": N},
        "read_probe_ms_same_bytes": round(read_ms, 5),
        "fraction_of_read_probe": round(read_ms / ms, 4),
        "roofline": {"kernel": "k_linear", "bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0,
                     "unit": "GB/s", "frac": round(gbs / 8000.0, 4), "traffic": None, "alg_bytes_per_launch": alg},
    }
    print(json.dumps(out), flush=True)


def model_alg_bytes(mc) -> float:
    """Bytes a stack verify must move: every projection weight once, each attention layer's KV prefix
    once per sequence, the committed windows and IIR states read, and the block tensors written
    (residual streams, in-projection streams, u / s) -- activations in bf16, retained tensors in fp32."""
    d, rows, N = mc.d, mc.rows, mc.poles
    total = 0.0
    for l, kind in enumerate(mc.kinds):
        total += 2.0 * (3 * d * d + d * d)                               # W_in, W_out
        total += rows * d * 2 * 2                                        # a and the new x
        if kind == "attn":
            total += sum(2.0 * 2 * L * d for L in mc.kv_lens)            # K and V prefix, bf16
            total += 3 * rows * d * 2 + rows * d * 2                     # q/k/v, o
        else:
            total += 3 * rows * d * 4 + rows * d * 2                     # z (fp32), y
            total += mc.nb * (mc.taps_short - 1) * 3 * d * 4             # short window
            if kind == "fir":
                total += rows * d * 4 + mc.nb * (mc.taps_long[l] - 1) * d * 4 + mc.taps_long[l] * d * 4
            else:
                total += rows * d * N * 4 + mc.nb * d * N * 4 + 3 * d * N * 4
    return total


def bench_model(args, hip):
    """One verify of the block through the whole layer stack (+ the slice), inputs resident."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import model as dm
    from hybrid_conv_iir_amd import synth
    mc = synth.MODEL_CONFIGS[args.model]
    params = synth.make_model(mc, 0, device="cuda")
    dmod = dm.DeviceModel(mc, params)
    del params
    st0 = synth.make_model_state(mc, 0, device="cuda")
    st = dm.DeviceModelState(dmod, (max(mc.kv_lens) + 64 + 31) // 32 * 32)
    st.load(st0)
    del st0
    blk = dm.DeviceModelBlock(dmod, mc.nb, mc.nc, mc.gamma)
    blk.set_input(synth.model_block_input(mc, 0, 0, device="cuda"))
    bound = max(mc.kv_lens)
    n_acc = torch.zeros((mc.nb, mc.nc), dtype=torch.int32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(args.warmup):
        dm.verify(dmod, st, blk, bound)
    evs = [_events(hip, 3) for _ in range(args.steps)]
    for i in range(args.steps):
        hip.hipEventRecord(evs[i][0], sp)
        dm.verify(dmod, st, blk, bound)
        hip.hipEventRecord(evs[i][1], sp)
        dm.slice_state(dmod, st, blk, bound, n_acc)              # commits k = 0 (one row): state changes
        hip.hipEventRecord(evs[i][2], sp)
        bound += 1
    torch.cuda.synchronize()
    v_ms = float(np.median([_ms(hip, e[0], e[1]) for e in evs]))
    s_ms = float(np.median([_ms(hip, e[1], e[2]) for e in evs]))
    alg = model_alg_bytes(mc)
    gbs = alg / (v_ms * 1e-3) / 1e9
    out = {
        "metric": "verified block-positions/sec through the layer stack",
        "value": round(mc.rows / (v_ms * 1e-3), 1), "unit": "block-positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(v_ms + s_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded weights, state and block rows; no trained weights)",
        "config": {"workload": f"{len(mc.kinds)}-layer stripe {'/'.join(mc.kinds)} at d={mc.d}, "
                               f"{mc.heads}x{mc.head_dim} heads, KV prefix {list(mc.kv_lens)}, gamma={mc.gamma}",
                   "layers": list(mc.kinds), "d": mc.d, "kv_len": list(mc.kv_lens), "gamma": mc.gamma},
        "verify_ms": round(v_ms, 4), "slice_ms": round(s_ms, 4),
        "roofline": {"kernel": "hci_model_verify, all launches", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4), "traffic": None,
                     "alg_bytes_per_launch": alg},
    }
    print(json.dumps(out), flush=True)


def bench_draft(args, hip):
    """Drafting one block: the trunk pass and the serial Markov-biased sampling, eagerly and as a
    replayed HIP graph (the whole draft is launch-bound: ~20 small launches)."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import drafter as ddr
    from hybrid_conv_iir_amd import synth
    dc = synth.DRAFTER_CONFIGS["d1k"]
    nb, gamma = 1, 12
    dd = ddr.DeviceDrafter(dc, synth.make_drafter(dc, 0, device="cuda"))
    rd = synth.draft_round(dc, nb, gamma, 0, 0, device="cuda")
    win, anchor, u = rd["window"], rd["anchor"].cuda(), rd["uniforms"].cuda()
    out = dd.buffers(nb, gamma)

    def timed(fn, stream):
        sp = stream.cuda_stream
        for _ in range(args.warmup):
            fn()
        evs = [_events(hip, 2) for _ in range(args.steps)]
        for i in range(args.steps):
            hip.hipEventRecord(evs[i][0], sp)
            fn()
            hip.hipEventRecord(evs[i][1], sp)
        torch.cuda.synchronize()
        return float(np.median([_ms(hip, e[0], e[1]) for e in evs]))

    cur = torch.cuda.current_stream()
    eager_ms = timed(lambda: dd.draft(win, anchor, u, 1.0, out), cur)
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        dd.draft(win, anchor, u, 1.0, out, stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            dd.draft(win, anchor, u, 1.0, out, stream=s)
    cur.wait_stream(s)
    graph_ms = timed(graph.replay, cur)
    d, F, L = dc.d, dc.ffn, dc.layers
    weights = 2.0 * (dc.d_target * d + L * (3 * d * d + d * d + 2 * d * F) + d * dc.vocab)
    alg = weights + 2.0 * nb * dc.window * dc.d_target + 4.0 * dc.vocab * dc.vocab
    gbs = alg / (graph_ms * 1e-3) / 1e9
    out_json = {
        "metric": "drafted blocks/sec (trunk + serial sampling, graph replay)",
        "value": round(nb / (graph_ms * 1e-3), 1), "unit": "blocks/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(graph_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded weights and window; no trained drafter)",
        "config": {"workload": f"drafter d={d}, {dc.heads}x{dc.head_dim} heads, ffn {F}, {L} layers, "
                               f"window {dc.window} x {dc.d_target}, vocab {dc.vocab}, gamma={gamma}, nb={nb}"},
        "eager_ms": round(eager_ms, 4), "graph_ms": round(graph_ms, 4),
        "roofline": {"kernel": "hci_draft_logits + hci_draft_sample (launch-bound)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                     "traffic": None, "alg_bytes_per_launch": alg},
    }
    print(json.dumps(out_json), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="long262k", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU-oracle sample (0 = all)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="repetitions of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="verify", choices=["verify", "prefill", "linear", "model", "draft", "tree"],
                    help="verify: the verify->accept->slice step (default); prefill: prompt -> committed state; "
                         "linear: one dense projection of the verified block; tree: the candidate blocks of "
                         "--config merged into token trees (tree verify -> accept -> slice), beside the chain step")
    ap.add_argument("--tree-vocab", type=int, default=4,
                    help="alphabet of the drafted tokens in --mode tree (4: nucleotides)")
    ap.add_argument("--linear-shape", default="13,4096,12288", help="M,K,N for --mode linear")
    ap.add_argument("--model", default="m4_long", help="layer stack for --mode model")
    ap.add_argument("--prompt", type=int, default=262144, help="prompt length for --mode prefill")
    ap.add_argument("--replay-reps", type=int, default=3, help="repetitions of the replay-equivalent timing")
    ap.add_argument("--event-every", type=int, default=4,
                    help="time the streaming kernel with events on every n-th timed step")
    ap.add_argument("--accept-rounds", type=int, default=64,
                    help="seeded rounds of hci_accept for the k histogram / survival curve (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run the known-size copy kernel once on this many MiB (byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    hip = _hip()
    cfg = synth.CONFIGS[args.config]
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        csrc = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        cdst = torch.empty_like(csrc)
        hci.probe_copy(cdst, csrc)
        torch.cuda.synchronize()
        del csrc, cdst
    if args.mode == "prefill":
        return bench_prefill(args, cfg, hip)
    if args.mode == "linear":
        return bench_linear(args, hip)
    if args.mode == "model":
        return bench_model(args, hip)
    if args.mode == "draft":
        return bench_draft(args, hip)
    if args.mode == "tree":
        return bench_tree(args, cfg, hip)
    return bench_verify(args, cfg, hip)


MALL_BYTES = 256 << 20          # MI355X Infinity Cache; a prefix below this could be served from it


def kv_sets_for(cfg) -> int:
    """KV sets the timed steps rotate over: one when the workload's KV prefix is far larger than the
    256 MB MALL, otherwise enough copies (at least 3) that together they exceed 1 GiB, so that no step
    finds its prefix left in the MALL by the previous one."""
    act = 2 if cfg.act == "bf16" else 4
    kv = sum(2 * cfg.heads * L * cfg.head_dim * act for L in cfg.kv_lens)
    if kv >= 4 * MALL_BYTES:
        return 1
    return int(min(16, max(3, -(-(1 << 30) // max(kv, 1)))))


def acceptance_stats(cfg, rounds, hip):
    """k histogram, survival curve and smallest decision margin of hci_accept over `rounds` seeded
    rounds of this workload's synthetic logits and drafts (fresh inputs per round)."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci, synth
    mode = hci.GREEDY if cfg.mode == "greedy" else hci.SAMPLE
    acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    ks, margins = [], []
    for r in range(1, rounds + 1):
        ri = synth.round_inputs(cfg, synth.anchors(cfg, r), r)
        acc.set_inputs(ri["target_logits"], ri["drafts"], ri["draft_logits"], ri["uniforms"])
        dv.accept(acc, mode, cfg.temperature)
        n_acc, best, marg = (dv.to_host(t) for t in (acc.n_acc, acc.best, acc.margin))
        for b in range(cfg.nb):
            ks.append(int(n_acc[b, int(best[b])]))
        margins.append(float(np.min(marg)))
    hist = np.bincount(np.asarray(ks), minlength=cfg.gamma + 1)[: cfg.gamma + 1]
    n = len(ks)
    return {"rounds": rounds, "blocks": n,
            "k_histogram": [int(v) for v in hist],
            "survival": [round(float(np.sum(np.asarray(ks) >= j)) / n, 4) for j in range(1, cfg.gamma + 1)],
            "mean_accepted_drafts": round(float(np.mean(ks)), 3),
            "min_decision_margin": float(np.min(margins)),
            "margin_note": ("greedy: smallest top-1 logit gap of the rows read" if cfg.mode == "greedy" else
                            "sampling: smallest relative distance of a ratio test or inverse-CDF draw from its "
                            "threshold")}


def bench_verify(args, cfg, hip):
    """verify -> accept -> slice steps on inputs resident in HBM (the metric's workload)."""
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci, synth
    W, K = args.warmup, args.steps
    P = cfg.P
    n_sets = kv_sets_for(cfg)
    per_set = (W + 2 * K) // n_sets + 2
    kv_cap = (cfg.max_kv_len + (per_set + 2) * P + 31) // 32 * 32

    # ---------------------------------------------------------------- inputs (resident before timing)
    params = synth.make_layer(cfg)
    small = synth.make_state_small(cfg)
    tables = synth.make_tables(cfg)
    anchor = synth.anchors(cfg)
    ri = synth.round_inputs(cfg, anchor)
    bn = synth.gather_block(cfg, tables, ri["tokens"])
    lay = dv.DeviceLayer(cfg, params)
    heads = list(range(cfg.heads if args.cpu_heads <= 0 else min(args.cpu_heads, cfg.heads)))
    kpre_host = vpre_host = None
    sets = []
    for si in range(n_sets):
        st = dv.DeviceState(lay, cfg.nb, kv_cap)
        st.load_small(small)
        for b in range(cfg.nb):
            kp = synth.kv_prefix(cfg, b, "k", device="cuda")
            vp = synth.kv_prefix(cfg, b, "v", device="cuda")
            st.write_prefix(b, kp, vp)
            if si == 0 and b == 0 and not args.no_cpu_baseline:
                kpre_host, vpre_host = dv.to_host(kp[heads]), dv.to_host(vp[heads])
            del kp, vp
        st.kv_len.copy_(torch.tensor(cfg.kv_lens, dtype=torch.int32))
        sets.append(st)
    blk = dv.DeviceBlock(lay, cfg.nb, cfg.nc, cfg.gamma)
    blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
    acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    acc.set_inputs(ri["target_logits"], ri["drafts"], ri["draft_logits"], ri["uniforms"])
    mode = hci.GREEDY if cfg.mode == "greedy" else hci.SAMPLE
    bounds = [cfg.max_kv_len] * n_sets
    blk.ensure_workspace(kv_cap - P)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    # ---------------------------------------------------------------- HBM read ceiling (probe)
    sink = torch.empty(hci.probe_sink_words(), dtype=torch.float32, device="cuda")
    pe = _events(hip, 2)
    hci.probe_read(sets[0].k_cache, sink)
    probe_ms = []
    for _ in range(5):
        hip.hipEventRecord(pe[0], sp)
        hci.probe_read(sets[0].k_cache, sink)
        hip.hipEventRecord(pe[1], sp)
        hip.hipEventSynchronize(pe[1])
        probe_ms.append(_ms(hip, pe[0], pe[1]))
    probe_gbs = sets[0].k_cache.numel() * 2 / (min(probe_ms) * 1e-3) / 1e9

    # ---------------------------------------------------------------- warm-up
    launch_lens = []                     # committed lengths each timed launch streamed (host bookkeeping)
    counter = [0]

    def step(evs=None):
        si = counter[0] % n_sets
        counter[0] += 1
        st, bound = sets[si], bounds[si]
        if evs is None:
            dv.verify(lay, st, blk, bound)
        else:
            hci.verify_block_timed(lay.c, st.c, blk.c, blk.nb, blk.nc, blk.gamma, bound, blk.ws, evs)
        dv.accept(acc, mode, cfg.temperature, status=st.status)
        if evs is not None and evs[4]:
            hip.hipEventRecord(evs[4], sp)
        dv.slice_state(lay, st, blk, acc, bound)
        if evs is not None and evs[5]:
            hip.hipEventRecord(evs[5], sp)
        bounds[si] = bound + P
        return si

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    lens_before = [dv.to_host(st.kv_len).astype(np.int64) for st in sets]

    # ---------------------------------------------------------------- timed region
    # Only the two events around the streaming kernel are recorded here (its
    # average launch time is the roofline's denominator), on every
    # --event-every-th step: an event record costs a few microseconds of device
    # time, so the sampled steps carry it and the per-part breakdown comes from
    # a second, untimed pass below.
    every = max(1, args.event_every)
    stream_evs = []
    for i in range(K):
        if i % every:
            stream_evs.append(None)
            continue
        e = _events(hip, 6)
        e[0] = e[3] = e[4] = e[5] = None
        stream_evs.append(e)
    used = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        used.append(step(stream_evs[i]))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lens_after = [dv.to_host(st.kv_len).astype(np.int64) for st in sets]
    ms_step = (t1 - t0) * 1e3 / K
    sampled = [i for i, e in enumerate(stream_evs) if e is not None]
    stream_ms = [_ms(hip, stream_evs[i][1], stream_evs[i][2]) for i in sampled]
    # every step commits the same k + 1 rows to the set it used: the lengths each launch read
    n_on = [used.count(si) for si in range(n_sets)]
    adv = [(lens_after[si] - lens_before[si]) // max(n_on[si], 1) for si in range(n_sets)]
    seen = [0] * n_sets
    for si in used:
        launch_lens.append(lens_before[si] + adv[si] * seen[si])
        seen[si] += 1
    mean_lens = [float(np.mean([launch_lens[i][b] for i in sampled])) for b in range(cfg.nb)]

    # ---------------------------------------------------------------- breakdown pass (not timed)
    evsets = [_events(hip, 6) for _ in range(K)]
    for i in range(K):
        step(evsets[i])
    torch.cuda.synchronize()
    combine_ms = [_ms(hip, e[2], e[3]) for e in evsets]
    verify_ms = [_ms(hip, e[0], e[3]) for e in evsets]
    accept_ms = [_ms(hip, e[3], e[4]) for e in evsets]
    slice_ms = [_ms(hip, e[4], e[5]) for e in evsets]
    step_dev_ms = [_ms(hip, e[0], e[5]) for e in evsets]
    status = [int(v) for st in sets for v in dv.to_host(st.status)]
    assert not any(status), f"device status bits set: {[hci.device_status_string(v) for v in status]}"

    # ---------------------------------------------------------------- replay-equivalent (not timed)
    replay = replay_equivalent(cfg, lay, sets[0], bn, acc, bounds[0], hip, sp, args.replay_reps)

    alg_verify = verify_alg_bytes(cfg, mean_lens)
    alg_stream = stream_alg_bytes(cfg, mean_lens)
    avg_stream_s = float(np.mean(stream_ms)) * 1e-3
    achieved = alg_stream / avg_stream_s / 1e9
    positions = cfg.nb * cfg.nc * P
    value = positions / (ms_step * 1e-3)
    slice_med = float(np.median(slice_ms))

    out = {
        "metric": "verified block-positions/sec per layer",
        "value": round(value, 2),
        "unit": "block-positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations and KV, N(0,2) logits; no trained weights)",
        "config": {"workload": WORKLOAD_NAMES[args.config], "config_id": cfg.name, "nb": cfg.nb, "nc": cfg.nc,
                   "gamma": cfg.gamma, "kv_len": list(cfg.kv_lens), "d": cfg.d, "heads": cfg.heads,
                   "head_dim": cfg.head_dim, "parallelism": "single GPU"},
        "kv_sets_rotated": n_sets,
        "verify_ms": round(float(np.median(verify_ms)), 4),
        "verify_hbm_GBs": round(alg_verify / (float(np.median(verify_ms)) * 1e-3) / 1e9, 1),
        "verify_pct_of_8TBs": round(100.0 * alg_verify / (float(np.median(verify_ms)) * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "verify_positions_per_s": round(positions / (float(np.median(verify_ms)) * 1e-3), 1),
        "breakdown_ms_median": {"verify_stream": round(float(np.median([_ms(hip, e[1], e[2]) for e in evsets])), 4),
                                "verify_finish": round(float(np.median(combine_ms)), 4),
                                "accept": round(float(np.median(accept_ms)), 4),
                                "slice": round(slice_med, 4),
                                "step_device": round(float(np.median(step_dev_ms)), 4)},
        "slice_ms": round(slice_med, 4),
        "replay_equiv_ms": replay["replay_equiv_ms"],
        "replay_equiv_over_slice": round(replay["replay_equiv_ms"] / slice_med, 1),
        "replay": replay,
        "hbm_probe_read_GBs": round(probe_gbs, 1),
        "roofline": {"kernel": stream_kernel_name(cfg),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": _traffic(args.config, traffic_file(args.config)),
                     "alg_bytes_per_launch": int(alg_stream),
                     "avg_launch_ms": round(avg_stream_s * 1e3, 4),
                     "launches_timed": len(sampled), "timed_every_nth_step": every},
        "accepted_per_step": [int(x) for x in adv[0]],
    }
    if args.accept_rounds > 0:
        out["acceptance"] = acceptance_stats(cfg, args.accept_rounds, hip)
    if not args.no_cpu_baseline:
        case_np = {"params": params, "small": small, "blk": bn, "ri": ri, "kpre": kpre_host, "vpre": vpre_host}
        out["cpu_baseline"] = cpu_baseline(cfg, case_np, heads, max(1, args.cpu_reps))
    print(json.dumps(out), flush=True)


def bench_tree(args, cfg, hip):
    """Token-tree verification against the chain form of the same candidates.

    The nc candidate blocks of each sequence (gamma drafts each, over a small alphabet, drawn from
    prefix-keyed draft rows) share prefixes; merged into a trie they are n <= nc * (gamma + 1)
    nodes, each computed once (EvSpark digest, Interpretation: several candidates per round;
    ReaDy summary, section 5: tree verification with state recovery).  One tree step =
    hci_verify_tree -> hci_accept_tree (sampling) -> hci_slice_tree; the chain step verifies the
    same candidates as nc blocks (hci_verify_block -> hci_accept -> hci_slice_state) on a
    second state with the same prefixes.
    """
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci, synth
    W, K = args.warmup, args.steps
    cfg = synth.scaled(cfg, vocab=args.tree_vocab, mode="sample")
    tr = synth.tree_round(cfg)
    n = int(tr["n"])
    P = cfg.P
    n_ev = max(3, K // 4)                                  # steps of the per-part breakdown
    kv_cap = (cfg.max_kv_len + (W + K + n_ev + 2) * max(n, P) + 31) // 32 * 32

    params = synth.make_layer(cfg)
    small = synth.make_state_small(cfg)
    tables = synth.make_tables(cfg)
    lay = dv.DeviceLayer(cfg, params)

    def new_state():
        st = dv.DeviceState(lay, cfg.nb, kv_cap)
        st.load_small(small)
        for b in range(cfg.nb):
            st.write_prefix(b, synth.kv_prefix(cfg, b, "k", device="cuda"), synth.kv_prefix(cfg, b, "v", device="cuda"))
        st.kv_len.copy_(torch.tensor(cfg.kv_lens, dtype=torch.int32))
        return st

    st_t, st_c = new_state(), new_state()
    tok = tr["tokens"]
    tree = dv.DeviceTree(lay, cfg.nb, n, cfg.vocab)
    tree.set_inputs(tr["parent"], tables["E_x"][tok], tables["E_q"][tok], tables["E_k"][tok], tables["E_v"][tok])
    tree.set_accept_inputs(tok, tr["target_logits"], tr["draft_logits"], tr["uniforms"])
    # the chain form: the same candidate blocks (the tries were built from them)
    cand_zt, cand_zd, drafts, cand_u = synth.prefix_keyed_round(cfg)
    bn = synth.gather_block(cfg, tables, synth.block_tokens(synth.anchors(cfg), drafts))
    blk = dv.DeviceBlock(lay, cfg.nb, cfg.nc, cfg.gamma)
    blk.set_inputs(bn["x"], bn["q"], bn["k"], bn["v"])
    acc = dv.DeviceAccept(cfg.nb, cfg.nc, cfg.gamma, cfg.vocab)
    acc.set_inputs(cand_zt, drafts, cand_zd, cand_u)
    bound_t = [cfg.max_kv_len]
    bound_c = [cfg.max_kv_len]
    tree.ensure_workspace(kv_cap - n)
    blk.ensure_workspace(kv_cap - P)
    sp = torch.cuda.current_stream().cuda_stream

    def tree_step(evs=None):
        if evs is not None:
            hip.hipEventRecord(evs[0], sp)
        dv.verify_tree(lay, st_t, tree, bound_t[0])
        if evs is not None:
            hip.hipEventRecord(evs[1], sp)
        dv.accept_tree(tree, hci.SAMPLE, cfg.temperature, status=st_t.status)
        if evs is not None:
            hip.hipEventRecord(evs[2], sp)
        dv.slice_tree(lay, st_t, tree, bound_t[0])
        if evs is not None:
            hip.hipEventRecord(evs[3], sp)
        bound_t[0] += n

    def chain_step():
        dv.verify(lay, st_c, blk, bound_c[0])
        dv.accept(acc, hci.SAMPLE, cfg.temperature, status=st_c.status)
        dv.slice_state(lay, st_c, blk, acc, bound_c[0])
        bound_c[0] += P

    def timed(fn, steps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    for _ in range(W):
        tree_step()
        chain_step()
    half = max(1, K // 2)
    tree_ms = timed(tree_step, half)
    chain_ms = timed(chain_step, half)
    tree_ms = min(tree_ms, timed(tree_step, K - half) if K > half else tree_ms)
    chain_ms = min(chain_ms, timed(chain_step, K - half) if K > half else chain_ms)
    evs = [_events(hip, 4) for _ in range(n_ev)]
    for e in evs:
        tree_step(e)
    torch.cuda.synchronize()
    parts = {"verify_tree": float(np.median([_ms(hip, e[0], e[1]) for e in evs])),
             "accept_tree": float(np.median([_ms(hip, e[1], e[2]) for e in evs])),
             "slice_tree": float(np.median([_ms(hip, e[2], e[3]) for e in evs]))}
    status = [int(v) for st in (st_t, st_c) for v in dv.to_host(st.status)]
    assert not any(status), f"device status bits set: {[hci.device_status_string(v) for v in status]}"
    n_acc = [int(v) for v in dv.to_host(tree.n_acc)]
    positions = cfg.nb * cfg.nc * P
    out = {
        "metric": "verified tree nodes/sec per layer",
        "value": round(cfg.nb * n / (tree_ms * 1e-3), 1),
        "unit": "nodes/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(tree_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.act == "bf16" else "f32",
        "data": f"synthetic (seeded N(0,1) activations and KV; drafts over a {cfg.vocab}-letter alphabet "
                f"from prefix-keyed draft rows; no trained weights)",
        "config": {"workload": f"token-tree verify: {cfg.nb} sequences x {cfg.nc} candidate blocks (gamma="
                               f"{cfg.gamma}) merged into tries of {n} nodes, KV prefixes "
                               + "/".join(str(L) for L in cfg.kv_lens),
                   "config_id": cfg.name, "nb": cfg.nb, "nc": cfg.nc, "gamma": cfg.gamma, "nodes": n,
                   "trie_sizes": [int(v) for v in tr["trie_sizes"]], "vocab": cfg.vocab,
                   "kv_len": list(cfg.kv_lens), "d": cfg.d, "heads": cfg.heads, "head_dim": cfg.head_dim,
                   "parallelism": "single GPU"},
        "candidate_positions_per_s": round(positions / (tree_ms * 1e-3), 1),
        "chain_ms_per_step": round(chain_ms, 4),
        "chain_candidate_positions_per_s": round(positions / (chain_ms * 1e-3), 1),
        "tree_over_chain_speedup": round(chain_ms / tree_ms, 3),
        "query_rows": {"tree": cfg.nb * n, "chain": positions},
        "breakdown_ms_median": {k: round(v, 4) for k, v in parts.items()},
        "accepted_depths_last_step": n_acc,
    }
    print(json.dumps(out), flush=True)


def replay_equivalent(cfg, lay, st, bn, acc, bound, hip, sp, reps):
    """What slicing replaces: the accepted tokens run again through the target from the committed state.

    replay_equiv_ms: the k + 1 accepted positions (k of the last accept, the winning candidate's rows)
    as k + 1 sequential single-position steps -- verify with gamma = 0, then slice at 0 -- each reading
    the whole KV prefix; for several sequences max_b k_b + 1 batched steps.  replay_block_forward_ms:
    the same positions as one block forward (gamma = k) plus a slice at k.  Both run on a copy of the
    committed state (windows, IIR state and lengths are restored between repetitions; cache rows past
    kv_len are not state); medians of `reps` repetitions, HIP events on the stream.
    """
    import numpy as np
    import torch
    from hybrid_conv_iir_amd import device as dv
    from hybrid_conv_iir_amd import hci
    torch.cuda.synchronize()
    n_acc, best = dv.to_host(acc.n_acc), dv.to_host(acc.best)
    cstar = [int(best[b]) if cfg.nc > 1 else 0 for b in range(cfg.nb)]
    ks = [int(n_acc[b, cstar[b]]) for b in range(cfg.nb)]
    n = max(ks) + 1
    saved = {name: getattr(st, name).clone() for name in ("short_win", "outer_win", "iir", "kv_len")}

    def restore():
        for name, t in saved.items():
            getattr(st, name).copy_(t)

    def rows(i0, i1):
        pick = lambda a: np.stack([a[b, cstar[b], i0:i1] for b in range(cfg.nb)])[:, None]
        return pick(bn["x"]), pick(bn["q"]), pick(bn["k"]), pick(bn["v"])

    one = []
    for i in range(n):
        blk = dv.DeviceBlock(lay, cfg.nb, 1, 0)
        blk.set_inputs(*rows(i, i + 1))
        if i == 0:
            blk.ensure_workspace(bound + n)
        else:
            blk.ws = one[0].ws                                # one workspace serves the sequential steps
        one.append(blk)
    acc0 = dv.DeviceAccept(cfg.nb, 1, 0, cfg.vocab)           # n_accepted = 0: commit the one position
    whole = dv.DeviceBlock(lay, cfg.nb, 1, n - 1)
    whole.set_inputs(*rows(0, n))
    whole.ensure_workspace(bound)
    accn = dv.DeviceAccept(cfg.nb, 1, n - 1, cfg.vocab)
    accn.n_acc.fill_(n - 1)
    ev = _events(hip, 2)
    seq_ms, blk_ms = [], []
    for r in range(reps + 1):                                 # the first repetition warms up
        restore()
        hip.hipEventRecord(ev[0], sp)
        for i in range(n):
            dv.verify(lay, st, one[i], bound + i)
            dv.slice_state(lay, st, one[i], acc0, bound + i)
        hip.hipEventRecord(ev[1], sp)
        hip.hipEventSynchronize(ev[1])
        if r:
            seq_ms.append(_ms(hip, ev[0], ev[1]))
        restore()
        hip.hipEventRecord(ev[0], sp)
        dv.verify(lay, st, whole, bound)
        dv.slice_state(lay, st, whole, accn, bound)
        hip.hipEventRecord(ev[1], sp)
        hip.hipEventSynchronize(ev[1])
        if r:
            blk_ms.append(_ms(hip, ev[0], ev[1]))
    restore()
    torch.cuda.synchronize()
    return {"replay_equiv_ms": round(float(np.median(seq_ms)), 4), "steps": n, "accepted_k": ks,
            "replay_block_forward_ms": round(float(np.median(blk_ms)), 4), "reps": reps}


if __name__ == "__main__":
    main()
