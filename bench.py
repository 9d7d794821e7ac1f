"""Benchmark of the fused RoPE + block-FP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--only irq|qnr|kvi|idx|variants|decode|copy|stream]

A step is one launch of ``inv_rope_fp8_quant`` over the prefill workload
(16384 tokens x 32 heads in 4 groups of 8, head dim 512, bf16 in, e4m3 +
fp32 block-128 scales out; synthetic inputs already resident in HBM).  The
timed region is K back-to-back launches on one stream, bracketed by HIP
events recorded on that same stream and by device synchronizations.  Launch
i works on buffer set i mod S, each set its own copy of the input and its own
outputs, with S >= 2 and S sets totalling >= 1 GiB, so that no launch finds
the lines it writes still in the last-level cache.  The JSON
line reports achieved HBM throughput over the algorithmic bytes, tokens/s,
the roofline fraction against the 8 TB/s HBM3E peak, HBM traffic from
rocprofv3 counters when they were taken on the current kernel source, and
the CPU oracle timed on this host.  The other ops (qnorm_rope and
kv_rope_quant_insert on the forward workload, their one-launch fusion, the
indexer query path, the output variants - bf16 inverse RoPE, q to FP8, kv into
the bf16 token-strided cache and the fused full-cache forms - and decode
latencies) are timed the same way and reported under "extra", beside the
streaming ceiling of this part for the same access patterns (kernels in
bench_stream.hip: reads, writes and inv_rope_fp8_quant's byte pattern with no
arithmetic, and the cost of an empty launch).  Launches too short to time
through Python (the kv paths on the forward workload, decode) are also timed
as calls inside a HIP graph.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
STREAM_SRC = os.path.join(ROOT, "bench_stream.hip")
STREAM_LIB = os.path.join(ROOT, "bench_stream.so")
STREAM_DIRECT = 0x100  # bench_stream_irq: rows read with LDS-direct loads
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "irq_prefill_n16384_h32_counters.json")
KERNEL_SRC = os.path.join(ROOT, "rope_fp8_quant_amd", "csrc", "ropequant.hip")

# Algorithmic bytes (what the op must move; caches assumed cold):
#   inv_rope_fp8_quant per (token, head): 1024 B bf16 read + 512 B e4m3 write
#     + 16 B fp32 scales (4 B in ue8m0); per token: 8 B position + 256 B cos/sin row.
#   qnorm_rope per live head: 1024 B read + 1024 B write; per pad head 1024 B
#     write; per token 8 + 256 B; plus the 1024 B weight once.
#   kv_rope_quant_insert per token: 1024 B read + 528 B record + 8 B slot
#     + 8 + 256 B.
#   indexer_q_rope_quant per (token, head): 256 B read + 128 B codes + 8 B of
#     weights; per token 8 + 256 B.
#   inv_rope_bf16 per (token, head): 1024 B read + 1024 B write; per token 8 + 256 B.
#   qnorm_rope_fp8 per live head: 1024 B read; per head (live or pad): 512 B
#     codes + 16 B scales; per token 8 + 256 B; plus the 1024 B weight once.
#   kv_rope_insert_full per token: 1024 B read + 1024 B row + 8 B slot + 8 + 256 B.


def irq_bytes(N, H, fmt="fp32"):
    return N * H * (1024 + 512 + (16 if fmt == "fp32" else 4)) + N * (8 + 256)


def qnr_bytes(N, Hq, Hpad):
    return N * Hq * 2048 + N * (Hpad - Hq) * 1024 + N * 264 + 1024


def kvi_bytes(N):
    return N * (1024 + 528 + 8 + 264)


def idx_bytes(N, H):
    # per (token, head): 256 B bf16 read + 128 B codes + 4 B weight in + 4 B out;
    # per token: 8 B position + 256 B cos/sin row
    return N * H * (256 + 128 + 4 + 4) + N * (8 + 256)


def irb_bytes(N, H):
    return N * H * 2048 + N * 264


def qf8_bytes(N, Hq, Hpad):
    return N * Hq * 1024 + N * Hpad * (512 + 16) + N * 264 + 1024


def kvf_bytes(N):
    return N * (1024 + 1024 + 8 + 264)


def _rate(name, us, b):
    return dict(workload=name, us=us, bytes=b, gbs=b / us / 1e3, frac=b / us / 1e3 / HBM_PEAK_GBS)


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


_SETTLE = {}


def settle_clocks(ms=25.0):
    """Keep the GPU busy with unrelated device work (a 256 MiB fill, over and
    over) for about `ms` milliseconds before a measurement's warm-up.  Input
    preparation on the host leaves the GPU idle for seconds, and after idle
    the first ~100 launches (about 12 ms of work) run at lower clocks, more
    than a warm-up of a few steps covers.  None of this is in a timed region,
    and the warm-up and timed steps are still exactly the ones asked for."""
    import time

    import torch
    buf = _SETTLE.get("buf")
    if buf is None:
        buf = _SETTLE["buf"] = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(16):
            buf.fill_(i & 0xFF)
            i += 1
        torch.cuda.synchronize()


def time_launches(fn, steps, warmup, stream):
    import torch
    settle_clocks()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per launch


# MI355X's MALL (last-level cache) holds 256 MB, and written lines stay in
# it: relaunching on the same buffers lets plain stores overwrite lines the
# last launch left there, which made an inv_rope_fp8_quant with plain code
# stores 16% faster than with cold buffers (the nontemporal stores used now
# gain about 1%).  In a model the next call on a buffer comes a layer later,
# after other traffic has flushed the cache, so every config is timed cycling
# through at least two copies of its buffers, and through enough copies that
# they total ROTATE_BYTES.
ROTATE_BYTES = 1 << 30


def rotation_sets(set_bytes):
    return max(2, -(-ROTATE_BYTES // int(set_bytes)))


def time_rotating(fns, steps, warmup, stream):
    """time_launches over a list of equivalent launches on distinct buffers."""
    it = [0]

    def step():
        fns[it[0] % len(fns)]()
        it[0] += 1
    return time_launches(step, steps, warmup, stream)


def build_stream_lib(verbose=False):
    """Compile the streaming-ceiling kernels (bench_stream.hip) for gfx950."""
    from rope_fp8_quant_amd import build as lib_build
    return lib_build.compile_hip(STREAM_SRC, STREAM_LIB, verbose)


_stream_lib = None


def stream_lib():
    import ctypes
    global _stream_lib
    if _stream_lib is None:
        if not os.path.exists(STREAM_LIB):
            build_stream_lib()
        L = ctypes.CDLL(STREAM_LIB)
        P, U64, U32, I = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
        L.bench_stream_read.argtypes = [P, U64, U32, P, P]
        L.bench_stream_write.argtypes = [P, U64, I, P]
        L.bench_stream_irq.argtypes = [P, P, P, U64, I, P]
        L.bench_stream_rows_gm.argtypes = [P, P, U64, U32, U32, P]
        L.bench_stream_q.argtypes = [P, P, P, U64, U32, U32, I, P]
        L.bench_stream_empty.argtypes = [P]
        for f in (L.bench_stream_read, L.bench_stream_write, L.bench_stream_irq,
                  L.bench_stream_rows_gm, L.bench_stream_q, L.bench_stream_empty):
            f.restype = I
        _stream_lib = L
    return _stream_lib


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: launch refused")


def bench_stream(args, device, stream):
    """What HBM sustains on this part for the kernels' access patterns, with
    no arithmetic: 512 MiB of 1 KiB rows read (nontemporal), written
    (nontemporal, plain, sc1), and inv_rope_fp8_quant's traffic for the
    prefill workload's 524288 units and for the unit counts of the shorter
    launches; each over rotating buffers like the kernels.  Also the fixed
    cost of one empty launch, eager and in a graph."""
    import torch
    L = stream_lib()

    def h():  # torch's current stream (a graph's capture stream while capturing)
        return torch.cuda.current_stream().cuda_stream
    res = {}
    rows = 1 << 19  # 512 MiB of 1 KiB rows
    nbytes = rows * 1024
    sets = rotation_sets(nbytes) + 1
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=device).fill_(i + 1)
            for i in range(sets)]
    sink = torch.zeros(64, dtype=torch.int32, device=device)
    # the XOR of 64 bytes each equal to i+1 is 0 per lane, never 0xDEADBEEF
    fns = [lambda b=b: _ok(L.bench_stream_read(b.data_ptr(), rows, 0xDEADBEEF, sink.data_ptr(),
                                               h()), "read") for b in bufs]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["read_nt"] = dict(_rate("512 MiB read, 1 KiB rows, nontemporal", ms * 1e3, nbytes),
                          buffer_sets=sets)
    for pol, name in ((0, "write_nt"), (1, "write_plain"), (2, "write_sc1")):
        fns = [lambda b=b, pol=pol: _ok(L.bench_stream_write(b.data_ptr(), rows, pol, h()),
                                        "write") for b in bufs]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res[name] = dict(_rate(f"512 MiB written, 1 KiB rows, {name[6:]}", ms * 1e3, nbytes),
                         buffer_sets=sets)
    del bufs
    torch.cuda.empty_cache()
    # the pattern at the prefill workload's 524288 units, four units per
    # wave as the kernel (and two, finer waves), then at the unit counts of
    # the shorter launches: a launch's fixed cost weighs more on fewer bytes,
    # for a plain stream as for a kernel
    sizes = [("irq_pattern", 16384 * 32, "inv_rope_fp8_quant's bytes for 16384 x 32 units")]
    sizes += [(key, units, f"the same pattern for {units} units ({what})")
              for key, units, what in SAME_SIZE_STREAMS]
    for key, units, what in sizes:
        b = units * (1024 + 512 + 16)
        sets = rotation_sets(b)
        rot = [(torch.empty(units * 1024, dtype=torch.uint8, device=device).fill_(3),
                torch.empty(units * 512, dtype=torch.uint8, device=device),
                torch.empty(units * 16, dtype=torch.uint8, device=device)) for _ in range(sets)]
        for upw, suffix in ((4, ""), (2, "_2_per_wave"), (4 | STREAM_DIRECT, "_direct"),
                            (2 | STREAM_DIRECT, "_2_per_wave_direct")):
            fns = [lambda s_=s_, c=c, sc=sc, u=units, upw=upw: _ok(L.bench_stream_irq(
                s_.data_ptr(), c.data_ptr(), sc.data_ptr(), u, upw, h()), "irq")
                for s_, c, sc in rot]
            ms = time_rotating(fns, args.steps, args.warmup, stream)
            how = " read straight into LDS" if upw & STREAM_DIRECT else ""
            res[key + suffix] = dict(_rate(f"{what}, {upw & 0xFF} units per wave{how}, no math",
                                           ms * 1e3, b), buffer_sets=sets)
            del fns
        del rot
        torch.cuda.empty_cache()

    # inv_rope_bf16's pattern at its workload (16384 x 32 units, 1 KiB read
    # and 1 KiB written group-major per unit, 4 groups of 8 heads)
    units, heads, hpg = 16384 * 32, 32, 8
    b = units * 2048
    sets = rotation_sets(b)
    rot = [(torch.empty(units * 1024, dtype=torch.uint8, device=device).fill_(3),
            torch.empty(units * 1024, dtype=torch.uint8, device=device)) for _ in range(sets)]
    fns = [lambda s_=s_, d=d: _ok(L.bench_stream_rows_gm(s_.data_ptr(), d.data_ptr(), units, heads,
                                                         hpg, h()), "rows_gm")
           for s_, d in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["irb_pattern"] = dict(_rate("inv_rope_bf16's bytes for 16384 x 32 units (1 KiB read, "
                                    "1 KiB written group-major), 4 units per wave, no math",
                                    ms * 1e3, b), buffer_sets=sets)
    del fns, rot
    torch.cuda.empty_cache()

    # the q paths' pattern at their workload (8192 tokens, 64 live heads padded
    # to 128): qnorm_rope's bf16 rows, and qnorm_rope_fp8's codes and scales
    tokens, hq, hpad = 8192, 64, 128
    units = tokens * hpad
    for key, out_bytes, what in (("qnr_pattern", 1024, "qnorm_rope"),
                                 ("qf8_pattern", 512, "qnorm_rope_fp8")):
        b = tokens * hq * 1024 + units * (out_bytes + (16 if out_bytes == 512 else 0))
        sets = rotation_sets(b)
        rot = [(torch.empty(tokens * hq * 1024, dtype=torch.uint8, device=device).fill_(3),
                torch.empty(units * out_bytes, dtype=torch.uint8, device=device),
                torch.empty(units * 16, dtype=torch.uint8, device=device)) for _ in range(sets)]
        fns = [lambda s_=s_, d=d, sc=sc, ob=out_bytes: _ok(L.bench_stream_q(
            s_.data_ptr(), d.data_ptr(), sc.data_ptr(), units, hq, hpad, ob, h()), "q")
            for s_, d, sc in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res[key] = dict(_rate(f"{what}'s bytes for 8192 x 64 -> 128 heads, 4 units per wave, "
                              "no math", ms * 1e3, b), buffer_sets=sets)
        del fns, rot
        torch.cuda.empty_cache()

    # at the kv insert's size (8192 units, 12.7 MB), timed as that kernel is:
    # per call inside a HIP graph, over enough buffer sets to total 1 GiB
    units = 8192
    b = units * (1024 + 512 + 16)
    sets = rotation_sets(b)
    rot = [(torch.empty(units * 1024, dtype=torch.uint8, device=device).fill_(3),
            torch.empty(units * 512, dtype=torch.uint8, device=device),
            torch.empty(units * 16, dtype=torch.uint8, device=device)) for _ in range(sets)]
    for upw, suffix in ((4, ""), (2, "_2_per_wave")):
        fns = [lambda s_=s_, c=c, sc=sc, upw=upw: _ok(L.bench_stream_irq(
            s_.data_ptr(), c.data_ptr(), sc.data_ptr(), units, upw, h()), "irq")
            for s_, c, sc in rot]
        us = graph_rotating_per_call_us(fns)
        res["irq_pattern_8192_units" + suffix] = dict(
            _rate(f"the same pattern for 8192 units (kv_rope_quant_insert's size), {upw} units "
                  "per wave, no math, per call in a HIP graph", us, b), buffer_sets=sets)
        del fns
    del rot
    torch.cuda.empty_cache()

    def empty():
        _ok(L.bench_stream_empty(h()), "empty")
    res["empty_launch"] = dict(us_eager=round(time_launches(empty, 500, 100, stream) * 1e3, 3),
                               us_graph=round(graph_per_call_us(empty), 3))
    return res


def graph_rotating_per_call_us(fns, calls=None, replays=5):
    """Per-call time of launches captured in one HIP graph, call i on buffer
    set i mod len(fns) (median of `replays` replays): the GPU-side cost of a
    launch, without Python dispatch, on buffers the previous calls did not
    touch."""
    calls = calls or max(100, 2 * len(fns))
    it = [0]

    def step():
        fns[it[0] % len(fns)]()
        it[0] += 1
    return graph_per_call_us(step, calls, replays)


def to_dev(a, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def bench_irq(args, device, stream, fmt="fp32", same_buffers=False):
    """The prefill workload over rotating buffer sets (the headline), or, with
    same_buffers, relaunched on one set (reported beside it, cache-assisted)."""
    import rope_fp8_quant_amd as rq
    from rope_fp8_quant_amd import synth
    cfg = synth.IRQ_PREFILL
    t0 = time.time()
    o, pos, cache = synth.irq_inputs(cfg)
    progress(f"irq inputs drawn in {time.time() - t0:.1f}s")
    N, H, hpg = cfg["N"], cfg["H"], cfg["hpg"]
    od, pd, cd = to_dev(o, device), to_dev(pos, device), to_dev(cache, device)
    sets = 1 if same_buffers else rotation_sets(irq_bytes(N, H, fmt))
    rot = [(od if i == 0 else od.clone(),) + rq.empty_inv_rope_fp8_quant_outputs(N, H, hpg, device, fmt)
           for i in range(sets)]
    fns = [lambda x=x, out=out, sc=sc: rq.inv_rope_fp8_quant(x, pd, cd, hpg, out, sc, fmt)
           for x, out, sc in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    del rot, fns, od
    return cfg, ms, (o, pos, cache), sets


# Streaming-pattern sizes matched to shorter launches: (ceiling key, 512-dim
# units of 1 KiB read and 528 B written, the kernel it stands beside).  The
# indexer moves 1 KiB in and 544 B out per 4-head item, 65536 items at 4096
# tokens x 64 heads; the irregular IRQ 4096 x 48 units.
SAME_SIZE_STREAMS = (
    ("irq_pattern_196608_units", 4096 * 48, "inv_rope_fp8_quant_irregular"),
    ("irq_pattern_65536_units", 4096 * 16, "indexer_q_rope_quant"),
)


def vs_same_size_stream(extra, ceiling):
    """Beside each shorter launch, the streaming pattern's rate at its size
    (four units per wave, as the kernels, and two); beside inv_rope_bf16, the
    stream of its own byte pattern, and so beside the q paths."""
    if not ceiling:
        return
    for what, key in (("inv_rope_bf16", "irb_pattern"), ("qnorm_rope", "qnr_pattern"),
                      ("qnorm_rope_fp8", "qf8_pattern")):
        if what in extra and key in ceiling:
            # time ratio: the pattern moves the op's bytes less its per-token
            # positions and cos/sin rows
            extra[what]["pattern_stream_us"] = round(ceiling[key]["us"], 2)
            extra[what]["frac_of_pattern_stream"] = round(
                ceiling[key]["us"] / extra[what]["us"], 4)
    for key, _, what in SAME_SIZE_STREAMS:
        if what in extra and key in ceiling:
            extra[what]["same_size_stream_gbs"] = round(ceiling[key]["gbs"], 1)
            extra[what]["frac_of_same_size_stream"] = round(
                extra[what]["gbs"] / ceiling[key]["gbs"], 4)
            k2 = key + "_2_per_wave"
            extra[what]["same_size_stream_2_per_wave_gbs"] = round(ceiling[k2]["gbs"], 1)
            extra[what]["frac_of_same_size_stream_2_per_wave"] = round(
                extra[what]["gbs"] / ceiling[k2]["gbs"], 4)


# Filled by bench_stream when it runs: the empty-launch cost in a graph, the
# streaming rate of inv_rope_fp8_quant's byte pattern, and that pattern's
# per-call time at the kv insert's size, for the comparisons beside short
# launches.
CEILING = {}


def small_launch_record(name, b, us_graph, us_python, sets):
    """A launch too short to time through Python: `us` is its per-call time in
    a HIP graph over rotating buffers; beside it the Python-loop time and,
    when the streaming ceiling was measured, the estimate of an empty launch
    plus its bytes at the ceiling rate, and the per-call time of the plain
    streaming pattern at the kv insert's size, timed the same way."""
    rec = dict(_rate(name, us_graph, b), us_python=round(us_python, 3), buffer_sets=sets,
               timing="per call inside a HIP graph, call i on buffer set i mod buffer_sets")
    if CEILING:
        est = CEILING["floor_us"] + b / CEILING["gbs"] / 1e3
        rec.update(launch_floor_us=CEILING["floor_us"], ceiling_gbs=CEILING["gbs"],
                   estimate_us=round(est, 3), residual_us=round(us_graph - est, 3),
                   small_stream_us=CEILING["small_us"],
                   small_stream_2_per_wave_us=CEILING["small_us_2"])
    return rec


def bench_qnr_kvi(args, device, stream):
    import torch

    import rope_fp8_quant_amd as rq
    from rope_fp8_quant_amd import synth
    res = {}
    if args.only in (None, "qnr"):
        cfg = synth.QNR_FORWARD
        q, w, pos, cache = synth.qnr_inputs(cfg)
        qd, wd, pd, cd = (to_dev(x, device) for x in (q, w, pos, cache))
        del q
        b = qnr_bytes(cfg["N"], cfg["Hq"], cfg["Hpad"])
        sets = rotation_sets(b)
        rot = [(qd if i == 0 else qd.clone(),
                torch.empty((cfg["N"], cfg["Hpad"], 512), dtype=torch.bfloat16, device=device))
               for i in range(sets)]
        fns = [lambda x=x, o=o: rq.qnorm_rope(x, wd, pd, cd, o, cfg["eps"]) for x, o in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res["qnorm_rope"] = dict(workload=cfg["name"], us=ms * 1e3, bytes=b,
                                 gbs=b / ms / 1e6, frac=b / ms / 1e6 / HBM_PEAK_GBS,
                                 buffer_sets=sets)
        del qd, rot, fns
    if args.only in (None, "kvi"):
        cfg = synth.KVI_FORWARD
        if args.kvi_tokens is not None or args.kvi_slots == "seq":
            # a traffic probe of the same op: another token count (the cache
            # grows to twice the tokens when 16384 slots are too few) or
            # slots in token order
            n = cfg["N"] if args.kvi_tokens is None else args.kvi_tokens
            cfg = dict(cfg, N=n, num_blocks=max(cfg["num_blocks"], -(-2 * n // cfg["block_size"])),
                       max_pos=max(cfg["max_pos"], n))
            cfg["name"] = f"kvi_n{n}_{cfg['num_blocks']}x{cfg['block_size']}_{args.kvi_slots}"
        kv, pos, slots, cache = synth.kvi_inputs(cfg)
        if args.kvi_slots == "seq":
            slots = np.arange(cfg["N"], dtype=np.int64)
        kd, pd, sd, cd = (to_dev(x, device) for x in (kv, pos, slots, cache))
        k_cache = rq.empty_kv_cache(cfg["num_blocks"], cfg["block_size"], device, fill=0xAA)
        b = kvi_bytes(cfg["N"])
        sets = rotation_sets(kd.nbytes + k_cache.nbytes)
        rot = [(kd.clone(), sd.clone(), k_cache.clone()) for _ in range(sets)]
        fns = [lambda k=k, s=s, c=c: rq.kv_rope_quant_insert(k, pd, cd, s, c, cfg["block_size"])
               for k, s, c in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res["kv_rope_quant_insert"] = small_launch_record(
            cfg["name"], b, graph_rotating_per_call_us(fns), ms * 1e3, sets)
        del rot, fns
        if cfg is not synth.KVI_FORWARD:
            return res
        # the same q and kv work in one launch (positions 0..8191 serve both)
        qc = synth.QNR_FORWARD
        q, w, qpos, qcache = synth.qnr_inputs(qc)
        qd, wd = to_dev(q, device), to_dev(w, device)
        del q
        b = qnr_bytes(qc["N"], qc["Hq"], qc["Hpad"]) + kvi_bytes(cfg["N"]) - cfg["N"] * 264
        sets = rotation_sets(b)
        rot = [(qd if i == 0 else qd.clone(), kd.clone(),
                torch.empty((qc["N"], qc["Hpad"], 512), dtype=torch.bfloat16, device=device),
                k_cache.clone()) for i in range(sets)]
        fns = [lambda x=x, k=k, o=o, c=c: rq.qnorm_rope_kv_rope_quant_insert(
            x, wd, k, pd, cd, sd, o, c, cfg["block_size"], qc["eps"]) for x, k, o, c in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        # The same work as two launches back to back, and the one launch with
        # the slots in token order (records written contiguously instead of
        # scattered over the cache): what the fusion saves, and what the
        # scattered record writes cost inside the q stream.
        fns2 = [lambda x=x, k=k, o=o, c=c: (
            rq.qnorm_rope(x, wd, pd, cd, o, qc["eps"]),
            rq.kv_rope_quant_insert(k, pd, cd, sd, c, cfg["block_size"])) for x, k, o, c in rot]
        ms_sep = time_rotating(fns2, args.steps, args.warmup, stream)
        sd_seq = to_dev(np.arange(cfg["N"], dtype=np.int64), device)
        fns3 = [lambda x=x, k=k, o=o, c=c: rq.qnorm_rope_kv_rope_quant_insert(
            x, wd, k, pd, cd, sd_seq, o, c, cfg["block_size"], qc["eps"]) for x, k, o, c in rot]
        ms_seq = time_rotating(fns3, args.steps, args.warmup, stream)
        res["qnorm_rope_kv_rope_quant_insert"] = dict(
            workload="qnr_forward + kvi_forward, one launch", us=ms * 1e3, bytes=b,
            gbs=b / ms / 1e6, frac=b / ms / 1e6 / HBM_PEAK_GBS, buffer_sets=sets,
            us_two_launches=ms_sep * 1e3, us_slots_in_token_order=ms_seq * 1e3)
        del qd, rot, fns, fns2, fns3
    if args.only in (None, "idx"):
        N, H = 4096, 64
        q = synth.normal_bf16((N, H, 128), 55, synth.T_Q)
        w = np.random.default_rng([55, 9]).uniform(0, 1, (N, H)).astype(np.float32)
        qd, wd = to_dev(q, device), to_dev(w, device)
        pd = to_dev(np.arange(N, dtype=np.int64), device)
        cd = to_dev(synth.cos_sin_cache(N), device)
        b = idx_bytes(N, H)
        sets = rotation_sets(b)
        rot = [(qd.clone(), wd.clone(), torch.empty((N, H, 128), dtype=torch.uint8, device=device),
                torch.empty((N, H), dtype=torch.float32, device=device)) for _ in range(sets)]
        fns = [lambda q=q, w=w, o=o, x=x: rq.indexer_q_rope_quant(q, pd, cd, w, o, x, 128 ** -0.5)
               for q, w, o, x in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res["indexer_q_rope_quant"] = dict(workload="idx_n4096_h64_d128", us=ms * 1e3, bytes=b,
                                           gbs=b / ms / 1e6, frac=b / ms / 1e6 / HBM_PEAK_GBS,
                                           buffer_sets=sets)
        del rot, fns
        # irregular grouping: 4096 tokens x 48 heads in groups of 6
        cfg = synth.IRQ_IRREGULAR
        o, pos, cache = synth.irq_inputs(cfg)
        N, H, hpg = cfg["N"], cfg["H"], cfg["hpg"]
        od, pd, cd = to_dev(o, device), to_dev(pos, device), to_dev(cache, device)
        del o
        b = irq_bytes(N, H)
        sets = rotation_sets(b)
        rot = [(od.clone(),) + rq.empty_inv_rope_fp8_quant_outputs(N, H, hpg, device)
               for _ in range(sets)]
        fns = [lambda x=x, out=out, sc=sc: rq.inv_rope_fp8_quant(x, pd, cd, hpg, out, sc)
               for x, out, sc in rot]
        ms = time_rotating(fns, args.steps, args.warmup, stream)
        res["inv_rope_fp8_quant_irregular"] = dict(
            workload=cfg["name"], us=ms * 1e3, bytes=b, gbs=b / ms / 1e6,
            frac=b / ms / 1e6 / HBM_PEAK_GBS, buffer_sets=sets)
        del rot, fns, od
    return res


def bench_variants(args, device, stream):
    """The output variants on the same workloads as their quantized forms."""
    import torch

    import rope_fp8_quant_amd as rq
    from rope_fp8_quant_amd import synth
    res = {}
    cfg = synth.IRQ_PREFILL
    o, pos, cache = synth.irq_inputs(cfg)
    N, H, hpg = cfg["N"], cfg["H"], cfg["hpg"]
    od, pd, cd = to_dev(o, device), to_dev(pos, device), to_dev(cache, device)
    del o
    sets = rotation_sets(irb_bytes(N, H))
    rot = [(od if i == 0 else od.clone(),
            torch.empty((H // hpg, N, hpg * 512), dtype=torch.bfloat16, device=device))
           for i in range(sets)]
    fns = [lambda x=x, o=o: rq.inv_rope_bf16(x, pd, cd, hpg, o) for x, o in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["inv_rope_bf16"] = dict(_rate(cfg["name"], ms * 1e3, irb_bytes(N, H)), buffer_sets=sets)
    del od, rot, fns
    torch.cuda.empty_cache()

    qc, kc = synth.QNR_FORWARD, synth.KVI_FORWARD
    q, w, pos, cache = synth.qnr_inputs(qc)
    kv, _, slots, _ = synth.kvi_inputs(kc)
    N, Hq, Hpad = qc["N"], qc["Hq"], qc["Hpad"]
    qd, wd, pd, cd, kd, sd = (to_dev(x, device) for x in (q, w, pos, cache, kv, slots))
    del q
    b = qf8_bytes(N, Hq, Hpad)
    sets = rotation_sets(b)
    rot = [(qd if i == 0 else qd.clone(),) + rq.empty_qnorm_rope_fp8_outputs(N, Hpad, device)
           for i in range(sets)]
    fns = [lambda x=x, c=c, s=s: rq.qnorm_rope_fp8(x, wd, pd, cd, c, s, qc["eps"])
           for x, c, s in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["qnorm_rope_fp8"] = dict(_rate(qc["name"], ms * 1e3, b), buffer_sets=sets)
    del rot, fns
    ns = kc["num_blocks"] * kc["block_size"]
    full = torch.empty((ns, 512), dtype=torch.bfloat16, device=device)
    sets = rotation_sets(kd.nbytes + full.nbytes)
    rot = [(kd.clone(), torch.empty_like(full)) for _ in range(sets)]
    fns = [lambda k=k, f=f: rq.kv_rope_insert_full(k, pd, cd, sd, f) for k, f in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["kv_rope_insert_full"] = small_launch_record(
        f"kvf_forward_n{N}_{ns}slots", kvf_bytes(N), graph_rotating_per_call_us(fns), ms * 1e3,
        sets)
    del rot, fns
    b = qf8_bytes(N, Hq, Hpad) + kvf_bytes(N) - N * 264
    sets = rotation_sets(b)
    rot = [(qd if i == 0 else qd.clone(), kd.clone(), torch.empty_like(full))
           + rq.empty_qnorm_rope_fp8_outputs(N, Hpad, device) for i in range(sets)]
    fns = [lambda x=x, k=k, f=f, c=c, s=s: rq.qnorm_rope_fp8_kv_rope_insert_full(
        x, wd, k, pd, cd, sd, c, s, f, qc["eps"]) for x, k, f, c, s in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["qnorm_rope_fp8_kv_rope_insert_full"] = dict(_rate(
        "qnr_forward (fp8) + kvf_forward, one launch", ms * 1e3, b), buffer_sets=sets)
    del rot, fns
    # bf16 full-cache form in place: q_head_padded == Hq, q_out is q_in (each
    # launch rotates q again, which leaves it a rotated copy of itself: the
    # traffic is the same)
    b = N * Hq * 2048 + N * 264 + 1024 + kvf_bytes(N) - N * 264
    sets = rotation_sets(b)
    rot = [(qd if i == 0 else qd.clone(), kd.clone(), torch.empty_like(full))
           for i in range(sets)]
    fns = [lambda x=x, k=k, f=f: rq.qnorm_rope_kv_rope_insert_full(
        x, wd, k, pd, cd, sd, x, f, qc["eps"]) for x, k, f in rot]
    ms = time_rotating(fns, args.steps, args.warmup, stream)
    res["qnorm_rope_kv_rope_insert_full"] = dict(_rate(
        f"q in place n{N}_h{Hq} + kvf_forward, one launch", ms * 1e3, b), buffer_sets=sets)
    return res


def graph_per_call_us(fn, calls=100, replays=5):
    """Per-call time of `calls` launches captured in one HIP graph (median of
    `replays` replays): the GPU-side cost without Python dispatch."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    settle_clocks()
    times = []
    for _ in range(replays + 1):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3 / calls)
    times = sorted(times[1:])
    return times[len(times) // 2]


def cold_single_us(fn, scratch, reps=21):
    """One launch on its own, timed with events right around it, after a 1 GiB
    write has flushed the caches (median over reps)."""
    import torch
    times = []
    for _ in range(reps):
        scratch.fill_(1)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    times.sort()
    return times[len(times) // 2]


def bench_decode(args, device, stream):
    """Decode sizes: per call through Python (host-bound), through a prepared
    call (checks and marshalling done once), in a HIP graph (GPU-side cost
    with warm caches), and one cold launch on its own."""
    import torch

    import rope_fp8_quant_amd as rq
    from rope_fp8_quant_amd import synth
    res = {}
    cache = to_dev(synth.cos_sin_cache(65536), device)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=device)
    for N in synth.DECODE_NS:
        cfg = dict(synth.IRQ_TINY, N=N, H=32, hpg=8, max_pos=65536, seed=40 + N)
        o, pos, _ = synth.irq_inputs(cfg)
        od, pd = to_dev(o, device), to_dev(pos, device)
        out, sc = rq.empty_inv_rope_fp8_quant_outputs(N, 32, 8, device)
        q = to_dev(synth.normal_bf16((N, 32, 512), 50 + N, synth.T_Q), device)
        q_out = torch.empty((N, 128, 512), dtype=torch.bfloat16, device=device)

        def irq():
            rq.inv_rope_fp8_quant(od, pd, cache, 8, out, sc)

        def qnr():
            rq.qnorm_rope(q, None, pd, cache, q_out, 1e-6)

        # the decode step's q + kv op [P1]: the same q, and the token's kv
        # into a 4 x 64-slot paged cache at seeded slots
        kvd = to_dev(synth.normal_bf16((N, 512), 60 + N, synth.T_KV), device)
        sd = to_dev(synth.slot_permutation(N, 256, 60 + N), device)
        kc = rq.empty_kv_cache(4, 64, device, fill=0xAA)

        def fused():
            rq.qnorm_rope_kv_rope_quant_insert(q, None, kvd, pd, cache, sd, q_out, kc, 64, 1e-6)

        ms = time_launches(irq, 200, 20, stream)
        msq = time_launches(qnr, 200, 20, stream)
        irq_p = rq.prepare(rq.inv_rope_fp8_quant, od, pd, cache, 8, out, sc)
        qnr_p = rq.prepare(rq.qnorm_rope, q, None, pd, cache, q_out, 1e-6)
        msp = time_launches(irq_p, 200, 20, stream)
        msqp = time_launches(qnr_p, 200, 20, stream)
        gi, gq = graph_per_call_us(irq), graph_per_call_us(qnr)
        gf = graph_per_call_us(fused)
        ci, cq = cold_single_us(irq, scratch), cold_single_us(qnr, scratch)
        res[f"N{N}"] = dict(irq_us_python=round(ms * 1e3, 2),
                            irq_us_prepared=round(msp * 1e3, 2), irq_us_graph=round(gi, 2),
                            irq_gbs_graph=round(irq_bytes(N, 32) / gi / 1e3, 1),
                            irq_us_single_cold=round(ci, 2),
                            qnr_us_python=round(msq * 1e3, 2),
                            qnr_us_prepared=round(msqp * 1e3, 2), qnr_us_graph=round(gq, 2),
                            qnr_gbs_graph=round(qnr_bytes(N, 32, 128) / gq / 1e3, 1),
                            qnr_us_single_cold=round(cq, 2),
                            qnr_kvi_fused_us_graph=round(gf, 2))
    del scratch
    return res


def bench_copy(args, device, stream):
    """Plain 1 GiB device copy, the calibration kernel for HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
    dst = torch.empty_like(src)
    ms = time_launches(lambda: dst.copy_(src), args.steps, args.warmup, stream)
    return dict(bytes_read=n, bytes_written=n, us=ms * 1e3, gbs=2 * n / ms / 1e6)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(irq_inputs, budget_s=4.0, runs=3):
    """The CPU oracle (single-threaded C) on this host, pinned to one core:
    the median of `runs` runs over a token prefix of the prefill workload
    sized to about budget_s seconds each (the whole workload if it fits)."""
    import oracle
    o, pos, cache = irq_inputs
    N, H = o.shape[0], o.shape[1]
    try:
        old_aff = os.sched_getaffinity(0)
        core = min(old_aff)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        old_aff, core = None, None
    try:
        n = 256
        t = time.perf_counter()
        oracle.inv_rope_fp8_quant(o[:n], pos[:n], cache, 8)
        dt = time.perf_counter() - t
        n2 = int(min(N, max(n, n * budget_s / max(dt, 1e-6))))
        oc, pc = np.ascontiguousarray(o[:n2]), pos[:n2].copy()
        times = []
        for _ in range(runs):
            t = time.perf_counter()
            oracle.inv_rope_fp8_quant(oc, pc, cache, 8)
            times.append(time.perf_counter() - t)
    finally:
        if old_aff is not None:
            os.sched_setaffinity(0, old_aff)
    dt = sorted(times)[len(times) // 2]
    gbs = irq_bytes(n2, H) / dt / 1e9
    return dict(value=round(gbs, 4), unit="GB/s", cores=1, kind="oracle",
                tokens_per_s=round(n2 / dt, 1), cpu=cpu_model(),
                sample=f"first {n2} of {N} tokens x {H} heads of the same workload, one "
                       f"thread pinned to core {core}, median of {runs} runs of {dt:.1f} s")


def _oracle_shard_proc(spec, results):
    """Process body of the sharded CPU baseline: runs one shard and reports its
    compute time (or the error) through `results`, then exits normally."""
    try:
        results.put(_oracle_shard(spec))
    except Exception as e:  # reported to the parent, which raises
        results.put(f"{type(e).__name__}: {e}")


def _oracle_shard(spec):
    """Worker of the sharded CPU baseline (a fresh process): the same oracle
    call on one token range of the shared inputs; returns its compute time."""
    from multiprocessing import shared_memory

    import oracle
    (o_name, o_shape, c_name, c_shape, pos, lo, hi) = spec
    so = shared_memory.SharedMemory(name=o_name)
    sc = shared_memory.SharedMemory(name=c_name)
    try:
        o = np.ndarray(o_shape, dtype=np.uint16, buffer=so.buf)
        cache = np.ndarray(c_shape, dtype=np.float32, buffer=sc.buf)
        mine = np.ascontiguousarray(o[lo:hi])
        oracle.lib()
        t = time.perf_counter()
        oracle.inv_rope_fp8_quant(mine, pos, cache, 8)
        return time.perf_counter() - t
    finally:
        del o, cache
        so.close()
        sc.close()


def cpu_baseline_sharded(irq_inputs):
    """The same oracle on every host core of this GPU's share, tokens split
    evenly; the slowest shard's compute time is the run's time."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    o, pos, cache = irq_inputs
    N, H = o.shape[0], o.shape[1]
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    workers = max(1, min(16, ncpu))
    so = shared_memory.SharedMemory(create=True, size=o.nbytes)
    sc = shared_memory.SharedMemory(create=True, size=cache.nbytes)
    try:
        np.ndarray(o.shape, dtype=np.uint16, buffer=so.buf)[:] = o
        np.ndarray(cache.shape, dtype=np.float32, buffer=sc.buf)[:] = cache
        cuts = [N * i // workers for i in range(workers + 1)]
        specs = [(so.name, o.shape, sc.name, cache.shape, pos[a:b].copy(), a, b)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        # one process per shard, each exiting on its own once done (no
        # terminate(): a profiler attached to the children may not survive it)
        ctx = mp.get_context("spawn")
        results = ctx.SimpleQueue()
        procs = [ctx.Process(target=_oracle_shard_proc, args=(sp, results)) for sp in specs]
        for pr in procs:
            pr.start()
        times = []
        while len(times) < len(procs):
            if not results.empty():
                times.append(results.get())
            elif not any(pr.is_alive() for pr in procs) and results.empty():
                # a worker died before reporting (e.g. it could not start)
                times.append("a worker exited without a result")
            else:
                time.sleep(0.02)
        for pr in procs:
            pr.join()
        bad = [t for t in times if not isinstance(t, float)]
        if bad:
            raise RuntimeError(f"sharded oracle failed: {bad[0]}")
    finally:
        so.close()
        so.unlink()
        sc.close()
        sc.unlink()
    dt = max(times)
    return dict(value=round(irq_bytes(N, H) / dt / 1e9, 4), unit="GB/s", cores=workers,
                kind="oracle", tokens_per_s=round(N / dt, 1), cpu=cpu_model(),
                sample=f"all {N} tokens x {H} heads split over {workers} processes, "
                       f"slowest shard {dt:.2f} s")


def traffic_from_profile():
    try:
        with open(PROFILE_COUNTERS) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


# ---------------------------------------------------- rocprofv3 summaries

def _csv_rows(path):
    import csv
    import glob
    files = [path] if os.path.isfile(path) else sorted(
        glob.glob(os.path.join(path, "**", "*.csv"), recursive=True))
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _short(name):
    """Kernel name without the parameter list and anonymous namespaces."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    depth, out = 0, []
    for ch in name:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)


def counter_medians(path):
    """{(kernel, grid, counter): (median value, dispatches)} from a rocprofv3
    --pmc output directory (or its counter_collection CSV)."""
    import statistics
    vals = {}
    for r in _csv_rows(path):
        if "Counter_Name" not in r:
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]), r["Counter_Name"])
        vals.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: (statistics.median(v), len(v)) for k, v in vals.items()}


def trace_stats(path):
    """{(kernel, grid, workgroup): [durations in us]} from a rocprofv3
    --kernel-trace output directory (its kernel_trace CSV)."""
    out = {}
    for r in _csv_rows(path):
        if "Start_Timestamp" not in r or "Counter_Name" in r or "Kernel_Name" not in r:
            continue
        grid = int(r.get("Grid_Size") or r["Grid_Size_X"])
        wg = int(r.get("Workgroup_Size") or r["Workgroup_Size_X"])
        key = (_short(r["Kernel_Name"]), grid, wg)
        out.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return out


def summarize(paths):
    """Print per-kernel medians of every counter / trace directory given."""
    import statistics
    for path in paths:
        print(f"## {path}")
        med = counter_medians(path)
        for (k, g, c), (v, n) in sorted(med.items()):
            print(f"| {k} | {g:,} | {c} | {v:,.3f} | {n} |")
        for (k, g, w), d in sorted(trace_stats(path).items(), key=lambda x: -sum(x[1])):
            print(f"| {k} | {g:,} | {w} | {len(d)} | {sum(d) / len(d):.2f} | "
                  f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")


def write_counters_json(irq_fetch, irq_write, copy_fetch, copy_write, sq=None):
    """profiles/irq_prefill_n16384_h32_counters.json from four rocprofv3 --pmc
    runs: FETCH_SIZE and WRITE_SIZE of `bench.py --only irq` and of
    `bench.py --only copy` (the calibration), plus optionally SQ counters."""
    from rope_fp8_quant_amd import synth
    cfg = synth.IRQ_PREFILL
    N, H = cfg["N"], cfg["H"]
    grid = N * H * 32  # 64 threads per two units

    def pick(path, kernel, counter, grid_size=None):
        for (k, g, c), (v, _) in counter_medians(path).items():
            if k.startswith(kernel) and c == counter and (grid_size is None or g == grid_size):
                return v
        raise RuntimeError(f"{path}: no {counter} for {kernel}")
    copy_bytes = 1 << 30
    cf = pick(copy_fetch, "__amd_rocclr_copyBuffer", "FETCH_SIZE") * 1024 / copy_bytes
    cw = pick(copy_write, "__amd_rocclr_copyBuffer", "WRITE_SIZE") * 1024 / copy_bytes
    f = pick(irq_fetch, "irq_kernel<0>", "FETCH_SIZE", grid)
    w = pick(irq_write, "irq_kernel<0>", "WRITE_SIZE", grid)
    rd, wr = round(f * 1024 / cf), round(w * 1024 / cw)
    alg_r = N * H * 1024 + N * (8 + 256)
    alg_w = N * H * (512 + 16)
    rec = {"kernel": "irq_kernel<0> (inv_rope_fp8_quant, fp32 scales)",
           "workload": cfg["name"], "kernel_sha256_16": kernel_hash(),
           "fetch_size_kib_per_dispatch": f, "write_size_kib_per_dispatch": w,
           "calibration": {"kernel": "__amd_rocclr_copyBuffer, 1 GiB device copy "
                                     "(bench.py --only copy)",
                           "fetch_factor": cf, "write_factor": cw},
           "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
           "traffic_bytes_per_launch": rd + wr,
           "algorithmic_read_bytes": alg_r, "algorithmic_write_bytes": alg_w,
           "traffic_over_algorithmic": (rd + wr) / (alg_r + alg_w)}
    if sq:
        rec["sq_counters_per_dispatch"] = {
            c: v for (k, g, c), (v, _) in counter_medians(sq).items()
            if k.startswith("irq_kernel<0>") and g == grid}
    with open(PROFILE_COUNTERS, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: the GPU's clocks need ~100 launches (~12 ms) to ramp up
    # from idle, so the timed region starts after 100 untimed launches
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--only", choices=["irq", "qnr", "kvi", "idx", "variants", "decode", "copy",
                                       "stream"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kvi-tokens", type=int, default=None,
                    help="with --only kvi: tokens inserted (default 8192)")
    ap.add_argument("--kvi-slots", choices=["perm", "seq"], default="perm",
                    help="with --only kvi: a seeded permutation of the slots (default) or "
                         "slots 0..N-1 in token order")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="print per-kernel medians of rocprofv3 output directories and exit")
    ap.add_argument("--write-counters-json", nargs="+", metavar="DIR",
                    help="IRQ_FETCH IRQ_WRITE COPY_FETCH COPY_WRITE [SQ]: write the counter "
                         "record bench lines read their traffic from, and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.write_counters_json:
        write_counters_json(*args.write_counters_json)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path has no cross-GPU step, and "
              "each GPU would run the same kernels on its own shard (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if (args.kvi_tokens is not None or args.kvi_slots != "perm") and args.only != "kvi":
        ap.error("--kvi-tokens and --kvi-slots go with --only kvi")
    if args.kvi_tokens is not None and not 1 <= args.kvi_tokens <= 1 << 20:
        ap.error("--kvi-tokens must be in [1, 2^20]")

    import torch

    import rope_fp8_quant_amd as rq
    rq.abi_version()  # loads libropequant.so or raises
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    stream = torch.cuda.current_stream(device)

    if args.only == "copy":
        print(json.dumps({"copy_calibration": bench_copy(args, device, stream)}))
        return
    ceiling = None
    if args.only in (None, "stream", "kvi", "idx", "variants"):
        progress("streaming ceiling")
        ceiling = bench_stream(args, device, stream)
        CEILING.update(floor_us=ceiling["empty_launch"]["us_graph"],
                       gbs=round(ceiling["irq_pattern"]["gbs"], 1),
                       small_us=round(ceiling["irq_pattern_8192_units"]["us"], 3),
                       small_us_2=round(ceiling["irq_pattern_8192_units_2_per_wave"]["us"], 3))
        torch.cuda.empty_cache()
    if args.only == "stream":
        print(json.dumps({"stream_ceiling": ceiling}))
        return
    if args.only in ("qnr", "kvi", "idx"):
        extra = bench_qnr_kvi(args, device, stream)
        vs_same_size_stream(extra, ceiling)
        print(json.dumps({"extra": extra, "stream_ceiling": ceiling}))
        return
    if args.only == "decode":
        print(json.dumps({"decode": bench_decode(args, device, stream)}))
        return
    if args.only == "variants":
        print(json.dumps({"extra": bench_variants(args, device, stream),
                          "stream_ceiling": ceiling}))
        return

    cfg, ms, host_inputs, sets = bench_irq(args, device, stream)
    N, H = cfg["N"], cfg["H"]
    b = irq_bytes(N, H)
    gbs = b / ms / 1e6
    extra = {}
    if args.only is None:
        torch.cuda.empty_cache()
        progress("headline done; same buffers back to back")
        _, ms_1, _, _ = bench_irq(args, device, stream, same_buffers=True)
        extra["inv_rope_fp8_quant_same_buffers"] = dict(
            note="one buffer set relaunched back to back: writes land on lines the last "
                 "launch left in the 256 MB MALL, so this is faster than cold HBM",
            us=ms_1 * 1e3, gbs=b / ms_1 / 1e6, frac=b / ms_1 / 1e6 / HBM_PEAK_GBS)
        torch.cuda.empty_cache()
        progress("ue8m0")
        _, ms_ue, _, sets_ue = bench_irq(args, device, stream, "ue8m0")
        bu = irq_bytes(N, H, "ue8m0")
        extra["inv_rope_fp8_quant_ue8m0"] = dict(
            us=ms_ue * 1e3, gbs=bu / ms_ue / 1e6, frac=bu / ms_ue / 1e6 / HBM_PEAK_GBS,
            buffer_sets=sets_ue)
        torch.cuda.empty_cache()
        progress("qnr / kvi / fused / indexer / irregular")
        extra.update(bench_qnr_kvi(args, device, stream))
        torch.cuda.empty_cache()
        progress("output variants")
        extra.update(bench_variants(args, device, stream))
        torch.cuda.empty_cache()
        progress("decode")
        extra["decode"] = bench_decode(args, device, stream)
    line = {
        "metric": "achieved HBM GB/s (% of peak) + tokens/s, inv_rope_fp8_quant 16k tok\u00d732 heads",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded bf16 N(0,1) with 1% x20 outliers; positions 0..16383)",
        "config": {"workload": cfg["name"], "n_tokens": N, "n_heads": H,
                   "heads_per_group": cfg["hpg"], "head_dim": 512, "scale_fmt": "fp32",
                   "algorithmic_bytes": b, "pages_convention_bytes": N * H * 1536,
                   "buffer_sets": sets},
        "tokens_per_s": round(N / (ms / 1e3), 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile()},
    }
    if not args.no_cpu_baseline:
        progress("cpu baseline (oracle, one thread)")
        line["cpu_baseline"] = cpu_baseline(host_inputs)
        progress("cpu baseline (oracle, sharded)")
        line["cpu_baseline_sharded"] = cpu_baseline_sharded(host_inputs)
    if extra:
        line["extra"] = extra
    vs_same_size_stream(extra, ceiling)
    if ceiling:
        line["stream_ceiling"] = ceiling
        line["frac_of_stream_ceiling"] = round(gbs / ceiling["irq_pattern"]["gbs"], 4)
        line["frac_of_stream_ceiling_2_per_wave"] = round(
            gbs / ceiling["irq_pattern_2_per_wave"]["gbs"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
