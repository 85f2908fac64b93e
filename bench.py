"""Decode-attention benchmark on one MI355X.

One step = one decode token for every request: for each of the 16 layers,
pkv_decode_attention (split-KV tile partials) then pkv_merge_partials (FP32
LSE merge) on the same stream (with --overlap, layer l's merge runs on a
second stream while layer l+1 decodes, and the step ends when every merge
has; the line reports the other schedule too).  Default workload: 1 request x
262,144 tokens, 16 layers, 24 q / 4 KV heads, head_dim 256, bf16, 64-token
pages in a 16 GiB arena in random physical order, 1 % of keys scaled by 4;
each 32,768-token staging window of the history is split-KV eight ways into
4,096-token tiles and all 64 partials are merged in FP32.  Inputs are
synthetic (seeded) and resident in HBM before timing.

`value` comes from K steps timed with nothing but the path between two
events; `roofline.achieved` from K further steps with an event pair around
every pkv_decode_attention call.

Prints one JSON line.  `value` is KV GB/s: K+V bytes the exact path must read
per step (sum of lengths x 4,096 B x 16 layers) over the step time.

    python bench.py [--steps K] [--warmup W] [--workload long262k|conc|mixed]
                    [--tile T] [--split S] [--kernel mfma|valu] [--no-cpu-baseline]
"""

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published

# HBM traffic of one decode-kernel launch on the 262K workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
# scaled by the factor the same counter shows on a plain 1 GiB device copy
# (FETCH_SIZE reads 0.5x of the bytes a copy must read, WRITE_SIZE 1.0x).
# Valid only for the kernel code it was measured on (source_sha256 hashes the
# code without comments, see code_text).
PMC_TRAFFIC = {
    "source_sha256": "a950b23bf0cf8c5dcb12f3dc4e9c7c2c5ff553a34187b072a7db2d9568dd4ef2",
    "workload": "long262k", "tile": 4096, "split": 4096,
    "fetch_kib": 524503.3, "fetch_scale": 1048576 / 524300.1,
    "write_kib": 1584.0, "write_scale": 1.0,
}
KERNEL_SOURCES = ("paged_kv_cache_10_amd/csrc/decode_mfma.hip", "paged_kv_cache_10_amd/csrc/decode_exact.h",
                  "paged_kv_cache_10_amd/csrc/device.h")

# The same for the 4-request workload's decode call (LAUNCH["conc"]): the
# decode kernel plus the tile finalize launch, FETCH_SIZE and WRITE_SIZE of
# both dispatches added, calibrated on the plain copy of the same runs.
PMC_TRAFFIC_CONC = {
    "source_sha256": "aed1d9749dd54b077c9ebed44cf2c2c2ba450c8451d74ce95a95bd288f412b3e",
    "workload": "conc", "tile": 8192, "split": 2048,
    "fetch_kib": 254293.9 + 845.0, "fetch_scale": 1048576 / 524300.1,
    "write_kib": 1584.4 + 387.0, "write_scale": 1.0,
}
CONC_SOURCES = KERNEL_SOURCES + ("paged_kv_cache_10_amd/csrc/merge.hip",)

# The same for the mixed batch's decode call with per-request tiles planned
# for LAUNCH["mixed"]["plan"] work-groups (the decode kernel alone).
PMC_TRAFFIC_MIXED = {
    "source_sha256": PMC_TRAFFIC["source_sha256"],
    "workload": "mixed", "plan": 256,
    "fetch_kib": 854230.6, "fetch_scale": 1048576 / 524301.2,
    "write_kib": 5922.5, "write_scale": 1.0,
}

# The same for the compact kernel on the 262K compact-older workload
# (COMPACT_LAUNCH), calibrated on the same plain copy in the same runs.
PMC_TRAFFIC_FP8 = {
    "source_sha256": "26051ccbf69d5f419e8fa9c0320be1a6b824a4573358e9306c72fda63a33c0a0",
    "workload": "long262k", "tile": 4800, "split": 4800,
    "fetch_kib": 230053.1, "fetch_scale": 1048576 / 524299.5,
    "write_kib": 1188.0, "write_scale": 1.0,
}
FP8_SOURCES = ("paged_kv_cache_10_amd/csrc/decode_fp8.hip", "paged_kv_cache_10_amd/csrc/decode_compact.h",
               "paged_kv_cache_10_amd/csrc/compact.h", "paged_kv_cache_10_amd/csrc/device.h")

# The same for the one-launch kernel of both runs (COMPACT_LAUNCH, "one_launch").
PMC_TRAFFIC_RUNS = {
    "source_sha256": "011204fb636cf51a8966593aa409ca4424a6f58b53c923a6ff6da57d0c1877cf",
    "workload": "long262k", "tile": 4800, "exact_tile": 2560,
    "fetch_kib": 295722.7, "fetch_scale": 1048576 / 524299.5,
    "write_kib": 1507.5, "write_scale": 1.0,
}
RUNS_SOURCES = ("paged_kv_cache_10_amd/csrc/decode_runs.hip", "paged_kv_cache_10_amd/csrc/decode_compact.h",
                "paged_kv_cache_10_amd/csrc/decode_exact.h", "paged_kv_cache_10_amd/csrc/compact.h",
                "paged_kv_cache_10_amd/csrc/device.h")


# The same for the merge alone on the merge-stress shape (merge_kernel, 64 x
# 24 rows x 256 partials), calibrated on the plain copy of the same runs.
PMC_TRAFFIC_MERGE = {
    "source_sha256": "e3f12e65f1287392e7c45f3360af71f04782a96851f2b181cbeb6fbaf2965a3a",
    "fetch_kib": 197466.5, "fetch_scale": 1048576 / 524301.2,
    "write_kib": 1584.0, "write_scale": 1.0,
}
MERGE_SOURCES = ("paged_kv_cache_10_amd/csrc/merge.hip", "paged_kv_cache_10_amd/csrc/device.h")


def code_text(text):
    """C/C++ source without its comments, whitespace runs collapsed to one
    space: what the compiler sees, so that a comment edit does not count as
    a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def sources_sha256(files, root=None):
    """SHA-256 over the code (code_text) of each file, in order; paths are
    relative to `root` (default: the repository)."""
    import hashlib
    h = hashlib.sha256()
    root = root or os.path.dirname(os.path.abspath(__file__))
    for f in files:
        with open(os.path.join(root, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def time_graph(L, K, stream, use_merged, decode_layer, pkv, pool, qs, dt, dc, span, T, w, po, pl,
               outs, lses, ws, args, timed_o, timed_l, same):
    """The timed step (every layer's decode and merge) captured once in a HIP
    graph on a side stream and replayed: the replay time per step, and three
    replays, each after the outputs are poisoned by eager work, checked bit
    for bit against the eager step."""
    import torch
    gs = torch.cuda.Stream()               # default priority

    def gstep():
        for layer in range(L):
            if use_merged:
                pkv.decode_attention_merged(pool, layer, qs[layer], dt, dc, span, T, w.scale,
                                            po[layer], pl[layer], outs[layer], lses[layer],
                                            workspace=ws, kernel=args.kernel,
                                            split_tokens=args.split, stream=gs)
            else:
                decode_layer(layer, gs)
                pkv.merge_partials(po[layer], pl[layer], outs[layer], lses[layer], stream=gs)

    gs.wait_stream(stream)
    gstep()                                 # eager, on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=gs):
        gstep()
    torch.cuda.synchronize()
    ok = True
    for _ in range(3):
        outs.fill_(float("nan"))
        lses.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = ok and same(outs, timed_o) and same(lses, timed_l)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    for _ in range(K):
        g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    del g
    torch.cuda.synchronize()
    return {"ms_per_step": round(ms, 4), "replays_equal_eager_bitwise": ok,
            "kv_GBs": round(w.kv_bytes_per_step / (ms * 1e-3) / 1e9, 1)}


def pmc_traffic(workload, tile, split, kernel, plan=0):
    """Counter-derived HBM bytes per launch, or None if they were not taken
    on this kernel source and launch configuration."""
    if plan:
        t = PMC_TRAFFIC_MIXED
        if ((workload, plan, kernel) != (t["workload"], t["plan"], "mfma")
                or sources_sha256(KERNEL_SOURCES) != t["source_sha256"]):
            return None
        return int(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])
    for t, sources in ((PMC_TRAFFIC, KERNEL_SOURCES), (PMC_TRAFFIC_CONC, CONC_SOURCES)):
        if (workload, tile, split, kernel) != (t["workload"], t["tile"], t["split"], "mfma"):
            continue
        if sources_sha256(sources) != t["source_sha256"]:
            return None
        return int(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])
    return None


# Launch configuration timed for each workload (tile tokens; tokens per
# work-group).  The full-size parity tests run exactly these.
# Every layer's merge follows its decode on the same stream, as a model whose
# next layer needs this layer's output runs them; --overlap instead runs
# layer l's merge on a second stream while layer l+1 decodes (the synthetic
# layers are independent), and the line reports the other schedule as well.
LAUNCH = {
    "long262k": dict(tile=4096, split=4096),   # 32K windows split-KV 8 ways
    "conc": dict(tile=8192, split=2048),       # the workload's 8,192-token tiles, split-KV 4 ways
    # per-request tiles planned for 256 work-groups (one per CU); --plan 0
    # runs the fixed 4,096-token tiling instead
    "mixed": dict(tile=4096, split=4096, plan=256),
    "tiny": dict(tile=1024, split=1024),
}


# Runs of two representations (--compact-older): every page older than the
# newest `exact_tail` tokens is served from compact (E4M3) pages.  Schedules:
# "one_launch" (both runs' work-groups in one pkv_decode_attention_runs
# grid), "tail_stream" (the exact run on a second stream beside the compact
# run's launch), "serial" (one call after the other on one stream).  The
# compact run's 4,800-token splits give 192 work-groups at 262K (48 splits x
# 4 KV heads, the last split 3,776 tokens), the exact tail's 2,048-token
# splits 64, so the two runs fill the 256 CUs once (each work-group reads
# 2.1-2.5 MB either way).  The full-size compact parity test runs exactly
# these.
COMPACT_LAUNCH = {
    # 192 compact work-groups of 4,800 tokens and 52 exact ones of 2,560 in
    # one grid (244 of 256 CUs): in a sweep of both tile sizes the fastest
    # (1.575 ms per step against 1.590 with 2,048-token exact tiles)
    "long262k": dict(exact_tail=32768, tile=4800, split=4800, exact_tile=2560, exact_split=2560,
                     schedule="one_launch"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long262k")
    ap.add_argument("--tile", type=int, default=0, help="tile tokens (default: LAUNCH)")
    ap.add_argument("--split", type=int, default=0, help="tokens per work-group (default: LAUNCH)")
    ap.add_argument("--kernel", default="mfma", choices=["mfma", "valu"])
    ap.add_argument("--separate", action="store_true",
                    help="decode and merge as separate calls (default: one merged call per "
                         "layer where the tiling allows)")
    ap.add_argument("--plan", type=int, default=None,
                    help="per-request tiles planned for this many work-groups (0: the fixed "
                         "tiling; default: LAUNCH)")
    ap.add_argument("--staged", action="store_true",
                    help="decode each 32,768-token staging window with its own call")
    ap.add_argument("--serial", action="store_true",
                    help="merge on the decode stream (the default)")
    ap.add_argument("--overlap", action="store_true",
                    help="merge layer l on a second stream while layer l+1 decodes")
    ap.add_argument("--window-streams", type=int, default=2,
                    help="--staged: streams the windows of a layer are spread over (they write "
                         "disjoint slots and run concurrently; 1 = one after the other)")
    ap.add_argument("--host-staged", action="store_true",
                    help="history in pinned host memory, staged per 32K window under leases")
    ap.add_argument("--compact-older", action="store_true",
                    help="serve pages older than the newest 32,768 tokens from compact (E4M3) "
                         "pages converted on the GPU; prints its own JSON line")
    ap.add_argument("--buffers", type=int, default=2,
                    help="staging buffers of the --host-staged mode")
    ap.add_argument("--merge-stress", action="store_true",
                    help="time pkv_merge_partials alone on 64 x 24 rows x 256 partials; "
                         "prints its own JSON line")
    ap.add_argument("--live", action="store_true",
                    help="the live pool: four ~31,744-token requests growing by one token per "
                         "step, device pool 3/4 of the pages, histories in pinned host memory")
    ap.add_argument("--live-compact", action="store_true",
                    help="the live pool with compact older pages: every page not resident is "
                         "staged as E4M3 codes and scales (half the bus bytes) and decoded as a "
                         "second run in the same launch")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the timed step in a HIP graph and time its replays")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the 4-request, mixed, merge-stress, live-pool and host-staged "
                         "lines the default run adds")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work budget of the oracle baseline sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also time a plain 1 GiB device copy (the PMC calibration kernel)")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the measured HBM read ceiling (probe_read, run first as a child)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only; --gpus {args.gpus} is not supported "
              "(no multi-GPU path exists)", file=sys.stderr)
        return 2
    ceiling = None if args.no_read_probe else read_probe()
    if args.merge_stress:
        print(json.dumps(merge_stress(args, ceiling)), flush=True)
        return 0
    if args.live or args.live_compact:
        print(json.dumps(live_pool(args)), flush=True)
        return 0
    import torch
    from paged_kv_cache_10_amd import inputs as I
    from paged_kv_cache_10_amd import pkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pkv.lib()

    w = I.workload(args.workload)
    launch = LAUNCH.get(args.workload, {})
    # per-request tiles (LAUNCH "plan"): only where nothing asks for the fixed tiling
    plan = launch.get("plan", 0) if args.plan is None else args.plan
    if (args.tile or args.split or args.staged or args.kernel != "mfma" or args.host_staged
            or args.compact_older):
        plan = 0
    # a 32,768-token window decoded alone holds 1/8 of the history: 512-token
    # splits give its launch 256 work-groups (4,096-token ones only 32), and
    # 512-token tiles (64 partials per head per window) need no tile finalize
    # staged windows spread over two streams run two at a time: 1,024-token
    # tiles give each window 128 work-groups, two windows fill the GPU; one
    # window at a time needs 512-token tiles to fill it alone (measured at
    # 262K: 3.27 ms per step against 3.72 one window at a time; 2,048-token
    # tiles on 4 streams 3.33, 1,024 on 3 or 4 streams 3.30 / 3.43)
    st_tile = 1024 if args.window_streams > 1 else 512
    w.tile_tokens = args.tile or (st_tile if args.staged else launch.get("tile", w.tile_tokens))
    args.split = args.split or (st_tile if args.staged else launch.get("split", 0))
    overlap = args.overlap and not args.serial
    T = w.tile_tokens
    B, Hq, Hkv, D, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_layers

    # ---------------------------------------------------------------- inputs
    t_gen = time.time()
    if plan:
        row_tiles, max_tiles = pkv.plan_tiles(w.ctx_lens, Hkv, plan)
        max_row = int(row_tiles.max())
        slots = max_tiles
        span = max_tiles * max_row
    else:
        slots = -(-w.max_ctx // T)
        span = slots * T
    width = span // w.page_tokens
    table = I.draw_page_tables(w, width)
    ctx = np.array(w.ctx_lens, dtype=np.int32)
    arena = torch.empty(w.num_pages * w.page_layer_bytes * L // 2, dtype=torch.int16, device=dev)
    arena.zero_()
    pool = pkv.Pool(arena, L, Hkv, D, w.page_tokens)
    dt = torch.empty(table.shape, dtype=torch.int32, device=dev)
    dc = torch.empty(B, dtype=torch.int32, device=dev)
    pkv.page_table_write(pool, table, ctx, dt, dc)
    qs = []
    for layer in range(L):
        qs.append(I.device_q(w, layer, dev))
        for b in range(B):
            k, v = I.device_kv(w, layer, b, dev)
            I.device_scatter(arena, w, layer, b, table[b], k, v)
            del k, v
    d_rt = torch.from_numpy(row_tiles).to(dev) if plan else None
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    # per-layer partial buffers: layer l's merge (second stream) overlaps
    # layer l+1's decode (main stream)
    po = torch.empty((L, B, Hq, slots, D), device=dev)
    pl = torch.empty((L, B, Hq, slots), device=dev)
    outs = torch.empty((L, B, Hq, D), device=dev)
    lses = torch.empty((L, B, Hq), device=dev)
    window = 32768 if args.staged else span
    ws_bytes = pkv.decode_workspace_bytes(B, Hq, window, T, D, args.kernel, args.split)
    ws = torch.zeros(max(16, ws_bytes) // 4 + 4, dtype=torch.float32, device=dev)
    # concurrent staged windows: one workspace and one stream each
    n_ws = max(1, args.window_streams) if args.staged else 1
    wss = [ws] + [torch.zeros_like(ws) for _ in range(n_ws - 1)]
    wstreams = [None] + [torch.cuda.Stream() for _ in range(n_ws - 1)]
    w_start = torch.cuda.Event()
    w_done = [torch.cuda.Event() for _ in range(n_ws)]
    stream = torch.cuda.current_stream()
    merge_stream = torch.cuda.Stream()          # default priority
    decoded = [torch.cuda.Event() for _ in range(L)]
    merged = torch.cuda.Event()

    def decode_layer(layer, s=None):
        s = stream if s is None else s
        if plan:
            pkv.decode_attention_rows(pool, layer, qs[layer], dt, dc, d_rt, max_row, max_tiles,
                                      w.scale, po[layer], pl[layer], stream=s)
            return
        if n_ws > 1:                       # windows round-robin over n_ws streams
            w_start.record(s)
            for ws_s in wstreams[1:]:
                ws_s.wait_event(w_start)
        for i, begin in enumerate(range(0, span, window)):
            k = i % n_ws
            pkv.decode_attention(pool, layer, qs[layer], dt[:, begin // w.page_tokens:], dc,
                                 begin, min(window, span - begin), T, w.scale, po[layer],
                                 pl[layer], workspace=wss[k], kernel=args.kernel,
                                 split_tokens=args.split, stream=s if k == 0 else wstreams[k])
        if n_ws > 1:                       # the merge waits for every window
            for k in range(1, n_ws):
                w_done[k].record(wstreams[k])
                s.wait_event(w_done[k])

    # a whole-history fixed tiling decodes and merges each layer in one call
    # (one kernel boundary fewer where tiles hold several splits); the
    # per-call roofline events and the overlapped schedule use separate calls
    use_merged = not plan and not args.staged and not args.separate

    def step(evs=None, overlap=overlap):
        for layer in range(L):
            if use_merged and evs is None and not overlap:
                pkv.decode_attention_merged(pool, layer, qs[layer], dt, dc, span, T, w.scale,
                                            po[layer], pl[layer], outs[layer], lses[layer],
                                            workspace=ws, kernel=args.kernel,
                                            split_tokens=args.split, stream=stream)
                continue
            if evs is not None:
                evs[layer][0].record(stream)
            decode_layer(layer)
            if evs is not None:
                evs[layer][1].record(stream)
            if overlap:
                decoded[layer].record(stream)
                merge_stream.wait_event(decoded[layer])
            pkv.merge_partials(po[layer], pl[layer], outs[layer], lses[layer],
                               stream=merge_stream if overlap else stream)
        if overlap:
            merged.record(merge_stream)
            stream.wait_event(merged)              # the step ends when every merge has

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # value: K steps with nothing but the path between two events
    K = args.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for k in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / K
    # five more passes of K steps: median and spread of the step time
    passes = []
    for _ in range(5):
        e0.record(stream)
        for k in range(K):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        passes.append(e0.elapsed_time(e1) / K)
    # the same steps in the other merge schedule, for comparison
    e0.record(stream)
    for k in range(K):
        step(overlap=not overlap)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_other = e0.elapsed_time(e1) / K
    # roofline: K more steps with an event pair around every decode call
    ev_dec = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(K)]
    for k in range(K):
        step(ev_dec[k])
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for evk in ev_dec for (a, b) in evk]
    dec_pairs_ms = float(np.mean(dec_ms))
    # and the decode calls alone, back to back: K passes of the L layers'
    # calls between one pair of events, so no event pair's own cost sits
    # inside every call; the mean duration of one call (the gaps between
    # consecutive kernels included)
    e0.record(stream)
    for k in range(K):
        for layer in range(L):
            decode_layer(layer)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_avg_ms = e0.elapsed_time(e1) / (K * L)

    # the timed schedule and the overlapped one against a serialized
    # recompute (separate decode and merge calls on one stream)
    def same(a, b):
        return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
    step()
    torch.cuda.synchronize()
    timed_o, timed_l = outs.clone(), lses.clone()
    step(overlap=True)
    torch.cuda.synchronize()
    ref_o, ref_l = outs.clone(), lses.clone()
    for layer in range(L):
        po[layer].fill_(float("nan"))
        decode_layer(layer)
        pkv.merge_partials(po[layer], pl[layer], outs[layer], lses[layer], stream=stream)
    torch.cuda.synchronize()
    self_check = same(ref_o, outs) and same(ref_l, lses)

    # optionally: the timed step captured once in a HIP graph and replayed
    graph_res = None
    if args.graph:
        graph_res = time_graph(L, K, stream, use_merged, decode_layer, pkv, pool, qs, dt, dc,
                               span, T, w, po, pl, outs, lses, ws, args, timed_o, timed_l, same)
    timed_check = same(timed_o, outs) and same(timed_l, lses)
    staged_vs_resident = None
    if args.staged:
        # one resident call over the whole history at the same tiling
        ws_r = torch.zeros(max(16, pkv.decode_workspace_bytes(B, Hq, span, T, D, args.kernel,
                                                              args.split)) // 4 + 4,
                           dtype=torch.float32, device=dev)
        staged_vs_resident = True
        for layer in range(L):
            rpo = torch.full_like(po[layer], float("nan"))
            rpl = torch.full_like(pl[layer], float("nan"))
            ro = torch.empty_like(outs[layer])
            rl = torch.empty_like(lses[layer])
            pkv.decode_attention(pool, layer, qs[layer], dt, dc, 0, span, T, w.scale, rpo, rpl,
                                 workspace=ws_r, kernel=args.kernel, split_tokens=args.split,
                                 stream=stream)
            pkv.merge_partials(rpo, rpl, ro, rl, stream=stream)
            torch.cuda.synchronize()
            staged_vs_resident = (staged_vs_resident and same(ro, timed_o[layer])
                                  and same(rl, timed_l[layer]))

    if args.host_staged and args.compact_older:
        res = host_staged_hybrid(args, w, pool, arena, table, ctx, qs, outs, lses, T, span)
        print(json.dumps(res), flush=True)
        return 0
    if args.host_staged:
        res = host_staged(args, w, pool, arena, table, ctx, qs, outs, lses, T, span)
        print(json.dumps(res), flush=True)
        return 0
    if args.compact_older:
        res = compact_older(args, w, pool, table, ctx, qs, outs, lses)
        if ceiling is not None:
            res["read_ceiling"] = ceiling
            res["roofline"]["frac_of_measured_ceiling"] = round(
                res["roofline"]["achieved"] / ceiling["blocks_nt_GBs"], 4)
        if args.copy_probe:
            res["copy_probe"] = copy_probe(dev, stream)
        print(json.dumps(res), flush=True)
        return 0

    kv_bytes_step = w.kv_bytes_per_step
    kv_gbs = kv_bytes_step / (ms_step * 1e-3) / 1e9
    tok_s = B / (ms_step * 1e-3)
    kv_bytes_layer = kv_bytes_step // L
    dec_gbs = kv_bytes_layer / (dec_avg_ms * 1e-3) / 1e9
    lengths = w.max_ctx if len(set(w.ctx_lens)) == 1 else "mixed"

    res = {
        "metric": "decode attention KV GB/s (% of HBM peak) and tokens/s at 262K ctx, 1 GPU",
        "value": round(kv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: {B} x {lengths} tokens, {L} layers, "
                        f"{Hq} q / {Hkv} kv heads, head_dim {D}, 64-token pages, "
                        + (f"per-request tiles planned for {plan} work-groups (at most "
                           f"{max_row} tokens, {max_tiles} per request)" if plan else f"tile {T}")
                        + (f", staged 32768-token windows ({n_ws} streams)" if args.staged
                           else ""),
            "batch": B, "ctx_lens_sum": int(sum(w.ctx_lens)), "layers": L,
            "tile_tokens": row_tiles.tolist() if plan else T,
            "kernel": args.kernel, "split_tokens": args.split or "default",
            "merge_overlapped": overlap,
            "decode_and_merge": ("pkv_decode_attention_merged, one call per layer"
                                 if use_merged and not overlap else "separate calls"),
            "parallelism": "none (1 GPU)",
        },
        "tokens_per_s": round(tok_s, 2),
        "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv_bytes_step,
        "total_bytes_per_step": total_bytes_step(
            w, slots, ws_bytes // (B * Hq * (D + 1) * 4) * (span // window)),
        "passes": {"n": len(passes), "ms_per_step_median": round(float(np.median(passes)), 4),
                   "ms_per_step_min": round(min(passes), 4),
                   "ms_per_step_max": round(max(passes), 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_mfma_kernel" if args.kernel == "mfma" else "decode_valu_kernel",
            "launch": ("one pkv_decode_attention_rows call per layer = the decode kernel" if plan
                       else (f"{span // window} pkv_decode_attention calls per layer (one per "
                             f"{window}-token window), each" if window < span
                             else "one pkv_decode_attention call per layer =")
                       + " the decode kernel"
                       + ("" if ws_bytes == 0 else " + the tile finalize")),
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": kv_bytes_layer,
            "avg_launch_ms": round(dec_avg_ms, 5),
            "timing": "HIP events on the decode stream around K passes of the layers' decode "
                      "calls back to back, divided by the calls",
            "avg_launch_ms_event_pair_per_call": round(dec_pairs_ms, 5),
            "traffic": pmc_traffic(args.workload, T, args.split, args.kernel, plan),
        },
        "setup_s": round(t_gen, 1),
        "overlapped_equals_serial_bitwise": self_check,
        **({"graph": graph_res} if graph_res is not None else {}),
        "timed_equals_serial_bitwise": timed_check,
        **({"staged_equals_resident_bitwise": staged_vs_resident,
            "window_streams": n_ws} if args.staged else {}),
        ("serial_merges" if overlap else "overlapped_merges"): {
            "ms_per_step": round(ms_other, 4),
            "value": round(kv_bytes_step / (ms_other * 1e-3) / 1e9, 1),
            "hbm_frac": round(kv_bytes_step / (ms_other * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }

    if ceiling is not None:
        res["read_ceiling"] = ceiling
        res["roofline"]["frac_of_measured_ceiling"] = round(dec_gbs / ceiling["blocks_nt_GBs"], 4)

    if args.copy_probe:
        res["copy_probe"] = copy_probe(dev, stream)

    res["append"] = append_probe(w, dev, stream)
    res["append"]["share_of_step"] = round(L * res["append"]["us_per_layer"] * 1e-3 / ms_step, 4)
    res["admission"] = admission_probe(w)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, qs, args.cpu_seconds)

    default_run = (args.workload == "long262k" and not (args.tile or args.staged or args.separate
                                                        or args.overlap or args.graph
                                                        or args.kernel != "mfma"))
    if default_run and not args.no_others:
        del arena, pool, po, pl, outs, lses, qs
        torch.cuda.empty_cache()
        res["other_workloads"] = other_workloads(args)

    print(json.dumps(res), flush=True)
    return 0


def host_staged(args, w, pool, arena, table, ctx, qs, ref_outs, ref_lses, T, span):
    """The history in pinned host memory (a copy of the arena), every layer
    decoded window by window from a staging buffer under a lease: the
    staged path of the pages, bound by host-to-device bandwidth."""
    import torch
    from paged_kv_cache_10_amd import pkv
    dev = arena.device
    L, B, Hq, D = w.num_layers, w.batch, w.num_q_heads, w.head_dim
    window = 32768
    # Host pool: each history contiguous, one segment per layer (GPU memory
    # management page, "A host pool that explains its own size"): host page
    # base_b + i holds logical page i of request b.
    npg = [-(-c // w.page_tokens) for c in w.ctx_lens]
    bases = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int64)
    Ph = int(sum(npg))
    blk = w.page_layer_bytes // 2
    host = torch.empty((L, Ph, blk), dtype=torch.int16, pin_memory=True)
    dev_slab = arena.view(L, -1, blk)
    for layer in range(L):
        for b, n in enumerate(npg):
            idx = torch.as_tensor(table[b, :n].astype(np.int64), device=dev)
            host[layer, bases[b]:bases[b] + n].copy_(dev_slab[layer].index_select(0, idx))
    torch.cuda.synchronize()
    host_table = np.full(table.shape, -1, dtype=np.int32)
    for b, n in enumerate(npg):
        host_table[b, :n] = bases[b] + np.arange(n)
    wpp = window // w.page_tokens
    nbuf = args.buffers
    st_arena = torch.empty(nbuf * B * wpp * w.page_layer_bytes // 2, dtype=torch.int16,
                           device=dev)
    st_pool = pkv.Pool(st_arena, 1, w.num_kv_heads)
    compute = torch.cuda.current_stream()
    copy_s, wb_s = torch.cuda.Stream(), torch.cuda.Stream()
    stager = pkv.Stager(st_pool, host, L, B, window, nbuf, copy_s, compute, wb_s)
    slots = span // T
    wspan = -(-span // window) * window
    po = torch.empty((B, Hq, wspan // T, D), device=dev)
    pl = torch.empty((B, Hq, wspan // T), device=dev)
    outs = torch.empty_like(ref_outs)
    lses = torch.empty_like(ref_lses)
    dc = torch.tensor(ctx, dtype=torch.int32, device=dev)
    nb = pkv.decode_workspace_bytes(B, Hq, window, T, D, args.kernel, args.split)
    ws = torch.zeros(max(16, nb) // 4 + 4, device=dev)
    pos = po[:, :, :slots]
    pls = pl[:, :, :slots]

    def step():
        for layer in range(L):
            for begin in range(0, wspan, window):
                lease = stager.begin(layer, host_table, ctx, begin)
                pkv.decode_attention(st_pool, lease.staging_layer, qs[layer], stager.table(lease),
                                     dc, begin, window, T, w.scale, po, pl, workspace=ws,
                                     kernel=args.kernel, split_tokens=args.split, stream=compute)
                stager.seal(lease)
            pkv.merge_partials(pos.contiguous(), pls.contiguous(), outs[layer], lses[layer],
                               stream=compute)

    step()
    stager.retire()
    ok = bool(torch.equal(outs.view(torch.int32), ref_outs.view(torch.int32))
              and torch.equal(lses.view(torch.int32), ref_lses.view(torch.int32)))
    K = max(1, min(args.steps, 5))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(compute)
    for _ in range(K):
        step()
    e1.record(compute)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    receipts = stager.retire()
    stager.destroy()
    h2d_ceiling = h2d_ceiling_GBs(host, dev, compute, copy_s)
    copied = sum(-(-c // w.page_tokens) for c in w.ctx_lens) * w.page_layer_bytes * L
    kv = w.kv_bytes_per_step
    return {
        "metric": "decode attention KV GB/s (% of HBM peak) and tokens/s at 262K ctx, 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": 1, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: history in pinned host memory (each history "
                               f"contiguous per layer), staged per 32,768-token window under "
                               f"leases ({nbuf} buffers, each window copied as two halves on "
                               f"two copy streams), tile {T}",
                   "tile_tokens": T, "split_tokens": args.split},
        "tokens_per_s": round(B / (ms * 1e-3), 3),
        "staged_equals_resident_bitwise": ok,
        "leases_per_step": L * (wspan // window), "receipts": receipts,
        "roofline": {"bound": "host-to-device", "achieved": round(copied / (ms * 1e-3) / 1e9, 2),
                     "peak": round(h2d_ceiling, 2), "unit": "GB/s",
                     "frac": round(copied / (ms * 1e-3) / 1e9 / h2d_ceiling, 4),
                     "peak_kind": "measured: plain 1 GiB pinned-to-device copy (faster of one "
                                  "copy and two halves on two streams)"},
    }


def h2d_ceiling_GBs(host, dev, compute, copy_s):
    """Host-to-device ceiling: a plain 1 GiB pinned-to-device copy from the
    pinned tensor `host`, as one copy and as two halves on two streams; the
    faster of the two, in GB/s."""
    import torch
    src = host.view(-1)[: 1 << 29]
    dst = torch.empty(src.shape, dtype=torch.int16, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h = src.numel() // 2

    def h2d(halves):
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(compute)
        copy_s.wait_event(c0)
        for _ in range(3):
            if halves:
                dst[:h].copy_(src[:h], non_blocking=True)
                with torch.cuda.stream(copy_s):
                    dst[h:].copy_(src[h:], non_blocking=True)
            else:
                dst.copy_(src, non_blocking=True)
        done = torch.cuda.Event()
        done.record(copy_s)
        compute.wait_event(done)
        c1.record(compute)
        torch.cuda.synchronize()
        return 3 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    return max(h2d(False), h2d(True))


def live_pool(args):
    """The live pool (pkv_live_*) on the 4-request shape: each history in
    pinned host memory (contiguous per layer), a device pool of 1,491 pages
    (3/4 of the histories' pages), admission per step, hot pages copied in,
    the rest staged per layer, the new token appended and its rows written
    back, one decode over the composed table per layer.  First the 20-step
    schedule of the GPU test (targets change, a request pauses), every layer
    checked bitwise against a resident decode; then `steps` timed steps with
    all four requests growing, against the resident decode of the same
    histories.

    With --live-compact every page full in the final histories has a compact
    copy (converted once on the GPU, kept in pinned host memory) published
    from the start, so each page the pool does not hold is staged compact:
    the exact run (2,048-token tiles over the composed table, compact pages
    masked) and the compact run (2,048-token tiles) in one launch, then one
    merge.  Checked bitwise against the same two runs over resident copies
    (tables read back after each schedule step)."""
    import torch
    from paged_kv_cache_10_amd import inputs as I
    from paged_kv_cache_10_amd import pkv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    compact = bool(args.live_compact)
    sc = I.live_schedule(20)
    grow = args.warmup + args.steps
    final = [f + grow for f in sc["final"]]
    W = I.Workload("live", seed=81, ctx_lens=final, num_layers=16, tile_tokens=8192)
    L, Hq, Hkv, D, PT = W.num_layers, W.num_q_heads, W.num_kv_heads, W.head_dim, W.page_tokens
    width = 4 * 8192 // PT
    T, SPLIT, CT = (2048, 0, 2048) if compact else (8192, 2048, 0)
    npg = [-(-c // PT) for c in final]
    bases = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int64)
    Ph = int(sum(npg))
    table = np.full((W.batch, width), -1, dtype=np.int32)
    for b, n in enumerate(npg):
        table[b, :n] = bases[b] + np.arange(n)        # each history contiguous per layer
    plb = W.page_layer_bytes
    resident = torch.zeros(Ph * plb * L // 2, dtype=torch.int16, device=dev)
    new_k, new_v = {}, {}
    qs = []
    for layer in range(L):
        qs.append(I.device_q(W, layer, dev))
        for b in range(W.batch):
            k, v = I.device_kv(W, layer, b, dev)
            I.device_scatter(resident, W, layer, b, table[b], k, v)
            new_k[layer, b] = k[:, sc["start"][b]:].contiguous()
            new_v[layer, b] = v[:, sc["start"][b]:].contiguous()
            del k, v
    host = torch.empty(resident.numel(), dtype=torch.int16, pin_memory=True)
    host.copy_(resident)
    rpool = pkv.Pool(resident, L, Hkv)
    dev_rtab = torch.tensor(table, dtype=torch.int32, device=dev)
    arena = torch.zeros(sc["pool_pages"] * plb * L // 2, dtype=torch.int16, device=dev)
    pool = pkv.Pool(arena, L, Hkv)
    K_BUF = 2
    sarena = torch.zeros(K_BUF * Ph * plb // 2, dtype=torch.int16, device=dev)
    spool = pkv.Pool(sarena, K_BUF, Hkv)
    copy_s, wb_s = torch.cuda.Stream(), torch.cuda.Stream()
    compute = torch.cuda.current_stream()
    live = pkv.Live(pool, spool, host, W.batch, width, copy_s, compute, wb_s)
    for c, (t, bu) in sc["contexts"].items():
        live.add(c, t, bu)
    E = width * PT // T
    CS = width * PT // CT if compact else 0
    S = E + CS
    if compact:
        cpb = pkv.compact_page_bytes(L, Hkv)
        cfull_arena = torch.zeros(Ph * cpb, dtype=torch.uint8, device=dev)
        cfull = pkv.Pool(cfull_arena, L, Hkv, compact=True)
        full_pages = np.concatenate([bases[b] + np.arange(c // PT)
                                     for b, c in enumerate(final)]).astype(np.int32)
        ids_dev = torch.from_numpy(full_pages).to(dev)
        crc = torch.zeros(ids_dev.numel(), dtype=torch.int32, device=dev)
        pkv.compact_convert(rpool, cfull, ids_dev, ids_dev, crc)
        torch.cuda.synchronize()
        chost = torch.empty(cfull_arena.numel(), dtype=torch.uint8, pin_memory=True)
        chost.copy_(cfull_arena)
        carena = torch.zeros(K_BUF * Ph * cpb // L, dtype=torch.uint8, device=dev)
        cstage = pkv.Pool(carena, K_BUF, Hkv, compact=True)
        live.attach_compact(cstage, chost, CT)
        live.publish(full_pages)
        cplb_all = cpb // L                      # codes and scales of one (layer, page)
    nbw = pkv.decode_workspace_bytes(W.batch, Hq, E * T, T, D, 0, SPLIT or T)
    ws = torch.zeros(max(16, nbw) // 4 + 4, device=dev)
    ws_r = torch.zeros_like(ws)
    po = torch.empty((L, W.batch, Hq, S, D), device=dev)
    pl = torch.empty((L, W.batch, Hq, S), device=dev)
    outs = torch.empty((L, W.batch, Hq, D), device=dev)
    lses = torch.empty((L, W.batch, Hq), device=dev)
    rpo, rpl, routs, rlses = (torch.empty_like(x) for x in (po, pl, outs, lses))
    length = list(sc["start"])

    def live_step(ids, lens):
        n = len(ids)
        status, info = live.begin(ids, lens, table[ids])
        for layer in range(L):
            kn = torch.stack([new_k[layer, c][:, lens[i] - 1 - sc["start"][c]]
                              for i, c in enumerate(ids)])
            vn = torch.stack([new_v[layer, c][:, lens[i] - 1 - sc["start"][c]]
                              for i, c in enumerate(ids)])
            live.layer(layer, qs[layer][:n], kn, vn, T, W.scale, po[layer, :n], pl[layer, :n],
                       outs[layer, :n], lses[layer, :n], workspace=ws, split_tokens=SPLIT)
        return status, info

    def resident_tables(ids, lens):
        """With compact pages: the open step's composition read back, as
        tables over resident copies (the exact run masked where the page is
        compact, the compact run naming host pages = compact copies)."""
        n = len(ids)
        comp = live.table(n)[0].cpu().numpy()
        clen = live.compact_table(n)[1].cpu().numpy()
        ref_e = table[ids].copy()
        ref_c = np.full((n, width), -1, np.int32)
        for i, ln in enumerate(lens):
            need = -(-ln // PT)
            lps = np.nonzero(comp[i, :need] == -1)[0]
            ref_e[i, lps] = -1
            ref_c[i, :lps.size] = table[ids[i], lps]
        return (torch.from_numpy(ref_e).to(dev), torch.from_numpy(ref_c).to(dev),
                torch.from_numpy(clen.astype(np.int32)).to(dev))

    def resident_step(ids, lens, tabs=None):
        n = len(ids)
        dl = torch.tensor(lens, dtype=torch.int32, device=dev)
        if compact:
            de, dc, dcl = tabs
            for layer in range(L):
                pkv.decode_attention_runs(layer, qs[layer][:n],
                                          [(rpool, de, dl, E * T, T, 0),
                                           (cfull, dc, dcl, CS * CT, CT, E)],
                                          W.scale, rpo[layer, :n], rpl[layer, :n])
                pkv.merge_partials(rpo[layer, :n], rpl[layer, :n], routs[layer, :n],
                                   rlses[layer, :n])
            return
        rows = dev_rtab[ids].contiguous()
        for layer in range(L):
            pkv.decode_attention_merged(rpool, layer, qs[layer][:n], rows, dl, S * T, T, W.scale,
                                        rpo[layer, :n], rpl[layer, :n], routs[layer, :n],
                                        rlses[layer, :n], workspace=ws_r, split_tokens=SPLIT)

    def same(a, b):
        return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
    # the schedule, every step and layer against the resident decode
    ok = True
    kinds = {}
    for st in sc["steps"]:
        for c, (t, bu) in st["set_target"].items():
            live.set_target(c, t, bu)
        ids, lens = st["ids"], st["lengths"]
        for c, ln in zip(ids, lens):
            length[c] = ln
        live_step(ids, lens)
        resident_step(ids, lens, resident_tables(ids, lens) if compact else None)
        torch.cuda.synchronize()
        n = len(ids)
        ok = ok and all(same(x[:, :n], y[:, :n]) for x, y in
                        ((po, rpo), (pl, rpl), (outs, routs), (lses, rlses)))
        for e in live.admission.events():
            kinds[e["kind"]] = kinds.get(e["kind"], 0) + 1
    # steady steps: all four growing
    ids = [0, 1, 2, 3]
    infos = []

    def grow_step():
        for c in ids:
            length[c] += 1
        infos.append(live_step(ids, [length[c] for c in ids])[1])
    for _ in range(args.warmup):
        grow_step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    first = len(infos)
    lens_timed = []
    e0.record(compute)
    for _ in range(args.steps):
        grow_step()
        lens_timed.append([length[c] for c in ids])
    # the step ends when its last write-back has landed
    done = torch.cuda.Event()
    done.record(wb_s)
    compute.wait_event(done)
    e1.record(compute)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    timed = infos[first:]
    # the resident decode of the same histories, same tiling (with compact
    # pages: the last timed step's composition for every step)
    tabs = resident_tables(ids, lens_timed[-1]) if compact else None
    e0.record(compute)
    for lens in lens_timed:
        resident_step(ids, lens, tabs)
    e1.record(compute)
    torch.cuda.synchronize()
    ms_res = e0.elapsed_time(e1) / args.steps
    live.destroy()
    ceiling = h2d_ceiling_GBs(host, dev, compute, copy_s)
    staged = float(np.mean([i["staged_pages"] for i in timed]))
    hot = float(np.mean([i["copied_in_pages"] for i in timed]))
    cstaged = float(np.mean([i["compact_staged_pages"] for i in timed]))
    kv = float(np.mean([sum(x) for x in lens_timed])) * 4096 * L
    h2d = (staged + hot) * plb * L + W.batch * (width + 2) * 4
    kv_read = kv
    if compact:
        h2d += cstaged * cplb_all * L + W.batch * (width + 1) * 4
        kv_read = kv - cstaged * PT * 4096 * L + cstaged * cplb_all * L
    d2h = W.batch * L * 2 * Hkv * D * 2
    hbm = kv_read + (staged + hot) * plb * L + d2h + (cstaged * cplb_all * L if compact else 0)
    return {
        "metric": "decode attention KV GB/s (% of HBM peak) and tokens/s at 262K ctx, 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "data": "synthetic",
        "dtype": "bf16 + e4m3 (pages not resident)" if compact else "bf16",
        "config": {"workload": "live pool: 4 requests of ~31,744 tokens growing by one token per "
                               "step, 16 layers, histories in pinned host memory (contiguous per "
                               "layer), device pool of 1,491 pages (3/4 of the histories' pages), "
                               + ("every page not resident staged compact (E4M3 codes + FP32 block "
                                  "scales), exact and compact runs with 2,048-token tiles in one "
                                  "launch, 2 staging buffers of each kind; value counts every "
                                  "token at its bf16 size"
                                  if compact else "tile 8192 / split 2048, 2 staging buffers"),
                   "pool_pages": sc["pool_pages"], "history_pages": Ph},
        "tokens_per_s": round(W.batch / (ms * 1e-3), 2),
        "schedule_equals_resident_bitwise": ok,
        "schedule_page_sources": kinds,
        "per_step": {"staged_pages_per_layer": staged, "copied_in_pages": hot,
                     "compact_staged_pages_per_layer": cstaged,
                     "host_to_device_bytes": int(h2d), "device_to_host_bytes": int(d2h),
                     "hbm_bytes": int(hbm), "kv_bytes_read": int(kv_read)},
        "roofline": {"bound": "host-to-device", "achieved": round(h2d / (ms * 1e-3) / 1e9, 2),
                     "peak": round(ceiling, 2), "unit": "GB/s",
                     "frac": round(h2d / (ms * 1e-3) / 1e9 / ceiling, 4),
                     "peak_kind": "measured: plain 1 GiB pinned-to-device copy (faster of one "
                                  "copy and two halves on two streams)"},
        "resident_same_histories": {"ms_per_step": round(ms_res, 3),
                                    "tokens_per_s": round(W.batch / (ms_res * 1e-3), 1),
                                    "value": round(kv / (ms_res * 1e-3) / 1e9, 1)},
    }


def merge_stress(args, ceiling):
    """The FP32 merge alone on the merge-stress shape: 64 requests x 24 heads
    x 256 partials of 256 channels, lse uniform in [-40, 40], 10 % of the
    partials empty (lse = -inf, output 0); seeded, generated on the device.
    Bytes per call: every partial output and lse read, out and lse written."""
    import torch
    from paged_kv_cache_10_amd import pkv
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pkv.lib()
    B, H, S, D = 64, 24, 256, 256
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    po = torch.randn((B, H, S, D), generator=g, device=dev)
    pl = torch.rand((B, H, S), generator=g, device=dev) * 80.0 - 40.0
    empty = torch.rand((B, H, S), generator=g, device=dev) < 0.1
    pl[empty] = float("-inf")
    po[empty] = 0.0
    out = torch.empty((B, H, D), device=dev)
    lse = torch.empty((B, H), device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pkv.merge_partials(po, pl, out, lse, stream=stream)
    K = max(args.steps, 20)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(K):
        pkv.merge_partials(po, pl, out, lse, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    nbytes = (po.numel() + pl.numel() + out.numel() + lse.numel()) * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "FP32 LSE merge GB/s on the merge-stress shape (64 x 24 x 256 partials)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "merge stress: 64 x 24 rows x 256 partials x 256 channels, lse "
                               "U[-40, 40], 10 % empty"},
        "bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "kernel": "merge_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5),
                     "traffic": merge_traffic()},
    }
    if ceiling is not None:
        res["read_ceiling"] = ceiling
    if args.copy_probe:
        res["copy_probe"] = copy_probe(dev, stream)
    return res


def merge_traffic():
    """Counter-derived HBM bytes of one merge-stress call, or None if they
    were not taken on this merge source."""
    t = PMC_TRAFFIC_MERGE
    if t["source_sha256"] is None or sources_sha256(MERGE_SOURCES) != t["source_sha256"]:
        return None
    return int(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])


def other_workloads(args):
    """The 4-request, mixed and merge-stress workloads, the live pool and the
    262K history staged from host memory (each exact and with compact
    pages), each measured by a child run of this script (its own process and
    device memory) with the same step counts: the key figures of each
    line."""
    import subprocess
    here = os.path.abspath(__file__)
    runs = {"conc": ["--workload", "conc"], "mixed": ["--workload", "mixed"],
            "merge_stress": ["--merge-stress"], "live": ["--live"],
            "live_compact": ["--live-compact"], "host_staged": ["--host-staged"],
            "host_staged_compact": ["--host-staged", "--compact-older"]}
    out = {}
    for name, extra in runs.items():
        cmd = [sys.executable, here, "--no-cpu-baseline", "--no-read-probe", "--no-others",
               "--steps", str(args.steps), "--warmup", str(args.warmup)] + extra
        p = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
        if p.returncode != 0 or not lines:
            out[name] = {"error": f"exit {p.returncode}: {p.stderr.strip()[-300:]}"}
            continue
        d = json.loads(lines[-1])
        r = d["roofline"]
        if r.get("bound") == "host-to-device":        # staged from host memory: the bus
            out[name] = {"workload": d["config"]["workload"], "ms_per_step": d["ms_per_step"],
                         "tokens_per_s": d["tokens_per_s"],
                         **{k: v for k, v in d.items() if k.endswith("_bitwise")},
                         "roofline": {k: r.get(k) for k in ("bound", "achieved", "peak", "unit",
                                                            "frac")}}
            continue
        out[name] = {"workload": d["config"]["workload"], "ms_per_step": d["ms_per_step"],
                     "value": d["value"], "unit": d["unit"],
                     "hbm_frac": round(d["value"] / HBM_PEAK_GBS, 4),
                     **({"tokens_per_s": d["tokens_per_s"]} if "tokens_per_s" in d else {}),
                     "roofline": {k: r.get(k) for k in ("kernel", "achieved", "frac",
                                                        "avg_launch_ms",
                                                        "algorithmic_bytes_per_launch",
                                                        "traffic")}}
    return out


def total_bytes_step(w, slots, split_slots=0):
    """Every byte one step moves, not only KV: per layer the KV history, q,
    the page-table entries read, the tile partials written (slots per row;
    and, where a tile has several splits, the split_slots split partials
    written and read back), the partials read by the merge, and out and lse
    written."""
    PT = w.page_tokens
    rows = w.batch * w.num_q_heads
    pages = sum(-(-c // PT) for c in w.ctx_lens)
    per_layer = (w.kv_bytes_per_step // w.num_layers
                 + rows * w.head_dim * 2                        # q (bf16)
                 + pages * 4                                    # page-table entries
                 + 2 * rows * slots * (w.head_dim + 1) * 4      # partials written, then read
                 + rows * (w.head_dim + 1) * 4)                 # out + lse
    per_layer += 2 * rows * split_slots * (w.head_dim + 1) * 4  # split partials, written and read
    return per_layer * w.num_layers


def append_probe(w, dev, stream):
    """pkv_append_kv, the step's new K/V rows into their pages, timed on a
    pool of its own (one page per request) so the history stays untouched:
    average time of one call for one layer over 200 calls."""
    import torch
    from paged_kv_cache_10_amd import pkv
    B, Hkv = w.batch, w.num_kv_heads
    arena = torch.zeros(B * w.page_layer_bytes // 2, dtype=torch.int16, device=dev)
    pool = pkv.Pool(arena, 1, Hkv, w.head_dim, w.page_tokens)
    table = torch.arange(B, dtype=torch.int32, device=dev).view(B, 1)
    pos = torch.full((B,), 5, dtype=torch.int32, device=dev)
    k = torch.randn((B, Hkv, w.head_dim), device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, w.head_dim), device=dev).to(torch.bfloat16)
    for _ in range(10):
        pkv.append_kv(pool, 0, table, pos, k, v, stream=stream)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(200):
        pkv.append_kv(pool, 0, table, pos, k, v, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / 200
    return {"us_per_layer": round(us, 2), "bytes_per_layer": B * Hkv * w.head_dim * 2 * 2}


def admission_probe(w, steps=200):
    """pkv_admit_step on the host: this workload's requests as contexts whose
    targets together exceed the pool, so every step reuses, reclaims and
    refuses; average host time of one planned step."""
    from paged_kv_cache_10_amd import pkv
    PT = w.page_tokens
    need = [-(-c // PT) for c in w.ctx_lens]
    pool_pages = max(2 * len(need), sum(need) * 3 // 4)          # 3/4 of what all would need
    a = pkv.Admission(pool_pages, PT)
    for i, n in enumerate(need):
        a.add(i, max(2, n * 2 // 3), burst=max(0, n // 3))
    lengths = list(w.ctx_lens)
    stride = max(need) + steps // PT + 2
    t0 = time.perf_counter()
    a.step(list(range(len(need))), lengths, stride)              # first fill of the pool
    fill_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    for k in range(1, steps + 1):
        active = [i for i in range(len(need)) if (i + k) % 3]   # a third idle each step
        a.step(active, [lengths[i] + k for i in active], stride)
    dt = time.perf_counter() - t0
    c = a.counts()
    a.close()
    return {"us_per_step": round(dt / steps * 1e6, 1), "first_fill_ms": round(fill_ms, 2),
            "contexts": len(need),
            "pool_pages": pool_pages, "counts": c,
            "note": "host time including the Python binding"}


def copy_probe(dev, stream):
    """A plain 1 GiB device-to-device copy (the kernel the PMC byte counters
    are calibrated on), timed over 10 runs."""
    import torch
    n = 1 << 29
    src = torch.empty(n, dtype=torch.int16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    cms = c0.elapsed_time(c1) / 10
    return {"bytes_read": n * 2, "bytes_written": n * 2, "ms": round(cms, 4),
            "GBs_read_plus_write": round(4 * n / (cms * 1e-3) / 1e9, 1)}


def compact_older(args, w, pool, table, ctx, qs, ref_outs, ref_lses):
    """Runs of two representations: each request's pages older than its
    newest exact_tail tokens are converted on the GPU into compact (E4M3)
    pages with their CRC and decoded from there; the tail stays exact; the
    two runs write disjoint slots and one FP32 merge combines them."""
    import torch
    from paged_kv_cache_10_amd import pkv
    dev = qs[0].device
    cl = COMPACT_LAUNCH[w.name]
    L, B, Hq, Hkv, D = w.num_layers, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    PT = w.page_tokens
    c = np.array([max(0, (n - cl["exact_tail"]) // PT * PT) for n in w.ctx_lens], np.int32)
    npc = c // PT
    P = int(npc.sum())
    cpb = pkv.compact_page_bytes(L, Hkv)
    carena = torch.zeros(P * cpb, dtype=torch.uint8, device=dev)
    cpool = pkv.Pool(carena, L, Hkv, compact=True)
    ids = np.random.default_rng(w.seed + 7).permutation(P).astype(np.int32)
    width = table.shape[1]
    ctab = np.full((B, width), -1, np.int32)
    etab = np.full((B, width), -1, np.int32)
    src, k = [], 0
    for b in range(B):
        ctab[b, :npc[b]] = ids[k:k + npc[b]]
        src.extend(table[b, :npc[b]].tolist())
        k += npc[b]
        rest = table[b, npc[b]:]
        rest = rest[rest >= 0]
        etab[b, :rest.size] = rest
    ectx = (ctx - c).astype(np.int32)
    dct, dcc = torch.empty((B, width), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev)
    det, dec = torch.empty((B, width), dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev)
    pkv.page_table_write(cpool, ctab, c, dct, dcc)
    pkv.page_table_write(pool, etab, ectx, det, dec)
    dsrc = torch.tensor(src, dtype=torch.int32, device=dev)
    ddst = torch.tensor(ids[:P], dtype=torch.int32, device=dev)
    crc = torch.empty(P, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pkv.compact_convert(pool, cpool, dsrc, ddst, crc)          # warm
    torch.cuda.synchronize()
    e0.record(stream)
    pkv.compact_convert(pool, cpool, dsrc, ddst, crc)
    e1.record(stream)
    torch.cuda.synchronize()
    convert_ms = e0.elapsed_time(e1)
    crc_host = crc.cpu().numpy().view(np.uint32)
    again = torch.empty_like(crc)
    pkv.compact_crc(cpool, ddst, again)
    torch.cuda.synchronize()
    crc_ok = bool(np.array_equal(crc_host, again.cpu().numpy().view(np.uint32)))

    T, S, Te, Se_ = cl["tile"], cl["split"], cl["exact_tile"], cl["exact_split"]
    if cl.get("schedule") == "one_launch" and (S != T or Se_ != Te):
        raise SystemExit("bench.py: the one-launch schedule runs one work-group per tile "
                         "(split = tile in both runs)")
    Sc = max(1, -(-int(c.max()) // T))
    Se = max(1, -(-int(ectx.max()) // Te))
    po = torch.empty((L, B, Hq, Sc + Se, D), device=dev)
    pl = torch.empty((L, B, Hq, Sc + Se), device=dev)
    outs = torch.empty_like(ref_outs)
    lses = torch.empty_like(ref_lses)
    nb = max(pkv.decode_workspace_bytes(B, Hq, Sc * T, T, D, 0, S),
             pkv.decode_workspace_bytes(B, Hq, Se * Te, Te, D, 0, Se_))
    ws = torch.zeros(max(16, nb) // 4 + 4, device=dev)

    ws2 = torch.zeros_like(ws)          # the tail's own workspace: the runs may overlap
    schedule = cl.get("schedule", "serial")
    side = torch.cuda.Stream() if schedule == "tail_stream" else None
    forks = [torch.cuda.Event() for _ in range(L)]
    joins = [torch.cuda.Event() for _ in range(L)]

    def runs_call(layer):
        pkv.decode_attention_runs(layer, qs[layer], [(cpool, dct, dcc, Sc * T, T, 0),
                                                     (pool, det, dec, Se * Te, Te, Sc)],
                                  w.scale, po[layer], pl[layer], stream=stream)

    def step(evs=None, pair=None, serial=False):
        """One 16-layer step.  evs: events around each compact launch; pair:
        events around each layer's two decode runs (fork to join)."""
        tail = stream if (serial or side is None) else side
        for layer in range(L):
            if pair is not None:
                pair[layer][0].record(stream)
            if schedule == "one_launch" and not serial and evs is None:
                runs_call(layer)
                if pair is not None:
                    pair[layer][1].record(stream)
                pkv.merge_partials(po[layer], pl[layer], outs[layer], lses[layer], stream=stream)
                continue
            if tail is not stream:
                forks[layer].record(stream)
                tail.wait_event(forks[layer])
            pkv.decode_attention(pool, layer, qs[layer], det, dec, 0, Se * Te, Te, w.scale,
                                 po[layer], pl[layer], workspace=ws2, split_tokens=Se_,
                                 slot_offset=Sc, stream=tail)
            if tail is not stream:
                joins[layer].record(tail)
            if evs is not None:
                evs[layer][0].record(stream)
            pkv.decode_attention(cpool, layer, qs[layer], dct, dcc, 0, Sc * T, T, w.scale,
                                 po[layer], pl[layer], workspace=ws, split_tokens=S, stream=stream)
            if evs is not None:
                evs[layer][1].record(stream)
            if tail is not stream:
                stream.wait_event(joins[layer])
            if pair is not None:
                pair[layer][1].record(stream)
            pkv.merge_partials(po[layer], pl[layer], outs[layer], lses[layer], stream=stream)

    def timed(**kw):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            step(**kw)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    def event_pass(kind, serial=False):
        """Mean ms between the two events a step records per layer: kind
        "evs" brackets the compact launch, "pair" the layer's two runs."""
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(args.steps)]
        for k in range(args.steps):
            step(serial=serial, **{kind: ev[k]})
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for evk in ev for (a, b) in evk]))

    for _ in range(args.warmup):
        step()
        step(serial=True)
    K = args.steps
    ms = timed()
    serial_ms = timed(serial=True)
    comp_ms = event_pass("evs", serial=True)   # the compact kernel alone on the GPU
    pair_ms = event_pass("pair")               # both runs of a layer, as timed
    # the compact run's own calls alone, back to back between one pair of events
    a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a0.record(stream)
    for _ in range(args.steps):
        for layer in range(L):
            pkv.decode_attention(cpool, layer, qs[layer], dct, dcc, 0, Sc * T, T, w.scale,
                                 po[layer], pl[layer], workspace=ws, split_tokens=S,
                                 stream=stream)
    b0.record(stream)
    torch.cuda.synchronize()
    comp_pairs_ms = comp_ms
    comp_ms = a0.elapsed_time(b0) / (args.steps * L)
    runs_b2b_ms = None
    if schedule == "one_launch":
        # the one-launch calls alone, back to back between one pair of events
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            for layer in range(L):
                runs_call(layer)
        b.record(stream)
        torch.cuda.synchronize()
        runs_b2b_ms = a.elapsed_time(b) / (args.steps * L)
    # one schedule's result must equal the other's bit for bit; the reported
    # result is the timed schedule's
    step(serial=True)
    torch.cuda.synchronize()
    serial_out, serial_lse = outs.clone(), lses.clone()
    step()
    torch.cuda.synchronize()
    same = bool(torch.equal(outs, serial_out) and torch.equal(lses, serial_lse))
    # the cost of the representation, against the exact path's own result
    d_out = (outs - ref_outs).abs()
    d_lse = (lses - ref_lses).abs()
    t = PMC_TRAFFIC_FP8
    fp8_traffic = None
    if ((w.name, T, S) == (t["workload"], t["tile"], t["split"])
            and sources_sha256(FP8_SOURCES) == t["source_sha256"]):
        fp8_traffic = int(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"])

    comp_bytes_layer = int(c.sum()) * 2 * Hkv * D + int(npc.sum()) * 2 * Hkv * 4
    exact_bytes_layer = int(ectx.sum()) * 2 * Hkv * D * 2
    moved = (comp_bytes_layer + exact_bytes_layer) * L
    if schedule == "one_launch":
        # the dominant kernel of the timed schedule: both runs in one launch,
        # timed by the events around each layer's decode_attention_runs call
        t = PMC_TRAFFIC_RUNS
        runs_traffic = None
        if ((w.name, T, Te) == (t["workload"], t["tile"], t["exact_tile"])
                and sources_sha256(RUNS_SOURCES) == t["source_sha256"]):
            runs_traffic = int(t["fetch_kib"] * 1024 * t["fetch_scale"]
                               + t["write_kib"] * 1024 * t["write_scale"])
        both = comp_bytes_layer + exact_bytes_layer
        roofline = {"bound": "hbm", "kernel": "decode_runs_kernel",
                    "launch": "one pkv_decode_attention_runs call per layer: the compact run "
                              "and the exact tail",
                    "achieved": round(both / (runs_b2b_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(both / (runs_b2b_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": both,
                    "avg_launch_ms": round(runs_b2b_ms, 5),
                    "timing": "HIP events on the decode stream around the layers' calls back "
                              "to back, K passes, divided by the calls",
                    "avg_launch_ms_event_pair_per_call": round(pair_ms, 5),
                    "traffic": runs_traffic}
    else:
        roofline = {"bound": "hbm", "kernel": "decode_fp8_kernel",
                    "achieved": round(comp_bytes_layer / (comp_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(comp_bytes_layer / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "algorithmic_bytes_per_launch": comp_bytes_layer,
                    "avg_launch_ms": round(comp_ms, 5), "traffic": fp8_traffic}
    kv = w.kv_bytes_per_step
    return {
        "metric": "decode attention KV GB/s (% of HBM peak) and tokens/s at 262K ctx, 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "value_kind": "exact-history bytes served per second (compact pages move fewer)",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: pages older than the newest {cl['exact_tail']} tokens "
                               f"served from compact E4M3 pages (per-block FP32 scale), the tail "
                               f"exact; compact run tile {T} split {S}, exact run tile {Te} "
                               f"split {Se_}" + {"one_launch": ", both runs in one launch",
                                                 "tail_stream": ", the tail on a second stream "
                                                                "concurrent with the compact run",
                                                 "serial": ", the runs one after the other"}[
                                                     schedule],
                   "compact_tokens": int(c.sum()), "exact_tokens": int(ectx.sum())},
        "tokens_per_s": round(B / (ms * 1e-3), 2),
        "bytes_moved_per_step": moved,
        "moved_GBs": round(moved / (ms * 1e-3) / 1e9, 1),
        "serial_ms_per_step": round(serial_ms, 4),
        "decode_runs_ms_per_layer": round(pair_ms, 5),
        "schedules_bitwise_equal": same,
        "bytes_per_token_layer": {"exact": 2 * Hkv * D * 2,
                                  "compact": round(comp_bytes_layer / max(1, int(c.sum())), 3)},
        "vs_exact_path": {"max_abs_out": round(float(d_out.max()), 5),
                          "mean_abs_out": round(float(d_out.mean()), 6),
                          "max_abs_lse": round(float(d_lse.max()), 5),
                          "mean_abs_lse": round(float(d_lse.mean()), 6),
                          "mean_abs_exact_out": round(float(ref_outs.abs().mean()), 5)},
        "convert": {"pages": P, "ms": round(convert_ms, 3),
                    "GBs_read": round(P * pool.page_bytes / (convert_ms * 1e-3) / 1e9, 1),
                    "crc_recomputed_equal": crc_ok},
        "roofline": roofline,
        "compact_kernel_alone": {
            "kernel": "decode_fp8_kernel", "schedule": "serial (the compact run's own launch)",
            "achieved": round(comp_bytes_layer / (comp_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(comp_bytes_layer / (comp_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": comp_bytes_layer,
            "avg_launch_ms": round(comp_ms, 5),
            "avg_launch_ms_event_pair_per_call": round(comp_pairs_ms, 5),
            "traffic": fp8_traffic},
    }


def host_staged_hybrid(args, w, pool, arena, table, ctx, qs, ref_outs, ref_lses, T, span):
    """The pages' hybrid tier: the whole history in pinned host memory, the
    windows older than the newest 32,768 tokens as compact pages (codes and
    scales, converted on the GPU from the exact pages, then copied to the
    host), the newest window exact; every layer staged window by window
    under leases from two stagers and decoded, one FP32 merge.  The bus
    carries 2,048.5 B per older token instead of 4,096."""
    import torch
    from paged_kv_cache_10_amd import pkv
    dev = arena.device
    L, B, Hq, Hkv, D, PT = (w.num_layers, w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                            w.page_tokens)
    window = 32768
    wpp = window // PT
    # compact boundary: whole windows older than the newest one
    c = np.array([max(0, (n - window) // window * window) for n in w.ctx_lens], np.int32)
    if len(set(c.tolist())) != 1:
        raise SystemExit("bench.py: --host-staged --compact-older needs one compact boundary for "
                         "every request (the single-request 262K workload)")
    npc = c // PT
    # exact host history, each history contiguous per layer (as the exact mode)
    npg = [-(-n // PT) for n in w.ctx_lens]
    bases = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int64)
    blk = w.page_layer_bytes // 2
    host = torch.empty((L, int(sum(npg)), blk), dtype=torch.int16, pin_memory=True)
    dev_slab = arena.view(L, -1, blk)
    for layer in range(L):
        for b, n in enumerate(npg):
            idx = torch.as_tensor(table[b, :n].astype(np.int64), device=dev)
            host[layer, bases[b]:bases[b] + n].copy_(dev_slab[layer].index_select(0, idx))
    host_table = np.full(table.shape, -1, dtype=np.int32)
    for b, n in enumerate(npg):
        host_table[b, :n] = bases[b] + np.arange(n)
    # compact pages of the older windows: converted on the GPU into a compact
    # pool whose page ids are contiguous per request, then copied to the host
    Pc = int(npc.sum())
    cpb = pkv.compact_page_bytes(L, Hkv)
    carena = torch.zeros(Pc * cpb, dtype=torch.uint8, device=dev)
    cpool = pkv.Pool(carena, L, Hkv, compact=True)
    cbase = np.concatenate([[0], np.cumsum(npc)[:-1]]).astype(np.int64)
    ctab = np.full(table.shape, -1, np.int32)
    src = []
    for b in range(B):
        ctab[b, :npc[b]] = cbase[b] + np.arange(npc[b])
        src.extend(table[b, :npc[b]].tolist())
    crc = torch.empty(max(1, Pc), dtype=torch.int32, device=dev)
    if Pc:
        pkv.compact_convert(pool, cpool, torch.tensor(src, dtype=torch.int32, device=dev),
                            torch.arange(Pc, dtype=torch.int32, device=dev), crc[:Pc])
    chost = torch.empty(carena.numel(), dtype=torch.uint8, pin_memory=True)
    chost.copy_(carena)
    torch.cuda.synchronize()
    # two stagers: compact windows and exact windows, two buffers each
    nbuf = args.buffers
    compute = torch.cuda.current_stream()
    copy_s, wb_s = torch.cuda.Stream(), torch.cuda.Stream()
    copy_c, wb_c = torch.cuda.Stream(), torch.cuda.Stream()
    st_arena = torch.empty(nbuf * B * wpp * w.page_layer_bytes // 2, dtype=torch.int16, device=dev)
    st_pool = pkv.Pool(st_arena, 1, Hkv)
    sc_arena = torch.zeros(nbuf * B * wpp * pkv.compact_page_bytes(1, Hkv), dtype=torch.uint8,
                           device=dev)
    sc_pool = pkv.Pool(sc_arena, 1, Hkv, compact=True)
    ex_stager = pkv.Stager(st_pool, host, L, B, window, nbuf, copy_s, compute, wb_s)
    c_stager = pkv.Stager(sc_pool, chost, L, B, window, nbuf, copy_c, compute, wb_c)
    wspan = -(-span // window) * window
    po = torch.empty((B, Hq, wspan // T, D), device=dev)
    pl = torch.empty((B, Hq, wspan // T), device=dev)
    slots = span // T
    outs = torch.empty_like(ref_outs)
    lses = torch.empty_like(ref_lses)
    dc = torch.tensor(ctx, dtype=torch.int32, device=dev)
    dcc = torch.tensor(c, dtype=torch.int32, device=dev)
    nb = pkv.decode_workspace_bytes(B, Hq, window, T, D, args.kernel, args.split)
    ws = torch.zeros(max(16, nb) // 4 + 4, device=dev)
    cmax = int(c.max())

    def step(resident=False):
        for layer in range(L):
            for begin in range(0, wspan, window):
                compact = begin < cmax
                if resident:
                    pool_, tab, dctx = ((cpool, torch.as_tensor(ctab[:, begin // PT:], device=dev).contiguous(), dcc)
                                        if compact else (pool, torch.as_tensor(table[:, begin // PT:], device=dev).contiguous(), dc))
                    pkv.decode_attention(pool_, layer, qs[layer], tab, dctx, begin, window, T,
                                         w.scale, po, pl, workspace=ws, split_tokens=args.split,
                                         stream=compute)
                    continue
                stg, spool, htab, hctx, dctx = ((c_stager, sc_pool, ctab, c, dcc) if compact
                                                else (ex_stager, st_pool, host_table, ctx, dc))
                lease = stg.begin(layer, htab, hctx, begin)
                pkv.decode_attention(spool, lease.staging_layer, qs[layer], stg.table(lease), dctx,
                                     begin, window, T, w.scale, po, pl, workspace=ws,
                                     split_tokens=args.split, stream=compute)
                stg.seal(lease)
            pkv.merge_partials(po[:, :, :slots].contiguous(), pl[:, :, :slots].contiguous(),
                               outs[layer], lses[layer], stream=compute)

    # the resident two-run decode at the same tiling, for the bitwise check
    step(resident=True)
    torch.cuda.synchronize()
    ref_o, ref_l = outs.clone(), lses.clone()
    step()
    ex_stager.retire()
    c_stager.retire()
    ok = bool(torch.equal(outs.view(torch.int32), ref_o.view(torch.int32))
              and torch.equal(lses.view(torch.int32), ref_l.view(torch.int32)))
    d_out = float((outs - ref_outs).abs().max())
    d_lse = float((lses - ref_lses).abs().max())
    K = max(1, min(args.steps, 5))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(compute)
    for _ in range(K):
        step()
    e1.record(compute)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    receipts = ex_stager.retire() + c_stager.retire()
    ex_stager.destroy()
    c_stager.destroy()
    # host-to-device ceiling, as the exact mode measures it
    src_h = host.view(-1)[: 1 << 29]
    dst = torch.empty(src_h.shape, dtype=torch.int16, device=dev)
    dst.copy_(src_h, non_blocking=True)
    torch.cuda.synchronize()
    h = src_h.numel() // 2
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(compute)
    copy_s.wait_event(c0)
    for _ in range(3):
        dst[:h].copy_(src_h[:h], non_blocking=True)
        with torch.cuda.stream(copy_s):
            dst[h:].copy_(src_h[h:], non_blocking=True)
    done = torch.cuda.Event()
    done.record(copy_s)
    compute.wait_event(done)
    c1.record(compute)
    torch.cuda.synchronize()
    h2d = 3 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    sb = 2 * Hkv * 4
    moved = 0
    for b, n in enumerate(w.ctx_lens):
        moved += int(npc[b]) * (w.page_layer_bytes // 2 + sb)                 # compact pages
        moved += (-(-n // PT) - int(npc[b])) * w.page_layer_bytes             # exact pages
    moved *= L
    kv = w.kv_bytes_per_step
    return {
        "metric": "decode attention KV GB/s (% of HBM peak) and tokens/s at 262K ctx, 1 GPU",
        "value": round(kv / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
        "value_kind": "exact-history bytes served per second; the bus moves fewer",
        "n_gpus": 1, "steps": K, "warmup": 1, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16+e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: history in pinned host memory, windows older than the "
                               f"newest {window} tokens as compact E4M3 pages, the newest exact; "
                               f"staged per window under leases ({nbuf} buffers per stager), "
                               f"tile {T}", "tile_tokens": T, "split_tokens": args.split,
                   "compact_tokens": int(c.sum())},
        "tokens_per_s": round(B / (ms * 1e-3), 3),
        "bus_bytes_per_step": moved,
        "staged_equals_resident_two_runs_bitwise": ok,
        "vs_exact_path": {"max_abs_out": round(d_out, 5), "max_abs_lse": round(d_lse, 5)},
        "leases_per_step": L * (wspan // window), "receipts": receipts,
        "roofline": {"bound": "host-to-device", "achieved": round(moved / (ms * 1e-3) / 1e9, 2),
                     "peak": round(h2d, 2), "unit": "GB/s",
                     "frac": round(moved / (ms * 1e-3) / 1e9 / h2d, 4),
                     "peak_kind": "measured: 1 GiB pinned-to-device copy as two halves on two "
                                  "streams"},
    }


def read_probe():
    """Measured HBM read ceiling: probe_read, run as a child process before
    this process touches the GPU; None if the probe is not built."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_10_amd",
                       "probe_read")
    if not os.path.exists(exe):
        return None
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, check=True).stdout
    return json.loads(out.strip().splitlines()[-1])


def cpu_baseline(w, qs, budget_s):
    """The float64 oracle on this host's cores, on a bounded sample: whole
    layers of the same workload (all requests, all heads, one-pass exact
    attention), as many as fit the budget; scaled to tokens/s per step."""
    import torch
    import oracle
    from paged_kv_cache_10_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    spent = 0.0
    layers = 0
    for layer in range(w.num_layers):
        qb = qs[layer].view(torch.int16).cpu().numpy().view(np.uint16)
        kv = []
        for b in range(w.batch):
            k, v = I.device_kv(w, layer, b, "cuda:0")
            kv.append((k.view(torch.int16).cpu().numpy().view(np.uint16),
                       v.view(torch.int16).cpu().numpy().view(np.uint16)))
            del k, v
        t = time.time()
        for b in range(w.batch):
            oracle.decode_one_pass(oracle.widen_bf16(qb[b]), oracle.widen_bf16(kv[b][0]),
                                   oracle.widen_bf16(kv[b][1]), w.ctx_lens[b], w.scale,
                                   w.num_kv_heads)
        spent += time.time() - t
        layers += 1
        del kv
        if spent >= budget_s:
            break
    s_per_step = spent / layers * w.num_layers
    return {
        "value": round(w.batch / s_per_step, 4),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{layers} of {w.num_layers} layers of the same workload (all "
                  f"{w.batch} request(s), all heads, float64 one-pass), scaled x{w.num_layers / layers:.1f}",
        "seconds": round(spent, 2),
        "kv_GBs_equiv": round(w.kv_bytes_per_step / s_per_step / 1e9, 3),
        "cpu_model": cpu_model(),
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    sys.exit(main())
