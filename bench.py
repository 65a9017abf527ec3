"""Benchmark of the paged <-> Full Block KV-move path on one MI355X.

One step = the layerwise loop of the Llama-3-8B-like workload (L=32, H_kv=8,
d=128, bf16, B=16; 8 requests of T_hit=32768 hit and T_miss=512 miss tokens;
24576-block pool, shuffled block tables): for every layer l, unpack_layer(l)
of the hit slice into the paged slots, then merge_layer(l) of hit || miss into
each request's complete_layer[l]; then pack_full of all T_all tokens of every
request. All inputs are resident in HBM before timing.

value = algorithmic bytes (read + write) of one step / step time, whole job.
Also reported: each op's average launch time from HIP events on the launch
stream, the roofline of the dominant kernel, the same step with unpack and
merge fused per layer (kvm_unpack_merge_layer), the host tier (a pinned host
Full Block / complete_layer over PCIe), the layerwise overlap of the moves
with a stand-in compute stream under workgroup budgets, two plain device
copies (reference rates), the MLA agentic layer loop (61 layers, 576-element
latent, 64 requests), the small-object batched copy (200000 objects of
256*U{16..512} bytes), the 256,000-object restore list, the per-call cost of
small calls, and the oracle timed on the host cores on one request of the
same workload. The layer loop, the MLA loop, the small-object copy and the
restore list each carry a roofline entry for their dominant kernel.

Inputs are seeded: --seed S (default 1002) draws the layer loop from S, the
restore list from S+1, the MLA loop from S+2 and the small-object list from
S+3 (the defaults are the workloads' own seeds).

--verify checks, after each timed section and outside its timing, every
output of the layer loop, the MLA loop and the two copy lists on the device
against the operations' definitions (no oracle: plain torch indexing).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--seed S] [--verify]
                      [--config c3,c4,c5] [--reps R] [--no-cpu] [--no-batch-copy]
                      [--no-host] [--no-pipeline] [--no-mla] [--no-restore] [--no-small]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PCIE_PEAK_GBS = 63.0   # PCIe 5.0 x16 host link, per direction


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=1002,
                    help="base seed of the synthetic inputs (layer loop S, restore list S+1, "
                         "MLA loop S+2, small objects S+3)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-batch-copy", action="store_true", help="skip the batched-copy section")
    ap.add_argument("--no-host", action="store_true", help="skip the pinned-host-buffer section")
    ap.add_argument("--no-mla", action="store_true", help="skip the MLA agentic layer loop")
    ap.add_argument("--no-restore", action="store_true",
                    help="skip the 256,000-object restore list")
    ap.add_argument("--no-small", action="store_true", help="skip the small-call section")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the layerwise overlap section (workgroup-bounded moves)")
    ap.add_argument("--config", default="c3,c4,c5",
                    help="comma list of the other workloads to run after the layer loop (C2, "
                         "always run): c3 the restore list, c4 the MLA loop, c5 the small-object "
                         "copy; 'none' for the layer loop alone")
    ap.add_argument("--reps", type=int, default=0,
                    help="timed repetitions of each copy list and of the MLA loops "
                         "(0: 10 per copy list, 5 per MLA loop)")
    ap.add_argument("--verify", action="store_true",
                    help="after each timed section, check its outputs on the device against the "
                         "operations' defining properties (untimed; exits 1 on a mismatch)")
    args = ap.parse_args()
    cfg = {c.strip().lower() for c in args.config.split(",") if c.strip()} - {"none"}
    unknown = cfg - {"c3", "c4", "c5"}
    if unknown:
        ap.error(f"--config: unknown workload(s) {sorted(unknown)}; choose from c3, c4, c5")
    args.no_restore |= "c3" not in cfg
    args.no_mla |= "c4" not in cfg
    args.no_batch_copy |= "c5" not in cfg
    if args.reps < 0:
        ap.error("--reps must be >= 0")
    return args


class Events:
    """Per-op launch timing with HIP events on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def around(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))

    def all_ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs[name]]

    def mean_ms(self, name):
        return statistics.fmean(self.all_ms(name))


def quantile(xs, q):
    """Linear-interpolated quantile of a non-empty list."""
    xs = sorted(xs)
    pos = q * (len(xs) - 1)
    lo = int(pos)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (pos - lo)


class VerifyError(RuntimeError):
    pass


def expect(ok, what):
    if not bool(ok):
        raise VerifyError(what)


def verify_layer_loop(torch, s):
    """The layer loop's outputs on the device, by the operations' definitions:
    complete_layer[r][l] is the hit slice of layer l then its miss rows; the
    slot row of every hit token t holds full[r][t][l]; and packed[r][t][l][s]
    is the pool row pool[l][s][bt[t / B]][t % B] for every token (pack after the
    loop)."""
    bts, fbs, misses, complete, packed = s["keep"]
    sh = s["w"].shape
    L, S, B, rb, N, C = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, s["w"].pool_blocks, s["C"]
    th, tm = s["w"].t_hit[0], s["w"].t_miss[0]
    ta = th + tm
    pv = s["pool"].view(L, S, N, B, rb)
    for r in range(len(fbs)):
        fb, ms = fbs[r].view(th, L, C), misses[r].view(tm, L, C)
        cm = complete[r * L * ta * C:(r + 1) * L * ta * C].view(L, ta, C)
        for l in range(L):
            expect(torch.equal(cm[l, :th], fb[:, l]), f"complete_layer hit rows, request {r} layer {l}")
            expect(torch.equal(cm[l, th:], ms[:, l]), f"complete_layer miss rows, request {r} layer {l}")
        pk, bt = packed[r].view(ta, L, S, rb), bts[r].long()
        for t0 in range(0, ta, 4096):
            t = torch.arange(t0, min(ta, t0 + 4096), device=pv.device)
            rows = pv[:, :, bt[t // B], t % B].permute(2, 0, 1, 3)      # [tokens][L][S][rb]
            expect(torch.equal(pk[t0:t0 + len(t)], rows), f"pack_full request {r} tokens from {t0}")
            h = int((t < th).sum().item())
            if h:
                expect(torch.equal(rows[:h], fbs[r].view(th, L, S, rb)[t0:t0 + h]),
                       f"unpack_layer slot rows, request {r} tokens from {t0}")
            del rows


def verify_copies(torch, src, dst, descs_np, granule=256, batch=4096):
    """Every object of a copy list: dst[dst_off, +n) == src[src_off, +n), on the
    device. Offsets are multiples of `granule`, so each length is compared
    through strided windows of the two buffers."""
    import numpy as np
    d = torch.from_numpy(descs_np.astype(np.int64)).to(src.device)
    expect(bool(((d[:, 0] % granule) == 0).all()) and bool(((d[:, 1] % granule) == 0).all()),
           "offsets are whole granules")
    for n in np.unique(descs_np[:, 2]):
        n = int(n)
        sel = d[d[:, 2] == n]
        ws, wd = src.unfold(0, n, granule), dst.unfold(0, n, granule)
        for a in range(0, len(sel), batch):
            part = sel[a:a + batch]
            expect(torch.equal(wd[part[:, 1] // granule], ws[part[:, 0] // granule]),
                   f"an object of {n} bytes differs")


def llama_setup(torch, kv, wl, dev, seed):
    import dataclasses
    w = dataclasses.replace(wl.LLAMA8B, seed=seed)
    sh = w.shape
    L, S, B, rb, N = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, w.pool_blocks
    C = sh.c_kv_bytes
    R = len(w.t_hit)
    t_hit, t_miss = w.t_hit[0], w.t_miss[0]
    t_all = t_hit + t_miss
    pool_bytes = L * S * N * B * rb
    fb_bytes = t_hit * L * C
    need = pool_bytes + R * (fb_bytes + t_miss * L * C + 2 * t_all * L * C)
    free, _ = torch.cuda.mem_get_info(dev)
    log(f"[bench] {w.name}: allocating {need / 2**30:.1f} GiB of {free / 2**30:.1f} GiB free")
    if need > free:
        raise SystemExit(f"workload needs {need} bytes, {free} free")
    u8 = dict(dtype=torch.uint8, device=dev)
    pool = torch.empty(pool_bytes, **u8)
    wl.fill_bf16_normal_(pool, w.seed, 1)
    tables = wl.block_tables(w.seed, 2, N, [wl.blocks_needed(t_all, B)] * R)
    bts = [torch.from_numpy(t).to(dev) for t in tables]
    fbs = [torch.empty(fb_bytes, **u8) for _ in range(R)]
    misses = [torch.empty(t_miss * L * C, **u8) for _ in range(R)]
    for r in range(R):
        wl.fill_bf16_normal_(fbs[r], w.seed, 10 + r)
        wl.fill_bf16_normal_(misses[r], w.seed, 30 + r)
    complete = torch.empty(R * L * t_all * C, **u8)      # [R][L][T_all][C]
    packed = [torch.empty(t_all * L * C, **u8) for _ in range(R)]
    torch.cuda.synchronize()
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    unpack_seqs = [kv.seq(bts[r], fbs[r], t_hit) for r in range(R)]
    pack_seqs = [kv.seq(bts[r], packed[r], t_all) for r in range(R)]
    merge_by_layer = []
    for l in range(L):
        merge_by_layer.append([
            kv.merge_seq(fbs[r].data_ptr() + l * C, L * C, t_hit,
                         misses[r].data_ptr() + l * C, L * C, t_miss,
                         complete.data_ptr() + (r * L + l) * t_all * C, C)
            for r in range(R)])
    fused_by_layer = []
    for l in range(L):
        fused_by_layer.append([
            kv.layer_seq(bts[r], fbs[r], t_hit, misses[r].data_ptr() + l * C, L * C, t_miss,
                         complete.data_ptr() + (r * L + l) * t_all * C, C)
            for r in range(R)])
    bytes_unpack = 2 * R * t_hit * C
    bytes_merge = 2 * R * t_all * C
    bytes_pack = 2 * R * t_all * L * C
    # fused layer: read hit + miss once, write the pool slots and complete_layer
    bytes_fused = R * C * (3 * t_hit + 2 * t_miss)
    return dict(w=w, L=L, layout=layout, pool=pool, unpack_seqs=unpack_seqs, pack_seqs=pack_seqs,
                merge_by_layer=merge_by_layer, fused_by_layer=fused_by_layer, bytes_fused=bytes_fused,
                C=C, keep=(bts, fbs, misses, complete, packed),
                bytes=dict(unpack_layer=bytes_unpack, merge_layer=bytes_merge,
                           pack_full=bytes_pack),
                launches=dict(unpack_layer=L, merge_layer=L, pack_full=1))


def llama_step(kv, ctx, s):
    L = s["L"]
    for l in range(L):
        kv.kvm_unpack_layer(ctx.handle, s["layout"], s["pool"], L, l, s["unpack_seqs"])
        kv.kvm_merge_layer(ctx.handle, s["C"], s["merge_by_layer"][l])
    kv.kvm_pack_full(ctx.handle, s["layout"], s["pool"], L, s["pack_seqs"])


def llama_fused_step(kv, ctx, s):
    L = s["L"]
    for l in range(L):
        kv.kvm_unpack_merge_layer(ctx.handle, s["layout"], s["pool"], L, l, s["fused_by_layer"][l])
    kv.kvm_pack_full(ctx.handle, s["layout"], s["pool"], L, s["pack_seqs"])


def fused_section(torch, kv, ctx, s, steps, warmup, ms_separate):
    """The same step with unpack_layer + merge_layer fused per layer."""
    for _ in range(warmup):
        llama_fused_step(kv, ctx, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        llama_fused_step(kv, ctx, s)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = Events(torch)
    L = s["L"]
    for _ in range(max(3, steps // 2)):
        ev.around("fused", lambda: [kv.kvm_unpack_merge_layer(
            ctx.handle, s["layout"], s["pool"], L, l, s["fused_by_layer"][l]) for l in range(L)])
    torch.cuda.synchronize()
    per = ev.mean_ms("fused") / L
    gbs = s["bytes_fused"] / (per * 1e6)
    # the fused step's own algorithmic bytes: it reads each hit row once
    fused_step_bytes = L * s["bytes_fused"] + s["bytes"]["pack_full"]
    return {"step": "32 x unpack_merge_layer + pack_full", "ms_per_step": round(ms, 3),
            "speedup_vs_separate": round(ms_separate / ms, 3),
            "bytes_per_step": fused_step_bytes,
            "GBps": round(fused_step_bytes / (ms * 1e6), 1),
            "pct_hbm_peak": round(100 * fused_step_bytes / (ms * 1e6) / HBM_PEAK_GBS, 2),
            "unpack_merge_layer": {"bytes_per_launch": s["bytes_fused"],
                                   "ms_per_launch": round(per, 4), "GBps": round(gbs, 1),
                                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}}


def host_tier_section(torch, kv, ctx, s, reps=3):
    """The pages' host-DRAM prompt buffers: request 0's Full Block in pinned host
    memory. Per layer: unpack_layer reads its hit slice over PCIe into the HBM
    pool (Prefill side); merge_layer writes complete_layer into a pinned host
    buffer (Decode side, hit rows from HBM); pack_full writes the request's whole
    Full Block (all T_all tokens) into pinned host memory (persisting it). Rates
    are PCIe bytes per second, next to torch's pinned host<->device copy rates
    and the PCIe 5.0 x16 peak (63 GB/s per direction)."""
    L, C = s["L"], s["C"]
    bts, fbs, misses, _, _ = s["keep"]
    t_hit, t_miss = 32768, 512
    t_all = t_hit + t_miss
    host_fb = torch.empty(fbs[0].numel(), dtype=torch.uint8, pin_memory=True)
    host_fb.copy_(fbs[0])
    host_out = torch.empty(t_all * C, dtype=torch.uint8, pin_memory=True)
    host_packed = torch.empty(t_all * L * C, dtype=torch.uint8, pin_memory=True)
    dev_buf = torch.empty(1 << 30, dtype=torch.uint8, device=fbs[0].device)
    host_buf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    seqs = [kv.seq(bts[0], host_fb, t_hit)]
    ev = Events(torch)

    def unpack_loop():
        for l in range(L):
            kv.kvm_unpack_layer(ctx.handle, s["layout"], s["pool"], L, l, seqs)

    def merge_loop():
        for l in range(L):
            kv.kvm_merge_layer(ctx.handle, C, [kv.merge_seq(
                fbs[0].data_ptr() + l * C, L * C, t_hit, misses[0].data_ptr() + l * C, L * C,
                t_miss, host_out, C)])

    def pack_host():
        kv.kvm_pack_full(ctx.handle, s["layout"], s["pool"], L, [kv.seq(bts[0], host_packed, t_all)])

    # one layer of a restore from a host-DRAM staging buffer: 4,000 K/V objects
    # of 128 KiB packed in pinned host memory, copied by kvm_batch_copy into
    # 4,000 shuffled 128 KiB slots of a device buffer (the restore list's
    # per-layer call, from host memory)
    import numpy as np
    nobj, obj = 4000, 128 << 10
    host_stage = torch.empty(nobj * obj, dtype=torch.uint8, pin_memory=True)
    dev_slots = torch.empty(nobj * obj, dtype=torch.uint8, device=fbs[0].device)
    perm = np.random.default_rng(1234).permutation(nobj).astype(np.uint64)
    d = np.stack([np.arange(nobj, dtype=np.uint64) * obj, perm * obj,
                  np.full(nobj, obj, np.uint64)], axis=1)
    host_descs = torch.from_numpy(d.view(np.uint8).reshape(-1)).to(fbs[0].device)

    def restore_from_host():
        kv.kvm_batch_copy(ctx.handle, dev_slots, nobj * obj, host_stage, nobj * obj,
                          host_descs, nobj)

    unpack_loop()
    merge_loop()
    pack_host()
    restore_from_host()
    for _ in range(reps):
        ev.around("h2d_unpack", unpack_loop)
        ev.around("d2h_merge", merge_loop)
        ev.around("d2h_pack", pack_host)
        ev.around("h2d_restore", restore_from_host)
        ev.around("h2d_copy", lambda: dev_buf.copy_(host_buf, non_blocking=True))
        ev.around("d2h_copy", lambda: host_buf.copy_(dev_buf, non_blocking=True))
    torch.cuda.synchronize()
    up_gbs = L * t_hit * C / (ev.mean_ms("h2d_unpack") * 1e6)
    mg_gbs = L * t_all * C / (ev.mean_ms("d2h_merge") * 1e6)
    h2d = (1 << 30) / (ev.mean_ms("h2d_copy") * 1e6)
    d2h = (1 << 30) / (ev.mean_ms("d2h_copy") * 1e6)
    pk_gbs = t_all * L * C / (ev.mean_ms("d2h_pack") * 1e6)
    rs_gbs = nobj * obj / (ev.mean_ms("h2d_restore") * 1e6)
    del host_fb, host_out, host_packed, dev_buf, host_buf, host_stage, dev_slots, host_descs
    return {"workload": "request 0 of the layer loop, Full Block / complete_layer in pinned host memory",
            "unpack_layer_from_host": {"pcie_bytes_per_launch": t_hit * C,
                                       "ms_per_launch": round(ev.mean_ms("h2d_unpack") / L, 3),
                                       "pcie_GBps": round(up_gbs, 1),
                                       "frac_of_h2d_copy": round(up_gbs / h2d, 3),
                                       "frac_of_pcie_peak": round(up_gbs / PCIE_PEAK_GBS, 3)},
            "merge_layer_into_host": {"pcie_bytes_per_launch": t_all * C,
                                      "ms_per_launch": round(ev.mean_ms("d2h_merge") / L, 3),
                                      "pcie_GBps": round(mg_gbs, 1),
                                      "frac_of_d2h_copy": round(mg_gbs / d2h, 3),
                                      "frac_of_pcie_peak": round(mg_gbs / PCIE_PEAK_GBS, 3)},
            "pack_full_into_host": {"pcie_bytes_per_launch": t_all * L * C,
                                    "ms_per_launch": round(ev.mean_ms("d2h_pack"), 3),
                                    "pcie_GBps": round(pk_gbs, 1),
                                    "frac_of_d2h_copy": round(pk_gbs / d2h, 3),
                                    "frac_of_pcie_peak": round(pk_gbs / PCIE_PEAK_GBS, 3)},
            "batch_copy_restore_layer_from_host": {"objects": nobj, "object_bytes": obj,
                                                   "pcie_bytes_per_call": nobj * obj,
                                                   "ms_per_call": round(ev.mean_ms("h2d_restore"), 3),
                                                   "pcie_GBps": round(rs_gbs, 1),
                                                   "frac_of_h2d_copy": round(rs_gbs / h2d, 3),
                                                   "frac_of_pcie_peak": round(rs_gbs / PCIE_PEAK_GBS, 3)},
            "torch_pinned_copy_GBps": {"h2d": round(h2d, 1), "d2h": round(d2h, 1)},
            "pcie_peak_GBps_per_direction": PCIE_PEAK_GBS}


def pipeline_section(torch, kv, ctx, s, reps=3, d_model=4096, d_ff=14336):
    """Layerwise overlap of the KV moves with compute, the moves bounded to a
    workgroup budget (kvm_ctx_set_max_workgroups).

    (1) The fused layer loop (L x unpack_merge_layer) alone at budgets k: how
    many workgroups the moves need to reach HBM speed. (2) A stand-in for each
    layer's compute, the MLP GEMMs of the step's miss tokens (R * T_miss rows,
    bf16, d_model -> 2*d_ff -> d_model, random weights), on a second stream,
    while the moves run ahead on the first: layer l's compute waits for layer
    l's moves, and layer l's moves wait for layer l-d's compute (d layer
    buffers, d = 2 and 4), or nothing waits. Timed against the same work run
    back to back on one stream."""
    L = s["L"]
    layers = s["fused_by_layer"]
    rows = sum(t for t in s["w"].t_miss)
    st_kv, st_cmp = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(rows, d_model, device="cuda", dtype=torch.bfloat16, generator=g)
    w_up = torch.randn(d_model, 2 * d_ff, device="cuda", dtype=torch.bfloat16, generator=g)
    w_down = torch.randn(d_ff, d_model, device="cuda", dtype=torch.bfloat16, generator=g)
    h = torch.empty(rows, 2 * d_ff, device="cuda", dtype=torch.bfloat16)
    y = torch.empty(rows, d_model, device="cuda", dtype=torch.bfloat16)
    flops_layer = 2 * rows * d_model * 2 * d_ff + 2 * rows * d_ff * d_model

    def moves(l, st=None):
        kv.kvm_unpack_merge_layer(ctx.handle, s["layout"], s["pool"], L, l, layers[l], stream=st)

    def compute():
        torch.mm(x, w_up, out=h)
        torch.mm(h[:, :d_ff], w_down, out=y)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) * 1e3
            best = dt if best is None else min(best, dt)
        return best

    def serial():
        for l in range(L):
            moves(l)
            compute()

    def overlapped(depth):
        # `depth` layer buffers: layer l's moves wait until layer l-depth's
        # compute is done, layer l's compute waits for its moves
        ready = [torch.cuda.Event() for _ in range(L)]
        done = [torch.cuda.Event() for _ in range(L)]
        st_kv.wait_stream(torch.cuda.current_stream())
        st_cmp.wait_stream(torch.cuda.current_stream())
        for l in range(L):
            if l >= depth:
                st_kv.wait_event(done[l - depth])
            moves(l, st_kv)
            ready[l].record(st_kv)
            with torch.cuda.stream(st_cmp):
                st_cmp.wait_event(ready[l])
                compute()
                done[l].record(st_cmp)
        torch.cuda.current_stream().wait_stream(st_cmp)
        torch.cuda.current_stream().wait_stream(st_kv)

    def compute_all():
        for _ in range(L):
            compute()

    def concurrent():
        # no dependencies: every layer's moves on one stream, every layer's
        # compute on the other (the most overlap the two streams can give)
        st_kv.wait_stream(torch.cuda.current_stream())
        st_cmp.wait_stream(torch.cuda.current_stream())
        for l in range(L):
            moves(l, st_kv)
        with torch.cuda.stream(st_cmp):
            compute_all()
        torch.cuda.current_stream().wait_stream(st_cmp)
        torch.cuda.current_stream().wait_stream(st_kv)

    try:
        curve = {}
        for k in (16, 32, 64, 128, 256, 512, 1024, 0):
            ctx.set_max_workgroups(k)
            ms = timed(lambda: [moves(l) for l in range(L)])
            curve[str(k) if k else "unbounded"] = round(L * s["bytes_fused"] / (ms * 1e6), 1)
        ctx.set_max_workgroups(0)
        t_moves = timed(lambda: [moves(l) for l in range(L)])
        t_comp = timed(compute_all)
        t_serial = timed(serial)
        over = {}
        for k in (64, 128, 256, 0):
            ctx.set_max_workgroups(k)
            row = {f"ms_{d}_layer_buffers": round(timed(lambda: overlapped(d)), 3)
                   for d in (2, 4)}
            row["ms_no_dependencies"] = round(timed(concurrent), 3)
            row["best_speedup_vs_back_to_back"] = round(t_serial / min(row.values()), 3)
            over[str(k) if k else "unbounded"] = row
    finally:
        ctx.set_max_workgroups(0)
        torch.cuda.synchronize()
    return {"moves_GBps_by_workgroup_budget": curve,
            "stand_in_compute": f"per layer: bf16 GEMMs {rows}x{d_model}x{2 * d_ff} and "
                                f"{rows}x{d_ff}x{d_model} (MLP of the miss tokens)",
            "compute_TFLOPs": round(L * flops_layer / (t_comp * 1e9), 1),
            "ms_moves_alone": round(t_moves, 3), "ms_compute_alone": round(t_comp, 3),
            "ms_back_to_back": round(t_serial, 3),
            "overlapped_by_workgroup_budget": over}


def plain_copies(torch, kv, ctx, dev, nbytes=2 << 30, reps=10):
    """Two device-to-device copies of nbytes, read+write GB/s: torch's copy
    (the runtime's blit kernel), and this library's batched copy of one
    nbytes object."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    desc = torch.tensor([0, 0, nbytes], dtype=torch.int64, device=dev)

    def rate(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 2 * nbytes / (e0.elapsed_time(e1) / reps * 1e6)

    torch_copy = rate(lambda: b.copy_(a))
    stream_copy = rate(lambda: kv.kvm_batch_copy(ctx.handle, b, nbytes, a, nbytes, desc, 1))
    assert ctx.take_device_errors() == 0
    del a, b
    return torch_copy, stream_copy


def batch_copy_section(torch, kv, wl, ctx, dev, seed, reps=10, verify=False):
    import dataclasses
    w = dataclasses.replace(wl.SMALL_OBJS, seed=seed)
    descs_np = wl.small_object_descs(w)
    total = int(descs_np[:, 2].sum())
    log(f"[bench] {w.name}: {len(descs_np)} objects, {total / 1e9:.2f} GB each way")
    u8 = dict(dtype=torch.uint8, device=dev)
    src = torch.empty(w.src_arena, **u8)
    wl.fill_random_bytes_(src, w.seed, 1)
    dst = torch.empty(w.dst_arena, **u8)
    descs = torch.from_numpy(descs_np.view(__import__("numpy").uint8).reshape(-1)).to(dev)
    ctx.reserve(64, len(descs_np))
    for _ in range(2):
        kv.kvm_batch_copy(ctx.handle, dst, w.dst_arena, src, w.src_arena, descs, len(descs_np))
    torch.cuda.synchronize()
    ev = Events(torch)
    for _ in range(reps):
        ev.around("batch_copy", lambda: kv.kvm_batch_copy(ctx.handle, dst, w.dst_arena, src,
                                                          w.src_arena, descs, len(descs_np)))
    torch.cuda.synchronize()
    ms = ev.mean_ms("batch_copy")
    spread = [round(quantile(ev.all_ms("batch_copy"), q), 4) for q in (0.1, 0.5, 0.9)]
    gbs = 2 * total / (ms * 1e6)
    if verify:
        verify_copies(torch, src, dst, descs_np)
    del src, dst, descs
    torch.cuda.empty_cache()
    return {"workload": w.name, "objects": len(descs_np), "bytes_rw": 2 * total,
            "ms_per_call": round(ms, 4), "ms_p10_p50_p90": spread, "repetitions": reps,
            "GBps": round(gbs, 1),
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "descriptors_per_s": round(len(descs_np) / (ms * 1e-3), 0),
            "roofline": roofline("k_bc_copy", "batch_copy (200000 small objects)", 2 * total, ms,
                                 "one call: HIP events around its metadata launches (k_bc_sums, "
                                 "k_bc_scan2, k_bc_map) and its k_bc_copy launch")}


def mla_section(torch, kv, wl, ctx, dev, seed, reps=5, verify=False):
    """The MLA agentic layer loop (64 requests, T_hit ~ U{16384..65536},
    T_miss ~ U{128..1024}, 61 layers of one 576-element bf16 latent, B=64, a
    one-layer slot pool): per layer unpack + merge into a 2-deep complete_layer
    ring, and the same loop with the fused call."""
    w = wl.mla_agentic(seed)
    sh = w.shape
    L, S, B, rb, C = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, sh.c_kv_bytes
    R = len(w.t_hit)
    per_req = [wl.blocks_needed(t, B) for t in w.t_all]
    N = sum(per_req)
    miss_all = sum(w.t_miss) * C
    ring_bytes = sum(w.t_all) * C
    need = sum(w.t_hit) * L * C + L * miss_all + N * B * rb + 2 * ring_bytes
    free, _ = torch.cuda.mem_get_info(dev)
    log(f"[bench] {w.name}: allocating {need / 2**30:.1f} GiB of {free / 2**30:.1f} GiB free")
    if need + (2 << 30) > free:
        return {"workload": w.name, "skipped": f"needs {need} bytes, {free} free"}
    u8 = dict(dtype=torch.uint8, device=dev)
    bts = [torch.from_numpy(t).to(dev) for t in wl.block_tables(w.seed, 2, N, per_req)]
    fbs = []
    for r in range(R):
        fbs.append(torch.empty(w.t_hit[r] * L * C, **u8))
        wl.fill_bf16_normal_(fbs[r], w.seed, 100 + r)
    misses = torch.empty(L * miss_all, **u8)                  # [L][request][T_miss][C]
    wl.fill_bf16_normal_(misses, w.seed, 7)
    slot = torch.empty(N * B * rb, **u8)
    rings = [torch.empty(ring_bytes, **u8) for _ in range(2)]
    moff, roff = [0], [0]
    for r in range(R):
        moff.append(moff[-1] + w.t_miss[r] * C)
        roff.append(roff[-1] + w.t_all[r] * C)
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, 0, N)
    seqs = [kv.seq(bts[r], fbs[r], w.t_hit[r]) for r in range(R)]
    merge_l, fused_l = [], []
    for l in range(L):
        mbase = misses.data_ptr() + l * miss_all
        out = rings[l % 2].data_ptr()
        merge_l.append([kv.merge_seq(fbs[r].data_ptr() + l * C, L * C, w.t_hit[r],
                                     mbase + moff[r], C, w.t_miss[r], out + roff[r], C)
                        for r in range(R)])
        fused_l.append([kv.layer_seq(bts[r], fbs[r], w.t_hit[r], mbase + moff[r], C,
                                     w.t_miss[r], out + roff[r], C) for r in range(R)])

    def separate():
        for l in range(L):
            kv.kvm_unpack_layer(ctx.handle, layout, slot, L, l, seqs)
            kv.kvm_merge_layer(ctx.handle, C, merge_l[l])

    def fused():
        for l in range(L):
            kv.kvm_unpack_merge_layer(ctx.handle, layout, slot, L, l, fused_l[l])

    th, ta, tm = sum(w.t_hit), sum(w.t_all), sum(w.t_miss)
    bytes_sep = L * (2 * th * C + 2 * ta * C)
    bytes_fused = L * (3 * th + 2 * tm) * C
    ev = Events(torch)
    out = {"workload": w.name, "sum_t_hit": th, "sum_t_miss": tm}
    for name, fn, nbytes in (("separate", separate, bytes_sep), ("fused", fused, bytes_fused)):
        fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            ev.around(name, fn)
        torch.cuda.synchronize()
        ms = ev.mean_ms(name)
        all_ms = ev.all_ms(name)
        out[name] = {"ms_per_loop": round(ms, 3),
                     "ms_p10_p50_p90": [round(quantile(all_ms, q), 3) for q in (0.1, 0.5, 0.9)],
                     "repetitions": reps, "bytes_per_loop": nbytes,
                     "GBps": round(nbytes / (ms * 1e6), 1),
                     "pct_hbm_peak": round(100 * nbytes / (ms * 1e6) / HBM_PEAK_GBS, 2)}
    # each op of the separate loop alone (its 61 launches back to back), for
    # per-launch times and the dominant kernel's roofline
    per_op = {"unpack_layer": ("k_unpack", 2 * th * C,
                               lambda: [kv.kvm_unpack_layer(ctx.handle, layout, slot, L, l, seqs)
                                        for l in range(L)]),
              "merge_layer": ("k_merge", 2 * ta * C,
                              lambda: [kv.kvm_merge_layer(ctx.handle, C, merge_l[l])
                                       for l in range(L)])}
    for name, (_, _, fn) in per_op.items():
        for _ in range(reps):
            ev.around(name, fn)
    torch.cuda.synchronize()
    ops = {}
    for name, (kernel, nbytes, _) in per_op.items():
        per_launch = [t / L for t in ev.all_ms(name)]
        ms = statistics.fmean(per_launch)
        ops[name] = {"kernel": kernel, "bytes_per_launch": nbytes, "ms_per_launch": round(ms, 4),
                     "ms_per_launch_p10_p50_p90": [round(quantile(per_launch, q), 4)
                                                   for q in (0.1, 0.5, 0.9)],
                     "GBps": round(nbytes / (ms * 1e6), 1),
                     "pct_hbm_peak": round(100 * nbytes / (ms * 1e6) / HBM_PEAK_GBS, 2)}
    out["ops"] = ops
    dom = max(ops, key=lambda k: ops[k]["ms_per_launch"])
    out["roofline"] = roofline(ops[dom]["kernel"], f"mla {dom}", ops[dom]["bytes_per_launch"],
                               ops[dom]["ms_per_launch"],
                               f"one launch: HIP events around the op's {L} launches back to "
                               f"back, divided by {L}")
    assert ctx.take_device_errors() == 0
    if verify:
        # every layer of one more separate loop, then of one more fused loop
        # (its slot pool and complete_layer ring reset to the sentinel first),
        # each checked right after its moves
        slots = slot.view(N, B, C)
        for l in list(range(L)) + [-1 - l for l in range(L)]:
            fused_pass = l < 0
            l = -1 - l if fused_pass else l
            ring = rings[l % 2]
            if fused_pass:
                slot.fill_(0xA5)
                ring.fill_(0xA5)
                kv.kvm_unpack_merge_layer(ctx.handle, layout, slot, L, l, fused_l[l])
            else:
                kv.kvm_unpack_layer(ctx.handle, layout, slot, L, l, seqs)
                kv.kvm_merge_layer(ctx.handle, C, merge_l[l])
            mbase = l * miss_all
            for r in range(R):
                th = w.t_hit[r]
                fbl = fbs[r].view(th, L, C)[:, l]
                o = ring[roff[r]:roff[r + 1]].view(-1, C)
                tag = "fused " if fused_pass else ""
                expect(torch.equal(o[:th], fbl), f"mla {tag}complete_layer hit rows, layer {l} request {r}")
                expect(torch.equal(o[th:], misses[mbase + moff[r]:mbase + moff[r + 1]].view(-1, C)),
                       f"mla {tag}complete_layer miss rows, layer {l} request {r}")
                t = torch.arange(th, device=slot.device)
                expect(torch.equal(slots[bts[r].long()[t // B], t % B], fbl),
                       f"mla {tag}slot rows, layer {l} request {r}")
    del fbs, misses, slot, rings, bts
    torch.cuda.empty_cache()
    return out


def small_call_section(torch, kv, wl, ctx, dev, calls=2000):
    """Per-call cost of small calls, back to back on one stream with no sync in
    between: the pages' case for batching is the submission cost per object.
    unpack_layer of the tiny workload (one request of 240 hit tokens, 30 KiB),
    the fused unpack_merge_layer of the same request with its 16 miss tokens,
    a batched copy of 64 objects of 4 KiB, and for reference one torch device
    copy of 4 KiB per call. Microseconds per call on the host clock, pipelined."""
    w = wl.TINY
    sh = w.shape
    L, S, B, rb, N = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes, w.pool_blocks
    u8 = dict(dtype=torch.uint8, device=dev)
    pool = torch.empty(L * S * N * B * rb, **u8)
    t_hit = w.t_hit[0]
    bt = torch.from_numpy(wl.block_tables(w.seed, 2, N, [wl.blocks_needed(t_hit, B)])[0]).to(dev)
    full = torch.empty(t_hit * L * S * rb, **u8)
    layout = kv.pool_layout(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    seqs = [kv.seq(bt, full, t_hit)]
    t_miss, C = w.t_miss[0], S * rb
    miss = torch.empty(t_miss * C, **u8)
    out = torch.empty((t_hit + t_miss) * C, **u8)
    fused = kv.records([kv.layer_seq(bt, full, t_hit, miss.data_ptr(), C, t_miss, out, C)])
    import numpy as np
    lens = np.full(64, 4096, np.int64)
    d = np.stack([wl.placements(9, 1, lens, 1 << 22), wl.placements(9, 2, lens, 1 << 22), lens],
                 axis=1).astype(np.uint64)
    descs = torch.from_numpy(d.view(np.uint8).reshape(-1)).to(dev)
    src, dst = torch.empty(1 << 22, **u8), torch.empty(1 << 22, **u8)
    a, b = torch.empty(4096, **u8), torch.empty(4096, **u8)

    def per_call(fn):
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / calls

    import ctypes
    lib = kv.load()
    arr = kv.records(seqs)
    lay = ctypes.byref(layout)
    st = torch.cuda.current_stream().cuda_stream
    pool_p, src_p, dst_p, descs_p = pool.data_ptr(), src.data_ptr(), dst.data_ptr(), descs.data_ptr()
    return {"unpack_layer_tiny_us": round(per_call(
                lambda: kv.kvm_unpack_layer(ctx.handle, layout, pool, L, 1, seqs)), 2),
            "unpack_layer_tiny_records_us": round(per_call(
                lambda: kv.kvm_unpack_layer(ctx.handle, layout, pool, L, 1, arr)), 2),
            "unpack_layer_tiny_c_us": round(per_call(
                lambda: lib.kvm_unpack_layer(ctx.handle, lay, pool_p, L, 1, arr, 1, st)), 2),
            "pack_full_tiny_c_us": round(per_call(
                lambda: lib.kvm_pack_full(ctx.handle, lay, pool_p, L, arr, 1, st)), 2),
            "unpack_merge_layer_tiny_c_us": round(per_call(
                lambda: lib.kvm_unpack_merge_layer(ctx.handle, lay, pool_p, L, 1, fused, 1, st)), 2),
            "batch_copy_64x4KiB_us": round(per_call(
                lambda: kv.kvm_batch_copy(ctx.handle, dst, 1 << 22, src, 1 << 22, descs, 64)), 2),
            "batch_copy_64x4KiB_c_us": round(per_call(
                lambda: lib.kvm_batch_copy(ctx.handle, dst_p, 1 << 22, src_p, 1 << 22, descs_p, 64,
                                           st)), 2),
            "torch_copy_4KiB_us": round(per_call(lambda: b.copy_(a)), 2),
            "ctypes_call_us": round(per_call(lambda: lib.kvm_version()), 2),
            "calls": calls,
            "note": "host clock per call, back to back, no sync between calls; *_us through "
                    "the Python binding with a list of records, *_records_us with a reused "
                    "records() array, *_c_us straight through ctypes with every argument "
                    "prepared once (the C entry point's own cost plus ctypes_call_us, a "
                    "call of kvm_version)"}


def restore_section(torch, kv, wl, ctx, dev, seed, reps=10, verify=False):
    """The long-sequence restore list (one 128,000-token sequence of a
    Qwen3-32B-like model, L=64, B=64: 256,000 K/V objects of 128 KiB from
    random staging offsets into their paged slots), as one batched copy and as
    one call per layer (4,000 objects each)."""
    descs_np, _, pool_bytes = wl.qwen32b_object_descs(seed)
    n, L = len(descs_np), wl.QWEN32B_SHAPE.layers
    total = int(descs_np[:, 2].sum())
    log(f"[bench] restore: {n} objects of 128 KiB, {total / 1e9:.2f} GB each way")
    u8 = dict(dtype=torch.uint8, device=dev)
    staging = torch.empty(wl.QWEN32B_STAGING, **u8)
    wl.fill_random_bytes_(staging, seed, 3)
    pool = torch.empty(pool_bytes, **u8)
    descs = torch.from_numpy(descs_np.view(__import__("numpy").uint8).reshape(-1)).to(dev)
    per = n // L
    ctx.reserve(64, n)

    def one_call():
        kv.kvm_batch_copy(ctx.handle, pool, pool_bytes, staging, wl.QWEN32B_STAGING, descs, n)

    def per_layer():
        for l in range(L):
            kv.kvm_batch_copy(ctx.handle, pool, pool_bytes, staging, wl.QWEN32B_STAGING,
                              descs.data_ptr() + l * per * 24, per)

    out = {"workload": f"restore list: {n} objects x 128 KiB (L={L}, 2000 blocks, K and V)",
           "bytes_rw": 2 * total, "objects_per_layer_call": per}
    ev = Events(torch)
    for name, fn in (("one_call", one_call), ("per_layer_calls", per_layer)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            ev.around(name, fn)
        torch.cuda.synchronize()
        ms = ev.mean_ms(name)
        gbs = 2 * total / (ms * 1e6)
        out[name] = {"ms": round(ms, 4),
                     "ms_p10_p50_p90": [round(quantile(ev.all_ms(name), q), 4)
                                        for q in (0.1, 0.5, 0.9)],
                     "repetitions": reps, "GBps": round(gbs, 1),
                     "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                     "descriptors_per_s": round(n / (ms * 1e-3), 0)}
    # every object is one 128 KiB piece, so after the first call of each list
    # shape a call is a single k_bc_each launch (one workgroup per object)
    out["roofline"] = roofline("k_bc_each", "restore list, one call", 2 * total,
                               out["one_call"]["ms"],
                               "one call: HIP events around its single k_bc_each launch")
    assert ctx.take_device_errors() == 0
    if verify:
        for fn in (one_call, per_layer):
            pool.fill_(0xA5)
            fn()
            torch.cuda.synchronize()
            verify_copies(torch, staging, pool, descs_np)
    del staging, pool, descs
    torch.cuda.empty_cache()
    return out


def device_info(torch):
    """What the runtime reports of the GPU, to tell boxes apart when their
    rates differ."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}
    for attr in ("clock_rate", "memory_clock_rate", "memory_bus_width"):
        if hasattr(p, attr):
            info[attr] = getattr(p, attr)
    return info


def host_cpu():
    """The host CPU's model name and the hardware threads this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline(wl, reps=12, host_threads=16):
    """The oracle on the host cores, on request 0 of the same workload: its 32
    unpack_layer + merge_layer calls and its pack_full (1/8 of a step). The
    request's 2080 blocks sit in a host pool of exactly that many blocks under
    a random permutation table (the same random 32 KiB object accesses without
    a 48 GiB host pool); every page is touched before timing. Timed on one
    thread, then from up to host_threads threads (a GPU's share of the host)
    over disjoint parts of the same sample."""
    import numpy as np
    import oracle
    w = wl.LLAMA8B
    sh = w.shape
    L, S, B, rb = sh.layers, sh.sides, sh.block_tokens, sh.row_bytes
    C = sh.c_kv_bytes
    t_hit, t_miss = w.t_hit[0], w.t_miss[0]
    t_all = t_hit + t_miss
    N = wl.blocks_needed(t_all, B)
    table = wl.block_tables(w.seed, 2, N, [N])[0]
    ref = oracle.pool_struct(S, B, rb, B * rb, N * B * rb, S * N * B * rb, N)
    pool = np.full(L * S * N * B * rb, 1, np.uint8)
    fb = np.full(t_hit * L * C, 3, np.uint8)
    miss = np.full(t_miss * L * C, 5, np.uint8)
    complete = np.full(L * t_all * C, 7, np.uint8)
    packed = np.full(t_all * L * C, 9, np.uint8)

    def sample():
        for l in range(L):
            oracle.unpack_layer(pool, ref, L, l, table, t_hit, fb)
            oracle.merge_layer(C, fb[l * C:], L * C, t_hit, miss[l * C:], L * C, t_miss,
                               complete[l * t_all * C:], C)
        oracle.pack_full(pool, ref, L, table, t_all, packed)

    model, threads = host_cpu()
    nthreads = max(1, min(threads, host_threads))
    per = -(-N // nthreads)                  # blocks of each thread's pack_full share
    spans = [(b * B, min(t_all, (b + per) * B)) for b in range(0, N, per)]

    def layers_of(k):
        for l in range(k, L, nthreads):      # disjoint pool layers and complete_layer rows
            oracle.unpack_layer(pool, ref, L, l, table, t_hit, fb)
            oracle.merge_layer(C, fb[l * C:], L * C, t_hit, miss[l * C:], L * C, t_miss,
                               complete[l * t_all * C:], C)

    def pack_span(span):                     # a block-aligned token range is a sequence
        t0, t1 = span
        oracle.pack_full(pool, ref, L, table[t0 // B:-(-t1 // B)], t1 - t0,
                         packed[t0 * L * C:t1 * L * C])

    def sample_threaded(ex):
        list(ex.map(layers_of, range(min(nthreads, L))))
        list(ex.map(pack_span, spans))

    def timed(fn, *a):
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn(*a)
            times.append(time.perf_counter() - t0)
        return statistics.median(times), sum(times)

    nbytes = L * 2 * t_hit * C + L * 2 * t_all * C + 2 * t_all * L * C
    dt, total = timed(sample)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(nthreads) as ex:   # ctypes calls release the GIL
        dt_mt, total_mt = timed(sample_threaded, ex)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"request 0 of 8 ({L} unpack_layer + {L} merge_layer + pack_full, "
                      f"{nbytes / 1e9:.1f} GB), median of {reps} runs ({total:.1f} s), "
                      f"single thread, host pool of the request's {N} blocks",
            "host": f"{model}; {threads} hardware threads available",
            "threaded": {"value": round(nbytes / dt_mt / 1e9, 3), "unit": "GB/s",
                         "cores": nthreads,
                         "sample": f"the same sample, median of {reps} runs ({total_mt:.1f} s): "
                                   f"the unchanged oracle called from {nthreads} threads, "
                                   f"unpack_layer + merge_layer split by layer, pack_full by "
                                   f"block-aligned token ranges"}}


PROFILES = os.path.join(ROOT, "profiles")
# The sources that decide what a launch moves and how: the kernels, and the
# host code that picks their tiles and grids.
KERNEL_SOURCES = ("paged_kv_cache_kvm_amd/csrc/kernels.hip",
                  "paged_kv_cache_kvm_amd/csrc/kvm_internal.h",
                  "paged_kv_cache_kvm_amd/csrc/api.cpp")


def kernel_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def measured_traffic(op):
    """HBM bytes (read + write) per launch of `op`'s kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summaries under profiles/ (their
    "traffic-json:" lines), or None when no summary taken on the sources built
    now has it."""
    want = kernel_source_sha256()
    try:
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return None
    for name in names:
        try:
            lines = open(os.path.join(PROFILES, name)).read().splitlines()
        except OSError:
            continue
        for line in lines:
            if not line.startswith("traffic-json: "):
                continue
            rec = json.loads(line[len("traffic-json: "):])
            if rec.get("kernel_source_sha256") == want and op in rec.get("bytes_per_launch", {}):
                return rec["bytes_per_launch"][op]
    return None


def roofline(kernel, op, bytes_per_launch, ms_per_launch, timed):
    """The HBM roofline entry of one kernel: algorithmic bytes per launch over
    its launch time (HIP events on the launch stream; `timed` says what the
    events bracket), against the 8 TB/s peak, with the measured traffic when a
    current profile has it."""
    gbs = bytes_per_launch / (ms_per_launch * 1e6)
    return {"bound": "hbm", "kernel": kernel, "op": op, "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(op), "algorithmic_bytes_per_launch": bytes_per_launch,
            "ms_per_launch": round(ms_per_launch, 4), "timed": timed}


def run_verify(fn):
    """Run fn; a VerifyError (an output that breaks its definition) ends the
    run with status 1 and the failing check on stderr."""
    try:
        return fn()
    except VerifyError as e:
        log(f"[bench] verify FAILED: {e}")
        sys.exit(1)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards "
              "by request with no exchange, so per-GPU throughput is the one-GPU figure",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from paged_kv_cache_kvm_amd import kvmove as kv
    from paged_kv_cache_kvm_amd import workloads as wl
    dev = torch.device("cuda:0")
    kv.load()
    ctx = kv.Context(0)

    s = llama_setup(torch, kv, wl, dev, args.seed)
    step_bytes = sum(s["bytes"][k] * s["launches"][k] for k in s["bytes"])
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        llama_step(kv, ctx, s)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        llama_step(kv, ctx, s)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    value = step_bytes * args.steps / dt / 1e9
    verified = {}
    if args.verify:
        run_verify(lambda: verify_layer_loop(torch, s))
        verified["layer_loop"] = "pass"

    # per-launch durations: HIP events on the launch stream around a loop of
    # each op alone (its launches back to back), divided by the launch count
    ev = Events(torch)
    L = s["L"]
    for _ in range(max(5, args.steps)):
        ev.around("unpack_layer", lambda: [kv.kvm_unpack_layer(
            ctx.handle, s["layout"], s["pool"], L, l, s["unpack_seqs"]) for l in range(L)])
        ev.around("merge_layer", lambda: [kv.kvm_merge_layer(
            ctx.handle, s["C"], s["merge_by_layer"][l]) for l in range(L)])
        ev.around("pack_full", lambda: kv.kvm_pack_full(ctx.handle, s["layout"], s["pool"], L,
                                                        s["pack_seqs"]))
    torch.cuda.synchronize()
    ops = {}
    for name in ("unpack_layer", "merge_layer", "pack_full"):
        per_launch = [t / s["launches"][name] for t in ev.all_ms(name)]
        ms = statistics.fmean(per_launch)
        gbs = s["bytes"][name] / (ms * 1e6)
        ops[name] = {"launches_per_step": s["launches"][name],
                     "bytes_per_launch": s["bytes"][name], "ms_per_launch": round(ms, 4),
                     "ms_per_launch_p10_p50_p90": [round(quantile(per_launch, q), 4)
                                                   for q in (0.1, 0.5, 0.9)],
                     "repetitions": len(per_launch),
                     "GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
    dom = max(ops, key=lambda k: ops[k]["ms_per_launch"] * ops[k]["launches_per_step"])
    fused = fused_section(torch, kv, ctx, s, args.steps, args.warmup, ms_step)
    if args.verify:
        def verify_fused():
            # one more fused step (32 x unpack_merge_layer + pack_full) into
            # complete_layer, Full Blocks and the hit tokens' pool slots reset
            # to the sentinel, checked as the separate loop is
            bts, complete, packed = s["keep"][0], s["keep"][3], s["keep"][4]
            complete.fill_(0xA5)
            for p in packed:
                p.fill_(0xA5)
            sh = s["w"].shape
            B, th = sh.block_tokens, s["w"].t_hit[0]
            pv = s["pool"].view(s["L"], sh.sides, s["w"].pool_blocks, B, sh.row_bytes)
            for bt in bts:
                for t0 in range(0, th, 4096):
                    t = torch.arange(t0, min(th, t0 + 4096), device=pv.device)
                    pv[:, :, bt.long()[t // B], t % B] = 0xA5
            llama_fused_step(kv, ctx, s)
            torch.cuda.synchronize()
            verify_layer_loop(torch, s)
        run_verify(verify_fused)
        verified["fused_layer_loop"] = "pass"
    host = None if args.no_host else host_tier_section(torch, kv, ctx, s)
    pipe = None
    if not args.no_pipeline:
        # its own context: it uses two streams, and a context that has seen a
        # second stream records an event per call from then on
        pctx = kv.Context(0)
        try:
            pipe = pipeline_section(torch, kv, pctx, s)
            assert pctx.take_device_errors() == 0
        finally:
            pctx.close()
    assert ctx.take_device_errors() == 0
    workload = s["w"].name
    del s
    torch.cuda.empty_cache()

    # Plain copies, for reference only: pack and the fused kernel move more than
    # either, so neither bounds the ops and no op is reported as a share of them.
    torch_copy, stream_copy = plain_copies(torch, kv, ctx, dev)
    copy_reps, mla_reps = (args.reps, args.reps) if args.reps else (10, 5)
    mla = None if args.no_mla else run_verify(
        lambda: mla_section(torch, kv, wl, ctx, dev, args.seed + 2, reps=mla_reps,
                            verify=args.verify))
    bc = None if args.no_batch_copy else run_verify(
        lambda: batch_copy_section(torch, kv, wl, ctx, dev, args.seed + 3, reps=copy_reps,
                                   verify=args.verify))
    restore = None if args.no_restore else run_verify(
        lambda: restore_section(torch, kv, wl, ctx, dev, args.seed + 1, reps=copy_reps,
                                verify=args.verify))
    if args.verify:
        for name, sec in (("mla_layer_loop", mla), ("batch_copy", bc),
                          ("batch_copy_restore", restore)):
            if sec is not None and "skipped" not in sec:
                verified[name] = "pass"
    small = None if args.no_small else small_call_section(torch, kv, wl, ctx, dev)
    ctx.close()
    cpu = None if args.no_cpu else cpu_baseline(wl)

    kernel = {"unpack_layer": "k_unpack", "merge_layer": "k_merge", "pack_full": "k_pack"}[dom]
    out = {
        "metric": "effective KV-move GB/s (read+write) and % of HBM peak; descriptors/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": {"workload": workload, "payload": "bf16 ~ N(0,1)", "layers": 32, "h_kv": 8,
                   "head_dim": 128, "block_tokens": 16, "requests": 8, "t_hit": 32768,
                   "t_miss": 512, "pool_blocks": 24576, "seed": args.seed,
                   "step": "32 x (unpack_layer + merge_layer) + pack_full",
                   "bytes_per_step": step_bytes},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "ops": ops,
        "roofline": roofline(kernel, dom, ops[dom]["bytes_per_launch"], ops[dom]["ms_per_launch"],
                             "one launch: HIP events around the op's 32 launches (1 for "
                             "pack_full) back to back, divided by their count"),
        "fused_layer_loop": fused,
        "host_tier": host,
        "pipeline": pipe,
        "plain_copy_2GiB_GBps": {"torch_copy": round(torch_copy, 1),
                                 "kvm_batch_copy_one_object": round(stream_copy, 1),
                                 "note": "reference rates of a plain device copy, not a "
                                         "ceiling: pack and the fused kernel move more"},
        "mla_layer_loop": mla,
        "batch_copy": bc,
        "batch_copy_restore": restore,
        "small_calls": small,
        "cpu_baseline": cpu,
        "verify": verified if args.verify else None,
        "device": device_info(torch),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
