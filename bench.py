#!/usr/bin/env python3
"""Benchmark of libq4gemv on one MI355X.

Default run (one JSON line on stdout): the headline workload, the fused
gate+up Q4_K GEMV at M=1, K=4096, N=14336 per matrix (66,060,288 weight bytes
per call), timed over --steps calls after --warmup untimed calls.

  value        whole-job effective weight bandwidth: weight bytes of the
               --steps timed calls (HIP graphs of >= 100 back-to-back launches,
               or one graph of all of them) / wall time between two device
               synchronizations (GB/s)
  roofline     the kernel itself: weight bytes per launch / mean launch
               duration, from HIP events recorded on the launch stream around
               4 replays of HIP graphs of 100 back-to-back launches each (no
               host gaps, graph-launch overhead amortized; whatever --steps
               is), against the 8 TB/s HBM3E peak
  pure_read    the same for the pure-read ceiling kernel (same bytes, same
               addressing, no arithmetic), for the reference stream (the same
               byte count read the fastest way measured: contiguous
               non-temporal 1 KiB wave loads), and a plain device-to-device
               copy of the same bytes (read + write) as an external reference
  cpu_baseline the CPU oracle (plain C, float64) timed on this host's cores on
               a bounded sample of the same workload

Weights stay resident in HBM; to measure HBM and not the 256 MB Infinity Cache
every call reads a different copy of the weights, from a rotation of copies
totalling at least 1 GiB.

  --all REPORT   additionally time every named workload and its ceiling and
                 write REPORT.json and REPORT.md
  --ceilings     only time the read ceilings of this part: the reference
                 stream and a device copy at the headline's 66 MB and at 8
                 times that
  --copy-calibration MIB
                 only run a plain device-to-device copy of MIB MiB 20 times:
                 the known-size reference that scales the FETCH_SIZE and
                 WRITE_SIZE counters of a profiler run into bytes

roofline.traffic is the HBM bytes per launch of the headline kernel measured
with those counters (FETCH_SIZE + WRITE_SIZE, each scaled by the copy's
factor); it is read from the counter summary in profiles/ and reported only
while the kernel sources hash to the value recorded there, else null.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s and % of HBM peak, Q4_K GEMV M=1 K=4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fused_gate_up_q4k_M1_K4096_N14336x2.txt")
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--all", metavar="REPORT", default=None,
                    help="also time every named workload; write REPORT.json / REPORT.md")
    ap.add_argument("--chain", action="store_true",
                    help="only time dispatch chains (the smallest call back to back, a dense "
                         "FFN decode step, an expert decode step; eager and as HIP graph "
                         "replays) and the submit+wait / submit+spin turnaround")
    ap.add_argument("--ceilings", action="store_true",
                    help="only time the reference stream and a device copy at the headline's "
                         "66 MB and at 8 times that (the read ceilings of this part)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB 20 times (counter scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound of the CPU-oracle sample (0 skips it)")
    return ap.parse_args()


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Rotation:
    """`ncopies` copies of one packed weight buffer inside one device allocation."""

    def __init__(self, torch, dev, host_bytes, min_total=ROTATE_BYTES):
        import numpy as np
        nbytes = int(host_bytes.nbytes)
        self.nbytes = nbytes
        self.stride = (nbytes + 4095) // 4096 * 4096
        self.ncopies = max(2, math.ceil(min_total / self.stride))
        self.buf = torch.empty(self.ncopies * self.stride, dtype=torch.uint8, device=dev)
        src = torch.from_numpy(np.ascontiguousarray(host_bytes).reshape(-1)).to(dev)
        self.buf.view(self.ncopies, self.stride)[:, :nbytes].copy_(
            src.view(1, nbytes).expand(self.ncopies, nbytes))
        self.base = self.buf.data_ptr()
        del src

    def ptr(self, i):
        return self.base + (i % self.ncopies) * self.stride


GRAPH_LAUNCHES = 100  # launches per graph of the kernel-duration measurement
DURATION_BATCHES = 4  # graphs of the kernel-duration measurement


def _capture(torch, s, launch, first, count):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.capture_begin()
        for k in range(count):
            launch(first + k, s.cuda_stream)
        g.capture_end()
    return g


def time_launches(torch, launch, warmup, steps, outs):
    """launch(i, stream) enqueues call i.  Three phases on one stream:
      1. `warmup` untimed calls, eagerly;
      2. the timed region: exactly `steps` calls, captured as HIP graphs of
         at least GRAPH_LAUNCHES back-to-back launches (one graph if steps is
         smaller), replayed between two device synchronizations -> the wall
         time of the whole job;
      3. the kernel duration: DURATION_BATCHES graphs of GRAPH_LAUNCHES
         launches each, whatever `steps` is, each replay bracketed by HIP
         events recorded on the replay stream, so graph-launch overhead is
         amortized over 100 launches -> per-launch mean of each batch.
    Afterwards the last graph's outputs (`outs`) are checked to be
    bit-identical to an eager launch of the same call.  Returns (wall
    seconds of phase 2, per-launch ms of each phase-3 batch, launches per
    batch)."""
    s = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(s):
        for i in range(warmup):
            launch(i, s.cuda_stream)
    torch.cuda.synchronize()
    n = warmup
    # phase 2: the timed steps
    steps = max(1, int(steps))
    ngraph = max(1, steps // GRAPH_LAUNCHES)
    cnts = [steps // ngraph] * ngraph
    cnts[-1] += steps - sum(cnts)
    graphs = []
    for cnt in cnts:
        graphs.append(_capture(torch, s, launch, n, cnt))
        n += cnt
    for g in graphs:  # first replays upload the graphs
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(s):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # phase 3: kernel duration
    dgraphs = []
    for _ in range(DURATION_BATCHES):
        dgraphs.append(_capture(torch, s, launch, n, GRAPH_LAUNCHES))
        n += GRAPH_LAUNCHES
    for g in dgraphs:
        g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in dgraphs]
    with torch.cuda.stream(s):
        for (e0, e1), g in zip(ev, dgraphs):
            e0.record()
            g.replay()
            e1.record()
    torch.cuda.synchronize()
    got = [o.clone() for o in outs]
    with torch.cuda.stream(s):
        launch(n - 1, s.cuda_stream)
    torch.cuda.synchronize()
    for a_, b_ in zip(got, outs):
        if not torch.equal(a_.view(torch.int32), b_.view(torch.int32)):
            raise RuntimeError("graph replay and eager launch of the same call differ")
    dcnts = [GRAPH_LAUNCHES] * DURATION_BATCHES
    return wall, [e0.elapsed_time(e1) / c for (e0, e1), c in zip(ev, dcnts)], dcnts


def stats(batch_ms, cnts):
    s = sorted(batch_ms)
    mean = sum(m * c for m, c in zip(batch_ms, cnts)) / sum(cnts)
    return dict(mean_ms=mean, median_ms=s[len(s) // 2], min_ms=s[0], max_ms=s[-1],
                spread=s[-1] / s[0] - 1.0 if s[0] > 0 else None)


def check(status, what):
    if status != 0:
        import bit_block_quantized_dequant_amd as q4
        raise RuntimeError("%s failed: %s" % (what, q4.q4_strerror(status)))


# ---------------------------------------------------------------------------
# workloads: each returns (weight bytes per call, launch(i), ceiling launch(i), notes)
# ---------------------------------------------------------------------------
def setup_workload(torch, dev, index, M, distinct=False, silu=False, norm=False, soa=False,
                   splitk=False):
    import numpy as np

    import bit_block_quantized_dequant_amd as q4
    from bit_block_quantized_dequant_amd import synth

    L = q4.lib()
    if index == 6:
        d = synth.down_inputs(M, distinct)
    elif index == 7:
        # the dense down-projection after workload 4's gate+up pair: Q4_K,
        # 4096 rows x 14336, x ~ N(0, 1), its own seed
        rng7 = synth.make_rng(synth.SEED_BASE + 7)
        N7, K7 = synth.DENSE_DOWN["N"], synth.DENSE_DOWN["K"]
        d = dict(N=N7, K=K7, w=synth.q4k_matrix(rng7, N7, K7),
                 x=synth.activations(rng7, M, K7))
    else:
        d = synth.workload_inputs(index, M=M, distinct=distinct)
    N, K = d["N"], d["K"]
    keep = []

    def T(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        keep.append(t)
        return t

    x = T(d["h"] if index == 6 else d["x"])
    notes = {}
    rot = None
    if index in (1, 2) and soa:
        # split arrays, one copy = [nibble blocks | f16 scales]
        sc, qs = synth.q4_0_soa_split(d["w"])
        qbytes = qs.nbytes
        rot = Rotation(torch, dev, np.concatenate([qs.reshape(-1), sc.reshape(-1)]))
        y = torch.empty(M, N, device=dev)
        cks = torch.empty(N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes

        def launch(i, stream):
            p = rot.ptr(i)
            check(L.q4_0_gemv_soa(y.data_ptr(), p + qbytes, p, x.data_ptr(), M, N, K, stream),
                  "q4_0_gemv_soa")

        def ceil_launch(i, stream):  # (no mirror of its own: the 18-byte call's addressing)
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_Q4_0_GEMV, rot.ptr(i), None, None,
                                 M, 0, 0, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    elif index in (1, 2) and splitk:
        rot = Rotation(torch, dev, d["w"])
        y = torch.empty(M, N, device=dev)
        cks = torch.empty(N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes
        need = q4.splitk_workspace_bytes(q4.Q4_FORMAT_Q4_0, M, N, K)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        notes = dict(splitk_workspace_bytes=need)
        keep.append(ws)

        def launch(i, stream):
            check(L.q4_0_gemv_splitk(y.data_ptr(), rot.ptr(i), x.data_ptr(), M, N, K,
                                     ws.data_ptr(), need, stream), "q4_0_gemv_splitk")

        def ceil_launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_Q4_0_GEMV, rot.ptr(i), None, None,
                                 M, 0, 0, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    elif index in (1, 2):
        rot = Rotation(torch, dev, d["w"])
        y = torch.empty(M, N, device=dev)
        cks = torch.empty(N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes

        def launch(i, stream):
            check(L.q4_0_gemv(y.data_ptr(), rot.ptr(i), x.data_ptr(), M, N, K, stream),
                  "q4_0_gemv")

        def ceil_launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_Q4_0_GEMV, rot.ptr(i), None, None,
                                 M, 0, 0, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    elif index == 7:
        rot = Rotation(torch, dev, d["w"])
        y = torch.empty(M, N, device=dev)
        cks = torch.empty(N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes
        need = q4.splitk_workspace_bytes(q4.Q4_FORMAT_Q4K, M, N, K) if splitk else 0
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        keep.append(ws)

        def launch(i, stream):
            if splitk:
                check(L.q4k_gemv_splitk(y.data_ptr(), rot.ptr(i), x.data_ptr(), M, N, K,
                                        ws.data_ptr(), need, stream), "q4k_gemv_splitk")
                return
            check(L.q4k_gemv(y.data_ptr(), rot.ptr(i), x.data_ptr(), M, N, K, stream), "q4k_gemv")

        def ceil_launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_Q4K_GEMV, rot.ptr(i), None, None,
                                 M, 0, 0, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    elif index == 3:
        rot = Rotation(torch, dev, d["w"])
        g = T(d["gamma"])
        y = torch.empty(M, N, device=dev)
        cks = torch.empty(N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes

        def launch(i, stream):
            check(L.fused_rmsnorm_q4k_gemv(y.data_ptr(), rot.ptr(i), x.data_ptr(), g.data_ptr(),
                                           d["eps"], M, N, K, stream), "fused_rmsnorm_q4k_gemv")

        def ceil_launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_Q4K_GEMV, rot.ptr(i), None, None,
                                 M, 0, 0, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    elif index == 4:
        both = np.concatenate([d["w_gate"].reshape(-1), d["w_up"].reshape(-1)])
        rot = Rotation(torch, dev, both)
        half = d["w_gate"].nbytes
        gate = torch.empty(M, N, device=dev)
        up = torch.empty(M, N, device=dev)
        cks = torch.empty(2 * N, dtype=torch.int32, device=dev)
        wbytes = rot.nbytes

        gam = T(synth.gamma(synth.make_rng(8500), K)) if norm else None  # (K floats)

        def launch(i, stream):
            p = rot.ptr(i)
            if silu and norm:
                check(L.fused_rmsnorm_gate_up_silu_q4k_gemv(gate.data_ptr(), p, p + half,
                                                            x.data_ptr(), gam.data_ptr(), 1e-5,
                                                            M, N, K, stream),
                      "fused_rmsnorm_gate_up_silu_q4k_gemv")
                return
            if silu:
                check(L.fused_gate_up_silu_q4k_gemv(gate.data_ptr(), p, p + half, x.data_ptr(),
                                                    M, N, K, stream),
                      "fused_gate_up_silu_q4k_gemv")
                return
            if norm:
                check(L.fused_rmsnorm_gate_up_q4k_gemv(gate.data_ptr(), up.data_ptr(), p,
                                                       p + half, x.data_ptr(), gam.data_ptr(),
                                                       1e-5, M, N, K, stream),
                      "fused_rmsnorm_gate_up_q4k_gemv")
                return
            check(L.fused_gate_up_q4k_gemv(gate.data_ptr(), up.data_ptr(), p, p + half,
                                           x.data_ptr(), M, N, K, stream),
                  "fused_gate_up_q4k_gemv")

        def ceil_launch(i, stream):
            p = rot.ptr(i)
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_GATE_UP, p, p + half, None, M, 0, 0,
                                 N, K, stream), "q4_pure_read")
        keep += [rot, gate, up, cks]
        outs, couts = ([gate] if silu else [gate, up]), [cks]
    elif index == 5:
        E, top_k = d["E"], d["top_k"]
        both = np.concatenate([d["w_gate"].reshape(-1), d["w_up"].reshape(-1)])
        rot = Rotation(torch, dev, both)
        half = d["w_gate"].nbytes
        ids = T(d["ids"])
        gate = torch.empty(M, top_k, N, device=dev)
        up = torch.empty(M, top_k, N, device=dev)
        cks = torch.empty(2 * M * top_k * N, dtype=torch.int32, device=dev)
        uniq = len(set(int(e) for e in d["ids"].reshape(-1)))
        per_expert = 2 * N * synth.q4_0_row_bytes(K)
        wbytes = uniq * per_expert
        notes = dict(unique_experts=uniq, pairs=M * top_k,
                     pair_counted_bytes=M * top_k * per_expert)

        def launch(i, stream):
            p = rot.ptr(i)
            if silu:
                check(L.moe_q4_gemv_silu(gate.data_ptr(), p, p + half, x.data_ptr(),
                                         ids.data_ptr(), M, top_k, E, N, K, stream),
                      "moe_q4_gemv_silu")
                return
            check(L.moe_q4_gemv(gate.data_ptr(), up.data_ptr(), p, p + half, x.data_ptr(),
                                ids.data_ptr(), M, top_k, E, N, K, stream), "moe_q4_gemv")

        def ceil_launch(i, stream):
            p = rot.ptr(i)
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_MOE, p, p + half, ids.data_ptr(), M,
                                 top_k, E, N, K, stream), "q4_pure_read")
        keep += [rot, gate, up, cks]
        outs, couts = ([gate] if silu else [gate, up]), [cks]
    elif index == 6:
        # the expert down-projection (x holds the pair rows h[M, top_k, K])
        E, top_k = d["E"], d["top_k"]
        rot = Rotation(torch, dev, d["w_down"])
        ids = T(d["ids"])
        y = torch.empty(M, top_k, N, device=dev)
        cks = torch.empty(M * top_k * N, dtype=torch.int32, device=dev)
        uniq = len(set(int(e) for e in d["ids"].reshape(-1)))
        per_expert = N * synth.q4_0_row_bytes(K)
        wbytes = uniq * per_expert
        notes = dict(unique_experts=uniq, pairs=M * top_k,
                     pair_counted_bytes=M * top_k * per_expert)

        def launch(i, stream):
            check(L.moe_q4_gemv_down(y.data_ptr(), rot.ptr(i), x.data_ptr(), ids.data_ptr(), M,
                                     top_k, E, N, K, stream), "moe_q4_gemv_down")

        def ceil_launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_MOE_DOWN, rot.ptr(i), None,
                                 ids.data_ptr(), M, top_k, E, N, K, stream), "q4_pure_read")
        keep += [rot, y, cks]
        outs, couts = [y], [cks]
    notes["copies"] = rot.ncopies
    # reference stream: the same byte count as contiguous rows of 256 * 9/16
    # bytes (rounded down to whole rows)
    srb = synth.q4k_row_bytes(256)
    srows = wbytes // srb
    scks = torch.empty((srows * srb + 4095) // 4096, dtype=torch.int32, device=dev)
    keep.append(scks)

    def stream_launch(i, stream):
        check(L.q4_pure_read(scks.data_ptr(), q4.Q4_READ_STREAM, rot.ptr(i), None, None, 1, 0, 0,
                             srows, 256, stream), "q4_pure_read")
    return wbytes, launch, ceil_launch, notes, keep, outs, couts, (stream_launch, [scks])


def measure(torch, dev, index, M, warmup, steps, distinct=False, silu=False, norm=False,
            soa=False, splitk=False):
    (wbytes, launch, ceil_launch, notes, keep, outs, couts,
     (stream_launch, souts)) = setup_workload(torch, dev, index, M, distinct, silu, norm, soa,
                                              splitk)
    wall, durs, cnts = time_launches(torch, launch, warmup, steps, outs)
    cwall, cdurs, ccnts = time_launches(torch, ceil_launch, warmup, steps, couts)
    swall, sdurs, scnts = time_launches(torch, stream_launch, warmup, steps, souts)
    st, cst, sst = stats(durs, cnts), stats(cdurs, ccnts), stats(sdurs, scnts)
    res = dict(index=index, M=M, distinct=distinct, silu=silu, norm=norm, soa=soa, splitk=splitk,
               weight_bytes=wbytes,
               wall_s=wall,
               steps=steps,
               value_gbs=wbytes * steps / wall / 1e9,
               kernel=st, kernel_gbs=wbytes / (st["mean_ms"] * 1e-3) / 1e9,
               kernel_gbs_median=wbytes / (st["median_ms"] * 1e-3) / 1e9,
               ceiling=cst, ceiling_gbs=wbytes / (cst["mean_ms"] * 1e-3) / 1e9,
               stream=sst, stream_gbs=wbytes / (sst["mean_ms"] * 1e-3) / 1e9, **notes)
    res["frac_of_peak"] = res["kernel_gbs"] / HBM_PEAK_GBS
    res["frac_of_ceiling"] = res["kernel_gbs"] / res["ceiling_gbs"]
    res["frac_of_stream"] = res["kernel_gbs"] / res["stream_gbs"]
    del keep
    torch.cuda.empty_cache()
    return res


def measure_router(torch, dev, warmup, steps):
    """The router at the expert call's shape (4 tokens, 64 experts, K = 2048,
    top-6, normalized): 73,728 bytes of Q4_0 router weights per call, rotated
    over 1 GiB of copies like the other workloads; one launch, latency-bound,
    so only its duration is reported."""
    import numpy as np

    import bit_block_quantized_dequant_amd as q4
    from bit_block_quantized_dequant_amd import synth
    L = q4.lib()
    d = synth.workload_inputs(5)
    M, E, K, top_k = d["M"], d["E"], d["K"], d["top_k"]
    rng = synth.make_rng(8100)
    wr = synth.q4_0_matrix(rng, E, K)
    rot = Rotation(torch, dev, wr)
    x = torch.from_numpy(np.ascontiguousarray(d["x"])).to(dev)
    ids = torch.empty(M, top_k, dtype=torch.int32, device=dev)
    wts = torch.empty(M, top_k, device=dev)

    def launch(i, stream):
        check(L.moe_router_q4_0(ids.data_ptr(), wts.data_ptr(), rot.ptr(i), x.data_ptr(), M, E,
                                K, top_k, 1, stream), "moe_router_q4_0")
    wall, durs, cnts = time_launches(torch, launch, warmup, steps, [ids, wts])
    st = stats(durs, cnts)
    return dict(M=M, E=E, K=K, top_k=top_k, weight_bytes=int(wr.nbytes), kernel=st)


def measure_chain(torch, dev, n=300, reps=50):
    """Dispatch cost on one stream (inferencelayer kernel_lab: the dependent-
    dispatch chain probe, N tiny dispatches in one submission, and the
    submit + wait against submit + spin turnaround probe).

    Chains, each run n times back to back eagerly (one host launch per call,
    through the binding's ctypes calls) and as one captured HIP graph, wall
    time per call or step between two device synchronizations:
      small_call       the smallest workload (Q4_0 K=512 N=256, M=1), each
                       call ordered after the previous one by the stream;
      dense_ffn_step   one decode step of a dense FFN: RMSNorm + gate/up +
                       SiLU (Q4_K, K=4096, N=14336 per matrix) writing h, then
                       the down-projection of h (Q4_K, 4096 rows x 14336);
      moe_step         one decode step of the expert path at the expert
                       call's shape: the router over 64 Q4_0 expert rows, the
                       SiLU-gated expert gate/up on the ids it wrote (which
                       never leave the device), then the expert down-
                       projection of those rows (2048 rows x 1408 per expert).
    Turnaround (reps single launches of the smallest call, each alone on an
    idle device): submit then hipDeviceSynchronize (wait), against submit
    then polling an event recorded after it (spin)."""
    import numpy as np

    import bit_block_quantized_dequant_amd as q4
    from bit_block_quantized_dequant_amd import synth
    L = q4.lib()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    d1 = synth.workload_inputs(1)
    w1, x1 = T(d1["w"]), T(d1["x"])
    y1 = torch.empty(d1["M"], d1["N"], device=dev)
    # dense FFN: gate/up of workload 4, a down matrix of its own seed
    d4 = synth.workload_inputs(4, M=1)
    K4, N4 = d4["K"], d4["N"]
    wg4, wu4, x4 = T(d4["w_gate"]), T(d4["w_up"]), T(d4["x"])
    rng = synth.make_rng(8600)
    gam4 = T(synth.gamma(rng, K4))
    DN, DK = synth.DENSE_DOWN["N"], synth.DENSE_DOWN["K"]
    wd4 = T(synth.q4k_matrix(rng, DN, DK))
    h4 = torch.empty(1, N4, device=dev)
    y4 = torch.empty(1, DN, device=dev)
    assert DK == N4
    # expert path
    d5 = synth.workload_inputs(5)
    M, E, N, K, top_k = d5["M"], d5["E"], d5["N"], d5["K"], d5["top_k"]
    dd = synth.down_inputs(M)
    wr = T(synth.q4_0_matrix(synth.make_rng(8100), E, K))
    wg, wu, x5 = T(d5["w_gate"]), T(d5["w_up"]), T(d5["x"])
    wd = T(dd["w_down"])
    ids = torch.empty(M, top_k, dtype=torch.int32, device=dev)
    wts = torch.empty(M, top_k, device=dev)
    h = torch.empty(M, top_k, N, device=dev)
    y5 = torch.empty(M, top_k, dd["N"], device=dev)
    assert dd["K"] == N

    def small(stream):
        check(L.q4_0_gemv(y1.data_ptr(), w1.data_ptr(), x1.data_ptr(), 1, d1["N"], d1["K"],
                          stream), "q4_0_gemv")

    def ffn(stream):
        check(L.fused_rmsnorm_gate_up_silu_q4k_gemv(h4.data_ptr(), wg4.data_ptr(), wu4.data_ptr(),
                                                    x4.data_ptr(), gam4.data_ptr(), 1e-5, 1, N4,
                                                    K4, stream),
              "fused_rmsnorm_gate_up_silu_q4k_gemv")
        check(L.q4k_gemv(y4.data_ptr(), wd4.data_ptr(), h4.data_ptr(), 1, DN, DK, stream),
              "q4k_gemv")

    def moe(stream):
        check(L.moe_router_q4_0(ids.data_ptr(), wts.data_ptr(), wr.data_ptr(), x5.data_ptr(), M,
                                E, K, top_k, 1, stream), "moe_router_q4_0")
        check(L.moe_q4_gemv_silu(h.data_ptr(), wg.data_ptr(), wu.data_ptr(), x5.data_ptr(),
                                 ids.data_ptr(), M, top_k, E, N, K, stream), "moe_q4_gemv_silu")
        check(L.moe_q4_gemv_down(y5.data_ptr(), wd.data_ptr(), h.data_ptr(), ids.data_ptr(), M,
                                 top_k, E, dd["N"], N, stream), "moe_q4_gemv_down")

    out = {}
    s = torch.cuda.Stream()  # default priority
    for name, fn, cnt in (("small_call", small, n), ("dense_ffn_step", ffn, n // 3),
                          ("moe_step", moe, n // 3)):
        with torch.cuda.stream(s):
            for _ in range(10):
                fn(s.cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            for _ in range(cnt):
                fn(s.cuda_stream)
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / cnt
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            g.capture_begin()
            for _ in range(cnt):
                fn(s.cuda_stream)
            g.capture_end()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        graph = (time.perf_counter() - t0) / cnt
        out[name] = dict(n=cnt, eager_us=eager * 1e6, graph_us=graph * 1e6)
        print("chain %-16s %d in a row: eager %.2f us each, graph replay %.2f us each"
              % (name, cnt, eager * 1e6, graph * 1e6), file=sys.stderr, flush=True)
        del g
    # turnaround of one submission on an idle device
    waits, spins = [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            small(s.cuda_stream)
        torch.cuda.synchronize()
        waits.append(time.perf_counter() - t0)
        ev = torch.cuda.Event()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            small(s.cuda_stream)
            ev.record()
        while not ev.query():
            pass
        spins.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    waits.sort()
    spins.sort()
    out["turnaround"] = dict(reps=reps, wait_us_median=waits[reps // 2] * 1e6,
                             wait_us_min=waits[0] * 1e6, spin_us_median=spins[reps // 2] * 1e6,
                             spin_us_min=spins[0] * 1e6)
    print("turnaround of one small call: submit+wait %.1f us, submit+spin %.1f us (medians of %d)"
          % (waits[reps // 2] * 1e6, spins[reps // 2] * 1e6, reps), file=sys.stderr, flush=True)
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds):
    """The oracle's gate+up GEMV of the headline workload, timed on the host."""
    from bit_block_quantized_dequant_amd import synth
    from oracle import oracle

    o = oracle.default()
    d = synth.workload_inputs(4, M=1)
    N, K = d["N"], d["K"]
    nt = host_threads()
    wbytes = d["w_gate"].nbytes + d["w_up"].nbytes
    o.gate_up_q4k_gemv(d["w_gate"][:64], d["w_up"][:64], d["x"], 64, K, nt)  # warm
    calls, t0 = 0, time.perf_counter()
    while True:
        o.gate_up_q4k_gemv(d["w_gate"], d["w_up"], d["x"], N, K, nt)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= 1000:
            break
    t1 = time.perf_counter()
    o.gate_up_q4k_gemv(d["w_gate"], d["w_up"], d["x"], N, K, 1)
    one = time.perf_counter() - t1
    return dict(value=wbytes * calls / el / 1e9, unit="GB/s", cores=nt, kind="oracle",
                cpu_model=cpu_model(), single_thread_value=wbytes / one / 1e9,
                sample="%d full calls of the oracle's gate+up Q4_K GEMV (M=1, K=4096, "
                       "N=14336x2; float64 accumulation) in %.1f s on %d threads; "
                       "single_thread_value: one full call on 1 thread (%.2f s)"
                       % (calls, el, nt, one))


def source_sha256():
    """Hash of the HIP sources and the C header the library is built from."""
    import hashlib

    csrc = os.path.join(ROOT, "bit_block_quantized_dequant_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith((".h", ".hip")))
    files.append(os.path.join(ROOT, "include", "q4gemv.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != source_sha256():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measure_copy(torch, dev, nbytes, reps=50):
    """A plain device-to-device copy (torch's copy_, the runtime's copy
    kernel) of nbytes, from a rotation of sources totalling at least 1 GiB
    into one destination, timed with HIP events over `reps` copies after 5
    warmup copies.  An external reference beside the read ceilings: each copy
    reads and writes nbytes.  Returns the read+write GB/s and the mean us."""
    n = nbytes // 4
    ncopies = max(2, math.ceil(ROTATE_BYTES / nbytes))
    src = torch.ones(ncopies, n, dtype=torch.float32, device=dev)
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    for i in range(5):
        dst.copy_(src[i % ncopies])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dst.copy_(src[i % ncopies])
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return dict(bytes=n * 4, us_mean=us, read_write_gbs=2 * n * 4 / (us * 1e-6) / 1e9)


CEILING_BYTES = (66060288, 8 * 66060288)  # the headline's weight bytes, and 8 times that


def measure_ceilings(torch, dev, warmup=10, steps=100):
    """The read ceilings of this part at the headline's size and at 8 times it:
    the reference stream (Q4_READ_STREAM: 16-byte loads per lane, 4 KiB per
    wave step, the next block's loads ahead, non-temporal) over a rotation of
    at least 1 GiB, timed like every workload (HIP graphs of 100 launches,
    events), and a device-to-device copy of the same bytes beside it."""
    import numpy as np

    import bit_block_quantized_dequant_amd as q4
    from bit_block_quantized_dequant_amd import synth
    L = q4.lib()
    out = []
    for nbytes in CEILING_BYTES:
        rng = np.random.default_rng(7000 + nbytes % 997)
        rot = Rotation(torch, dev, rng.integers(0, 256, nbytes, dtype=np.uint8))
        srb = synth.q4k_row_bytes(256)
        srows = nbytes // srb
        cks = torch.empty((srows * srb + 4095) // 4096, dtype=torch.int32, device=dev)

        def launch(i, stream):
            check(L.q4_pure_read(cks.data_ptr(), q4.Q4_READ_STREAM, rot.ptr(i), None, None, 1,
                                 0, 0, srows, 256, stream), "q4_pure_read")
        wall, durs, cnts = time_launches(torch, launch, warmup, steps, [cks])
        st = stats(durs, cnts)
        cp = measure_copy(torch, dev, nbytes)
        gbs = nbytes / (st["mean_ms"] * 1e-3) / 1e9
        out.append(dict(bytes=nbytes, copies=rot.ncopies, stream_us_mean=st["mean_ms"] * 1e3,
                        stream_us_median=st["median_ms"] * 1e3, stream_gbs=gbs,
                        stream_frac_of_peak=gbs / HBM_PEAK_GBS,
                        copy_us_mean=cp["us_mean"], copy_read_write_gbs=cp["read_write_gbs"]))
        print("read ceiling %d bytes: stream %.2f us (%.0f GB/s, %.1f%% of 8 TB/s); device copy "
              "%.2f us (%.0f GB/s read+write)" % (nbytes, st["mean_ms"] * 1e3, gbs,
                                                  100 * gbs / HBM_PEAK_GBS, cp["us_mean"],
                                                  cp["read_write_gbs"]),
              file=sys.stderr, flush=True)
        del rot, cks
        torch.cuda.empty_cache()
    return out


def copy_calibration(torch, dev, mib):
    """A plain device-to-device copy of known size, run 20 times."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("copy calibration: %d launches, %d bytes read and %d bytes written per launch"
          % (20, n * 4, n * 4), flush=True)


def write_report(path, rows, headline, router=None):
    with open(path + ".json", "w") as f:
        json.dump(dict(headline=headline, workloads=rows, router=router), f, indent=1)
    names = {1: "q4_0_gemv K=512 N=256", 2: "q4_0_gemv K=4096 N=4096",
             3: "fused_rmsnorm_q4k_gemv K=3584 N=18944", 4: "fused_gate_up_q4k_gemv K=4096 N=14336x2",
             5: "moe_q4_gemv E=64 top6 N=1408 K=2048",
             6: "moe_q4_gemv_down E=64 top6 N=2048 K=1408",
             7: "q4k_gemv (dense down-projection) K=14336 N=4096"}
    lines = ["| workload | M | weight MB | kernel us (median) | GB/s (mean dur) | % of 8 TB/s | "
             "ceiling GB/s | % of ceiling | stream GB/s | % of stream | spread |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = names[r["index"]]
        if r.get("silu"):
            name = name.replace("fused_gate_up_q4k_gemv", "fused_gate_up_silu_q4k_gemv").replace(
                "moe_q4_gemv", "moe_q4_gemv_silu")
        if r.get("norm"):
            name = name.replace("fused_gate_up", "fused_rmsnorm_gate_up")
        if r.get("soa"):
            name = name.replace("q4_0_gemv", "q4_0_gemv_soa")
        if r.get("splitk"):
            name = name.replace("q4_0_gemv", "q4_0_gemv_splitk").replace("q4k_gemv",
                                                                        "q4k_gemv_splitk")
        if r["index"] in (5, 6):
            name += " (%s, %d experts)" % ("all distinct" if r["distinct"] else "seeded ids",
                                           r["unique_experts"])
        lines.append("| %s | %d | %.2f | %.2f | %.0f | %.1f%% | %.0f | %.1f%% | %.0f | %.1f%% | "
                     "%.2f |" % (
                         name, r["M"], r["weight_bytes"] / 1e6, r["kernel"]["median_ms"] * 1e3,
                         r["kernel_gbs"], 100 * r["frac_of_peak"], r["ceiling_gbs"],
                         100 * r["frac_of_ceiling"], r["stream_gbs"], 100 * r["frac_of_stream"],
                         r["kernel"]["spread"]))
    if router:
        lines += ["", "router (moe_router_q4_0) M=%d E=%d K=%d top-%d: %.2f us median, %.2f us "
                  "min (latency-bound: %d bytes of weights)"
                  % (router["M"], router["E"], router["K"], router["top_k"],
                     router["kernel"]["median_ms"] * 1e3, router["kernel"]["min_ms"] * 1e3,
                     router["weight_bytes"])]
    with open(path + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    args = parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_block_quantized_dequant_amd as q4

    q4.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration > 0:
        copy_calibration(torch, dev, args.copy_calibration)
        return
    if args.chain:
        print(json.dumps({"chain": measure_chain(torch, dev)}), flush=True)
        return
    if args.ceilings:
        print(json.dumps({"ceilings": measure_ceilings(torch, dev)}), flush=True)
        return

    head = measure(torch, dev, 4, 1, args.warmup, args.steps)
    print("headline: kernel %.2f us (median %.2f), %.0f GB/s; ceiling %.0f GB/s; wall %.0f GB/s"
          % (head["kernel"]["mean_ms"] * 1e3, head["kernel"]["median_ms"] * 1e3,
             head["kernel_gbs"], head["ceiling_gbs"], head["value_gbs"]), file=sys.stderr,
          flush=True)

    copy_ref = measure_copy(torch, dev, head["weight_bytes"])
    print("device copy of the same bytes: %.2f us, %.0f GB/s read+write"
          % (copy_ref["us_mean"], copy_ref["read_write_gbs"]), file=sys.stderr, flush=True)

    rows = []
    if args.all:
        # (workload, batch sizes, all-distinct expert ids, SiLU-gated single output,
        #  RMSNorm feeding the pair, split-array Q4_0); 6 is the expert
        # down-projection, 7 the dense down-projection (4096 x 14336)
        # (index, Ms, all-distinct ids, SiLU, RMSNorm, split arrays, split-K)
        for index, Ms, dist, silu, norm, soa, sk in (
                (1, (1,), 0, 0, 0, 0, 0), (2, (1, 2, 4, 8, 16), 0, 0, 0, 0, 0),
                (2, (4, 8, 16), 0, 0, 0, 0, 1), (2, (1, 2, 4, 8), 0, 0, 0, 1, 0),
                (3, (1,), 0, 0, 0, 0, 0), (4, (1, 2, 4, 8, 16), 0, 0, 0, 0, 0),
                (4, (1, 4), 0, 1, 0, 0, 0), (4, (1, 4), 0, 0, 1, 0, 0),
                (4, (1, 4), 0, 1, 1, 0, 0),
                (5, (4,), 0, 0, 0, 0, 0), (5, (4,), 1, 0, 0, 0, 0),
                (5, (4,), 0, 1, 0, 0, 0), (6, (1, 4, 8), 0, 0, 0, 0, 0),
                (7, (1, 4), 0, 0, 0, 0, 0), (7, (4,), 0, 0, 0, 0, 1)):
            for M in Ms:
                r = measure(torch, dev, index, M, args.warmup, args.steps, bool(dist), bool(silu),
                            bool(norm), bool(soa), bool(sk))
                rows.append(r)
                print("workload %d%s%s%s%s%s M=%d: %.2f us, %.0f GB/s (%.1f%% of peak, %.1f%% "
                      "of ceiling, %.1f%% of stream)"
                      % (index, " distinct" if dist else "", " silu" if silu else "",
                         " norm" if norm else "", " soa" if soa else "",
                         " splitk" if sk else "", M,
                         r["kernel"]["median_ms"] * 1e3, r["kernel_gbs"],
                         100 * r["frac_of_peak"], 100 * r["frac_of_ceiling"],
                         100 * r["frac_of_stream"]), file=sys.stderr, flush=True)

    router = None
    if args.all:
        router = measure_router(torch, dev, args.warmup, args.steps)
        print("router M=4 E=64 K=2048 top-6: %.2f us (median)"
              % (router["kernel"]["median_ms"] * 1e3), file=sys.stderr, flush=True)

    cpu = cpu_baseline(args.cpu_seconds) if args.cpu_seconds > 0 else None

    ms_per_step = head["wall_s"] / head["steps"] * 1e3
    line = {
        "metric": METRIC,
        "value": round(head["value_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fused_gate_up_q4k_gemv Q4_K M=1 K=4096 N=14336x2 "
                               "(66,060,288 weight bytes per call; %d rotating copies)"
                               % head["copies"]},
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["kernel_gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["frac_of_peak"], 4),
            "traffic": recorded_traffic(),
            "kernel_us_mean": round(head["kernel"]["mean_ms"] * 1e3, 3),
            "kernel_us_median": round(head["kernel"]["median_ms"] * 1e3, 3),
        },
        "pure_read": {
            "achieved": round(head["ceiling_gbs"], 2),
            "unit": "GB/s",
            "kernel_frac_of_ceiling": round(head["frac_of_ceiling"], 4),
            "stream_achieved": round(head["stream_gbs"], 2),
            "kernel_frac_of_stream": round(head["frac_of_stream"], 4),
            "device_copy_read_write": round(copy_ref["read_write_gbs"], 2),
        },
        "cpu_baseline": cpu,
    }
    if args.all:
        write_report(args.all, rows, line, router)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
