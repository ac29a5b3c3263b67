"""Benchmark of the SC bipolar XNOR matmul hot path on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input
already resident in device memory: quantise + encode the row side X and the
weight side W, classify the rows into stream-length rungs and bucket them,
run the XNOR contraction with K-band partial sums and the fused decode.  The
Sobol table is built once before timing (it is resident, built at layer
load) and its build time is reported separately.

Prints one JSON line.  ``value`` is SC bit-MACs per second,
sum over output elements of D * L (L the element's stream length).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--algo auto|mfma|bitserial] [--no-cpu-baseline]
"""

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SC bit-MACs/s (M*N*D*L_eff) + % of int-VALU/HBM roofline, ViT-L fc1 MP"
DEFAULT_WORKLOAD = "vitl_fc1_mp"

# MI355X published peaks used for the roofline fractions.
PEAK_FP4_TOPS = 10100.0          # dense fp4 MFMA, 10.1 PFLOP/s
PEAK_HBM_GBS = 8000.0            # HBM3E, 8 TB/s
# Vector-ALU bit-serial bound: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz int32
# ops, two ops (bit-select, popcount) per 32 stream positions.
PEAK_VALU_BITMACS = 256 * 4 * 16 * 2.4e9 * 16
# LDS gather bound of the pair-count table form: 32 banks of 4 bytes per CU
# per clock, one 2-byte table entry per lane: 256 x 32 x 2.4 GHz lookups.
PEAK_LDS_GATHERS = 256 * 32 * 2.4e9


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--algo", default="auto",
                    choices=["auto", "mfma", "bitserial", "mfma_persistent", "mfma_onepass", "gather", "mfma_quarter"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="rows for the oracle sample (0 = 2 per worker)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 256 MiB float32 buffer three times (the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    return ap.parse_args()


def copy_calibration():
    """Three plain device copies of 64 Mi float32 (256 MiB): under rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE their counts per dispatch give the factor
    from counter units to bytes."""
    import torch
    a = torch.empty(64 * 1024 * 1024, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": a.numel() * a.element_size(), "copies": 3}), flush=True)


def sources_sha256():
    """SHA-256 of the library's sources (csrc/ and include/), so that a
    profile's counters are used only for the kernels they were taken on."""
    import hashlib
    h = hashlib.sha256()
    dirs = [os.path.join(ROOT, "mixed_precision_quantization_amd", "csrc"), os.path.join(ROOT, "include")]
    for d in dirs:
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".h", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


class TimingEvents:
    """Pairs of HIP timing events recorded on one stream, created before the
    timed steps.  They are created with hipEventDisableSystemFence: an event
    that only times the work between two records needs no system-scope
    fence, so recording one adds no cache writeback or invalidation to the
    stream and leaves the following kernels unperturbed.  Read them after a
    device synchronisation."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)

    def __init__(self, n):
        import ctypes
        self._c = ctypes
        self._lib = ctypes.CDLL("libamdhip64.so")
        self._pairs = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                st = self._lib.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(self.FLAGS))
                if st != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
                pair.append(e)
            self._pairs.append(pair)
        self._used = 0

    def start(self, stream):
        self._check(self._lib.hipEventRecord(self._pairs[self._used][0], self._c.c_void_p(stream.cuda_stream)))

    def stop(self, stream):
        self._check(self._lib.hipEventRecord(self._pairs[self._used][1], self._c.c_void_p(stream.cuda_stream)))
        self._used += 1

    def mean_ms(self):
        out = []
        for a, b in self._pairs[:self._used]:
            ms = self._c.c_float(0.0)
            self._check(self._lib.hipEventElapsedTime(self._c.byref(ms), a, b))
            out.append(ms.value)
        return float(sum(out) / len(out))

    def close(self):
        for pair in self._pairs:
            for e in pair:
                self._lib.hipEventDestroy(e)
        self._pairs = []

    @staticmethod
    def _check(st):
        if st != 0:
            raise RuntimeError(f"HIP event call failed ({st})")


def profiled_traffic(workload, algo, dispatches):
    """HBM bytes of the contraction kernel per timed call from the committed
    rocprofv3 summary of this workload and algo (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy), or None when there is none or the sources have
    changed since it was taken."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"k_*_{workload}.md"))):
        text = open(path).read()
        marker = "```json\n"
        if marker not in text:
            continue
        rec = json.loads(text.split(marker)[-1].split("```")[0])
        if rec.get("workload") != workload or rec.get("algo") != algo:
            continue
        if rec.get("sources_sha256") != sources_sha256():
            return None
        if "fetch_bytes_per_dispatch" not in rec or "write_bytes_per_dispatch" not in rec:
            return None
        return (rec["fetch_bytes_per_dispatch"] + rec["write_bytes_per_dispatch"]) * dispatches
    return None


def git_sha():
    try:
        return subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                              text=True, timeout=10).stdout.strip() or None
    except Exception:
        return None


def work_per_step(plan, M, N, G, heads=0):
    """Algorithmic work of one product: bit-MACs sum_i N * sum_b D_b L[b][rung_i],
    and the paired int8 MACs sum_i N * sum_b D_b ceil(L/2) of the matrix-core form.
    With ``heads`` the rungs are per head: per image, the plan's cuts split
    the heads, and every row of a head runs its head's length."""
    if heads:
        hc = plan.row_cuts(heads)
        cuts = [c * M for c in hc]
        G = G // heads
    else:
        cuts = plan.row_cuts(M)
    cols = plan.band_columns()
    L = plan.band_lengths()
    bitmacs = 0
    paired = 0
    for k in range(plan.n_rungs):
        rows = cuts[k + 1] - cuts[k]
        for b in range(plan.n_bands):
            Db = cols[b + 1] - cols[b]
            bitmacs += rows * Db * L[b][k]
            paired += rows * Db * ((L[b][k] + 1) // 2)
    return bitmacs * N * G, paired * N * G


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


def cpu_baseline(w, A, B, n_rows_req, bitmacs_per_step, seconds=12.0):
    """Time the CPU oracle, as it stands, on a bounded sample of output rows
    of the same workload (all columns, all of D), one worker process per
    core (at most 16).  Rows are taken batch by batch (per-row rungs:
    sampled rows of every rung; per-group workloads: whole groups in order;
    per-head rungs: whole images) until about ``seconds`` of wall time have
    been spent, or ``n_rows_req`` rows when that is given.  A fixed slice
    (the first sorted row of every rung; group 0; image 0's first head) is
    also timed in this process alone, for the one-core rate."""
    import numpy as np
    import oracle as o
    from oracle.pool import OraclePool, workers
    from mixed_precision_quantization_amd.workloads import sample_rows

    okw = dict(p=8, Lmax=256, D=w.D, chunk_d=w.chunk_d, levels=w.levels, fractions=w.fractions,
               n_bands=w.n_bands, tilt=w.tilt, metric=w.metric, mode=w.mode)
    oplan = o.OraclePlan(**okw)
    widths = np.diff(oplan.chunk_bounds(), axis=1).T          # (1, n_chunks)
    nw = workers()
    heads = w.extra.get("heads", 0)
    A3 = A if A.ndim == 3 else A[None]
    B3 = B if B.ndim == 3 else B[None]
    N = B3.shape[1]

    def batches():
        """Lists of (A_rows, rungs, B) jobs with a description of each batch."""
        if heads:
            for img in range(A3.shape[0] // heads):
                hs = slice(img * heads, (img + 1) * heads)
                hr = o.head_rungs(A3[hs], oplan)
                yield [(A3[img * heads + h], np.full(w.M, int(hr["rung"][h])), B3[img * heads + h])
                       for h in range(heads)], f"image {img} (all {heads} heads x {w.M} query rows)"
        elif A3.shape[0] > 1:
            for g in range(A3.shape[0]):
                cls = o.classify(A3[g], oplan)
                yield [(A3[g], cls["rung"], B3[g])], f"group {g} (all {w.M} rows)"
        else:
            cls = o.classify(A3[0], oplan)
            per = max(2, -(-(n_rows_req or 4 * nw) // len(w.levels)))
            for seed in range(11, 10 ** 6):
                pos = sample_rows(w.M, cls["cuts"], per_rung=per, seed=seed)
                if n_rows_req:
                    pos = pos[:n_rows_req]
                rows = cls["order"][pos]
                yield [(A3[0][rows], cls["rung"][rows], B3[0])], f"{len(rows)} sampled rows"

    def one_core_slice():
        if heads:
            hr = o.head_rungs(A3[:heads], oplan)
            return A3[0], np.full(w.M, int(hr["rung"][0])), B3[0], f"image 0 head 0 ({w.M} query rows)"
        cls = o.classify(A3[0], oplan)
        if A3.shape[0] > 1:
            return A3[0], cls["rung"], B3[0], f"group 0 (all {w.M} rows)"
        first = [int(c) for c in cls["cuts"][:-1] if c < w.M]
        rows = cls["order"][first]
        return A3[0][rows], cls["rung"][rows], B3[0], f"the first sorted row of each of {len(rows)} rungs"

    t0 = time.perf_counter()
    bitmacs = 0
    rows_done = 0
    parts = []
    with OraclePool(okw, nw) as pool:
        for jobs, what in batches():
            for out in pool.run(jobs):
                bitmacs += int(np.sum(out["L"] * widths)) * N
                rows_done += out["L"].shape[0]
            parts.append(what)
            if (n_rows_req and rows_done >= n_rows_req) or time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    rate = bitmacs / dt

    A1, r1, B1, what1 = one_core_slice()
    t1 = time.perf_counter()
    out1 = o.rows_product(A1, r1, B1, oplan)
    dt1 = time.perf_counter() - t1
    bm1 = int(np.sum(out1["L"] * widths)) * N

    kind = ("query rows of whole images, each head at its rung" if heads else
            "rows of whole groups" if A3.shape[0] > 1 else
            "output rows of every rung (sorted-position edges plus seeded picks)")
    return {
        "value": rate,
        "unit": "bit-MAC/s",
        "cores": nw,
        "kind": "oracle",
        "sample": f"{rows_done} {kind} in {len(parts)} batches ({parts[0]}, ...) x all {N} columns x all "
                  f"D={w.D}, materialised C-BSG streams, {bitmacs:.3e} bit-MACs in {dt:.1f} s wall incl. "
                  f"classification and quantisation, {nw} worker processes",
        "seconds": dt,
        "host_cpu_count": os.cpu_count(),
        "cpu_model": cpu_model(),
        "one_core": {"value": bm1 / dt1, "unit": "bit-MAC/s", "seconds": dt1, "bit_macs": bm1,
                     "sample": f"{what1} x all {N} columns x all D={w.D}, one process"},
        "full_config_seconds_extrapolated": bitmacs_per_step / rate,
        "full_config_seconds_extrapolated_one_core": bitmacs_per_step / (bm1 / dt1),
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              f"mode: sharded, each GPU would take a block of X rows with a replicated W and exchange only the "
              f"row-metric maximum and quantile cuts", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mixed_precision_quantization_amd import scmp
    from mixed_precision_quantization_amd.workloads import WORKLOADS, draw, draw_bias

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = WORKLOADS[args.workload]
    A_np, B_np = draw(w)
    dev = torch.device("cuda:0")
    A = torch.from_numpy(A_np).to(dev)
    B = torch.from_numpy(B_np).to(dev)
    if A.dim() == 2:
        A, B = A.unsqueeze(0), B.unsqueeze(0)
    G, M, D = A.shape
    N = B.shape[1]
    bias = None
    if w.extra.get("bias"):
        bias = torch.from_numpy(draw_bias(w)).to(dev).reshape(G, N)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    table = scmp.scmp_build_sobol_table(8, 256)
    torch.cuda.synchronize()
    table_ms = (time.perf_counter() - t0) * 1e3
    ranged = bool(w.extra.get("range_mp"))
    plan = scmp.scmp_plan_create(op=w.kind, D=w.D, chunk_d=w.chunk_d, levels=w.levels, fractions=w.fractions,
                                 n_bands=w.n_bands, tilt=w.tilt, mode=w.mode, range_mp=ranged,
                                 range_threshold=w.extra.get("range_threshold", 0.3),
                                 range_group=w.extra.get("range_group", 128))
    nch = plan.n_chunks
    # Every buffer of the step is allocated before timing.
    qA = torch.empty((G, M, D), dtype=torch.int8, device=dev)
    sA = torch.empty((G, M, nch), dtype=torch.float32, device=dev)
    mA = torch.empty((G, M), dtype=torch.float32, device=dev)
    qB = torch.empty((G, N, D), dtype=torch.int8, device=dev)
    sB = torch.empty((G, N, nch), dtype=torch.float32, device=dev)
    pB = torch.empty((G, N, D, table.words), dtype=torch.int32, device=dev) if plan.needs_packed(args.algo) else None
    gh = torch.empty((G, M), dtype=torch.float32, device=dev)
    rg = torch.empty((G, M), dtype=torch.uint8, device=dev)
    pm = torch.empty((G, M), dtype=torch.int32, device=dev)
    th = torch.empty((G, max(plan.n_rungs - 1, 1)), dtype=torch.float32, device=dev)
    heads = w.extra.get("heads", 0)
    if heads:
        # Per-head rungs: one metric, rung and rank per (image, head).
        hm = torch.empty(G, dtype=torch.float32, device=dev)
        gh = torch.empty((G // heads, heads), dtype=torch.float32, device=dev)
        rg = torch.empty((G // heads, heads), dtype=torch.uint8, device=dev)
        pm = torch.empty((G // heads, heads), dtype=torch.int32, device=dev)
        th = torch.empty((G // heads, max(plan.n_rungs - 1, 1)), dtype=torch.float32, device=dev)
    C = torch.empty((G, M, N), dtype=torch.float32, device=dev)
    ws_bytes = scmp.scmp_matmul_workspace_bytes(table, plan, G, M, N, args.algo)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = TimingEvents(args.steps)
    if ranged:
        # Range MP: W's groups are classified once, at load time (the weights
        # are static; the call synchronises); each step quantises W and
        # stores it in level order, then runs one contraction per level.
        _, _, rcols, n_lv = scmp.scmp_range_classify(plan, B[0], stream=stream)
        qBs = torch.empty_like(qB)
        sBs = torch.empty_like(sB)
        pBs = torch.empty_like(pB) if pB is not None else None
        offs = [0, n_lv[0], N]
        wsk = [torch.empty(max(scmp.scmp_matmul_workspace_bytes(table, plan, G, M, max(n, 1), args.algo), 1),
                           dtype=torch.uint8, device=dev) for n in n_lv]

    def gather_into(src, dst):
        scmp.scmp_gather_rows(src, rcols, out=dst, stream=stream)

    def step_range(timed):
        scmp.scmp_quantize_encode(table, plan, A, q_out=qA, scales_out=sA, metric_out=mA, stream=stream)
        scmp.scmp_quantize_encode(table, plan, B, q_out=qB, scales_out=sB, packed_out=pB, want_metric=False,
                                  stream=stream)
        gather_into(qB, qBs)
        gather_into(sB, sBs)
        if pB is not None:
            gather_into(pB, pBs)
        if timed:
            ev.start(stream)
        for k in range(2):
            a0, a1 = offs[k], offs[k + 1]
            if a1 > a0:
                scmp.scmp_matmul_range(table, plan, k, qA, sA, qBs[:, a0:a1], sBs[:, a0:a1], rcols[a0:a1], C,
                                       packedB=None if pBs is None else pBs[:, a0:a1], algo=args.algo,
                                       workspace=wsk[k], stream=stream)
        if timed:
            ev.stop(stream)

    def step(timed):
        scmp.scmp_quantize_encode(table, plan, A, q_out=qA, scales_out=sA, metric_out=mA, stream=stream)
        scmp.scmp_quantize_encode(table, plan, B, q_out=qB, scales_out=sB, packed_out=pB, want_metric=False,
                                  stream=stream)
        perm = group_rung = None
        if heads:
            scmp.scmp_group_max(mA, out=hm, stream=stream)
            scmp.scmp_classify_rows(plan, hm.view(G // heads, heads), ghat_out=gh, rung_out=rg, perm_out=pm,
                                    thresholds_out=th, stream=stream)
            group_rung = rg.view(G)
        elif plan.n_rungs > 1:
            scmp.scmp_classify_rows(plan, mA, ghat_out=gh, rung_out=rg, perm_out=pm, thresholds_out=th,
                                    stream=stream)
            perm = pm
        if timed:
            ev.start(stream)
        scmp.scmp_matmul(table, plan, qA, sA, qB, sB, permA=perm, packedB=pB, algo=args.algo, C_out=C,
                         want_C=True, workspace=ws, bias=bias, group_rung=group_rung, stream=stream)
        if timed:
            ev.stop(stream)

    run = step_range if ranged else step
    for _ in range(args.warmup):
        run(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = ev.mean_ms()
    ev.close()
    if ranged:
        lv = plan.band_lengths()[0]
        bitmacs = G * M * D * (n_lv[0] * lv[0] + n_lv[1] * lv[1])
        paired = G * M * D * (n_lv[0] * ((lv[0] + 1) // 2) + n_lv[1] * ((lv[1] + 1) // 2))
    else:
        bitmacs, paired = work_per_step(plan, M, N, G, heads)
    value = bitmacs / (ms_per_step / 1e3)
    L_eff = bitmacs / (G * M * N * D)

    on_valu = args.algo == "bitserial"
    if args.algo == "gather":
        lookups = G * M * N * D
        achieved = lookups / (kern_ms / 1e3) / 1e9
        roof = {"bound": "lds", "achieved": achieved, "peak": PEAK_LDS_GATHERS / 1e9, "unit": "G lookups/s",
                "frac": achieved / (PEAK_LDS_GATHERS / 1e9), "traffic": None,
                "work": "one 2-byte LDS table lookup per (row, column, index)", "lookups": lookups}
    elif on_valu:
        achieved = bitmacs / (kern_ms / 1e3) / 1e12
        roof = {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_BITMACS / 1e12,
                "unit": "T bit-MAC/s", "frac": achieved / (PEAK_VALU_BITMACS / 1e12), "traffic": None,
                "work": "bit-MACs (D * L per output element), two VALU ops per 32"}
    else:
        # The windowed contraction: per output element and contraction index
        # the exact count needs the row's window of paired positions (the
        # useful multiply-accumulates, recorded by the library's encode
        # pass); the kernel issues, per 128 x 128 tile and index, every
        # 16-position block up to the tile's largest window.  Both are fp4
        # (e2m1) MFMA work, priced at the dense fp4 peak.
        if ranged:
            issued = sum(scmp.scmp_matmul_issued_macs(table, plan, G, M, n, wsk[k], algo=args.algo, stream=stream)
                         for k, n in enumerate(n_lv) if n)
            window = sum(scmp.scmp_matmul_window_macs(table, plan, G, M, n, wsk[k], algo=args.algo, stream=stream)
                         for k, n in enumerate(n_lv) if n)
        else:
            issued = scmp.scmp_matmul_issued_macs(table, plan, G, M, N, ws, algo=args.algo, stream=stream)
            window = scmp.scmp_matmul_window_macs(table, plan, G, M, N, ws, algo=args.algo, stream=stream)
        achieved = 2.0 * window / (kern_ms / 1e3) / 1e12
        issued_rate = 2.0 * issued / (kern_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP4_TOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_FP4_TOPS, "traffic": None,
                "work": "window MACs x 2 per launch: per output element and contraction index the "
                        "half-window ceil(|n1 - n0| / 2) of paired positions the exact count needs "
                        "(unipolar: the prefix n1), summed by the library; priced at the dense fp4 "
                        "(e2m1) MFMA peak, the instruction the kernel runs",
                "window_macs": window, "issued_macs": issued,
                "issued_frac": issued_rate / PEAK_FP4_TOPS,
                "padding_frac": 1.0 - window / issued if issued else None,
                "issued_work": "every 16-position block up to the tile's largest window at each index, "
                               "per 128 x 128 tile (what the matrix cores execute)"}
    # The events bracket one scmp_matmul call: the contraction kernel plus, on
    # the matrix-core path, its encode kernel (k_prep: row and column
    # encodes in one launch), which runs first on the same stream.
    roof["kernel"] = ("scmp_matmul = k_matmul_bitserial" if on_valu else
                      "scmp_matmul = k_pc_tables + k_matmul_gather" if args.algo == "gather"
                      else "scmp_matmul = k_prep (row and column encode) + k_mfma")
    if ranged:
        roof["kernel"] = "two scmp_matmul_range calls (one per level), each " + roof["kernel"].split(" = ")[1]
    roof["traffic"] = profiled_traffic(w.name, args.algo, 2 if ranged else 1)
    roof["traffic_source"] = ("profiles/ summary of this workload (FETCH_SIZE + WRITE_SIZE of the contraction "
                              "kernel per timed call, scaled by a plain copy); null when the library sources "
                              "differ from the profiled ones")
    roof["kernel_ms"] = kern_ms
    # HBM: the call's algorithmic bytes, the int8 operands read once and the
    # float32 output written once.
    alg_bytes = G * (M + N) * D + 4 * G * M * N
    roof["algorithmic_bytes"] = alg_bytes
    roof["hbm_frac"] = alg_bytes / (kern_ms / 1e3) / (PEAK_HBM_GBS * 1e9)
    roof["bitmacs_per_s_kernel"] = bitmacs / (kern_ms / 1e3)

    # Arithmetic of the contraction: integer stream counts, on e2m1 (fp4,
    # exact for these operands) matrix-core operands with float32
    # accumulators, on 32-bit words (bit-serial) or 16-bit table entries.
    if on_valu:
        dtype = "u32 bit-ops"
    elif args.algo == "gather":
        dtype = "u16 table lookups"
    else:
        dtype = "fp4(e2m1)"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "bit-MAC/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "G": G, "M": M, "N": N, "D": D, "levels": list(w.levels),
            "fractions": list(w.fractions) if w.fractions else None, "chunk_d": w.chunk_d,
            "n_bands": w.n_bands, "tilt": w.tilt, "L_eff": L_eff, "algo": args.algo, "mode": w.mode,
            "range_mp": {"threshold": w.extra.get("range_threshold", 0.3), "group": plan.range_group, "rows_per_level": list(n_lv)}
            if ranged else None,
            "bit_macs_per_step": bitmacs,
        },
        "roofline": roof,
        "table_build_ms": table_ms,
        "device": torch.cuda.get_device_name(0),
        "git": git_sha(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, A_np, B_np, args.cpu_rows, bitmacs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
