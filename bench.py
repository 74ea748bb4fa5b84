"""Throughput of the simulated-quantization hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The default workload is the dense 8B-class transformer
layer (fused QKV 6144x4096, fused gate/up 28672x4096, down 4096x14336, O
4096x4096, bf16), quantized NVFP4 W4A16.  One step is the whole hot path over
that layer:
  1. grouped tensor scales (one tied group per fused matrix): amax pass + reduce,
  2. grouped QDQ + pack of all four matrices in one launch (bf16 QDQ'd weights
     for the BF16 matmul, packed E2M1 codes + E4M3 block scales for the engine),
  3. the identity STE backward of the upstream gradient of all four matrices
     (one contiguous bf16 buffer -> fp32).
Inputs are resident in HBM before timing starts.  `value` is algorithmic bytes
per step / time per step; the roofline object describes the step's dominant
kernel, timed with HIP events on the stream it runs on.  The CPU baseline is
the oracle (test infrastructure) on a bounded sample of the same workload.

Other workloads: --workload q4k_set (Q4_K grouped QDQ + pack over the layer set
plus a 151936x4096 vocabulary projection) and the ones listed by --help.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
METRIC = "QDQ+pack GB/s (% HBM peak) per format; fused W4A4 QDQ-GEMM TFLOP/s (% MFMA)"


# sources of the streaming QDQ / pack / STE kernels whose traffic profiles/traffic.json records
TRAFFIC_SOURCES = ("qf_device.h", "qf_kernels.h", "qf_quant.hip", "qf_api.cpp")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "fp4_fake_quant_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel_key, launches_per_step):
    """HBM-side bytes per launch of the dominant kernel from the committed counter summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_key)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def _counter_rows(folder):
    import csv
    rows = []
    for root, _, files in os.walk(folder):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    rows += list(csv.DictReader(fh))
    return rows


def pmc_summary(fetch_dir, write_dir, workload):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by the same
    counters of the 1 GiB calibration copy (the last device copy of the run), written to
    profiles/traffic.json under the current kernel-source hash."""
    out = {}
    per = {}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(folder) if r.get("Counter_Name") == counter]
        by_dispatch = {}
        for r in rows:
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            by_dispatch[key] = by_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        copies = sorted((int(d), v) for (d, k), v in by_dispatch.items() if "copyBuffer" in k)
        if not copies:
            raise SystemExit(f"{folder}: no calibration copy dispatch found")
        kib_copy = copies[-1][1]
        scale = (1 << 30) / (kib_copy * 1024.0)           # true bytes per counted byte
        for (d, k), v in by_dispatch.items():
            if "copyBuffer" in k:
                continue
            per.setdefault(k, {}).setdefault(counter, []).append(v * 1024.0 * scale)
        out.setdefault("_calibration", {})[counter] = {"copy_KiB_counted": kib_copy, "scale": scale}
    path = os.path.join(PROFILE_DIR, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    short = {"k_nvfp4_amax": "nvfp4_amax", "k_nvfp4_scale_reduce": "nvfp4_amax", "k_nvfp4<": "nvfp4_qdq_pack",
             "k_mxfp4<": "mxfp4_qdq_pack", "k_q4k<": "q4k_qdq_pack", "k_ste<": "ste_backward"}
    for k, cnt in per.items():
        tag = next((v for s_, v in short.items() if s_ in k), None)
        if tag is None:
            continue
        f = sum(cnt.get("FETCH_SIZE", [0])) / max(1, len(cnt.get("FETCH_SIZE", [1])))
        w = sum(cnt.get("WRITE_SIZE", [0])) / max(1, len(cnt.get("WRITE_SIZE", [1])))
        entry = data.setdefault(f"{workload}:{tag}", {"kernels": {}, "source_hash": kernel_source_hash()})
        entry["source_hash"] = kernel_source_hash()
        entry["kernels"][k] = {"fetch_bytes": round(f), "write_bytes": round(w)}
        entry["bytes_per_launch"] = sum(v["fetch_bytes"] + v["write_bytes"] for v in entry["kernels"].values())
    data["_calibration"] = out["_calibration"]
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps(data, indent=1, sort_keys=True))


def counter_summary(folders):
    """Markdown table: per kernel, the number of dispatches and the average of every counter
    (summed over the counter's hardware instances within a dispatch)."""
    per = {}
    for folder in folders:
        for r in _counter_rows(folder):
            k = r["Kernel_Name"]
            key = (r["Dispatch_Id"], k, r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    table = {}
    for (d, k, c), v in per.items():
        table.setdefault(k, {}).setdefault(c, []).append(v)
    counters = sorted({c for v in table.values() for c in v})
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---" * (len(counters) + 2) + "|")
    for k in sorted(table):
        row = table[k]
        n = max(len(v) for v in row.values())
        cells = [f"{sum(row[c]) / len(row[c]):.4g}" if c in row else "" for c in counters]
        print(f"| `{k[:90]}` | {n} | " + " | ".join(cells) + " |")


# ------------------------------------------------------------ workloads ----
def _no_mark(kernel, edge):
    pass


class DenseLayerNVFP4:
    name = "dense_layer_8b_nvfp4_w4a16"

    def __init__(self, torch, fq):
        import numpy as np
        import workloads
        self.torch, self.fq = torch, fq
        layer = workloads.dense_layer_8b(with_grad=True)
        self.names = list(layer)
        dev = torch.device("cuda")

        def to_dev(b):
            return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

        self.host = layer
        self.W = {n: to_dev(layer[n][0]) for n in self.names}
        self.numel = sum(self.W[n].numel() for n in self.names)
        # one contiguous upstream-gradient buffer for the whole layer (a flat grad buffer)
        self.G = torch.empty(self.numel, dtype=torch.bfloat16, device=dev)
        off = 0
        for n in self.names:
            k = self.W[n].numel()
            self.G[off:off + k].copy_(to_dev(layer[n][1]).reshape(-1))
            off += k
        self.g_latent = torch.empty(self.numel, dtype=torch.float32, device=dev)
        self.Y = {n: torch.empty_like(self.W[n]) for n in self.names}
        self.codes = {n: torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev) for n, w in self.W.items()}
        self.scl = {n: torch.empty((w.shape[0], w.shape[1] // 16), dtype=torch.uint8, device=dev) for n, w in self.W.items()}
        self.amax_items = [dict(x=self.W[n], group=i) for i, n in enumerate(self.names)]
        self.qitems = [dict(x=self.W[n], y=self.Y[n], codes=self.codes[n], scales=self.scl[n], group=i)
                       for i, n in enumerate(self.names)]
        self.ws = torch.empty(fq.qf_nvfp4_tensor_scale_workspace(self.amax_items), dtype=torch.uint8, device=dev)
        self.scales = torch.empty(len(self.names), dtype=torch.float32, device=dev)
        n = self.numel
        # algorithmic bytes: amax reads bf16 (2 B); QDQ+pack reads bf16, writes bf16 + codes
        # (0.5 B) + E4M3 scales (1/16 B); STE reads bf16 and writes fp32
        self.kernels = {
            "nvfp4_amax": 2 * n,
            "nvfp4_qdq_pack": n * (2 + 2 + 0.5 + 1 / 16),
            "ste_backward": n * (2 + 4),
        }
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {
            "workload": self.name,
            "matrices": {k: list(v.shape) for k, v in self.W.items()},
            "elements": n,
            "format": "NVFP4 (E2M1, block 16, E4M3 + FP32 tensor scale tied per fused matrix)",
            "tied_groups": len(self.names),
        }

    def step(self, mark=None):
        fq = self.fq
        t = mark or _no_mark
        t("nvfp4_amax", 0)
        fq.qf_nvfp4_tensor_scale_grouped(self.amax_items, len(self.names), self.scales, None, self.ws)
        t("nvfp4_amax", 1)
        t("nvfp4_qdq_pack", 0)
        fq.qf_qdq_pack_nvfp4_grouped(self.qitems, self.scales)
        t("nvfp4_qdq_pack", 1)
        t("ste_backward", 0)
        fq.qf_ste_backward(self.G, self.g_latent)
        t("ste_backward", 1)

    def cpu_baseline(self, budget_s=15.0):
        """The oracle's full step on the first rows of every matrix, sized to ~budget_s."""
        import numpy as np
        from oracle import nvfp4, ste

        def run(frac):
            t0 = time.perf_counter()
            nbytes = 0.0
            for n in self.names:
                W, G = self.host[n]
                r = max(1, int(W.shape[0] * frac))
                Ws, Gs = W[:r], G[:r]
                s_t = nvfp4.tensor_scale([Ws])
                c, S = nvfp4.quantize(Ws, s_t)
                nvfp4.dequantize(c, S, s_t)
                nvfp4.pack(c, S)
                ste.ste_backward(Gs)
                nbytes += Ws.size * (2 + 4.5625 + 6)
            return time.perf_counter() - t0, nbytes

        dt, nb = run(0.002)
        frac = min(1.0, 0.002 * budget_s / max(dt, 1e-3))
        dt, nb = run(frac)
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's amax + QDQ + pack + STE on the first {frac * 100:.2f}% of rows of each "
                          f"of the four matrices ({nb / 12.5625 / 1e6:.1f} M elements, {dt:.1f} s, numpy, 1 thread)"}


class Q4KSet:
    """Q4_K weight-only QDQ + GGUF-style packing in one grouped launch over the Q4_K set:
    the 256x512 matrix, the four 8B-layer matrices and the 151936x4096 vocabulary
    projection (inputs drawn on the device with the same recipe as the tests' set)."""
    name = "q4k_set_qdq_pack"

    def __init__(self, torch, fq):
        import workloads
        self.torch, self.fq = torch, fq
        self.T = workloads.q4k_set_device(seed=0)
        dev = torch.device("cuda")
        self.items = []
        for n, w in self.T.items():
            y = torch.empty_like(w)
            b = torch.empty((w.shape[0], w.shape[1] // 256, 144), dtype=torch.uint8, device=dev)
            self.items.append(dict(x=w, y=y, codes=b))
        n = sum(w.numel() for w in self.T.values())
        self.numel = n
        self.kernels = {"q4k_qdq_pack": n * (2 + 2 + 144 / 256)}
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {"workload": self.name, "matrices": {k: list(v.shape) for k, v in self.T.items()},
                       "elements": n, "format": "Q4_K (INT4, 32-blocks in 256 super-blocks, 6-bit scales/mins, FP16 d/dmin)"}

    def step(self, mark=None):
        t = mark or _no_mark
        t("q4k_qdq_pack", 0)
        self.fq.qf_qdq_pack_q4k_grouped(self.items)
        t("q4k_qdq_pack", 1)

    rule = "minmax"

    def cpu_baseline(self, budget_s=10.0):
        import numpy as np
        import workloads
        from oracle import q4k
        W = workloads.q4k_set(names=["o"])["o"]
        t0 = time.perf_counter()
        r = 64
        p = q4k.quantize(W[:r], self.rule); q4k.dequantize(p); q4k.pack(p)
        dt = time.perf_counter() - t0
        r = max(64, min(W.shape[0], int(64 * budget_s / max(dt, 1e-3))))
        t0 = time.perf_counter()
        p = q4k.quantize(W[:r], self.rule); q4k.dequantize(p); q4k.pack(p)
        dt = time.perf_counter() - t0
        nb = W[:r].size * (2 + 2 + 144 / 256)
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's Q4_K QDQ + pack ({self.rule} rule) on the first {r} rows of the "
                          f"4096x4096 matrix ({dt:.1f} s)"}


class SteClippedDense:
    """The clipped STE over the dense 8B layer's four matrices (218 M elements): the
    gradient of each latent weight, or +0.0 where the quantizer saturated it, from the
    weight x, the upstream gradient g (N(0,1)) and, for NVFP4, the matrix's tensor scale
    (computed once, before timing).  NVFP4 and MXFP4 (floor rule), four launches each."""
    name = "dense_layer_8b_ste_clipped"

    def __init__(self, torch, fq):
        import workloads
        self.torch, self.fq = torch, fq
        x = workloads.dense_layer_8b_device(seed=0)
        self.mats = []
        n = 0
        for w, g in x.values():
            self.mats.append(dict(x=w, g=g, s=fq.qf_nvfp4_tensor_scale(w),
                                  out=torch.empty(w.shape, dtype=torch.float32, device="cuda")))
            n += w.numel()
        self.numel = n
        # algorithmic bytes: x and g in (bf16), fp32 out
        self.kernels = {"ste_clipped_nvfp4": n * 8.0, "ste_clipped_mxfp4": n * 8.0}
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {"workload": self.name, "elements": n,
                       "formats": "NVFP4 (per-matrix tensor scale), MXFP4 floor rule"}

    def step(self, mark=None):
        fq = self.fq
        t = mark or _no_mark
        t("ste_clipped_nvfp4", 0)
        for m in self.mats:
            fq.qf_ste_backward_clipped_nvfp4(m["g"], m["x"], m["s"], m["out"])
        t("ste_clipped_nvfp4", 1)
        t("ste_clipped_mxfp4", 0)
        for m in self.mats:
            fq.qf_ste_backward_clipped_mxfp4(m["g"], m["x"], m["out"])
        t("ste_clipped_mxfp4", 1)

    def cpu_baseline(self, budget_s=6.0):
        """The oracle's saturation masks and clipped STE (NVFP4 and MXFP4) on the first rows
        of the 4096x4096 O projection."""
        import workloads
        from oracle import mxfp4, nvfp4, ste
        W, G = workloads.dense_layer_8b(names=["o"])["o"]
        s_t = nvfp4.tensor_scale([W])

        def run(r):
            t0 = time.perf_counter()
            ste.ste_backward_clipped(G[:r], nvfp4.saturated(W[:r], s_t))
            ste.ste_backward_clipped(G[:r], mxfp4.saturated(W[:r]))
            return time.perf_counter() - t0

        dt = run(64)
        r = max(64, min(W.shape[0], int(64 * budget_s / max(dt, 1e-3))))
        dt = run(r)
        nb = 2 * r * W.shape[1] * 8.0
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's clipped STE under both FP4 masks on the first {r} rows of the 4096x4096 "
                          f"O projection ({dt:.1f} s, numpy, 1 thread)"}


class Q4KSetMSE(Q4KSet):
    """The Q4_K set under the mse sub-block scale rule (8 candidate scales per sub-block,
    each judged by the sub-block's squared error), one grouped launch."""
    name = "q4k_set_qdq_pack_mse"
    rule = "mse"

    def __init__(self, torch, fq):
        super().__init__(torch, fq)
        self.kernels = {"q4k_qdq_pack_mse": self.kernels["q4k_qdq_pack"]}
        self.config = dict(self.config, workload=self.name, rule="mse (8 candidate scales per sub-block)")

    def step(self, mark=None):
        t = mark or _no_mark
        t("q4k_qdq_pack_mse", 0)
        self.fq.qf_qdq_pack_q4k_rule(self.items, self.fq.QF_Q4K_RULE_MSE)
        t("q4k_qdq_pack_mse", 1)


class DequantDense:
    """Dequant of the dense 8B layer's four matrices (218 M elements) from each packed
    layout back to bf16: NVFP4 (per-matrix tensor scales), MXFP4 and Q4_K, four launches
    per format.  The packed inputs are written once, before timing, by the pack calls."""
    name = "dense_layer_8b_dequant"

    def __init__(self, torch, fq):
        import workloads
        self.torch, self.fq = torch, fq
        x = workloads.dense_layer_8b_device(seed=0)
        dev = torch.device("cuda")
        self.mats = []
        n = 0
        for w, _ in x.values():
            rows, cols = w.shape
            s = fq.qf_nvfp4_tensor_scale(w)
            nc, ns = fq.qf_pack_nvfp4(w, s)
            mc, ms = fq.qf_pack_mxfp4(w)
            qb = fq.qf_pack_q4k(w)
            self.mats.append(dict(rows=rows, cols=cols, s=s, nc=nc, ns=ns, mc=mc, ms=ms, qb=qb,
                                  y=torch.empty((rows, cols), dtype=torch.bfloat16, device=dev)))
            n += w.numel()
        del x
        torch.cuda.empty_cache()
        self.numel = n
        # algorithmic bytes: packed codes + scale bytes (or 144-byte blocks) in, bf16 out
        self.kernels = {
            "dequant_nvfp4": n * (0.5 + 1 / 16 + 2),
            "dequant_mxfp4": n * (0.5 + 1 / 32 + 2),
            "dequant_q4k": n * (144 / 256 + 2),
        }
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {"workload": self.name, "elements": n,
                       "formats": "NVFP4, MXFP4, Q4_K packed layouts -> bf16"}

    def step(self, mark=None):
        fq = self.fq
        t = mark or _no_mark
        t("dequant_nvfp4", 0)
        for m in self.mats:
            fq.qf_dequant_nvfp4(m["nc"], m["ns"], m["s"], m["y"])
        t("dequant_nvfp4", 1)
        t("dequant_mxfp4", 0)
        for m in self.mats:
            fq.qf_dequant_mxfp4(m["mc"], m["ms"], m["y"])
        t("dequant_mxfp4", 1)
        t("dequant_q4k", 0)
        for m in self.mats:
            fq.qf_dequant_q4k(m["qb"], m["rows"], m["cols"], m["y"])
        t("dequant_q4k", 1)

    def cpu_baseline(self, budget_s=10.0):
        """The oracle's unpack + dequantize of all three layouts on the first rows of the
        4096x4096 O projection, packed by the oracle."""
        import workloads
        from oracle import mxfp4, nvfp4, q4k
        W = workloads.dense_layer_8b(names=["o"], with_grad=False)["o"][0]
        s_t = nvfp4.tensor_scale([W])

        def run(r):
            x = W[:r]
            pn = nvfp4.pack(*nvfp4.quantize(x, s_t))
            pm = mxfp4.pack(*mxfp4.quantize(x))
            pq = q4k.pack(q4k.quantize(x))
            t0 = time.perf_counter()
            nvfp4.dequantize(*nvfp4.unpack(*pn), s_t)
            mxfp4.dequantize(*mxfp4.unpack(*pm))
            q4k.dequantize(q4k.unpack(pq))
            return time.perf_counter() - t0

        r = 64
        dt = run(r)
        r = max(64, min(W.shape[0], int(r * budget_s / max(dt, 1e-3))))
        dt = run(r)
        nb = W[:r].size * ((0.5 + 1 / 16 + 2) + (0.5 + 1 / 32 + 2) + (144 / 256 + 2))
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's unpack + dequantize of the three layouts on the first {r} rows of the "
                          f"4096x4096 O projection ({dt:.1f} s)"}


class MXFP4Operands:
    """MXFP4 QDQ + pack of the W4A4 GEMM operands, X 32768x4096 (activations, Student-t
    with outlier columns) and W 14336x4096, one grouped launch."""
    name = "mxfp4_gemm_operands_qdq_pack"

    def __init__(self, torch, fq):
        import workloads
        self.torch, self.fq = torch, fq
        g = workloads.w4a4_gemm_device(seed=0)
        dev = torch.device("cuda")
        self.items = []
        for w in (g["X"], g["W"]):
            self.items.append(dict(x=w, y=torch.empty_like(w),
                                   codes=torch.empty((w.shape[0], w.shape[1] // 2), dtype=torch.uint8, device=dev),
                                   scales=torch.empty((w.shape[0], w.shape[1] // 32), dtype=torch.uint8, device=dev)))
        n = sum(it["x"].numel() for it in self.items)
        self.kernels = {"mxfp4_qdq_pack": n * (2 + 2 + 0.5 + 1 / 32)}
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {"workload": self.name, "matrices": {"X": [32768, 4096], "W": [14336, 4096]}, "elements": n,
                       "format": "MXFP4 (E2M1, block 32, E8M0)"}

    def step(self, mark=None):
        t = mark or _no_mark
        t("mxfp4_qdq_pack", 0)
        self.fq.qf_qdq_pack_mxfp4_grouped(self.items)
        t("mxfp4_qdq_pack", 1)

    rule = "floor"

    def cpu_baseline(self, budget_s=6.0):
        """The oracle's MXFP4 QDQ + pack on the first rows of the activations X (host-drawn
        with the same recipe)."""
        import workloads
        from oracle import mxfp4
        X = workloads.w4a4_gemm(M=4096)["X"]

        def run(r):
            t0 = time.perf_counter()
            c, E = mxfp4.quantize(X[:r], self.rule)
            mxfp4.dequantize(c, E), mxfp4.pack(c, E)
            return time.perf_counter() - t0

        dt = run(64)
        r = max(64, min(X.shape[0], int(64 * budget_s / max(dt, 1e-3))))
        dt = run(r)
        nb = r * X.shape[1] * (2 + 2 + 0.5 + 1 / 32)
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's MXFP4 QDQ + pack ({self.rule} rule) on the first {r} rows of X "
                          f"({dt:.1f} s, numpy, 1 thread)"}


class MXFP4OperandsNoclip(MXFP4Operands):
    """The same operands under the noclip shared-exponent rule (the block maximum is never
    clipped onto 6 X), one grouped launch."""
    name = "mxfp4_gemm_operands_qdq_pack_noclip"

    def __init__(self, torch, fq):
        super().__init__(torch, fq)
        self.kernels = {"mxfp4_qdq_pack_noclip": self.kernels["mxfp4_qdq_pack"]}
        self.config = dict(self.config, workload=self.name, rule="noclip (E = ceil(log2(amax / 6)), at most 252)")

    rule = "noclip"

    def step(self, mark=None):
        t = mark or _no_mark
        t("mxfp4_qdq_pack_noclip", 0)
        self.fq.qf_qdq_pack_mxfp4_rule(self.items, self.fq.QF_MX_RULE_NOCLIP)
        t("mxfp4_qdq_pack_noclip", 1)


class Single256x512:
    """The 256x512 matrix (N(0, 0.02^2) with 131 N(0, 0.5^2) outliers) under each format:
    launch-latency bound, reported in microseconds per call."""
    name = "single_256x512_all_formats"

    def __init__(self, torch, fq):
        import numpy as np
        import workloads
        self.torch, self.fq = torch, fq
        w = workloads.single_256x512()
        dev = torch.device("cuda")

        def to_dev(b):
            return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)

        self.W, self.G = to_dev(w["W"]), to_dev(w["G"])
        self.g = torch.empty(self.G.shape, dtype=torch.float32, device=dev)
        self.items = [dict(x=self.W, group=0)]
        self.ws = torch.empty(fq.qf_nvfp4_tensor_scale_workspace(self.items), dtype=torch.uint8, device=dev)
        self.sc = torch.empty(1, dtype=torch.float32, device=dev)
        self.y = torch.empty_like(self.W)
        self.c = torch.empty((256, 256), dtype=torch.uint8, device=dev)
        self.s16 = torch.empty((256, 32), dtype=torch.uint8, device=dev)
        self.s32 = torch.empty((256, 16), dtype=torch.uint8, device=dev)
        self.b = torch.empty((256, 2, 144), dtype=torch.uint8, device=dev)
        n = self.W.numel()
        self.kernels = {"nvfp4_tensor_scale": 2 * n, "nvfp4_qdq_pack": n * 4.5625, "mxfp4_qdq_pack": n * 4.53125,
                        "q4k_qdq_pack": n * 4.5625, "ste_backward": 6 * n}
        self.bytes_per_step = sum(self.kernels.values())
        self.config = {"workload": self.name, "matrices": {"W": [256, 512]}, "elements": n}

    def step(self, mark=None):
        fq = self.fq
        t = mark or _no_mark
        t("nvfp4_tensor_scale", 0)
        fq.qf_nvfp4_tensor_scale(self.W, self.sc, None, self.ws)
        t("nvfp4_tensor_scale", 1)
        t("nvfp4_qdq_pack", 0)
        fq.qf_qdq_pack_nvfp4(self.W, self.sc, self.y, self.c, self.s16)
        t("nvfp4_qdq_pack", 1)
        t("mxfp4_qdq_pack", 0)
        fq.qf_qdq_pack_mxfp4(self.W, self.y, self.c, self.s32)
        t("mxfp4_qdq_pack", 1)
        t("q4k_qdq_pack", 0)
        fq.qf_qdq_pack_q4k(self.W, self.y, self.b)
        t("q4k_qdq_pack", 1)
        t("ste_backward", 0)
        fq.qf_ste_backward(self.G, self.g)
        t("ste_backward", 1)

    def controls(self, reps=500):
        """The same step captured once in a HIP graph and replayed: the GPU-side time of its
        six launches without the per-call host overhead."""
        return {"graph_replay": graph_replay(self.torch, self.step, reps, self.bytes_per_step)}

    def cpu_baseline(self, budget_s=5.0):
        """The oracle's whole step (NVFP4 tensor scale, QDQ + pack of all three formats, STE)
        on the 256x512 matrix, repeated for about budget_s."""
        import workloads
        from oracle import mxfp4, nvfp4, q4k, ste
        w = workloads.single_256x512()
        W, G = w["W"], w["G"]
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s or reps == 0:
            s_t = nvfp4.tensor_scale([W])
            c, S = nvfp4.quantize(W, s_t)
            nvfp4.dequantize(c, S, s_t), nvfp4.pack(c, S)
            c, E = mxfp4.quantize(W)
            mxfp4.dequantize(c, E), mxfp4.pack(c, E)
            p = q4k.quantize(W)
            q4k.dequantize(p), q4k.pack(p)
            ste.ste_backward(G)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        return {"value": round(dt * 1e6, 1), "unit": "us per step", "cores": 1, "kind": "oracle",
                "GB/s": self.bytes_per_step / dt / 1e9,
                "sample": f"the oracle's whole step on the 256x512 matrix, {reps} repetitions (numpy, 1 thread)"}


MFMA_BF16_PEAK_TFS = 2516.6     # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz (dense)


class W4A4GemmMXFP4:
    """Y = QDQ(X) . QDQ(W)^T, X 32768x4096 (Student-t activations with outlier columns),
    W 14336x4096, MXFP4 on both operands, through qf_linear_forward_mxfp4: the streaming
    QDQ of X and of W into bf16 buffers, then the BF16 MFMA GEMM on them (bit for bit the
    fused kernel's result, which is timed among the controls)."""
    name = "w4a4_mxfp4_gemm"

    def __init__(self, torch, fq):
        import workloads
        self.torch, self.fq = torch, fq
        g = workloads.w4a4_gemm_device(seed=0)
        self.X, self.W = g["X"], g["W"]
        self.M, self.K = self.X.shape
        self.N = self.W.shape[0]
        self.Y = torch.empty((self.M, self.N), dtype=torch.bfloat16, device="cuda")
        self.Xq, self.Wq = torch.empty_like(self.X), torch.empty_like(self.W)
        self.flop = 2.0 * self.M * self.N * self.K
        # per kernel: algorithmic bytes of the QDQ passes (bf16 in, bf16 out), flop of the GEMM
        self.kernels = {"mxfp4_qdq_x": 4.0 * self.M * self.K, "mxfp4_qdq_w": 4.0 * self.N * self.K,
                        "gemm_bf16_on_qdq_operands": self.flop}
        self.bytes_per_step = self.flop
        self.config = {"workload": self.name, "M": self.M, "N": self.N, "K": self.K,
                       "format": "MXFP4 W4A4 (E2M1, block 32, E8M0): QDQ of X and W once each, then the "
                                 "BF16 MFMA GEMM, fp32 accumulate, bf16 out"}

    def step(self, mark=None):
        fq = self.fq
        if mark is None:
            fq.qf_linear_forward_mxfp4(self.X, self.W, self.Y, Xq=self.Xq, Wq=self.Wq)
            return
        # the three launches the entry point makes, each bracketed on its own
        mark("mxfp4_qdq_x", 0)
        fq.qf_qdq_mxfp4(self.X, self.Xq)
        mark("mxfp4_qdq_x", 1)
        mark("mxfp4_qdq_w", 0)
        fq.qf_qdq_mxfp4(self.W, self.Wq)
        mark("mxfp4_qdq_w", 1)
        mark("gemm_bf16_on_qdq_operands", 0)
        fq.qf_gemm_mxfp4(self.Xq, self.Wq, self.Y, flags=0)
        mark("gemm_bf16_on_qdq_operands", 1)

    def cpu_baseline(self, budget_s=8.0):
        """The oracle's path on a sample: MXFP4 QDQ of the first r rows of X and of W, then
        the float64 BLAS reference product of those rows with the first c rows of W (host-
        drawn with the same recipe); TFLOP/s over 2 r c K of the product and the QDQ time."""
        import os as _os
        import threadpoolctl
        import workloads
        from oracle import gemm, mxfp4
        g = workloads.w4a4_gemm(M=2048, N=2048)
        X, W = g["X"], g["W"]
        K = X.shape[1]

        def run(r):
            t0 = time.perf_counter()
            Xq, Wq = mxfp4.qdq(X[:r]), mxfp4.qdq(W[:r])
            gemm.reference(Xq, Wq)
            return time.perf_counter() - t0

        dt = run(128)
        r = max(128, min(X.shape[0], int(128 * (budget_s / max(dt, 1e-3)) ** 0.5)))
        dt = run(r)
        blas = [i.get("num_threads") for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        return {"value": 2.0 * r * r * K / dt / 1e12, "unit": "TFLOP/s", "cores": blas[0] if blas else None,
                "kind": "oracle", "host_cores": len(_os.sched_getaffinity(0)),
                "sample": f"the oracle's MXFP4 QDQ of {r} rows of X and of W, then the float64 BLAS reference "
                          f"product {r}x{r}x{K} ({dt:.1f} s; numpy, {blas[0] if blas else '?'} BLAS threads)"}

    def controls(self, reps=10):
        """ms of: the fused kernel (QDQ inside the GEMM); the same kernel on the raw operands
        (flags = 0); the same forward under the MXFP4 noclip rule, in two passes and fused; torch.matmul
        (hipBLASLt) on the raw and on the QDQ'd operands; the NVFP4 W4A4 product,
        fused and in two passes (tensor scales of X and W included in the two-pass time and
        timed on their own); the layer's backward (dX = dY . Wq and dW = dY^T . Xq with
        their three transposes; TFLOP/s over both products)."""
        torch = self.torch
        fq = self.fq
        out = {}
        sx, sw = fq.qf_nvfp4_tensor_scale(self.X), fq.qf_nvfp4_tensor_scale(self.W)
        # backward of the quantized linear: an N(0,1) upstream gradient of Y's shape
        gen = torch.Generator(device="cuda").manual_seed(11)
        dY = torch.randn((self.M, self.N), generator=gen, device="cuda").to(torch.bfloat16)
        dX = torch.empty_like(self.X)
        dW = torch.empty_like(self.W)
        bws = torch.empty(fq.qf_linear_backward_workspace(self.M, self.N, self.K), dtype=torch.uint8,
                          device="cuda")
        Xq, Wq = self.Xq, self.Wq                         # MXFP4 QDQ'd by the workload's steps
        Xq_nv, Wq_nv = torch.empty_like(self.X), torch.empty_like(self.W)

        def two_pass_nv():
            fq.qf_nvfp4_tensor_scale(self.X, sx)
            fq.qf_nvfp4_tensor_scale(self.W, sw)
            fq.qf_linear_forward_nvfp4(self.X, self.W, sx, sw, self.Y, Xq=Xq_nv, Wq=Wq_nv)

        noclip = fq.QF_QDQ_A | fq.QF_QDQ_W | fq.QF_MX_NOCLIP
        for name, fn in (("w4a4_mxfp4_fused", lambda: fq.qf_gemm_mxfp4(self.X, self.W, self.Y, flags=3)),
                         ("w4a4_mxfp4_noclip_two_pass",
                          lambda: fq.qf_linear_forward_mxfp4(self.X, self.W, self.Y, flags=noclip, Xq=Xq_nv, Wq=Wq_nv)),
                         ("w4a4_mxfp4_noclip_fused", lambda: fq.qf_gemm_mxfp4(self.X, self.W, self.Y, flags=noclip)),
                         ("gemm_bf16_same_kernel_raw_operands",
                          lambda: fq.qf_gemm_mxfp4(self.X, self.W, self.Y, flags=0)),
                         ("w4a4_nvfp4_fused", lambda: fq.qf_gemm_nvfp4(self.X, self.W, sx, sw, self.Y)),
                         ("w4a4_nvfp4_two_pass", two_pass_nv),
                         ("tensor_scales_nvfp4", lambda: (fq.qf_nvfp4_tensor_scale(self.X, sx),
                                                          fq.qf_nvfp4_tensor_scale(self.W, sw))),
                         ("backward_dx_dw_mxfp4", lambda: fq.qf_linear_backward_mxfp4(self.X, self.W, dY, dX, dW,
                                                                                        ws=bws)),
                         ("torch_matmul_hipblaslt", lambda: torch.matmul(self.X, self.W.t(), out=self.Y)),
                         ("torch_matmul_hipblaslt_qdq_operands", lambda: torch.matmul(Xq, Wq.t(), out=self.Y))):

            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            if name.startswith("tensor_scales"):
                out[name] = {"ms": round(ms, 4)}
                continue
            flop = 2 * self.flop if name.startswith("backward") else self.flop   # dX and dW: two products
            tf = flop / ms / 1e9
            out[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFS, 4)}
        return out


class MoELoRANVFP4:
    """MoE layer share with LoRA: 128 experts, each with a fused gate/up 3072x3072 and a
    down 3072x1536 bf16 base weight and rank-16 adapters.  Per expert, in expert order:
      1. merge M = W + B.A and take the NVFP4 tensor scale of each fused matrix (one tied
         group per expert per matrix),
      2. merge again and NVFP4 QDQ + pack (the QDQ'd bf16 into a bounded scratch that holds
         the experts of one launch; packed codes and E4M3 block scales of every expert
         are kept),
      3. the adapter gradients dA = B^T.G, dB = G.A^T from the upstream gradient G of the
         QDQ'd weight (identity STE).
    `experts_per_launch` experts share one launch of each call.  With merge_scratch=True
    step 1 also stores M in a scratch of the launch's experts and step 2 quantizes M from
    there (same bits; M is written and read once more, W read once less).
    Algorithmic bytes are the method's minimum, 8.5625 per element: W read by each pass
    (2 + 2), the QDQ'd bf16 (2), codes and block scales (0.5625) and G (2) (the adapters
    and their gradients, 0.02 G elements, are not counted).  The scratch form's extra
    traffic (the M write, 2 bytes per element, less nothing: M's read replaces W's) is
    reported next to it, not in the figure.
    The passes of different launches are independent except that a launch's QDQ pass needs
    its tensor scales, and the adapter gradients depend on the inputs only (A, B, G), so a
    timed step runs the gradient passes on a stream of their own (default priority, with a
    workspace of their own) and, with several experts per launch, the QDQ passes on a third
    (each after its launch's scales, through an event); the streams join at the end.  (With
    one expert per launch the per-launch events cost more than the third stream gains:
    5.5 -> 9.3 ms per step.)  The per-kernel timings run everything on one stream."""
    name = "moe_lora_nvfp4"

    def __init__(self, torch, fq, experts_per_launch=1, merge_scratch=False, api="grouped"):
        import workloads
        self.torch, self.fq = torch, fq
        self.api = api
        mo = workloads.MOE
        E, r = mo["experts"], mo["rank"]
        k = experts_per_launch
        assert E % k == 0 and 2 * k <= (64 if api == "experts" else 16)
        x = workloads.moe_experts_device(seed=0)
        dev = torch.device("cuda")
        mats = ("gate_up", "down")
        self.x = x
        scratch = {m: (torch.empty((k,) + tuple(x[m]["W"].shape[1:]), dtype=torch.bfloat16, device=dev)
                       if merge_scratch else None,
                       torch.empty((k,) + tuple(x[m]["W"].shape[1:]), dtype=torch.bfloat16, device=dev)) for m in mats}
        self.scratch = scratch
        self.codes, self.scl, self.dA, self.dB = {}, {}, {}, {}
        for m in mats:
            _, rows, cols = x[m]["W"].shape
            self.codes[m] = torch.empty((E, rows, cols // 2), dtype=torch.uint8, device=dev)
            self.scl[m] = torch.empty((E, rows, cols // 16), dtype=torch.uint8, device=dev)
            self.dA[m] = torch.empty((E, r, cols), dtype=torch.float32, device=dev)
            self.dB[m] = torch.empty((E, rows, r), dtype=torch.float32, device=dev)
        self.tscale = torch.empty(2 * E, dtype=torch.float32, device=dev)
        self.chunks = []
        for c0 in range(0, E, k):
            if api == "experts":
                # one stacked-experts descriptor per matrix: expert e of the call in groups 2e, 2e + 1
                assert not merge_scratch
                descs = [dict(W=x[m]["W"][c0:c0 + k], A=x[m]["A"][c0:c0 + k], B=x[m]["B"][c0:c0 + k],
                              G=x[m]["G"][c0:c0 + k], y=scratch[m][1], codes=self.codes[m][c0:c0 + k],
                              scales=self.scl[m][c0:c0 + k], dA=self.dA[m][c0:c0 + k], dB=self.dB[m][c0:c0 + k],
                              group=j, group_stride=2) for j, m in enumerate(mats)]
                self.chunks.append((fq.LoraExperts(descs), self.tscale[2 * c0: 2 * (c0 + k)]))
                continue
            items = []
            for e in range(c0, c0 + k):
                for j, m in enumerate(mats):
                    items.append(dict(W=x[m]["W"][e], A=x[m]["A"][e], B=x[m]["B"][e], G=x[m]["G"][e],
                                      M=scratch[m][0][e - c0] if merge_scratch else None,
                                      y=scratch[m][1][e - c0],
                                      codes=self.codes[m][e], scales=self.scl[m][e],
                                      dA=self.dA[m][e], dB=self.dB[m][e], group=2 * (e - c0) + j))
            self.chunks.append((fq.LoraBatch(items), self.tscale[2 * c0: 2 * (c0 + k)]))
        self.ws = torch.empty(self.chunks[0][0].workspace_bytes, dtype=torch.uint8, device=dev)
        self.ws_grads = torch.empty(self.chunks[0][0].workspace_bytes, dtype=torch.uint8, device=dev)
        self.experts_per_launch = k
        self.qdq_stream, self.grad_stream = side_streams(torch)
        self.scale_ready = [torch.cuda.Event() for _ in self.chunks]
        n = sum(x[m]["W"].numel() for m in mats)
        self.numel = n
        self.kernels = {"lora_merge_amax": 2.0 * n, "lora_merge_qdq_pack": (2 + 2 + 0.5 + 1 / 16) * n,
                        "lora_adapter_grads": 2.0 * n}
        self.bytes_per_step = sum(self.kernels.values())
        layout = (fq.qf_lora_experts_layout(self.chunks[0][0]) if api == "experts"
                  else fq.qf_lora_layout(self.chunks[0][0]))
        self.config = {"workload": self.name,
                       "experts": E, "matrices_per_expert": {m: list(x[m]["W"].shape[1:]) for m in mats},
                       "rank": r, "elements": n, "experts_per_launch": k,
                       "calls": ("stacked-experts calls (one descriptor per matrix, experts stacked)"
                                 if api == "experts" else "grouped calls (one descriptor per expert matrix)"),
                       "merge_scratch": merge_scratch,
                       "bytes_per_element": 8.5625,
                       "extra_traffic_bytes": int(2 * n) if merge_scratch else 0,
                       "merge_tiles_per_wave": layout[0], "merge_workgroups": layout[1],
                       "qdq_rows_per_unit": layout[4], "qdq_workgroups": layout[5], "gradient_rows_per_workgroup": layout[2],
                       "scratch_bytes": sum(t.numel() * 2 for p in scratch.values() for t in p if t is not None),
                       "streams": ("tensor-scale, QDQ and gradient passes on three streams" if k > 1
                                   else "merge passes and gradient passes on two streams"),
                       "format": "NVFP4 (E2M1, block 16, E4M3 + FP32 tensor scale per expert per fused matrix)"}

    def _scale(self, items, sc, ws):
        if self.api == "experts":
            self.fq.qf_lora_experts_merge_tensor_scale_nvfp4(items, len(sc), sc, None, ws)
        else:
            self.fq.qf_lora_merge_tensor_scale_nvfp4_grouped(items, items.n, sc, None, ws)

    def _qdq(self, items, sc):
        if self.api == "experts":
            self.fq.qf_lora_experts_merge_qdq_pack_nvfp4(items, sc)
        else:
            self.fq.qf_lora_merge_qdq_pack_nvfp4_grouped(items, sc)

    def _grads(self, items, ws):
        if self.api == "experts":
            self.fq.qf_lora_experts_adapter_grads(items, ws=ws)
        else:
            self.fq.qf_lora_adapter_grads_grouped(items, ws=ws)

    def step(self, mark=None):
        fq, ws = self.fq, self.ws
        if mark is None:
            torch = self.torch
            cur = torch.cuda.current_stream()
            self.grad_stream.wait_stream(cur)
            self.qdq_stream.wait_stream(cur)
            three = self.experts_per_launch > 1
            for (items, sc), ready in zip(self.chunks, self.scale_ready):
                self._scale(items, sc, ws)
                if three:
                    ready.record(cur)
                    with torch.cuda.stream(self.qdq_stream):
                        self.qdq_stream.wait_event(ready)
                        self._qdq(items, sc)
                else:
                    self._qdq(items, sc)
                with torch.cuda.stream(self.grad_stream):
                    self._grads(items, self.ws_grads)
            cur.wait_stream(self.qdq_stream)
            cur.wait_stream(self.grad_stream)
            return
        t = mark
        for items, sc in self.chunks:
            t("lora_merge_amax", 0)
            self._scale(items, sc, ws)
            t("lora_merge_amax", 1)
            t("lora_merge_qdq_pack", 0)
            self._qdq(items, sc)
            t("lora_merge_qdq_pack", 1)
            t("lora_adapter_grads", 0)
            self._grads(items, ws)
            t("lora_adapter_grads", 1)

    def controls(self, reps=20):
        """The whole 128-expert step captured once as a HIP graph and replayed (the launch
        overhead of the many small launches of the one-expert-per-launch reading)."""
        return {"graph_replay": graph_replay(self.torch, self.step, reps, self.bytes_per_step)}

    def cpu_baseline(self, budget_s=8.0):
        """The oracle's merge + tensor scale + NVFP4 QDQ + pack + adapter gradients on the first
        rows of expert 0's two matrices (host-drawn with the same recipe)."""
        import workloads
        from oracle import lora, nvfp4
        e0 = workloads.moe_expert(0)

        def run(rows):
            t0 = time.perf_counter()
            nb = 0.0
            for m in ("gate_up", "down"):
                W, A, B, G = e0[m]
                M = lora.merge(W[:rows], A, B[:rows])
                s_t = nvfp4.tensor_scale([M])
                c, S = nvfp4.quantize(M, s_t)
                nvfp4.dequantize(c, S, s_t)
                nvfp4.pack(c, S)
                lora.adapter_grads(G[:rows], A, B[:rows])
                nb += M.size * 8.5625
            return time.perf_counter() - t0, nb

        dt, _ = run(16)
        rows = max(16, min(3072, int(16 * budget_s / max(dt, 1e-3))))
        dt, nb = run(rows)
        return {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"the oracle's merge + tensor scale + QDQ + pack + adapter gradients on the first {rows} "
                          f"rows of expert 0's gate/up and down matrices ({dt:.1f} s, numpy, 1 thread)"}


class MoELoRANVFP4x8(MoELoRANVFP4):
    """The same step with 8 experts per launch (the QDQ'd scratch of 8 experts, no merge
    scratch): the MoE share's figure."""
    name = "moe_lora_nvfp4_x8"

    def __init__(self, torch, fq):
        super().__init__(torch, fq, experts_per_launch=8)

    def controls(self, reps=20):
        return {}


class MoELoRANVFP4x32(MoELoRANVFP4):
    """The same step through the stacked-experts calls, 32 experts per call (two
    descriptors, 64 tied groups; 4 calls of each pass per step)."""
    name = "moe_lora_nvfp4_x32"

    def __init__(self, torch, fq):
        super().__init__(torch, fq, experts_per_launch=32, api="experts")

    def controls(self, reps=20):
        return {}


class MoELoRANVFP4x8Scratch(MoELoRANVFP4):
    """8 experts per launch with the merged weights kept in a scratch between the passes."""
    name = "moe_lora_nvfp4_x8_scratch"

    def __init__(self, torch, fq):
        super().__init__(torch, fq, experts_per_launch=8, merge_scratch=True)

    def controls(self, reps=20):
        return {}


_SIDE = []


def side_streams(torch):
    """The two default-priority side streams of the MoE steps, created once per process.
    The runtime binds streams to a few hardware queues as they are first used; streams made
    per workload, or first used after other side streams (graph captures make their own),
    could share a queue with the default stream or with each other and run their passes
    one after another instead of side by side.  main() creates and uses these first."""
    if not _SIDE:
        _SIDE.extend((torch.cuda.Stream(), torch.cuda.Stream()))
        # a first command on each: the runtime binds a stream to its hardware queue on first use
        for st in _SIDE:
            with torch.cuda.stream(st):
                torch.zeros(1, device="cuda")
        torch.cuda.synchronize()
    return _SIDE[0], _SIDE[1]


def graph_replay(torch, step, reps, nbytes):
    """us per step of `step` captured once in a HIP graph (on a side stream) and replayed."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / reps
    del graph
    return {"us_per_step": round(us, 2), "replays": reps, "GB/s": round(nbytes / us / 1e3, 1)}


WORKLOADS = {c.name: c for c in (DenseLayerNVFP4, Q4KSet, MXFP4Operands, MXFP4OperandsNoclip, Single256x512,
                                 W4A4GemmMXFP4,
                                 MoELoRANVFP4, MoELoRANVFP4x8, MoELoRANVFP4x32, MoELoRANVFP4x8Scratch, DequantDense,
                                 SteClippedDense, Q4KSetMSE)}
# measured next to the headline workload in a default run (fewer steps each)
SECONDARY = [MXFP4Operands.name, MXFP4OperandsNoclip.name, Q4KSet.name, Single256x512.name, W4A4GemmMXFP4.name,
             MoELoRANVFP4x32.name, MoELoRANVFP4x8.name, MoELoRANVFP4.name, MoELoRANVFP4x8Scratch.name,
             DequantDense.name,
             SteClippedDense.name, Q4KSetMSE.name]


FLUSH_BYTES = 512 << 20      # an untimed write of this size before each flushed iteration
FLUSH_ITERS = 20


_SPIN_CYCLES_PER_MS = None


def gpu_backlog(torch, ms):
    """Keep the current stream busy for about `ms` milliseconds (torch's one-wave spin
    kernel, calibrated once against HIP events), so that work enqueued behind it finds
    the GPU already loaded."""
    global _SPIN_CYCLES_PER_MS
    if _SPIN_CYCLES_PER_MS is None:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(min(ms, 2000.0) * _SPIN_CYCLES_PER_MS))


def measure(torch, wl, steps, warmup, flush_iters=FLUSH_ITERS):
    """(ms per step over `steps` back-to-back steps, per-kernel dict, flushed dict).

    Per-kernel durations come from a second pass of `steps` steps with a HIP event pair
    around every launch (events add a few microseconds between kernels, so they stay out
    of the headline loop), queued behind a spin kernel so that the GPU never waits for the
    host inside a pair; the events sit on torch's current stream, where the library
    launches.  The flushed figures time `flush_iters` further steps one at a time, each
    after an untimed 512 MiB device write that evicts the 256 MB memory-side cache, and
    report the median and the minimum (per step, and per kernel from a second such pass
    with the per-launch events)."""
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    pairs = {k: [] for k in wl.kernels}

    def mark(kernel, edge):
        if edge == 0:
            pairs[kernel].append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        pairs[kernel][-1][edge].record()

    # Enqueueing a step with an event pair around every launch can take the host longer
    # than the GPU needs for the step; the GPU then idles inside an event pair while the
    # host prepares the next launch, and that gap would be booked to the kernel.  So the
    # marked steps are queued behind a spin kernel that lasts longer than their enqueue:
    # a first marked pass measures the host's enqueue time, the second is the timed one.
    t0 = time.perf_counter()
    for _ in range(steps):
        wl.step(mark)
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    for k in pairs:
        pairs[k] = []
    gpu_backlog(torch, 1.5 * host_ms + 2.0)
    for _ in range(steps):
        wl.step(mark)
    torch.cuda.synchronize()
    kern = {}
    for k, nbytes in wl.kernels.items():
        ms = sum(a.elapsed_time(b) for a, b in pairs[k]) / steps
        kern[k] = {"ms": round(ms, 5), "GB/s": round(nbytes / ms / 1e6, 1),
                   "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": int(nbytes),
                   "launches_per_step": len(pairs[k]) // steps}
    # flushed iterations: median and min of single steps after a cache-evicting write
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    step_ms = []
    for i in range(flush_iters):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wl.step()
        e1.record()
        torch.cuda.synchronize()
        step_ms.append(e0.elapsed_time(e1))
    per_kernel = {k: [] for k in wl.kernels}
    for i in range(flush_iters):
        for k in pairs:
            pairs[k] = []
        gpu_backlog(torch, 3.0 * host_ms / steps + 2.0)
        flush.fill_((i + 7) & 0xFF)
        wl.step(mark)
        torch.cuda.synchronize()
        for k in wl.kernels:
            per_kernel[k].append(sum(a.elapsed_time(b) for a, b in pairs[k]))
    del flush
    med = lambda v: sorted(v)[len(v) // 2]
    flushed = {"iters": flush_iters, "flush_bytes": FLUSH_BYTES,
               "step_ms_median": round(med(step_ms), 5), "step_ms_min": round(min(step_ms), 5),
               "kernels": {k: {"ms_median": round(med(v), 5), "ms_min": round(min(v), 5)}
                           for k, v in per_kernel.items()}}
    return ms_per_step, kern, flushed


def gemm_kernel_figures(wl, kern):
    """Per-kernel figures of the GEMM workload: TFLOP/s for the GEMM, GB/s for the QDQ passes."""
    out = {}
    for k, v in kern.items():
        if k.startswith("gemm"):
            tf = round(wl.flop / v["ms"] / 1e9, 1)
            out[k] = {"ms": v["ms"], "TFLOP/s": tf, "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFS, 4),
                      "launches_per_step": v["launches_per_step"]}
        else:
            out[k] = v
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DenseLayerNVFP4.name, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads of a default run")
    ap.add_argument("--no-controls", action="store_true", help="skip the control timings (GEMM workload; graph replay of the 256x512 case)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one 1 GiB device copy (the counter reference of a rocprofv3 --pmc run)")
    ap.add_argument("--flush-iters", type=int, default=FLUSH_ITERS,
                    help="single steps timed after a 512 MiB cache-evicting write (median and min reported)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc output folders into profiles/traffic.json and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print per-kernel averages of every counter in rocprofv3 --pmc output folders and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}): the hot path here is a "
              "single-GPU kernel set and no multi-GPU run is made", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_fake_quant_amd as fq
    torch.cuda.set_device(0)
    side_streams(torch)                          # before any other stream: hardware queues of their own
    wl = WORKLOADS[args.workload](torch, fq)

    print(f"bench: {wl.name}", file=sys.stderr, flush=True)
    ms_per_step, kern, flushed = measure(torch, wl, args.steps, args.warmup, args.flush_iters)
    dom = max(kern, key=lambda k: kern[k]["ms"])
    gemm = isinstance(wl, W4A4GemmMXFP4)
    if gemm:
        # a contraction: TFLOP/s against the dense BF16 MFMA peak
        kern = gemm_kernel_figures(wl, kern)
        achieved = kern[dom]["TFLOP/s"]
        roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4), "traffic": None}
        value, unit = wl.flop / (ms_per_step / 1e3) / 1e12, "TFLOP/s"
    else:
        achieved = kern[dom]["GB/s"]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(f"{wl.name}:{dom}", 1)}
        value, unit = wl.bytes_per_step / (ms_per_step / 1e3) / 1e9, "GB/s"
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": wl.config,
        "roofline": roofline,
        "kernels": kern,
        "flushed": flushed,
    }
    if hasattr(wl, "controls") and not args.no_controls:
        c = wl.controls()
        if c:
            line["controls"] = c
    if not args.no_cpu_baseline and hasattr(wl, "cpu_baseline"):
        line["cpu_baseline"] = wl.cpu_baseline()
    if args.calibrate_copy:
        # a plain device copy of exactly 1 GiB (read 1 GiB, write 1 GiB): the reference
        # that scales the FETCH_SIZE / WRITE_SIZE counters of a --pmc run to bytes
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == DenseLayerNVFP4.name and not args.no_secondary:
        # the other configurations and formats, each on its own inputs, fewer steps
        del wl
        torch.cuda.empty_cache()
        other = {}
        for name in SECONDARY:
            print(f"bench: {name}", file=sys.stderr, flush=True)
            w2 = WORKLOADS[name](torch, fq)
            ms2, kern2, fl2 = measure(torch, w2, max(5, args.steps // 4), 3, args.flush_iters)
            if isinstance(w2, W4A4GemmMXFP4):
                tf = w2.flop / ms2 / 1e9
                other[name] = {"config": w2.config, "ms_per_step": round(ms2, 5), "TFLOP/s": round(tf, 1),
                               "frac_mfma_bf16": round(tf / MFMA_BF16_PEAK_TFS, 4),
                               "kernels": gemm_kernel_figures(w2, kern2), "flushed": fl2}
            else:
                other[name] = {"config": w2.config, "ms_per_step": round(ms2, 5),
                               "GB/s": round(w2.bytes_per_step / ms2 / 1e6, 1),
                               "frac_hbm": round(w2.bytes_per_step / ms2 / 1e6 / HBM_PEAK_GBS, 4),
                               "kernels": kern2, "flushed": fl2}
            if hasattr(w2, "controls") and not args.no_controls:
                c = w2.controls()
                if c:
                    other[name]["controls"] = c
            if not args.no_cpu_baseline and hasattr(w2, "cpu_baseline"):
                other[name]["cpu_baseline"] = w2.cpu_baseline()
            del w2
            torch.cuda.empty_cache()
        line["per_workload"] = other
        # the metric per format: each QDQ+pack kernel against the HBM peak, and the W4A4 GEMM
        fmt = {"nvfp4": (kern, "nvfp4_qdq_pack"),
               "mxfp4": (other[MXFP4Operands.name]["kernels"], "mxfp4_qdq_pack"),
               "q4k": (other[Q4KSet.name]["kernels"], "q4k_qdq_pack")}
        line["per_format"] = {f: {"kernel": k, "GB/s": d[k]["GB/s"], "frac_hbm": d[k]["frac_hbm"]}
                              for f, (d, k) in fmt.items()}
        g = other[W4A4GemmMXFP4.name]
        line["per_format"]["w4a4_mxfp4_forward"] = {"TFLOP/s": g["TFLOP/s"], "frac_mfma_bf16": g["frac_mfma_bf16"],
                                                    "gemm_kernel": g["kernels"]["gemm_bf16_on_qdq_operands"]}
    print(json.dumps(line))

if __name__ == "__main__":
    main()
