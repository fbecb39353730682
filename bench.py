"""Benchmark of the block-scaled FP8 GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--settle-seconds S] [--reps R] [--timing eager|graph]
                    [--workload dense|contiguous|masked|masked_graph|bf16_dense|dense_rowb|dense_fp8_out|
                                dense_nn|dense_tn|dense_tt|moe_decode|moe_prefill]
                    [--no-masked] [--no-cpu-baseline]

Default workload ("dense"): the five DeepSeek-V3-shaped dense GEMMs,
M = 4096 with (N, K) in {(2112, 7168), (24576, 1536), (7168, 16384),
(4096, 7168), (7168, 2048)}, N(0, 1) float32 inputs already resident in HBM.
One step = for every shape: per-token FP8 cast of A (1x128 scales),
per-block FP8 cast of B (128x128 scales), and the block-scaled FP8 GEMM
with BF16 output -- the whole hot path, no work skipped.

Prints ONE JSON line.

* `value`: GEMM FLOPs (2*M*N*K summed over the shapes) per second of
  whole-step time over the K timed steps (after untimed settle steps for S
  seconds -- the GPU clock dips for the first milliseconds of sustained load
  -- and W warmup steps).
* `roofline`: the dominant kernel (the FP8 GEMM), timed per GEMM call:
  5 untimed calls, then R calls with HIP events around the call on the
  launch stream; a 1 GiB cache flush (a read of a 1 GiB scratch tensor) runs
  before every timed call, outside the events, so every call starts with
  cold, clean L2s and MALL (a writing flush, whose dirty lines the call
  would then write back, is reported beside it).  The flush keeps the queue
  busy while the call is issued, so the events bracket the kernel alone
  (within 2-4 us of the kernel durations a rocprofv3 kernel trace records).
  `--timing graph` replays a captured hipGraph instead, the protocol of the
  pages' test suite ("DeepGEMM CUDA Graph Compatibility for Masked Grouped
  GEMMs", Verification via Test Suite: graph-mode timing, median); on this
  runtime each replay adds about 10 us of graph-launch work inside the
  events.  `achieved` = the shapes' FLOPs / the sum of their median call
  times; the spread (min, p10, p90, max) is listed per shape, next to the
  warm in-step figure (HIP events around the GEMM calls of the timed steps).
* `masked`: the second half of the metric -- the masked grouped GEMMs
  against HBM bandwidth, by the same protocol: MoE decode (32 experts x 256
  rows, masked_m ~ floor(192 U(0.7, 1.3)), (N, K) = (4096, 7168) and
  (7168, 2048), FP32 scales) and the graph workload (64 experts x 128 rows,
  N 7168, K 2048, always as hipGraph replays: a fresh uniform masked_m is
  written before every replay, outside the events; FP8 with packed UE8M0
  scales and BF16).  GB/s = algorithmic bytes of the draw (B once per
  active expert, A and D over valid rows, scales) / median call time.
* `cpu_baseline`: the CPU oracle timed per configuration on bounded samples
  (about 10-30 s in total), with the host's core count and CPU model.

Other workloads (each run on its own with --workload):
  contiguous   -- MoE prefill: 4 groups x 8192 rows, (N, K) = (4096, 7168) and (7168, 2048)
  masked       -- MoE decode: 32 experts, max_m 256, masked_m ~ floor(192 U(0.7, 1.3)),
                  (N, K) = (4096, 7168) and (7168, 2048); metric GB/s
  masked_graph -- 64 experts, max_m 128, N 7168, K 2048, UE8M0 scales packed by
                  pack_ue8m0_to_int, FP8 and BF16 masked GEMMs replayed as one hipGraph
  bf16_dense   -- the five dense shapes with BF16 operands through bf16_gemm_nt
                  (metric against the 2.5 PFLOP/s BF16 MFMA peak)
  dense_rowb   -- the five dense shapes with one B scale per row of B (B cast per
                  token, scales [N, K/128]), as in the pages' dense example
  dense_fp8_out -- the five dense shapes with FP8 output: the GEMM's BF16 result
                  cast per token to E4M3 in its epilogue (fp8_gemm_nt_fp8_out)
  dense_nn, dense_tn, dense_tt -- the five dense shapes with A stored [K, M] (T) and / or
                  B stored [K, N] (N), through fp8_gemm_nn / _tn / _tt; one step = the
                  GEMMs (the operands are cast and transposed once at set-up)
  moe_decode   -- 768 tokens to 8 of 32 experts: moe_dispatch_masked_fp8 (routing +
                  per-token cast), the masked FP8 GEMM (N 4096, K 7168), moe_combine
  moe_prefill  -- 4096 tokens to 8 of 32 experts: moe_dispatch_contiguous_fp8, the
                  contiguous FP8 GEMM (N 4096, K 7168), moe_combine
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 1 << 30      # cache flush before every timed call (L2 4 MB x 8, MALL 256 MB)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

class DenseWorkload:
    name = "dense_fp8_v3_shapes"

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        self.M = synth.DENSE_V3_M
        self.shapes = list(synth.DENSE_V3_SHAPES)
        self.bufs = []
        for i, (N, K) in enumerate(self.shapes):
            sa, sb = synth.dense_v3_seeds(i)
            xa = torch.from_numpy(synth.normal_f32(sa, (self.M, K))).to(dev)
            xb = torch.from_numpy(synth.normal_f32(sb, (N, K))).to(dev)
            buf = dict(
                xa=xa, xb=xb,
                a=torch.empty((self.M, K), dtype=torch.uint8, device=dev),
                sfa=torch.empty((K // 128, self.M), dtype=torch.float32, device=dev).t(),
                b=torch.empty((N, K), dtype=torch.uint8, device=dev),
                sfb=torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=dev),
                d=torch.empty((self.M, N), dtype=torch.bfloat16, device=dev),
            )
            self.bufs.append(buf)
        self.flops = [2.0 * self.M * N * K for N, K in self.shapes]
        # algorithmic bytes of one GEMM launch: A, B, both scales once, D once
        self.gemm_bytes = [self.M * K + N * K + 4 * (self.M * K // 128 + ((N + 127) // 128) * (K // 128)) + 2 * self.M * N
                           for N, K in self.shapes]

    def step(self, events=None):
        mg = self.mg
        for i, b in enumerate(self.bufs):
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            mg.per_block_cast_to_fp8(b["xb"], b["b"], b["sfb"])
            if events is not None:
                events[i][0].record()
            mg.fp8_gemm_nt(b["a"], b["b"], b["sfa"], b["sfb"], None, b["d"])
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        b = self.bufs[i]
        return lambda: self.mg.fp8_gemm_nt(b["a"], b["b"], b["sfa"], b["sfb"], None, b["d"])

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_DENSE", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes,
                "scales": "fp32 1x128 (A) / 128x128 (B)", "out": "bf16"}


class DenseRowBWorkload(DenseWorkload):
    """The five dense shapes with one B scale per row of B (the per-row b_sf
    of the pages' dense example): B is cast per token like A, its scales
    [N, K/128]; one step = both casts and the GEMM per shape."""
    name = "dense_fp8_v3_shapes_row_b_scales"

    def __init__(self, torch, mg, synth):
        super().__init__(torch, mg, synth)
        for (N, K), buf in zip(self.shapes, self.bufs):
            buf["sfb"] = torch.empty((N, K // 128), dtype=torch.float32, device=buf["xb"].device)
        self.gemm_bytes = [self.M * K + N * K + 4 * (self.M * K // 128 + N * (K // 128)) + 2 * self.M * N
                           for N, K in self.shapes]

    def step(self, events=None):
        mg = self.mg
        for i, b in enumerate(self.bufs):
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            mg.per_token_cast_to_fp8(b["xb"], b["b"], b["sfb"])
            if events is not None:
                events[i][0].record()
            mg.fp8_gemm_nt(b["a"], b["b"], b["sfa"], b["sfb"], None, b["d"])
            if events is not None:
                events[i][1].record()

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_DENSE_ROWB", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes,
                "scales": "fp32 1x128 (A) / 1x128 per row (B)", "out": "bf16"}


class DenseFp8OutWorkload(DenseWorkload):
    """The five dense shapes with FP8 output: fp8_gemm_nt_fp8_out casts the
    BF16 result per token in the GEMM's epilogue (q [M, N] E4M3 and scales
    [M, N/128]); one step = both input casts and the GEMM per shape."""
    name = "dense_fp8_v3_shapes_fp8_out"

    def __init__(self, torch, mg, synth):
        super().__init__(torch, mg, synth)
        for (N, K), buf in zip(self.shapes, self.bufs):
            dev = buf["xa"].device
            del buf["d"]
            buf["q"] = torch.empty((self.M, N), dtype=torch.uint8, device=dev)
            buf["sfq"] = torch.empty((self.M, (N + 127) // 128), dtype=torch.float32, device=dev)
        self.gemm_bytes = [self.M * K + N * K + 4 * (self.M * K // 128 + ((N + 127) // 128) * (K // 128))
                           + self.M * N + 4 * self.M * ((N + 127) // 128) for N, K in self.shapes]

    def step(self, events=None):
        mg = self.mg
        for i, b in enumerate(self.bufs):
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            mg.per_block_cast_to_fp8(b["xb"], b["b"], b["sfb"])
            if events is not None:
                events[i][0].record()
            mg.fp8_gemm_nt_fp8_out(b["a"], b["b"], b["sfa"], b["sfb"], None, b["q"], b["sfq"])
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        b = self.bufs[i]
        return lambda: self.mg.fp8_gemm_nt_fp8_out(b["a"], b["b"], b["sfa"], b["sfb"], None, b["q"], b["sfq"])

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_DENSE_FP8_OUT", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes,
                "scales": "fp32 1x128 (A) / 128x128 (B)", "out": "fp8 e4m3, fp32 1x128 scales (per-token cast fused)"}


class DenseLayoutWorkload(DenseWorkload):
    """The five dense shapes with an operand stored MN-major (the NN, TN and
    TT layouts of the FP8 GEMM): A as [K, M] (TN, TT) and / or B as [K, N]
    (NN, TN), quantized once at set-up (the K-major casts, then a transposed
    copy); one step = the GEMM per shape (fp8_gemm_nn / _tn / _tt)."""

    def __init__(self, torch, mg, synth, layout):
        super().__init__(torch, mg, synth)
        self.layout = layout
        self.name = f"dense_fp8_v3_shapes_{layout}"
        for b in self.bufs:
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            mg.per_block_cast_to_fp8(b["xb"], b["b"], b["sfb"])
            if layout[0] == "t":
                b["a"] = b["a"].t().contiguous()  # [K, M]
            if layout[1] == "n":
                b["b"] = b["b"].t().contiguous()  # [K, N]
            del b["xa"], b["xb"]
        torch.cuda.synchronize()
        self.fn = getattr(mg, f"fp8_gemm_{layout}")

    def step(self, events=None):
        for i, b in enumerate(self.bufs):
            if events is not None:
                events[i][0].record()
            self.fn(b["a"], b["b"], b["sfa"], b["sfb"], None, b["d"])
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        b = self.bufs[i]
        return lambda: self.fn(b["a"], b["b"], b["sfa"], b["sfb"], None, b["d"])

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_DENSE_MN", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes,
                "layout": {"nn": "A [M, K], B [K, N]", "tn": "A [K, M], B [K, N]", "tt": "A [K, M], B [N, K]"}[self.layout],
                "scales": "fp32 1x128 (A) / 128x128 (B)", "out": "bf16", "step": "the GEMMs only (operands cast at set-up)"}


class Bf16DenseWorkload:
    """The five dense shapes with BF16 operands (converted once, outside the
    step) through bf16_gemm_nt; one step = the five GEMMs."""
    name = "dense_bf16_v3_shapes"

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        self.M = synth.DENSE_V3_M
        self.shapes = list(synth.DENSE_V3_SHAPES)
        self.bufs = []
        for i, (N, K) in enumerate(self.shapes):
            sa, sb = synth.dense_v3_seeds(i)
            a = torch.from_numpy(synth.normal_f32(sa, (self.M, K))).to(dev).to(torch.bfloat16)
            b = torch.from_numpy(synth.normal_f32(sb, (N, K))).to(dev).to(torch.bfloat16)
            d = torch.empty((self.M, N), dtype=torch.bfloat16, device=dev)
            self.bufs.append((a, b, d))
        self.flops = [2.0 * self.M * N * K for N, K in self.shapes]
        self.gemm_bytes = [2 * (self.M * K + N * K + self.M * N) for N, K in self.shapes]

    def step(self, events=None):
        for i, (a, b, d) in enumerate(self.bufs):
            if events is not None:
                events[i][0].record()
            self.mg.bf16_gemm_nt(a, b, None, d)
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        a, b, d = self.bufs[i]
        return lambda: self.mg.bf16_gemm_nt(a, b, None, d)

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_BF16_DENSE", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes, "out": "bf16"}


class ContiguousWorkload:
    name = "contiguous_fp8_moe_prefill"

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        c = synth.CONTIG
        self.G, per = c["G"], c["rows_per_group"]
        self.Msum = self.G * per
        self.shapes = list(c["shapes"])
        self.layout = torch.from_numpy(synth.contiguous_layout(self.G, per)).to(dev)
        self.bufs = []
        for si, (N, K) in enumerate(self.shapes):
            xa = torch.from_numpy(synth.normal_f32(c["seed_a"] + 10 * si, (self.Msum, K))).to(dev)
            xb = torch.empty((self.G, N, K), dtype=torch.float32, device=dev)
            for g, chunk in enumerate(synth.normal_f32_chunks(c["seed_b"] + 10 * si, (self.G, N, K))):
                xb[g].copy_(torch.from_numpy(chunk))
            self.bufs.append(dict(
                xa=xa, xb=xb,
                a=torch.empty((self.Msum, K), dtype=torch.uint8, device=dev),
                sfa=torch.empty((K // 128, self.Msum), dtype=torch.float32, device=dev).t(),
                b=torch.empty((self.G, N, K), dtype=torch.uint8, device=dev),
                sfb=torch.empty((self.G, (N + 127) // 128, K // 128), dtype=torch.float32, device=dev),
                d=torch.empty((self.Msum, N), dtype=torch.bfloat16, device=dev)))
        self.flops = [2.0 * self.Msum * N * K for N, K in self.shapes]
        self.gemm_bytes = [self.Msum * K + self.G * N * K + 2 * self.Msum * N for N, K in self.shapes]

    def step(self, events=None):
        mg = self.mg
        for i, b in enumerate(self.bufs):
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            mg.per_block_cast_to_fp8(b["xb"], b["b"], b["sfb"])
            if events is not None:
                events[i][0].record()
            mg.m_grouped_fp8_gemm_nt_contiguous(b["a"], b["b"], b["sfa"], b["sfb"], b["d"], self.layout)
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        b = self.bufs[i]
        return lambda: self.mg.m_grouped_fp8_gemm_nt_contiguous(b["a"], b["b"], b["sfa"], b["sfb"], b["d"],
                                                                self.layout)

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_CONTIGUOUS", self.G, self.Msum, N, K)

    def config(self):
        return {"workload": self.name, "groups": self.G, "rows": self.Msum, "shapes_NK": self.shapes}


class MaskedWorkload:
    name = "masked_fp8_moe_decode"
    uniform_m = None  # every expert's masked_m set to this value instead of the seeded draw

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        c = synth.MASKED
        self.G, self.max_m = c["G"], c["max_m"]
        self.shapes = list(c["shapes"])
        if self.uniform_m is None:
            mm = synth.masked_m_decode(c["seed_m"], self.G)
        else:
            mm = np.full(self.G, self.uniform_m, dtype=np.int32)
        self.mm_host = mm
        self.masked_m = torch.from_numpy(mm).to(dev)
        self.bufs = []
        for si, (N, K) in enumerate(self.shapes):
            xa = torch.from_numpy(synth.normal_f32(c["seed_a"] + 10 * si, (self.G, self.max_m, K))).to(dev)
            b = torch.empty((self.G, N, K), dtype=torch.uint8, device=dev)
            sfb = torch.empty((self.G, (N + 127) // 128, K // 128), dtype=torch.float32, device=dev)
            xb = torch.empty((N, K), dtype=torch.float32, device=dev)
            for g, chunk in enumerate(synth.normal_f32_chunks(c["seed_b"] + 10 * si, (self.G, N, K))):
                xb.copy_(torch.from_numpy(chunk))
                mg.per_block_cast_to_fp8(xb, b[g], sfb[g])  # expert weights: quantized once
            del xb
            self.bufs.append(dict(
                xa=xa, b=b, sfb=sfb,
                a=torch.empty((self.G, self.max_m, K), dtype=torch.uint8, device=dev),
                # M-major per expert (the 256 row scales of a K-block contiguous: eight cache lines
                # per slice of a tile instead of one per row)
                sfa=torch.empty((self.G, K // 128, self.max_m), dtype=torch.float32, device=dev).transpose(1, 2),
                d=torch.empty((self.G, self.max_m, N), dtype=torch.bfloat16, device=dev)))
        rows = int(mm.sum())
        active = int((mm > 0).sum())
        self.flops = [2.0 * rows * N * K for N, K in self.shapes]
        self.gemm_bytes = [active * (N * K + 4 * ((N + 127) // 128) * (K // 128)) + rows * (K + 4 * (K // 128) + 2 * N) + 4 * self.G
                           for N, K in self.shapes]

    def step(self, events=None):
        mg = self.mg
        for i, b in enumerate(self.bufs):
            mg.per_token_cast_to_fp8(b["xa"], b["a"], b["sfa"])
            if events is not None:
                events[i][0].record()
            mg.m_grouped_fp8_gemm_nt_masked(b["a"], b["b"], b["sfa"], b["sfb"], b["d"], self.masked_m, self.max_m)
            if events is not None:
                events[i][1].record()

    def gemm_call(self, i):
        b = self.bufs[i]
        return lambda: self.mg.m_grouped_fp8_gemm_nt_masked(b["a"], b["b"], b["sfa"], b["sfb"], b["d"],
                                                            self.masked_m, self.max_m)

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_MASKED", self.G, self.max_m, N, K)

    def config(self):
        cfg = {"workload": self.name, "experts": self.G, "max_m": self.max_m,
               "sum_masked_m": int(self.mm_host.sum()), "shapes_NK": self.shapes}
        if self.uniform_m is not None:
            cfg["masked_m"] = f"every expert {self.uniform_m}"
        return cfg


class MoeDecodeWorkload:
    """MoE decode on one GPU around the masked GEMM: 768 tokens routed to 8
    of 32 experts (256-row buffers, about 192 rows each), N 4096, K 7168.
    One step = moe_dispatch_masked_fp8 (routing + per-token cast of the
    routed tokens), the masked FP8 GEMM, and moe_combine.  With contig=True
    (MoePrefillWorkload): moe_dispatch_contiguous_fp8, the contiguous FP8
    GEMM and moe_combine on 4096 tokens."""
    name = "moe_decode_dispatch_gemm_combine"
    contig = False
    align = 128  # contiguous regions: row granule (set by --moe-align)

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        c = synth.MOE_PREFILL if self.contig else synth.MOE_DECODE
        T, k, G, N, K = c["T"], c["k"], c["G"], c["N"], c["K"]
        # contiguous layout: one "group" of Mcap rows holding every region
        max_m = -(-(T * k + 255 * G) // 256) * 256 if self.contig else c["max_m"]
        self.T, self.k, self.G, self.max_m, self.N, self.K = T, k, G, max_m, N, K
        self.shapes = [(N, K)]
        topk, w = synth.moe_routing(c["seed_r"], T, G, k)
        self.x = torch.from_numpy(synth.normal_f32(c["seed_x"], (T, K))).to(dev)
        self.topk = torch.from_numpy(topk).to(dev)
        self.w = torch.from_numpy(w).to(dev)
        self.b = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
        self.sfb = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
        xb = torch.empty((N, K), dtype=torch.float32, device=dev)
        for g, chunk in enumerate(synth.normal_f32_chunks(c["seed_b"], (G, N, K))):
            xb.copy_(torch.from_numpy(chunk))
            mg.per_block_cast_to_fp8(xb, self.b[g], self.sfb[g])  # expert weights: quantized once
        del xb
        ga = 1 if self.contig else G
        self.a = torch.empty((ga, max_m, K), dtype=torch.uint8, device=dev)
        # M-major per expert, as for the masked decode workload
        self.sfa = torch.empty((ga, K // 128, max_m), dtype=torch.float32, device=dev).transpose(1, 2)
        self.masked_m = torch.empty((G,), dtype=torch.int32, device=dev)  # contiguous: the counts
        self.layout = torch.empty((max_m // 128,), dtype=torch.int32, device=dev)
        self.slot = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.src = None if self.contig else torch.empty((G, max_m), dtype=torch.int32, device=dev)
        self.d = torch.empty((ga, max_m, N), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        self.step()
        torch.cuda.synchronize()
        mm = self.masked_m.cpu().numpy()
        self.mm_host = mm
        placed = int((self.slot.cpu().numpy() >= 0).sum())
        if self.contig:
            # the GEMM computes every block of every region (padding included)
            rows = int(sum(-(-int(c_) // self.align) * self.align for c_ in mm))
        else:
            rows = int(mm.sum())
        active = int((mm > 0).sum())
        self.flops = [2.0 * rows * N * K]
        self.gemm_bytes = [active * (N * K + 4 * (N // 128) * (K // 128)) + rows * (K + 4 * (K // 128) + 2 * N) + 4 * G]
        # x read once, routing tables, the routed rows written with their scales
        self.dispatch_bytes = 4 * T * K + 2 * 4 * T * k + placed * (K + 4 * (K // 128)) + 4 * G
        self.combine_bytes = placed * 2 * N + 2 * 4 * T * k + 2 * T * N
        self.step_bytes_total = self.dispatch_bytes + self.gemm_bytes[0] + self.combine_bytes
        self.extra_events = []

    def step(self, events=None):
        mg = self.mg
        ev = None
        if events is not None:
            ev = [self.torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
        if self.contig:
            mg.moe_dispatch_contiguous_fp8(self.x, self.topk, self.a[0], self.sfa[0], self.layout, self.masked_m,
                                           self.slot, align=self.align)
        else:
            mg.moe_dispatch_masked_fp8(self.x, self.topk, self.a, self.sfa, self.masked_m, self.slot, self.src)
        if events is not None:
            ev[1].record()
            events[0][0].record()
        if self.contig:
            mg.m_grouped_fp8_gemm_nt_contiguous(self.a[0], self.b, self.sfa[0], self.sfb, self.d[0], self.layout)
        else:
            mg.m_grouped_fp8_gemm_nt_masked(self.a, self.b, self.sfa, self.sfb, self.d, self.masked_m, self.max_m)
        if events is not None:
            events[0][1].record()
            ev[2].record()
        mg.moe_combine(self.d, self.slot, self.w, self.y)
        if events is not None:
            ev[3].record()
            self.extra_events.append(ev)

    def extra(self):
        disp = float(np.mean([e[0].elapsed_time(e[1]) for e in self.extra_events])) * 1e3
        comb = float(np.mean([e[2].elapsed_time(e[3]) for e in self.extra_events])) * 1e3
        return {"dispatch_us": disp, "dispatch_gbs": self.dispatch_bytes / (disp * 1e-6) / 1e9,
                "combine_us": comb, "combine_gbs": self.combine_bytes / (comb * 1e-6) / 1e9,
                "dispatch_bytes": self.dispatch_bytes, "combine_bytes": self.combine_bytes}

    def gemm_call(self, i):
        mg = self.mg
        if self.contig:
            return lambda: mg.m_grouped_fp8_gemm_nt_contiguous(self.a[0], self.b, self.sfa[0], self.sfb, self.d[0],
                                                               self.layout)
        return lambda: mg.m_grouped_fp8_gemm_nt_masked(self.a, self.b, self.sfa, self.sfb, self.d, self.masked_m,
                                                       self.max_m)

    def plan_args(self, i):
        if self.contig:
            return ("DG_KIND_CONTIGUOUS", self.G, self.max_m, self.N, self.K)
        return ("DG_KIND_MASKED", self.G, self.max_m, self.N, self.K)

    def config(self):
        if self.contig:
            return {"workload": self.name, "tokens": self.T, "topk": self.k, "experts": self.G, "rows": self.max_m,
                    "N": self.N, "K": self.K, "routed_pairs": int(self.mm_host.sum()), "region_align": self.align,
                    "step": "moe_dispatch_contiguous_fp8 (count, place, per-token cast), contiguous FP8 GEMM, "
                            "moe_combine"}
        return {"workload": self.name, "tokens": self.T, "topk": self.k, "experts": self.G, "max_m": self.max_m,
                "N": self.N, "K": self.K, "sum_masked_m": int(self.mm_host.sum()),
                "step": "moe_dispatch_masked_fp8 (route + per-token cast), masked FP8 GEMM, moe_combine"}


class MoePrefillWorkload(MoeDecodeWorkload):
    name = "moe_prefill_dispatch_gemm_combine"
    contig = True


class MaskedGraphWorkload:
    """64 experts x 128 rows, N 7168, K 2048: per-token UE8M0 cast of the
    activations, pack_ue8m0_to_int of both scale tensors, the masked FP8 GEMM
    on the packed scales and the masked BF16 GEMM on the same shapes, captured
    once as one hipGraph and replayed with a new masked_m (uniform integers in
    [0, 128]) written into the device tensor before each replay."""
    name = "masked_graph_ue8m0_fp8_and_bf16"

    def __init__(self, torch, mg, synth):
        self.torch, self.mg, self.synth = torch, mg, synth
        dev = torch.device("cuda")
        c = synth.MASKED_GRAPH
        G, max_m, N, K = c["G"], c["max_m"], c["N"], c["K"]
        KB = K // 128
        self.G, self.max_m, self.N, self.K = G, max_m, N, K
        self.shapes = [(N, K), (N, K)]  # FP8 masked, BF16 masked
        self.seed_m = c["seed_m"]
        self.xa = torch.from_numpy(synth.normal_f32(c["seed_a"], (G, max_m, K))).to(dev)
        self.qb = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
        self.sfb = torch.empty((G, N // 128, KB), dtype=torch.float32, device=dev)
        self.b16 = torch.empty((G, N, K), dtype=torch.bfloat16, device=dev)
        xb = torch.empty((N, K), dtype=torch.float32, device=dev)
        for g, chunk in enumerate(synth.normal_f32_chunks(c["seed_b"], (G, N, K))):
            xb.copy_(torch.from_numpy(chunk))
            mg.per_block_cast_to_fp8(xb, self.qb[g], self.sfb[g], True)  # expert weights: quantized once
            self.b16[g].copy_(xb)
        del xb
        self.a16 = self.xa.to(torch.bfloat16)
        self.qa = torch.empty((G, max_m, K), dtype=torch.uint8, device=dev)
        self.sfa = torch.empty((G, max_m, KB), dtype=torch.float32, device=dev)
        self.pa = torch.empty((G, max_m, (KB + 3) // 4), dtype=torch.int32, device=dev)
        self.pb = torch.empty((G, N // 128, (KB + 3) // 4), dtype=torch.int32, device=dev)
        self.d8 = torch.empty((G, max_m, N), dtype=torch.bfloat16, device=dev)
        self.d16 = torch.empty((G, max_m, N), dtype=torch.bfloat16, device=dev)
        self.masked_m = torch.zeros(G, dtype=torch.int32, device=dev)
        self.draw = 0
        self.mm_host = []
        self.flops, self.gemm_bytes = [0.0, 0.0], [0.0, 0.0]
        self.nsteps = 0

        self._calls()  # eager warm-up before capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.graph.capture_begin()
            self._calls()
            self.graph.capture_end()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

    def _calls(self, events=None):
        mg = self.mg
        mg.per_token_cast_to_fp8(self.xa, self.qa, self.sfa, True)
        mg.pack_ue8m0_to_int(self.sfa, self.pa)
        mg.pack_ue8m0_to_int(self.sfb, self.pb)
        if events is not None:
            events[0][0].record()
        mg.m_grouped_fp8_gemm_nt_masked(self.qa, self.qb, self.pa, self.pb, self.d8, self.masked_m, self.max_m)
        if events is not None:
            events[0][1].record()
            events[1][0].record()
        mg.m_grouped_bf16_gemm_nt_masked(self.a16, self.b16, self.d16, self.masked_m, self.max_m)
        if events is not None:
            events[1][1].record()

    def _next_masked_m(self):
        mm = self.synth.masked_m_uniform(self.seed_m + 2 + self.draw, self.G, self.max_m)
        self.draw += 1
        return mm

    def step(self, events=None):
        """One replay of the captured graph with a fresh masked_m."""
        mm = self._next_masked_m()
        self.masked_m.copy_(self.torch.from_numpy(mm))
        self.graph.replay()
        self.mm_host.append(mm)

    def _bytes(self, mm):
        rows, active = int(mm.sum()), int((mm > 0).sum())
        N, K = self.N, self.K
        KB = K // 128
        nb = (N + 127) // 128
        fp8 = active * (N * K + 4 * nb * ((KB + 3) // 4)) + rows * (K + 4 * ((KB + 3) // 4) + 2 * N) + 4 * self.G
        bf16 = active * (2 * N * K) + rows * (2 * K + 2 * N) + 4 * self.G
        return 2.0 * rows * N * K, fp8, bf16

    def step_bytes(self):
        """Mean algorithmic GEMM bytes (FP8 + BF16) per replayed step."""
        return float(np.mean([sum(self._bytes(m)[1:]) for m in self.mm_host]))

    def timing_pass(self, events):
        """Eager pass over the same calls with HIP events around each GEMM
        (events cannot be recorded inside a replay); per-kernel figures come
        from these passes, the step time from the replays."""
        mm = self._next_masked_m()
        self.masked_m.copy_(self.torch.from_numpy(mm))
        self._calls(events)
        f, b8, b16 = self._bytes(mm)
        self.flops[0] += f
        self.flops[1] += f
        self.gemm_bytes[0] += b8
        self.gemm_bytes[1] += b16
        self.nsteps += 1

    def finish(self):
        n = max(self.nsteps, 1)
        self.flops = [f / n for f in self.flops]
        self.gemm_bytes = [b / n for b in self.gemm_bytes]

    def gemm_call(self, i):
        mg = self.mg
        if i == 0:
            return lambda: mg.m_grouped_fp8_gemm_nt_masked(self.qa, self.qb, self.pa, self.pb, self.d8,
                                                           self.masked_m, self.max_m)
        return lambda: mg.m_grouped_bf16_gemm_nt_masked(self.a16, self.b16, self.d16, self.masked_m, self.max_m)

    def plan_args(self, i):
        return ("DG_KIND_MASKED" if i == 0 else "DG_KIND_BF16_MASKED", self.G, self.max_m, self.N, self.K)

    def config(self):
        return {"workload": self.name, "experts": self.G, "max_m": self.max_m, "N": self.N, "K": self.K,
                "mean_sum_masked_m": float(np.mean([m.sum() for m in self.mm_host])) if self.mm_host else 0.0,
                "kernels": ["gemm_kernel FP8 kind (UE8M0 packed scales)", "gemm_kernel BF16 kind"],
                "step": "one hipGraph replay: UE8M0 cast of A, 2 packs, FP8 masked GEMM, BF16 masked GEMM"}


# ---------------------------------------------------------------------------
# timing: one call, eager or as hipGraph replays, with a cold cache
# ---------------------------------------------------------------------------

def _stats(us):
    a = np.sort(np.asarray(us, dtype=np.float64))
    return {"median_us": float(np.median(a)), "min_us": float(a[0]), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "max_us": float(a[-1]), "calls": int(a.size)}


class CallTimer:
    """Times a call with HIP events on the current stream, a 1 GiB flush before
    each timed call (outside the events): eager calls, or replays of the call
    captured once (torch.cuda.graph).

    The flush reads the 1 GiB scratch tensor (a sum): afterwards neither the
    per-XCD L2s nor the 256 MB MALL hold any of the call's operands, and no
    dirty line is left behind.  A flush that writes 1 GiB instead leaves the
    MALL full of dirty lines, whose write-back to HBM the next call then pays
    for out of its own bandwidth; that variant is reported separately
    (write_flush)."""

    def __init__(self, torch, write_flush=False, graph=True):
        self.torch = torch
        self.write_flush = write_flush
        self.graph = graph
        self.flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = None

    def _flush(self):
        if self.write_flush:
            self.flush.fill_(1.0)
        else:
            self.sink = self.flush.sum()

    def capture(self, fn):
        torch = self.torch
        fn()  # eager call first (nothing lazy left for the capture)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time(self, fn, reps, warm=5, before=None):
        """Returns (per-call microseconds, per-call results of before())."""
        torch = self.torch
        g = self.capture(fn) if self.graph else None
        run = g.replay if g is not None else fn
        for _ in range(warm):
            if before is not None:
                before()
            run()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        tags = []
        for e0, e1 in evs:
            if before is not None:
                tags.append(before())
            self._flush()
            e0.record()
            run()
            e1.record()
        torch.cuda.synchronize()
        us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
        del g
        return us, tags


def time_gemms(torch, W, timer, reps):
    """Cold-cache timing of every GEMM call of a workload."""
    out = []
    for i in range(len(W.flops)):
        us, _ = timer.time(W.gemm_call(i), reps)
        out.append(_stats(us))
    return out


# ---------------------------------------------------------------------------
# masked block: the masked grouped GEMMs against HBM
# ---------------------------------------------------------------------------

def masked_block(torch, mg, synth, timer, reps):
    """MoE decode (32 x 256 rows, FP32 scales) and the graph workload (64 x
    128 rows, FP8 UE8M0 and BF16), each GEMM call timed after a cache flush
    (the graph workload always as hipGraph replays)."""
    res = {}
    log("masked block: decode workload (32 experts x 256 rows)")
    Wd = MaskedWorkload(torch, mg, synth)
    Wd.step()  # the per-token casts of A
    torch.cuda.synchronize()
    dec = []
    for i, (N, K) in enumerate(Wd.shapes):
        st = _stats(timer.time(Wd.gemm_call(i), reps)[0])
        st.update({"N": N, "K": K, "algorithmic_bytes": Wd.gemm_bytes[i],
                   "gbs": Wd.gemm_bytes[i] / (st["median_us"] * 1e-6) / 1e9,
                   "tflops": Wd.flops[i] / (st["median_us"] * 1e-6) / 1e12})
        dec.append(st)
    tot_b = float(sum(Wd.gemm_bytes))
    tot_t = sum(s["median_us"] for s in dec) * 1e-6
    res["decode"] = {"workload": Wd.name, "experts": Wd.G, "max_m": Wd.max_m,
                     "sum_masked_m": int(Wd.mm_host.sum()), "scales": "fp32 1x128 (A) / 128x128 (B)",
                     "gbs": tot_b / tot_t / 1e9, "frac": tot_b / tot_t / 1e9 / HBM_PEAK_GBS, "per_shape": dec}
    del Wd
    torch.cuda.empty_cache()

    log("masked block: graph workload (64 experts x 128 rows, FP8 UE8M0 and BF16)")
    Wg = MaskedGraphWorkload(torch, mg, synth)
    draws = []

    def fresh():
        mm = Wg._next_masked_m()
        Wg.masked_m.copy_(torch.from_numpy(mm))
        draws.append(mm)
        return mm

    graph = {}
    eager, timer.graph = not timer.graph, True  # this workload is timed as graph replays in either mode
    for i, kind in enumerate(("fp8_ue8m0", "bf16")):
        us, tags = timer.time(Wg.gemm_call(i), reps, before=fresh)
        b = np.array([Wg._bytes(m)[1 + i] for m in tags])
        gbs = b / (np.asarray(us) * 1e-6) / 1e9
        st = _stats(us)
        st.update({"gbs_median": float(np.median(gbs)), "gbs_p10": float(np.percentile(gbs, 10)),
                   "gbs_p90": float(np.percentile(gbs, 90)), "mean_algorithmic_bytes": float(b.mean()),
                   "mean_sum_masked_m": float(np.mean([m.sum() for m in tags]))})
        st["frac"] = st["gbs_median"] / HBM_PEAK_GBS
        graph[kind] = st
    timer.graph = not eager
    res["graph"] = {"workload": Wg.name, "experts": Wg.G, "max_m": Wg.max_m, "N": Wg.N, "K": Wg.K,
                    "masked_m": "uniform integers 0..128, a fresh draw before every replay", **graph}
    del Wg
    torch.cuda.empty_cache()
    res["roofline"] = {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "decode_frac": res["decode"]["frac"],
                       "graph_fp8_ue8m0_frac": graph["fp8_ue8m0"]["frac"], "graph_bf16_frac": graph["bf16"]["frac"]}
    return res


# ---------------------------------------------------------------------------
# recorded HBM traffic of the GEMM kernel (rocprofv3 PMC), valid for one source
# ---------------------------------------------------------------------------

def recorded_traffic(workload):
    """Bytes per launch of the dominant GEMM kernel (HBM-side reads + writes, calibrated
    against a 1 GiB copy) from profiles/gemm_traffic.txt, or None when the
    record is missing or was taken on a different version of the kernel
    source."""
    import hashlib

    rec_path = os.path.join(ROOT, "profiles", "gemm_traffic.txt")
    src_path = os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "csrc", "gemm.hip")
    if not os.path.exists(rec_path):
        return None
    rec = {}
    for line in open(rec_path):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        rec[k.strip()] = v.strip()
    cur = hashlib.sha256(open(src_path, "rb").read()).hexdigest()[:16]
    if rec.get("gemm_source_sha256_16") != cur:
        return None
    try:
        return float(rec[f"{workload}_fetch_bytes_per_launch"]) + float(rec[f"{workload}_write_bytes_per_launch"])
    except KeyError:
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle per configuration on bounded samples
# ---------------------------------------------------------------------------

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_cpu_baseline():
    """The oracle (numpy float64; the per-128-block products go through the
    BLAS matmul, the rest is single-threaded numpy) on a bounded sample of
    every configuration.  Returns the dense sample's TFLOP/s as `value`."""
    import oracle
    from moe_grouped_gemm_x128_amd import synth

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    per = {}

    def timed(fn):
        t = time.perf_counter()
        fn()
        return time.perf_counter() - t

    # dense small, whole: quantize both operands + GEMM
    c = synth.DENSE_SMALL
    xa, xb = synth.normal_f32(c["seed_a"], (c["M"], c["K"])), synth.normal_f32(c["seed_b"], (c["N"], c["K"]))

    def run_small():
        a, sfa = oracle.per_token_cast_to_fp8(xa)
        b, sfb = oracle.per_block_cast_to_fp8(xb)
        oracle.fp8_gemm_nt(a, b, sfa, sfb)

    s = timed(run_small)
    f = 2.0 * c["M"] * c["N"] * c["K"]
    per["dense_small"] = {"seconds": s, "gflops": f / s / 1e9, "sample": "whole (128 x 256 x 512)"}

    # dense V3 shapes: 256 rows of A x 2048 rows of B per shape, full K
    rows_a, rows_b = 256, 2048
    flops, spent = 0.0, 0.0
    for i, (N, K) in enumerate(synth.DENSE_V3_SHAPES):
        sa, sb = synth.dense_v3_seeds(i)
        ra = synth.normal_f32(sa, (rows_a, K))
        rb = synth.normal_f32(sb, (min(rows_b, N), K))

        def run():
            a, sfa = oracle.per_token_cast_to_fp8(ra)
            b, sfb = oracle.per_block_cast_to_fp8(rb)
            oracle.fp8_gemm_nt(a, b, sfa, sfb)

        spent += timed(run)
        flops += 2.0 * rows_a * min(rows_b, N) * K
    per["dense_v3"] = {"seconds": spent, "gflops": flops / spent / 1e9,
                       "sample": f"per shape: {rows_a} rows of A x {rows_b} rows of B, full K, quantize + GEMM"}
    dense_tflops = flops / spent / 1e12

    # contiguous prefill: one 128-row block per group, 1024 rows of each group's B
    cc = synth.CONTIG
    G = cc["G"]
    flops, spent = 0.0, 0.0
    for si, (N, K) in enumerate(cc["shapes"]):
        xa = synth.normal_f32(cc["seed_a"] + 10 * si, (G * 128, K))
        xb = synth.normal_f32(cc["seed_b"] + 10 * si, (G, 1024, K))
        layout = np.arange(G, dtype=np.int32)

        def run():
            a, sfa = oracle.per_token_cast_to_fp8(xa)
            b, sfb = oracle.per_block_cast_to_fp8(xb)
            oracle.m_grouped_fp8_gemm_nt_contiguous(a, b, sfa, sfb, layout)

        spent += timed(run)
        flops += 2.0 * G * 128 * 1024 * K
    per["contiguous_prefill"] = {"seconds": spent, "gflops": flops / spent / 1e9,
                                 "sample": "per shape: one 128-row block per group x 1024 rows of its B"}

    # masked decode: 2 experts (their masked_m rows) x 1024 rows of B
    cm = synth.MASKED
    mm = synth.masked_m_decode(cm["seed_m"], cm["G"])[:2]
    flops, spent = 0.0, 0.0
    for si, (N, K) in enumerate(cm["shapes"]):
        xa = synth.normal_f32(cm["seed_a"] + 10 * si, (2, cm["max_m"], K))
        xb = synth.normal_f32(cm["seed_b"] + 10 * si, (2, 1024, K))

        def run():
            a, sfa = oracle.per_token_cast_to_fp8(xa)
            b, sfb = oracle.per_block_cast_to_fp8(xb)
            oracle.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, mm, cm["max_m"])

        spent += timed(run)
        flops += 2.0 * int(mm.sum()) * 1024 * K
    per["masked_decode"] = {"seconds": spent, "gflops": flops / spent / 1e9,
                            "sample": "per shape: 2 experts (their masked_m rows) x 1024 rows of B"}

    # masked graph: 4 experts, FP8 with UE8M0 scales and BF16, 1024 rows of B
    cg = synth.MASKED_GRAPH
    mm = synth.masked_m_uniform(cg["seed_m"] + 2, cg["G"], cg["max_m"])[:4]
    xa = synth.normal_f32(cg["seed_a"], (4, cg["max_m"], cg["K"]))
    xb = synth.normal_f32(cg["seed_b"], (4, 1024, cg["K"]))

    def run_g():
        a, sfa = oracle.per_token_cast_to_fp8(xa, use_ue8m0=True)
        b, sfb = oracle.per_block_cast_to_fp8(xb, use_ue8m0=True)
        oracle.m_grouped_fp8_gemm_nt_masked(a, b, sfa, sfb, mm, cg["max_m"])
        ab = synth.bf16_bits_from_f32(xa)
        bb = synth.bf16_bits_from_f32(xb)
        oracle.m_grouped_bf16_gemm_nt_masked(ab, bb, mm, cg["max_m"])

    s = timed(run_g)
    f = 2 * 2.0 * int(mm.sum()) * 1024 * cg["K"]
    per["masked_graph"] = {"seconds": s, "gflops": f / s / 1e9,
                           "sample": "4 experts (their masked_m rows) x 1024 rows of B, FP8 UE8M0 + BF16"}
    total = sum(v["seconds"] for v in per.values())
    return {
        "value": dense_tflops,
        "unit": "TFLOPS",
        "cores": blas_threads,
        "kind": "oracle",
        "sample": (f"dense V3 shapes, {rows_a} rows of A x {rows_b} rows of B per shape, quantize + block-scaled "
                   f"GEMM in float64 (numpy; the block products on {blas_threads} BLAS threads, the rest "
                   f"single-threaded); every configuration under per_config; {total:.1f} s of oracle time"),
        "host_cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "per_config": per,
        "seconds": total,
    }


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense",
                    choices=["dense", "contiguous", "masked", "masked_graph", "bf16_dense", "dense_rowb",
                             "dense_fp8_out", "dense_nn", "dense_tn", "dense_tt", "moe_decode", "moe_prefill"])
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed steps run for this long before the warmup steps, so that the timed steps see "
                         "the GPU's steady sustained clock rather than the dip of its first milliseconds under load")
    ap.add_argument("--reps", type=int, default=25, help="timed calls per GEMM call (kernel timing)")
    ap.add_argument("--timing", choices=("graph", "eager"), default="eager",
                    help="kernel timing: eager calls (default), or replays of a captured hipGraph (each replay "
                         "adds about 10 us of graph-launch work inside the events on this runtime); the masked "
                         "graph workload is always timed as graph replays")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record HIP events around the GEMM calls of one timed step in this many (plus the last)")
    ap.add_argument("--moe-align", type=int, choices=(128, 256), default=128,
                    help="moe_prefill: row granule of the experts' regions in the contiguous layout")
    ap.add_argument("--masked-m", type=int, default=None,
                    help="masked: set every expert's masked_m to this many rows (1..256) instead of the seeded "
                         "draw, to time the decode GEMM against the number of valid rows")
    ap.add_argument("--no-masked", action="store_true", help="dense: skip the masked grouped GEMM block")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 1 GiB device copy (calibrates rocprofv3 FETCH/WRITE_SIZE counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(expert/column sharding across GPUs is a design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_grouped_gemm_x128_amd as mg
    from moe_grouped_gemm_x128_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    mg.dgmi_init()

    log(f"setting up workload {args.workload}")
    MoeDecodeWorkload.align = args.moe_align
    if args.masked_m is not None:
        if args.workload != "masked" or not 1 <= args.masked_m <= 256:
            print("--masked-m takes 1..256 rows, with --workload masked", file=sys.stderr)
            sys.exit(2)
        MaskedWorkload.uniform_m = args.masked_m
    if args.workload in ("dense_nn", "dense_tn", "dense_tt"):
        W = DenseLayoutWorkload(torch, mg, synth, args.workload[-2:])
    else:
        W = {"dense": DenseWorkload, "contiguous": ContiguousWorkload, "masked": MaskedWorkload,
             "masked_graph": MaskedGraphWorkload, "bf16_dense": Bf16DenseWorkload,
             "dense_rowb": DenseRowBWorkload, "dense_fp8_out": DenseFp8OutWorkload,
             "moe_decode": MoeDecodeWorkload, "moe_prefill": MoePrefillWorkload}[args.workload](torch, mg, synth)
    torch.cuda.synchronize()

    # Power-state settle: under sustained GEMM load the clock dips for the first
    # few milliseconds and recovers within a few tens of milliseconds; steps run
    # here are not timed and not counted.
    settle_steps = 0
    t_settle = time.perf_counter() + args.settle_seconds
    while time.perf_counter() < t_settle:
        W.step()
        settle_steps += 1
        if settle_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"settle done ({settle_steps} steps in {args.settle_seconds:.2f} s)")
    for _ in range(args.warmup):
        W.step()
    torch.cuda.synchronize()
    graph_wl = hasattr(W, "timing_pass")
    if graph_wl:
        W.mm_host = []  # count the timed replays only
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    nshape = len(W.flops)
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nshape)]
              for _ in range(args.steps)]
    # HIP events around the GEMM calls of one timed step in `event_every` (and
    # of the last step): an event record is a marker that the next kernel waits
    # behind, so recording them on every step would add gaps to the step
    timed = [s for s in range(args.steps) if s % args.event_every == args.event_every - 1]
    if args.steps - 1 not in timed:
        timed.append(args.steps - 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        W.step(events[s] if (s in timed and not graph_wl) else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("timed region done")
    if graph_wl:
        timed = list(range(args.steps))
        for s in timed:
            W.timing_pass(events[s])
        torch.cuda.synchronize()
        W.finish()

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # warm in-step GEMM durations (ms) from the timed steps' events
    step_ms = [float(np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in timed])) for i in range(nshape)]
    ms_per_step = wall * 1e3 / args.steps
    total_flops = float(sum(W.flops))
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    # kernel timing (cold cache, median)
    log(f"{args.timing} timing of the GEMM calls ({args.reps} calls each, 1 GiB flush before each)")
    timer = CallTimer(torch, graph=args.timing == "graph")
    if graph_wl:
        kt = []
        for i in range(nshape):
            us, tags = timer.time(W.gemm_call(i), args.reps,
                                  before=lambda: (W.masked_m.copy_(torch.from_numpy(W._next_masked_m())), None)[1])
            kt.append(_stats(us))
    else:
        kt = time_gemms(torch, W, timer, args.reps)
        wtimer = CallTimer(torch, write_flush=True, graph=args.timing == "graph")
        wflush = [k["median_us"] for k in time_gemms(torch, W, wtimer, args.reps)]
        del wtimer
        for k, w in zip(kt, wflush):
            k["write_flush_median_us"] = w
    gemm_us = [k["median_us"] for k in kt]

    is_masked = args.workload in ("masked", "masked_graph", "moe_decode")
    peak = BF16_PEAK_TFLOPS if args.workload == "bf16_dense" else FP8_PEAK_TFLOPS
    if is_masked:
        if graph_wl:
            dom = int(np.argmax(gemm_us))
            achieved = W.gemm_bytes[dom] / (gemm_us[dom] * 1e-6) / 1e9
            alg = float(W.gemm_bytes[dom])
            avg_us = gemm_us[dom]
        else:
            alg = float(np.mean(W.gemm_bytes))
            avg_us = float(np.mean(gemm_us))
            achieved = float(sum(W.gemm_bytes)) / (sum(gemm_us) * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
    else:
        achieved = total_flops / (sum(gemm_us) * 1e-6) / 1e12
        alg = float(np.mean(W.gemm_bytes))
        avg_us = float(np.mean(gemm_us))
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    roof["traffic"] = recorded_traffic(args.workload)
    roof["traffic_unit"] = ("HBM-side bytes per GEMM call: rocprofv3 TCC_EA0 read requests by size (32/64/128 B) plus "
                           "write requests, calibrated against a 1 GiB copy")
    roof["algorithmic_bytes_per_launch"] = alg
    roof["kernel"] = "gemm_kernel (BF16 kind)" if args.workload == "bf16_dense" else "gemm_kernel (FP8 kind)"
    roof["avg_launch_us"] = avg_us
    roof["per_launch"] = ("each GEMM call: 5 untimed calls, then %d calls (%s) with HIP events around the call on the "
                          "launch stream and a 1 GiB cache flush (a read of a 1 GiB scratch tensor) before each, "
                          "outside the events; achieved = the calls' algorithmic work / the sum of their median times "
                          "(a call is one kernel launch, or two in stream order where the launch plan splits the "
                          "columns)" % (args.reps, "eager" if args.timing == "eager" else "replays of a hipGraph"))
    if not is_masked and not graph_wl:
        wf = total_flops / (sum(k["write_flush_median_us"] for k in kt) * 1e-6) / 1e12
        roof["write_flush"] = {"achieved": wf, "frac": wf / peak,
                               "note": "the same protocol with a flush that writes 1 GiB: the call also pays the "
                                       "write-back of the dirty lines the flush leaves in the MALL"}
    in_step = total_flops / (sum(step_ms) * 1e-3) / 1e12 if not is_masked else None
    roof["warm_in_step"] = {"achieved": in_step, "frac": in_step / peak if in_step else None,
                            "per_call_us": [m * 1e3 for m in step_ms],
                            "note": "HIP events around the GEMM calls of %d of the %d timed steps (warm cache, "
                                    "operands just written by the casts)" % (len(timed), args.steps)}

    per_shape = []
    for i in range(nshape):
        N, K = W.shapes[i]
        kind, G, Mq, Nq, Kq = W.plan_args(i)
        plan = binding.query_config(getattr(binding, kind), G, Mq, Nq, Kq)
        tiles = f"{plan['block_m']}x{plan['block_n']}"
        if plan["block_n2"]:
            tiles += f" on columns [0, {plan['n_split']}), {plan['block_m']}x{plan['block_n2']} on the rest"
        e = {"N": N, "K": K, "tflops": W.flops[i] / (gemm_us[i] * 1e-6) / 1e12,
             "gbs": W.gemm_bytes[i] / (gemm_us[i] * 1e-6) / 1e9,
             "in_step_us": step_ms[i] * 1e3, "launches": 2 if plan["block_n2"] else 1, "tiles": tiles}
        e.update(kt[i])
        per_shape.append(e)

    if graph_wl:
        metric = "masked grouped FP8 (UE8M0) + BF16 GEMM GB/s under graph replay (% HBM)"
        unit = "GB/s"
        value = W.step_bytes() / (ms_per_step * 1e-3) / 1e9
        per_shape[0]["kernel"] = "fp8 masked, UE8M0 packed scales"
        per_shape[1]["kernel"] = "bf16 masked"
    elif args.workload == "moe_decode":
        metric = "MoE decode (dispatch + per-token cast, masked FP8 GEMM, combine) GB/s (% HBM)"
        unit = "GB/s"
        value = W.step_bytes_total / (ms_per_step * 1e-3) / 1e9
        per_shape[0]["kernel"] = "fp8 masked"
        per_shape[0].update(W.extra())
        per_shape[0]["tokens_per_s"] = W.T / (ms_per_step * 1e-3)
    elif args.workload == "moe_prefill":
        metric = "MoE prefill (dispatch + per-token cast, contiguous FP8 GEMM, combine) TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
        per_shape[0]["kernel"] = "fp8 contiguous"
        per_shape[0].update(W.extra())
        per_shape[0]["tokens_per_s"] = W.T / (ms_per_step * 1e-3)
    elif is_masked:
        metric = "masked grouped FP8 GEMM GB/s (% HBM)"
        unit = "GB/s"
        value = float(sum(W.gemm_bytes)) / (ms_per_step * 1e-3) / 1e9
    elif args.workload == "bf16_dense":
        metric = "BF16 GEMM TFLOPS (% BF16 MFMA peak)"
        unit = "TFLOPS"
    elif args.workload == "dense_rowb":
        metric = "FP8 GEMM with one FP32 B scale per row of B, TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
    elif args.workload == "contiguous":
        metric = "contiguous grouped FP8 block-scaled GEMM TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
    elif args.workload in ("dense_nn", "dense_tn", "dense_tt"):
        metric = f"FP8 block-scaled GEMM, {args.workload[-2:].upper()} layout, TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
    elif args.workload == "dense_fp8_out":
        metric = "FP8 block-scaled GEMM with per-token FP8 output TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
        roof["kernel"] = "gemm_kernel (FP8 kind, FP8-output epilogue)"
    else:
        metric = "FP8 block-scaled GEMM TFLOPS (% FP8 MFMA peak); masked-grouped GB/s (% HBM)"
        unit = "TFLOPS"

    out = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": args.settle_seconds, "steps": settle_steps},
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+bf16" if graph_wl else ("bf16" if args.workload == "bf16_dense" else "fp8_e4m3"),
        "data": "synthetic N(0,1) float32 inputs, seeded (numpy PCG64); no real activations or weights",
        "config": W.config(),
        "roofline": roof,
        "gemm_per_shape": per_shape,
    }
    del W
    torch.cuda.empty_cache()
    if args.workload == "dense" and not args.no_masked:
        out["masked"] = masked_block(torch, mg, synth, timer, args.reps)
    if not args.no_cpu_baseline and args.workload == "dense":
        log("timing the CPU oracle on bounded samples")
        out["cpu_baseline"] = time_cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
