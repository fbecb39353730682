"""Benchmark of the block-scaled FP8 GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--settle-seconds S]
                    [--workload dense|contiguous|masked|masked_graph|bf16_dense|dense_rowb|dense_fp8_out|
                                moe_decode|moe_prefill]

Before the W warmup steps, untimed steps run for S seconds (default 1): under
sustained GEMM load the GPU clock dips for the first few milliseconds and
settles within a few tens of milliseconds, and the K timed steps measure the
settled, sustained rate.

Default workload ("dense"): the five DeepSeek-V3-shaped dense GEMMs,
M = 4096 with (N, K) in {(2112, 7168), (24576, 1536), (7168, 16384),
(4096, 7168), (7168, 2048)}, N(0, 1) float32 inputs already resident in HBM.
One step = for every shape: per-token FP8 cast of A (1x128 scales),
per-block FP8 cast of B (128x128 scales), and the block-scaled FP8 GEMM
with BF16 output -- the whole hot path, no work skipped.

Prints ONE JSON line.  `value` is GEMM FLOPs (2*M*N*K summed over the
shapes) per second of whole-step time; `roofline` describes the dominant
kernel (the FP8 GEMM) from HIP events recorded around each GEMM call on the
launch stream (a call is one kernel launch, or two in stream order where the
launch plan splits the columns); `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload.

Other workloads (for the measurements in the design notes):
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

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_DENSE_FP8_OUT", 1, self.M, N, K)

    def config(self):
        return {"workload": self.name, "M": self.M, "shapes_NK": self.shapes,
                "scales": "fp32 1x128 (A) / 128x128 (B)", "out": "fp8 e4m3, fp32 1x128 scales (per-token cast fused)"}


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

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_CONTIGUOUS", self.G, self.Msum, N, K)

    def config(self):
        return {"workload": self.name, "groups": self.G, "rows": self.Msum, "shapes_NK": self.shapes}


class MaskedWorkload:
    name = "masked_fp8_moe_decode"

    def __init__(self, torch, mg, synth):
        self.torch, self.mg = torch, mg
        dev = torch.device("cuda")
        c = synth.MASKED
        self.G, self.max_m = c["G"], c["max_m"]
        self.shapes = list(c["shapes"])
        mm = synth.masked_m_decode(c["seed_m"], self.G)
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
                sfa=torch.empty((self.G, self.max_m, K // 128), dtype=torch.float32, device=dev),
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

    def plan_args(self, i):
        N, K = self.shapes[i]
        return ("DG_KIND_MASKED", self.G, self.max_m, N, K)

    def config(self):
        return {"workload": self.name, "experts": self.G, "max_m": self.max_m,
                "sum_masked_m": int(self.mm_host.sum()), "shapes_NK": self.shapes}


class MoeDecodeWorkload:
    """MoE decode on one GPU around the masked GEMM: 768 tokens routed to 8
    of 32 experts (256-row buffers, about 192 rows each), N 4096, K 7168.
    One step = moe_dispatch_masked_fp8 (routing + per-token cast of the
    routed tokens), the masked FP8 GEMM, and moe_combine.  With contig=True
    (MoePrefillWorkload): moe_dispatch_contiguous_fp8, the contiguous FP8
    GEMM and moe_combine on 4096 tokens."""
    name = "moe_decode_dispatch_gemm_combine"
    contig = False

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
        self.sfa = torch.empty((ga, max_m, K // 128), dtype=torch.float32, device=dev)
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
            rows = int(sum(-(-int(c_) // 256) * 256 for c_ in mm))
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
            # regions in 256-row granules: no 256-row tile of the GEMM holds two experts
            mg.moe_dispatch_contiguous_fp8(self.x, self.topk, self.a[0], self.sfa[0], self.layout, self.masked_m,
                                           self.slot, align=256)
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

    def plan_args(self, i):
        if self.contig:
            return ("DG_KIND_CONTIGUOUS", self.G, self.max_m, self.N, self.K)
        return ("DG_KIND_MASKED", self.G, self.max_m, self.N, self.K)

    def config(self):
        if self.contig:
            return {"workload": self.name, "tokens": self.T, "topk": self.k, "experts": self.G, "rows": self.max_m,
                    "N": self.N, "K": self.K, "routed_pairs": int(self.mm_host.sum()),
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

    def plan_args(self, i):
        return ("DG_KIND_MASKED" if i == 0 else "DG_KIND_BF16_MASKED", self.G, self.max_m, self.N, self.K)

    def config(self):
        return {"workload": self.name, "experts": self.G, "max_m": self.max_m, "N": self.N, "K": self.K,
                "mean_sum_masked_m": float(np.mean([m.sum() for m in self.mm_host])) if self.mm_host else 0.0,
                "kernels": ["gemm_kernel FP8 kind (UE8M0 packed scales)", "gemm_kernel BF16 kind"],
                "step": "one hipGraph replay: UE8M0 cast of A, 2 packs, FP8 masked GEMM, BF16 masked GEMM"}


# ---------------------------------------------------------------------------
# recorded HBM traffic of the GEMM kernel (rocprofv3 PMC), valid for one source
# ---------------------------------------------------------------------------

def recorded_traffic(workload):
    """Bytes per launch of the dominant GEMM kernel (FETCH + WRITE, calibrated
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
# CPU baseline: the oracle on a bounded sample of the dense workload
# ---------------------------------------------------------------------------

def time_cpu_baseline(rows_a=512, rows_b=8192):
    import oracle
    from moe_grouped_gemm_x128_amd import synth

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    flops = 0.0
    spent = 0.0
    for i, (N, K) in enumerate(synth.DENSE_V3_SHAPES):
        sa, sb = synth.dense_v3_seeds(i)
        rng_a = synth.normal_f32(sa, (synth.DENSE_V3_M, K))[:rows_a]
        rng_b = synth.normal_f32(sb, (N, K))[:rows_b]
        t = time.perf_counter()
        a, sfa = oracle.per_token_cast_to_fp8(rng_a)
        b, sfb = oracle.per_block_cast_to_fp8(rng_b)
        oracle.fp8_gemm_nt(a, b, sfa, sfb)
        spent += time.perf_counter() - t
        flops += 2.0 * rows_a * min(rows_b, N) * K
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOPS",
        "cores": blas_threads,
        "kind": "oracle",
        "sample": (f"per shape: first {rows_a} rows of A x first {rows_b} rows of B, per-token + per-block quantize "
                   f"+ block-scaled GEMM in float64 (numpy; elementwise work single-threaded, matmul on "
                   f"{blas_threads} BLAS threads); {spent:.1f} s of oracle time"),
        "seconds": spent,
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
                             "dense_fp8_out", "moe_decode", "moe_prefill"])
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed steps run for this long before the warmup steps, so that the timed steps see "
                         "the GPU's steady sustained clock rather than the dip of its first milliseconds under load")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record HIP events around the GEMM calls of one timed step in this many (plus the last)")
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
    W = {"dense": DenseWorkload, "contiguous": ContiguousWorkload, "masked": MaskedWorkload,
         "masked_graph": MaskedGraphWorkload, "bf16_dense": Bf16DenseWorkload,
         "dense_rowb": DenseRowBWorkload, "dense_fp8_out": DenseFp8OutWorkload,
         "moe_decode": MoeDecodeWorkload, "moe_prefill": MoePrefillWorkload}[args.workload](torch, mg, synth)
    torch.cuda.synchronize()

    # Power-state settle: under sustained GEMM load the clock dips for the first
    # few milliseconds (to ~1.4 GHz) and recovers to its steady level within a
    # few tens of milliseconds; steps run here are not timed and not counted.
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
    if hasattr(W, "timing_pass"):
        W.mm_host = []  # count the timed replays only
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    nshape = len(W.flops)
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nshape)]
              for _ in range(args.steps)]
    # HIP events around the GEMM calls of one timed step in `event_every`
    # (and of the last step): each event record is a marker in the stream
    # that the next kernel waits behind (about 5.6 us on this GPU), so
    # recording them on every step would add ~10% of gaps to a step of
    # fifteen kernels
    timed = [s for s in range(args.steps) if s % args.event_every == args.event_every - 1]
    if args.steps - 1 not in timed:
        timed.append(args.steps - 1)
    torch.cuda.synchronize()
    graph_wl = hasattr(W, "timing_pass")
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

    # per-shape average GEMM launch duration (ms)
    gemm_ms = [float(np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in timed])) for i in range(nshape)]
    ms_per_step = wall * 1e3 / args.steps
    total_flops = float(sum(W.flops))
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    mean_launch_ms = float(np.mean(gemm_ms))
    mean_flops = total_flops / nshape
    is_masked = args.workload in ("masked", "masked_graph", "moe_decode")
    is_moe = args.workload in ("moe_decode", "moe_prefill")
    if graph_wl:
        # dominant kernel: the GEMM with the longest launches
        dom = int(np.argmax(gemm_ms))
        achieved = W.gemm_bytes[dom] / (gemm_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    elif is_masked:
        mean_bytes = float(np.mean(W.gemm_bytes))
        achieved = mean_bytes / (mean_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None}
    else:
        peak = BF16_PEAK_TFLOPS if args.workload == "bf16_dense" else FP8_PEAK_TFLOPS
        achieved = mean_flops / (mean_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["traffic"] = recorded_traffic(args.workload)
    roof["traffic_unit"] = "HBM bytes per GEMM call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roof["algorithmic_bytes_per_launch"] = float(np.mean(W.gemm_bytes))
    roof["kernel"] = "gemm_kernel (FP8 kind)"
    roof["avg_launch_us"] = mean_launch_ms * 1e3
    roof["per_launch"] = ("mean over the workload's GEMM calls of one step (algorithmic work / HIP-event duration "
                          "around the call; a call is one kernel launch, or two in stream order where the launch "
                          "plan splits the columns, see gemm_per_shape); events recorded on %d of the %d timed "
                          "steps" % (len(timed), args.steps))
    if graph_wl:
        roof["algorithmic_bytes_per_launch"] = float(W.gemm_bytes[dom])
        roof["kernel"] = ["gemm_kernel (FP8 kind, UE8M0)", "gemm_kernel (BF16 kind)"][dom]
        roof["avg_launch_us"] = gemm_ms[dom] * 1e3
        roof["per_launch"] = "the longer of the two GEMM kernels (algorithmic bytes / HIP-event duration of eager launches)"

    per_shape = []
    for i in range(nshape):
        N, K = W.shapes[i]
        kind, G, Mq, Nq, Kq = W.plan_args(i)
        plan = binding.query_config(getattr(binding, kind), G, Mq, Nq, Kq)
        tiles = f"{plan['block_m']}x{plan['block_n']}"
        if plan["block_n2"]:
            tiles += f" on columns [0, {plan['n_split']}), {plan['block_m']}x{plan['block_n2']} on the rest"
        per_shape.append({"N": N, "K": K, "gemm_us": gemm_ms[i] * 1e3,
                          "tflops": W.flops[i] / (gemm_ms[i] * 1e-3) / 1e12,
                          "gbs": W.gemm_bytes[i] / (gemm_ms[i] * 1e-3) / 1e9,
                          "launches": 2 if plan["block_n2"] else 1, "tiles": tiles})

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
        step_bytes = float(sum(W.gemm_bytes))
        value = step_bytes / (ms_per_step * 1e-3) / 1e9
    elif args.workload == "bf16_dense":
        metric = "BF16 GEMM TFLOPS (% BF16 MFMA peak)"
        unit = "TFLOPS"
        roof["kernel"] = "gemm_kernel (BF16 kind)"
    elif args.workload == "dense_fp8_out":
        metric = "FP8 block-scaled GEMM with per-token FP8 output TFLOPS (% FP8 MFMA peak)"
        unit = "TFLOPS"
        roof["kernel"] = "gemm_kernel (FP8 kind, FP8-output epilogue)"
    else:
        metric = "FP8 block-scaled GEMM TFLOPS (% FP8 MFMA peak)"
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
        "gemm_only_value": mean_flops / (mean_launch_ms * 1e-3) / 1e12 if not is_masked else achieved,
    }
    if not args.no_cpu_baseline and args.workload == "dense":
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = time_cpu_baseline()
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
