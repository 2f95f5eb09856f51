"""Benchmark of the fused low-bit dequant-GEMV hot path on one MI355X.

Default workload: INT4 group-128 fused dequant-GEMV, W 8192 x 8192 (Student-t(4)
* 0.015, synthetic), x bf16 N(0, 1), batch 1.  A step is one fused GEMV over the
whole matrix.  The weights are cycled through a rotation pool of distinct
device copies (>= 1.1 GiB in total) so every step reads HBM rather than the
256 MB Infinity Cache; activations and outputs stay resident.  The K timed steps
are captured once in a HIP graph and replayed, bracketed by device syncs, and
timed with HIP events on the launch stream.

Prints one JSON line: effective weight GB/s (algorithmic bytes per step / time),
the roofline fraction against the 8 TB/s HBM peak and, for context, the fp64
oracle timed on the host cores on the same workload.

Other workloads (``--workload``): ternary_1k, int4_8k_b4, moe_t1, moe_t8,
cassandra_spec, cassandra_restore, cassandra_verify, mx_verify and the FFN-shaped
int4/ternary matrices; ``--all FILE`` measures every one and appends a JSON line
per workload to FILE (the stdout line is still the default workload's).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
POOL_BYTES = int(1.1 * 2 ** 30)
METRIC = "effective weight GB/s (fraction of HBM peak), fused dequant-GEMV batch 1"


def _x_dev(x_bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)


class Workload:
    """A device-resident workload: `launch(i)` enqueues step i (rotation copy i % n)."""
    name = ""
    kernel = ""          # kernel symbol substring, for profiles
    fmt_name = ""
    dtype = "bf16"

    def bytes_per_step(self) -> int: ...
    def launch(self, i: int) -> None: ...


def synth_zero_frac():
    import synth
    return synth.ZERO_BLOCK_FRAC


def _pool_copies(bytes_weights):
    return max(1, math.ceil(POOL_BYTES / max(1, bytes_weights)))


class BlockQuantGemv(Workload):
    def __init__(self, kind, M, K, B, dev, name, seed_name):
        import torch
        import memory_bound_decode_amd as mbd
        import synth
        self.name, self.kind, self.M, self.K, self.B = name, kind, M, K, B
        self.kernel = "gemv_bn_kernel" if B <= 4 else "gemv_mq_kernel"
        self.fmt_name = {"int4": "int4_g128", "ternary": "ternary_b128", "ternary_skip": "ternary_b128_skip"}[kind]
        wl = synth.WORKLOADS[seed_name]
        if (wl.M, wl.K) == (M, K):
            self.w = synth.gen_weights(wl)
        else:
            seed = wl.seed + 1000 * M + K
            self.w = synth.f32_to_bf16_bits(
                synth.gen_weight_rows(seed, M, K, wl.dist, wl.scale).astype(np.float32))
            if kind == "ternary_skip":         # block-sparse: whole 128-blocks zero
                self.w = synth.zero_out_blocks(self.w, synth.gen_zero_blocks(seed, M, K))
        self.x = synth.gen_x(wl, B, K)
        fmt = {"int4": mbd.MBD_INT4_G128, "ternary": mbd.MBD_TERNARY_B128,
               "ternary_skip": mbd.MBD_TERNARY_SKIP}[kind]
        self.packed = mbd.mbd_pack(fmt, self.w)
        st = self.packed.stats()
        self.bpw = st.bpw
        wbytes = sum(b for _, b in self.packed.sections().values())
        self.weight_bytes = wbytes
        self.n = _pool_copies(wbytes)
        self.copies = [mbd.to_device(self.packed, dev) for _ in range(self.n)]
        self.xt = _x_dev(self.x, dev)
        self.y = torch.empty((B, M), dtype=torch.float32, device=dev)
        self.mbd = mbd

    def bytes_per_step(self):
        return self.weight_bytes + self.B * self.K * 2 + self.B * self.M * 4

    def launch(self, i):
        self.mbd.mbd_gemv(self.copies[i % self.n], self.xt, self.y)

    def config(self):
        c = {"workload": self.name, "M": self.M, "K": self.K, "batch": self.B,
             "weight_format": self.fmt_name, "bits_per_weight": round(self.bpw, 4),
             "rotation_copies": self.n, "bytes_per_step": self.bytes_per_step()}
        if self.kind == "ternary_skip":
            c["zero_block_fraction"] = synth_zero_frac()
            c["dense_format_bytes"] = self.M * self.K // 4 + self.M * (self.K // 128) * 2
        return c

    def oracle_pack(self):
        """The oracle's pack of the whole matrix (quantize + code packing), once."""
        from oracle import int4, ternary, ternary_skip
        if self.kind == "ternary_skip":
            return ternary_skip.pack(self.w)
        return (int4 if self.kind == "int4" else ternary).pack(self.w)

    def bf16_bytes(self):
        return 2 * self.M * self.K

    def oracle_call(self):
        """One oracle call: unpack + dequant from the packed sections + fp64 matvec."""
        from oracle import gemv, int4, ternary, ternary_skip
        if self.kind == "ternary_skip":
            sec = {k: self.packed.section(k, dt) for k, dt in
                   (("codes", np.uint32), ("scales", np.uint16), ("slabs", np.uint32), ("tile_base", np.uint32))}
            return gemv.gemv(ternary_skip.unpack_dequant(sec, self.M, self.K), self.x)
        mod = int4 if self.kind == "int4" else ternary
        codes = self.packed.section("codes", np.uint32).reshape(self.M, -1)
        scales = self.packed.section("scales", np.uint16).reshape(self.M, -1)
        return gemv.gemv(mod.unpack_dequant(codes, scales, self.K), self.x)

    def device_output(self):
        import torch
        self.launch(0)
        torch.cuda.synchronize()
        return self.y.cpu().numpy()


class MoeGemv(Workload):
    def __init__(self, T, dev):
        import torch
        import memory_bound_decode_amd as mbd
        import synth
        wl = synth.WORKLOADS["ternary_moe"]
        self.name, self.T, self.kernel, self.fmt_name = "ternary_moe_t%d" % T, T, (
            "moe_b1_kernel" if T == 1 else "moe_mq_kernel"), "ternary_b128"
        self.routes = synth.gen_routes(wl, T)
        ups = np.concatenate([synth.gen_expert(wl, e, "up") for e in range(wl.experts)])
        dns = np.concatenate([synth.gen_expert(wl, e, "down") for e in range(wl.experts)])
        pu = mbd.mbd_pack(mbd.MBD_TERNARY_B128, ups, n_mats=wl.experts)
        pd = mbd.mbd_pack(mbd.MBD_TERNARY_B128, dns, n_mats=wl.experts)
        per_expert = (sum(b for _, b in pu.sections().values()) + sum(b for _, b in pd.sections().values())) // wl.experts
        self.distinct = len(set(self.routes.reshape(-1).tolist()))
        self.weight_bytes = per_expert * self.distinct
        self.n = _pool_copies(per_expert * wl.experts)
        self.up = [mbd.to_device(pu, dev, n_mats=wl.experts) for _ in range(self.n)]
        self.dn = [mbd.to_device(pd, dev, n_mats=wl.experts) for _ in range(self.n)]
        self.x = _x_dev(synth.gen_x(wl, T, wl.K), dev)
        self.a = _x_dev(synth.gen_down_inputs(wl, T).reshape(T * wl.topk, wl.M), dev)
        self.r = torch.from_numpy(self.routes).to(dev)
        self.yu = torch.empty((T, wl.topk, wl.M), dtype=torch.float32, device=dev)
        self.yd = torch.empty((T, wl.topk, wl.K), dtype=torch.float32, device=dev)
        self.ws = torch.empty(mbd.mbd_moe_workspace_bytes(wl.experts, T, wl.topk), dtype=torch.uint8, device=dev)
        self.wl, self.mbd = wl, mbd

    def bf16_bytes(self):
        return 2 * 2 * self.wl.M * self.wl.K * self.distinct      # up and down matrices of each distinct expert

    def bytes_per_step(self):
        wl, T = self.wl, self.T
        act = T * wl.K * 2 + T * wl.topk * wl.M * 2 + T * wl.topk * 4
        out = T * wl.topk * (wl.M + wl.K) * 4
        return self.weight_bytes + act + out

    def launch(self, i):
        m = self.mbd
        m.mbd_moe_gemv(self.up[i % self.n], self.r, self.x, False, self.yu, self.ws)
        m.mbd_moe_gemv(self.dn[i % self.n], self.r, self.a, True, self.yd, self.ws)

    def config(self):
        return {"workload": self.name, "experts": 64, "topk": 8, "tokens": self.T, "distinct_experts": self.distinct,
                "up": [1536, 4096], "down": [4096, 1536], "weight_format": self.fmt_name,
                "rotation_copies": self.n, "bytes_per_step": self.bytes_per_step()}


class CassandraWl(Workload):
    def __init__(self, mode, dev):
        import torch
        import memory_bound_decode_amd as mbd
        import synth
        draft = mode in ("spec", "spec_mx", "decode", "decode_mx")
        wl = synth.WORKLOADS["cassandra_spec" if draft else "cassandra_verify"]
        self.mode, self.M, self.K = mode, wl.M, wl.K
        self.w = synth.gen_weights(wl)
        norms = synth.gen_act_norms(wl)
        self.fmt_name = {"mx": "mx32", "spec_mx": "cassandra2_mx32_spec", "decode_mx": "cassandra2_mx32_spec"}.get(
            mode, "cassandra")
        if mode == "mx":
            p = mbd.mbd_pack(mbd.MBD_MX32, self.w)
            used = list(p.sections().keys())
        elif mode in ("spec_mx", "decode_mx"):
            p = mbd.mbd_pack(mbd.MBD_CASSANDRA_MX, self.w, norms)
            used = list(p.sections().keys())
        else:
            p = mbd.mbd_pack(mbd.MBD_CASSANDRA, self.w, norms)
            used = list(mbd.SPEC_SECTIONS) if mode in ("spec", "decode") else list(mbd.SECTION_NAMES[mbd.MBD_CASSANDRA])
        st = p.stats()
        self.stats = {"spec_bpw": round(st.spec_bpw, 4), "bpw": round(st.bpw, 4),
                      "exp_entropy_bits": round(st.exp_entropy_bits, 4), "unary_avg_bits": round(st.unary_avg_bits, 4),
                      "n_sym": st.n_sym, "kept": st.n_kept}
        secs = p.sections()
        self.weight_bytes = sum(secs[k][1] for k in used)
        self.n = _pool_copies(self.weight_bytes)
        self.copies = [mbd.to_device(p, dev, only=used) for _ in range(self.n)]
        self.B = {"spec": 1, "spec_mx": 1, "restore": 0, "decode": 0, "decode_mx": 0, "verify": 16, "mx": 16}[mode]
        self.name = {"spec": "cassandra_spec_gemv_4096x14336_b1", "restore": "cassandra_restore_8192x28672",
                     "verify": "cassandra_verify_gemm_8192x28672_b16", "mx": "mx32_gemm_8192x28672_b16",
                     "spec_mx": "cassandra2_mx_spec_gemv_4096x14336_b1",
                     "decode": "cassandra_spec_decode_4096x14336", "decode_mx": "cassandra2_mx_spec_decode_4096x14336"}[mode]
        self.kernel = {"spec": "spec_gemv_kernel", "restore": "decode_dense_kernel", "verify": "verify_gemm_kernel",
                       "mx": "mx_gemm_kernel", "spec_mx": "mx_spec_gemv_kernel", "decode": "decode_dense_kernel",
                       "decode_mx": "mx_spec_decode_kernel"}[mode]
        if self.B:
            self.xt = _x_dev(synth.gen_x(wl, self.B), dev)
            self.y = torch.empty((self.B, self.M), dtype=torch.float32, device=dev)
        else:
            self.out = torch.empty((self.M, self.K), dtype=torch.int16, device=dev)
        self.mbd = mbd

    def bf16_bytes(self):
        return 2 * self.M * self.K

    def bytes_per_step(self):
        if self.B == 0:                                  # restore / draft decode: sections read, bf16 written
            return self.weight_bytes + self.M * self.K * 2
        return self.weight_bytes + self.B * self.K * 2 + self.B * self.M * 4

    def launch(self, i):
        m, c = self.mbd, self.copies[i % self.n]
        if self.mode in ("spec", "spec_mx"):
            m.mbd_spec_gemv(c, self.xt, self.y)
        elif self.mode == "restore":
            m.mbd_verify_restore(c, self.out)
        elif self.mode in ("decode", "decode_mx"):
            m.mbd_spec_decode(c, self.out)
        else:
            m.mbd_gemv(c, self.xt, self.y)

    def config(self):
        d = {"workload": self.name, "M": self.M, "K": self.K, "batch": self.B, "weight_format": self.fmt_name,
             "rotation_copies": self.n, "bytes_per_step": self.bytes_per_step()}
        d.update(self.stats)
        return d


class CassandraStep(Workload):
    """Draft/verify step of speculative decoding over a stack of layer-shaped
    Cassandra matrices (Cassandra review, speculative decoding and the ideal-speedup
    figure): N draft tokens, each through every layer as a GEMV over the speculation
    data only, then every layer's batch-(N+1) fused restore + verify GEMM.  The
    activations are synthetic (no trained weights), drawn per call.  Acceptance is a
    parameter: with per-token acceptance a, a step yields (1 - a^(N+1)) / (1 - a)
    tokens on average; the weight bytes per token against bf16 give the byte side of
    the ideal speedup."""

    def __init__(self, dev, n_draft=4, layers=2, alpha=0.8):
        import torch
        import memory_bound_decode_amd as mbd
        import synth
        wl = synth.WORKLOADS["cassandra_verify"]
        self.M, self.K, self.N, self.L, self.alpha = wl.M, wl.K, n_draft, layers, alpha
        self.name, self.kernel, self.fmt_name = "cassandra_draft_verify_step", "verify_gemm_kernel", "cassandra"
        norms = synth.gen_act_norms(wl)
        packs = []
        for l in range(layers):
            w = synth.f32_to_bf16_bits(synth.gen_weight_rows(wl.seed + 101 * (l + 1), wl.M, wl.K, wl.dist,
                                                             wl.scale).astype(np.float32))
            packs.append(mbd.mbd_pack(mbd.MBD_CASSANDRA, w, norms))
        secs = packs[0].sections()
        self.spec_bytes = sum(secs[k][1] for k in mbd.SPEC_SECTIONS)
        self.full_bytes = sum(b for _, b in secs.values())
        weight_step = sum(self._layer_bytes(p, mbd) for p in packs)
        self.n = _pool_copies(weight_step)
        self.copies = [[mbd.to_device(p, dev) for p in packs] for _ in range(self.n)]
        self.weight_step = weight_step
        xs = synth.gen_x(wl, n_draft * layers)              # one activation row per draft call
        self.xd = [[_x_dev(xs[l * n_draft + t:l * n_draft + t + 1], dev) for t in range(n_draft)]
                   for l in range(layers)]
        self.X = [_x_dev(synth.gen_x(wl, n_draft + 1), dev) for _ in range(layers)]
        self.yd = torch.empty((layers, n_draft, 1, wl.M), dtype=torch.float32, device=dev)
        self.Y = torch.empty((layers, n_draft + 1, wl.M), dtype=torch.float32, device=dev)
        self.mbd = mbd

    def _layer_bytes(self, p, mbd):
        secs = p.sections()
        return self.N * sum(secs[k][1] for k in mbd.SPEC_SECTIONS) + sum(b for _, b in secs.values())

    def bytes_per_step(self):
        M, K, N, L = self.M, self.K, self.N, self.L
        act = L * (N * (2 * K + 4 * M) + (N + 1) * (2 * K + 4 * M))
        return self.weight_step + act

    def launch(self, i):
        m, layers = self.mbd, self.copies[i % self.n]
        for t in range(self.N):                      # draft: token by token through the stack
            for l, dw in enumerate(layers):
                m.mbd_spec_gemv(dw, self.xd[l][t], self.yd[l, t])
        for l, dw in enumerate(layers):              # verify: all N + 1 positions at once
            m.mbd_gemv(dw, self.X[l], self.Y[l])

    def config(self):
        a, N = self.alpha, self.N
        tokens = (1 - a ** (N + 1)) / (1 - a)
        bf16_per_token = self.L * self.M * self.K * 2
        return {"workload": self.name, "layers": self.L, "layer": [self.M, self.K], "n_draft": N,
                "verify_batch": N + 1, "weight_format": "cassandra", "rotation_copies": self.n,
                "spec_bytes_per_layer": self.spec_bytes, "full_bytes_per_layer": self.full_bytes,
                "weight_bytes_per_step": self.weight_step, "bytes_per_step": self.bytes_per_step(),
                "acceptance": a, "tokens_per_step": round(tokens, 4),
                "bf16_weight_bytes_per_token": bf16_per_token,
                "weight_bytes_per_token": round(self.weight_step / tokens),
                "byte_speedup_vs_bf16": round(bf16_per_token / (self.weight_step / tokens), 4)}


class CassandraEncode(Workload):
    """Device encoder: the eight Cassandra sections of the 4096 x 14336 draft
    workload's weight from device bf16 weights and activation norms (the encode
    call; its plan is made once, outside the timed region)."""
    kernel = "enc_select_kernel"

    def __init__(self, dev):
        import torch
        import memory_bound_decode_amd as mbd
        import synth
        wl = synth.WORKLOADS["cassandra_spec"]
        self.M, self.K = wl.M, wl.K
        w = synth.gen_weights(wl)
        norms = synth.gen_act_norms(wl)
        self.n = _pool_copies(w.nbytes)
        self.wd = [torch.from_numpy(w.view(np.int16)).to(dev) for _ in range(self.n)]
        self.nd = torch.from_numpy(norms).to(dev)
        self.ws = torch.empty(mbd.mbd_encode_workspace_bytes(self.M), dtype=torch.uint8, device=dev)
        self.plan = mbd.mbd_encode_plan(self.wd[0], self.nd, 3, 10, self.ws)
        self.secs = [torch.empty(int(self.plan.padded_bytes[i]), dtype=torch.uint8, device=dev) for i in range(8)]
        self.name = "cassandra_encode_4096x14336"
        self.fmt_name = "cassandra"
        self.mbd = mbd

    def bytes_per_step(self):
        return self.M * self.K * 2 + self.K * 4 + sum(int(b) for b in self.plan.bytes)

    def launch(self, i):
        self.mbd.mbd_encode_cassandra(self.wd[i % self.n], self.nd, 3, 10, self.plan, self.secs, self.ws)

    def config(self):
        return {"workload": self.name, "M": self.M, "K": self.K, "weight_format": self.fmt_name,
                "kept": int(self.plan.n_kept), "n_sym": int(self.plan.n_sym), "unary_bits": int(self.plan.unary_bits),
                "rotation_copies": self.n, "bytes_per_step": self.bytes_per_step()}


def make_workload(name, dev):
    if name == "int4_8k":
        return BlockQuantGemv("int4", 8192, 8192, 1, dev, "int4_g128_gemv_8192x8192_b1", "int4_8k")
    if name == "int4_8k_b4":
        return BlockQuantGemv("int4", 8192, 8192, 4, dev, "int4_g128_gemv_8192x8192_b4", "int4_8k")
    if name == "int4_8k_b8":
        return BlockQuantGemv("int4", 8192, 8192, 8, dev, "int4_g128_gemv_8192x8192_b8", "int4_8k")
    if name == "int4_8k_b16":
        return BlockQuantGemv("int4", 8192, 8192, 16, dev, "int4_g128_gemv_8192x8192_b16", "int4_8k")
    if name == "ternary_1k":
        return BlockQuantGemv("ternary", 1024, 1024, 1, dev, "ternary_b128_gemv_1024x1024_b1", "ternary_1k")
    for kind, tag in (("int4", "int4_8k"), ("ternary", "ternary_moe")):
        for (M, K) in ((4096, 14336), (14336, 4096), (8192, 28672)):
            if name == "%s_%dx%d" % (kind, M, K):
                return BlockQuantGemv(kind, M, K, 1, dev, "%s_gemv_%dx%d_b1" % (
                    "int4_g128" if kind == "int4" else "ternary_b128", M, K), tag)
    for (M, K) in ((4096, 14336), (8192, 28672)):
        for B in (1, 4, 8):
            if name == "ternary_skip_%dx%d%s" % (M, K, "" if B == 1 else "_b%d" % B):
                return BlockQuantGemv("ternary_skip", M, K, B, dev, "ternary_skip_gemv_%dx%d_b%d" % (M, K, B),
                                      "ternary_moe")
    if name == "moe_t1":
        return MoeGemv(1, dev)
    if name == "moe_t8":
        return MoeGemv(8, dev)
    if name == "cassandra_step":
        return CassandraStep(dev)
    if name == "cassandra_encode":
        return CassandraEncode(dev)
    if name in ("cassandra_spec", "cassandra_restore", "cassandra_verify", "mx_verify", "cassandra_spec_mx",
                "cassandra_decode", "cassandra_decode_mx"):
        return CassandraWl({"cassandra_spec": "spec", "cassandra_restore": "restore", "cassandra_spec_mx": "spec_mx",
                            "cassandra_verify": "verify", "mx_verify": "mx", "cassandra_decode": "decode",
                            "cassandra_decode_mx": "decode_mx"}[name], dev)
    raise SystemExit("unknown workload %s" % name)


ALL = ["int4_8k", "int4_8k_b4", "int4_8k_b8", "int4_8k_b16", "ternary_1k", "int4_4096x14336", "int4_14336x4096", "int4_8192x28672",
       "ternary_4096x14336", "ternary_14336x4096", "ternary_8192x28672", "moe_t1", "moe_t8",
       "cassandra_spec", "cassandra_restore", "cassandra_verify", "mx_verify", "cassandra_step",
       "cassandra_decode", "cassandra_decode_mx",
       "ternary_skip_8192x28672", "ternary_skip_4096x14336", "ternary_skip_8192x28672_b4",
       "ternary_skip_8192x28672_b8", "cassandra_spec_mx", "cassandra_encode"]


_HOLD_CYCLES = None


def hold_gpu(us=400.0):
    """Enqueue a spin kernel of about ``us`` microseconds on the current stream.  The
    host submits the timed launches while the GPU spins, so the start event, which
    the stream reaches only after the spin, is not delayed by the host's submission
    of the first launches: the timed region holds the K steps and nothing else."""
    import torch
    global _HOLD_CYCLES
    if _HOLD_CYCLES is None:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 1 << 20
        e0.record()
        torch.cuda._sleep(n)
        e1.record()
        torch.cuda.synchronize()
        _HOLD_CYCLES = n / max(1e-3, e0.elapsed_time(e1) * 1000.0)     # cycles per microsecond
    torch.cuda._sleep(int(_HOLD_CYCLES * us))


EAGER_MAX_STEPS = 512


def time_workload(wl, steps, warmup, use_graph=None):
    """(seconds for `steps` steps, per-step ms) with HIP events on the launch stream.

    use_graph None picks by step count: a HIP graph replay costs about 13 us once per
    replay (measured: 20 steps of the INT4 8192 x 8192 GEMV 8.70 us per step from a
    graph, 8.05 us eager), while eager launches are gapless only while the host has
    queued them all behind the hold kernel, so up to EAGER_MAX_STEPS steps launch
    eagerly and longer runs replay one graph."""
    import torch
    if use_graph is None:
        use_graph = steps > EAGER_MAX_STEPS
    stream = torch.cuda.current_stream()
    # Set-up, not steps: every rotation copy is read once by the step's own launch, so
    # that the timed steps, like those of a decode loop that reads all its weights
    # every token, find the copies' address translations resident (the first read of
    # a copy untouched since its upload costs ~0.5 us more at 8192 x 8192).
    for i in range(getattr(wl, "n", 1)):
        wl.launch(i)
    torch.cuda.synchronize()
    for i in range(min(warmup, 3)):
        wl.launch(i)                                     # eager warm-up (first-call set-up)
    torch.cuda.synchronize()
    if use_graph:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            for i in range(warmup):
                wl.launch(i)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                wl.launch(warmup + i)
        torch.cuda.synchronize()
        gw.replay()
        hold_us = 400.0
    else:
        # the host time per step, so that the hold outlasts the host's queueing of
        # every timed launch
        hold_gpu(2000.0)
        t0 = time.perf_counter()
        for i in range(warmup):
            wl.launch(i)
        host_us = (time.perf_counter() - t0) * 1e6 / max(1, warmup)
        # a wide margin: the host can queue more slowly during the timed loop than
        # during the warm-up, and a GPU that catches up with it times the gaps
        hold_us = 1000.0 + 4.0 * host_us * steps
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    hold_gpu(hold_us)
    e0.record(stream)
    if use_graph:
        g.replay()
    else:
        for i in range(steps):
            wl.launch(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1000.0
    time_workload.last_mode = "graph replay" if use_graph else "eager"
    return sec, 1000.0 * sec / steps


def read_peak(nbytes, dev, steps=100, shapes=None):
    """Best streaming-read rate over launch shapes for a read of ``nbytes`` per launch
    (the library's probe kernel: 16-byte non-temporal loads, eight in flight per
    thread), cycling through copies of >= 1.1 GiB in total as the workloads do.
    Returns (best record, all records); a record gives the shape, the per-launch
    microseconds and GB/s."""
    import torch
    import memory_bound_decode_amd as mbd
    n16 = max(1, nbytes // 16)
    nbytes = 16 * n16
    copies = [torch.empty(n16 * 4, dtype=torch.int32, device=dev) for _ in range(_pool_copies(nbytes))]
    for c in copies:
        c.fill_(1)
    if shapes is None:
        shapes = []
        for threads in (256, 512, 1024):
            one_round = -(-n16 // (threads * 8))
            for blocks in sorted({256, 512, 1024, 2048, 4096, 8192, one_round}):
                if blocks <= 4 * one_round:
                    shapes.append((blocks, threads))
    sink = torch.zeros(max(b for b, _ in shapes), dtype=torch.int32, device=dev)
    recs = []
    class _Probe:                                        # the probe as a workload for time_workload
        n = len(copies)

        def __init__(self, blocks, threads):
            self.blocks, self.threads = blocks, threads

        def launch(self, i):
            mbd.mbd_probe_stream_read(copies[i % len(copies)], sink, self.blocks, self.threads)

    for blocks, threads in shapes:
        # the workloads' protocol (every copy read once, warm-up, the timed launches
        # queued behind a hold, HIP events around them), eager and from a graph: the
        # faster of the two, so that the peak is not understated
        us = 1000.0 * min(time_workload(_Probe(blocks, threads), steps, 10, g)[1] for g in (False, True))
        recs.append({"blocks": blocks, "threads": threads, "us": round(us, 3), "gbs": round(nbytes / us / 1e3, 1)})
    best = max(recs, key=lambda r: r["gbs"])
    return dict(best, bytes=nbytes), recs


def traffic_from_profiles(wl):
    """Measured HBM bytes per step from a committed counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_traffic.json" % wl.name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_sha256") != source_hash():
        return None
    return d.get("hbm_bytes_per_step")


def source_hash():
    """Hash of the sources the default workload's kernel is built from; the stored
    traffic counters apply only while it matches."""
    h = hashlib.sha256()
    for s in ("gemv.hip", "mbd_internal.h"):
        with open(os.path.join(ROOT, "memory_bound_decode_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def cpu_baseline(wl, budget_s=15.0):
    """Time the fp64 oracle (unpack + dequant + matvec) on the host for ~budget_s."""
    if not hasattr(wl, "oracle_call"):
        return None, None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                                    # pragma: no cover
        blas = 1
    t0 = time.perf_counter()
    ref = wl.oracle_call()
    calls, elapsed = 1, time.perf_counter() - t0
    while elapsed < budget_s and calls < 50:
        t1 = time.perf_counter()
        wl.oracle_call()
        elapsed += time.perf_counter() - t1
        calls += 1
    gbs = wl.bytes_per_step() * calls / elapsed / 1e9
    extra = {"cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": int(blas)}
    if hasattr(wl, "oracle_pack"):
        t1 = time.perf_counter()
        wl.oracle_pack()
        extra["oracle_pack_s"] = round(time.perf_counter() - t1, 2)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(blas), "kind": "oracle", **extra,
            "sample": "%d full oracle calls (unpack + fp64 dequant + numpy fp64 matvec) over the whole "
                      "%s matrix in %.1f s; elementwise steps single-threaded, matvec on %d BLAS threads"
                      % (calls, wl.name, elapsed, blas)}, ref


def measure(name, dev, steps, warmup, with_cpu, use_graph=None, with_read_peak=False):
    wl = make_workload(name, dev)
    sec, ms = time_workload(wl, steps, warmup, use_graph)
    bps = wl.bytes_per_step()
    gbs = bps * steps / sec / 1e9
    traffic = traffic_from_profiles(wl)
    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": wl.config(),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
        "kernel": wl.kernel,
        "launch": time_workload.last_mode,
    }
    if hasattr(wl, "B") and getattr(wl, "B", 0):
        out["tok_per_s_equiv"] = round(wl.B / (ms / 1000.0), 1)
    if hasattr(wl, "bf16_bytes"):
        # the same weights read as bf16 in the same time (not comparable to the peak)
        out["bf16_equiv_gbs"] = round(wl.bf16_bytes() / (ms / 1000.0) / 1e9, 1)
    if hasattr(wl, "bpw"):
        # context: tokens/s of a 9B-active model whose weights stream at this rate
        out["tok_per_s_9b_active_equiv"] = round(gbs * 1e9 / (9e9 * wl.bpw / 8.0), 1)
    if with_read_peak:
        best, _ = read_peak(bps, dev)
        out["read_peak"] = best
        out["roofline"]["read_peak"] = best["gbs"]
        out["roofline"]["frac_of_read_peak"] = round(gbs / best["gbs"], 4)
    if with_cpu:
        cb, ref = cpu_baseline(wl)
        out["cpu_baseline"] = cb
        if ref is not None:
            from oracle import gemv
            out["parity_rel_l2"] = gemv.rel_l2(wl.device_output(), ref)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="int4_8k")
    ap.add_argument("--all", default=None, help="append one JSON line per workload to this file")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the timed steps eagerly")
    ap.add_argument("--graph", action="store_true", help="replay the timed steps from one HIP graph "
                    "(default: eager up to %d steps, a graph above)" % EAGER_MAX_STEPS)
    ap.add_argument("--read-peak", type=int, default=0, metavar="BYTES",
                    help="only sweep the streaming-read probe over launch shapes for reads of BYTES per launch")
    ap.add_argument("--no-read-peak", action="store_true", help="leave the read-peak field out of the bench line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain elementwise copy (y = -x, fp32) reading and writing BYTES per "
                         "launch, --steps times: the reference kernel for scaling the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the hot path is a single-GPU kernel; a sharded run "
              "over several GPUs is not implemented (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": args.steps}), flush=True)
        return
    mode = False if args.no_graph else True if args.graph else None
    if args.all:
        for name in ALL:
            if name == args.workload:
                continue
            print("measuring", name, file=sys.stderr, flush=True)
            r = measure(name, dev, args.steps, args.warmup, with_cpu=False, use_graph=mode)
            with open(args.all, "a") as f:
                f.write(json.dumps(r) + "\n")
            torch.cuda.empty_cache()
    if args.read_peak:
        best, recs = read_peak(args.read_peak, dev, steps=args.steps)
        for r in recs:
            print(json.dumps(dict(r, bytes=best["bytes"])), flush=True)
        print(json.dumps({"read_peak": best, "peak_gbs": HBM_PEAK_GBS, "frac": round(best["gbs"] / HBM_PEAK_GBS, 4)}),
              flush=True)
        return
    res = measure(args.workload, dev, args.steps, args.warmup, with_cpu=not args.no_cpu, use_graph=mode,
                  with_read_peak=not args.no_read_peak)
    if args.all:
        with open(args.all, "a") as f:
            f.write(json.dumps(res) + "\n")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
