"""Benchmark: sliding-window (W=750) RoPE attention on one MI355X.

One step = the whole hot path on synthetic inputs already resident in HBM:
  * prefill of one encoder layer's attention, B1 T1500 H32 D64, bf16 in and
    out, RoPE fused into the tile loads (cos/sin table built once, outside the
    timed region, like any RoPE cache); a grid this small runs 64-query
    workgroups whose waves each take one half of every key tile;
  * one batched streaming step, 64 streams x 4 new frames, H32 D64, 750-slot
    bf16 rings: attention plus ring append in one call
    (vx_swa_attn_stream_step_append; the two-call form is timed beside it).
Positions advance 4 per step; two ring sets alternate so the working set
(786 MB) exceeds the 256 MB last-level cache; new frames cycle through 8
pre-drawn batches.

Printed value: prefill TFLOP/s over the unmasked band FLOPs
(4*64*pairs*H*B, pairs = W(W+1)/2 + (T-W)W), from HIP events around
back-to-back launches on the launch stream: every leg is timed in 5 passes
(at least 200 calls each for calls under a millisecond), interleaved with the
other legs, and the per-call median is reported.  The
streaming step runs 200 consecutive steps per pass with positions advancing
and is reported in microseconds and GB/s of algorithmic HBM bytes.  The CPU
baseline is the float64 oracle timed on the host on the same prefill
workload (all host threads, and one thread on a slice of it); the other
workloads' oracle times ride along, measured on a share and scaled where the
whole would take minutes.  `attainable` gives this GPU's measured bf16 GEMM
rate (hipBLASLt through torch) and device-copy bandwidth, for scale beside the
published peaks the rooflines use.

Beside the step, the same line reports the 32-layer attention stack (B4
T1500 per layer) and the long-form prefill (B8 T6000), the batched first-chunk
prefill, the
text decoder's grouped-query attention (32 query / 8 key-value heads,
head_dim 128, window 8192): one decode step of 64 streams over full 8192-slot
rings (ring append fused) and a 16384-token prompt prefill, each with its
roofline; the encoder's attention block (projections + attention); and the
whole streaming encoder step (conv stem + 32 layers, 64 streams x 4 frames).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0

# HBM bytes per launch measured with rocprofv3 (FETCH_SIZE and WRITE_SIZE passes, calibrated
# against a 1 GiB device copy: read = FETCH_SIZE x 2, written = WRITE_SIZE x 1), for the kernel
# sources whose SHA-256 is given.  A changed source reports null until it is measured again.
CSRC = os.path.join(ROOT, "sliding_window_attention_vx_amd", "csrc")
MEASURED_TRAFFIC = {
    "prefill": (("prefill_mfma.hip", "vx_device.h", "vx_launch.h"),
               "70385c15869df08b761bb7315b018f75da4ea7edaab5c8be07aa83d62461ef55",
               21_644_768 + 6_144_000),
    "stream": (("stream.hip", "vx_device.h", "vx_launch.h"),
              "735e9f9bf00ba20ab84eec779c6a8fe18c87926d3e6cd79d91dcdbc3f46b5cda",
              396_079_413 + 3_146_672),
    "first_chunk": (("prefill_mfma.hip", "vx_device.h", "vx_launch.h"),
                   "70385c15869df08b761bb7315b018f75da4ea7edaab5c8be07aa83d62461ef55",
                   155_812_800 + 107_363_920),
    "gqa_decode": (("gqa_decode.hip", "gqa_launch.h", "vx_device.h"),
                   "71d51d1bade315e29fb14b1164cdef63eb44efb65221e448a1e6a7302bfe4288",
                   2_148_346_558 + 786_944),
    "qkv": (("linear.hip", "linear_launch.h", "vx_device.h"),
            "1d6eb355dc43e46fce1a5168c9e141740c392831e2ec3de3bc91d3a938287d67",
            21_103_073 + 3_145_728),
    "oproj": (("linear.hip", "linear_launch.h", "vx_device.h"),
              "1d6eb355dc43e46fce1a5168c9e141740c392831e2ec3de3bc91d3a938287d67",
              13_718_730 + 655_360),
    "gqa_prefill": (("gqa_prefill.hip", "gqa_launch.h", "vx_device.h"),
                    "5feee362e008dbf0c8734e53c411e85c079a11a14a2749654e18950708698381",
                    450_948_348 + 134_504_800),
    "stack": (("prefill_mfma.hip", "vx_device.h", "vx_launch.h"),
             "70385c15869df08b761bb7315b018f75da4ea7edaab5c8be07aa83d62461ef55",
             103_764_736 + 24_576_000),
    "long": (("prefill_mfma.hip", "rope.hip", "vx_device.h", "vx_launch.h"),
            "a324a3a587e03e18df83ffe59dc4a70ad091cc8fcb18baec0de92f504796039c",
            (952_918_304 + 196_612_264) + (208_812_960 + 196_608_288)),
}


def measured_traffic(kind):
    """Bytes per launch from the counters if the kernel source is the one measured, else None."""
    import hashlib
    files, digest, nbytes = MEASURED_TRAFFIC[kind]
    if digest is None:
        return None
    m = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            m.update(fh.read())
    return nbytes if m.hexdigest() == digest else None


def band_flops(B, T, H, W, D=64):
    from sliding_window_attention_vx_amd.synth import band_pairs
    return 4.0 * D * band_pairs(T, W) * H * B


def stream_bytes(S, n, H, W, D=64, elem=2):
    """Algorithmic HBM bytes of one streaming step (attend + append).

    Per (stream, head): the ring keys and values the queries need (W-1 slots
    each, since the oldest slot's frame has left every query's window once
    the new frames arrive), the new q, k, v rows, the output rows, and the
    appended k and v rows; plus pos read and written per stream.
    """
    row = D * elem
    per_sh = 2 * (W - 1) * row + 3 * n * row + n * row + 2 * n * row
    return S * H * per_sh + S * 16


def gqa_decode_bytes(S, n, Hq, Hkv, W, D=128, elem=2):
    """Algorithmic HBM bytes of one grouped-query decode step (attend + append).

    Per (stream, key/value head): the W-1 ring keys and values the new
    tokens need, the G*n query rows and G*n output rows (G = Hq/Hkv), the n
    new key and value rows read and the same rows appended; plus pos read
    and written per stream.
    """
    row = D * elem
    G = Hq // Hkv
    per = 2 * (W - 1) * row + G * n * row + 2 * n * row + G * n * row + 2 * n * row
    return S * Hkv * per + S * 16


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=60,
                    help="oracle repetitions of the prefill workload for the CPU baseline")
    ap.add_argument("--only", choices=["prefill", "stream", "first_chunk", "gqa_prefill",
                                       "gqa_decode", "qkv", "oproj", "enc_block", "enc_step",
                                       "stack", "long", "copy"],
                    default=None,
                    help="profiling aid: launch only this kernel (or a plain device copy of "
                         "--copy-mib MiB, to calibrate HBM byte counters) and print its timing")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--enc-layers", type=int, default=None,
                    help="layers of the whole encoder step (default: the model's 32)")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the 32-layer stack and long-form prefill legs (their inputs take "
                         "about 30 s to draw on the host)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the work shards by batch, head or stream with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sliding_window_attention_vx_amd as vx
    from sliding_window_attention_vx_amd import synth

    if not os.path.exists(vx.LIB_PATH):
        from sliding_window_attention_vx_amd import build
        build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "copy":
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e_.record()
        torch.cuda.synchronize()
        us = s_.elapsed_time(e_) * 1e3 / args.steps
        print(json.dumps({"only": "copy", "bytes_read": n, "bytes_written": n, "us": round(us, 2),
                          "GBps_read_plus_write": round(2 * n / us / 1e3, 1)}))
        return

    def to(x, dt=torch.bfloat16):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev, dt)

    def need(*legs):
        # --only builds the inputs of its own leg only
        return args.only is None or args.only in legs

    # ---- prefill workload: one encoder layer, T=1500
    pc = synth.CONFIGS["layer"]
    x = synth.make_config("layer")
    q, k, v = to(x["q"]), to(x["k"]), to(x["v"])
    o = torch.empty_like(q)
    table = vx.rope_table(0, pc.T)
    flops = band_flops(pc.B, pc.T, pc.H, pc.W)
    # a 500-frame chunk of the same layer: 128 query tiles, half a query tile
    # per CU (the halves-split schedule, like the layer), and the same call
    # on the split walk (VX_FLAG_SPLIT_WALK with a workspace)
    spT = 500
    spq, spk, spv = q[:, :spT].contiguous(), k[:, :spT].contiguous(), v[:, :spT].contiguous()
    spo = torch.empty_like(spq)
    sws = vx.prefill_workspace(1, spT, pc.H, pc.W, force_split=True)
    sp_flops = band_flops(1, spT, pc.H, pc.W)

    # ---- streaming workload
    sc = synth.CONFIGS["stream"]
    rings = []
    for r in range(2 if need("stream") else 0):
        st = synth.make_stream_state(sc.S, sc.H, sc.W, seed=[sc.seed, r], pos_lo=sc.pos_lo,
                                     pos_hi=sc.pos_hi)
        p0 = torch.from_numpy(st["pos"].copy()).to(dev)
        # two position arrays per ring set: the fused call reads one, writes the other
        rings.append({"k": to(st["ring_k"]), "v": to(st["ring_v"]), "pos": [p0, p0.clone()],
                      "c": 0})
    frames = []
    for i in range(8 if need("stream") else 0):
        fr = synth.make_stream_frames(sc.S, sc.n, sc.H, seed=sc.seed, step=i)
        frames.append((to(fr["q"]), to(fr["k"]), to(fr["v"])))
    so = torch.empty_like(frames[0][0]) if frames else None
    sbytes = stream_bytes(sc.S, sc.n, sc.H, sc.W)

    # ---- batched first chunks (varlen prefill seeding the rings)
    fc = synth.FIRST_CHUNK
    fc_len = synth.first_chunk_lengths(fc["S"], fc["t_lo"], fc["t_hi"], seed=fc["seed"])
    xf = synth.make_first_chunks(fc["S"], fc["H"], fc_len, seed=fc["seed"], scale=fc["scale"])
    # (small: drawn for every leg)
    fq, fk, fv = to(xf["q"]), to(xf["k"]), to(xf["v"])
    fcu = torch.from_numpy(xf["cu"]).to(dev)
    fo = torch.empty_like(fq)
    frk = torch.zeros((fc["S"], fc["H"], fc["W"], 64), dtype=torch.bfloat16, device=dev)
    frv = torch.zeros_like(frk)
    fpos = torch.zeros(fc["S"], dtype=torch.int64, device=dev)
    ftab = vx.rope_table(0, fc["t_hi"])
    fc_flops = sum(4.0 * 64 * synth.band_pairs(int(t), fc["W"]) * fc["H"] for t in fc_len)
    # algorithmic bytes: q, k, v read, o written, the seeded ring rows (each
    # stream's last W frames, rotated keys and values) and pos written
    fc_tot = int(xf["cu"][-1])
    fc_bytes = (4 * fc_tot * fc["H"] * 128
                + 2 * sum(min(int(t), fc["W"]) for t in fc_len) * fc["H"] * 128 + 8 * fc["S"])
    fc_slices = [(int(xf["cu"][i]), int(xf["cu"][i + 1])) for i in range(fc["S"])]

    # ---- 32-layer attention stack (B4 T1500, fresh seeded Q/K/V per layer) and long-form
    # prefill (B8 T6000, 1 % of key rows x8), both with fused RoPE; each call gets a
    # workspace, in which grids of at least 8 query tiles per CU (the long form, the
    # stack as one B128 call) keep their keys rotated once, ahead of the attention
    # kernel (the same bits as rotating them in the kernel's staging)
    stack_in, long_in = [], None
    if not args.no_stack and args.only in (None, "stack", "long"):
        stc, lgc = synth.CONFIGS["stack"], synth.CONFIGS["long"]
        for l in range(stc.layers):
            xx = synth.make_config("stack", layer=l)
            stack_in.append((to(xx["q"]), to(xx["k"]), to(xx["v"])))
        stack_o = torch.empty_like(stack_in[0][0])
        xx = synth.make_config("long")
        long_in = (to(xx["q"]), to(xx["k"]), to(xx["v"]))
        del xx
        long_o = torch.empty_like(long_in[0])
        long_tab = vx.rope_table(0, lgc.T)
        stack_ws = vx.prefill_workspace(stc.B, stc.T, stc.H, stc.W)
        long_ws = vx.prefill_workspace(lgc.B, lgc.T, lgc.H, lgc.W)
        stack_flops = band_flops(stc.B, stc.T, stc.H, stc.W) * stc.layers
        long_flops = band_flops(lgc.B, lgc.T, lgc.H, lgc.W)

    def stack_pass(i):
        for sq, sk, sv in stack_in:
            vx.prefill(sq, sk, sv, window=stc.W, table=table, out=stack_o, workspace=stack_ws)

    # the same 32 layers as one call of B = 128 (an upper bound: one launch,
    # four times the workgroups of a layer)
    stack_all = None
    if stack_in and args.only is None:
        stack_all = tuple(torch.cat([l_[j] for l_ in stack_in]) for j in range(3))
        stack_all_o = torch.empty_like(stack_all[0])
        stack_all_ws = vx.prefill_workspace(stack_all[0].shape[0], stc.T, stc.H, stc.W)

    def stack_one_call(i):
        vx.prefill(*stack_all, window=stc.W, table=table, out=stack_all_o, workspace=stack_all_ws)

    def long_pass(i):
        vx.prefill(*long_in, window=lgc.W, table=long_tab, out=long_o, workspace=long_ws)

    # one stack layer on q and k rotated upstream (RoPE applied by the q/k/v
    # projection's epilogue, as in the encoder step): no cos/sin staging at all
    def stack_layer_rope_upstream(i):
        sq, sk, sv = stack_in[0]
        vx.prefill(sq, sk, sv, window=stc.W, rope_applied=True, out=stack_o)

    # the same call without a workspace: keys rotated in the kernel's staging
    def long_in_kernel(i):
        vx.prefill(*long_in, window=lgc.W, table=long_tab, out=long_o)

    # ---- text decoder (grouped-query attention, head_dim 128)
    dc = synth.GQA_CONFIGS["dec_decode"]
    gc = synth.GQA_CONFIGS["dec_prefill"]
    dbytes = gqa_decode_bytes(dc.B, dc.T, dc.Hq, dc.Hkv, dc.W)
    g_flops = band_flops(gc.B, gc.T, gc.Hq, gc.W, D=gc.D)
    dring, dframes, do = {}, [], None
    if need("gqa_decode"):
        dst = synth.make_gqa_decode_state("dec_decode")
        dring = {"k": to(dst["ring_k"]), "v": to(dst["ring_v"]), "c": 0,
                 "pos": [torch.from_numpy(dst["pos"].copy()).to(dev)]}
        dring["pos"].append(dring["pos"][0].clone())
        del dst
        for i in range(8):
            fr = synth.make_gqa_frames(dc.B, dc.T, dc.Hq, dc.Hkv, seed=dc.seed, step=i)
            dframes.append((to(fr["q"]), to(fr["k"]), to(fr["v"])))
        do = torch.empty_like(dframes[0][0])
    if need("gqa_prefill"):
        xg = synth.make_gqa_config("dec_prefill")
        gq, gk, gv = to(xg["q"]), to(xg["k"]), to(xg["v"])
        del xg
        go = torch.empty_like(gq)
        gkr = torch.empty_like(gk)  # rotated keys, written once per call
        gtab = vx.rope_table(0, gc.T, head_dim=vx.DEC_HEAD_DIM)

    def gqa_decode(i):
        qn, kn, vn = dframes[i % 8]
        c = dring["c"]
        vx.gqa_decode(qn, kn, vn, dring["k"], dring["v"], dring["pos"][c % 2],
                      dring["pos"][(c + 1) % 2], window=dc.W, out=do)
        dring["c"] = c + 1

    def gqa_prefill(i):
        vx.gqa_prefill(gq, gk, gv, window=gc.W, table=gtab, out=go, k_rot=gkr)

    def gqa_prefill_fused(i):
        vx.gqa_prefill(gq, gk, gv, window=gc.W, table=gtab, out=go)

    # ---- encoder attention block: q/k/v projection + RoPE, attention step, output projection
    ec = synth.ENC_BLOCK
    if need("enc_block", "qkv", "oproj", "enc_step"):
        ew = {k_: to(v_) for k_, v_ in synth.make_enc_block_weights(ec["d_model"], ec["H"],
                                                                     seed=ec["seed"]).items()}
        est = synth.make_stream_state(ec["S"], ec["H"], ec["W"], seed=[ec["seed"], 1],
                                      pos_lo=ec["pos_lo"], pos_hi=ec["pos_hi"])
        ering = {"k": to(est["ring_k"]), "v": to(est["ring_v"]), "c": 0,
                 "pos": [torch.from_numpy(est["pos"].copy()).to(dev)]}
        ering["pos"].append(ering["pos"][0].clone())
        del est
        ex = [to(synth.make_enc_block_input(ec["S"], ec["n"], ec["d_model"], seed=ec["seed"],
                                            step=i)) for i in range(8)]
        eshape = (ec["S"], ec["n"], ec["H"], 64)
        ework = {k_: torch.empty(eshape, dtype=torch.bfloat16, device=dev) for k_ in "qkvo"}
        ey = torch.empty_like(ex[0])
    eM, eHD, edm = ec["S"] * ec["n"], ec["H"] * 64, ec["d_model"]
    qkv_bytes = 3 * eHD * edm * 2 + eM * edm * 2 + 3 * eM * eHD * 2 + 2 * eHD * 2 + ec["S"] * 8
    oproj_bytes = edm * eHD * 2 + eM * eHD * 2 + eM * edm * 2 + edm * 2
    blk_bytes = qkv_bytes + stream_bytes(ec["S"], ec["n"], ec["H"], ec["W"]) + oproj_bytes

    def enc_block(i):
        c = ering["c"]
        vx.enc_attn_step(ex[i % 8], ew["w_qkv"], ew["b_q"], ew["b_v"], ew["w_o"], ew["b_o"],
                         ering["k"], ering["v"], ering["pos"][c % 2], ering["pos"][(c + 1) % 2],
                         window=ec["W"], H=ec["H"], work=ework, out=ey)
        ering["c"] = c + 1

    def qkv(i):
        vx.enc_qkv_rope(ex[i % 8], ew["w_qkv"], ew["b_q"], ew["b_v"], ering["pos"][0], H=ec["H"],
                        q=ework["q"], k=ework["k"], v=ework["v"])

    def oproj(i):
        vx.linear(ework["o"].view(eM, eHD), ew["w_o"], ew["b_o"], out=ey.view(eM, edm))

    # ---- whole streaming encoder step: conv stem + 32 pre-norm layers, 64 streams x 4 frames;
    # every layer's rings start as the encoder-block leg's full-ring draw
    cs = synth.ENC_STEP
    sL = args.enc_layers or cs["L"]
    sS, sn, sH, sdm, sffn, snm = cs["S"], cs["n"], cs["H"], cs["d_model"], cs["ffn"], cs["n_mels"]
    s_state = {"c": 0}
    if need("enc_step"):
        s_stem = {k_: to(v_) for k_, v_ in synth.make_enc_stem_weights(sdm, snm,
                                                                        seed=cs["seed"]).items()}
        s_layers = [{k_: to(v_) for k_, v_ in synth.make_enc_layer_weights(
            sdm, sH, sffn, seed=cs["seed"], layer=l).items()} for l in range(sL)]
        s_rk = ering["k"].unsqueeze(0).repeat(sL, 1, 1, 1, 1)
        s_rv = ering["v"].unsqueeze(0).repeat(sL, 1, 1, 1, 1)
        s_pos = [ering["pos"][0].clone(), ering["pos"][0].clone()]
        s_mel = [to(synth.make_mel(sS, 2 * sn, snm, seed=cs["seed"], step=i)) for i in range(8)]
        s_melbuf = torch.zeros((sS, 2 * sn + 2, snm), dtype=torch.bfloat16, device=dev)
        s_c1buf = torch.zeros((sS, 2 * sn + 2, sdm), dtype=torch.bfloat16, device=dev)
        s_x = torch.empty((sS, sn, sdm), dtype=torch.float32, device=dev)
        s_work = vx.enc_work(sS, sn, sH, sdm, sffn, device=dev)
    sM, sHD, sF = sS * sn, sH * 64, 2 * sn + 2
    s_stem_bytes = (sdm * 3 * snm * 2 + sS * sF * snm * 2 + sS * 2 * sn * sdm * 2  # conv1
                    + sdm * 3 * sdm * 2 + sS * sF * sdm * 2 + sM * sdm * 4          # conv2
                    + 2 * sS * 2 * (snm + sdm) * 2 + 2 * 2 * sdm)                   # shift, biases
    # per layer: each RMSNorm reads x and writes h; the output and down
    # projections read their weights and inputs and update x (read + write);
    # the split products' partial sums stay out (an implementation choice)
    s_layer_bytes = (2 * (sM * sdm * 4 + sM * sdm * 2 + sdm * 2)                    # two RMSNorms
                     + qkv_bytes + stream_bytes(sS, sn, sH, cs["W"])                # attention
                     + sdm * sHD * 2 + sM * sHD * 2 + 2 * sM * sdm * 4 + sdm * 2   # out proj
                     + 2 * sffn * sdm * 2 + sM * sdm * 2 + sM * sffn * 2           # gate/up
                     + sdm * sffn * 2 + sM * sffn * 2 + 2 * sM * sdm * 4 + sdm * 2)  # down
    s_bytes = s_stem_bytes + sL * s_layer_bytes

    def enc_step(i):
        c = s_state["c"]
        s_melbuf[:, 2:].copy_(s_mel[i % 8])
        vx.enc_step(s_melbuf, s_c1buf, s_stem, s_layers, s_rk, s_rv, s_pos[c % 2],
                    s_pos[(c + 1) % 2], x=s_x, window=cs["W"], H=sH, work=s_work)
        s_state["c"] = c + 1

    def prefill():
        vx.prefill(q, k, v, window=pc.W, table=table, out=o)

    def stream(i):
        R = rings[i % 2]
        qn, kn, vn = frames[i % 8]
        pos = R["pos"][R["c"] % 2]
        vx.stream_step(qn, kn, vn, R["k"], R["v"], pos, window=sc.W, out=so)
        return R["k"], R["v"], pos, kn, vn

    def append(args_):
        rk, rv, pos, kn, vn = args_
        vx.ring_append(rk, rv, kn, vn, pos, window=sc.W)

    def stream_fused(i):
        R = rings[i % 2]
        qn, kn, vn = frames[i % 8]
        c = R["c"]
        vx.stream_step_append(qn, kn, vn, R["k"], R["v"], R["pos"][c % 2], R["pos"][(c + 1) % 2],
                              window=sc.W, out=so)
        R["c"] = c + 1

    def step(i):
        prefill()
        stream_fused(i)

    if args.only is not None:
        fn = {"prefill": lambda j: prefill(), "stream": stream_fused,
              "first_chunk": lambda j: vx.prefill_varlen(fq, fk, fv, fcu, fc["t_hi"],
                                                         window=fc["W"], table=ftab, ring_k=frk,
                                                         ring_v=frv, pos=fpos, out=fo),
              "gqa_prefill": gqa_prefill, "gqa_decode": gqa_decode, "qkv": qkv, "oproj": oproj,
              "enc_block": enc_block, "enc_step": enc_step,
              "stack": lambda j: vx.prefill(*stack_in[j % len(stack_in)], window=stc.W,
                                            table=table, out=stack_o, workspace=stack_ws),
              "long": long_pass}[args.only]
        for j in range(args.warmup):
            fn(j)
        torch.cuda.synchronize()
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        for j in range(args.steps):
            fn(j)
        e_.record()
        torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "us_per_launch": round(s_.elapsed_time(e_) * 1e3 /
                                                                     args.steps, 3)}))
        return

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, with per-kernel events on the launch stream
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        e = evs[i]
        e[0].record()
        prefill()
        e[1].record()
        stream_fused(args.warmup + i)
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / K
    pre_in_step = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3
    str_in_step = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3

    # ---- per-call durations: back-to-back launches between two events on the
    # launch stream, 5 passes interleaved over the legs, median per leg
    def time_launches(fn, reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for j in range(reps):
            fn(j)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e3 / reps

    # at least 200 back-to-back calls per pass, so the pass's start (the first
    # launch reaching an idle GPU) weighs under 1 % of a 25 us call
    reps = max(K, 200)

    # the layer prefill as one HIP graph of 100 launches (no host launch cost
    # between kernels); the library's calls allocate nothing, so they capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prefill()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    pre_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(pre_graph):
        for _ in range(100):
            prefill()
    pre_graph.replay()
    torch.cuda.synchronize()

    # the whole encoder step captured as a HIP graph: two steps (the position
    # arrays ping-pong), so every replay advances the streams like the eager loop
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc_step(0)
        enc_step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    encs_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(encs_graph):
        s_state["c"] = 0
        enc_step(0)
        enc_step(1)
    encs_graph.replay()
    torch.cuda.synchronize()

    def serial_first_chunks(j):
        for a_, b_ in fc_slices:
            vx.prefill(fq[a_:b_][None], fk[a_:b_][None], fv[a_:b_][None], window=fc["W"],
                       table=ftab, out=fo[a_:b_][None])

    # name -> (function of the call index, calls per pass, calls counted per pass)
    legs = {
        "prefill": (lambda j: prefill(), reps, reps),
        "prefill_graph": (lambda j: pre_graph.replay(), 1, 100),
        # the same attention with q and k rotated upstream, as when the q/k/v
        # projection's epilogue applies RoPE (reported beside the fused figure)
        "prefill_rope_upstream": (lambda j: vx.prefill(q, k, v, window=pc.W, rope_applied=True,
                                                       out=o), reps, reps),
        # the 500-frame chunk on the default schedule, and on the split walk
        "chunk500": (lambda j: vx.prefill(spq, spk, spv, window=pc.W, table=table, out=spo),
                     reps, reps),
        "chunk500_split_walk": (lambda j: vx.prefill(spq, spk, spv, window=pc.W, table=table,
                                                     out=spo, workspace=sws, force_split=True),
                                reps, reps),
        # the cos/sin rows of the layer's 1500 positions (a cache built once per
        # position range, outside the headline)
        "rope_table": (lambda j: vx.rope_table(0, pc.T, out=table), reps, reps),
        # 200 consecutive steps with positions advancing, per pass
        "stream_step": (stream_fused, 200, 200),
        "stream_attend": (lambda j: stream(j), reps, reps),
        "stream_two_calls": (lambda j: append(stream(j)), reps, reps),
        "first_chunk": (lambda j: vx.prefill_varlen(fq, fk, fv, fcu, fc["t_hi"], window=fc["W"],
                                                    table=ftab, ring_k=frk, ring_v=frv, pos=fpos,
                                                    out=fo), reps, reps),
        "first_chunk_serial": (serial_first_chunks, max(K // 4, 5), max(K // 4, 5)),
        "enc_block": (enc_block, reps, reps),
        "qkv": (qkv, reps, reps),
        "oproj": (oproj, reps, reps),
        "enc_step": (enc_step, max(K // 5, 4), max(K // 5, 4)),
        "enc_step_graph": (lambda j: encs_graph.replay(), max(K // 10, 2), 2 * max(K // 10, 2)),
        "gqa_decode": (gqa_decode, reps, reps),
        "gqa_prefill": (gqa_prefill, max(K // 5, 4), max(K // 5, 4)),
        "gqa_prefill_fused": (gqa_prefill_fused, max(K // 5, 4), max(K // 5, 4)),
    }
    if stack_in:
        legs["stack"] = (stack_pass, 1, 1)
        legs["stack_one_call"] = (stack_one_call, 1, 1)
        legs["long"] = (long_pass, max(K // 5, 4), max(K // 5, 4))
        legs["long_in_kernel"] = (long_in_kernel, max(K // 5, 4), max(K // 5, 4))
        legs["stack_layer_rope_upstream"] = (stack_layer_rope_upstream, reps, reps)
    for name, (fn, n_, _) in legs.items():
        fn(-1)  # first-launch and first-touch costs stay out of the passes
    torch.cuda.synchronize()
    PASSES = 5
    samples = {name: [] for name in legs}
    for _ in range(PASSES):
        for name, (fn, n_, per) in legs.items():
            samples[name].append(time_launches(fn, n_) * n_ / per)
    med = {name: float(np.median(v_)) for name, v_ in samples.items()}
    pre_us, pre_graph_us, pre_rot_us = med["prefill"], med["prefill_graph"], med["prefill_rope_upstream"]
    step_us, attend_us, two_call_us = med["stream_step"], med["stream_attend"], med["stream_two_calls"]
    fc_us, fc_serial_us = med["first_chunk"], med["first_chunk_serial"]
    blk_us, qkv_us, oproj_us = med["enc_block"], med["qkv"], med["oproj"]
    encs_us, encs_graph_us = med["enc_step"], med["enc_step_graph"]
    dec_us, gpre_us, gpre_fused_us = med["gqa_decode"], med["gqa_prefill"], med["gqa_prefill_fused"]
    if stack_in:
        stack_us, stack_one_us, long_us = med["stack"], med["stack_one_call"], med["long"]

    tflops = flops / (pre_us * 1e-6) / 1e12
    stream_gbs = sbytes / (step_us * 1e-6) / 1e9

    out = {
        "metric": "SWA-750 attention TFLOP/s (T=1500, 32h x 64, bf16) + streaming step us",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill B1 T1500 H32 D64 W750 bf16 (RoPE theta 1e6 fused) + streaming "
                        "step S64 n4 H32 D64 W750 bf16 (attend + ring append)",
            "global_batch": pc.B,
            "seq_len": pc.T,
            "parallelism": "none (one GPU)",
        },
        "timing": "per-call median of 5 passes interleaved over the legs (HIP events around "
                  "back-to-back launches, at least 200 calls per pass for calls under a "
                  "millisecond); the streaming step over 200 consecutive steps per pass",
        "prefill_us": round(pre_us, 3),
        "prefill_us_passes": [round(x_, 3) for x_ in samples["prefill"]],
        "prefill_us_graph": round(pre_graph_us, 3),
        "prefill_us_rope_upstream": round(pre_rot_us, 3),
        "rope_table_us": round(med["rope_table"], 3),
        "chunk500": {
            "workload": f"prefill B1 T{spT} H{pc.H} D64 W{pc.W} bf16 (RoPE fused): 128 query "
                        "tiles of 128, run as 64-query workgroups whose waves split each key "
                        "tile's halves",
            "us": round(med["chunk500"], 3),
            "tflops": round(sp_flops / (med["chunk500"] * 1e-6) / 1e12, 2),
            "us_split_walk": round(med["chunk500_split_walk"], 3),
        },
        "stream_step_us": round(step_us, 3),
        "stream_step_two_calls_us": round(two_call_us, 3),
        "stream_attend_only_us": round(attend_us, 3),
        "in_step_event_us": {"prefill": round(pre_in_step, 3), "stream_step": round(str_in_step, 3)},
        "roofline": {
            "kernel": "prefill_mfma_kernel",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill"),
        },
        "roofline_stream": {
            "kernel": "stream_step_mfma_kernel",
            "bound": "hbm",
            "achieved": round(stream_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(stream_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("stream"),
        },
    }

    out["first_chunk"] = {
        "workload": f"{fc['S']} streams x first chunks of {fc['t_lo']}..{fc['t_hi']} frames "
                    f"(varlen, {int(xf['cu'][-1])} frames), H{fc['H']} D64 W{fc['W']} bf16, RoPE "
                    "fused, rings seeded",
        "us_per_call": round(fc_us, 3),
        "tflops": round(fc_flops / (fc_us * 1e-6) / 1e12, 2),
        "serialized_us": round(fc_serial_us, 3),
        "batching_speedup": round(fc_serial_us / fc_us, 2),
        # about 23 flops per byte, far below the 312 flop/B ridge: HBM-bound
        "roofline": {"bound": "hbm", "achieved": round(fc_bytes / (fc_us * 1e-6) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(fc_bytes / (fc_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic("first_chunk")},
    }

    dec_gbs = dbytes / (dec_us * 1e-6) / 1e9
    g_tflops = g_flops / (gpre_us * 1e-6) / 1e12
    out["decoder"] = {
        "decode": {
            "workload": f"grouped-query decode step S{dc.B} n{dc.T} Hq{dc.Hq} Hkv{dc.Hkv} "
                        f"D{dc.D} W{dc.W} bf16, full rings, RoPE fused, ring append fused",
            "us_per_step": round(dec_us, 3),
            "roofline": {"kernel": "gqa_decode_kernel", "bound": "hbm",
                         "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("gqa_decode")},
        },
        "prefill": {
            "workload": f"grouped-query prefill B{gc.B} T{gc.T} Hq{gc.Hq} Hkv{gc.Hkv} D{gc.D} "
                        f"W{gc.W} bf16, RoPE in the call (keys rotated once into k_rot, queries "
                        f"in the attention kernel)",
            "us_per_call": round(gpre_us, 3),
            "us_single_kernel_fused_rope": round(gpre_fused_us, 3),
            "roofline": {"kernel": "gqa_prefill_kernel", "bound": "mfma",
                         "achieved": round(g_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(g_tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("gqa_prefill")},
        },
    }

    out["enc_block"] = {
        "workload": f"encoder attention block step S{ec['S']} n{ec['n']} d_model {edm} "
                    f"H{ec['H']} D64 W{ec['W']} bf16: q/k/v projection with RoPE, attention "
                    f"step with ring append, output projection (three launches)",
        "us_per_step": round(blk_us, 3),
        "GBps_algorithmic": round(blk_bytes / (blk_us * 1e-6) / 1e9, 1),
        "qkv_rope_us": round(qkv_us, 3),
        "out_proj_us": round(oproj_us, 3),
        "roofline_qkv": {"kernel": "linear_kernel (q/k/v + RoPE epilogue)", "bound": "hbm",
                         "achieved": round(qkv_bytes / (qkv_us * 1e-6) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(qkv_bytes / (qkv_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("qkv")},
        "roofline_out_proj": {"kernel": "linear_kernel (bias epilogue)", "bound": "hbm",
                              "achieved": round(oproj_bytes / (oproj_us * 1e-6) / 1e9, 1),
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(oproj_bytes / (oproj_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                            4),
                              "traffic": measured_traffic("oproj")},
    }

    if stack_in:
        stack_tf = stack_flops / (stack_us * 1e-6) / 1e12
        long_tf = long_flops / (long_us * 1e-6) / 1e12
        out["stack"] = {
            "workload": f"{stc.layers} layers x prefill B{stc.B} T{stc.T} H{stc.H} D64 W{stc.W} bf16, "
                        "fresh Q/K/V per layer, RoPE fused, one call per layer (the B128 "
                        "call rotates its keys once, ahead of the attention kernel)",
            "us_per_stack": round(stack_us, 3),
            "us_per_layer": round(stack_us / stc.layers, 3),
            "us_per_layer_rope_upstream": round(med["stack_layer_rope_upstream"], 3),
            "us_one_call_B128": round(stack_one_us, 3),
            "tflops_one_call_B128": round(stack_flops / (stack_one_us * 1e-6) / 1e12, 2),
            "roofline": {"kernel": "prefill_mfma_kernel", "bound": "mfma",
                         "achieved": round(stack_tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(stack_tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("stack")},
        }
        out["long"] = {
            "workload": f"prefill B{lgc.B} T{lgc.T} H{lgc.H} D64 W{lgc.W} bf16, 1 % of key rows x8, "
                        "RoPE fused (keys rotated once, ahead of the attention kernel)",
            "us_per_call": round(long_us, 3),
            "us_per_call_keys_rotated_in_kernel": round(med["long_in_kernel"], 3),
            "roofline": {"kernel": "rope_k_table_kernel + prefill_mfma_kernel (per call)",
                         "bound": "mfma",
                         "achieved": round(long_tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(long_tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": measured_traffic("long")},
        }

    encs_gbs = s_bytes / (encs_us * 1e-6) / 1e9
    out["enc_step"] = {
        "workload": f"whole streaming encoder step S{sS} x {2 * sn} mel frames -> {sn} frames: "
                    f"causal conv stem ({snm}->{sdm} k3 s1, {sdm}->{sdm} k3 s2, GELU) + {sL} "
                    f"pre-norm layers (d_model {sdm}, H{sH} D64 W{cs['W']}, SwiGLU FFN {sffn}), "
                    f"bf16 weights/activations, float32 residual, {4 + 7 * sL} launches",
        "us_per_step": round(encs_us, 3),
        "us_per_step_graph": round(encs_graph_us, 3),
        "encoder_frames_per_s": round(sM / (encs_us * 1e-6), 1),
        "audio_s_per_s": round(sS * 0.08 / (encs_us * 1e-6), 1),
        "bytes_algorithmic": int(s_bytes),
        "roofline": {"kernel": "whole step (all launches)", "bound": "hbm",
                     "achieved": round(encs_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(encs_gbs / PEAK_HBM_GBS, 4), "traffic": None},
    }

    # attainable peaks on this GPU, for scale beside the published ones: a large
    # bf16 GEMM through torch (hipBLASLt) and a 1 GiB device-to-device copy
    ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gc_ = torch.empty(8192, 8192, device=dev, dtype=torch.bfloat16)
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_src.fill_(1)
    torch.matmul(ga, gb, out=gc_)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    gemm_us = float(np.median([time_launches(lambda j: torch.matmul(ga, gb, out=gc_), 5)
                               for _ in range(5)]))
    copy_us = float(np.median([time_launches(lambda j: cp_dst.copy_(cp_src), 5)
                               for _ in range(5)]))
    out["attainable"] = {
        "bf16_gemm_tflops": round(2 * 8192 ** 3 / gemm_us / 1e6, 1),
        "hbm_copy_gbs": round(2 * (1 << 30) / copy_us / 1e3, 1),
        "how": "torch.matmul of two 8192x8192 bf16 matrices (hipBLASLt) and a 1 GiB "
               "device-to-device copy (bytes read + written), medians of 5 passes of 5",
    }
    del ga, gb, gc_, cp_src, cp_dst

    if not args.no_cpu_baseline:
        import oracle
        nt = len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        for _ in range(args.cpu_reps):
            oracle.prefill(x["q"], x["k"], x["v"], pc.W, bf16=True, nthreads=nt)
        cpu_s = time.perf_counter() - t0
        # one thread on 4 of the 32 heads (the oracle's work is per (batch, head))
        hs = slice(0, 4)
        t1 = time.perf_counter()
        oracle.prefill(x["q"][:, :, hs], x["k"][:, :, hs], x["v"][:, :, hs], pc.W, bf16=True,
                       nthreads=1)
        one_s = time.perf_counter() - t1
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as fh:
                for line in fh:
                    if line.startswith("model name"):
                        cpu_model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        # the other workloads on the oracle: the tiny fp32 case and one streaming
        # step's worth in full or by a share scaled to the whole (labelled)
        others = {}

        def timed(fn):
            t = time.perf_counter()
            fn()
            return time.perf_counter() - t

        c1 = synth.CONFIGS["tiny"]
        x1 = synth.make_prefill(c1.B, c1.T, c1.H, seed=c1.seed, dtype=c1.dtype, scale=c1.scale)
        t_c1 = timed(lambda: oracle.prefill(x1["q"], x1["k"], x1["v"], c1.W, nthreads=nt))
        others["tiny_B1_T64_H4_W16_f32"] = {"seconds": round(t_c1, 6), "extrapolated": False}
        # one streaming step of 8 of the 64 streams (per-stream work is the same), x8
        sc_ = synth.CONFIGS["stream"]
        st8 = synth.make_stream_state(8, sc_.H, sc_.W, seed=[sc_.seed, 99], pos_lo=sc_.pos_lo,
                                      pos_hi=sc_.pos_hi)
        fr8 = synth.make_stream_frames(8, sc_.n, sc_.H, seed=[sc_.seed, 99], step=0)
        t_c4 = timed(lambda: oracle.stream_step(fr8["q"], fr8["k"], fr8["v"], st8["ring_k"],
                                                st8["ring_v"], st8["pos"], sc_.W, bf16=True,
                                                nthreads=nt)) * (sc_.S / 8)
        others["stream_step_S64_n4"] = {"seconds": round(t_c4, 4),
                                        "GBps": round(sbytes / t_c4 / 1e9, 3),
                                        "extrapolated": True,
                                        "sample": "8 of the 64 streams, one step, x8"}
        del st8, fr8
        # the stack: one batch entry of layer 0 (1/128 of the 32 layers x B4), x128
        x3 = synth.make_prefill(1, pc.T, pc.H, seed=[3, 0], dtype="bf16", scale=0.5)
        t_c3 = timed(lambda: oracle.prefill(x3["q"], x3["k"], x3["v"], pc.W, bf16=True,
                                            nthreads=nt)) * 128
        others["stack_32x_B4_T1500"] = {"seconds": round(t_c3, 2),
                                        "tflops": round(128 * flops / t_c3 / 1e12, 6),
                                        "extrapolated": True,
                                        "sample": "layer 0, batch entry 0, x128"}
        # the long form: batch entry 0 (1/8), x8
        x5 = synth.make_prefill(1, 6000, pc.H, seed=[5, 0], dtype="bf16", scale=1.0)
        f5 = band_flops(1, 6000, pc.H, pc.W)
        t_c5 = timed(lambda: oracle.prefill(x5["q"], x5["k"], x5["v"], pc.W, bf16=True,
                                            nthreads=nt)) * 8
        others["long_B8_T6000"] = {"seconds": round(t_c5, 2),
                                   "tflops": round(8 * f5 / t_c5 / 1e12, 6),
                                   "extrapolated": True, "sample": "batch entry 0, x8"}
        out["cpu_baseline"] = {
            "value": round(flops * args.cpu_reps / cpu_s / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": nt,
            "kind": "oracle",
            "sample": f"float64 oracle (bf16 contract), the full prefill workload B1 T1500 H32 "
                      f"W750 x {args.cpu_reps} repetitions, {cpu_s:.1f} s on {nt} threads; one "
                      f"thread: 4 of the 32 heads once, {one_s:.2f} s",
            "value_1thread": round(flops / 8 / one_s / 1e12, 6),
            "cpu_model": cpu_model,
            "other_workloads": others,
        }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
