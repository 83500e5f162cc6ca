#!/usr/bin/env python3
"""Throughput of the RWKV-7 WKV7 / time-mix hot path on one MI355X.

Prints ONE JSON line.  By default every workload below runs in turn; the
line's headline ("value") is the streaming decode, and "configs" holds one
record per workload (median ms per step, throughput, roofline of its
dominant kernel, CPU-oracle baseline).  --workload NAME runs one of them as
the headline alone.  Workloads:
  wkv7_small WKV7 forward+backward, B=1 T=64 H=4 N=64, fp32 (the small
             configuration; latency bound: microseconds per step)
  decode     streaming decode through a 12-layer RWKV-7 stack,
             C=256 H=4 FFN 1024, LoRA 32/32/32/64, vocab 256, 2048
             independent streams, fp32, one token per stream per step
             (steps/s); the step is replayed from a captured HIP graph
  timemix    time-mix block forward+backward, B=8 T=1024 C=768 (H=12),
             LoRA ranks w/a/v/g = 64/64/32/128, layer > 0, fp32 (tokens/s)
  wkv7_long  WKV7 forward+backward, B=4 T=8192 H=32 N=64, bf16 token
             tensors, fp32 state, checkpointed backward (tokens/s)
  online     online TBPTT training segments on the decode model (12 layers,
             C=256, vocab 256): 256 streams x 64 steps from their live state,
             backward through the segment, Adam update, live-state replay,
             fp32 (tokens/s)
  hybrid     hybrid training step: 12 RWKV-7 blocks and 4 MoBA attention
             blocks (one after every three), C=1024 H=16 FFN 4096, vocab 65536,
             B=4 T=2048, attention in chunks of 64 with top-4 chunks, bf16
             GEMM operands (tokens/s)
  gdn        GatedDeltaNet layer forward + through-gradient backward, B=2
             windows of T=4096, 12 key heads / 24 value heads of size 128,
             4 causal conv taps, fp32 (tokens/s)
  train      full training step: 24 blocks C=1024 H=16 FFN 4096, vocab
             65536, B=4 T=2048, embedding, LM head, fused CE, forward +
             backward; GEMMs with bf16 operands and fp32 accumulation,
             recurrence and elementwise steps fp32 (tokens/s)
A step is one pass of the whole workload over one batch of seeded synthetic
inputs that are resident in HBM before timing starts.  Each step is timed
with its own pair of HIP events on the stream the library launches on; the
K timed steps are bracketed by device synchronisation, and ms_per_step is
their median (the mean is reported beside it).

"roofline" reports the workload's dominant kernel, timed live here on the
same stream over its own loop of launches (HIP events), against MI355X peak.
"cpu_baseline" times the f64 CPU oracle on a bounded sample of the same
workload on the host cores (rank 0, one GPU only).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WKV7 time-mix fwd+bwd tokens/s and decode steps/s; % of HBM/MFMA peak"
PEAK = {"hbm": (8000.0, "GB/s"), "mfma_fp32": (157.3, "TFLOP/s"), "alu_fp32": (157.3, "TFLOP/s"),
        "mfma_bf16": (2500.0, "TFLOP/s")}
PEAK_ALU_NO_PACKED = 256 * 64 * 2 * 2.4e9 / 1e12  # 78.6 TFLOP/s
# The time-mix and training-step workloads overlap their weight-gradient GEMMs
# with the rest of the backward on the library's side stream; --one-stream runs
# them on the caller's stream alone, so that a counter run times every kernel
# by itself.
OPTS = {"side": True}
N = 64


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


CPU_MIN_S = 10.0  # seconds of oracle work per cpu_baseline sample


def repeat_for(fn, min_s=CPU_MIN_S):
    """Run fn until at least min_s seconds have passed: (repetitions, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return reps, dt


def time_calls(fn, iters):
    """Per-call ms of `iters` calls of fn(): one pair of HIP events per call on
    the current stream (the stream the library launches on), bracketed by
    device synchronisation.  Returns (median, mean, wall seconds)."""
    import statistics

    import torch
    ev = [_events() for _ in range(iters)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in ev]
    return statistics.median(ms), sum(ms) / len(ms), wall


def traffic_from_profile(kernel_key, src_files):
    """HBM bytes per launch from committed rocprofv3 --pmc counters, or None.

    profiles/pmc_<kernel_key>.json holds the FETCH_SIZE/WRITE_SIZE derived bytes
    and a hash of the kernel sources at measurement time; a changed source
    makes the figure stale (None).
    """
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in src_files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


# --------------------------------------------------------------- workloads --
def setup_wkv7_small():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    B, T, H = 1, 64, 4
    d = synth.wkv7_inputs(B, T, H, N, seed=0)
    dev = torch.device("cuda")
    names = ("r", "w", "k", "v", "a", "b")
    ins = [torch.from_numpy(d[n]).to(dev) for n in names]
    dy = torch.from_numpy(d["dy"]).to(dev)
    ck = torch.empty(binding.wkv7_checkpoint_floats(B, T, H), device=dev)

    def step():
        binding.wkv7_forward(*ins, ckpt=ck, want_state=False)
        binding.wkv7_backward(*ins, dy, ckpt=ck, want_ds0=False)

    def dom():
        binding.wkv7_backward(*ins, dy, ckpt=ck, want_ds0=False)

    flops = 26.0 * N * N * B * T * H
    roof = dict(kernel="wkv7 backward call (B=1 T=64 H=4: the single-pass reverse kernel and its "
                       "column reduction, 16 workgroups, latency bound)",
                bound="alu", work=flops, unit="TFLOP/s", peak=PEAK["alu_fp32"][0], fn=dom,
                key="wkv7_bwd_small", src=["rwkv_linear_attention_wkv7_amd/csrc/wkv7_seq.hip"])

    def cpu():
        from oracle import wkv7 as ow
        sub = [d[n].astype(np.float64) for n in names]
        dy64 = d["dy"].astype(np.float64)

        def one():
            ow.forward(*sub)
            ow.backward(*sub, dy64)

        reps, dt = repeat_for(one)
        return dict(value=reps * B * T / dt, unit="tokens/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"the whole workload (4 heads, T=64) {reps} times: f64 forward+backward, "
                           f"{dt:.1f} s")

    cfg = {"workload": "WKV7 forward+backward, small", "B": B, "T": T, "H": H, "N": N,
           "dtype": "fp32", "global_batch": B, "seq_len": T, "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="f32", config=cfg, roof=roof,
                cpu=cpu, extra=lambda v, ms: {"us_per_step": round(ms * 1e3, 2)})


def setup_timemix():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    B, T, C, H = 8, 1024, 768, 12
    ranks = (64, 64, 32, 128)
    p = synth.timemix_params(C, H, *ranks, layer_id=1, seed=0)
    d = synth.timemix_inputs(B, T, C, seed=1)
    dev = torch.device("cuda")
    W = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
    x, vf, dout = (torch.from_numpy(d[k]).to(dev) for k in ("x", "v_first", "dout"))
    s = binding.tm_shape(C, H, *ranks, layer_id=1)

    def step():
        f = binding.timemix_forward(s, W, x, v_first=vf, want_cache=True, want_state=False)
        binding.timemix_backward(s, W, x, dout, v_first=vf, cache=f["cache"], want_dx_prev=False,
                                 want_ds0=False, side=OPTS["side"])

    # dominant kernel: the fp32 MFMA GEMM of the C x C projections
    # (X [BT][C] . W [C][C]; 2*BT*C*C flop per launch)
    A = torch.from_numpy(d["x"].reshape(B * T, C)).to(dev)
    Wm = W["Wr"]
    Cout = torch.empty((B * T, C), device=dev)

    def dom():
        binding.wkv7_gemm_f32(A, Wm, Cout)

    flops = 2.0 * B * T * C * C
    roof = dict(kernel="gemm_f32 (X[8192][768] . W[768][768])", bound="mfma", work=flops,
                unit="TFLOP/s", peak=PEAK["mfma_fp32"][0], fn=dom, key="gemm_f32_c768",
                src=["rwkv_linear_attention_wkv7_amd/csrc/gemm.hip"])

    def cpu():
        from oracle import timemix as otm
        from oracle import wkv7 as ow
        def one():
            out, c = otm.forward(p, d["x"], H, 1, v_first=d["v_first"])
            otm.backward(p, c, d["dout"])

        reps, dt = repeat_for(one)
        return dict(value=reps * B * T / dt, unit="tokens/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"the whole workload (8 sequences, T=1024, C=768) {reps} times: f64 "
                           f"forward+backward, {dt:.1f} s")

    cfg = {"workload": "time-mix block forward+backward", "B": B, "T": T, "C": C, "H": H,
           "N": N, "lora_ranks_w_a_v_g": list(ranks), "layer_id": 1, "global_batch": B,
           "seq_len": T, "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="f32", config=cfg, roof=roof,
                cpu=cpu)


def setup_wkv7_long(chunked=False):
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    B, T, H = 4, 8192, 32
    d = synth.wkv7_inputs(B, T, H, N, seed=3, bf16=True)
    dev = torch.device("cuda")
    names = ("r", "w", "k", "v", "a", "b")
    ins = [torch.from_numpy(d[n]).to(dev).to(torch.bfloat16) for n in names]
    dy = torch.from_numpy(d["dy"]).to(dev).to(torch.bfloat16)
    ck = torch.empty(binding.wkv7_checkpoint_floats(B, T, H), device=dev)

    fws = None
    if chunked:
        fws = torch.empty(binding.lib().wkv7_forward_workspace_bytes(B, T, H, N), dtype=torch.uint8,
                          device=dev)

    def step():
        # token-sequential forward (no chunk workspace): the faster path here;
        # chunked=True times the chunked matrix-core forward instead
        binding.wkv7_forward(*ins, ckpt=ck, want_state=False, chunked=chunked, ws=fws)
        binding.wkv7_backward(*ins, dy, ckpt=ck, want_ds0=False)

    def dom():
        binding.wkv7_backward(*ins, dy, ckpt=ck, want_ds0=False)

    # backward algorithmic work per token-head: 19 N^2 flop for the reverse
    # step (G += dy r^T, dr, dv, dk, db, dsa, dw, da: 2 N^2 each; G update
    # 3 N^2) plus 7 N^2 to recompute sa and the state from the checkpoint
    # (the per-token recurrence's count, whatever form the kernels take).
    flops = 26.0 * N * N * B * T * H
    roof = dict(kernel="wkv7 backward call (reverse state-gradient scan + per-chunk matrix-core products)",
                bound="alu", work=flops, unit="TFLOP/s", peak=PEAK["alu_fp32"][0], fn=dom,
                key="wkv7_bwd_long", src=["rwkv_linear_attention_wkv7_amd/csrc/wkv7_bwd.hip"])

    def cpu():
        from oracle import wkv7 as ow
        sub = [d[n].astype(np.float64) for n in names]
        dy64 = d["dy"].astype(np.float64)

        def one():
            ow.forward(*sub)
            ow.backward(*sub, dy64)

        reps, dt = repeat_for(one)
        return dict(value=reps * B * T / dt, unit="tokens/s", cores=ow.num_threads(),
                    kind="oracle",
                    sample=f"the whole workload (128 (b,h) pairs, T=8192) {reps} times: f64 "
                           f"forward+backward, {dt:.1f} s")

    cfg = {"workload": "WKV7 forward+backward, long context", "B": B, "T": T, "H": H, "N": N,
           "forward": "chunked (matrix cores)" if chunked else "token-sequential",
           "inputs": "bf16", "state": "fp32", "checkpoint_interval": binding.wkv7_checkpoint_interval(),
           "global_batch": B, "seq_len": T, "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="bf16 in / f32 state", config=cfg,
                roof=roof, cpu=cpu)


def setup_decode():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    L, C, H, F, V, B, STEPS = 12, 256, 4, 1024, 256, 2048, 512
    ranks = (32, 32, 32, 64)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=0)
    dev = torch.device("cuda")
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    w = {k: d(v) for k, v in m.items() if k != "blocks"}
    w["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                    for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=1), w)
    tokens_np = synth.token_ids(STEPS, B, V, seed=0, name="decode_tokens")
    tokens = torch.from_numpy(tokens_np).to(dev)
    st = dm.new_state(B)
    cur = torch.empty(B, dtype=torch.int32, device=dev)
    logits = torch.empty((B, V), device=dev)
    ws = torch.empty(binding.rwkv7_decode_workspace_bytes(dm, B), dtype=torch.uint8, device=dev)
    cur.copy_(tokens[0])
    binding.rwkv7_decode_step(dm, cur, st, logits=logits, ws=ws)
    torch.cuda.synchronize()
    for k in st:
        st[k].zero_()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            binding.rwkv7_decode_step(dm, cur, st, logits=logits, ws=ws)
    torch.cuda.synchronize()
    pos = [0]

    def step():
        cur.copy_(tokens[pos[0] % STEPS])
        g.replay()
        pos[0] += 1

    # dominant kernel: wkv7_step on one layer's state (2048 streams x 4 heads)
    vec = [torch.from_numpy(synth.wkv7_inputs(B, 1, H, 64, seed=9)[n][:, 0].copy()).to(dev)
           for n in ("r", "w", "k", "v", "a", "b")]
    state1 = st["att_state"][0]
    y1 = torch.empty_like(vec[0])

    def dom():
        binding.wkv7_step(*vec, state1, y=y1)

    nbytes = 2.0 * B * H * 64 * 64 * 4 + 7.0 * B * H * 64 * 4
    roof = dict(kernel="wkv7_step (2048 streams x 4 heads, fp32 state in place)", bound="hbm",
                work=nbytes, unit="GB/s", peak=PEAK["hbm"][0], fn=dom, key="wkv7_step_decode",
                src=["rwkv_linear_attention_wkv7_amd/csrc/wkv7_step.hip"])

    def cpu():
        from oracle import stack
        from oracle import wkv7 as ow
        ns = 128
        idx = np.arange(ns) * (B // ns)
        ocfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
        box = dict(state=stack.init_state(ocfg, ns), t=0)

        def one():
            _, box["state"] = stack.decode_step(m, ocfg, tokens_np[box["t"] % STEPS, idx], box["state"])
            box["t"] += 1

        steps, dt = repeat_for(one)
        per_step_full = dt / steps * (B / ns)
        return dict(value=1.0 / per_step_full, unit="steps/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"{ns} of {B} streams x {steps} steps (f64), {dt:.1f} s; scaled to "
                           f"{B} streams")

    cfg = {"workload": "streaming decode, 12-layer RWKV-7 stack", "n_layer": L, "C": C, "H": H,
           "N": 64, "ffn": F, "vocab": V, "lora_ranks_w_a_v_g": list(ranks), "streams": B,
           "tokens_per_step": B, "token_steps_available": STEPS, "graph_replay": True,
           "global_batch": B, "seq_len": 1, "parallelism": "single GPU"}
    return dict(step=step, tokens=1, unit="steps/s", dtype="f32", config=cfg, roof=roof, cpu=cpu,
                extra=lambda v, ms: {"tokens_per_s": round(v * B, 1)})


def setup_train():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    L, C, H, F, V, B, T = 24, 1024, 16, 4096, 65536, 4, 2048
    ranks = (64, 64, 32, 128)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=0, use_ln0=False)
    dev = torch.device("cuda")
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    w = {k: d(v) for k, v in m.items() if k != "blocks"}
    w["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                    for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=0,
                                  gemm_dtype="bf16"), w)
    grads = binding.TrainGrads(dm)
    tok = synth.token_ids(B, T + 1, V, seed=0, name="train_tokens")
    x = torch.from_numpy(np.ascontiguousarray(tok[:, :-1])).to(dev)
    y = torch.from_numpy(np.ascontiguousarray(tok[:, 1:])).to(dev)
    loss = torch.empty(1, device=dev)
    ws = torch.empty(binding.rwkv7_train_workspace_bytes(dm, B, T), dtype=torch.uint8, device=dev)

    def step():
        binding.rwkv7_train_step(dm, grads, x, y, loss=loss, ws=ws, side=OPTS["side"])

    # dominant kernels: the bf16 matrix-core GEMMs; the timed one is the
    # channel-mix key projection [8192][1024] . [1024][4096], as the training
    # step runs it: both operands rounded to bf16 copies (k-contiguous), then
    # the direct-to-LDS product (the timed call includes the two copies)
    A = torch.randn(B * T, C, device=dev)
    Wk = w["blocks"][0]["cm_Wk"]
    out = torch.empty(B * T, F, device=dev)
    gws = torch.empty(binding.wkv7_gemm_bf16_workspace_bytes(B * T, F, C), dtype=torch.uint8,
                      device=dev)

    def dom():
        binding.wkv7_gemm_bf16(A, Wk, out, ws=gws)

    roof = dict(kernel="gemm_bf16 (X[8192][1024] . Wk[1024][4096]; bf16 operand copies + product)",
                bound="mfma",
                work=2.0 * B * T * C * F, unit="TFLOP/s", peak=PEAK["mfma_bf16"][0], fn=dom,
                key="gemm_bf16_c1024_f4096", src=["rwkv_linear_attention_wkv7_amd/csrc/gemm.hip"])

    def cpu():
        from oracle import stack
        from oracle import wkv7 as ow
        Ts = 768
        ocfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
        reps, dt = repeat_for(lambda: stack.train_step(m, ocfg, tok[:1, :Ts], tok[:1, 1:Ts + 1]))
        return dict(value=reps * Ts / dt, unit="tokens/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"1 sequence x {Ts} tokens of the same model (f64 forward+backward) "
                           f"{reps} times, {dt:.1f} s")

    cfg = {"workload": "RWKV-7 training step (24 blocks, LM head, log-softmax CE) forward+backward",
           "n_layer": L, "C": C, "H": H, "N": 64, "ffn": F, "vocab": V,
           "lora_ranks_w_a_v_g": list(ranks), "B": B, "T": T, "gemm": "bf16 operands, fp32 accumulation (matrix cores)",
           "global_batch": B, "seq_len": T, "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="bf16 GEMM / f32", config=cfg,
                roof=roof, cpu=cpu, extra=lambda v, ms: {"loss": round(float(loss.item()), 5)})


def moba_attended_keys(T, chunk, topk):
    """Keys each query attends, summed over the T queries of one head: its own
    chunk up to itself plus min(topk - 1, earlier chunks) full chunks."""
    return sum(t % chunk + 1 + chunk * min(topk - 1, t // chunk) for t in range(T))


def setup_hybrid():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    L, NA, C, H, F, V, B, T = 12, 4, 1024, 16, 4096, 65536, 4, 2048
    chunk, topk = 64, 4
    ranks = (64, 64, 32, 128)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=0, use_ln0=False)
    m["attn"] = synth.attn_blocks(C, F, NA, seed=0)
    dev = torch.device("cuda")
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    w = {k: d(v) for k, v in m.items() if k not in ("blocks", "attn")}
    w["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                    for k, v in b.items()} for b in m["blocks"]]
    w["attn"] = [{k: d(v) for k, v in a.items()} for a in m["attn"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=0,
                                  gemm_dtype="bf16", n_attn=NA, moba_chunk=chunk, moba_topk=topk), w)
    grads = binding.TrainGrads(dm)
    tok = synth.token_ids(B, T + 1, V, seed=0, name="hybrid_tokens")
    x = torch.from_numpy(np.ascontiguousarray(tok[:, :-1])).to(dev)
    y = torch.from_numpy(np.ascontiguousarray(tok[:, 1:])).to(dev)
    loss = torch.empty(1, device=dev)
    ws = torch.empty(binding.rwkv7_train_workspace_bytes(dm, B, T), dtype=torch.uint8, device=dev)

    def step():
        binding.rwkv7_train_step(dm, grads, x, y, loss=loss, ws=ws, side=OPTS["side"])

    # dominant kernel of the attention: the MoBA core backward of one block
    # ([4][2048][16 x 64] q, k, v); its products run as fp32 matrix-core tiles,
    # so the ceiling is the fp32 MFMA peak: 5 products of 2 N flop per attended
    # (query, key) pair (S recomputed, dP, dQ, dK, dV)
    g = torch.Generator(device=dev).manual_seed(0)
    q, k, v, dy = (torch.randn(B, T, C, device=dev, generator=g) for _ in range(4))
    yo, lse, sel = binding.moba_forward(q, k, v, H, chunk, topk)
    mws = torch.empty(binding.lib().moba_workspace_bytes(B, T, H, 64, chunk, topk), dtype=torch.uint8,
                      device=dev)

    def dom():
        binding.moba_backward(q, k, v, yo, lse, sel, dy, H, chunk, topk, ws=mws)

    flops = 5.0 * 2 * 64 * moba_attended_keys(T, chunk, topk) * B * H
    roof = dict(kernel=f"moba_backward (B={B} T={T} H={H}, chunks of {chunk}, top-{topk}: dQ pass + "
                       "dK/dV pass)", bound="mfma", work=flops, unit="TFLOP/s",
                peak=PEAK["mfma_fp32"][0], fn=dom, key="moba_bwd",
                src=["rwkv_linear_attention_wkv7_amd/csrc/moba.hip"])

    def cpu():
        from oracle import moba
        from oracle import wkv7 as ow
        Ts = 512
        ocfg = dict(C=C, H=H, F=F, V=V, n_layer=L, n_attn=NA, chunk=chunk, topk=topk)
        reps, dt = repeat_for(lambda: moba.train_step(m, ocfg, tok[:1, :Ts], tok[:1, 1:Ts + 1]))
        return dict(value=reps * Ts / dt, unit="tokens/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"1 sequence x {Ts} tokens of the same model (f64 forward+backward) "
                           f"{reps} times, {dt:.1f} s")

    cfg = {"workload": "hybrid RWKV-7 / MoBA training step (12 RWKV-7 + 4 attention blocks, LM head, "
                       "log-softmax CE) forward+backward",
           "n_layer": L, "n_attn": NA, "C": C, "H": H, "N": 64, "ffn": F, "vocab": V,
           "moba_chunk": chunk, "moba_topk": topk, "lora_ranks_w_a_v_g": list(ranks), "B": B, "T": T,
           "gemm": "bf16 operands, fp32 accumulation (matrix cores)", "global_batch": B, "seq_len": T,
           "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="bf16 GEMM / f32", config=cfg,
                roof=roof, cpu=cpu, extra=lambda v, ms: {"loss": round(float(loss.item()), 5)})


def setup_gdn():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    B, T, nk, nv, dk, dv, kk = 2, 4096, 12, 24, 128, 128, 4
    cfg = synth.gdn_config(nk, nv, dk, dv, kk=kk, seed=0)
    d = synth.gdn_inputs(B, T, cfg, seed=0)
    dev = torch.device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    layer = binding.Gdn(nk, nv, dk, dv, kk, cfg["rms_eps"], t(cfg["conv"]), t(cfg["A_log"]),
                        t(cfg["dt_bias"]), t(cfg["norm"]))
    ins = [t(d[k]) for k in ("raw", "z", "a", "b")]
    dout = t(d["dout"])
    cache = torch.empty(binding.gdn_cache_bytes(layer, B, T), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, nv * dv), device=dev)
    ws = torch.empty(binding.lib().gdn_backward_workspace_bytes(
        ctypes_byref(layer.shape), B, T, 1), dtype=torch.uint8, device=dev)

    def step():
        binding.gdn_forward(layer, *ins, out=out, cache=cache)
        binding.gdn_backward(layer, *ins, dout, cache=cache, ws=ws)

    def dom():
        binding.gdn_backward(layer, *ins, dout, cache=cache, ws=ws)

    # the backward's recurrence per token and value head: 5 dk dv flop to
    # recompute the state (decay, kv, update) and 14 dk dv for the reverse
    # step (dS += q^ do, S do, dS^T k^, dS_pre, dS u + S_pre dkv, <dS_pre, S>,
    # g dS_pre) -- the per-token recurrence's count, whatever form the
    # kernels take
    flops = 19.0 * dk * dv * B * T * nv
    roof = dict(kernel="gdn_backward call (RMSNorm backward, reverse state-gradient scan, "
                       "per-block matrix-core products, gate and l2-norm chain, conv backward)",
                bound="alu", work=flops,
                unit="TFLOP/s", peak=PEAK["alu_fp32"][0], fn=dom, key="gdn_bwd",
                src=["rwkv_linear_attention_wkv7_amd/csrc/gdn.hip"])

    def cpu():
        from oracle import gdn as og
        from oracle import wkv7 as ow
        kd = nk * dk
        heads = np.arange(2)
        ch = np.concatenate([np.arange(dk), kd + np.arange(dk),
                             2 * kd + (heads[:, None] * dv + np.arange(dv)).ravel()])
        vc = (heads[:, None] * dv + np.arange(dv)).ravel()
        f64 = lambda x: np.asarray(x, np.float64)
        sub = {k: (f64(v) if isinstance(v, np.ndarray) else v) for k, v in cfg.items()}
        sub.update(nk=1, nv=2, conv=f64(cfg["conv"])[ch], A_log=f64(cfg["A_log"])[heads],
                   dt_bias=f64(cfg["dt_bias"])[heads])
        ins64 = (f64(d["raw"][0][:, ch]), f64(d["z"][0][:, vc]), f64(d["a"][0][:, heads]),
                 f64(d["b"][0][:, heads]))
        dout64 = f64(d["dout"][0][:, vc])

        def one():
            _, c = og.forward(*ins64, sub)
            og.backward(c, dout64)

        reps, dt = repeat_for(one)
        scale = B * nk  # windows x key-head groups in the workload
        return dict(value=reps * B * T / (dt * scale), unit="tokens/s", cores=ow.num_threads(),
                    kind="oracle",
                    sample=f"one key-head group (2 value heads) of one window, T={T}, {reps} times: "
                           f"f64 forward+backward, {dt:.1f} s; scaled to the {scale} groups of the "
                           f"workload")

    cfgd = {"workload": "GatedDeltaNet layer forward+backward (through-gradients)", "B": B, "T": T,
            "nk": nk, "nv": nv, "dk": dk, "dv": dv, "conv_taps": kk, "global_batch": B,
            "seq_len": T, "parallelism": "single GPU"}
    return dict(step=step, tokens=B * T, unit="tokens/s", dtype="f32", config=cfgd, roof=roof,
                cpu=cpu)


def setup_online():
    import numpy as np
    import torch

    from rwkv_linear_attention_wkv7_amd import binding, synth
    L, C, H, F, V, B, S = 12, 256, 4, 1024, 256, 256, 64
    ranks = (32, 32, 32, 64)
    m = synth.stack_model(C, H, F, V, L, ranks, seed=0)
    dev = torch.device("cuda")
    d = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    w = {k: d(v) for k, v in m.items() if k != "blocks"}
    w["blocks"] = [{k: ({kk: d(vv) for kk, vv in v.items()} if k == "tm" else d(v))
                    for k, v in b.items()} for b in m["blocks"]]
    dm = binding.DecodeModel(dict(n_layer=L, C=C, H=H, F=F, V=V, ranks=ranks, use_ln0=1), w)
    grads = binding.TrainGrads(dm)
    am, av = binding.TrainGrads(dm, zero=True), binding.TrainGrads(dm, zero=True)
    nseg = 8
    tok = synth.token_ids(B, nseg * S + 1, V, seed=0, name="online_tokens")
    seg = lambda a, j: torch.from_numpy(np.ascontiguousarray(a[:, j * S:(j + 1) * S])).to(dev)
    xs = [seg(tok[:, :-1], j) for j in range(nseg)]
    ys = [seg(tok[:, 1:], j) for j in range(nseg)]
    state = dm.new_state(B)
    loss = torch.empty(1, device=dev)
    ws = torch.empty(binding.rwkv7_online_workspace_bytes(dm, B, S), dtype=torch.uint8, device=dev)
    pos = [0]

    def step():
        j = pos[0] % nseg
        t_ = pos[0] + 1
        binding.rwkv7_online_segment(dm, grads, xs[j], ys[j], state, optimizer="adam", lr=1e-4,
                                     step=t_, adam_m=am, adam_v=av, loss=loss, ws=ws)
        pos[0] += 1

    # dominant products: the fp32 channel-mix key GEMM of the segment,
    # [B*S][256] . [256][1024]
    A = torch.randn(B * S, C, device=dev)
    Wk = w["blocks"][0]["cm_Wk"]
    out = torch.empty(B * S, F, device=dev)

    def dom():
        binding.wkv7_gemm_f32(A, Wk, out)

    roof = dict(kernel="gemm_f32 (X[16384][256] . Wk[256][1024])", bound="mfma",
                work=2.0 * B * S * C * F, unit="TFLOP/s", peak=PEAK["mfma_fp32"][0], fn=dom,
                key="gemm_f32_online", src=["rwkv_linear_attention_wkv7_amd/csrc/gemm.hip"])

    def cpu():
        from oracle import online, stack
        from oracle import wkv7 as ow
        ns = 4
        ocfg = dict(C=C, H=H, F=F, V=V, n_layer=L)
        st0 = stack.init_state(ocfg, ns)
        reps, dt = repeat_for(lambda: online.train_segment(m, ocfg, tok[:ns, :S], tok[:ns, 1:S + 1],
                                                           st0, "adam", lr=1e-4))
        return dict(value=reps * ns * S / dt, unit="tokens/s", cores=ow.num_threads(), kind="oracle",
                    sample=f"one segment of {ns} of the {B} streams x {S} steps (f64 gradients, "
                           f"Adam update, replay) {reps} times, {dt:.1f} s; streams are independent")

    cfgd = {"workload": "online TBPTT training segments on the 12-layer decode model",
            "n_layer": L, "C": C, "H": H, "N": 64, "ffn": F, "vocab": V,
            "lora_ranks_w_a_v_g": list(ranks), "streams": B, "segment_steps": S,
            "optimizer": "Adam (lr 1e-4)", "global_batch": B, "seq_len": S,
            "parallelism": "single GPU"}
    return dict(step=step, tokens=B * S, unit="tokens/s", dtype="f32", config=cfgd, roof=roof,
                cpu=cpu, extra=lambda v, ms: {"loss": round(float(loss.item()), 5)})


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)


WORKLOADS = {"wkv7_small": setup_wkv7_small, "decode": setup_decode, "timemix": setup_timemix,
             "wkv7_long": setup_wkv7_long, "train": setup_train, "gdn": setup_gdn,
             "online": setup_online, "hybrid": setup_hybrid,
             "wkv7_long_chunked": lambda: setup_wkv7_long(chunked=True)}
ORDER = ("wkv7_small", "decode", "timemix", "wkv7_long", "train", "online", "gdn", "hybrid")


def run_workload(name, steps, warmup, roof_iters, with_cpu):
    """One workload: warm-up, K timed steps, the dominant kernel's roofline
    loop, optionally the CPU-oracle baseline.  Returns its record."""
    import torch
    w = WORKLOADS[name]()
    for _ in range(warmup):
        w["step"]()
    torch.cuda.synchronize()
    ms, ms_mean, wall = time_calls(w["step"], steps)
    value = w["tokens"] / (ms / 1e3)

    r = w["roof"]
    r["fn"]()
    kms, kms_mean, _ = time_calls(r["fn"], roof_iters)
    # work: algorithmic flop (unit TFLOP/s) or bytes (unit GB/s) per launch
    achieved = r["work"] / (kms / 1e3) / (1e12 if r["unit"] == "TFLOP/s" else 1e9)
    traffic = traffic_from_profile(r["key"], r["src"])
    roofline = {"bound": r["bound"], "kernel": r["kernel"], "achieved": round(achieved, 3),
                "peak": r["peak"], "unit": r["unit"], "frac": round(achieved / r["peak"], 4),
                "kernel_ms": round(kms, 4), "kernel_ms_mean": round(kms_mean, 4),
                "traffic": traffic}
    if r["bound"] == "alu":
        # the published fp32 vector peak counts packed FMA (two per lane); the
        # kernels here issue one fp32 FMA per lane: 256 CUs x 64 lanes x 2 flop
        # x 2.4 GHz
        roofline["peak_without_packed_fp32"] = PEAK_ALU_NO_PACKED
        roofline["frac_without_packed_fp32"] = round(achieved / PEAK_ALU_NO_PACKED, 4)
    cpu = None
    if with_cpu:
        cpu = w["cpu"]()
        cpu["value"] = round(cpu["value"], 2)
    rec = {"value": round(value, 1), "unit": w["unit"], "steps": steps, "warmup": warmup,
           "ms_per_step": round(ms, 4), "ms_per_step_mean": round(ms_mean, 4),
           "wall_s": round(wall, 3), "dtype": w["dtype"], "config": w["config"],
           "roofline": roofline, "cpu_baseline": cpu}
    if "extra" in w:
        rec.update(w["extra"](value, ms))
    del w
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=sorted(WORKLOADS) + ["all"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roof-iters", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (the known-size "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--one-stream", action="store_true",
                    help="run the time-mix and training-step workloads without the side stream (counter "
                         "runs that time each kernel alone)")
    args = ap.parse_args()
    OPTS["side"] = not args.one_stream
    if args.copy_calibration:
        import torch
        n = 64 * 1024 * 1024
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "repeats": 3}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); the library runs on one GPU and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from rwkv_linear_attention_wkv7_amd import binding
    binding.lib()

    names = ORDER if args.workload == "all" else (args.workload,)
    head = "decode" if args.workload == "all" else args.workload
    recs = {}
    for n in names:
        print(f"[bench] {n}", file=sys.stderr, flush=True)
        recs[n] = run_workload(n, args.steps, args.warmup, args.roof_iters,
                               not args.no_cpu_baseline)
    h = recs[head]
    out = {"metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
           "wall_s": h["wall_s"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": h["dtype"], "data": "synthetic (seeded)",
           "config": h["config"], "roofline": h["roofline"], "cpu_baseline": h["cpu_baseline"]}
    for k in ("ms_per_step_mean", "tokens_per_s", "us_per_step", "loss"):
        if k in h:
            out[k] = h[k]
    if len(recs) > 1:
        out["configs"] = recs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
