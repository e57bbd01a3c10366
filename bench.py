"""Benchmark of the KV codec's hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]
                    [--copies 4] [--reps 5] [--cache-state rotate|hot|flushed]
                    [--bits B] [--qjl-rows M] [--context L]
    python bench.py --copy-calibrate          # a device copy of known size

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: encode K and V into packed records, score
every cached key for every query head (attention logits), and run the fused
decode (softmax times values).  The default workload is one
Llama-3.1-8B-shaped layer: batch 8, 32 query heads over 8 KV heads, head dim
128, context 32768, bf16 K/V with one percent of channels scaled x100, RoPE
base 5e5, 3-bit Lloyd-Max codes plus a 64-row QJL sketch.

Timing.
* Steps: W untimed warmup steps, then K steps timed by the host clock
  between two device synchronisations (ms_per_step).  Every buffer the step
  touches exists in --copies copies (inputs, records, outputs) and step i uses
  copy i mod copies, so no step finds the previous step's data in the 256 MB
  memory-side cache.
* Calls: each call of the step (encode K, encode V, logits, decode) is then
  timed alone as N back-to-back launches between one pair of HIP events on
  the launch stream, N cycling through the buffer copies (about 3 ms per
  repeat); the figure is the median over --reps repeats of the per-launch
  time.  With --cache-state hot the same copy is relaunched (its data stays
  cached); with flushed every launch is timed alone after a 1 GiB read that
  evicts the cache.
* Device bandwidth: a 1 GiB device copy, fill and read (sum) are timed in the
  same run, and the kernels' rates are also given as a fraction of them.

Printed: one JSON line.  `value` is the logit scan's key throughput (keys of
the cached context scored per second for all their query heads) for the
decode workloads, encode tokens/s for the ESM-2 prefill encode, database
vectors scanned per second for vector search.  `roofline` relates the
dominant call's algorithmic bytes (or flops) per launch to its measured
duration; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload, and the tiny configuration on one and on all host threads.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attn-logit keys/sec + % of HBM peak; KV encode tokens/sec (1 MI355X)"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3
BF16_PEAK_TFLOPS = 2500.0
# the dense-rotation GEMMs run fp32 operands as three bf16 pieces each and
# issue six bf16 matrix products per fp32 multiply-add; the index scan's
# sketch part multiplies by exact +-1 (three products)
BF16_PRODUCTS_PER_FP32_MAC = 6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
REPEAT_MS = 3.0  # device time per timed repeat of a call


def device_code_digest() -> str:
    """sha256 over the library's device sources and build script: counter
    figures taken for another version of the kernels no longer apply."""
    import hashlib
    pkg = os.path.join(ROOT, "kv_cache_vector_05_amd")
    csrc = os.path.join(pkg, "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp")))
    files.append(os.path.join(pkg, "build.py"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, call: str):
    """HBM bytes per call from rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    (profiles/hbm_traffic.json), or None when absent or taken for other
    device code."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("device_code_sha256") != device_code_digest():
        return None
    return t.get("calls", {}).get(workload, {}).get(call, {}).get("traffic_bytes")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as fill about 0.3 s, at least one per buffer "
                         "copy: the GPU's clocks take some 100 ms of load to settle)")
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "llama70b", "esm650m", "vsearch", "llama8b-turboesm", "esm650m-turboesm",
                             "llama8b-serve", "llama8b-fib", "tiny"])
    ap.add_argument("--copies", type=int, default=4, help="buffer copies the steps and timed calls rotate over")
    ap.add_argument("--reps", type=int, default=5, help="timed repeats per call (the median is reported)")
    ap.add_argument("--cache-state", default="rotate", choices=["rotate", "hot", "flushed"])
    ap.add_argument("--bits", type=int, default=None, help="llama workloads: Lloyd-Max bits (default 3)")
    ap.add_argument("--context", type=int, default=None,
                    help="llama workloads: tokens per sequence (default 32768 for llama8b, 131072 for llama70b)")
    ap.add_argument("--qjl-rows", type=int, default=None,
                    help="llama workloads: QJL sketch rows m (default 64 for llama8b, 128 for llama70b)")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="only run a 1 GiB device copy, fill and read (counter calibration) and print their rates")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="keys in the oracle's sample (0: default)")
    return ap.parse_args(argv)


def host_cores():
    """Host CPUs this process may run on, and the oracle's BLAS thread count."""
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        blas = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = cores
    return cores, blas


class StepTimer:
    """HIP events on the launch stream around the calls of the timed steps
    (created up front, so that recording them costs the host little)."""

    def __init__(self, torch, events=0):
        self.torch = torch
        self.spans = {}
        self.stream = torch.cuda.current_stream()
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range(2 * events)]
        self.used = 0

    def _event(self):
        if self.used < len(self.pool):
            self.used += 1
            return self.pool[self.used - 1]
        return self.torch.cuda.Event(enable_timing=True)

    def call(self, name, fn):
        s, e = self._event(), self._event()
        s.record(self.stream)
        fn()
        e.record(self.stream)
        self.spans.setdefault(name, []).append((s, e))

    def mean_us(self, name):
        v = [s.elapsed_time(e) for s, e in self.spans.get(name, [])]
        return float(np.mean(v)) * 1e3 if v else None


class NoTimer:
    """Warmup steps: the calls only."""

    def call(self, name, fn):
        fn()


def run_step(st, timer, i=0):
    """Step i: the calls of buffer copy i mod copies."""
    for name, launch in st["rot"][i % len(st["rot"])]:
        timer.call(name, launch)


def run_calls(st, timer):
    """One step over buffer copy 0."""
    run_step(st, timer, 0)


def call_names(st):
    names = []
    for n, _ in st["rot"][0]:
        if n not in names:
            names.append(n)
    return names


def time_calls(torch, st, state, reps):
    """Per-launch device time (us) of each call, as the median over `reps`
    repeats of N back-to-back launches between one event pair on the launch
    stream.  rotate: the launches cycle through the buffer copies (and, for a
    call made several times per step, its instances); hot: one instance
    relaunched; flushed: each launch timed alone after a 1 GiB read."""
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if state == "flushed" else None
    out = {}
    for name in call_names(st):
        seq = [launch for rot in st["rot"] for n, launch in rot if n == name]
        if state == "hot":
            seq = seq[:1]
        if state == "flushed":
            ts = []
            for j in range(3 + 8 * reps):
                flush.sum()
                s, e = ev(), ev()
                s.record(stream)
                seq[j % len(seq)]()
                e.record(stream)
                torch.cuda.synchronize()
                ts.append(s.elapsed_time(e) * 1e3)
            ts = np.array(ts[3:])
            out[name] = {"us": float(np.median(ts)), "us_min": float(ts.min()), "us_max": float(ts.max()),
                         "launches": len(ts), "timing": "each launch alone after a 1 GiB read"}
            continue
        s, e = ev(), ev()
        s.record(stream)
        for f in seq:
            f()
        e.record(stream)
        torch.cuda.synchronize()
        t_seq = s.elapsed_time(e)
        n = len(seq) * max(2, int(math.ceil(REPEAT_MS / max(t_seq, 1e-3))))
        per = []
        for _ in range(reps):
            s, e = ev(), ev()
            s.record(stream)
            for j in range(n):
                seq[j % len(seq)]()
            e.record(stream)
            torch.cuda.synchronize()
            per.append(s.elapsed_time(e) * 1e3 / n)
        per = np.array(per)
        out[name] = {"us": float(np.median(per)), "us_min": float(per.min()), "us_max": float(per.max()),
                     "launches_per_repeat": n, "repeats": reps, "instances": len(seq),
                     "timing": "back-to-back launches, one event pair per repeat"}
    return out


def device_rates(torch, mib=1024, reps=5):
    """GB/s of a device copy (read + write), a fill (write) and a sum (read)
    of `mib` MiB, each the median of `reps` event-timed repeats of three
    back-to-back launches."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    nbytes = n * 4
    res = {}
    for label, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                             ("fill", lambda: dst.fill_(2.0), nbytes),
                             ("read", lambda: src.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        v = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(3):
                fn()
            e.record()
            torch.cuda.synchronize()
            v.append(3 * moved / (s.elapsed_time(e) * 1e-3) / 1e9)
        res[label + "_GBps"] = float(np.median(v))
    del src, dst
    torch.cuda.empty_cache()
    return res


def bf16_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _copies(t, n):
    return [t] + [t.clone() for _ in range(n - 1)]


def _rate(k):
    k["GBps"] = k["alg_bytes"] / (k["us"] * 1e-6) / 1e9
    k["hbm_frac"] = k["GBps"] / HBM_PEAK_GBS
    return k


# ------------------------------------------------------------ TurboESM tables
CALIB_TOKENS = 256  # calibration batch: the first tokens of the first sequence


def turboesm_codebooks(tq, synth, d, bits, k_sample, v_sample, rope_host):
    """Key codebook (Hadamard, RoPE'd calibration) and value codebook (no
    rotation), each with its own calibrated table and one mu per KV head
    (TurboESM-style records: codes, one residual sign per coordinate, nu)."""
    lk, mk = tq.calibrate(d, bits, k_sample, rotation="hadamard", seed=synth.K_SEED, rope=rope_host)
    lv, mv = tq.calibrate(d, bits, v_sample, rotation="none")
    ck = tq.Codebook(d, bits, d, "hadamard", seed=synth.K_SEED, correction="sign", levels=lk, mu=mk)
    cv = tq.Codebook(d, bits, d, "none", correction="sign", levels=lv, mu=mv)
    return ck, cv


# ------------------------------------------------------------ llama-shaped
def setup_llama(torch, tq, synth, kind, variant="qjl", copies=1, bits=None, m=None, ctx=None):
    if kind == "llama8b":
        B, Hq, H, L, d, b0, m0, rope_base = 8, 32, 8, 32768, 128, 3, 64, 5e5
    else:
        B, Hq, H, L, d, b0, m0, rope_base = 1, 64, 8, 131072, 128, 3, 128, 0.0
    L = L if ctx is None else ctx
    bits = b0 if bits is None else bits
    m = (d if variant == "turboesm" else m0) if m is None else m
    K, V = synth.llama_kv_inputs(kind, seed=0, batch=B, ctx=L, hkv=H, d=d)
    Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
    st = {"B": B, "Hq": Hq, "H": H, "L": L, "d": d, "bits": bits, "m": m, "rope_base": rope_base,
          "variant": variant, "kind": kind}
    Kd, Vd = bf16_dev(torch, K), bf16_dev(torch, V)
    st["Q"] = bf16_dev(torch, Q)
    st["host"] = (K, V, Q)
    if variant == "turboesm":
        rope_host = tq.rope_table(rope_base, d, L + 1, device=None) if rope_base else None
        st["ck"], st["cv"] = turboesm_codebooks(tq, synth, d, bits,
                                                synth.bf16_bits_to_f32(K[0, :CALIB_TOKENS]),
                                                synth.bf16_bits_to_f32(V[0, :CALIB_TOKENS]), rope_host)
    else:
        st["ck"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.K_SEED)
        st["cv"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.V_SEED)
    st["rope"] = tq.rope_table(rope_base, d, L + 1) if rope_base else None
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["ws_l"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    Ks, Vs = _copies(Kd, copies), _copies(Vd, copies)
    st["rot"] = []
    for c in range(copies):
        kp, vp = tq.Packed(st["ck"], B * H * L), tq.Packed(st["cv"], B * H * L)
        lg = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        if c == 0:
            st["K"], st["V"], st["kp"], st["vp"], st["logits"], st["out"] = Ks[0], Vs[0], kp, vp, lg, out
        # every call of the step with its arguments marshalled once
        st["rot"].append([
            ("encode_k", tq.encode_kv(st["ck"], None, Ks[c], None, kp, None, L_cap=L, rope=st["rope"],
                                      prepare=True)),
            ("encode_v", tq.encode_kv(None, st["cv"], None, Vs[c], None, vp, L_cap=L, prepare=True)),
            ("logits", tq.attn_logits(st["ck"], st["Q"], kp, H, L, st["sl"], rope=st["rope"], out=lg,
                                      workspace=st["ws_l"], prepare=True)[0]),
            ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], kp, vp, H, L, st["sl"], rope=st["rope"],
                                      out=out, workspace=st["ws_d"], prepare=True)[0]),
        ])
    st["calls"] = st["rot"][0]
    return st


def llama_report(st, ct, ms_step):
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    G = Hq // H
    keys = B * H * L
    sign = st["variant"] == "turboesm"
    rec = 4 + (4 if m and not sign else 0) + bits * d // 8 + m // 8
    in_bytes = 2 * d  # bf16
    kern = {
        "encode_k": {"alg_bytes": keys * (in_bytes + rec), "units": keys, "unit": "vectors"},
        "encode_v": {"alg_bytes": keys * (in_bytes + rec), "units": keys, "unit": "vectors"},
        "logits": {"alg_bytes": keys * (rec + 4 * G), "units": keys, "unit": "keys"},
        "decode": {"alg_bytes": keys * 2 * rec, "units": keys, "unit": "keys"},
    }
    for name, k in kern.items():
        k.update(ct[name])
        _rate(k)
    t = {n: kern[n]["us"] * 1e-6 for n in kern}
    extra = {
        "logit_keys_per_s": keys / t["logits"],
        "logits_per_s": keys * G / t["logits"],
        "logit_hbm_frac": kern["logits"]["hbm_frac"],
        "decode_keys_per_s": keys / t["decode"],
        "encode_tokens_per_s": B * L / (t["encode_k"] + t["encode_v"]),
        "encode_vectors_per_s": 2 * keys / (t["encode_k"] + t["encode_v"]),
        "step_keys_per_s": keys / (ms_step * 1e-3),
    }
    name = f"{'Llama-3.1-8B' if st['kind'] == 'llama8b' else 'Llama-70B'}-shaped decode layer"
    cfg = {"workload": name + (", TurboESM-style records" if sign else ""), "batch": B,
           "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "bits": bits,
           "input_dtype": "bf16", "rope_base": st["rope_base"], "record_bytes": rec}
    if sign:
        cfg.update({"residual_signs": "one per coordinate, mu per KV head", "key_table": "calibrated, rotated",
                    "value_table": "calibrated, original coordinates", "calibration_tokens": CALIB_TOKENS})
    else:
        cfg["qjl_rows"] = m
    return extra["logit_keys_per_s"], "keys/s", kern, extra, cfg


# ------------------------------------------------------------ FibQuant codebooks
FIB_BITS = 4  # 16 codewords per 2-coordinate block: 2 bits per coordinate


def setup_fib(torch, tq, synth, copies=1):
    """The Llama-3.1-8B-shaped layer with FibQuant vector codebooks for keys
    and values (k = 2, N = 16): encode K (RoPE), encode V, the logit scan of
    the 32 query heads over every cached key, and the fused decode."""
    B, Hq, H, L, d = 8, 32, 8, 32768, 128
    K, V = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L, hkv=H, d=d)
    Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
    st = {"B": B, "Hq": Hq, "H": H, "L": L, "d": d, "bits": FIB_BITS, "rope_base": 5e5, "host": (K, V, Q)}
    Kd, Vd = bf16_dev(torch, K), bf16_dev(torch, V)
    st["Q"] = bf16_dev(torch, Q)
    st["ck"] = tq.Codebook(d, FIB_BITS, 0, "hadamard", seed=synth.K_SEED, block=2)
    st["cv"] = tq.Codebook(d, FIB_BITS, 0, "hadamard", seed=synth.V_SEED, block=2)
    st["rope"] = tq.rope_table(5e5, d, L + 1)
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["ws_l"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    Ks, Vs = _copies(Kd, copies), _copies(Vd, copies)
    st["rot"] = []
    for c in range(copies):
        kp, vp = tq.Packed(st["ck"], B * H * L), tq.Packed(st["cv"], B * H * L)
        lg = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        if c == 0:
            st["K"], st["V"], st["kp"], st["vp"], st["logits"], st["out"] = Ks[0], Vs[0], kp, vp, lg, out
        st["rot"].append([
            ("encode_k", tq.encode_kv(st["ck"], None, Ks[c], None, kp, None, L_cap=L, rope=st["rope"],
                                      prepare=True)),
            ("encode_v", tq.encode_kv(None, st["cv"], None, Vs[c], None, vp, L_cap=L, prepare=True)),
            ("logits", tq.attn_logits(st["ck"], st["Q"], kp, H, L, st["sl"], rope=st["rope"], out=lg,
                                      workspace=st["ws_l"], prepare=True)[0]),
            ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], kp, vp, H, L, st["sl"], rope=st["rope"],
                                      out=out, workspace=st["ws_d"], prepare=True)[0]),
        ])
    st["calls"] = st["rot"][0]
    return st


def fib_report(st, ct, ms_step):
    B, Hq, H, L, d, bits = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits"))
    keys = B * H * L
    rec = 4 + 4 * ((d // 2 * bits + 31) // 32)
    kern = {"encode_k": {"alg_bytes": keys * (2 * d + rec), "units": keys, "unit": "vectors"},
            "encode_v": {"alg_bytes": keys * (2 * d + rec), "units": keys, "unit": "vectors"},
            "logits": {"alg_bytes": keys * (rec + 4 * Hq // H), "units": keys, "unit": "keys"},
            "decode": {"alg_bytes": keys * 2 * rec, "units": keys, "unit": "keys"}}
    for name, k in kern.items():
        k.update(ct[name])
        _rate(k)
    t = {n: kern[n]["us"] * 1e-6 for n in kern}
    extra = {"logit_keys_per_s": keys / t["logits"], "logit_hbm_frac": kern["logits"]["hbm_frac"],
             "decode_keys_per_s": keys / t["decode"],
             "encode_vectors_per_s": 2 * keys / (t["encode_k"] + t["encode_v"]),
             "step_keys_per_s": keys / (ms_step * 1e-3)}
    cfg = {"workload": "Llama-3.1-8B-shaped layer with FibQuant vector codebooks (encode K, V; logits; decode)",
           "batch": B, "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "block": 2,
           "codewords": 1 << bits, "bits_per_coordinate": bits / 2, "input_dtype": "bf16",
           "rope_base": st["rope_base"], "record_bytes": rec}
    return extra["logit_keys_per_s"], "keys/s", kern, extra, cfg


def cpu_baseline_fib(st, budget_s=10.0):
    """The oracle on a bounded sample of the FibQuant step: (sequence, KV
    head) pairs in order, keys (RoPE) and values encoded and the pair's 4
    query heads scored, until about budget_s seconds."""
    import synth
    from oracle import fibquant as F, rng, rope as orope
    K, V, Q = st["host"]
    B, Hq, H, L, d, bits = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits"))
    G = Hq // H
    t0 = time.perf_counter()
    ock = F.make_vq_codebook(d, 2, 1 << bits, rng.signs(synth.K_SEED, d))
    ocv = F.make_vq_codebook(d, 2, 1 << bits, rng.signs(synth.V_SEED, d), code=ock.code32)
    t_setup = time.perf_counter() - t0
    rope = orope.rope_table(st["rope_base"], d, L + 1)
    from oracle.rope import apply_rope
    done, pairs, dt = 0, 0, 0.0
    n = 4096  # keys per pair in the sample (the oracle's nearest-codeword search is slow)
    for b in range(B):
        for kh in range(H):
            if dt >= budget_s:
                break
            kx = synth.bf16_bits_to_f32(K[b, :n, kh])
            vx = synth.bf16_bits_to_f32(V[b, :n, kh])
            q = synth.bf16_bits_to_f32(Q[b, kh * G:(kh + 1) * G])
            t1 = time.perf_counter()
            ek = F.encode(ock, kx, pos=np.arange(n), rope=rope)
            ev = F.encode(ocv, vx)
            qp = apply_rope(q, np.full(G, L), rope[0], rope[1]) @ ock.pi.T
            F.logits(ock, qp, ek.norm, ek.codes)
            F.attention(ock, ocv, qp, ek.norm, ek.codes, ev.norm, ev.codes, 1.0 / math.sqrt(d))
            dt += time.perf_counter() - t1
            done += n
            pairs += 1
    return {"value": done / dt, "unit": "keys/s", "kind": "oracle",
            "sample": f"{pairs} (sequence, KV head) pairs, the first {n} keys and values of each encoded, scored "
                      f"and attended for {G} query heads by the oracle, {dt:.1f} s on the host (codebook built "
                      f"beforehand, {t_setup:.1f} s)"}


# ------------------------------------------------------------ serving step
PAGE = 256  # slots per page of the paged cache


def setup_serve(torch, tq, synth, copies=1):
    """One autoregressive step of the Llama-3.1-8B-shaped layer over a paged
    cache: the cache holds L - 1 tokens per sequence, spread over a shuffled
    pool of pages; a step appends token L - 1 (keys and values of every
    (sequence, KV head)) and runs the fused decode over the L tokens, the
    query at position L - 1 like its own key."""
    B, Hq, H, L, d, bits, m, rope_base = 8, 32, 8, 32768, 128, 3, 64, 5e5
    K, V = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L, hkv=H, d=d)
    Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
    st = {"B": B, "Hq": Hq, "H": H, "L": L, "d": d, "bits": bits, "m": m, "rope_base": rope_base,
          "variant": "qjl", "host": (K, V, Q)}
    J = L // PAGE
    n_pages = B * J
    table = synth.rng(3).permutation(n_pages).astype(np.int32).reshape(B, J)
    st["pages"] = tq.Pages(torch.from_numpy(table).cuda(), PAGE, n_pages)
    st["ck"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.K_SEED)
    st["cv"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.V_SEED)
    st["rope"] = tq.rope_table(rope_base, d, L + 1)
    Kd, Vd = bf16_dev(torch, K), bf16_dev(torch, V)
    st["K1"], st["V1"] = Kd[:, L - 1].contiguous(), Vd[:, L - 1].contiguous()
    st["pos"] = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["Q"] = bf16_dev(torch, Q)
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["rot"] = []
    for c in range(copies):
        kp, vp = tq.Packed(st["ck"], st["pages"].records(H)), tq.Packed(st["cv"], st["pages"].records(H))
        # prefill: the first L - 1 tokens
        tq.encode_kv(st["ck"], st["cv"], Kd[:, :L - 1], Vd[:, :L - 1], kp, vp, rope=st["rope"], pages=st["pages"])
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        if c == 0:
            st["kp"], st["vp"], st["out"] = kp, vp, out
        st["rot"].append([
            ("append", tq.append_kv(st["ck"], st["cv"], st["K1"], st["V1"], kp, vp, st["pos"], pages=st["pages"],
                                    rope=st["rope"], prepare=True)),
            ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], kp, vp, H, None, st["sl"], rope=st["rope"],
                                      out=out, workspace=st["ws_d"], prepare=True, pages=st["pages"],
                                      q_pos=st["pos"])[0]),
        ])
    del Kd, Vd
    st["calls"] = st["rot"][0]
    return st


def serve_report(st, ct, ms_step):
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    keys = B * H * L
    rec = 8 + bits * d // 8 + m // 8
    kern = {"append": {"alg_bytes": 2 * B * H * (2 * d + rec), "units": 2 * B * H, "unit": "vectors"},
            "decode": {"alg_bytes": keys * 2 * rec, "units": keys, "unit": "keys"}}
    for name, k in kern.items():
        k.update(ct[name])
        _rate(k)
    extra = {"decode_keys_per_s": keys / (kern["decode"]["us"] * 1e-6), "append_us": kern["append"]["us"],
             "decode_us": kern["decode"]["us"], "tokens_per_s": B / (ms_step * 1e-3)}
    cfg = {"workload": "Llama-3.1-8B-shaped decode step over a paged cache (append + fused decode)", "batch": B,
           "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "bits": bits, "qjl_rows": m,
           "input_dtype": "bf16", "rope_base": st["rope_base"], "record_bytes": rec, "page_size": PAGE,
           "pages": B * (L // PAGE), "page_order": "shuffled", "query_position": L - 1}
    return extra["decode_keys_per_s"], "keys/s", kern, extra, cfg


def cpu_baseline_serve(st, budget_s=8.0):
    """The oracle on a bounded sample of the serving step: whole (sequence,
    KV head) pairs in order, each cache encoded beforehand (untimed), then
    timed: the append of the pair's new key and value and the decode of its
    G query heads over all L keys, until about budget_s seconds."""
    import synth
    from oracle import codec, estimator, rope as orope
    K, V, Q = st["host"]
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    G = Hq // H
    ock = codec.make_codebook(d, bits, m, False, seed=synth.K_SEED)
    ocv = codec.make_codebook(d, bits, m, False, seed=synth.V_SEED)
    rope = orope.rope_table(st["rope_base"], d, L + 1)
    done, pairs, dt = 0, 0, 0.0
    for b in range(B):
        for kh in range(H):
            if dt >= budget_s:
                break
            kx = synth.bf16_bits_to_f32(K[b, :, kh])
            vx = synth.bf16_bits_to_f32(V[b, :, kh])
            ek = codec.encode(ock, kx[:L - 1], pos=np.arange(L - 1), rope=rope)
            ev = codec.encode(ocv, vx[:L - 1])
            q = synth.bf16_bits_to_f32(Q[b, kh * G:(kh + 1) * G])
            t1 = time.perf_counter()
            nk = codec.encode(ock, kx[L - 1:], pos=np.array([L - 1]), rope=rope)
            nv = codec.encode(ocv, vx[L - 1:])
            cat = lambda e, n: codec.Encoded(np.concatenate([e.norm, n.norm]), np.concatenate([e.rnorm, n.rnorm]),
                                             np.concatenate([e.codes, n.codes]), np.concatenate([e.signs, n.signs]))
            qp, s = estimator.prep_query(ock, q, L - 1, rope)
            estimator.attention(ock, ocv, qp, s, cat(ek, nk), cat(ev, nv), L, 1 / math.sqrt(d))
            dt += time.perf_counter() - t1
            done += L
            pairs += 1
    return {"value": done / dt, "unit": "keys/s", "kind": "oracle",
            "sample": f"{pairs} (sequence, KV head) pairs: the append of one key and value and the decode of "
                      f"{G} query heads over {L} cached keys each, {dt:.1f} s on the host (the caches encoded "
                      f"beforehand, untimed)"}


def cpu_baseline_llama(st, sample_keys, budget_s=12.0):
    """The oracle on a bounded sample: (sequence, KV head) pairs in order,
    each fully encoded (keys with RoPE, values), scored for its G query heads
    and decoded, until about budget_s seconds of host time or sample_keys
    keys.  `value` is the oracle's logit rate (keys scored per second for
    their G query heads, query preparation included), the GPU's `value`
    quantity; step_keys_per_s covers encode, logits and decode."""
    import synth
    from oracle import codec, estimator, rope as orope
    K, V, Q = st["host"]
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    G = Hq // H
    rope = orope.rope_table(st["rope_base"], d, L + 1) if st["rope_base"] else None
    t0 = time.perf_counter()
    if st["variant"] == "turboesm":
        ock, ocv = oracle_turboesm_codebooks(synth, d, bits, synth.bf16_bits_to_f32(K[0, :CALIB_TOKENS]),
                                             synth.bf16_bits_to_f32(V[0, :CALIB_TOKENS]), rope)
    else:
        ock = codec.make_codebook(d, bits, m, False, seed=synth.K_SEED)
        ocv = codec.make_codebook(d, bits, m, False, seed=synth.V_SEED)
    t_setup = time.perf_counter() - t0
    done, pairs, dt, dt_log = 0, 0, 0.0, 0.0
    for b in range(B):
        for kh in range(H):
            if done >= sample_keys or dt >= budget_s:
                break
            n = min(L, sample_keys - done)
            kx = synth.bf16_bits_to_f32(K[b, :n, kh])
            vx = synth.bf16_bits_to_f32(V[b, :n, kh])
            q = synth.bf16_bits_to_f32(Q[b, kh * G:(kh + 1) * G])
            t1 = time.perf_counter()
            ek = codec.encode(ock, kx, pos=np.arange(n), rope=rope)
            ev = codec.encode(ocv, vx)
            t2 = time.perf_counter()
            qp, s = estimator.prep_query(ock, q, n, rope)
            estimator.logits(ock, qp, s, ek, kh)
            t3 = time.perf_counter()
            estimator.attention(ock, ocv, qp, s, ek, ev, n, 1 / math.sqrt(d), kh)
            dt += time.perf_counter() - t1
            dt_log += t3 - t2
            done += n
            pairs += 1
    return {"value": done / dt_log, "unit": "keys/s", "kind": "oracle", "step_keys_per_s": done / dt,
            "sample": f"{done} keys: the first {pairs} (sequence, KV head) pairs, each encoded (keys with RoPE, and "
                      f"values), scored for its {G} query heads and decoded by the oracle in {dt:.1f} s on the host; "
                      f"value counts the {dt_log:.1f} s of query preparation and logits (codebook tables built once "
                      f"beforehand, {t_setup:.1f} s)"}


def oracle_turboesm_codebooks(synth, d, bits, k_sample, v_sample, rope):
    """The oracle's own calibration and sign-corrected codebooks for the same
    samples (the CPU baseline times the oracle as it stands)."""
    from oracle import calibration, codec, rng, rotation
    sigma = rng.signs(synth.K_SEED, d)  # the seeded signs the library derives from the same seed
    lk, mk = calibration.calibrate(rotation.rht_matrix(sigma), bits, k_sample, rope=rope)
    lv, mv = calibration.calibrate(np.eye(d), bits, v_sample)
    return (codec.make_sign_codebook(d, bits, "hadamard", sigma=sigma, levels=lk, mu=mk),
            codec.make_sign_codebook(d, bits, "none", levels=lv, mu=mv))


def cpu_tiny(threads):
    """The oracle on the tiny configuration (4096 fp32 keys, d = 128, 2-bit
    codes + 128-row sketch, 16 queries): encode every key, then score it for
    every query, with the BLAS pool limited to `threads`."""
    import threadpoolctl
    import synth
    from oracle import codec, estimator
    K, Q, _ = synth.tiny_inputs(0)
    ock = codec.make_codebook(128, 2, 128, False, seed=synth.K_SEED)
    ts = []
    with threadpoolctl.threadpool_limits(threads):
        for _ in range(5):
            t0 = time.perf_counter()
            enc = codec.encode(ock, K)
            qp, s = estimator.prep_query(ock, Q)
            estimator.logits(ock, qp, s, enc)
            ts.append(time.perf_counter() - t0)
    dt = float(np.median(ts))
    return {"keys_per_s": len(K) / dt, "threads": threads, "seconds_median_of_5": dt}


# ------------------------------------------------------------ ESM-2 prefill
def setup_esm(torch, tq, synth, variant="qjl", copies=1):
    """33 layers of K and V: the step's own layer buffers already rotate (one
    encode of each layer per step), so one copy serves."""
    S, T, H, d, layers, bits, m = 32, 1024, 20, 64, 33, 3, 64
    tok_h = synth.esm_tokens(0, S, T)
    tok = torch.from_numpy(tok_h).cuda()
    Ks, Vs, cks, cvs = [], [], [], []
    rope_host = tq.rope_table(1e4, d, T, device=None)
    for layer in range(layers):
        pk, pv = synth.esm_layer_tables(layer)
        Ks.append(torch.from_numpy(pk).cuda()[tok].view(S, T, H, d))
        Vs.append(torch.from_numpy(pv).cuda()[tok].view(S, T, H, d))
        if variant == "turboesm":
            # per layer: key and value tables, mu per head, from the first tokens of sequence 0
            ck, cv = turboesm_codebooks(tq, synth, d, bits, pk[tok_h[0, :CALIB_TOKENS]].reshape(-1, H, d),
                                        pv[tok_h[0, :CALIB_TOKENS]].reshape(-1, H, d), rope_host)
            cks.append(ck)
            cvs.append(cv)
    st = {"S": S, "T": T, "H": H, "d": d, "layers": layers, "bits": bits, "m": m, "K": Ks, "V": Vs,
          "variant": variant, "tok": tok_h}
    if variant != "turboesm":
        ck = tq.Codebook(d, bits, m, "hadamard", seed=synth.K_SEED)
        cv = tq.Codebook(d, bits, m, "hadamard", seed=synth.V_SEED)
        cks, cvs = [ck] * layers, [cv] * layers
    st["ck"], st["cv"] = cks, cvs
    st["kp"] = [tq.Packed(cks[i], S * H * T) for i in range(layers)]
    st["vp"] = [tq.Packed(cvs[i], S * H * T) for i in range(layers)]
    st["rope"] = tq.rope_table(1e4, d, T)
    calls = []
    for layer in range(layers):
        calls.append(("encode_k", tq.encode_kv(cks[layer], None, Ks[layer], None, st["kp"][layer], None,
                                               L_cap=T, rope=st["rope"], prepare=True)))
        calls.append(("encode_v", tq.encode_kv(None, cvs[layer], None, Vs[layer], None, st["vp"][layer],
                                               L_cap=T, prepare=True)))
    st["rot"] = [calls]
    st["calls"] = calls
    return st


def cpu_baseline_esm(st, budget_s=12.0):
    """The oracle on a bounded sample: layer 0's keys (RoPE) and values of
    whole (sequence, head) pairs in order, until about budget_s seconds of
    host time; reported as tokens/s of the whole 33-layer encode."""
    import synth
    from oracle import codec, rope as orope
    S, T, H, d, layers, bits, m = (st[k] for k in ("S", "T", "H", "d", "layers", "bits", "m"))
    pk, pv = synth.esm_layer_tables(0)
    rope = orope.rope_table(1e4, d, T)
    t0 = time.perf_counter()
    if st["variant"] == "turboesm":
        tok0 = st["tok"][0, :CALIB_TOKENS]
        ock, ocv = oracle_turboesm_codebooks(synth, d, bits, pk[tok0].reshape(-1, H, d), pv[tok0].reshape(-1, H, d),
                                             rope)
    else:
        ock = codec.make_codebook(d, bits, m, False, seed=synth.K_SEED)
        ocv = codec.make_codebook(d, bits, m, False, seed=synth.V_SEED)
    t_setup = time.perf_counter() - t0
    done, dt = 0, 0.0
    for s in range(S):
        for h in range(H):
            if dt >= budget_s:
                break
            kx = pk[st["tok"][s]].reshape(T, H, d)[:, h]
            vx = pv[st["tok"][s]].reshape(T, H, d)[:, h]
            t1 = time.perf_counter()
            codec.encode(ock, kx, pos=np.arange(T), rope=rope)
            codec.encode(ocv, vx)
            dt += time.perf_counter() - t1
            done += T
    # `done` key+value vector pairs of one layer; a token needs layers * H of them
    return {"value": done / dt / (layers * H), "unit": "tokens/s", "kind": "oracle",
            "sample": f"{done} key+value vector pairs of layer 0 ({done // T} (sequence, head) pairs of {T} tokens) "
                      f"encoded by the oracle in {dt:.1f} s on the host, scaled to tokens of the {layers}-layer, "
                      f"{H}-head encode (codebook tables built once beforehand, {t_setup:.1f} s)"}


def esm_report(st, ct, ms_step):
    S, T, H, d, layers, bits, m = (st[k] for k in ("S", "T", "H", "d", "layers", "bits", "m"))
    vec = S * T * H
    sign = st["variant"] == "turboesm"
    rec = 4 + (0 if sign else 4) + bits * d // 8 + m // 8
    kern = {"encode_k": {"alg_bytes": vec * (4 * d + rec), "units": vec, "unit": "vectors"},
            "encode_v": {"alg_bytes": vec * (4 * d + rec), "units": vec, "unit": "vectors"}}
    for name, k in kern.items():
        k.update(ct[name])
        _rate(k)
    t_layer = (kern["encode_k"]["us"] + kern["encode_v"]["us"]) * 1e-6
    extra = {"encode_tokens_per_s": S * T / (layers * t_layer),
             "encode_vectors_per_s": 2 * vec / t_layer,
             "step_tokens_per_s": S * T / (ms_step * 1e-3),
             "kv_bytes_fp32_per_sequence": 2 * layers * T * H * d * 4,
             "kv_bytes_packed_per_sequence": 2 * layers * T * H * rec,
             "kv_reduction_vs_fp32": (4 * d) / rec}
    cfg = {"workload": "ESM-2-650M-shaped prefill encode" + (", TurboESM-style records" if sign else ""),
           "layers": layers, "heads": H, "head_dim": d, "sequences": S, "length": T, "bits": bits,
           "input_dtype": "f32", "rope_base": 1e4, "record_bytes": rec}
    if sign:
        cfg.update({"residual_signs": "one per coordinate, mu per head", "key_table": "calibrated per layer, rotated",
                    "value_table": "calibrated per layer, original coordinates", "calibration_tokens": CALIB_TOKENS})
    else:
        cfg["qjl_rows"] = m
    return extra["encode_tokens_per_s"], "tokens/s", kern, extra, cfg


# ------------------------------------------------------------ vector search
def setup_vsearch(torch, tq, synth, copies=1):
    n, nq, d, bits, m = 1_000_000, 1024, 1536, 2, 1536
    X = torch.empty((n, d), dtype=torch.float32, device="cuda")
    step = 65536
    for s0 in range(0, n, step):
        c = min(step, n - s0)
        X[s0:s0 + c] = torch.from_numpy(synth.vsearch_rows(0, s0, c)).cuda()
    Qh = synth.vsearch_rows(1, 0, nq)
    st = {"n": n, "nq": nq, "d": d, "bits": bits, "m": m, "Q": torch.from_numpy(Qh).cuda()[None], "Qh": Qh}
    st["ck"] = tq.Codebook(d, bits, m, "dense", seed=synth.K_SEED)
    st["ws_e"] = torch.empty(tq.workspace_bytes(st["ck"], None, tq.TQ_OP_ENCODE, n), dtype=torch.uint8, device="cuda")
    st["ws_l"] = torch.empty(tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, 1, nq, 1, n, 10), dtype=torch.uint8,
                             device="cuda")
    st["sl"] = torch.tensor([n], dtype=torch.int32, device="cuda")
    Xs = _copies(X, copies)
    st["rot"] = []
    for c in range(copies):
        kp = tq.Packed(st["ck"], n)
        vals = torch.empty((1, nq, 10), dtype=torch.float32, device="cuda")
        if c == 0:
            st["X"], st["kp"] = Xs[0].view(1, n, 1, d), kp
        st["rot"].append([
            ("encode_k", tq.encode_kv(st["ck"], None, Xs[c].view(1, n, 1, d), None, kp, None, L_cap=n,
                                      workspace=st["ws_e"], prepare=True)),
            ("scan_topk", tq.attn_logits(st["ck"], st["Q"], kp, 1, n, st["sl"], top_k=10, out=vals,
                                         workspace=st["ws_l"], prepare=True)[0]),
        ])
    st["calls"] = st["rot"][0]
    return st


def vsearch_report(st, ct, ms_step):
    n, nq, d, bits, m = (st[k] for k in ("n", "nq", "d", "bits", "m"))
    rec = 8 + bits * d // 8 + m // 8
    kern = {"encode_k": {"alg_bytes": n * (4 * d + rec), "units": n, "unit": "vectors",
                         "alg_tflop": 2.0 * n * d * (d + m) / 1e12},
            "scan_topk": {"alg_bytes": n * rec, "units": n * nq, "unit": "scores",
                          "alg_tflop": 2.0 * n * nq * (d + m) / 1e12}}
    products = {"encode_k": BF16_PRODUCTS_PER_FP32_MAC,
                "scan_topk": (BF16_PRODUCTS_PER_FP32_MAC * d + 3 * m) / (d + m)}
    for name, k in kern.items():
        k.update(ct[name])
        _rate(k)
        k["TFLOPs"] = k["alg_tflop"] / (k["us"] * 1e-6)  # fp32 multiply-adds as the method counts them
        k["bf16_products_per_fp32_mac"] = products[name]
        k["bf16_TFLOPs"] = products[name] * k["TFLOPs"]  # what the matrix cores execute
    extra = {"scan_vectors_per_s": n / (kern["scan_topk"]["us"] * 1e-6),
             "scan_scores_per_s": n * nq / (kern["scan_topk"]["us"] * 1e-6),
             "index_vectors_per_s": n / (kern["encode_k"]["us"] * 1e-6),
             "step_vectors_per_s": n / (ms_step * 1e-3)}
    cfg = {"workload": "vector search, 1e6 x 1536 unit vectors, 1024 queries, top-10", "bits": bits, "qjl_rows": m,
           "rotation": "dense Haar", "record_bytes": rec}
    return extra["scan_vectors_per_s"], "vectors/s", kern, extra, cfg


# ------------------------------------------------------------ main
def roofline_of(name, k, rates):
    if "bf16_TFLOPs" in k:
        r = {"bound": "mfma", "achieved": k["bf16_TFLOPs"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": k["bf16_TFLOPs"] / BF16_PEAK_TFLOPS, "dtype": "bf16 (three-piece fp32)",
             "bf16_products_per_fp32_mac": k["bf16_products_per_fp32_mac"], "fp32_equivalent_TFLOPs": k["TFLOPs"],
             "frac_of_fp32_peak": k["TFLOPs"] / FP32_PEAK_TFLOPS}
    else:
        r = {"bound": "hbm", "achieved": k["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": k["GBps"] / HBM_PEAK_GBS, "frac_of_measured_copy": k["GBps"] / rates["copy_GBps"],
             "frac_of_measured_read": k["GBps"] / rates["read_GBps"]}
    r["traffic"] = k.get("traffic_bytes")
    r["kernel"] = name
    r["launch_us"] = k["us"]
    return r


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibrate:
        # a device copy of known size: FETCH_SIZE / WRITE_SIZE of this run calibrate the counters
        r = device_rates(torch, 1024, 3)
        print(json.dumps({"device_copy_MiB": 1024, **r}), flush=True)
        return 0
    import kv_cache_vector_05_amd as tq
    import synth
    wl = args.workload
    copies = max(1, args.copies) if args.cache_state != "hot" else 1
    print(f"[bench] setting up {wl} ({copies} buffer copies)", file=sys.stderr, flush=True)
    if wl in ("llama8b", "llama70b", "llama8b-turboesm"):
        st = setup_llama(torch, tq, synth, wl.split("-")[0], "turboesm" if wl.endswith("turboesm") else "qjl",
                         copies, args.bits, args.qjl_rows, args.context)
        report = llama_report
    elif wl in ("esm650m", "esm650m-turboesm"):
        st = setup_esm(torch, tq, synth, "turboesm" if wl.endswith("turboesm") else "qjl")
        report = esm_report
    elif wl == "vsearch":
        st = setup_vsearch(torch, tq, synth, copies)
        report = vsearch_report
    elif wl == "llama8b-serve":
        st = setup_serve(torch, tq, synth, copies)
        report = serve_report
    elif wl == "llama8b-fib":
        st = setup_fib(torch, tq, synth, copies)
        report = fib_report
    else:
        raise SystemExit("tiny is a parity case, not a benchmark workload")
    nrot = len(st["rot"])
    torch.cuda.synchronize()
    # every buffer copy once (fills all records), then enough steps for the clock ramp
    for i in range(nrot):
        run_step(st, NoTimer(), i)
    torch.cuda.synchronize()
    if args.warmup is None:
        t0 = time.perf_counter()
        run_step(st, NoTimer(), 0)
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        args.warmup = max(nrot + 1, min(2000, int(0.3 / max(one, 1e-6))))
        warm = args.warmup - nrot - 1
    else:
        warm = max(0, args.warmup - nrot)
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(warm):
        run_step(st, NoTimer(), i)
    torch.cuda.synchronize()
    timer = StepTimer(torch, events=args.steps * len(st["rot"][0]))
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(st, timer, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timing each call ({args.cache_state}, {args.reps} repeats)", file=sys.stderr, flush=True)
    ct = time_calls(torch, st, args.cache_state, args.reps)
    for name in ct:
        ct[name]["in_step_us"] = timer.mean_us(name)
    print("[bench] device copy, fill and read rates", file=sys.stderr, flush=True)
    rates = device_rates(torch)
    value, unit, kern, extra, cfg = report(st, ct, ms_step)
    # counter figures are kept per workload; a bit-width override is a workload of its own
    tkey = wl if (args.bits is None and args.qjl_rows is None) else f"{wl}-b{st['bits']}m{st['m']}"
    if args.context is not None:
        tkey += f"-L{args.context}"
    for name, k in kern.items():
        k["traffic_bytes"] = measured_traffic(tkey, name)
        k["frac_of_measured_copy"] = k["GBps"] / rates["copy_GBps"]
    dom = max(kern, key=lambda x: kern[x]["us"])
    roof = roofline_of(dom, kern[dom], rates)
    cores, blas = host_cores()
    line = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg, "roofline": roof}
    if "logits" in kern:
        line["logits_roofline"] = roofline_of("logits", kern["logits"], rates)
    line.update({"timing": {"cache_state": args.cache_state, "buffer_copies": nrot, "repeats": args.reps,
                            "per_call": "median over repeats of back-to-back launches per event pair",
                            "step": "host clock over the timed steps between device synchronisations"},
                 "device_rates": rates, "kernels": kern, **extra})
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        if wl == "llama8b-fib":
            cb = cpu_baseline_fib(st)
        elif wl == "llama8b-serve":
            cb = cpu_baseline_serve(st)
        elif wl in ("esm650m", "esm650m-turboesm"):
            cb = cpu_baseline_esm(st)
        elif wl == "vsearch":
            cb = None
        else:
            cb = cpu_baseline_llama(st, args.cpu_sample or 1 << 22)
        if cb is not None:
            cb["cores"] = blas
            cb["affinity_cores"] = cores
            cb["blas_threads"] = blas
            print("[bench] cpu baseline: tiny configuration on 1 and on all threads", file=sys.stderr, flush=True)
            cb["tiny_one_thread"] = cpu_tiny(1)
            cb["tiny_all_threads"] = cpu_tiny(blas)
            line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
