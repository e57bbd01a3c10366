"""Benchmark of the KV codec's hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

A step is one pass of the whole hot path over one batch of synthetic input
that is already resident in HBM: encode K and V into packed records, score
every cached key for every query head (attention logits), and run the fused
decode (softmax times values).  The default workload is one
Llama-3.1-8B-shaped layer: batch 8, 32 query heads over 8 KV heads, head dim
128, context 32768, bf16 K/V with one percent of channels scaled x100, RoPE
base 5e5, 3-bit Lloyd-Max codes plus a 64-row QJL sketch.

Printed: one JSON line.  `value` is whole-step key throughput (cached keys
encoded, scored and attended per second); per-kernel times come from HIP
events on the launch stream inside the timed region, and `roofline` relates
the dominant kernel's algorithmic bytes per launch to its measured duration.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


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
    import json as _json
    try:
        with open(TRAFFIC_FILE) as fh:
            t = _json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("device_code_sha256") != device_code_digest():
        return None
    return t.get("calls", {}).get(workload, {}).get(call, {}).get("traffic_bytes")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as fill about 0.3 s, at least 3: the "
                         "GPU's clocks take some 100 ms of load to settle)")
    ap.add_argument("--workload", default="llama8b",
                    choices=["llama8b", "llama70b", "esm650m", "vsearch", "llama8b-turboesm", "esm650m-turboesm",
                             "llama8b-serve", "llama8b-fib", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0, help="keys in the oracle's sample (0: default)")
    return ap.parse_args()


class Timer:
    """HIP events on the launch stream around individual API calls (events
    created up front, so that recording them costs the host little)."""

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

    def mean_ms(self, name):
        v = [s.elapsed_time(e) for s, e in self.spans[name]]
        return float(np.mean(v)), len(v)


class NoTimer:
    """Warmup steps: the calls only."""

    def call(self, name, fn):
        fn()


def bf16_dev(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


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
def setup_llama(torch, tq, synth, kind, variant="qjl"):
    if kind == "llama8b":
        B, Hq, H, L, d, bits, m, rope_base = 8, 32, 8, 32768, 128, 3, 64, 5e5
    else:
        B, Hq, H, L, d, bits, m, rope_base = 1, 64, 8, 131072, 128, 3, 128, 0.0
    if variant == "turboesm":
        m = d
    K, V = synth.llama_kv_inputs(kind, seed=0, batch=B, ctx=L, hkv=H, d=d)
    Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
    st = {"B": B, "Hq": Hq, "H": H, "L": L, "d": d, "bits": bits, "m": m, "rope_base": rope_base,
          "variant": variant}
    st["K"], st["V"], st["Q"] = bf16_dev(torch, K), bf16_dev(torch, V), bf16_dev(torch, Q)
    st["host"] = (K, V, Q)
    if variant == "turboesm":
        rope_host = tq.rope_table(rope_base, d, L + 1, device=None) if rope_base else None
        st["ck"], st["cv"] = turboesm_codebooks(tq, synth, d, bits,
                                                synth.bf16_bits_to_f32(K[0, :CALIB_TOKENS]),
                                                synth.bf16_bits_to_f32(V[0, :CALIB_TOKENS]), rope_host)
    else:
        st["ck"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.K_SEED)
        st["cv"] = tq.Codebook(d, bits, m, "hadamard", seed=synth.V_SEED)
    st["kp"] = tq.Packed(st["ck"], B * H * L)
    st["vp"] = tq.Packed(st["cv"], B * H * L)
    st["rope"] = tq.rope_table(rope_base, d, L + 1) if rope_base else None
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["logits"] = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    st["out"] = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    st["ws_l"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    # every call of the step with its arguments marshalled once
    st["calls"] = [
        ("encode_k", tq.encode_kv(st["ck"], None, st["K"], None, st["kp"], None, L_cap=L, rope=st["rope"],
                                  prepare=True)),
        ("encode_v", tq.encode_kv(None, st["cv"], None, st["V"], None, st["vp"], L_cap=L, prepare=True)),
        ("logits", tq.attn_logits(st["ck"], st["Q"], st["kp"], H, L, st["sl"], rope=st["rope"], out=st["logits"],
                                  workspace=st["ws_l"], prepare=True)[0]),
        ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], st["kp"], st["vp"], H, L, st["sl"], rope=st["rope"],
                                  out=st["out"], workspace=st["ws_d"], prepare=True)[0]),
    ]
    return st


def run_calls(st, timer):
    for name, launch in st["calls"]:
        timer.call(name, launch)


def llama_report(st, timer, ms_step):
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    G = Hq // H
    keys = B * H * L
    sign = st["variant"] == "turboesm"
    rec = 4 + (4 if m and not sign else 0) + bits * d // 8 + m // 8
    in_bytes = 2 * d  # bf16
    enc_ms, n_enc = timer.mean_ms("encode_k")
    encv_ms, _ = timer.mean_ms("encode_v")
    log_ms, _ = timer.mean_ms("logits")
    dec_ms, _ = timer.mean_ms("decode")
    kern = {
        "encode_k": {"ms": enc_ms, "launches": n_enc, "alg_bytes": keys * (in_bytes + rec),
                     "unit": "vectors", "units": keys},
        "encode_v": {"ms": encv_ms, "alg_bytes": keys * (in_bytes + rec), "units": keys},
        "logits": {"ms": log_ms, "alg_bytes": keys * (rec + 4 * G), "units": keys},
        "decode": {"ms": dec_ms, "alg_bytes": keys * 2 * rec, "units": keys},
    }
    for k in kern.values():
        k["GBps"] = k["alg_bytes"] / (k["ms"] * 1e-3) / 1e9
        k["hbm_frac"] = k["GBps"] / HBM_PEAK_GBS
    dom = max(("encode_k", "encode_v", "logits", "decode"), key=lambda k: kern[k]["ms"])
    extra = {
        "logit_keys_per_s": keys / (log_ms * 1e-3),
        "logit_hbm_frac": kern["logits"]["hbm_frac"],
        "decode_keys_per_s": keys / (dec_ms * 1e-3),
        "encode_tokens_per_s": B * L / ((enc_ms + encv_ms) * 1e-3),
        "encode_vectors_per_s": 2 * keys / ((enc_ms + encv_ms) * 1e-3),
    }
    name = f"{'Llama-3.1-8B' if L == 32768 else 'Llama-70B'}-shaped decode layer"
    cfg = {"workload": name + (", TurboESM-style records" if sign else ""), "batch": B,
           "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "bits": bits,
           "input_dtype": "bf16", "rope_base": st["rope_base"], "record_bytes": rec}
    if sign:
        cfg.update({"residual_signs": "one per coordinate, mu per KV head", "key_table": "calibrated, rotated",
                    "value_table": "calibrated, original coordinates", "calibration_tokens": CALIB_TOKENS})
    else:
        cfg["qjl_rows"] = m
    return keys / (ms_step * 1e-3), "keys/s", kern, dom, extra, cfg


# ------------------------------------------------------------ FibQuant codebooks
FIB_BITS = 4  # 16 codewords per 2-coordinate block: 2 bits per coordinate


def setup_fib(torch, tq, synth):
    """The Llama-3.1-8B-shaped layer with FibQuant vector codebooks for keys
    and values (k = 2, N = 16): encode K (RoPE), encode V, the logit scan of
    the 32 query heads over every cached key, and the fused decode."""
    B, Hq, H, L, d = 8, 32, 8, 32768, 128
    K, V = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L, hkv=H, d=d)
    Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
    st = {"B": B, "Hq": Hq, "H": H, "L": L, "d": d, "bits": FIB_BITS, "rope_base": 5e5, "host": (K, V, Q)}
    st["K"], st["V"], st["Q"] = bf16_dev(torch, K), bf16_dev(torch, V), bf16_dev(torch, Q)
    st["ck"] = tq.Codebook(d, FIB_BITS, 0, "hadamard", seed=synth.K_SEED, block=2)
    st["cv"] = tq.Codebook(d, FIB_BITS, 0, "hadamard", seed=synth.V_SEED, block=2)
    st["kp"], st["vp"] = tq.Packed(st["ck"], B * H * L), tq.Packed(st["cv"], B * H * L)
    st["rope"] = tq.rope_table(5e5, d, L + 1)
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["logits"] = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    st["ws_l"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["out"] = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["calls"] = [
        ("encode_k", tq.encode_kv(st["ck"], None, st["K"], None, st["kp"], None, L_cap=L, rope=st["rope"],
                                  prepare=True)),
        ("encode_v", tq.encode_kv(None, st["cv"], None, st["V"], None, st["vp"], L_cap=L, prepare=True)),
        ("logits", tq.attn_logits(st["ck"], st["Q"], st["kp"], H, L, st["sl"], rope=st["rope"], out=st["logits"],
                                  workspace=st["ws_l"], prepare=True)[0]),
        ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], st["kp"], st["vp"], H, L, st["sl"], rope=st["rope"],
                                  out=st["out"], workspace=st["ws_d"], prepare=True)[0]),
    ]
    return st


def fib_report(st, timer, ms_step):
    B, Hq, H, L, d, bits = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits"))
    keys = B * H * L
    rec = 4 + 4 * ((d // 2 * bits + 31) // 32)
    enc_ms, n = timer.mean_ms("encode_k")
    encv_ms, _ = timer.mean_ms("encode_v")
    log_ms, _ = timer.mean_ms("logits")
    dec_ms, _ = timer.mean_ms("decode")
    kern = {"encode_k": {"ms": enc_ms, "launches": n, "alg_bytes": keys * (2 * d + rec), "units": keys},
            "encode_v": {"ms": encv_ms, "alg_bytes": keys * (2 * d + rec), "units": keys},
            "logits": {"ms": log_ms, "alg_bytes": keys * (rec + 4 * Hq // H), "units": keys},
            "decode": {"ms": dec_ms, "alg_bytes": keys * 2 * rec, "units": keys}}
    for k in kern.values():
        k["GBps"] = k["alg_bytes"] / (k["ms"] * 1e-3) / 1e9
        k["hbm_frac"] = k["GBps"] / HBM_PEAK_GBS
    dom = max(kern, key=lambda x: kern[x]["ms"])
    extra = {"logit_keys_per_s": keys / (log_ms * 1e-3), "logit_hbm_frac": kern["logits"]["hbm_frac"],
             "decode_keys_per_s": keys / (dec_ms * 1e-3),
             "encode_vectors_per_s": 2 * keys / ((enc_ms + encv_ms) * 1e-3)}
    cfg = {"workload": "Llama-3.1-8B-shaped layer with FibQuant vector codebooks (encode K, V; logits; decode)",
           "batch": B,
           "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "block": 2, "codewords": 1 << bits,
           "bits_per_coordinate": bits / 2, "input_dtype": "bf16", "rope_base": st["rope_base"],
           "record_bytes": rec}
    return keys / (ms_step * 1e-3), "keys/s", kern, dom, extra, cfg


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
    try:
        import threadpoolctl
        threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": done / dt, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{pairs} (sequence, KV head) pairs, the first {n} keys and values of each encoded, scored "
                      f"and attended for {G} query heads by the oracle, {dt:.1f} s on the host (codebook built beforehand, "
                      f"{t_setup:.1f} s)"}


# ------------------------------------------------------------ serving step
PAGE = 256  # slots per page of the paged cache


def setup_serve(torch, tq, synth):
    """One autoregressive step of the Llama-3.1-8B-shaped layer over a paged
    cache: the cache holds L - 1 tokens per sequence, spread over a shuffled
    pool of pages; a step appends token L - 1 (keys and values of every
    (sequence, KV head)) and runs the fused decode over the L tokens."""
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
    st["kp"] = tq.Packed(st["ck"], st["pages"].records(H))
    st["vp"] = tq.Packed(st["cv"], st["pages"].records(H))
    st["rope"] = tq.rope_table(rope_base, d, L + 1)
    Kd, Vd = bf16_dev(torch, K), bf16_dev(torch, V)
    # prefill: the first L - 1 tokens
    tq.encode_kv(st["ck"], st["cv"], Kd[:, :L - 1], Vd[:, :L - 1], st["kp"], st["vp"], rope=st["rope"],
                 pages=st["pages"])
    st["K1"], st["V1"] = Kd[:, L - 1].contiguous(), Vd[:, L - 1].contiguous()
    st["pos"] = torch.full((B,), L - 1, dtype=torch.int32, device="cuda")
    st["sl"] = torch.full((B,), L, dtype=torch.int32, device="cuda")
    st["Q"] = bf16_dev(torch, Q)
    st["out"] = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    st["ws_d"] = torch.empty(max(1, tq.workspace_bytes(st["ck"], st["cv"], tq.TQ_OP_DECODE, B, Hq, H, L, 0)),
                             dtype=torch.uint8, device="cuda")
    st["calls"] = [
        ("append", tq.append_kv(st["ck"], st["cv"], st["K1"], st["V1"], st["kp"], st["vp"], st["pos"],
                                pages=st["pages"], rope=st["rope"], prepare=True)),
        ("decode", tq.attn_decode(st["ck"], st["cv"], st["Q"], st["kp"], st["vp"], H, None, st["sl"], rope=st["rope"],
                                  out=st["out"], workspace=st["ws_d"], prepare=True, pages=st["pages"])[0]),
    ]
    return st


def serve_report(st, timer, ms_step):
    B, Hq, H, L, d, bits, m = (st[k] for k in ("B", "Hq", "H", "L", "d", "bits", "m"))
    keys = B * H * L
    rec = 8 + bits * d // 8 + m // 8
    app_ms, n = timer.mean_ms("append")
    dec_ms, _ = timer.mean_ms("decode")
    kern = {"append": {"ms": app_ms, "launches": n, "alg_bytes": 2 * B * H * (2 * d + rec), "units": 2 * B * H},
            "decode": {"ms": dec_ms, "alg_bytes": keys * 2 * rec, "units": keys}}
    for k in kern.values():
        k["GBps"] = k["alg_bytes"] / (k["ms"] * 1e-3) / 1e9
        k["hbm_frac"] = k["GBps"] / HBM_PEAK_GBS
    extra = {"decode_keys_per_s": keys / (dec_ms * 1e-3), "append_us": app_ms * 1e3, "decode_us": dec_ms * 1e3,
             "tokens_per_s": B / (ms_step * 1e-3)}
    cfg = {"workload": "Llama-3.1-8B-shaped decode step over a paged cache (append + fused decode)", "batch": B,
           "q_heads": Hq, "kv_heads": H, "head_dim": d, "context": L, "bits": bits, "qjl_rows": m,
           "input_dtype": "bf16", "rope_base": st["rope_base"], "record_bytes": rec, "page_size": PAGE,
           "pages": B * (L // PAGE), "page_order": "shuffled"}
    return keys / (ms_step * 1e-3), "keys/s", kern, "decode", extra, cfg


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
            qp, s = estimator.prep_query(ock, q, L, rope)
            estimator.attention(ock, ocv, qp, s, cat(ek, nk), cat(ev, nv), L, 1 / math.sqrt(d))
            dt += time.perf_counter() - t1
            done += L
            pairs += 1
    try:
        import threadpoolctl
        threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": done / dt, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{pairs} (sequence, KV head) pairs: the append of one key and value and the decode of "
                      f"{G} query heads over {L} cached keys each, {dt:.1f} s on the host (the caches encoded "
                      f"beforehand, untimed)"}


def cpu_baseline_llama(st, sample_keys, budget_s=12.0):
    """The oracle on a bounded sample: (sequence, KV head) pairs in order,
    each fully encoded (keys with RoPE, values), scored for its G query heads
    and decoded, until about budget_s seconds of host time or sample_keys
    keys."""
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
    done, pairs, dt = 0, 0, 0.0
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
            qp, s = estimator.prep_query(ock, q, n, rope)
            estimator.logits(ock, qp, s, ek, kh)
            estimator.attention(ock, ocv, qp, s, ek, ev, n, 1 / math.sqrt(d), kh)
            dt += time.perf_counter() - t1
            done += n
            pairs += 1
    try:
        import threadpoolctl
        threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": done / dt, "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} keys+values: the first {pairs} (sequence, KV head) pairs, each encoded "
                      f"(keys with RoPE), scored for its {G} query heads and decoded by the oracle; "
                      f"{dt:.1f} s on the host (codebook tables built once beforehand, {t_setup:.1f} s)"}


def oracle_turboesm_codebooks(synth, d, bits, k_sample, v_sample, rope):
    """The oracle's own calibration and sign-corrected codebooks for the same
    samples (the CPU baseline times the oracle as it stands)."""
    from oracle import calibration, codec, rng, rotation
    sigma = rng.signs(synth.K_SEED, d)  # the seeded signs the library derives from the same seed
    lk, mk = calibration.calibrate(rotation.rht_matrix(sigma), bits, k_sample, rope=rope)
    lv, mv = calibration.calibrate(np.eye(d), bits, v_sample)
    return (codec.make_sign_codebook(d, bits, "hadamard", sigma=sigma, levels=lk, mu=mk),
            codec.make_sign_codebook(d, bits, "none", levels=lv, mu=mv))


# ------------------------------------------------------------ ESM-2 prefill
def setup_esm(torch, tq, synth, variant="qjl"):
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
    st["calls"] = []
    for layer in range(layers):
        st["calls"].append(("encode_k", tq.encode_kv(cks[layer], None, Ks[layer], None, st["kp"][layer], None,
                                                     L_cap=T, rope=st["rope"], prepare=True)))
        st["calls"].append(("encode_v", tq.encode_kv(None, cvs[layer], None, Vs[layer], None, st["vp"][layer],
                                                     L_cap=T, prepare=True)))
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
    try:
        import threadpoolctl
        threads = max(p["num_threads"] for p in threadpoolctl.threadpool_info()) or 1
    except Exception:
        threads = len(os.sched_getaffinity(0))
    # `done` key+value vector pairs of one layer; a token needs layers * H of them
    return {"value": done / dt / (layers * H), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} key+value vector pairs of layer 0 ({done // T} (sequence, head) pairs of {T} tokens) "
                      f"encoded by the oracle in {dt:.1f} s on the host, scaled to tokens of the {layers}-layer, "
                      f"{H}-head encode (codebook tables built once beforehand, {t_setup:.1f} s)"}


def esm_report(st, timer, ms_step):
    S, T, H, d, layers, bits, m = (st[k] for k in ("S", "T", "H", "d", "layers", "bits", "m"))
    vec = S * T * H
    sign = st["variant"] == "turboesm"
    rec = 4 + (0 if sign else 4) + bits * d // 8 + m // 8
    enc_ms, n = timer.mean_ms("encode_k")
    encv_ms, _ = timer.mean_ms("encode_v")
    kern = {"encode_k": {"ms": enc_ms, "launches": n, "alg_bytes": vec * (4 * d + rec), "units": vec},
            "encode_v": {"ms": encv_ms, "alg_bytes": vec * (4 * d + rec), "units": vec}}
    for k in kern.values():
        k["GBps"] = k["alg_bytes"] / (k["ms"] * 1e-3) / 1e9
        k["hbm_frac"] = k["GBps"] / HBM_PEAK_GBS
    extra = {"encode_tokens_per_s": S * T / (ms_step * 1e-3), "encode_vectors_per_s": 2 * layers * vec / (ms_step * 1e-3),
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
    return S * T / (ms_step * 1e-3), "tokens/s", kern, "encode_k", extra, cfg


# ------------------------------------------------------------ vector search
def setup_vsearch(torch, tq, synth):
    n, nq, d, bits, m = 1_000_000, 1024, 1536, 2, 1536
    X = torch.empty((n, d), dtype=torch.float32, device="cuda")
    step = 65536
    for s0 in range(0, n, step):
        c = min(step, n - s0)
        X[s0:s0 + c] = torch.from_numpy(synth.vsearch_rows(0, s0, c)).cuda()
    Qh = synth.vsearch_rows(1, 0, nq)
    st = {"n": n, "nq": nq, "d": d, "bits": bits, "m": m, "X": X.view(1, n, 1, d),
          "Q": torch.from_numpy(Qh).cuda()[None], "Qh": Qh}
    st["ck"] = tq.Codebook(d, bits, m, "dense", seed=synth.K_SEED)
    st["kp"] = tq.Packed(st["ck"], n)
    st["ws_e"] = torch.empty(tq.workspace_bytes(st["ck"], None, tq.TQ_OP_ENCODE, n), dtype=torch.uint8, device="cuda")
    st["ws_l"] = torch.empty(tq.workspace_bytes(st["ck"], None, tq.TQ_OP_LOGITS, 1, nq, 1, n, 10), dtype=torch.uint8,
                             device="cuda")
    st["sl"] = torch.tensor([n], dtype=torch.int32, device="cuda")
    st["calls"] = [
        ("encode_k", tq.encode_kv(st["ck"], None, st["X"], None, st["kp"], None, L_cap=n, workspace=st["ws_e"],
                                  prepare=True)),
        ("scan_topk", tq.attn_logits(st["ck"], st["Q"], st["kp"], 1, n, st["sl"], top_k=10, workspace=st["ws_l"],
                                     prepare=True)[0]),
    ]
    return st


def vsearch_report(st, timer, ms_step):
    n, nq, d, bits, m = (st[k] for k in ("n", "nq", "d", "bits", "m"))
    rec = 8 + bits * d // 8 + m // 8
    enc_ms, k = timer.mean_ms("encode_k")
    scan_ms, _ = timer.mean_ms("scan_topk")
    kern = {"encode_k": {"ms": enc_ms, "launches": k, "alg_bytes": n * (4 * d + rec), "units": n,
                         "alg_tflop": 2.0 * n * d * (d + m) / 1e12},
            "scan_topk": {"ms": scan_ms, "alg_bytes": n * rec, "units": n * nq,
                          "alg_tflop": 2.0 * n * nq * (d + m) / 1e12}}
    for kk in kern.values():
        kk["GBps"] = kk["alg_bytes"] / (kk["ms"] * 1e-3) / 1e9
        kk["hbm_frac"] = kk["GBps"] / HBM_PEAK_GBS
        kk["TFLOPs"] = kk["alg_tflop"] / (kk["ms"] * 1e-3)
    extra = {"scan_scores_per_s": n * nq / (scan_ms * 1e-3), "index_vectors_per_s": n / (enc_ms * 1e-3)}
    cfg = {"workload": "vector search, 1e6 x 1536 unit vectors, 1024 queries, top-10", "bits": bits, "qjl_rows": m,
           "rotation": "dense Haar", "record_bytes": rec}
    return n / (ms_step * 1e-3), "vectors/s", kern, max(kern, key=lambda x: kern[x]["ms"]), extra, cfg


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    import torch
    import kv_cache_vector_05_amd as tq
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    wl = args.workload
    print(f"[bench] setting up {wl}", file=sys.stderr, flush=True)
    if wl in ("llama8b", "llama70b", "llama8b-turboesm"):
        st = setup_llama(torch, tq, synth, wl.split("-")[0], "turboesm" if wl.endswith("turboesm") else "qjl")
        report = lambda t, ms: llama_report(st, t, ms)
    elif wl in ("esm650m", "esm650m-turboesm"):
        st = setup_esm(torch, tq, synth, "turboesm" if wl.endswith("turboesm") else "qjl")
        report = lambda t, ms: esm_report(st, t, ms)
    elif wl == "vsearch":
        st = setup_vsearch(torch, tq, synth)
        report = lambda t, ms: vsearch_report(st, t, ms)
    elif wl == "llama8b-serve":
        st = setup_serve(torch, tq, synth)
        report = lambda t, ms: serve_report(st, t, ms)
    elif wl == "llama8b-fib":
        st = setup_fib(torch, tq, synth)
        report = lambda t, ms: fib_report(st, t, ms)
    else:
        raise SystemExit("tiny is a parity case, not a benchmark workload")
    step = lambda t: run_calls(st, t)
    torch.cuda.synchronize()
    if args.warmup is None:
        # enough steps to cover the clock ramp under load (~0.3 s), at least 3,
        # sized from the second step (the first carries one-time set-up)
        step(NoTimer())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step(NoTimer())
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        args.warmup = max(3, min(2000, int(0.3 / max(one, 1e-6))))
        warm = args.warmup - 2
    else:
        warm = args.warmup
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(warm):
        step(NoTimer())
    torch.cuda.synchronize()
    timer = Timer(torch, events=args.steps * len(st["calls"]))
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    value, unit, kern, dom, extra, cfg = report(timer, ms_step)
    dk = kern[dom]
    for name, k in kern.items():
        k["traffic_bytes"] = measured_traffic(wl, name)
    if "TFLOPs" in dk and dom == "scan_topk":
        roof = {"bound": "mfma", "achieved": dk["TFLOPs"], "peak": 157.3, "unit": "TFLOP/s",
                "frac": dk["TFLOPs"] / 157.3, "traffic": dk["traffic_bytes"], "kernel": dom}
    else:
        roof = {"bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dk["GBps"] / HBM_PEAK_GBS, "traffic": dk["traffic_bytes"], "kernel": dom}
    line = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg, "roofline": roof,
            "kernels": kern, **extra}
    if not args.no_cpu_baseline and wl == "llama8b-fib":
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_fib(st)
    elif not args.no_cpu_baseline and wl == "llama8b-serve":
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_serve(st)
    elif not args.no_cpu_baseline and wl in ("llama8b", "llama70b", "llama8b-turboesm"):
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_llama(st, args.cpu_sample or 1 << 22)
    elif not args.no_cpu_baseline and wl in ("esm650m", "esm650m-turboesm"):
        print("[bench] cpu baseline (oracle on a sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_esm(st)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
