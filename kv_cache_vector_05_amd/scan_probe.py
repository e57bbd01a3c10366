"""Times the attention-logit scan at the Llama-3.1-8B decode shape (8
sequences, 32 query and 8 KV heads, d = 128, 3-bit codes with a 64-row
sketch) in two states of the memory-side cache, at contexts of 2048 and
32768 tokens:

* hot: the same launch repeated, so the key records (134 MB at 32768 tokens)
  stay in the 256 MB memory-side cache;
* flushed: a 1 GiB device fill before each launch evicts them.

A scan bound by HBM bandwidth runs faster hot than flushed; one bound by its
own instruction stream does not.

    python kv_cache_vector_05_amd/scan_probe.py [--reps 30]

Each (context, state) pair runs --reps launches in that order: 2048 hot,
2048 flushed, 32768 hot, 32768 flushed. The printed medians skip the first
five launches of each pair and include the query preparation.
"""
from __future__ import annotations

import argparse
import os
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=30)
    args = ap.parse_args(argv)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("scan_probe needs a GPU", file=sys.stderr)
        return 1
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    import kv_cache_vector_05_amd as tq
    import synth

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    torch.cuda.set_device(0)
    B, Hq, H, d = 8, 32, 8, 128
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    for L in (2048, 32768):
        K, _ = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L, hkv=H, d=d)
        Q = synth.llama_q_inputs(seed=100, batch=B, hq=Hq, d=d)
        ck = tq.Codebook(d, 3, 64, "hadamard", seed=synth.K_SEED)
        kp = tq.Packed(ck, B * H * L)
        rope = tq.rope_table(5e5, d, L + 1)
        tq.encode_kv(ck, None, bf16(K), None, kp, None, L_cap=L, rope=rope)
        sl = torch.full((B,), L, dtype=torch.int32, device="cuda")
        out = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, tq.workspace_bytes(ck, None, tq.TQ_OP_LOGITS, B, Hq, H, L, 0)),
                         dtype=torch.uint8, device="cuda")
        call = tq.attn_logits(ck, bf16(Q), kp, H, L, sl, rope=rope, out=out, workspace=ws, prepare=True)[0]
        torch.cuda.synchronize()
        for state in ("hot", "flushed"):
            ts = []
            for rep in range(args.reps):
                if state == "flushed":
                    flush.fill_(float(rep))
                s = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                s.record()
                call()
                e.record()
                torch.cuda.synchronize()
                ts.append(s.elapsed_time(e) * 1000.0)
            ts = sorted(ts[5:])
            med = ts[len(ts) // 2]
            keys = B * H * L
            print(f"context {L} {state}: median {med:.1f} us per launch, {keys / med / 1e3:.2f} G keys/s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
