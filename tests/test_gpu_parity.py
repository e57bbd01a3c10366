"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, for down-scaled versions of every workload shape plus
edge cases.  Full-size runs are in test_gpu_fullsize.py."""
import math

import numpy as np
import pytest

import synth
from oracle import codec, estimator, rope as orope

import parity

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_05_amd")

pytestmark = pytest.mark.gpu


def codebooks(d, bits, m, dense, seed):
    sigma, rg, sk = synth.codec_draws(d, m, dense, seed)
    o = codec.make_codebook(d, bits, m, dense, sigma, rg, sk)
    g = tq.Codebook(d, bits, m, "dense" if dense else "hadamard", sigma=sigma, rot_gauss=rg, sketch=sk)
    return o, g


def stored(enc: codec.Encoded) -> codec.Encoded:
    """The record as the cache stores it: nu and gamma rounded to float32."""
    return codec.Encoded(enc.norm.astype(np.float32).astype(np.float64),
                         enc.rnorm.astype(np.float32).astype(np.float64), enc.codes, enc.signs)


def rows(enc, lo, hi):
    return codec.Encoded(enc.norm[lo:hi], enc.rnorm[lo:hi], enc.codes[lo:hi], enc.signs[lo:hi])


def upload(gcb, enc):
    return tq.Packed.from_arrays(gcb, enc.norm, enc.rnorm, enc.codes, enc.signs)


def bf16_tensor(bits_u16):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).cuda().view(torch.bfloat16)


def check_logits_and_decode(ock, gck, ocv, gcv, encK, encV, q_f32, q_dev, B, Hq, H, L, sl, rope_o, rope_g,
                            label, do_decode=True):
    G = Hq // H
    sl_t = torch.tensor(sl, dtype=torch.int32, device="cuda")
    kpo = upload(gck, encK)
    sentinel = torch.full((B, Hq, L), float("nan"), device="cuda")
    lg = tq.attn_logits(gck, q_dev, kpo, H, L, sl_t, rope=rope_g, out=sentinel).cpu().numpy()
    if do_decode:
        vpo = upload(gcv, encV)
        out = tq.attn_decode(gck, gcv, q_dev, kpo, vpo, H, L, sl_t, rope=rope_g).cpu().numpy()
    for b in range(B):
        pos = min(max(sl[b], 0), L)
        qp, s = estimator.prep_query(ock, q_f32[b], pos, rope_o)
        for kh in range(H):
            n0 = (b * H + kh) * L
            ek = rows(encK, n0, n0 + L)
            gsl = slice(kh * G, (kh + 1) * G)
            ref = estimator.logits(ock, qp[gsl], s[gsl], ek, kh)[:, :pos]
            parity.assert_close(lg[b, gsl, :pos], ref, f"{label} logits b={b} kh={kh}")
            assert np.all(np.isnan(lg[b, gsl, pos:])), f"{label}: logits past seq_len were written"
            if do_decode:
                ev = rows(encV, n0, n0 + L)
                ref_o = estimator.attention(ock, ocv, qp[gsl], s[gsl], ek, ev, pos, 1.0 / math.sqrt(ock.d), kh)
                parity.assert_close(out[b, gsl], ref_o, f"{label} decode b={b} kh={kh}")


def test_tiny_encode_and_logits():
    """4096 fp32 keys with two x50 outlier channels, b=2, m=128, 16 queries."""
    k, q, _ = synth.tiny_inputs(0)
    ock, gck = codebooks(128, 2, 128, False, synth.K_SEED)
    kp = tq.Packed(gck, 4096)
    tq.encode_kv(gck, None, torch.from_numpy(k).cuda().view(1, 4096, 1, 128), None, kp, None, L_cap=4096)
    torch.cuda.synchronize()
    enc = codec.encode(ock, k)
    info = parity.compare_encoded(ock, enc, kp.numpy(), "tiny K")
    assert info["n"] == 4096
    check_logits_and_decode(ock, gck, None, None, stored(enc), None, q[None], torch.from_numpy(q).cuda()[None],
                            1, 16, 1, 4096, [4096], None, None, "tiny", do_decode=False)


def test_llama8b_shaped_small():
    """bf16 K/V with 1% outlier channels, RoPE base 5e5, b=3 + m=64, GQA 32/8,
    a ragged context and two different sequence lengths."""
    B, Hq, H, L, d = 2, 32, 8, 1000, 128
    K, V = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L)
    Q = synth.llama_q_inputs(seed=100, batch=B)
    ock, gck = codebooks(d, 3, 64, False, synth.K_SEED)
    ocv, gcv = codebooks(d, 3, 64, False, synth.V_SEED)
    rope_g = tq.rope_table(5e5, d, L + 1)
    rope_o = orope.rope_table(5e5, d, L + 1)
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, bf16_tensor(K), bf16_tensor(V), kp, vp, L_cap=L, rope=rope_g)
    torch.cuda.synchronize()
    kf, vf = synth.bf16_bits_to_f32(K), synth.bf16_bits_to_f32(V)
    ek = codec.encode(ock, parity.oracle_rows(kf), pos=np.tile(np.arange(L), B * H), rope=rope_o)
    ev = codec.encode(ocv, parity.oracle_rows(vf))
    parity.compare_encoded(ock, ek, kp.numpy(), "llama8b K")
    parity.compare_encoded(ocv, ev, vp.numpy(), "llama8b V")
    qf = synth.bf16_bits_to_f32(Q)
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), qf, bf16_tensor(Q), B, Hq, H, L,
                            [1000, 777], rope_o, rope_g, "llama8b")


def test_llama70b_shaped_small():
    """Student-t(3) channel scales, no RoPE, b=3 + m=128, GQA 64/8."""
    B, Hq, H, L, d = 1, 64, 8, 2500, 128
    K, V = synth.llama_kv_inputs("llama70b", seed=0, batch=B, ctx=L)
    Q = synth.llama_q_inputs(seed=101, batch=B, hq=Hq)
    ock, gck = codebooks(d, 3, 128, False, synth.K_SEED)
    ocv, gcv = codebooks(d, 3, 128, False, synth.V_SEED)
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, bf16_tensor(K), bf16_tensor(V), kp, vp, L_cap=L)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(synth.bf16_bits_to_f32(K)))
    ev = codec.encode(ocv, parity.oracle_rows(synth.bf16_bits_to_f32(V)))
    parity.compare_encoded(ock, ek, kp.numpy(), "llama70b K")
    parity.compare_encoded(ocv, ev, vp.numpy(), "llama70b V")
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), synth.bf16_bits_to_f32(Q), bf16_tensor(Q),
                            B, Hq, H, L, [2500], None, None, "llama70b")


def test_esm_shaped_small():
    """d=64 heads, 20 per layer, fp32 projections of a 20-letter alphabet,
    RoPE base 1e4, b=3 + m=64; keys and values of one layer."""
    S, T, H, d = 2, 300, 20, 64
    pk, pv = synth.esm_layer_tables(0)
    tok = synth.esm_tokens(0, S, T)
    K = pk[tok].reshape(S, T, H, d)
    V = pv[tok].reshape(S, T, H, d)
    ock, gck = codebooks(d, 3, 64, False, synth.K_SEED)
    ocv, gcv = codebooks(d, 3, 64, False, synth.V_SEED)
    rope_g = tq.rope_table(1e4, d, T)
    rope_o = orope.rope_table(1e4, d, T)
    kp, vp = tq.Packed(gck, S * H * T), tq.Packed(gcv, S * H * T)
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=T, rope=rope_g)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(K), pos=np.tile(np.arange(T), S * H), rope=rope_o)
    ev = codec.encode(ocv, parity.oracle_rows(V))
    parity.compare_encoded(ock, ek, kp.numpy(), "esm K")
    parity.compare_encoded(ocv, ev, vp.numpy(), "esm V")


def test_vector_search_shaped_small():
    """Dense Haar rotation at d=1536, b=2 + m=1536: index encode, full scan
    (dense logits) and top-10 per query."""
    n, nq, d = 3000, 32, 1536
    X = synth.vsearch_rows(0, 0, n)
    Q = synth.vsearch_rows(1, 0, nq)
    ock, gck = codebooks(d, 2, 1536, True, synth.K_SEED)
    kp = tq.Packed(gck, n)
    tq.encode_kv(gck, None, torch.from_numpy(X).cuda().view(1, n, 1, d), None, kp, None, L_cap=n)
    torch.cuda.synchronize()
    enc = codec.encode(ock, X)
    parity.compare_encoded(ock, enc, kp.numpy(), "vsearch index")
    st = stored(enc)
    kpo = upload(gck, st)
    qt = torch.from_numpy(Q).cuda()[None]
    sl = torch.tensor([n], dtype=torch.int32, device="cuda")
    lg = tq.attn_logits(gck, qt, kpo, 1, n, sl).cpu().numpy()[0]
    qp, s = estimator.prep_query(ock, Q)
    ref = estimator.logits(ock, qp, s, st)
    parity.assert_close(lg, ref, "vsearch scores")
    vals, idx = tq.attn_logits(gck, qt, kpo, 1, n, sl, top_k=10)
    vals, idx = vals.cpu().numpy()[0], idx.cpu().numpy()[0]
    ridx, rval = estimator.topk(ref, 10)
    check_topk(vals, idx, ref, rval)


@pytest.mark.parametrize("bits,m", [(1, 64), (3, 64), (4, 32), (2, 0)])
def test_dense_logits_bit_widths(bits, m):
    """Dense Haar rotation at d = 128: logits from records the oracle wrote,
    for the widths the score GEMM decodes from the records itself (1, 2, 4
    bits) and for 3 bits (dequantised first); a ragged key count."""
    n, nq, d = 700, 8, 128
    X = synth.vsearch_rows(2, 0, n, d=d)
    Q = synth.vsearch_rows(3, 0, nq, d=d)
    ock, gck = codebooks(d, bits, m, True, 11 + bits)
    st = stored(codec.encode(ock, X))
    kpo = upload(gck, st)
    qt = torch.from_numpy(Q).cuda()[None]
    sl = torch.tensor([n], dtype=torch.int32, device="cuda")
    lg = tq.attn_logits(gck, qt, kpo, 1, n, sl).cpu().numpy()[0]
    qp, s_ = estimator.prep_query(ock, Q)
    parity.assert_close(lg, estimator.logits(ock, qp, s_, st), f"dense logits b{bits} m{m}")


def check_topk(vals, idx, ref_scores, ref_vals, k=10):
    """Top-k sets agree up to near-ties (tests/parity.py::check_topk)."""
    parity.check_topk(vals, idx, ref_scores, k)


@pytest.mark.parametrize("d,bits,m", [(64, 1, 32), (64, 2, 0), (64, 4, 64), (128, 1, 128), (128, 2, 64),
                                      (128, 4, 0), (128, 4, 128)])
def test_bit_widths_and_sketch_sizes(d, bits, m):
    """Every table width with sketch off, at half width and at full width:
    encode (ragged tail), logits and decode, with GQA 6/2 (not a multiple of
    the kernel's query tile)."""
    B, Hq, H, L = 2, 6, 2, 333
    g = synth.rng(d * 10 + bits * 3 + m)
    K = g.standard_normal((B, L, H, d)).astype(np.float32)
    V = g.standard_normal((B, L, H, d)).astype(np.float32)
    Q = g.standard_normal((B, Hq, d)).astype(np.float32)
    ock, gck = codebooks(d, bits, m, False, 5)
    ocv, gcv = codebooks(d, bits, m, False, 6)
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=L)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(K))
    ev = codec.encode(ocv, parity.oracle_rows(V))
    parity.compare_encoded(ock, ek, kp.numpy(), f"K d{d} b{bits} m{m}")
    parity.compare_encoded(ocv, ev, vp.numpy(), f"V d{d} b{bits} m{m}")
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), Q, torch.from_numpy(Q).cuda(), B, Hq, H,
                            L, [333, 45], None, None, f"d{d} b{bits} m{m}")


@pytest.mark.parametrize("d,bits,m,dtype,rope,H", [
    (128, 3, 64, "bf16", True, 3),    # bf16 RoPE keys, heads not a multiple of 4: rows read per wave
    (128, 3, 64, "bf16", True, 4),    # bf16 RoPE keys, rows staged per block
    (128, 4, 128, "bf16", True, 8),   # 4-bit byte-packed codes, full-width sketch
    (128, 3, 64, "f32", True, 2),     # fp32 RoPE keys
    (128, 3, 0, "bf16", False, 5),    # raw bf16 operands, no sketch
    (128, 2, 128, "bf16", True, 1),   # per-coordinate packing with RoPE
    (64, 3, 64, "bf16", True, 4),     # d = 64, bf16 RoPE, staged
    (64, 4, 32, "bf16", False, 3),    # d = 64, 4-bit, one sketch row block
])
def test_encoder_paths(d, bits, m, dtype, rope, H):
    """The Hadamard encoder's paths (raw bf16 or split fp16 operands, RoPE rows
    staged or read per wave, 2/3/4-bit packing, sketch widths) at a token offset
    in a larger cache, with a ragged last tile: records match the oracle and
    every other slot keeps its sentinel."""
    B, T, off, L = 2, 77, 3, 90
    g = synth.rng(d + 7 * bits + m + 31 * H + (100 if rope else 0))
    X = g.standard_normal((B, T, H, d)).astype(np.float32)
    X[:, :, :, 5] *= np.float32(40.0)  # one outlier channel
    if dtype == "bf16":
        xb = synth.bf16_round_bits(X)
        X = synth.bf16_bits_to_f32(xb)
        x_dev = bf16_tensor(xb)
    else:
        x_dev = torch.from_numpy(X).cuda()
    ock, gck = codebooks(d, bits, m, False, 11)
    rope_g = tq.rope_table(1e4, d, L + 1) if rope else None
    rope_o = orope.rope_table(1e4, d, L + 1) if rope else None
    kp = tq.Packed(gck, B * H * L)
    kp.norm.fill_(-3.0)
    tq.encode_kv(gck, None, x_dev, None, kp, None, tok_offset=off, L_cap=L, rope=rope_g)
    torch.cuda.synchronize()
    got = kp.numpy()
    nrm = got[0].reshape(B * H, L)
    assert np.all(nrm[:, :off] == -3.0) and np.all(nrm[:, off + T:] == -3.0)
    pos = np.tile(off + np.arange(T), B * H)
    enc = codec.encode(ock, parity.oracle_rows(X), pos=pos if rope else None, rope=rope_o)
    def window(a):  # the records of tokens off .. off+T-1 of every (sequence, head)
        if a.size == 0:
            return a
        if a.ndim == 2:
            return a.reshape(B * H, L, -1)[:, off:off + T].reshape(B * H * T, -1)
        return a.reshape(B * H, L)[:, off:off + T].reshape(-1)
    parity.compare_encoded(ock, enc, tuple(window(a) for a in got), f"encoder d{d} b{bits} m{m} {dtype} rope={rope} H={H}")


def test_edge_cases_lengths_offsets_zero_vectors():
    """seq_len 0 (decode gives zeros, logits untouched), seq_len above L_cap
    (clamped), zero key vectors, and an append at a token offset that leaves
    the other cache slots untouched."""
    d, H, Hq, L = 128, 1, 4, 200
    ock, gck = codebooks(d, 3, 64, False, 0)
    ocv, gcv = codebooks(d, 3, 64, False, 1)
    g = synth.rng(9)
    K = g.standard_normal((3, L, H, d)).astype(np.float32)
    K[1, :17] = 0.0
    V = g.standard_normal((3, L, H, d)).astype(np.float32)
    Q = g.standard_normal((3, Hq, d)).astype(np.float32)
    kp, vp = tq.Packed(gck, 3 * H * L), tq.Packed(gcv, 3 * H * L)
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=L)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(K))
    ev = codec.encode(ocv, parity.oracle_rows(V))
    got = kp.numpy()
    parity.compare_encoded(ock, ek, got, "edge K")
    assert np.all(got[0][L:L + 17] == 0.0)
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), Q, torch.from_numpy(Q).cuda(), 3, Hq, H, L,
                            [0, 5000, 64], None, None, "edge")
    # append 40 tokens at slot 100 of a fresh cache: nothing else is written
    kp2 = tq.Packed(gck, 3 * H * L)
    kp2.norm.fill_(-7.0)
    tq.encode_kv(gck, None, torch.from_numpy(K[:, :40]).cuda(), None, kp2, None, tok_offset=100, L_cap=L)
    torch.cuda.synchronize()
    nrm = kp2.norm.cpu().numpy().reshape(3, L)
    assert np.all(nrm[:, :100] == -7.0) and np.all(nrm[:, 140:] == -7.0)
    ea = codec.encode(ock, parity.oracle_rows(K[:, :40]))
    sub = tuple(a.reshape(3, L, -1)[:, 100:140].reshape(3 * 40, -1) if a.ndim == 2 else
                a.reshape(3, L)[:, 100:140].reshape(-1) for a in kp2.numpy())
    parity.compare_encoded(ock, ea, sub, "append")


def test_runs_are_deterministic():
    d, H, Hq, L = 128, 2, 8, 3000
    ock, gck = codebooks(d, 3, 64, False, 0)
    gcv = codebooks(d, 3, 64, False, 1)[1]
    g = synth.rng(11)
    K = torch.from_numpy(g.standard_normal((1, L, H, d)).astype(np.float32)).cuda()
    V = torch.from_numpy(g.standard_normal((1, L, H, d)).astype(np.float32)).cuda()
    Q = torch.from_numpy(g.standard_normal((1, Hq, d)).astype(np.float32)).cuda()
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    res = []
    for _ in range(2):
        kp, vp = tq.Packed(gck, H * L), tq.Packed(gcv, H * L)
        tq.encode_kv(gck, gcv, K, V, kp, vp, L_cap=L)
        out = tq.attn_decode(gck, gcv, Q, kp, vp, H, L, sl)
        lg = tq.attn_logits(gck, Q, kp, H, L, sl)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in (kp.codes, kp.signs, kp.norm, vp.codes, out, lg)])
    for a, b in zip(*res):
        assert np.array_equal(a, b)


def test_api_rejects_bad_calls_on_gpu():
    d, H, Hq, L = 128, 1, 4, 64
    gck = codebooks(d, 3, 64, False, 0)[1]
    gcv = codebooks(d, 3, 64, False, 1)[1]
    kp = tq.Packed(gck, H * L)
    vp = tq.Packed(gcv, H * L)
    Q = torch.zeros((1, Hq, d), device="cuda")
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    with pytest.raises(tq.TQError) as ei:
        tq.attn_decode(gck, gcv, Q, kp, vp, H, L, sl, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == -1
    with pytest.raises(tq.TQError):
        tq.attn_logits(gck, Q, kp, 3, L, sl)                     # Hq not a multiple of h_kv
    small = tq.Packed(gck, 10)
    with pytest.raises(tq.TQError):
        tq.encode_kv(gck, None, torch.zeros((1, 64, 1, d), device="cuda"), None, small, None, L_cap=64)
    with pytest.raises(tq.TQError):
        tq.encode_kv(gck, None, torch.zeros((1, 64, 1, d), device="cuda"), None, kp, None, tok_offset=10, L_cap=64)
    # empty input is a no-op
    tq.encode_kv(gck, None, torch.zeros((1, 0, 1, d), device="cuda"), None, kp, None, L_cap=64)
    # the fused decode needs equal bits and m for keys and values, and no
    # dense rotation: refused before any launch with TQ_EUNSUPPORTED
    for cv_bad in (codebooks(d, 2, 64, False, 1)[1], codebooks(d, 3, 128, False, 1)[1],
                   codebooks(d, 3, 64, True, 1)[1]):
        with pytest.raises(tq.TQError) as ei:
            tq.attn_decode(gck, cv_bad, Q, kp, tq.Packed(cv_bad, H * L), H, L, sl)
        assert ei.value.code == -2 and "decode" in str(ei.value)
    gck_dense = codebooks(d, 3, 64, True, 0)[1]
    with pytest.raises(tq.TQError) as ei:
        tq.attn_decode(gck_dense, gcv, Q, tq.Packed(gck_dense, H * L), vp, H, L, sl)
    assert ei.value.code == -2


def test_prepared_launches_match_eager_calls():
    """A Launch (arguments marshalled once) enqueues the same work as the
    eager call, and can be replayed."""
    d, H, Hq, L = 128, 2, 8, 700
    gck = codebooks(d, 3, 64, False, 0)[1]
    gcv = codebooks(d, 3, 64, False, 1)[1]
    g = synth.rng(12)
    K = torch.from_numpy(g.standard_normal((1, L, H, d)).astype(np.float32)).cuda()
    V = torch.from_numpy(g.standard_normal((1, L, H, d)).astype(np.float32)).cuda()
    Q = torch.from_numpy(g.standard_normal((1, Hq, d)).astype(np.float32)).cuda()
    sl = torch.tensor([L - 3], dtype=torch.int32, device="cuda")
    kp, vp = tq.Packed(gck, H * L), tq.Packed(gcv, H * L)
    tq.encode_kv(gck, gcv, K, V, kp, vp, L_cap=L)
    lg = tq.attn_logits(gck, Q, kp, H, L, sl)
    out = tq.attn_decode(gck, gcv, Q, kp, vp, H, L, sl)
    kp2, vp2 = tq.Packed(gck, H * L), tq.Packed(gcv, H * L)
    enc = tq.encode_kv(gck, gcv, K, V, kp2, vp2, L_cap=L, prepare=True)
    run_l, lg2 = tq.attn_logits(gck, Q, kp2, H, L, sl, prepare=True)
    run_d, out2 = tq.attn_decode(gck, gcv, Q, kp2, vp2, H, L, sl, prepare=True)
    torch.cuda.synchronize()
    assert not kp2.norm.any()  # nothing ran yet
    for _ in range(2):
        enc()
        run_l()
        run_d()
        torch.cuda.synchronize()
        for a, b in [(kp.codes, kp2.codes), (kp.signs, kp2.signs), (kp.norm, kp2.norm), (vp.codes, vp2.codes),
                     (lg[..., :L - 3], lg2[..., :L - 3]), (out, out2)]:
            assert torch.equal(a, b)


def test_explicit_query_positions():
    """q_pos sets each sequence's query RoPE position (a decode step whose own
    key is already cached passes q_pos = seq_len - 1); positions below 0 and
    above L_cap are clamped like seq_len.  Logits, top-k and the fused decode
    all take it, for the contiguous and the paged forms."""
    d, H, Hq, L, B = 128, 2, 8, 257, 4
    ock, gck = codebooks(d, 3, 64, False, 0)
    ocv, gcv = codebooks(d, 3, 64, False, 1)
    g = synth.rng(21)
    K = g.standard_normal((B, L, H, d)).astype(np.float32)
    V = g.standard_normal((B, L, H, d)).astype(np.float32)
    Q = g.standard_normal((B, Hq, d)).astype(np.float32)
    rope_o = orope.rope_table(5e5, d, L + 1)
    rope_g = tq.rope_table(5e5, d, L + 1)
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=L, rope=rope_g)
    lens = np.array([L, 130, 1, L], np.int32)
    qpos = np.array([L - 1, 7, -5, 10 ** 6], np.int32)
    sl = torch.from_numpy(lens).cuda()
    qp_dev = torch.from_numpy(qpos).cuda()
    qd = torch.from_numpy(Q).cuda()
    lg = tq.attn_logits(gck, qd, kp, H, L, sl, rope=rope_g, q_pos=qp_dev).cpu().numpy()
    vals, idx = tq.attn_logits(gck, qd, kp, H, L, sl, rope=rope_g, q_pos=qp_dev, top_k=4)
    out = tq.attn_decode(gck, gcv, qd, kp, vp, H, L, sl, rope=rope_g, q_pos=qp_dev).cpu().numpy()
    lg_default = tq.attn_logits(gck, qd, kp, H, L, sl, rope=rope_g).cpu().numpy()
    torch.cuda.synchronize()
    vals, idx = vals.cpu().numpy(), idx.cpu().numpy()
    gk, gv = kp.numpy(), vp.numpy()
    ek = codec.Encoded(gk[0].astype(np.float64), gk[1].astype(np.float64), gk[2], gk[3])
    ev = codec.Encoded(gv[0].astype(np.float64), gv[1].astype(np.float64), gv[2], gv[3])
    G = Hq // H
    for b in range(B):
        p = int(min(max(qpos[b], 0), L))
        qp, s = estimator.prep_query(ock, Q[b], p, rope_o)
        qd0, sd0 = estimator.prep_query(ock, Q[b], int(lens[b]), rope_o)
        for h in range(H):
            gs = slice(h * G, (h + 1) * G)
            r = rows(ek, (b * H + h) * L, (b * H + h) * L + lens[b])
            rv = rows(ev, (b * H + h) * L, (b * H + h) * L + lens[b])
            ref = estimator.logits(ock, qp[gs], s[gs], r)
            parity.assert_close(lg[b, gs, :lens[b]], ref, f"q_pos logits b={b} h={h}")
            parity.check_topk(vals[b, gs], idx[b, gs], ref, 4, f"q_pos top-k b={b} h={h}")
            parity.assert_close(out[b, gs], estimator.attention(ock, ocv, qp[gs], s[gs], r, rv, int(lens[b]),
                                                                1 / math.sqrt(d), h), f"q_pos decode b={b} h={h}")
            parity.assert_close(lg_default[b, gs, :lens[b]], estimator.logits(ock, qd0[gs], sd0[gs], r),
                                f"default position logits b={b} h={h}")
