"""GPU parity for the TurboESM-style codebooks (one residual sign per
coordinate, a calibrated mean residual magnitude per KV head, separate key
and value tables, values optionally unrotated): the HIP path through the C
ABI against the CPU oracle on the same seeded inputs."""
import math

import numpy as np
import pytest

import synth
from oracle import calibration as ocal, codec, estimator, lloyd_max, rope as orope, rotation as orot

import parity
from test_gpu_parity import bf16_tensor, check_logits_and_decode, stored

torch = pytest.importorskip("torch")
tq = pytest.importorskip("kv_cache_vector_05_amd")

pytestmark = pytest.mark.gpu


def sign_codebooks(d, bits, rot, seed, levels=None, mu=None):
    """(oracle, GPU) sign-corrected codebooks with the same draws and tables."""
    sigma = synth.codec_draws(d, 0, False, seed)[0] if rot == "hadamard" else None
    o = codec.make_sign_codebook(d, bits, rot, sigma=sigma, levels=levels, mu=mu)
    g = tq.Codebook(d, bits, d, rot, sigma=sigma, correction="sign", levels=levels, mu=mu)
    return o, g


def test_default_mu_is_the_beta_law_mean_residual():
    """Without calibration a sign codebook's mu is E|Y - t[c(Y)]| under the
    rotated-coordinate law of its table."""
    for d, bits in [(64, 3), (128, 3), (128, 1), (64, 2)]:
        o, g = sign_codebooks(d, bits, "hadamard", 3)
        mu = g.mu()
        assert mu.shape == (1,)
        assert abs(float(mu[0]) - lloyd_max.mean_abs_error(o.t32, o.tau32, d)) <= 2e-7 * float(mu[0])
        assert float(mu[0]) == float(o.mu[0]) or abs(float(mu[0]) - float(o.mu[0])) <= 2e-7 * float(mu[0])


@pytest.mark.parametrize("d,bits,dtype,rope,rot,H", [
    (128, 3, "bf16", True, "hadamard", 4),   # RoPE rows staged per block, next-tile prefetch
    (128, 3, "bf16", True, "hadamard", 3),   # RoPE rows read per wave
    (128, 3, "f32", False, "hadamard", 2),
    (64, 3, "f32", True, "hadamard", 20),    # the ESM-2 head shape
    (64, 3, "bf16", False, "none", 5),       # values in their original coordinates
    (64, 3, "f32", True, "none", 4),         # unrotated with RoPE, staged
    (128, 3, "bf16", True, "none", 3),       # unrotated with RoPE, per wave
    (128, 2, "bf16", False, "none", 3),      # per-coordinate packing, unrotated
    (128, 1, "bf16", True, "hadamard", 1),
    (64, 2, "f32", False, "hadamard", 8),
])
def test_sign_encoder_paths(d, bits, dtype, rope, rot, H):
    """Encoder records (codes, per-coordinate sign bits, nu; no gamma plane)
    at a token offset inside a larger cache with a ragged last tile, plus a
    zero vector and negative-zero entries; every other slot keeps its
    sentinel."""
    B, T, off, L = 2, 77, 3, 90
    g = synth.rng(d + 7 * bits + 31 * H + (100 if rope else 0) + (500 if rot == "none" else 0))
    X = g.standard_normal((B, T, H, d)).astype(np.float32)
    X[:, :, :, 5] *= np.float32(40.0)   # one outlier channel
    X[0, 10] = 0.0                      # zero vectors (every head of one token)
    X[1, 20, :, :7] = -0.0              # negative zeros
    if dtype == "bf16":
        xb = synth.bf16_round_bits(X)
        X = synth.bf16_bits_to_f32(xb)
        x_dev = bf16_tensor(xb)
    else:
        x_dev = torch.from_numpy(X).cuda()
    ock, gck = sign_codebooks(d, bits, rot, 11)
    rope_g = tq.rope_table(1e4, d, L + 1) if rope else None
    rope_o = orope.rope_table(1e4, d, L + 1) if rope else None
    kp = tq.Packed(gck, B * H * L)
    assert kp.rnorm.numel() == 0
    kp.norm.fill_(-3.0)
    tq.encode_kv(gck, None, x_dev, None, kp, None, tok_offset=off, L_cap=L, rope=rope_g)
    torch.cuda.synchronize()
    got = kp.numpy()
    nrm = got[0].reshape(B * H, L)
    assert np.all(nrm[:, :off] == -3.0) and np.all(nrm[:, off + T:] == -3.0)
    pos = np.tile(off + np.arange(T), B * H)
    enc = codec.encode(ock, parity.oracle_rows(X), pos=pos if rope else None, rope=rope_o)

    def window(a):
        if a.size == 0:
            return a
        if a.ndim == 2:
            return a.reshape(B * H, L, -1)[:, off:off + T].reshape(B * H * T, -1)
        return a.reshape(B * H, L)[:, off:off + T].reshape(-1)
    parity.compare_encoded(ock, enc, tuple(window(a) for a in got),
                           f"sign encoder d{d} b{bits} {dtype} rope={rope} {rot} H={H}")


def _calibrated(d, bits, rot, seed, sample, rope_host=None, tok_offset=0):
    """(oracle, GPU) codebooks, each calibrated on the same batch by its own
    side: the oracle's calibration (oracle.calibration) and the library's
    (tq_calibrate), which agree to a unit or two in the last place."""
    sigma = synth.codec_draws(d, 0, False, seed)[0] if rot == "hadamard" else None
    lv, mu = tq.calibrate(d, bits, sample, rotation=rot, seed=0, sigma=sigma, tok_offset=tok_offset,
                          rope=rope_host)
    pi = orot.rht_matrix(sigma) if rot == "hadamard" else np.eye(d)
    olv, omu = ocal.calibrate(pi, bits, sample, tok_offset=tok_offset, rope=rope_host)
    o = codec.make_sign_codebook(d, bits, rot, sigma=sigma, levels=olv, mu=omu)
    g = tq.Codebook(d, bits, d, rot, sigma=sigma, correction="sign", levels=lv, mu=mu)
    return o, g


def test_llama8b_shaped_sign_logits_and_decode():
    """Calibrated key table (rotated, RoPE) and value table (original
    coordinates), one mu per KV head; GPU encode against the oracle, then
    logits and fused decode over the oracle's records (GQA 32/8, ragged
    context, two sequence lengths)."""
    B, Hq, H, L, d = 2, 32, 8, 1000, 128
    K, V = synth.llama_kv_inputs("llama8b", seed=0, batch=B, ctx=L)
    Q = synth.llama_q_inputs(seed=100, batch=B)
    kf, vf = synth.bf16_bits_to_f32(K), synth.bf16_bits_to_f32(V)
    rope_o = orope.rope_table(5e5, d, L + 1)
    rope_g = tq.rope_table(5e5, d, L + 1)
    ock, gck = _calibrated(d, 3, "hadamard", synth.K_SEED, kf[0, :256], rope_host=rope_o)
    ocv, gcv = _calibrated(d, 3, "none", synth.V_SEED, vf[0, :256])
    assert len(ock.mu) == H and len(ocv.mu) == H
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, bf16_tensor(K), bf16_tensor(V), kp, vp, L_cap=L, rope=rope_g)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(kf), pos=np.tile(np.arange(L), B * H), rope=rope_o)
    ev = codec.encode(ocv, parity.oracle_rows(vf))
    parity.compare_encoded(ock, ek, kp.numpy(), "sign llama8b K")
    parity.compare_encoded(ocv, ev, vp.numpy(), "sign llama8b V")
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), synth.bf16_bits_to_f32(Q), bf16_tensor(Q),
                            B, Hq, H, L, [1000, 777], rope_o, rope_g, "sign llama8b")


def test_esm_shaped_sign_records_and_decode():
    """ESM-2 head shape (d = 64, 20 heads, fp32, RoPE base 1e4): calibrated
    3-bit key and value tables, 36-byte records; logits and decode with one
    query per KV head."""
    S, T, H, d = 2, 300, 20, 64
    pk, pv = synth.esm_layer_tables(0)
    tok = synth.esm_tokens(0, S, T)
    K = pk[tok].reshape(S, T, H, d)
    V = pv[tok].reshape(S, T, H, d)
    rope_o = orope.rope_table(1e4, d, T + 1)
    rope_g = tq.rope_table(1e4, d, T + 1)
    ock, gck = _calibrated(d, 3, "hadamard", synth.K_SEED, K[0], rope_host=rope_o)
    ocv, gcv = _calibrated(d, 3, "none", synth.V_SEED, V[0])
    kp, vp = tq.Packed(gck, S * H * T), tq.Packed(gcv, S * H * T)
    assert 4 + 4 * kp.codes.shape[1] + 4 * kp.signs.shape[1] == 36
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=T, rope=rope_g)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(K), pos=np.tile(np.arange(T), S * H), rope=rope_o)
    ev = codec.encode(ocv, parity.oracle_rows(V))
    parity.compare_encoded(ock, ek, kp.numpy(), "sign esm K")
    parity.compare_encoded(ocv, ev, vp.numpy(), "sign esm V")
    Q = synth.rng(7).standard_normal((S, H, d)).astype(np.float32)
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), Q, torch.from_numpy(Q).cuda(), S, H, H, T,
                            [300, 123], rope_o, rope_g, "sign esm")


@pytest.mark.parametrize("kcorr,vcorr", [("sign", "qjl"), ("qjl", "sign")])
def test_mixed_key_and_value_corrections(kcorr, vcorr):
    """A sign-corrected key table with a QJL value table and the other way
    round (same d, bits and m), shared mu, GQA 6/2."""
    B, Hq, H, L, d, bits = 2, 6, 2, 333, 128, 2
    g = synth.rng(77)
    K = g.standard_normal((B, L, H, d)).astype(np.float32)
    V = g.standard_normal((B, L, H, d)).astype(np.float32)
    Q = g.standard_normal((B, Hq, d)).astype(np.float32)

    def make(corr, seed):
        if corr == "sign":
            return sign_codebooks(d, bits, "hadamard", seed, mu=[0.0123])
        sigma, rg, sk = synth.codec_draws(d, d, False, seed)
        return (codec.make_codebook(d, bits, d, False, sigma, rg, sk),
                tq.Codebook(d, bits, d, "hadamard", sigma=sigma, sketch=sk))
    ock, gck = make(kcorr, 5)
    ocv, gcv = make(vcorr, 6)
    kp, vp = tq.Packed(gck, B * H * L), tq.Packed(gcv, B * H * L)
    tq.encode_kv(gck, gcv, torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), kp, vp, L_cap=L)
    torch.cuda.synchronize()
    ek = codec.encode(ock, parity.oracle_rows(K))
    ev = codec.encode(ocv, parity.oracle_rows(V))
    parity.compare_encoded(ock, ek, kp.numpy(), f"mixed K {kcorr}")
    parity.compare_encoded(ocv, ev, vp.numpy(), f"mixed V {vcorr}")
    check_logits_and_decode(ock, gck, ocv, gcv, stored(ek), stored(ev), Q, torch.from_numpy(Q).cuda(), B, Hq, H, L,
                            [333, 45], None, None, f"mixed {kcorr}/{vcorr}")


def test_sign_calls_check_mu_count_and_top_k():
    """A per-head mu table must match h_kv; top-k over sign-corrected keys
    agrees with the oracle's scores."""
    d, H, Hq, L = 64, 4, 8, 500
    g = synth.rng(3)
    K = g.standard_normal((1, L, H, d)).astype(np.float32)
    Q = g.standard_normal((1, Hq, d)).astype(np.float32)
    mu = np.array([0.01, 0.02, 0.03, 0.04], np.float32)
    ock, gck = sign_codebooks(d, 3, "hadamard", 9, mu=mu)
    kp = tq.Packed(gck, H * L)
    tq.encode_kv(gck, None, torch.from_numpy(K).cuda(), None, kp, None, L_cap=L)
    sl = torch.tensor([L], dtype=torch.int32, device="cuda")
    qt = torch.from_numpy(Q).cuda()
    with pytest.raises(tq.TQError) as ei:
        tq.attn_logits(gck, qt[:, :4], tq.Packed(gck, 2 * L), 2, L, sl)   # 4 mu values, 2 KV heads
    assert ei.value.code == -1
    vals, idx = tq.attn_logits(gck, qt, kp, H, L, sl, top_k=10)
    torch.cuda.synchronize()
    enc = stored(codec.encode(ock, parity.oracle_rows(K)))
    qp, s = estimator.prep_query(ock, Q[0])
    G = Hq // H
    from test_gpu_parity import check_topk, rows
    for kh in range(H):
        ref = estimator.logits(ock, qp[kh * G:(kh + 1) * G], s[kh * G:(kh + 1) * G], rows(enc, kh * L, (kh + 1) * L), kh)
        ridx, rval = estimator.topk(ref, 10)
        check_topk(vals.cpu().numpy()[0, kh * G:(kh + 1) * G], idx.cpu().numpy()[0, kh * G:(kh + 1) * G], ref, rval)
