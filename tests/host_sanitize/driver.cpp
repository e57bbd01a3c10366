// Host-only driver for the sanitizer build of the library's host code: the
// table builders (Lloyd-Max, FibQuant, seeded draws, dense Haar rotation),
// the RoPE table, calibration and the argument checks that return before any
// HIP call.  Built with AddressSanitizer and UndefinedBehaviorSanitizer; any
// report, or any unexpected status, makes the process exit non-zero.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "tq.h"

static int g_fail = 0;

static void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (%s)\n", what, tq_last_error());
        g_fail = 1;
    }
}

static tq_spec spec(int d, int bits, int m, int rot, int corr = TQ_CORR_QJL, int block = 0) {
    tq_spec s{};
    s.d = d;
    s.bits = bits;
    s.m = m;
    s.rotation = rot;
    s.seed = 1234;
    s.correction = corr;
    s.block = block;
    return s;
}

static void tables(const tq_spec& s) {
    const int K = 1 << s.bits;
    const bool dense = s.rotation == TQ_ROT_DENSE || (s.rotation == TQ_ROT_AUTO && (s.d & (s.d - 1)) != 0);
    std::vector<float> lv((size_t)K * (s.block > 1 ? s.block : 1)), th(K > 1 ? K - 1 : 1);
    std::vector<float> rot(dense ? (size_t)s.d * s.d : (size_t)s.d), sk((size_t)(s.m ? s.m : 1) * s.d);
    const tq_status st = tq_codebook_tables(&s, nullptr, lv.data(), th.data(), rot.data(), sk.data());
    expect(st == TQ_OK, "tq_codebook_tables");
    if (st != TQ_OK) return;
    for (float x : lv) expect(std::isfinite(x), "finite levels");
    if (s.block <= 1)
        for (int j = 1; j < K; ++j) expect(lv[j] > lv[j - 1], "increasing levels");
    // the same call with every output skipped
    expect(tq_codebook_tables(&s, nullptr, nullptr, nullptr, nullptr, nullptr) == TQ_OK, "tables, no outputs");
}

int main() {
    // scalar Lloyd-Max tables over bit widths, Hadamard and dense rotations
    for (int bits = 1; bits <= 4; ++bits) {
        tables(spec(64, bits, 64, TQ_ROT_HADAMARD));
        tables(spec(128, bits, 128, TQ_ROT_HADAMARD));
        tables(spec(192, bits, 32, TQ_ROT_DENSE));
    }
    tables(spec(128, 3, 128, TQ_ROT_HADAMARD, TQ_CORR_SIGN));
    tables(spec(64, 3, 64, TQ_ROT_NONE, TQ_CORR_SIGN));
    // FibQuant vector codebooks: discs (k = 2) and spheres (k = 3)
    tables(spec(128, 4, 0, TQ_ROT_HADAMARD, TQ_CORR_QJL, 2));
    tables(spec(128, 6, 0, TQ_ROT_HADAMARD, TQ_CORR_QJL, 2));
    tables(spec(192, 5, 0, TQ_ROT_DENSE, TQ_CORR_QJL, 3));

    // explicit draws are read verbatim
    {
        const tq_spec s = spec(64, 2, 32, TQ_ROT_HADAMARD);
        std::vector<int8_t> sigma(64, 1);
        std::vector<float> sketch(32 * 64, 0.5f), rot(64), sk(32 * 64);
        tq_draws dr{sigma.data(), nullptr, sketch.data()};
        expect(tq_codebook_tables(&s, &dr, nullptr, nullptr, rot.data(), sk.data()) == TQ_OK, "given draws");
        expect(sk[0] == 0.5f && sk[32 * 64 - 1] == 0.5f, "sketch verbatim");
    }

    // RoPE table and plane sizes
    {
        std::vector<float> c(100 * 64), s(100 * 64);
        expect(tq_rope_table(5e5, 128, 100, c.data(), s.data()) == TQ_OK, "rope table");
        expect(c[0] == 1.0f && s[0] == 0.0f, "rope position 0");
        expect(tq_rope_table(5e5, 127, 100, c.data(), s.data()) != TQ_OK, "odd d rejected");
        const tq_spec sp = spec(128, 3, 64, TQ_ROT_HADAMARD);
        expect(tq_plane_words(&sp, 0) == 12, "code words at b = 3");
        expect(tq_plane_words(&sp, 1) == 2, "sign words at m = 64");
    }

    // calibration of a sign-corrected codebook on a host batch, with RoPE
    {
        const int d = 64, h = 2, n = 300;
        const tq_spec s = spec(d, 3, d, TQ_ROT_HADAMARD, TQ_CORR_SIGN);
        std::vector<float> x((size_t)n * h * d);
        uint64_t z = 7;
        for (float& v : x) {
            z = z * 6364136223846793005ull + 1442695040888963407ull;
            v = (float)((int64_t)(z >> 40) - (1ll << 23)) / (float)(1 << 23);
        }
        std::vector<float> c((size_t)(n + 5) * d / 2), sn((size_t)(n + 5) * d / 2), lv(8), mu(h);
        expect(tq_rope_table(1e4, d, n + 5, c.data(), sn.data()) == TQ_OK, "rope table for calibration");
        expect(tq_calibrate(&s, nullptr, x.data(), n, h, 5, c.data(), sn.data(), n + 5, lv.data(), mu.data()) ==
                   TQ_OK,
               "calibrate");
        expect(mu[0] > 0.0f && mu[1] > 0.0f, "positive mu");
        // RoPE rows that do not cover the last position
        expect(tq_calibrate(&s, nullptr, x.data(), n, h, 5, c.data(), sn.data(), n, lv.data(), mu.data()) != TQ_OK,
               "short RoPE table rejected");
    }

    // bad specs and null arguments are rejected before any device call
    {
        const tq_spec bad[] = {spec(0, 3, 64, TQ_ROT_HADAMARD), spec(128, 9, 64, TQ_ROT_HADAMARD),
                               spec(128, 3, 48, TQ_ROT_HADAMARD), spec(100, 3, 64, TQ_ROT_HADAMARD),
                               spec(128, 3, 64, TQ_ROT_NONE)};
        for (const tq_spec& s : bad) {
            tq_codebook* cb = reinterpret_cast<tq_codebook*>(1);
            expect(tq_codebook_init(&s, nullptr, nullptr, &cb) != TQ_OK && cb == nullptr, "bad spec rejected");
            expect(tq_codebook_tables(&s, nullptr, nullptr, nullptr, nullptr, nullptr) != TQ_OK, "bad tables");
        }
        expect(tq_codebook_init(nullptr, nullptr, nullptr, nullptr) == TQ_EINVAL, "null spec");
        tq_packed kp{};
        expect(tq_encode_kv(nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 1, nullptr, nullptr, 0, 1, nullptr,
                            nullptr, 0, &kp, nullptr, nullptr, 0, nullptr) == TQ_EINVAL,
               "null codebooks rejected");
        expect(tq_attn_logits(nullptr, nullptr, 0, &kp, 1, 8, 2, 64, nullptr, nullptr, nullptr, nullptr, 0, 0,
                              nullptr, nullptr, nullptr, 0, nullptr) == TQ_EINVAL,
               "null logits arguments rejected");
    }
    std::printf(g_fail ? "host sanitizer driver: FAILED\n" : "host sanitizer driver: ok\n");
    return g_fail;
}
