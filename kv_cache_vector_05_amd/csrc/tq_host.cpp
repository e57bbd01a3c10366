// Host side of libtq: argument validation, codebook table construction
// (Lloyd-Max solver, seeded draws, Haar rotation, RoPE table) and the C ABI
// entry points, which validate and then enqueue the HIP kernels.
//
// Table construction follows the FibQuant summary, sections 1 and 2.1
// (normalise, shared Haar rotation, scalar Lloyd-Max table for the
// spherical-Beta marginal; one offline table for all inputs) and the
// iaemfoco post, "TurboQuant: Uma Nova Abordagem" (randomized Hadamard
// rotation; Johnson-Lindenstrauss sketch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace tq {

static thread_local std::string g_last_error;

tq_status fail(tq_status code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

tq_status hip_fail(hipError_t e, const char* what) {
    g_last_error = std::string(what) + ": " + hipGetErrorString(e);
    return TQ_EHIP;
}

static bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

tq_status check_spec(const tq_spec& s, bool* dense) {
    if (s.block < 0 || s.block > 3) return fail(TQ_EINVAL, "block must be 0..3");
    if (s.block >= 2) {
        // a FibQuant vector codebook: N = 2^bits codewords per block of `block` coordinates
        if (s.bits < 1 || s.bits > 8) return fail(TQ_EINVAL, "a vector codebook has 1..8 index bits per block");
        if (s.d < 3 || s.d > 4096 || s.d % s.block) return fail(TQ_EINVAL, "d must be a multiple of block");
        if (s.m != 0 || s.correction != TQ_CORR_QJL)
            return fail(TQ_EINVAL, "vector codebooks take no residual correction (m = 0)");
        bool dn;
        if (s.rotation == TQ_ROT_AUTO) dn = !is_pow2(s.d);
        else if (s.rotation == TQ_ROT_HADAMARD) dn = false;
        else if (s.rotation == TQ_ROT_DENSE) dn = true;
        else return fail(TQ_EINVAL, "vector codebooks take the Hadamard or the dense rotation");
        if (!dn && !is_pow2(s.d)) return fail(TQ_EINVAL, "Hadamard rotation needs a power-of-two d");
        if (dn && s.d % 64) return fail(TQ_EUNSUPPORTED, "dense rotations need d a multiple of 64");
        if (dense) *dense = dn;
        return TQ_OK;
    }
    if (s.bits < 1 || s.bits > 4) return fail(TQ_EINVAL, "bits must be 1..4");
    if (s.d < 3 || s.d > 4096) return fail(TQ_EINVAL, "d must be 3..4096");
    if ((s.bits * s.d) % 32) return fail(TQ_EINVAL, "bits*d must be a multiple of 32");
    if (s.m < 0 || s.m > 4096 || (s.m % 32)) return fail(TQ_EINVAL, "m must be 0 or a multiple of 32 up to 4096");
    if (s.correction != TQ_CORR_QJL && s.correction != TQ_CORR_SIGN) return fail(TQ_EINVAL, "unknown correction");
    bool dn;
    if (s.rotation == TQ_ROT_AUTO) dn = !is_pow2(s.d);
    else if (s.rotation == TQ_ROT_HADAMARD || s.rotation == TQ_ROT_NONE) dn = false;
    else if (s.rotation == TQ_ROT_DENSE) dn = true;
    else return fail(TQ_EINVAL, "unknown rotation");
    if (s.rotation == TQ_ROT_NONE && s.correction != TQ_CORR_SIGN)
        return fail(TQ_EUNSUPPORTED, "rotation none is served with the sign correction only");
    if (s.correction == TQ_CORR_SIGN) {
        if (s.m != s.d) return fail(TQ_EINVAL, "the sign correction keeps one bit per coordinate: m must equal d");
        if (dn || (s.d != 64 && s.d != 128))
            return fail(TQ_EUNSUPPORTED, "the sign correction has kernels for d = 64 and 128, Hadamard or no rotation");
        if (s.bits > 3) return fail(TQ_EUNSUPPORTED, "the sign correction has kernels for bits 1..3");
    }
    if (!dn) {
        if (!is_pow2(s.d)) return fail(TQ_EINVAL, "Hadamard rotation needs a power-of-two d");
        if (s.d != 64 && s.d != 128) return fail(TQ_EUNSUPPORTED, "Hadamard kernels exist for d = 64 and 128");
        if (s.m != 0 && s.m != s.d / 2 && s.m != s.d)
            return fail(TQ_EUNSUPPORTED, "Hadamard kernels exist for m = 0, d/2 and d");
    } else {
        if (s.d % 64) return fail(TQ_EUNSUPPORTED, "dense kernels need d a multiple of 64");
    }
    if (dense) *dense = dn;
    return TQ_OK;
}

// ------------------------------------------------------------------------
// Lloyd-Max table for one coordinate of a uniform point on S^{d-1}.
// Density f(y) proportional to (1 - y^2)^((d-3)/2).  With y = sin(theta),
// f(y) dy is proportional to cos(theta)^(d-2) dtheta, smooth on
// [-pi/2, pi/2] for every d >= 3, so composite Gauss-Legendre quadrature in
// theta converges fast even where the y-density has an endpoint
// singularity (small d).  The normalising constant cancels in the level
// (a ratio of two integrals), so it is never formed.
// ------------------------------------------------------------------------
namespace {

struct GaussLegendre {
    std::vector<double> x, w;  // nodes and weights on [-1, 1]
    explicit GaussLegendre(int n) : x(n), w(n) {
        // Newton's method on P_n from the usual cosine starting points
        auto legendre = [n](double z, double* dp) {
            double p0 = 1.0, p1 = 0.0;
            for (int k = 1; k <= n; ++k) {
                const double p2 = p1;
                p1 = p0;
                p0 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p2) / k;
            }
            *dp = n * (z * p0 - p1) / (z * z - 1.0);
            return p0;
        };
        for (int i = 0; i < n; ++i) {
            double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
            double dp = 0.0;
            for (int it = 0; it < 100; ++it) {
                const double pz = legendre(z, &dp);
                const double dz = pz / dp;
                z -= dz;
                if (std::fabs(dz) < 1e-16) break;
            }
            legendre(z, &dp);
            x[i] = z;
            w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
        }
    }
};

// (mass, first moment) of cos^(d-2) over [ta, tb] in theta (unnormalised).
void cell_integrals(const GaussLegendre& gl, int d, double ta, double tb, double* mass,
                    double* mom) {
    const double width = 1.0 / std::sqrt((double)d);
    // beyond ~60 widths the integrand is below exp(-1800): skip it
    const double lim = std::min(M_PI / 2, 60.0 * width);
    ta = std::max(ta, -lim);
    tb = std::min(tb, lim);
    *mass = 0.0;
    *mom = 0.0;
    if (tb <= ta) return;
    const double h = std::min(0.05, 0.25 * width);
    const int panels = std::max(1, (int)std::ceil((tb - ta) / h));
    const double hp = (tb - ta) / panels;
    for (int p = 0; p < panels; ++p) {
        const double a = ta + p * hp, c = a + 0.5 * hp;
        for (size_t k = 0; k < gl.x.size(); ++k) {
            const double th = c + 0.5 * hp * gl.x[k];
            const double ct = std::cos(th);
            const double f = ct > 0 ? std::exp((d - 2) * std::log(ct)) : 0.0;
            const double wk = 0.5 * hp * gl.w[k];
            *mass += wk * f;
            *mom += wk * f * std::sin(th);
        }
    }
}

}  // namespace

void lloyd_max_table(int d, int bits, std::vector<double>* levels, std::vector<double>* thr) {
    static const GaussLegendre gl(24);
    const int K = 1 << bits, half = K / 2;
    std::vector<double> t(K), tau(K - 1), tn(K);
    // start: K evenly spread levels inside +-3 standard deviations
    const double sd = 1.0 / std::sqrt((double)d);
    for (int j = 0; j < K; ++j) t[j] = std::min(0.9, 3.0 * sd) * (2.0 * (j + 0.5) / K - 1.0);
    double prev = INFINITY;
    for (int it = 0; it < 2000000; ++it) {
        for (int j = 0; j + 1 < K; ++j) tau[j] = 0.5 * (t[j] + t[j + 1]);
        // upper-half cells [tau_{K/2-1} (= 0), ...), mirrored below (f is even)
        for (int j = half; j < K; ++j) {
            const double lo = tau[j - 1];
            const double hi = (j + 1 < K) ? tau[j] : 1.0;
            double mass, mom;
            cell_integrals(gl, d, std::asin(std::max(-1.0, std::min(1.0, lo))),
                           std::asin(std::max(-1.0, std::min(1.0, hi))), &mass, &mom);
            tn[j] = mom / mass;
            tn[K - 1 - j] = -tn[j];
        }
        double step = 0.0, big = 0.0;
        for (int j = 0; j < K; ++j) {
            step = std::max(step, std::fabs(tn[j] - t[j]));
            big = std::max(big, std::fabs(tn[j]));
        }
        step /= big;
        t = tn;
        if (step <= 1e-14 || (step <= 1e-12 && step >= prev)) break;
        prev = step;
    }
    for (int j = 0; j + 1 < K; ++j) tau[j] = 0.5 * (t[j] + t[j + 1]);
    *levels = t;
    *thr = tau;
}

// E|Y - t[c(Y)]| under the same density (the sign correction's mean residual
// magnitude when no calibration is given): per cell, the integrals of
// (t - y) f below the level and (y - t) f above it, from the cell's mass and
// first moment in theta, over the total mass.
double beta_mean_abs_error(int d, const std::vector<float>& levels, const std::vector<float>& thr) {
    static const GaussLegendre gl(24);
    const int K = (int)levels.size();
    auto th = [](double y) { return std::asin(std::max(-1.0, std::min(1.0, y))); };
    double mass = 0.0, acc = 0.0;
    for (int j = 0; j < K; ++j) {
        const double lo = j == 0 ? -1.0 : (double)thr[j - 1];
        const double hi = j + 1 < K ? (double)thr[j] : 1.0;
        const double t = levels[j];
        const double tm = std::min(std::max(t, lo), hi);
        double m1, s1, m2, s2;
        cell_integrals(gl, d, th(lo), th(tm), &m1, &s1);
        cell_integrals(gl, d, th(tm), th(hi), &m2, &s2);
        acc += (t * m1 - s1) + (s2 - t * m2);
        mass += m1 + m2;
    }
    return acc / mass;
}

// ------------------------------------------------------------------------
// FibQuant vector codebooks (FibQuant summary, section 2.2).  A block of k
// coordinates of a uniform point on S^{d-1} has |x|^2 ~ Beta(k/2, (d-k)/2).
// Initial codewords: Bennett-Gersho radii (point density proportional to
// f^(k/(k+2)), whose |x|^2 is Beta(k/2, a + 1), a = k (d-k-2) / (2 (k+2)),
// taken at the quantiles (n + 1/2) / N) with golden-angle directions (k = 2)
// or a Fibonacci sphere (k = 3, radius quantile frac((n + 1/2) / phi)).
// Refinement: Lloyd-Max on an equal-mass deterministic sample (64 radial
// quantiles times 256 directions; for k = 3 a Fibonacci sphere and its
// antipodes), several restarts rotated by 2 pi r / (R N).
// ------------------------------------------------------------------------
namespace {

// continued fraction of the regularised incomplete beta function (DLMF
// 8.17.22), evaluated by the modified Lentz method
double ibeta_cf(double a, double b, double x) {
    const double tiny = 1e-300;
    double c = 1.0, dd = 1.0 - (a + b) * x / (a + 1.0);
    if (std::fabs(dd) < tiny) dd = tiny;
    dd = 1.0 / dd;
    double f = dd;
    for (int m = 1; m < 10000; ++m) {
        // even step: m (b - m) x / ((a + 2m - 1)(a + 2m))
        double num = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
        dd = 1.0 + num * dd;
        if (std::fabs(dd) < tiny) dd = tiny;
        c = 1.0 + num / c;
        if (std::fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd;
        f *= dd * c;
        // odd step: -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1))
        num = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
        dd = 1.0 + num * dd;
        if (std::fabs(dd) < tiny) dd = tiny;
        c = 1.0 + num / c;
        if (std::fabs(c) < tiny) c = tiny;
        dd = 1.0 / dd;
        const double step = dd * c;
        f *= step;
        if (std::fabs(step - 1.0) < 1e-16) break;
    }
    return f;
}

// I_x(a, b)
double ibeta(double a, double b, double x) {
    if (x <= 0.0) return 0.0;
    if (x >= 1.0) return 1.0;
    const double lfront = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) + a * std::log(x) + b * std::log1p(-x);
    if (x < (a + 1.0) / (a + b + 2.0)) return std::exp(lfront) * ibeta_cf(a, b, x) / a;
    return 1.0 - std::exp(lfront) * ibeta_cf(b, a, 1.0 - x) / b;
}

// the p-quantile of Beta(a, b), by bisection
double ibeta_inv(double a, double b, double p) {
    double lo = 0.0, hi = 1.0;
    for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (ibeta(a, b, mid) < p) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

const double kPhi = 1.6180339887498949;  // (1 + sqrt 5) / 2

void fibonacci_sphere(int n, std::vector<double>* out) {
    const double ga = 2.0 * M_PI / (kPhi * kPhi);
    out->resize((size_t)n * 3);
    for (int i = 0; i < n; ++i) {
        const double z = 1.0 - 2.0 * (i + 0.5) / n;
        const double rho = std::sqrt(std::max(0.0, 1.0 - z * z));
        const double th = i * ga;
        (*out)[3 * i] = rho * std::cos(th);
        (*out)[3 * i + 1] = rho * std::sin(th);
        (*out)[3 * i + 2] = z;
    }
}

// Lloyd-Max on equal-weight points (row-major [P][k]) from code [N][k];
// returns the mean squared error
double vq_lloyd(const std::vector<double>& pts, int k, std::vector<double>* code, int N) {
    const size_t P = pts.size() / k;
    std::vector<int> assign(P, -1), next(P);
    std::vector<double> sum((size_t)N * k);
    std::vector<long> cnt(N);
    for (int it = 0; it < 5000; ++it) {
        for (size_t p = 0; p < P; ++p) {
            double best = 0.0;
            int bi = 0;
            for (int n = 0; n < N; ++n) {
                double dist = 0.0;
                for (int i = 0; i < k; ++i) {
                    const double df = pts[p * k + i] - (*code)[(size_t)n * k + i];
                    dist = dist + df * df;
                }
                if (n == 0 || dist < best) {
                    best = dist;
                    bi = n;
                }
            }
            next[p] = bi;
        }
        if (next == assign) break;
        assign = next;
        std::fill(sum.begin(), sum.end(), 0.0);
        std::fill(cnt.begin(), cnt.end(), 0);
        for (size_t p = 0; p < P; ++p) {
            ++cnt[assign[p]];
            for (int i = 0; i < k; ++i) sum[(size_t)assign[p] * k + i] += pts[p * k + i];
        }
        for (int n = 0; n < N; ++n)
            if (cnt[n])
                for (int i = 0; i < k; ++i) (*code)[(size_t)n * k + i] = sum[(size_t)n * k + i] / (double)cnt[n];
    }
    double mse = 0.0;
    for (size_t p = 0; p < P; ++p) {
        double dist = 0.0;
        for (int i = 0; i < k; ++i) {
            const double df = pts[p * k + i] - (*code)[(size_t)assign[p] * k + i];
            dist += df * df;
        }
        mse += dist;
    }
    return mse / (double)P;
}

}  // namespace

void fibquant_codebook(int d, int k, int N, std::vector<double>* out) {
    const int n_radii = 64, n_dirs = 256, restarts = 4;
    // equal-mass sample of the block law
    std::vector<double> r(n_radii), dirs;
    for (int i = 0; i < n_radii; ++i) r[i] = std::sqrt(ibeta_inv(k / 2.0, (d - k) / 2.0, (i + 0.5) / n_radii));
    int nd;
    if (k == 2) {
        nd = n_dirs;
        dirs.resize((size_t)nd * 2);
        for (int j = 0; j < nd; ++j) {
            const double th = 2.0 * M_PI * (j + 0.5) / nd;
            dirs[2 * j] = std::cos(th);
            dirs[2 * j + 1] = std::sin(th);
        }
    } else {
        std::vector<double> f;
        fibonacci_sphere(n_dirs, &f);
        nd = 2 * n_dirs;
        dirs.resize((size_t)nd * 3);
        for (size_t i = 0; i < f.size(); ++i) {
            dirs[i] = f[i];
            dirs[f.size() + i] = -f[i];
        }
    }
    std::vector<double> pts((size_t)n_radii * nd * k);
    for (int i = 0; i < n_radii; ++i)
        for (int j = 0; j < nd; ++j)
            for (int c = 0; c < k; ++c) pts[((size_t)i * nd + j) * k + c] = r[i] * dirs[(size_t)j * k + c];
    // initial codebook
    const double a = k * (d - k - 2) / (2.0 * (k + 2));
    std::vector<double> init((size_t)N * k);
    if (k == 2) {
        const double ga = 2.0 * M_PI / (kPhi * kPhi);
        for (int n = 0; n < N; ++n) {
            const double rn = std::sqrt(ibeta_inv(1.0, a + 1.0, (n + 0.5) / N));
            const double th = n * ga;
            init[2 * n] = rn * std::cos(th);
            init[2 * n + 1] = rn * std::sin(th);
        }
    } else {
        std::vector<double> f;
        fibonacci_sphere(N, &f);
        for (int n = 0; n < N; ++n) {
            const double lv = std::fmod((n + 0.5) / kPhi, 1.0);
            const double rn = std::sqrt(ibeta_inv(1.5, a + 1.0, lv));
            for (int c = 0; c < 3; ++c) init[3 * n + c] = rn * f[3 * n + c];
        }
    }
    double best_mse = 0.0;
    for (int rs = 0; rs < restarts; ++rs) {
        const double ang = 2.0 * M_PI * rs / (restarts * (double)N);
        const double ca = std::cos(ang), sa = std::sin(ang);
        std::vector<double> c = init;
        for (int n = 0; n < N; ++n) {
            c[(size_t)n * k] = ca * init[(size_t)n * k] - sa * init[(size_t)n * k + 1];
            c[(size_t)n * k + 1] = sa * init[(size_t)n * k] + ca * init[(size_t)n * k + 1];
        }
        const double mse = vq_lloyd(pts, k, &c, N);
        if (rs == 0 || mse < best_mse * (1.0 - 1e-9)) {
            best_mse = mse;
            *out = c;
        }
    }
}

// ------------------------------------------------------------------------
// Seeded draws: SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) streams,
// Box-Muller (1958) Gaussians.  Purpose p (1 signs, 2 rotation, 3 sketch)
// starts from output p of a SplitMix64 seeded with the codebook seed.
// ------------------------------------------------------------------------
namespace {
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
inline uint64_t stream_start(uint64_t seed, int purpose) {
    return mix64(seed + (uint64_t)purpose * kGamma);
}
}  // namespace

void splitmix_gaussians(uint64_t seed, int purpose, size_t n, double* out) {
    uint64_t s = stream_start(seed, purpose);
    for (size_t i = 0; i < n; i += 2) {
        s += kGamma;
        const double u1 = (double)(mix64(s) >> 11) * 0x1.0p-53;
        s += kGamma;
        const double u2 = (double)(mix64(s) >> 11) * 0x1.0p-53;
        const double r = std::sqrt(-2.0 * std::log(1.0 - u1));
        const double a = 2.0 * M_PI * u2;
        out[i] = r * std::cos(a);
        if (i + 1 < n) out[i + 1] = r * std::sin(a);
    }
}

void splitmix_signs(uint64_t seed, size_t n, int8_t* out) {
    uint64_t s = stream_start(seed, 1);
    for (size_t i = 0; i < n; ++i) {
        s += kGamma;
        out[i] = (mix64(s) >> 63) ? -1 : 1;
    }
}

// ------------------------------------------------------------------------
// Haar rotation: Householder QR of a d x d Gaussian matrix G = Q R, with the
// columns of Q multiplied by sign(R_jj) so that diag(R) > 0.  Works on a
// column-major copy; returns Q row-major.
// ------------------------------------------------------------------------
void haar_from_gaussians(int d, const double* g, std::vector<double>* qout) {
    const size_t n = (size_t)d;
    std::vector<double> a(n * n);  // column-major: a[j*n + i] = G[i][j]
    for (size_t i = 0; i < n; ++i)
        for (size_t j = 0; j < n; ++j) a[j * n + i] = g[i * n + j];
    std::vector<double> vs(n * n, 0.0);  // Householder vectors, column k in vs[k*n ...]
    std::vector<double> rdiag(n);
    for (size_t k = 0; k < n; ++k) {
        double* col = &a[k * n];
        double norm2 = 0.0;
        for (size_t i = k; i < n; ++i) norm2 += col[i] * col[i];
        const double nrm = std::sqrt(norm2);
        const double alpha = col[k] >= 0 ? -nrm : nrm;
        double* v = &vs[k * n];
        for (size_t i = k; i < n; ++i) v[i] = col[i];
        v[k] -= alpha;
        double vn2 = 0.0;
        for (size_t i = k; i < n; ++i) vn2 += v[i] * v[i];
        rdiag[k] = alpha;
        if (vn2 == 0.0) continue;
        const double inv = 1.0 / std::sqrt(vn2);
        for (size_t i = k; i < n; ++i) v[i] *= inv;
        for (size_t j = k; j < n; ++j) {
            double* cj = &a[j * n];
            double dot = 0.0;
            for (size_t i = k; i < n; ++i) dot += v[i] * cj[i];
            dot *= 2.0;
            for (size_t i = k; i < n; ++i) cj[i] -= dot * v[i];
        }
    }
    // Q = H_0 H_1 ... H_{n-1} I, accumulated from the right (column-major).
    std::vector<double> q(n * n, 0.0);
    for (size_t i = 0; i < n; ++i) q[i * n + i] = 1.0;
    for (size_t kk = n; kk-- > 0;) {
        const double* v = &vs[kk * n];
        for (size_t j = kk; j < n; ++j) {
            double* cj = &q[j * n];
            double dot = 0.0;
            for (size_t i = kk; i < n; ++i) dot += v[i] * cj[i];
            dot *= 2.0;
            if (dot != 0.0)
                for (size_t i = kk; i < n; ++i) cj[i] -= dot * v[i];
        }
    }
    qout->assign(n * n, 0.0);
    for (size_t i = 0; i < n; ++i)
        for (size_t j = 0; j < n; ++j) {
            const double sgn = rdiag[j] < 0 ? -1.0 : 1.0;  // R_jj = rdiag[j]
            (*qout)[i * n + j] = q[j * n + i] * sgn;
        }
}

// Levels as 24-bit fixed-point integers T_k ~= t_k * 2^shift split into three
// balanced base-256 digits, each in [-128, 127]: T = e0*2^16 + e1*2^8 + e2.
// The shift puts max|T| just under 127.5 * 2^16 so the top digit fits.
// Digit b of level c sits in byte c % 4 of word 8 (c / 8) + 2 b + (c % 8) / 4
// (levels 8-15 of a 4-bit table in the upper half).
void level_digits(const std::vector<float>& levels, uint32_t words[16], int* shift) {
    double mx = 0.0;
    for (float v : levels) mx = std::max(mx, (double)std::fabs(v));
    int e = 0;
    std::frexp(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    int sh = 23 - e;
    if (std::ldexp(mx, sh) > 127.0 * 65536.0) --sh;
    *shift = sh;
    for (int w = 0; w < 16; ++w) words[w] = 0u;
    for (size_t c = 0; c < levels.size() && c < 16; ++c) {
        long long T = std::llround(std::ldexp((double)levels[c], sh));
        int dig[3];
        for (int k = 2; k >= 1; --k) {
            const long long r = ((T + 128) % 256 + 256) % 256 - 128;
            dig[k] = (int)r;
            T = (T - r) / 256;
        }
        dig[0] = (int)T;
        for (int b = 0; b < 3; ++b) {
            const uint32_t byte = (uint32_t)(uint8_t)(int8_t)dig[b];
            words[8 * (c >> 3) + 2 * b + ((c & 7) >> 2)] |= byte << (8 * (c & 3));
        }
    }
}

// IEEE binary16 conversions (round to nearest even), for the MFMA tables.
uint16_t f32_to_f16(float f) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const int32_t exp = (int32_t)((x >> 23) & 0xFF) - 127 + 15;
    uint32_t man = x & 0x7FFFFFu;
    if (((x >> 23) & 0xFF) == 0xFF) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    if (exp >= 31) return (uint16_t)(sign | 0x7C00u);
    if (exp <= 0) {
        if (exp < -10) return (uint16_t)sign;
        man |= 0x800000u;
        const int shift = 14 - exp;
        uint32_t h = man >> shift;
        const uint32_t rem = man & ((1u << shift) - 1u), halfway = 1u << (shift - 1);
        if (rem > halfway || (rem == halfway && (h & 1u))) ++h;
        return (uint16_t)(sign | h);
    }
    uint32_t h = ((uint32_t)exp << 10) | (man >> 13);
    const uint32_t rem = man & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
}

float f16_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const uint32_t exp = (h >> 10) & 0x1F, man = h & 0x3FFu;
    float v;
    if (exp == 0) v = std::ldexp((float)man, -24);
    else if (exp == 31) v = man ? NAN : INFINITY;
    else v = std::ldexp((float)(man | 0x400u), (int)exp - 25);
    uint32_t bits;
    std::memcpy(&bits, &v, 4);
    bits |= sign;
    std::memcpy(&v, &bits, 4);
    return v;
}

// Candidate grid of a two-coordinate codebook for the encoder's nearest-codeword
// search (layout in tq_internal.h).  Cells cover |y_i| < 5 / sqrt(d): a
// rotated unit vector's coordinate has standard deviation 1 / sqrt(d), so
// blocks outside are rare (they fall back to the full search).  Codeword n
// is a candidate for the cell of centre m when
//   |m - c_n| <= min_k |m - c_k| + 2 rho + eps,
// rho the cell's half-diagonal with 2e-4 of slack for the float32 cell
// assignment, eps = 3e-4.  For any point p of the cell a codeword outside the
// list is then farther than the best candidate by more than eps, so its
// squared distance exceeds the best one's by more than eps^2 - far above the
// float32 rounding of the scores - and the first maximum over the candidates
// (ascending) is the first maximum over the whole codebook.
static void vq_candidate_grid(const std::vector<float>& code, int N, int d, std::vector<uint32_t>* grid,
                              float* inv_cell) {
    const double R = 5.0 / std::sqrt((double)d);
    *inv_cell = (float)(kVqGrid / (2.0 * R));
    const double cell = 1.0 / (double)*inv_cell;
    const double rho = cell * std::sqrt(0.5) * (1.0 + 2e-4), eps = 3e-4;
    grid->assign((size_t)kVqGrid * kVqGrid, 0u);
    std::vector<double> dist(N);
    for (int iy = 0; iy < kVqGrid; ++iy)
        for (int ix = 0; ix < kVqGrid; ++ix) {
            const double mx = (ix - kVqGrid / 2 + 0.5) * cell, my = (iy - kVqGrid / 2 + 0.5) * cell;
            double best = INFINITY;
            for (int n = 0; n < N; ++n) {
                const double dx = mx - code[2 * n], dy = my - code[2 * n + 1];
                dist[n] = std::sqrt(dx * dx + dy * dy);
                best = std::min(best, dist[n]);
            }
            uint32_t w = 0;
            int cnt = 0, last = 0;
            for (int n = 0; n < N && cnt <= 4; ++n)
                if (dist[n] <= best + 2.0 * rho + eps) {
                    if (cnt < 4) w |= (uint32_t)n << (8 * cnt);
                    last = n;
                    ++cnt;
                }
            if (cnt > 4) {
                w = 0xFFu;
            } else {
                for (int q = cnt; q < 4; ++q) w |= (uint32_t)last << (8 * q);
            }
            (*grid)[(size_t)iy * kVqGrid + ix] = w;
        }
}

// Builds every host table of a codebook.
static tq_status build_tables(const tq_spec& s, const tq_draws* dr, bool dense,
                              std::vector<float>* levels, std::vector<float>* thr,
                              std::vector<float>* rot, std::vector<float>* sk) {
    if (s.block >= 2) {
        // vector codebook: levels holds the N x block codewords
        std::vector<double> code;
        fibquant_codebook(s.d, s.block, 1 << s.bits, &code);
        levels->assign(code.begin(), code.end());
        thr->clear();
    } else {
        std::vector<double> t, tau;
        lloyd_max_table(s.d, s.bits, &t, &tau);
        levels->assign(t.begin(), t.end());
        thr->assign(tau.begin(), tau.end());
    }
    const size_t d = (size_t)s.d;
    if (dense) {
        std::vector<double> g;
        const double* gp = dr ? dr->rot_gauss : nullptr;
        if (!gp) {
            g.resize(d * d);
            splitmix_gaussians(s.seed, 2, d * d, g.data());
            gp = g.data();
        }
        std::vector<double> q;
        haar_from_gaussians(s.d, gp, &q);
        rot->assign(q.begin(), q.end());
    } else if (s.rotation == TQ_ROT_NONE) {
        rot->assign(d, 1.0f);  // no rotation: the kernels read no sigma
    } else {
        std::vector<int8_t> sg(d);
        if (dr && dr->sigma) {
            for (size_t i = 0; i < d; ++i) {
                if (dr->sigma[i] != 1 && dr->sigma[i] != -1) return fail(TQ_EINVAL, "sigma entries must be +1 or -1");
                sg[i] = dr->sigma[i];
            }
        } else {
            splitmix_signs(s.seed, d, sg.data());
        }
        rot->resize(d);
        for (size_t i = 0; i < d; ++i) (*rot)[i] = (float)sg[i];
    }
    const size_t md = (size_t)s.m * d;
    sk->resize(md);
    if (s.correction == TQ_CORR_SIGN) {
        // S = I: the sign of each residual coordinate
        if (dr && dr->sketch) return fail(TQ_EINVAL, "the sign correction takes no sketch draws");
        std::fill(sk->begin(), sk->end(), 0.0f);
        for (size_t i = 0; i < d; ++i) (*sk)[i * d + i] = 1.0f;
    } else if (md) {
        if (dr && dr->sketch) {
            std::memcpy(sk->data(), dr->sketch, md * sizeof(float));
        } else {
            std::vector<double> g(md);
            splitmix_gaussians(s.seed, 3, md, g.data());
            for (size_t i = 0; i < md; ++i) (*sk)[i] = (float)g[i];
        }
    }
    return TQ_OK;
}

}  // namespace tq

using namespace tq;

extern "C" {

const char* tq_last_error(void) { return g_last_error.c_str(); }

const char* tq_version(void) { return "libtq 0.1 (gfx950)"; }

int64_t tq_plane_words(const tq_spec* spec, int32_t plane) {
    if (!spec || check_spec(*spec, nullptr) != TQ_OK) return -1;
    if (plane == 0 && spec->block >= 2) return ((int64_t)spec->bits * (spec->d / spec->block) + 31) / 32;
    if (plane == 0) return (int64_t)spec->bits * spec->d / 32;
    if (plane == 1) return spec->m / 32;
    return -1;
}

tq_status tq_rope_table(double base, int32_t d, int32_t n_pos, float* cos_out, float* sin_out) {
    if (!cos_out || !sin_out) return fail(TQ_EINVAL, "null output");
    if (d <= 0 || (d & 1) || n_pos < 0 || !(base > 0)) return fail(TQ_EINVAL, "bad RoPE size or base");
    const int half = d / 2;
    std::vector<double> theta(half);
    for (int i = 0; i < half; ++i) theta[i] = std::pow(base, -2.0 * i / d);
    for (int64_t p = 0; p < n_pos; ++p)
        for (int i = 0; i < half; ++i) {
            const double ang = (double)p * theta[i];
            cos_out[p * half + i] = (float)std::cos(ang);
            sin_out[p * half + i] = (float)std::sin(ang);
        }
    return TQ_OK;
}

tq_status tq_codebook_tables(const tq_spec* spec, const tq_draws* draws, float* levels,
                             float* thresholds, float* rotation, float* sketch) {
    if (!spec) return fail(TQ_EINVAL, "null spec");
    bool dense;
    tq_status st = check_spec(*spec, &dense);
    if (st) return st;
    std::vector<float> lv, th, rot, sk;
    st = build_tables(*spec, draws, dense, &lv, &th, &rot, &sk);
    if (st) return st;
    // (an empty table, such as a vector codebook's thresholds, copies nothing:
    // memcpy from the null data() of an empty vector is undefined)
    if (levels && !lv.empty()) std::memcpy(levels, lv.data(), lv.size() * sizeof(float));
    if (thresholds && !th.empty()) std::memcpy(thresholds, th.data(), th.size() * sizeof(float));
    if (rotation && spec->rotation != TQ_ROT_NONE && !rot.empty())
        std::memcpy(rotation, rot.data(), rot.size() * sizeof(float));
    if (sketch && !sk.empty()) std::memcpy(sketch, sk.data(), sk.size() * sizeof(float));
    return TQ_OK;
}

}  // extern "C"

static tq_status codebook_create(const tq_spec* spec, const tq_draws* draws, const float* levels,
                                 const float* mu, int32_t n_mu, void* stream, tq_codebook** out) {
    if (!out) return fail(TQ_EINVAL, "null out");
    *out = nullptr;
    if (!spec) return fail(TQ_EINVAL, "null spec");
    bool dense;
    tq_status st = check_spec(*spec, &dense);
    if (st) return st;
    const int K = 1 << spec->bits;
    const bool vq = spec->block >= 2;
    if (levels && vq) {
        // explicit codewords of a vector codebook [N][block]
        for (int j = 0; j < K * spec->block; ++j)
            if (!std::isfinite(levels[j])) return fail(TQ_EINVAL, "codewords must be finite");
    } else if (levels) {
        // a calibrated table: strictly increasing, exactly symmetric
        for (int j = 0; j < K; ++j) {
            if (!std::isfinite(levels[j])) return fail(TQ_EINVAL, "levels must be finite");
            if (j && !(levels[j] > levels[j - 1])) return fail(TQ_EINVAL, "levels must be strictly increasing");
            if (levels[K - 1 - j] != -levels[j]) return fail(TQ_EINVAL, "levels must be symmetric about 0");
        }
    }
    const bool sign = spec->correction == TQ_CORR_SIGN;
    if (!sign && (mu || n_mu)) return fail(TQ_EINVAL, "mu is given only for the sign correction");
    if (mu && n_mu < 1) return fail(TQ_EINVAL, "n_mu must be >= 1 when mu is given");
    if (!mu && n_mu) return fail(TQ_EINVAL, "n_mu without mu");
    for (int32_t i = 0; mu && i < n_mu; ++i)
        if (!std::isfinite(mu[i]) || mu[i] < 0.0f) return fail(TQ_EINVAL, "mu must be finite and >= 0");
    tq_codebook* cb = new tq_codebook();
    cb->spec = *spec;
    cb->dense = dense;
    cb->K = K;
    st = build_tables(*spec, draws, dense, &cb->levels, &cb->thresholds, &cb->rotation, &cb->sketch);
    if (st) {
        delete cb;
        return st;
    }
    if (levels && vq) {
        cb->levels.assign(levels, levels + (size_t)K * spec->block);
    } else if (levels) {
        cb->levels.assign(levels, levels + K);
        for (int j = 0; j + 1 < K; ++j) cb->thresholds[j] = (float)(0.5 * ((double)levels[j] + (double)levels[j + 1]));
    }
    if (sign) {
        if (mu) cb->mu.assign(mu, mu + n_mu);
        else cb->mu.assign(1, (float)beta_mean_abs_error(spec->d, cb->levels, cb->thresholds));
    }
    if (cb->K <= 16 && !vq) level_digits(cb->levels, cb->lvl_digits, &cb->lvl_shift);
    const int d = spec->d, m = spec->m;
    if (vq && spec->block == 2 && !dense && cb->K <= kVqGridMaxN)
        vq_candidate_grid(cb->levels, cb->K, d, &cb->vq_grid, &cb->vq_inv_cell);
    // the encode kernel's sketch operand (Hadamard form): S split into fp16
    // hi + lo parts in the A-operand order of v_mfma_f32_32x32x16_f16, the
    // columns in the order the kernel's Hadamard MFMAs leave the residual in:
    // entry [(rb*(d/16) + p)*2 + piece][lane][s] = part `piece` of
    // S[rb*32 + lane%32][c],  c = 32(p/2) + 8(2(p%2) + s/4) + 4(lane/32) + s%4
    std::vector<float> sk_mfma((size_t)m * d);
    if (!dense && m && !sign) {
        const int np = d / 16;
        uint16_t* out = reinterpret_cast<uint16_t*>(sk_mfma.data());
        for (int rb = 0; rb < m / 32; ++rb)
            for (int p = 0; p < np; ++p)
                for (int l = 0; l < 64; ++l)
                    for (int sidx = 0; sidx < 8; ++sidx) {
                        const int c = 32 * (p / 2) + 8 * (2 * (p % 2) + sidx / 4) + 4 * (l >> 5) + sidx % 4;
                        const float v = cb->sketch[(size_t)(rb * 32 + (l & 31)) * d + c];
                        const uint16_t hi = f32_to_f16(v);
                        const uint16_t lo = f32_to_f16(v - f16_to_f32(hi));
                        const size_t base = ((((size_t)rb * np + p) * 2) * 64 + l) * 8 + sidx;
                        out[base] = hi;
                        out[base + 64 * 8] = lo;
                    }
    }
    // one device block: levels[16] | thresholds[16] | sigma[d] or rot[d*d] | sketch | sketch_mfma |
    // sketch transposed | mu | candidate grid (the sign correction's S = I is never read on the device)
    const size_t n_lv = vq ? std::max<size_t>(16, cb->levels.size()) : 16, n_th = 16;
    const size_t n_rot = dense ? (size_t)d * d : (size_t)d;
    const size_t n_sk = sign ? 0 : (size_t)m * d;
    const size_t n_mu_dev = cb->mu.size();
    const size_t n_grid = cb->vq_grid.size();
    const size_t total = n_lv + n_th + n_rot + 3 * n_sk + n_mu_dev + n_grid;
    std::vector<float> host(total, 0.0f);
    if (!cb->levels.empty()) std::memcpy(host.data(), cb->levels.data(), cb->levels.size() * 4);
    if (!cb->thresholds.empty()) std::memcpy(host.data() + n_lv, cb->thresholds.data(), cb->thresholds.size() * 4);
    if (n_rot) std::memcpy(host.data() + n_lv + n_th, cb->rotation.data(), n_rot * 4);
    if (n_sk) {
        std::memcpy(host.data() + n_lv + n_th + n_rot, cb->sketch.data(), n_sk * 4);
        std::memcpy(host.data() + n_lv + n_th + n_rot + n_sk, sk_mfma.data(), n_sk * 4);
        float* skt = host.data() + n_lv + n_th + n_rot + 2 * n_sk;
        for (int l = 0; l < m; ++l)
            for (int i = 0; i < d; ++i) skt[(size_t)i * m + l] = cb->sketch[(size_t)l * d + i];
    }
    if (n_mu_dev) std::memcpy(host.data() + n_lv + n_th + n_rot + 3 * n_sk, cb->mu.data(), n_mu_dev * 4);
    if (n_grid) std::memcpy(host.data() + n_lv + n_th + n_rot + 3 * n_sk + n_mu_dev, cb->vq_grid.data(), n_grid * 4);
    if (const char* f = std::getenv("TQ_TEST_FAIL_ALLOC"); f && std::atoi(f) == 1) {
        delete cb;
        return fail(TQ_ENOMEM, "allocation failure forced by TQ_TEST_FAIL_ALLOC");
    }
    hipError_t e = hipGetDevice(&cb->device);
    if (e != hipSuccess) {
        delete cb;
        return hip_fail(e, "hipGetDevice");
    }
    e = hipMalloc(&cb->block, total * sizeof(float));
    if (e != hipSuccess) {
        delete cb;
        (void)hipGetLastError();
        return e == hipErrorOutOfMemory ? fail(TQ_ENOMEM, "hipMalloc of codebook tables failed")
                                        : hip_fail(e, "hipMalloc");
    }
    float* base = (float*)cb->block;
    cb->dev.levels = base;
    cb->dev.thresholds = base + n_lv;
    if (dense) cb->dev.rot = base + n_lv + n_th;
    else cb->dev.sigma = base + n_lv + n_th;
    if (n_sk) {
        cb->dev.sketch = base + n_lv + n_th + n_rot;
        cb->dev.sketch_mfma = base + n_lv + n_th + n_rot + n_sk;
        cb->dev.sketch_t = base + n_lv + n_th + n_rot + 2 * n_sk;
    }
    if (n_mu_dev) cb->dev.mu = base + n_lv + n_th + n_rot + 3 * n_sk;
    if (n_grid) cb->dev.vq_grid = reinterpret_cast<uint32_t*>(base + n_lv + n_th + n_rot + 3 * n_sk + n_mu_dev);
    hipStream_t s = (hipStream_t)stream;
    e = hipMemcpyAsync(cb->block, host.data(), total * sizeof(float), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);  // host staging buffer is local
    if (e != hipSuccess) {
        (void)hipFree(cb->block);
        delete cb;
        return hip_fail(e, "uploading codebook tables");
    }
    *out = cb;
    return TQ_OK;
}

extern "C" {

tq_status tq_codebook_init(const tq_spec* spec, const tq_draws* draws, void* stream,
                           tq_codebook** out) {
    return codebook_create(spec, draws, nullptr, nullptr, 0, stream, out);
}

tq_status tq_codebook_init_calibrated(const tq_spec* spec, const tq_draws* draws, const float* levels,
                                      const float* mu, int32_t n_mu, void* stream, tq_codebook** out) {
    return codebook_create(spec, draws, levels, mu, n_mu, stream, out);
}

// Calibration (TurboESM summary, technical section 2: per-tensor tables and a
// calibrated mean residual magnitude).  Rotated unit vectors in double; the
// symmetric table's upper half is Lloyd's fixed point for |y|, computed on
// the sorted values with prefix sums (a cell's mean is a difference of two
// sums); mu per head with the float table, as the encoder decides codes.
tq_status tq_calibrate(const tq_spec* spec, const tq_draws* draws, const float* x, int64_t n_tok,
                       int32_t h, int32_t tok_offset, const float* rope_cos, const float* rope_sin,
                       int32_t rope_npos, float* levels, float* mu) {
    if (!spec || !x || !levels || !mu) return fail(TQ_EINVAL, "null argument");
    bool dense;
    tq_status st = check_spec(*spec, &dense);
    if (st) return st;
    if (dense) return fail(TQ_EUNSUPPORTED, "calibration is served for Hadamard and unrotated codebooks");
    if (n_tok <= 0 || h <= 0 || tok_offset < 0) return fail(TQ_EINVAL, "bad calibration sizes");
    if ((rope_cos == nullptr) != (rope_sin == nullptr)) return fail(TQ_EINVAL, "give both RoPE tables or neither");
    if (rope_cos && (int64_t)rope_npos < (int64_t)tok_offset + n_tok)
        return fail(TQ_EINVAL, "RoPE table shorter than the last position");
    const int d = spec->d, half_d = d / 2, K = 1 << spec->bits, half = K / 2;
    std::vector<float> sig(d, 1.0f);
    if (spec->rotation != TQ_ROT_NONE) {
        std::vector<int8_t> sg(d);
        if (draws && draws->sigma) {
            for (int i = 0; i < d; ++i) {
                if (draws->sigma[i] != 1 && draws->sigma[i] != -1) return fail(TQ_EINVAL, "sigma entries must be +1 or -1");
                sg[i] = draws->sigma[i];
            }
        } else {
            splitmix_signs(spec->seed, d, sg.data());
        }
        for (int i = 0; i < d; ++i) sig[i] = (float)sg[i];
    }
    const int64_t nvec = n_tok * h;
    std::vector<double> y((size_t)nvec * d);
    std::vector<char> keep((size_t)nvec, 0);
    std::vector<double> v(d);
    const double inv_sqrt_d = 1.0 / std::sqrt((double)d);
    for (int64_t t = 0; t < n_tok; ++t)
        for (int j = 0; j < h; ++j) {
            const int64_t n = t * h + j;
            const float* xr = x + n * d;
            for (int i = 0; i < d; ++i) v[i] = xr[i];
            if (rope_cos) {
                const int64_t pos = tok_offset + t;
                for (int i = 0; i < half_d; ++i) {
                    const double c = rope_cos[pos * half_d + i], sn = rope_sin[pos * half_d + i];
                    const double lo = v[i], hi = v[i + half_d];
                    v[i] = lo * c - hi * sn;
                    v[i + half_d] = hi * c + lo * sn;
                }
            }
            double ss = 0.0;
            for (int i = 0; i < d; ++i) ss += v[i] * v[i];
            const double nu = std::sqrt(ss);
            if (!(nu > 0.0)) continue;
            keep[n] = 1;
            double* yr = y.data() + n * d;
            for (int i = 0; i < d; ++i) yr[i] = v[i] / nu * sig[i];
            if (spec->rotation != TQ_ROT_NONE) {
                // Walsh-Hadamard butterflies (Sylvester order), then 1/sqrt(d)
                for (int len = 1; len < d; len <<= 1)
                    for (int i = 0; i < d; i += 2 * len)
                        for (int k = i; k < i + len; ++k) {
                            const double a = yr[k], b = yr[k + len];
                            yr[k] = a + b;
                            yr[k + len] = a - b;
                        }
                for (int i = 0; i < d; ++i) yr[i] *= inv_sqrt_d;
            }
        }
    std::vector<double> a;
    a.reserve((size_t)nvec * d);
    for (int64_t n = 0; n < nvec; ++n)
        if (keep[n])
            for (int i = 0; i < d; ++i) a.push_back(std::fabs(y[(size_t)n * d + i]));
    if (a.empty()) return fail(TQ_EINVAL, "no non-zero calibration vector");
    std::sort(a.begin(), a.end());
    const size_t N = a.size();
    std::vector<long double> pre(N + 1, 0.0L);
    for (size_t i = 0; i < N; ++i) pre[i + 1] = pre[i] + (long double)a[i];
    std::vector<double> lv(half);
    for (int j = 0; j < half; ++j) {
        size_t idx = (size_t)std::floor((j + 0.5) * (double)N / half);
        lv[j] = a[std::min(idx, N - 1)];
    }
    std::vector<size_t> cut(half + 1), prev;
    bool settled = false;
    for (int it = 0; it < 100000; ++it) {
        cut[0] = 0;
        cut[half] = N;
        for (int j = 1; j < half; ++j) {
            const double b = 0.5 * (lv[j - 1] + lv[j]);
            cut[j] = (size_t)(std::lower_bound(a.begin(), a.end(), b) - a.begin());  // ties go up
        }
        for (int j = 0; j < half; ++j)
            if (cut[j + 1] > cut[j]) lv[j] = (double)((pre[cut[j + 1]] - pre[cut[j]]) / (long double)(cut[j + 1] - cut[j]));
        if (!prev.empty() && prev == cut) {
            settled = true;
            break;
        }
        prev = cut;
    }
    if (!settled) return fail(TQ_EINVAL, "calibration did not settle");
    std::vector<float> t32(K), tau32(K - 1);
    for (int j = 0; j < half; ++j) {
        t32[half + j] = (float)lv[j];
        t32[half - 1 - j] = -(float)lv[j];
    }
    for (int j = 0; j + 1 < K; ++j) tau32[j] = (float)(0.5 * ((double)t32[j] + (double)t32[j + 1]));
    for (int j = 0; j < h; ++j) {
        double sum = 0.0;
        int64_t cnt = 0;
        for (int64_t t = 0; t < n_tok; ++t) {
            const int64_t n = t * h + j;
            if (!keep[n]) continue;
            for (int i = 0; i < d; ++i) {
                const double yy = y[(size_t)n * d + i];
                const float y32 = (float)yy;
                int c = 0;
                for (int k = 0; k + 1 < K; ++k) c += y32 >= tau32[k];
                sum += std::fabs(yy - (double)t32[c]);
                ++cnt;
            }
        }
        mu[j] = cnt ? (float)(sum / (double)cnt) : 0.0f;
    }
    std::memcpy(levels, t32.data(), K * sizeof(float));
    return TQ_OK;
}

tq_status tq_codebook_get_mu(const tq_codebook* cb, float* mu, int32_t* n_mu) {
    if (!cb || !n_mu) return fail(TQ_EINVAL, "null argument");
    *n_mu = (int32_t)cb->mu.size();
    if (mu && !cb->mu.empty()) std::memcpy(mu, cb->mu.data(), cb->mu.size() * 4);
    return TQ_OK;
}

tq_status tq_codebook_destroy(tq_codebook* cb) {
    if (!cb) return TQ_OK;
    hipError_t e = hipSuccess;
    if (cb->block) e = hipFree(cb->block);
    delete cb;
    return e == hipSuccess ? TQ_OK : hip_fail(e, "hipFree");
}

tq_status tq_codebook_get_spec(const tq_codebook* cb, tq_spec* out) {
    if (!cb || !out) return fail(TQ_EINVAL, "null argument");
    *out = cb->spec;
    return TQ_OK;
}

tq_status tq_codebook_export(const tq_codebook* cb, float* levels, float* thresholds,
                             float* rotation, float* sketch) {
    if (!cb) return fail(TQ_EINVAL, "null codebook");
    if (levels && !cb->levels.empty()) std::memcpy(levels, cb->levels.data(), cb->levels.size() * 4);
    if (thresholds && !cb->thresholds.empty())
        std::memcpy(thresholds, cb->thresholds.data(), cb->thresholds.size() * 4);
    if (rotation && !no_rotation(cb)) std::memcpy(rotation, cb->rotation.data(), cb->rotation.size() * 4);
    if (sketch && !cb->sketch.empty()) std::memcpy(sketch, cb->sketch.data(), cb->sketch.size() * 4);
    return TQ_OK;
}

static tq_status check_packed(const tq_codebook* cb, const tq_packed* p, int64_t need,
                              const char* what) {
    if (!p) return fail(TQ_EINVAL, std::string("null packed planes: ") + what);
    if (!p->norm || !p->codes) return fail(TQ_EINVAL, std::string("null norm/codes plane: ") + what);
    if (cb->spec.m && !p->signs) return fail(TQ_EINVAL, std::string("null signs plane with m > 0: ") + what);
    if (has_rnorm(cb) && !p->rnorm) return fail(TQ_EINVAL, std::string("null rnorm plane with m > 0: ") + what);
    if (p->n < need) return fail(TQ_EINVAL, std::string("packed capacity too small: ") + what);
    return TQ_OK;
}

}  // extern "C"

// page table checks: page size a multiple of 64, logical capacity below 2^31
static tq_status check_pages(const tq_pages* pg, PageRef* out) {
    if (!pg || !pg->pages) return fail(TQ_EINVAL, "null page table");
    if (pg->page_size <= 0 || pg->page_size % 64) return fail(TQ_EINVAL, "page_size must be a positive multiple of 64");
    if (pg->max_pages <= 0 || pg->n_pages <= 0) return fail(TQ_EINVAL, "max_pages and n_pages must be positive");
    if ((int64_t)pg->max_pages * pg->page_size >= ((int64_t)1 << 31))
        return fail(TQ_EINVAL, "max_pages * page_size must be below 2^31");
    out->table = pg->pages;
    out->size = pg->page_size;
    out->max_pages = pg->max_pages;
    out->n_pages = pg->n_pages;
    return TQ_OK;
}

// Shared body of the encode entry points.  pos != nullptr: one token per
// (sequence, head) at slot pos[sequence] (append); pg.table != nullptr: paged
// records.  cap_records: records the planes must hold.
static tq_status encode_common(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v,
                               int32_t dtype, int32_t n_seq, int32_t n_tok, int32_t h_kv, const int64_t ks[3],
                               const int64_t vs[3], int32_t tok_offset, int32_t L_cap, const PageRef& pg,
                               const int32_t* pos, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                               const tq_packed* kout, const tq_packed* vout, int64_t cap_records, void* ws,
                               size_t ws_bytes, void* stream) {
    if (dtype != TQ_F32 && dtype != TQ_BF16) return fail(TQ_EINVAL, "dtype must be TQ_F32 or TQ_BF16");
    if (n_seq < 0 || n_tok < 0 || h_kv < 0 || tok_offset < 0 || L_cap < 0) return fail(TQ_EINVAL, "negative size");
    const int64_t slots = pg.table ? (int64_t)pg.max_pages * pg.size : L_cap;
    if (!pos && (int64_t)tok_offset + n_tok > slots) return fail(TQ_EINVAL, "tok_offset + n_tok exceeds the cache's slots");
    if ((int64_t)n_seq * n_tok * h_kv == 0) return TQ_OK;  // nothing to encode
    if (!k && !v) return fail(TQ_EINVAL, "neither k nor v given");
    if ((rope_cos == nullptr) != (rope_sin == nullptr)) return fail(TQ_EINVAL, "give both RoPE tables or neither");
    const int64_t nvec = (int64_t)n_seq * n_tok * h_kv;
    const int align = dtype == TQ_F32 ? 4 : 8;
    struct Side { const tq_codebook* cb; const void* x; const int64_t* st; const tq_packed* o; bool rope; };
    Side sides[2] = {{ck, k, ks, kout, rope_cos != nullptr}, {cv, v, vs, vout, false}};
    for (auto& sd : sides) {
        if (!sd.x) continue;
        if (!sd.cb) return fail(TQ_EINVAL, "tensor given without a codebook");
        if (!sd.st) return fail(TQ_EINVAL, "null strides");
        for (int i = 0; i < 3; ++i)
            if (sd.st[i] < 0 || sd.st[i] % align) return fail(TQ_EINVAL, "strides must be non-negative multiples of 16 bytes");
        if (((uintptr_t)sd.x) % 16) return fail(TQ_EINVAL, "input must be 16-byte aligned");
        tq_status st = check_packed(sd.cb, sd.o, cap_records, sd.x == k ? "k" : "v");
        if (st) return st;
        if (sd.rope) {
            if (!pos && rope_npos < tok_offset + n_tok) return fail(TQ_EINVAL, "RoPE table shorter than the last position");
            if (pos && rope_npos <= 0) return fail(TQ_EINVAL, "empty RoPE table");
            if (sd.cb->spec.d % 2) return fail(TQ_EINVAL, "RoPE needs an even d");
        }
        if (sd.cb->dense && (pos || pg.table))
            return fail(TQ_EUNSUPPORTED, "appends and paged records are served for Hadamard and unrotated codebooks");
        if (sd.cb->spec.block >= 2) {
            if (!vq_supported(sd.cb))
                return fail(TQ_EUNSUPPORTED,
                            "vector codebooks encode on the GPU for block 2 with the Hadamard rotation at d = 64 or 128, "
                            "or any block with a dense rotation");
            if (nvec >= ((int64_t)1 << 31)) return fail(TQ_EUNSUPPORTED, "too many vectors in one encode call (split it)");
        }
        if (!sd.cb->dense && (int64_t)n_seq * ((n_tok + 31) / 32) * h_kv >= (int64_t)1 << 31)
            return fail(TQ_EUNSUPPORTED, "too many vectors in one encode call (split it)");
        if (sd.cb->dense && nvec > 0) {
            const size_t wsn = encode_workspace_bytes(sd.cb, nvec);
            if (!ws || ws_bytes < wsn) return fail(TQ_EINVAL, "workspace too small for the dense encoder");
        }
    }
    for (auto& sd : sides) {
        if (!sd.x) continue;
        EncodeArgs a{};
        a.x = sd.x;
        a.s_seq = sd.st[0];
        a.s_tok = sd.st[1];
        a.s_head = sd.st[2];
        a.n_seq = n_seq;
        a.n_tok = n_tok;
        a.h_kv = h_kv;
        a.tok_offset = tok_offset;
        a.L_cap = L_cap;
        a.bf16 = dtype == TQ_BF16;
        a.rope_cos = sd.rope ? rope_cos : nullptr;
        a.rope_sin = sd.rope ? rope_sin : nullptr;
        a.rope_npos = rope_npos;
        a.out = *sd.o;
        a.ws = ws;
        a.ws_bytes = ws_bytes;
        a.append = pos ? 1 : 0;
        a.pos = pos;
        a.pages = pg;
        hipError_t e = launch_encode(sd.cb, a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "encode launch");
    }
    return TQ_OK;
}

// a sign-corrected codebook has one mu per KV head of the call, or one shared
static tq_status check_mu(const tq_codebook* cb, int32_t h_kv) {
    if (sign_corr(cb) && cb->mu.size() != 1 && (int64_t)cb->mu.size() != h_kv)
        return fail(TQ_EINVAL, "the codebook's mu count matches neither 1 nor h_kv");
    return TQ_OK;
}

static tq_status check_attn(const tq_codebook* ck, const void* q, int32_t q_dtype, int32_t B,
                            int32_t Hq, int32_t h_kv, int32_t L_cap, const int32_t* seq_len,
                            const float* rope_cos, const float* rope_sin, int32_t rope_npos) {
    if (!ck) return fail(TQ_EINVAL, "null key codebook");
    if (!q || !seq_len) return fail(TQ_EINVAL, "null q or seq_len");
    if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return fail(TQ_EINVAL, "q dtype must be TQ_F32 or TQ_BF16");
    if (B < 0 || Hq < 0 || h_kv <= 0 || L_cap < 0) return fail(TQ_EINVAL, "bad sizes");
    if (Hq % h_kv) return fail(TQ_EINVAL, "Hq must be a multiple of h_kv");
    if ((rope_cos == nullptr) != (rope_sin == nullptr)) return fail(TQ_EINVAL, "give both RoPE tables or neither");
    if (rope_cos && rope_npos <= L_cap) return fail(TQ_EINVAL, "RoPE table must cover position L_cap");
    if (((uintptr_t)q) % 16) return fail(TQ_EINVAL, "q must be 16-byte aligned");
    return TQ_OK;
}

static tq_status logits_common(const tq_codebook* ck, const void* q, int32_t q_dtype, const tq_packed* k, int32_t B,
                               int32_t Hq, int32_t h_kv, int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos,
                               const PageRef& pg, int64_t cap_records, const float* rope_cos, const float* rope_sin,
                               int32_t rope_npos, int32_t top_k, float* out, int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
    tq_status st = check_attn(ck, q, q_dtype, B, Hq, h_kv, L_cap, seq_len, rope_cos, rope_sin, rope_npos);
    if (st) return st;
    if (top_k < 0 || top_k > 16) return fail(TQ_EINVAL, "top_k must be 0..16");
    if (!out || (top_k && !topk_idx)) return fail(TQ_EINVAL, "null output");
    st = check_packed(ck, k, cap_records, "k");
    if (st) return st;
    st = check_mu(ck, h_kv);
    if (st) return st;
    if (ck->spec.block >= 2) {
        if (!vq_supported(ck)) return fail(TQ_EUNSUPPORTED, "no logit kernel for this vector codebook");
        if (ck->dense && pg.table) return fail(TQ_EUNSUPPORTED, "paged scans are served for Hadamard codebooks");
    } else if ((sign_corr(ck) || pg.table) && !logits_mfma_supported(ck)) {
        return fail(TQ_EUNSUPPORTED, "no logit kernel for this codebook (paged and sign-corrected scans need "
                                     "a Hadamard or unrotated codebook with bits <= 4 and m <= 128)");
    }
    if ((int64_t)B * Hq == 0 || (L_cap == 0 && top_k == 0)) return TQ_OK;
    const size_t need = logits_workspace_bytes(ck, B, Hq, h_kv, L_cap, top_k);
    if (ws_bytes < need || (need && !ws)) return fail(TQ_EINVAL, "workspace too small");
    AttnArgs a{};
    a.q = q;
    a.bf16 = q_dtype == TQ_BF16;
    a.B = B;
    a.Hq = Hq;
    a.h_kv = h_kv;
    a.L_cap = L_cap;
    a.seq_len = seq_len;
    a.q_pos = q_pos;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.top_k = top_k;
    a.out = out;
    a.topk_idx = topk_idx;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    a.pages = pg;
    hipError_t e = launch_logits(ck, *k, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : hip_fail(e, "logits launch");
}

static tq_status decode_common(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                               const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                               int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos, const PageRef& pg,
                               int64_t cap_records, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                               float scale,
                               float* out, void* ws, size_t ws_bytes, void* stream) {
    tq_status st = check_attn(ck, q, q_dtype, B, Hq, h_kv, L_cap, seq_len, rope_cos, rope_sin, rope_npos);
    if (st) return st;
    if (!cv) return fail(TQ_EINVAL, "null value codebook");
    if (!out) return fail(TQ_EINVAL, "null output");
    if (!(scale >= 0.0f) || std::isinf(scale)) return fail(TQ_EINVAL, "scale must be finite and >= 0");
    if (ck->spec.d != cv->spec.d) return fail(TQ_EINVAL, "key and value dimensions differ");
    const bool vq = ck->spec.block >= 2 || cv->spec.block >= 2;
    if (vq && !vq_attn_supported(ck, cv))
        return fail(TQ_EUNSUPPORTED, "the fused decode takes vector codebooks for keys and values together (block 2, "
                                     "Hadamard, d = 64 or 128, at most 5 key index bits at d = 128 and 6 at d = 64); "
                                     "rebuild other vector-coded values with tq_decode_vectors");
    if (vq) {
        int nsplit = 1, split_len = 0;
        vq_attn_plan(L_cap, &nsplit, &split_len);
        if (nsplit > 65535) return fail(TQ_EUNSUPPORTED, "the vector-codebook decode takes at most 65535 splits of keys");
    }
    st = check_packed(ck, k, cap_records, "k");
    if (st) return st;
    st = check_packed(cv, v, cap_records, "v");
    if (st) return st;
    st = check_mu(ck, h_kv);
    if (st) return st;
    st = check_mu(cv, h_kv);
    if (st) return st;
    if (!vq && (ck->dense || cv->dense))
        return fail(TQ_EUNSUPPORTED, "the fused decode serves Hadamard or unrotated scalar codebooks; a dense "
                                     "rotation is served by tq_attn_logits only");
    if (!vq && (ck->spec.bits != cv->spec.bits || ck->spec.m != cv->spec.m))
        return fail(TQ_EUNSUPPORTED, "the fused decode needs key and value codebooks of equal bits and m");
    if (!vq && (sign_corr(ck) || sign_corr(cv) || pg.table) && !decode_mfma_supported(ck, cv))
        return fail(TQ_EUNSUPPORTED, "paged and sign-corrected decodes need key and value tables of equal d, bits "
                                     "and m (bits <= 4)");
    if ((int64_t)B * Hq == 0) return TQ_OK;
    const size_t need = decode_workspace_bytes(ck, cv, B, Hq, h_kv, L_cap);
    if (ws_bytes < need || (need && !ws)) return fail(TQ_EINVAL, "workspace too small");
    AttnArgs a{};
    a.q = q;
    a.bf16 = q_dtype == TQ_BF16;
    a.B = B;
    a.Hq = Hq;
    a.h_kv = h_kv;
    a.L_cap = L_cap;
    a.seq_len = seq_len;
    a.q_pos = q_pos;
    a.rope_cos = rope_cos;
    a.rope_sin = rope_sin;
    a.scale = scale > 0 ? scale : 1.0f / std::sqrt((float)ck->spec.d);
    a.out = out;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    a.pages = pg;
    hipError_t e = launch_decode(ck, cv, *k, *v, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : hip_fail(e, "decode launch");
}

extern "C" {

tq_status tq_encode_kv(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v,
                       int32_t dtype, int32_t n_seq, int32_t n_tok, int32_t h_kv,
                       const int64_t* k_stride, const int64_t* v_stride, int32_t tok_offset,
                       int32_t L_cap, const float* rope_cos, const float* rope_sin,
                       int32_t rope_npos, const tq_packed* kout, const tq_packed* vout, void* ws,
                       size_t ws_bytes, void* stream) {
    return encode_common(ck, cv, k, v, dtype, n_seq, n_tok, h_kv, k_stride, v_stride, tok_offset, L_cap, PageRef{},
                         nullptr, rope_cos, rope_sin, rope_npos, kout, vout, (int64_t)n_seq * h_kv * L_cap, ws,
                         ws_bytes, stream);
}

tq_status tq_encode_kv_paged(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v,
                             int32_t dtype, int32_t n_seq, int32_t n_tok, int32_t h_kv, const int64_t* k_stride,
                             const int64_t* v_stride, int32_t tok_offset, const tq_pages* pages,
                             const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                             const tq_packed* kout, const tq_packed* vout, void* stream) {
    PageRef pg;
    tq_status st = check_pages(pages, &pg);
    if (st) return st;
    return encode_common(ck, cv, k, v, dtype, n_seq, n_tok, h_kv, k_stride, v_stride, tok_offset, 0, pg, nullptr,
                         rope_cos, rope_sin, rope_npos, kout, vout, pg.n_pages * h_kv * (int64_t)pg.size, nullptr, 0,
                         stream);
}

tq_status tq_append_kv(const tq_codebook* ck, const tq_codebook* cv, const void* k, const void* v, int32_t dtype,
                       int32_t B, int32_t h_kv, const int64_t* k_stride, const int64_t* v_stride,
                       const int32_t* pos, const tq_pages* pages, int32_t L_cap, const float* rope_cos,
                       const float* rope_sin, int32_t rope_npos, const tq_packed* kout, const tq_packed* vout,
                       void* stream) {
    if (!pos) return fail(TQ_EINVAL, "null pos");
    PageRef pg;
    int64_t cap = 0;
    if (pages) {
        tq_status st = check_pages(pages, &pg);
        if (st) return st;
        cap = pg.n_pages * h_kv * (int64_t)pg.size;
        L_cap = 0;
    } else {
        if (L_cap <= 0) return fail(TQ_EINVAL, "L_cap must be positive without a page table");
        cap = (int64_t)B * h_kv * L_cap;
    }
    if ((int64_t)B * h_kv >= ((int64_t)1 << 31)) return fail(TQ_EUNSUPPORTED, "too many vectors in one append");
    const int64_t ks[3] = {k_stride ? k_stride[0] : 0, 0, k_stride ? k_stride[1] : 0};
    const int64_t vs[3] = {v_stride ? v_stride[0] : 0, 0, v_stride ? v_stride[1] : 0};
    return encode_common(ck, cv, k, v, dtype, B, 1, h_kv, k_stride ? ks : nullptr, v_stride ? vs : nullptr, 0, L_cap,
                         pg, pos, rope_cos, rope_sin, rope_npos, kout, vout, cap, nullptr, 0, stream);
}

tq_status tq_attn_logits(const tq_codebook* ck, const void* q, int32_t q_dtype, const tq_packed* k,
                         int32_t B, int32_t Hq, int32_t h_kv, int32_t L_cap, const int32_t* seq_len,
                         const int32_t* q_pos, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                         int32_t top_k, float* out, int32_t* topk_idx, void* ws, size_t ws_bytes,
                         void* stream) {
    return logits_common(ck, q, q_dtype, k, B, Hq, h_kv, L_cap, seq_len, q_pos, PageRef{}, (int64_t)B * h_kv * L_cap,
                         rope_cos, rope_sin, rope_npos, top_k, out, topk_idx, ws, ws_bytes, stream);
}

tq_status tq_attn_logits_paged(const tq_codebook* ck, const void* q, int32_t q_dtype, const tq_packed* k, int32_t B,
                               int32_t Hq, int32_t h_kv, const int32_t* seq_len, const int32_t* q_pos,
                               const tq_pages* pages, const float* rope_cos, const float* rope_sin, int32_t rope_npos,
                               int32_t top_k, float* out, int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
    PageRef pg;
    tq_status st = check_pages(pages, &pg);
    if (st) return st;
    return logits_common(ck, q, q_dtype, k, B, Hq, h_kv, pg.max_pages * pg.size, seq_len, q_pos, pg,
                         pg.n_pages * h_kv * (int64_t)pg.size, rope_cos, rope_sin, rope_npos, top_k, out, topk_idx, ws,
                         ws_bytes, stream);
}

tq_status tq_attn_decode(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                         const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                         int32_t L_cap, const int32_t* seq_len, const int32_t* q_pos, const float* rope_cos,
                         const float* rope_sin, int32_t rope_npos, float scale, float* out,
                         void* ws, size_t ws_bytes, void* stream) {
    return decode_common(ck, cv, q, q_dtype, k, v, B, Hq, h_kv, L_cap, seq_len, q_pos, PageRef{},
                         (int64_t)B * h_kv * L_cap,
                         rope_cos, rope_sin, rope_npos, scale, out, ws, ws_bytes, stream);
}

tq_status tq_attn_decode_paged(const tq_codebook* ck, const tq_codebook* cv, const void* q, int32_t q_dtype,
                               const tq_packed* k, const tq_packed* v, int32_t B, int32_t Hq, int32_t h_kv,
                               const int32_t* seq_len, const int32_t* q_pos, const tq_pages* pages,
                               const float* rope_cos, const float* rope_sin, int32_t rope_npos, float scale,
                               float* out, void* ws, size_t ws_bytes, void* stream) {
    PageRef pg;
    tq_status st = check_pages(pages, &pg);
    if (st) return st;
    return decode_common(ck, cv, q, q_dtype, k, v, B, Hq, h_kv, pg.max_pages * pg.size, seq_len, q_pos, pg,
                         pg.n_pages * h_kv * (int64_t)pg.size, rope_cos, rope_sin, rope_npos, scale, out, ws, ws_bytes,
                         stream);
}

tq_status tq_decode_vectors(const tq_codebook* cb, const tq_packed* packed, int64_t first, int64_t count, float* out,
                            void* stream) {
    if (!cb || !packed || !out) return fail(TQ_EINVAL, "null argument");
    if (!packed->norm || !packed->codes) return fail(TQ_EINVAL, "null norm/codes plane");
    if (first < 0 || count < 0 || first + count > packed->n) return fail(TQ_EINVAL, "records out of range");
    if (cb->spec.block < 2 || !vq_supported(cb))
        return fail(TQ_EUNSUPPORTED, "vectors are rebuilt for vector codebooks");
    if (count == 0) return TQ_OK;
    hipError_t e = launch_vq_decode(cb, *packed, first, count, out, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : hip_fail(e, "decode launch");
}

size_t tq_workspace_bytes(const tq_codebook* ck, const tq_codebook* cv, int32_t op, int64_t B,
                          int32_t Hq, int32_t h_kv, int32_t L_cap, int32_t top_k) {
    if (!ck || B < 0) return 0;
    switch (op) {
        case TQ_OP_ENCODE: {
            size_t a = encode_workspace_bytes(ck, B);
            size_t b = cv ? encode_workspace_bytes(cv, B) : 0;
            return std::max(a, b);
        }
        case TQ_OP_LOGITS:
            if (h_kv <= 0 || Hq < 0 || L_cap < 0) return 0;
            return logits_workspace_bytes(ck, B, Hq, h_kv, L_cap, top_k);
        case TQ_OP_DECODE:
            if (!cv || h_kv <= 0 || Hq < 0 || L_cap < 0) return 0;
            return decode_workspace_bytes(ck, cv, B, Hq, h_kv, L_cap);
        default:
            return 0;
    }
}

}  // extern "C"
