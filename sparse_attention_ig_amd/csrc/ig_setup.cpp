// Host-side offline setup of the InfiniGen decode path: skew rotation, weight
// rotation, storage rounding and the partial-weight channel pick.
//
// Method: InfiniGen (arXiv 2406.19707), paper-graph-ui summary, section 3.4:
// "Skewed Partial Weights" (A = V of the sample query's SVD, W~ = W A) and
// "Prefill Stage: Partial Weight Index Generation" (column sums of |W~_Q| and
// |K~|, top channels, partial weight extraction).
//
// Everything here is plain float64 host code with no GPU calls.  The SVD is a
// one-sided (Hestenes) Jacobi iteration: it orthogonalises the columns of the
// source matrix by plane rotations and accumulates the same rotations in V,
// which is accurate to a few ulps for the small d x d problems of one head.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <numeric>
#include <thread>
#include <vector>

#include "ig_internal.h"

namespace ig {

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    unsigned hw = std::thread::hardware_concurrency();
    return hw ? static_cast<int>(hw) : 1;
}

// Run f(i) for i in [0, count) on up to nthreads threads (static blocks).
static void parallel_for(int64_t count, int nthreads, const std::function<void(int64_t)>& f) {
    int nt = static_cast<int>(std::min<int64_t>(resolve_threads(nthreads), std::max<int64_t>(count, 1)));
    if (nt <= 1) {
        for (int64_t i = 0; i < count; ++i) f(i);
        return;
    }
    std::vector<std::thread> pool;
    int64_t per = (count + nt - 1) / nt;
    for (int t = 0; t < nt; ++t) {
        int64_t lo = t * per, hi = std::min(count, lo + per);
        if (lo >= hi) break;
        pool.emplace_back([lo, hi, &f] { for (int64_t i = lo; i < hi; ++i) f(i); });
    }
    for (auto& th : pool) th.join();
}

// One head: V (d x d, row-major, column j = j-th right singular vector) of the
// m x d row-major matrix src, columns by descending singular value, signed so
// that each column's largest-magnitude entry is positive.
static void jacobi_right_vectors(const double* src, int m, int d, double* V, double* sigma) {
    // column-major working copies: U columns are contiguous
    std::vector<double> U(static_cast<size_t>(m) * d), W(static_cast<size_t>(d) * d, 0.0);
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < d; ++j) U[static_cast<size_t>(j) * m + i] = src[static_cast<size_t>(i) * d + j];
    for (int j = 0; j < d; ++j) W[static_cast<size_t>(j) * d + j] = 1.0;

    const double eps = 1e-15;
    for (int sweep = 0; sweep < 60; ++sweep) {
        int rotated = 0;
        for (int p = 0; p < d - 1; ++p) {
            double* up = &U[static_cast<size_t>(p) * m];
            double* vp = &W[static_cast<size_t>(p) * d];
            for (int q = p + 1; q < d; ++q) {
                double* uq = &U[static_cast<size_t>(q) * m];
                double a = 0, b = 0, g = 0;
                for (int i = 0; i < m; ++i) {
                    a += up[i] * up[i];
                    b += uq[i] * uq[i];
                    g += up[i] * uq[i];
                }
                if (std::fabs(g) <= eps * std::sqrt(a * b) || g == 0.0) continue;
                ++rotated;
                // rotation that zeroes the inner product of columns p and q
                double zeta = (b - a) / (2.0 * g);
                double t = (zeta >= 0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
                double c = 1.0 / std::sqrt(1.0 + t * t), s = c * t;
                for (int i = 0; i < m; ++i) {
                    double x = up[i], y = uq[i];
                    up[i] = c * x - s * y;
                    uq[i] = s * x + c * y;
                }
                double* vq = &W[static_cast<size_t>(q) * d];
                for (int i = 0; i < d; ++i) {
                    double x = vp[i], y = vq[i];
                    vp[i] = c * x - s * y;
                    vq[i] = s * x + c * y;
                }
            }
        }
        if (!rotated) break;
    }
    std::vector<double> norm(d);
    for (int j = 0; j < d; ++j) {
        double acc = 0;
        const double* u = &U[static_cast<size_t>(j) * m];
        for (int i = 0; i < m; ++i) acc += u[i] * u[i];
        norm[j] = std::sqrt(acc);
    }
    std::vector<int> order(d);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return norm[x] > norm[y]; });
    for (int jj = 0; jj < d; ++jj) {
        const double* v = &W[static_cast<size_t>(order[jj]) * d];
        int piv = 0;
        for (int i = 1; i < d; ++i)
            if (std::fabs(v[i]) > std::fabs(v[piv])) piv = i;
        double sgn = v[piv] < 0 ? -1.0 : 1.0;
        for (int i = 0; i < d; ++i) V[static_cast<size_t>(i) * d + jj] = sgn * v[i];
        if (sigma) sigma[jj] = norm[order[jj]];
    }
}

// out[r][h*d + j] = sum_i M[r][h*d + i] A_h[i][j]
static void rotate_rows(const double* A, int H, int d, const double* M, int64_t rows,
                        double* out, int nthreads) {
    const int64_t ncol = static_cast<int64_t>(H) * d;
    parallel_for(rows, nthreads, [&](int64_t r) {
        const double* mrow = M + r * ncol;
        double* orow = out + r * ncol;
        for (int h = 0; h < H; ++h) {
            const double* Ah = A + static_cast<size_t>(h) * d * d;
            double* o = orow + static_cast<size_t>(h) * d;
            for (int j = 0; j < d; ++j) o[j] = 0.0;
            for (int i = 0; i < d; ++i) {
                double mv = mrow[static_cast<size_t>(h) * d + i];
                const double* arow = Ah + static_cast<size_t>(i) * d;
                for (int j = 0; j < d; ++j) o[j] += mv * arow[j];
            }
        }
    });
}

int skew_weights(const ig_skew_args* a) {
    if (!a) return fail(IG_EINVAL, "ig_skew_weights: args is NULL");
    if (a->H < 1 || a->d < 1 || a->m < a->d)
        return fail(IG_EINVAL, "ig_skew_weights: need H >= 1, d >= 1, m >= d (got H=%d d=%d m=%d)", a->H, a->d, a->m);
    if (!a->skew_src || !a->A) return fail(IG_EINVAL, "ig_skew_weights: skew_src and A are required");
    if ((a->Wq || a->Wk) && a->D < 1) return fail(IG_EINVAL, "ig_skew_weights: D must be >= 1");
    if (!a->Wq != !a->Wq_s || !a->Wk != !a->Wk_s || !a->bq != !a->bq_s || !a->bk != !a->bk_s)
        return fail(IG_EINVAL, "ig_skew_weights: each output must be given exactly when its input is");
    const int H = a->H, d = a->d, m = a->m;
    parallel_for(H, a->nthreads, [&](int64_t h) {
        jacobi_right_vectors(a->skew_src + static_cast<size_t>(h) * m * d, m, d,
                             a->A + static_cast<size_t>(h) * d * d,
                             a->sigma ? a->sigma + static_cast<size_t>(h) * d : nullptr);
    });
    if (a->Wq) rotate_rows(a->A, H, d, a->Wq, a->D, a->Wq_s, a->nthreads);
    if (a->Wk) rotate_rows(a->A, H, d, a->Wk, a->D, a->Wk_s, a->nthreads);
    if (a->bq) rotate_rows(a->A, H, d, a->bq, 1, a->bq_s, 1);
    if (a->bk) rotate_rows(a->A, H, d, a->bk, 1, a->bk_s, 1);
    return ok();
}

int skew_apply(const double* A, int H, int d, const double* M, int64_t rows, double* out, int nthreads) {
    if (!A || !M || !out) return fail(IG_EINVAL, "ig_skew_apply: NULL pointer");
    if (H < 1 || d < 1 || rows < 0) return fail(IG_EINVAL, "ig_skew_apply: bad sizes");
    if (out == M) return fail(IG_EINVAL, "ig_skew_apply: out must not alias M");
    rotate_rows(A, H, d, M, rows, out, nthreads);
    return ok();
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;  // NaN
    uint32_t lsb = (u >> 16) & 1u;
    return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

int store(const double* vals, int64_t count, int dtype, void* out) {
    if (!vals || !out || count < 0) return fail(IG_EINVAL, "ig_store: bad arguments");
    if (dtype == IG_F32) {
        float* o = static_cast<float*>(out);
        for (int64_t i = 0; i < count; ++i) o[i] = static_cast<float>(vals[i]);
    } else if (dtype == IG_BF16) {
        uint16_t* o = static_cast<uint16_t*>(out);
        for (int64_t i = 0; i < count; ++i) o[i] = f32_to_bf16_rne(static_cast<float>(vals[i]));
    } else {
        return fail(IG_EINVAL, "ig_store: unknown dtype %d", dtype);
    }
    return ok();
}

static inline double stored_value(const void* base, int64_t i, int dtype) {
    if (dtype == IG_F32) return static_cast<double>(static_cast<const float*>(base)[i]);
    uint32_t u = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return static_cast<double>(f);
}

int partial_weight_index(const void* Wq_s, int D, int H, int d, int r, const void* K_s, int B,
                         int n_cap, int n, int dtype, int32_t* chan, void* Wq_part, int nthreads) {
    if (!Wq_s || !K_s || !chan || !Wq_part) return fail(IG_EINVAL, "ig_partial_weight_index: NULL pointer");
    if (D < 1 || H < 1 || d < 1 || r < 1 || r > d || B < 1 || n < 1 || n > n_cap)
        return fail(IG_EINVAL, "ig_partial_weight_index: bad sizes (D=%d H=%d d=%d r=%d B=%d n=%d n_cap=%d)",
                    D, H, d, r, B, n, n_cap);
    if (dtype != IG_F32 && dtype != IG_BF16) return fail(IG_EINVAL, "ig_partial_weight_index: bad dtype");
    const int64_t ncol = static_cast<int64_t>(H) * d;
    std::vector<double> score(static_cast<size_t>(ncol), 0.0);
    // column sums of |W~_Q| over the D rows, then of |K~| over every cached row of the batch
    parallel_for(H, nthreads, [&](int64_t h) {
        double* sc = &score[static_cast<size_t>(h) * d];
        for (int64_t i = 0; i < D; ++i)
            for (int c = 0; c < d; ++c) sc[c] += std::fabs(stored_value(Wq_s, i * ncol + h * d + c, dtype));
        std::vector<double> ks(d, 0.0);
        for (int b = 0; b < B; ++b) {
            int64_t base = ((static_cast<int64_t>(b) * H + h) * n_cap) * d;
            for (int64_t j = 0; j < n; ++j)
                for (int c = 0; c < d; ++c) ks[c] += std::fabs(stored_value(K_s, base + j * d + c, dtype));
        }
        for (int c = 0; c < d; ++c) sc[c] += ks[c];
        std::vector<int> order(d);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return sc[x] > sc[y]; });
        std::vector<int> pick(order.begin(), order.begin() + r);
        std::sort(pick.begin(), pick.end());
        for (int k = 0; k < r; ++k) chan[h * r + k] = pick[k];
    });
    const size_t esz = dtype == IG_F32 ? 4 : 2;
    const char* src = static_cast<const char*>(Wq_s);
    char* dst = static_cast<char*>(Wq_part);
    // one row of D inputs per partial column (h, k): the layout the projection's matrix-core operands
    // read with 16-byte loads along the reduction
    for (int h = 0; h < H; ++h)
        for (int k = 0; k < r; ++k) {
            char* row = dst + (static_cast<int64_t>(h) * r + k) * D * esz;
            const int64_t c = static_cast<int64_t>(h) * d + chan[h * r + k];
            for (int64_t i = 0; i < D; ++i) std::memcpy(row + i * esz, src + (i * ncol + c) * esz, esz);
        }
    return ok();
}

}  // namespace ig
