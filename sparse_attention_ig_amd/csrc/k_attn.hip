// Attention over the selected rows only (InfiniGen, arXiv 2406.19707,
// paper-graph-ui summary, section 3.2 Inference Controller; section 2,
// softmax(QK^T)V over the cached rows).
//
// Decode attention with one query per (b, h) and its own index set is a set of
// matrix-vector products, not a dense contraction, so it runs on the vector
// ALUs: a row of K or V (d elements) is read by LPR lanes with 16-byte loads,
// the q.k dot product is reduced across those lanes with xor shuffles, and
// every lane group keeps an online-softmax state (running max m, running sum l,
// and its slice of the weighted V accumulator).  Rows are gathered straight
// from the cache through the index list (no staging copy in HBM).
//
// Each lane group keeps 8 rows of K and V in flight at once and folds them into
// its running state with one rescale per 8 rows.  Split-K: when there are too
// few (b, h) units to fill the chip, the selected rows of one (b, h) are cut
// into splits of at least 128 rows, one workgroup each.  Lane groups of a
// workgroup are merged through LDS; splits are merged by k_attn_combine with
// the usual (m, l, acc) rescaling.
#include <cmath>

#include "ig_device.h"
#include "ig_internal.h"

namespace ig {

constexpr int kAttnThreads = 256;
constexpr int kAttnUnroll = 8;  // rows per lane group in flight at once (K and V: 16 x 16 bytes per lane)


template <typename T, int LPR>
__global__ __launch_bounds__(kAttnThreads) void k_attn_split(
    const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V, int ld_rows,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int d, int max_out,
    int rows_per_split, int nsplit, float scale, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part) {
    constexpr int VEC = Vec<T>::N;
    constexpr int G = kAttnThreads / LPR;  // lane groups (one row each) per workgroup
    constexpr int U = kAttnUnroll;
    __shared__ float s_m[G], s_l[G];
    __shared__ float s_acc[G * LPR * VEC];

    const int bh = blockIdx.y, split = blockIdx.x, tid = threadIdx.x;
    const int li = tid % LPR, gi = tid / LPR;
    // round trip 1: the count, the query slice and the first batch of indices are loaded together
    // (indices past the count are loaded from the idx row and ignored)
    const int c_raw = count[bh];
    const uint4 qraw = load_raw16(q + static_cast<size_t>(bh) * d + li * VEC);
    const int32_t* irow = idx ? idx + static_cast<size_t>(bh) * max_out : nullptr;
    const int r0 = split * rows_per_split;
    const int rcap = min(max_out, r0 + rows_per_split);
    int ipre[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = r0 + u * G + gi;
        ipre[u] = (irow && i < rcap) ? irow[i] : i;
    }
    int c = min(c_raw, max_out);
    if (!idx) c = min(c, ld_rows);
    const int r1 = min(c, rcap);

    float qv[VEC];
    unpack_raw(qraw, qv);
#pragma unroll
    for (int v = 0; v < VEC; ++v) qv[v] *= scale;

    const T* Kh = K + static_cast<size_t>(bh) * ld_rows * d + li * VEC;
    const T* Vh = V + static_cast<size_t>(bh) * ld_rows * d + li * VEC;
    float m = -INFINITY, l = 0.f, acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

    for (int ib = r0; ib < r1; ib += G * U) {
        int rows[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = ib + u * G + gi;
            int row = -1;
            if (i < r1) row = min(max(ib == r0 ? ipre[u] : (irow ? irow[i] : i), 0), ld_rows - 1);
            rows[u] = row;
        }
        // round trip 2: every K and V row slice of this batch in flight at once
        uint4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (rows[u] >= 0) {
                kr[u] = load_raw16(Kh + static_cast<size_t>(rows[u]) * d);
                vr[u] = load_raw16(Vh + static_cast<size_t>(rows[u]) * d);
            } else {
                kr[u] = make_uint4(0, 0, 0, 0);
                vr[u] = make_uint4(0, 0, 0, 0);
            }
        }
        float sc[U];
        float mb = m;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kv[VEC];
            unpack_raw(kr[u], kv);
            float s = 0.f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) s = fmaf(qv[v], kv[v], s);
            s = group_sum<LPR>(s);
            sc[u] = rows[u] >= 0 ? s : -INFINITY;
            mb = fmaxf(mb, sc[u]);
        }
        if (mb != -INFINITY) {  // this lane group has at least one live row (now or before)
            const float corr = __expf(m - mb);  // m = -inf before the first row: exp(-inf) = 0
            l *= corr;
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] *= corr;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pw = __expf(sc[u] - mb);  // dead rows: exp(-inf) = 0
                float vv[VEC];
                unpack_raw(vr[u], vv);
                l += pw;
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = fmaf(pw, vv[v], acc[v]);
            }
            m = mb;
        }
    }
    if (li == 0) {
        s_m[gi] = m;
        s_l[gi] = l;
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) s_acc[gi * LPR * VEC + li * VEC + v] = acc[v];
    __syncthreads();

    // merge the lane groups: thread t owns output element t of the d values
    for (int t = tid; t < d; t += kAttnThreads) {
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g) M = fmaxf(M, s_m[g]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll 4
            for (int g = 0; g < G; ++g) {
                const float w = (s_m[g] == -INFINITY) ? 0.f : __expf(s_m[g] - M);
                L += s_l[g] * w;
                A += s_acc[g * LPR * VEC + t] * w;
            }
        }
        if (nsplit == 1) {
            out[static_cast<size_t>(bh) * d + t] = L > 0.f ? A / L : 0.f;
            if (lse && t == 0) lse[bh] = L > 0.f ? M + __logf(L) : -INFINITY;
        } else {
            float* pp = part + (static_cast<size_t>(bh) * nsplit + split) * (2 + d);
            if (t == 0) {
                pp[0] = M;
                pp[1] = L;
            }
            pp[2 + t] = A;
        }
    }
}

__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ part, int nsplit, int d,
                                                      float* __restrict__ out, float* __restrict__ lse) {
    const int bh = blockIdx.x;
    const float* pp = part + static_cast<size_t>(bh) * nsplit * (2 + d);
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pp[s * (2 + d)]);
    for (int t = threadIdx.x; t < d; t += blockDim.x) {
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int s = 0; s < nsplit; ++s) {
                const float ms = pp[s * (2 + d)];
                const float w = (ms == -INFINITY) ? 0.f : __expf(ms - M);
                L += pp[s * (2 + d) + 1] * w;
                A += pp[s * (2 + d) + 2 + t] * w;
            }
        }
        out[static_cast<size_t>(bh) * d + t] = L > 0.f ? A / L : 0.f;
        if (lse && t == 0) lse[bh] = L > 0.f ? M + __logf(L) : -INFINITY;
    }
}

AttnPlan plan_attn(int B, int H, int d, int max_out) {
    AttnPlan p{};
    const int64_t bh = static_cast<int64_t>(B) * H;
    // one workgroup per (b, h) when there are enough of them to fill the chip; otherwise split the
    // selected rows so that about 512 workgroups run, each with at least 128 rows
    int64_t nsplit = 1;
    if (bh < 256) {
        nsplit = (512 + bh - 1) / bh;
        nsplit = std::max<int64_t>(1, std::min<int64_t>(nsplit, (max_out + 127) / 128));
    }
    int64_t rps = (max_out + nsplit - 1) / nsplit;
    rps = ((rps + 15) / 16) * 16;
    p.rows_per_split = static_cast<int>(rps);
    p.nsplit = static_cast<int>((max_out + rps - 1) / rps);
    p.ws_bytes = p.nsplit > 1 ? static_cast<size_t>(B) * H * p.nsplit * (2 + d) * sizeof(float) : 0;
    return p;
}

template <typename T>
static int launch_attn_t(const T* q, const T* K, const T* V, int ld_rows, const int32_t* idx, const int32_t* count,
                         int B, int H, int d, int max_out, float scale, float* out, float* lse, float* part,
                         const AttnPlan& p, hipStream_t s) {
    constexpr int VEC = Vec<T>::N;
    const dim3 grid(p.nsplit, B * H);
#define IG_ATTN_CASE(L)                                                                                   \
    case L:                                                                                               \
        hipLaunchKernelGGL((k_attn_split<T, L>), grid, dim3(kAttnThreads), 0, s, q, K, V, ld_rows, idx, \
                           count, d, max_out, p.rows_per_split, p.nsplit, scale, out, lse, part);        \
        break;
    switch (d / VEC) {
        IG_ATTN_CASE(4)
        IG_ATTN_CASE(8)
        IG_ATTN_CASE(16)
        IG_ATTN_CASE(32)
        default: return static_cast<int>(hipErrorInvalidValue);
    }
#undef IG_ATTN_CASE
    int e = static_cast<int>(hipGetLastError());
    if (e || p.nsplit == 1) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(B * H), dim3(std::min(256, d)), 0, s, part, p.nsplit, d, out, lse);
    return static_cast<int>(hipGetLastError());
}

int launch_attn(const void* q, const void* K, const void* V, int ld_rows, const int32_t* idx, const int32_t* count,
                int B, int H, int d, int max_out, int dtype, float scale, float* out, float* lse, void* ws,
                hipStream_t s) {
    const AttnPlan p = plan_attn(B, H, d, max_out);
    float* part = static_cast<float*>(ws);
    if (dtype == IG_BF16)
        return launch_attn_t(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                             static_cast<const uint16_t*>(V), ld_rows, idx, count, B, H, d, max_out, scale, out,
                             lse, part, p, s);
    return launch_attn_t(static_cast<const float*>(q), static_cast<const float*>(K), static_cast<const float*>(V),
                         ld_rows, idx, count, B, H, d, max_out, scale, out, lse, part, p, s);
}

}  // namespace ig
