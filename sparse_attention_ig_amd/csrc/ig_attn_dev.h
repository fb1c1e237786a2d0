// Attention over the selected rows of one (b, h), one split of them (InfiniGen,
// arXiv 2406.19707, paper-graph-ui summary, section 3.2 Inference Controller;
// section 2, softmax(QK^T)V over the cached rows), as a device function for NT
// threads: the standalone attention kernel runs it with 256, the fused decode
// kernel with 1024.
//
// Decode attention with one query per (b, h) and its own index set is a set of
// matrix-vector products, not a dense contraction, so it runs on the vector
// ALUs: a row of K or V (d elements) is read by LPR lanes with 16-byte loads,
// the q.k dot product is reduced across those lanes with DPP moves, and every
// lane group keeps an online-softmax state (running max m, running sum l, and
// its slice of the weighted V accumulator).  Rows are gathered straight from
// the cache through the index list (no staging copy in HBM).  Each lane group
// keeps 8 rows of K and V in flight at once and folds them into its running
// state with one rescale per 8 rows.  Lane groups are merged through LDS;
// splits of one (b, h) are merged by k_attn_combine with the usual (m, l, acc)
// rescaling.
#pragma once

#include <cmath>

#include "ig_device.h"

namespace ig {

constexpr int kAttnUnroll = 8;  // default rows per lane group in flight at once (K and V: 16 x 16 bytes per lane)

struct AttnArgs {
    const void* q;
    const void* K;
    const void* V;
    int ld_rows;
    const int32_t* idx;     // NULL: rows 0 .. count-1
    const int32_t* count;
    int d, max_out, rows_per_split, nsplit;
    float scale;
    float* out;
    float* lse;
    float* part;            // [B*H][nsplit][2 + d] when nsplit > 1
};

template <int NT, int LPR, int VEC>
struct AttnShared {
    static constexpr int G = NT / LPR;
    float m[G], l[G];
    float acc[G * LPR * VEC];
};

template <typename T, int LPR, int NT, int U = kAttnUnroll>
__device__ __forceinline__ void attn_item(const AttnArgs& a, int bh, int split, AttnShared<NT, LPR, Vec<T>::N>& sm) {
    constexpr int VEC = Vec<T>::N;
    constexpr int G = NT / LPR;  // lane groups (one row each) per workgroup
    const T* __restrict__ q = static_cast<const T*>(a.q);
    const T* __restrict__ K = static_cast<const T*>(a.K);
    const T* __restrict__ V = static_cast<const T*>(a.V);
    const int32_t* __restrict__ idx = a.idx;
    const int32_t* __restrict__ count = a.count;
    const int ld_rows = a.ld_rows, d = a.d, max_out = a.max_out, rows_per_split = a.rows_per_split;
    const int nsplit = a.nsplit;
    const float scale = a.scale;
    float* __restrict__ out = a.out;
    float* __restrict__ lse = a.lse;
    float* __restrict__ part = a.part;
    float* s_m = sm.m;
    float* s_l = sm.l;
    float* s_acc = sm.acc;
    const int tid = threadIdx.x;
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
    for (int t = tid; t < d; t += NT) {
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

// The split-K combine of one (b, h): the splits' (m, l, acc) rescaled to the largest m and added, then
// o = acc / l and lse = m + log l.  Run by the threads t < d of a workgroup (each owns output element t).
struct CombineArgs {
    const float* part;   // [B*H][nsplit][2 + d]; NULL: nothing to combine
    int nsplit, d;
    float* out;
    float* lse;
};

__device__ __forceinline__ void combine_item(const CombineArgs& c, int bh) {
    const int nsplit = c.nsplit, d = c.d;
    const float* pp = c.part + static_cast<size_t>(bh) * nsplit * (2 + d);
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
        c.out[static_cast<size_t>(bh) * d + t] = L > 0.f ? A / L : 0.f;
        if (c.lse && t == 0) c.lse[bh] = L > 0.f ? M + __logf(L) : -INFINITY;
    }
}

// The same combine with the splits' partials loaded ahead (at most kCombinePre splits): combine_load
// issues the loads into registers, combine_store adds them exactly as combine_item does (splits in
// order), so a workgroup can start the loads before other work and finish the combine after it.
constexpr int kCombinePre = 8;
struct CombinePre {
    float m[kCombinePre], l[kCombinePre], a[kCombinePre];
};

__device__ __forceinline__ void combine_load(const CombineArgs& c, int bh, CombinePre& pre) {
    const int t = threadIdx.x, d = c.d;
    const float* pp = c.part + static_cast<size_t>(bh) * c.nsplit * (2 + d);
#pragma unroll
    for (int s = 0; s < kCombinePre; ++s) {
        const bool on = s < c.nsplit && t < d;
        pre.m[s] = on ? pp[s * (2 + d)] : -INFINITY;
        pre.l[s] = on ? pp[s * (2 + d) + 1] : 0.f;
        pre.a[s] = on ? pp[s * (2 + d) + 2 + t] : 0.f;
    }
}

__device__ __forceinline__ void combine_store(const CombineArgs& c, int bh, const CombinePre& pre) {
    const int t = threadIdx.x, d = c.d;
    if (t >= d) return;
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kCombinePre; ++s) M = fmaxf(M, pre.m[s]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int s = 0; s < kCombinePre; ++s) {
            if (s < c.nsplit) {
                const float ms = pre.m[s];
                const float w = (ms == -INFINITY) ? 0.f : __expf(ms - M);
                L += pre.l[s] * w;
                A += pre.a[s] * w;
            }
        }
    }
    c.out[static_cast<size_t>(bh) * d + t] = L > 0.f ? A / L : 0.f;
    if (c.lse && t == 0) c.lse[bh] = L > 0.f ? M + __logf(L) : -INFINITY;
}

}  // namespace ig
